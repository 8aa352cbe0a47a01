/*
 * sscan_oracle_conv.c -- plain fp64 depthwise 1-D convolution in front of the scan.
 *
 * TEST INFRASTRUCTURE ONLY (see sscan_oracle.c).  Shares no code with the HIP path.
 *
 * Each channel is convolved with its own kernel of `width` taps before the scan
 * (Hand-written simplified Mamba2 page, section 4.4: a depthwise Conv1d of d_conv
 * taps, padded by d_conv - 1 and cut back to the sequence length, i.e. causal;
 * Reproducing Vision Mamba page, section 3.2: kernel 3 with 'same' padding so 197
 * tokens stay 197).  Cross-correlation as in those layers:
 *   causal: out[t] = bias + sum_{j<width} w[j] * x[t - (width-1) + j]
 *   same:   out[t] = bias + sum_{j<width} w[j] * x[t - (width-1)/2 + j]   (odd width)
 * with x = 0 outside [0, len), then optionally silu(out).
 * Layouts: x, out [batch, dim, len]; w [dim, width]; bias [dim] (nullable).
 */
#include <math.h>
#include <stdint.h>

int oracle_conv1d(const double* x, const double* w, const double* bias, double* out, int64_t batch, int64_t dim,
                  int64_t len, int64_t width, int same, int silu) {
    if (batch < 0 || dim < 0 || len < 0 || width < 1) return -2;
    if (same && width % 2 == 0) return -3;
    const int64_t left = same ? (width - 1) / 2 : width - 1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const double* xr = x + (b * dim + d) * len;
            double* o = out + (b * dim + d) * len;
            for (int64_t t = 0; t < len; ++t) {
                double acc = bias ? bias[d] : 0.0;
                for (int64_t j = 0; j < width; ++j) {
                    const int64_t s = t - left + j;
                    if (s >= 0 && s < len) acc += w[d * width + j] * xr[s];
                }
                o[t] = silu ? acc / (1.0 + exp(-acc)) : acc;
            }
        }
    }
    return 0;
}
