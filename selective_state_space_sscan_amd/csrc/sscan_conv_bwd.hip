// sscan_conv_bwd.hip -- backward of the depthwise convolution in front of the scan
// (gfx950).  Training differentiates the block by hand (Reproducing Vision Mamba
// page, section 1.3; Hand-written simplified Mamba2 page, sections 4.4 and 5.1);
// given du = dLoss/du (float32) of the scan's input u = act(pre), pre[t] = bias +
// sum_j w[j] x[t - left + j] (x = 0 outside the row), with g = du * act'(pre):
//   dx[s]   = sum_j w[j] g[s + left - j]          (t = s + left - j inside the row)
//   dw[j]   = sum over batch rows and t of g[t] x[t - left + j]
//   dbias   = sum over batch rows and t of g[t]
// The taps sit in the same fixed five-token window as the forward's (x[t-3 .. t+1],
// zeros where the kernel has no tap), so every index below is a compile-time one.
// dx is written per run of eight tokens; a thread takes four runs (each pass of the
// wave covers 64 consecutive runs) and keeps its weight and bias sums in registers,
// which are then reduced over the wave with a fixed butterfly, stored per (run
// chunk, batch row, channel), and summed in a fixed order by a second kernel:
// results are bitwise reproducible (no atomics).
#include "sscan_device.h"

namespace sscan {
namespace {

constexpr int kRun = 8;                      // tokens per thread and pass
constexpr int kReps = 4;                     // passes per thread before the weight sums leave registers
constexpr int kRows = 4;                     // channels per block (one wave each)
constexpr int kParts = kConvTaps + 1;        // five window taps + bias per partial
constexpr int kXSpan = kRun + 8;             // x[t0 - 4 .. t0 + 12)
constexpr int kGSpan = kRun + 4;             // g[t0 - 1 .. t0 + 11)

__device__ __forceinline__ float wave_sum(float v) {
  // fixed butterfly over the 64 lanes (xor 1, 2, 4, 8, 16, 32)
#pragma unroll
  for (int m = 1; m < kLanes; m <<= 1) v += __shfl_xor(v, m, kLanes);
  return v;
}

template <bool IO_BF16, bool SILU>
__global__ __launch_bounds__(kLanes * kRows) void conv1d_bwd_kernel(ConvBwdArgs a, float* __restrict__ part, int vec,
                                                                    int duvec) {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  const int64_t chunk = blockIdx.x;
  for (int64_t d = int64_t(blockIdx.y) * kRows + threadIdx.y; d < a.dim; d += int64_t(gridDim.y) * kRows) {
    // tap k of the window multiplies x[t - 3 + k]: tap j of the kernel sits at k = 3 - left + j
    float cw[kConvTaps];
#pragma unroll
    for (int k = 0; k < kConvTaps; ++k) {
      const int j = k - (kConvBack - a.left);
      cw[k] = (j >= 0 && j < a.width) ? a.w[d * a.width + j] : 0.0f;
    }
    const float cb = a.b ? a.b[d] : 0.0f;
    for (int64_t b = blockIdx.z; b < a.batch; b += gridDim.z) {
      const int64_t row = (b * a.dim + d) * a.len;
      const T* x = static_cast<const T*>(a.x) + row;
      const float* du = a.du + row;
      auto ld = [&](const T* p, int64_t t) { return (t >= 0 && t < a.len) ? IO::load(p, t) : 0.0f; };
      auto ldu = [&](int64_t t) { return (t >= 0 && t < a.len) ? du[t] : 0.0f; };
      // the weight and bias sums of this thread's kReps runs (each pass of the wave
      // covers 64 consecutive runs)
      float ps[kParts];
#pragma unroll
      for (int k = 0; k < kParts; ++k) ps[k] = 0.0f;
      for (int rep = 0; rep < kReps; ++rep) {
        const int64_t pass0 = (chunk * kReps + rep) * kLanes * kRun;  // first token of this pass
        if (pass0 >= a.len) break;                                      // wave-uniform
        const int64_t t0 = pass0 + int64_t(threadIdx.x) * kRun;       // may be past the row's end (zeros)
        const bool full = vec && t0 + kRun <= a.len;
        float xs[kXSpan];  // x[t0 - 4 + i]
        float gs[kGSpan];  // g[t0 - 1 + i]
        if (full) {
          if (IO_BF16) {
            const uint4 v = *reinterpret_cast<const uint4*>(x + t0);
            const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              xs[4 + 2 * k] = bf16_lo(ws[k]);
              xs[5 + 2 * k] = bf16_hi(ws[k]);
            }
          } else {
            const float4* p = reinterpret_cast<const float4*>(x + t0);
            const float4 v0 = p[0], v1 = p[1];
            const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) xs[4 + k] = f[k];
          }
        } else {
#pragma unroll
          for (int k = 0; k < kRun; ++k) xs[4 + k] = ld(x, t0 + k);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          xs[k] = ld(x, t0 - 4 + k);
          xs[kRun + 4 + k] = ld(x, t0 + kRun + k);
        }
        // du over t0 - 1 .. t0 + 10: the run's own eight as two 16-byte loads where the
        // rows allow, the halo as single loads
        float dus[kGSpan];
        if (full && duvec) {
          const float4* q = reinterpret_cast<const float4*>(du + t0);
          const float4 v0 = q[0], v1 = q[1];
          dus[1] = v0.x, dus[2] = v0.y, dus[3] = v0.z, dus[4] = v0.w;
          dus[5] = v1.x, dus[6] = v1.y, dus[7] = v1.z, dus[8] = v1.w;
        } else {
#pragma unroll
          for (int k = 0; k < kRun; ++k) dus[1 + k] = ldu(t0 + k);
        }
        dus[0] = ldu(t0 - 1);
#pragma unroll
        for (int k = 0; k < kGSpan - 1 - kRun; ++k) dus[1 + kRun + k] = ldu(t0 + kRun + k);
        // g over t = t0 - 1 + i: pre from the window x[t - 3 .. t + 1] = xs[i .. i + 4]
#pragma unroll
        for (int i = 0; i < kGSpan; ++i) {
          const float d_u = dus[i];
          if (SILU) {
            float pre = cb;
#pragma unroll
            for (int k = 0; k < kConvTaps; ++k) pre = fmaf(cw[k], xs[i + k], pre);
            const float s = rcp_hw(1.0f + exp2_hw(-pre * kLog2e));
            gs[i] = d_u * (s * fmaf(pre, 1.0f - s, 1.0f));
          } else {
            gs[i] = d_u;
          }
        }
        // dx[t0 + m] = sum_k cw[k] g[t0 + m + 3 - k] = sum_k cw[k] gs[m + 4 - k]
        float dxo[kRun];
#pragma unroll
        for (int m = 0; m < kRun; ++m) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < kConvTaps; ++k) acc = fmaf(cw[k], gs[m + 4 - k], acc);
          dxo[m] = acc;
        }
        T* dx = static_cast<T*>(a.dx) + row;
        if (full) {
          if (IO_BF16) {
            *reinterpret_cast<uint4*>(dx + t0) = make_uint4(pack_bf16x2(dxo[0], dxo[1]), pack_bf16x2(dxo[2], dxo[3]),
                                                            pack_bf16x2(dxo[4], dxo[5]), pack_bf16x2(dxo[6], dxo[7]));
          } else {
            float4* p = reinterpret_cast<float4*>(dx + t0);
            p[0] = make_float4(dxo[0], dxo[1], dxo[2], dxo[3]);
            p[1] = make_float4(dxo[4], dxo[5], dxo[6], dxo[7]);
          }
        } else {
#pragma unroll
          for (int m = 0; m < kRun; ++m)
            if (t0 + m < a.len) IO::store(dx, t0 + m, dxo[m]);
        }
        // this run's share of the weight and bias sums: t = t0 + m inside the row (g is
        // zero outside it), window x[t - 3 + k] = xs[m + 1 + k]
#pragma unroll
        for (int m = 0; m < kRun; ++m) {
          const float g = gs[m + 1];
#pragma unroll
          for (int k = 0; k < kConvTaps; ++k) ps[k] = fmaf(g, xs[m + 1 + k], ps[k]);
          ps[kConvTaps] += g;
        }
      }
#pragma unroll
      for (int k = 0; k < kParts; ++k) ps[k] = wave_sum(ps[k]);
      if (threadIdx.x < kParts) {
        float v = ps[0];
#pragma unroll
        for (int k = 1; k < kParts; ++k) v = (int(threadIdx.x) == k) ? ps[k] : v;
        part[((size_t(chunk) * a.batch + b) * a.dim + d) * kParts + threadIdx.x] = v;
      }
    }
  }
}

// dw and dbias: per (channel, window tap), the partials of every (run chunk, batch
// row) summed in that order.
__global__ __launch_bounds__(256) void conv1d_bwd_reduce_kernel(ConvBwdArgs a, const float* __restrict__ part,
                                                                int64_t nchunk) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.dim * kParts) return;
  const int64_t d = i / kParts;
  const int k = int(i % kParts);
  const int j = k - (kConvBack - a.left);
  if (k < kConvTaps && (j < 0 || j >= a.width)) return;  // a window slot without a tap
  double acc = 0.0;
  for (int64_t c = 0; c < nchunk; ++c)
    for (int64_t b = 0; b < a.batch; ++b) acc += part[((size_t(c) * a.batch + b) * a.dim + d) * kParts + k];
  if (k == kConvTaps) {
    if (a.db) a.db[d] = float(acc);
  } else {
    a.dw[d * a.width + j] = float(acc);
  }
}

__global__ __launch_bounds__(256) void conv1d_bwd_zero_kernel(ConvBwdArgs a) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < a.dim * a.width) a.dw[i] = 0.0f;
  if (a.db && i < a.dim) a.db[i] = 0.0f;
}

bool aligned16_c(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int64_t conv_bwd_chunks(int64_t len) {
  const int64_t runs = (len + kRun - 1) / kRun;
  return std::max<int64_t>(1, (runs + kLanes * kReps - 1) / (kLanes * kReps));
}

size_t conv_bwd_partial_floats(int64_t batch, int64_t dim, int64_t len) {
  return size_t(conv_bwd_chunks(len)) * size_t(batch) * size_t(dim) * kParts;
}

hipError_t launch_conv1d_bwd(const ConvBwdArgs& a, float* part, hipStream_t stream) {
  if (a.batch == 0 || a.len == 0) {
    if (a.dim > 0)
      hipLaunchKernelGGL(conv1d_bwd_zero_kernel, dim3(unsigned((a.dim * a.width + 255) / 256)), dim3(256), 0, stream,
                         a);
    return hipGetLastError();
  }
  constexpr int64_t kMaxGridYZ = 65535;
  const int64_t nchunk = conv_bwd_chunks(a.len);
  const int64_t quads = (a.dim + kRows - 1) / kRows;
  const dim3 grid(unsigned(nchunk), unsigned(std::min(quads, kMaxGridYZ)), unsigned(std::min(a.batch, kMaxGridYZ)));
  const dim3 block(kLanes, kRows);
  const size_t esz = a.io_bf16 ? 2 : 4;
  const int vec = (size_t(a.len) * esz) % 16 == 0 && aligned16_c(a.x) && aligned16_c(a.dx);
  const int duvec = vec && a.len % 4 == 0 && aligned16_c(a.du);
  if (a.io_bf16) {
    if (a.silu) {
      hipLaunchKernelGGL((conv1d_bwd_kernel<true, true>), grid, block, 0, stream, a, part, vec, duvec);
    } else {
      hipLaunchKernelGGL((conv1d_bwd_kernel<true, false>), grid, block, 0, stream, a, part, vec, duvec);
    }
  } else {
    if (a.silu) {
      hipLaunchKernelGGL((conv1d_bwd_kernel<false, true>), grid, block, 0, stream, a, part, vec, duvec);
    } else {
      hipLaunchKernelGGL((conv1d_bwd_kernel<false, false>), grid, block, 0, stream, a, part, vec, duvec);
    }
  }
  hipLaunchKernelGGL(conv1d_bwd_reduce_kernel, dim3(unsigned((a.dim * kParts + 255) / 256)), dim3(256), 0, stream, a,
                     static_cast<const float*>(part), nchunk);
  return hipGetLastError();
}

}  // namespace sscan
