// sscan_multi.hip -- scans of a 2-D feature map along several visiting orders.
//
// A [height, width] map is flattened row-major (token t = r * width + c).  Each
// direction visits the tokens in its own order -- by rows, by columns, or along a
// caller-given permutation, forward or reversed (Mamba in the YOLO26 backbone
// page, sections 1.2, 2.2 and 4.4: row, column and crosswise scans, four
// directions; Samba page, section 3.1: a centre-out spiral) -- with its own
// parameters; every direction's output lands at the tokens' own positions, the
// directions are summed and the gate is applied once.
//
// Directions are grouped by family (row, column, index).  A family's forward and
// reverse directions run as one two-direction scan (the bidirectional kernels of
// sscan_kernels.hip, without the gate) on inputs gathered into the family's
// visiting order: nothing to gather for rows; an LDS-tiled transpose for columns
// (the column order of an H x W map is the row order of its W x H transpose);
// a gather through the index for permutations.  Each family's output is put back
// at the token positions and summed into an fp32 accumulator in a fixed order
// (rows, columns, index); a last pass gates it and stores the result.
#include "sscan_internal.h"

#include <algorithm>
#include <cstring>

namespace sscan {
namespace {

constexpr int kTT = 32;  // transpose tile

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }
__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 x = {v, 0.0f};
  p[i] = uint16_t(__builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2)) & 0xffffu);
}

// What a put-back does with the accumulator.
enum Put : int { kCopy = 0, kSet = 1, kAdd = 2 };

// out[row][c][r] = in[row][r][c] for every row of [rows][h][w] (kCopy, same type),
// or acc[row][c][r] = / += in[row][r][c] (kSet / kAdd into fp32).  Grid:
// (ceil(w/32), ceil(h/32), up to 65535 row slots striding over the rows); block 32 x 8.
constexpr int64_t kMaxGridZ = 65535;

template <typename TI, typename TO, int PUT>
__global__ __launch_bounds__(256) void transpose_kernel(const TI* __restrict__ in, TO* __restrict__ out, int64_t rows,
                                                        int64_t h, int64_t w) {
  __shared__ float tile[kTT][kTT + 1];
  const int64_t c0 = int64_t(blockIdx.x) * kTT, r0 = int64_t(blockIdx.y) * kTT;
  for (int64_t row = blockIdx.z; row < rows; row += gridDim.z) {
    const TI* src = in + row * h * w;
    TO* dst = out + row * h * w;
    __syncthreads();  // the previous row's tile has been read out
    for (int k = threadIdx.y; k < kTT; k += 8) {
      const int64_t r = r0 + k, c = c0 + threadIdx.x;
      tile[k][threadIdx.x] = (r < h && c < w) ? ld(src, r * w + c) : 0.0f;
    }
    __syncthreads();
    for (int k = threadIdx.y; k < kTT; k += 8) {
      const int64_t c = c0 + k, r = r0 + threadIdx.x;
      if (r < h && c < w) {
        const float v = tile[threadIdx.x][k];
        const int64_t o = c * h + r;
        if (PUT == kAdd) {
          st(dst, o, ld(dst, o) + v);
        } else {
          st(dst, o, v);
        }
      }
    }
  }
}

dim3 transpose_grid(int64_t rows, int64_t h, int64_t w) {
  return dim3(unsigned((w + kTT - 1) / kTT), unsigned((h + kTT - 1) / kTT), unsigned(std::min(rows, kMaxGridZ)));
}

// out[row][s] = in[row][index[s]]; entries outside [0, len) read as 0.
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                     const int32_t* __restrict__ index, int64_t rows, int64_t len) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * len) return;
  const int64_t row = i / len, s = i % len;
  const int64_t p = index[s];
  st(out, i, (p >= 0 && p < len) ? ld(in, row * len + p) : 0.0f);
}

// acc[row][index[s]] = / += y[row][s] (index a permutation; entries outside
// [0, len) are skipped).  With index == nullptr the identity.
template <typename T, int PUT>
__global__ __launch_bounds__(256) void put_kernel(const T* __restrict__ y, float* __restrict__ acc,
                                                  const int32_t* __restrict__ index, int64_t rows, int64_t len) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * len) return;
  const int64_t row = i / len, s = i % len;
  const int64_t p = index ? int64_t(index[s]) : s;
  if (p < 0 || p >= len) return;
  const float v = ld(y, i);
  float* o = acc + row * len + p;
  *o = PUT == kAdd ? *o + v : v;
}

// y = acc * silu(z) (or acc), in the I/O dtype.
template <typename T>
__global__ __launch_bounds__(256) void gate_kernel(const float* __restrict__ acc, const T* __restrict__ z,
                                                   T* __restrict__ y, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float v = acc[i];
  if (z) {
    const float zv = ld(z, i);
    // silu(z) = z / (1 + 2^(-z log2 e)), as in the scan kernels
    v *= zv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * 1.4426950408889634f));
  }
  st(y, i, v);
}

unsigned blocks_for(int64_t n) { return unsigned((n + 255) / 256); }

template <typename T>
void launch_transpose(const void* in, void* out, int64_t rows, int64_t h, int64_t w, hipStream_t s) {
  hipLaunchKernelGGL((transpose_kernel<T, T, kCopy>), transpose_grid(rows, h, w), dim3(kTT, 8), 0, s,
                     static_cast<const T*>(in), static_cast<T*>(out), rows, h, w);
}

template <typename T>
void launch_gather(const void* in, void* out, const int32_t* index, int64_t rows, int64_t len, hipStream_t s) {
  hipLaunchKernelGGL((gather_kernel<T>), dim3(blocks_for(rows * len)), dim3(256), 0, s, static_cast<const T*>(in),
                     static_cast<T*>(out), index, rows, len);
}

// Gathers one [rows][len] tensor into a family's visiting order (forward order;
// the reverse directions scan the same sequence backwards).
void gather_family(int family, bool bf16, const void* in, void* out, const int32_t* index, int64_t rows,
                   int64_t h, int64_t w, hipStream_t s) {
  if (family == kFamilyCol) {
    if (bf16) {
      launch_transpose<uint16_t>(in, out, rows, h, w, s);
    } else {
      launch_transpose<float>(in, out, rows, h, w, s);
    }
  } else if (bf16) {
    launch_gather<uint16_t>(in, out, index, rows, h * w, s);
  } else {
    launch_gather<float>(in, out, index, rows, h * w, s);
  }
}

template <typename T>
void put_family(int family, const void* y, float* acc, const int32_t* index, int64_t rows, int64_t h, int64_t w,
                bool first, hipStream_t s) {
  const T* yy = static_cast<const T*>(y);
  if (family == kFamilyCol) {
    // y is in column order: the [w][h] map transposed back onto [h][w]
    const dim3 grid = transpose_grid(rows, w, h);
    if (first) {
      hipLaunchKernelGGL((transpose_kernel<T, float, kSet>), grid, dim3(kTT, 8), 0, s, yy, acc, rows, w, h);
    } else {
      hipLaunchKernelGGL((transpose_kernel<T, float, kAdd>), grid, dim3(kTT, 8), 0, s, yy, acc, rows, w, h);
    }
  } else {
    const int32_t* idx = family == kFamilyIndex ? index : nullptr;
    if (first) {
      hipLaunchKernelGGL((put_kernel<T, kSet>), dim3(blocks_for(rows * h * w)), dim3(256), 0, s, yy, acc, idx, rows,
                         h * w);
    } else {
      hipLaunchKernelGGL((put_kernel<T, kAdd>), dim3(blocks_for(rows * h * w)), dim3(256), 0, s, yy, acc, idx, rows,
                         h * w);
    }
  }
}

}  // namespace

MultiPlan make_multi_plan(int64_t batch, int64_t dim, int64_t height, int64_t width, const int* kinds, int ndir,
                          bool io_bf16, bool bc_bf16) {
  MultiPlan p{};
  const int64_t len = height * width;
  const size_t io = io_bf16 ? 2 : 4, bc = bc_bf16 ? 2 : 4;
  auto up = [](size_t n) { return (n + 255) / 256 * 256; };
  size_t scan = 0;
  for (int f = 0; f < kFamilies; ++f) {
    int n = 0;
    for (int k = 0; k < ndir; ++k) n += kinds[k] / 2 == f;
    if (n > 0) scan = std::max(scan, make_plan(batch, dim, len, n).workspace_bytes);
  }
  size_t off = 0;
  p.off_acc = off;
  off += up(size_t(batch) * dim * len * 4);
  p.off_y = off;
  off += up(size_t(batch) * dim * len * 4);  // fp32 partial output
  p.off_u = off;
  off += up(size_t(batch) * dim * len * io);
  for (int j = 0; j < 2; ++j) {
    p.off_delta[j] = off;
    off += up(size_t(batch) * dim * len * io);
    p.off_B[j] = off;
    off += up(size_t(batch) * kDState * len * bc);
    p.off_C[j] = off;
    off += up(size_t(batch) * kDState * len * bc);
  }
  p.off_scan = off;
  off += up(scan);
  p.workspace_bytes = off;
  return p;
}

hipError_t launch_multi(const MultiArgs& a, const MultiPlan& p, char* ws, hipStream_t stream) {
  const int64_t len = a.height * a.width;
  const int64_t rows = a.batch * a.dim, bc_rows = a.batch * kDState;
  float* acc = reinterpret_cast<float*>(ws + p.off_acc);
  bool first = true;
  for (int f = 0; f < kFamilies; ++f) {
    int idx[2] = {-1, -1};  // forward, reverse direction of this family
    for (int k = 0; k < a.ndir; ++k)
      if (a.kind[k] / 2 == f) idx[a.kind[k] % 2] = k;
    if (idx[0] < 0 && idx[1] < 0) continue;
    ScanArgs s;
    std::memset(&s, 0, sizeof(s));
    s.u = a.u;
    s.y = ws + p.off_y;
    s.y_f32 = 1;  // the families' outputs are summed before any rounding
    s.softplus = a.softplus;
    s.io_bf16 = a.io_bf16;
    s.bc_bf16 = a.bc_bf16;
    s.batch = a.batch;
    s.dim = a.dim;
    s.len = len;
    if (f != kFamilyRow) s.u = ws + p.off_u;
    if (f != kFamilyRow)
      gather_family(f, a.io_bf16, a.u, ws + p.off_u, a.index, rows, a.height, a.width, stream);
    int slot = 0;
    for (int j = 0; j < 2; ++j) {
      if (idx[j] < 0) continue;
      DirArgs d = a.dir[idx[j]];
      if (f != kFamilyRow) {
        gather_family(f, a.io_bf16, d.delta, ws + p.off_delta[slot], a.index, rows, a.height, a.width, stream);
        gather_family(f, a.bc_bf16, d.B, ws + p.off_B[slot], a.index, bc_rows, a.height, a.width, stream);
        gather_family(f, a.bc_bf16, d.C, ws + p.off_C[slot], a.index, bc_rows, a.height, a.width, stream);
        d.delta = ws + p.off_delta[slot];
        d.B = ws + p.off_B[slot];
        d.C = ws + p.off_C[slot];
      }
      s.dir[slot++] = d;
    }
    s.ndir = slot;
    s.reverse = (slot == 1 && idx[1] >= 0) ? 1 : 0;  // a lone reverse direction
    // for the gathered families the visiting order's tokens are in the order the
    // scan expects; a column map is a [width][height] map in that order
    const Plan plan = make_plan(a.batch, a.dim, len, s.ndir);
    hipError_t e = launch_scan(s, plan, reinterpret_cast<float*>(ws + p.off_scan), stream);
    if (e != hipSuccess) return e;
    put_family<float>(f, ws + p.off_y, acc, a.index, rows, a.height, a.width, first, stream);
    first = false;
  }
  const int64_t n = rows * len;
  if (a.io_bf16) {
    hipLaunchKernelGGL((gate_kernel<uint16_t>), dim3(blocks_for(n)), dim3(256), 0, stream, acc,
                       static_cast<const uint16_t*>(a.z), static_cast<uint16_t*>(a.y), n);
  } else {
    hipLaunchKernelGGL((gate_kernel<float>), dim3(blocks_for(n)), dim3(256), 0, stream, acc,
                       static_cast<const float*>(a.z), static_cast<float*>(a.y), n);
  }
  return hipGetLastError();
}

}  // namespace sscan
