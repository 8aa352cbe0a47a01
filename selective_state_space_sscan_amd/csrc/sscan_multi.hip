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
// a gather through the index for permutations.  Each family's fp32 output is put
// back at the token positions and summed into an fp32 accumulator in a fixed order
// (rows, columns, index; the row family scans straight into it), and the last
// family's put-back applies the gate and stores the result.
#include "sscan_internal.h"

#include <algorithm>
#include <type_traits>
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

// out[row][c][r] = in[row][r][c] for every row of [rows][h][w].  Grid:
// (ceil(w/32), ceil(h/32), up to 65535 row slots striding over the rows); block 32 x 8.
constexpr int64_t kMaxGridZ = 65535;

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, T* __restrict__ out, int64_t rows,
                                                        int64_t h, int64_t w) {
  __shared__ float tile[kTT][kTT + 1];
  const int64_t c0 = int64_t(blockIdx.x) * kTT, r0 = int64_t(blockIdx.y) * kTT;
  for (int64_t row = blockIdx.z; row < rows; row += gridDim.z) {
    const T* src = in + row * h * w;
    T* dst = out + row * h * w;
    __syncthreads();  // the previous row's tile has been read out
    for (int k = threadIdx.y; k < kTT; k += 8) {
      const int64_t r = r0 + k, c = c0 + threadIdx.x;
      tile[k][threadIdx.x] = (r < h && c < w) ? ld(src, r * w + c) : 0.0f;
    }
    __syncthreads();
    for (int k = threadIdx.y; k < kTT; k += 8) {
      const int64_t c = c0 + k, r = r0 + threadIdx.x;
      if (r < h && c < w) st(dst, c * h + r, tile[threadIdx.x][k]);
    }
  }
}

dim3 transpose_grid(int64_t rows, int64_t h, int64_t w) {
  return dim3(unsigned((w + kTT - 1) / kTT), unsigned((h + kTT - 1) / kTT), unsigned(std::min(rows, kMaxGridZ)));
}

// The same for bf16 maps with even sides, on 64 x 64 tiles moving element pairs:
// a thread loads two neighbours of a row as one 4-byte word and stores two
// neighbours of an output row as one word (128 contiguous bytes per 32 lanes
// either way, where single 2-byte elements give 64).  The LDS tile keeps the loaded
// words; a column's pair is taken from two of them.  Block 32 x 8.
constexpr int kPT = 64;

__device__ __forceinline__ uint32_t half_of(uint32_t w, int hi) { return hi ? w >> 16 : w & 0xffffu; }

// two floats rounded to bf16 (nearest even) in one word, lo in the low half
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2));
}

__global__ __launch_bounds__(256) void transpose_pairs_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                              int64_t rows, int64_t h, int64_t w) {
  __shared__ uint32_t tile[kPT][kPT / 2 + 1];  // [row in tile][column pair]
  const int64_t c0 = int64_t(blockIdx.x) * kPT, r0 = int64_t(blockIdx.y) * kPT;
  const int tx = threadIdx.x, ty = threadIdx.y;
  for (int64_t row = blockIdx.z; row < rows; row += gridDim.z) {
    const uint16_t* src = in + row * h * w;
    uint16_t* dst = out + row * h * w;
    __syncthreads();  // the previous row's tile has been read out
    for (int k = ty; k < kPT; k += 8) {
      const int64_t r = r0 + k, c = c0 + 2 * tx;
      tile[k][tx] = (r < h && c < w) ? *reinterpret_cast<const uint32_t*>(src + r * w + c) : 0u;
    }
    __syncthreads();
    for (int k = ty; k < kPT; k += 8) {
      // output row c0 + k holds input column c0 + k; this thread's pair: input rows
      // r0 + 2 tx and r0 + 2 tx + 1
      const int64_t c = c0 + k, r = r0 + 2 * tx;
      if (c < w && r < h) {
        const uint32_t lo = half_of(tile[2 * tx][k >> 1], k & 1), hi = half_of(tile[2 * tx + 1][k >> 1], k & 1);
        *reinterpret_cast<uint32_t*>(dst + c * h + r) = lo | (hi << 16);
      }
    }
  }
}

dim3 pairs_grid(int64_t rows, int64_t h, int64_t w) {
  return dim3(unsigned((w + kPT - 1) / kPT), unsigned((h + kPT - 1) / kPT), unsigned(std::min(rows, kMaxGridZ)));
}

// The index family's kernels.  On large maps the gather takes one element per
// thread in flat (row, position) order, so the whole GPU works through a few
// channel rows at a time: the column runs of a spatial order (a spiral) read a new
// 128-byte line per element, and a channel row (a few hundred KB) stays in the
// caches while its lines are reused.  On small maps, and for the put-back (which
// reads through the inverse permutation and writes coalesced), a thread walks
// groups of kIndexRows rows with their loads in flight together, which measured
// faster there.
constexpr int kIndexRows = 4;

// The gather in row groups, for maps small enough that the flat order's cache
// reuse does not matter: a thread walks groups of kIndexRows rows with their loads
// in flight together (same result as gather_kernel).
template <typename T>
__global__ __launch_bounds__(256) void gather_rows_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                          const int32_t* __restrict__ index, int64_t rows,
                                                          int64_t len) {
  const int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (s >= len) return;
  const int64_t p = index[s];
  const bool valid = p >= 0 && p < len;
  const int64_t pp = valid ? p : 0;
  for (int64_t row0 = int64_t(blockIdx.y) * kIndexRows; row0 < rows; row0 += int64_t(gridDim.y) * kIndexRows) {
    float v[kIndexRows];
#pragma unroll
    for (int j = 0; j < kIndexRows; ++j) {
      const int64_t row = row0 + j;
      v[j] = (valid && row < rows) ? ld(in, row * len + pp) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kIndexRows; ++j)
      if (row0 + j < rows) st(out, (row0 + j) * len + s, v[j]);
  }
}

// out[row][s] = in[row][index[s]]; entries outside [0, len) read as 0.
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                     const int32_t* __restrict__ index, int64_t rows, int64_t len) {
  const int64_t n = rows * len;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t row = i / len, s = i - row * len;
    const int64_t p = index[s];
    st(out, i, (p >= 0 && p < len) ? ld(in, row * len + p) : 0.0f);
  }
}

// inv[p] = s for index[s] = p (inv filled with -1 first): the position at which
// the index family visits token p.
__global__ __launch_bounds__(256) void fill_kernel(int32_t* __restrict__ a, int64_t n, int32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) a[i] = v;
}
__global__ __launch_bounds__(256) void invert_kernel(const int32_t* __restrict__ index, int32_t* __restrict__ inv,
                                                     int64_t len) {
  for (int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x; s < len; s += int64_t(gridDim.x) * 256) {
    const int64_t p = index[s];
    if (p >= 0 && p < len) inv[p] = int32_t(s);
  }
}

__device__ __forceinline__ float silu_gate(float v, float zv) {
  // v * silu(z), silu(z) = z / (1 + 2^(-z log2 e)), as in the scan kernels
  return v * (zv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * 1.4426950408889634f)));
}

// Puts one family's fp32 output back at the token positions: FIRST sets the
// accumulator, later families add to it; the LAST family adds, gates and stores
// the result in the I/O dtype instead.  The index family reads, for token t, the
// value at the position inv[t] that visits it (nothing where no position does), so
// every store is coalesced and the permutation only scatters the reads.
template <typename TIO, bool FIRST, bool LAST>
__global__ __launch_bounds__(256) void put_index_kernel(const float* __restrict__ yf, float* __restrict__ acc,
                                                        const int32_t* __restrict__ inv, const TIO* __restrict__ z,
                                                        TIO* __restrict__ y, int64_t rows, int64_t len) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= len) return;
  const int64_t s = inv[t];
  for (int64_t row0 = int64_t(blockIdx.y) * kIndexRows; row0 < rows; row0 += int64_t(gridDim.y) * kIndexRows) {
    float yv[kIndexRows];
#pragma unroll
    for (int j = 0; j < kIndexRows; ++j) {
      const int64_t row = row0 + j;
      yv[j] = (s >= 0 && row < rows) ? yf[row * len + s] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kIndexRows; ++j) {
      const int64_t row = row0 + j;
      if (row >= rows) break;
      const int64_t o = row * len + t;
      const float v = FIRST ? yv[j] : acc[o] + yv[j];
      if (LAST) {
        st(y, o, z ? silu_gate(v, ld(z, o)) : v);
      } else {
        acc[o] = v;
      }
    }
  }
}

// The put-back's grid: x over token positions (256 per block), y over groups of
// kIndexRows rows (about 64K blocks, striding above that).
dim3 index_grid(int64_t rows, int64_t len) {
  const int64_t gx = (len + 255) / 256;
  const int64_t groups = (rows + kIndexRows - 1) / kIndexRows;
  const int64_t slots = std::min(std::min(groups, kMaxGridZ), std::max<int64_t>(16, 65536 / gx));
  return dim3(unsigned(gx), unsigned(slots));
}

// The column family: its output is the [w][h] map of the visiting order,
// transposed back onto [h][w] through an LDS tile (grid as transpose_kernel with
// the [w][h] shape).
template <typename TIO, bool FIRST, bool LAST>
__global__ __launch_bounds__(256) void put_col_kernel(const float* __restrict__ yf, float* __restrict__ acc,
                                                      const TIO* __restrict__ z, TIO* __restrict__ y, int64_t rows,
                                                      int64_t h, int64_t w) {
  __shared__ float tile[kTT][kTT + 1];
  const int64_t c0 = int64_t(blockIdx.x) * kTT, r0 = int64_t(blockIdx.y) * kTT;
  for (int64_t row = blockIdx.z; row < rows; row += gridDim.z) {
    const float* src = yf + row * h * w;
    __syncthreads();
    for (int k = threadIdx.y; k < kTT; k += 8) {
      const int64_t r = r0 + k, c = c0 + threadIdx.x;
      tile[k][threadIdx.x] = (r < h && c < w) ? src[r * w + c] : 0.0f;
    }
    __syncthreads();
    for (int k = threadIdx.y; k < kTT; k += 8) {
      const int64_t c = c0 + k, r = r0 + threadIdx.x;
      if (r < h && c < w) {
        const int64_t o = row * h * w + c * h + r;
        const float v = FIRST ? tile[threadIdx.x][k] : acc[o] + tile[threadIdx.x][k];
        if (LAST) {
          st(y, o, z ? silu_gate(v, ld(z, o)) : v);
        } else {
          acc[o] = v;
        }
      }
    }
  }
}

// put_col_kernel for bf16 maps with even sides, on 64 x 64 tiles moving pairs: the
// family's fp32 output ([w][h], a column per row) is read as float2 along the
// column, and two neighbouring tokens of a map row are handled per thread (float2
// accumulator, a 4-byte word of z and of y).  Block 32 x 8; grid as
// transpose_pairs_kernel with the [w][h] shape.
template <bool FIRST, bool LAST>
__global__ __launch_bounds__(256) void put_col_pairs_kernel(const float* __restrict__ yf, float* __restrict__ acc,
                                                            const uint16_t* __restrict__ z, uint16_t* __restrict__ y,
                                                            int64_t rows, int64_t h, int64_t w) {
  __shared__ float tile[kPT][kPT + 1];  // [column in tile][map row in tile]
  // the tile covers map rows r0 .. r0+63 (yf's columns) and map columns c0 .. c0+63
  const int64_t r0 = int64_t(blockIdx.x) * kPT, c0 = int64_t(blockIdx.y) * kPT;
  const int tx = threadIdx.x, ty = threadIdx.y;
  for (int64_t row = blockIdx.z; row < rows; row += gridDim.z) {
    const float* src = yf + row * h * w;
    __syncthreads();
    for (int k = ty; k < kPT; k += 8) {
      const int64_t c = c0 + k, r = r0 + 2 * tx;
      float2 v = make_float2(0.0f, 0.0f);
      if (c < w && r < h) v = *reinterpret_cast<const float2*>(src + c * h + r);
      tile[k][2 * tx] = v.x;
      tile[k][2 * tx + 1] = v.y;
    }
    __syncthreads();
    for (int k = ty; k < kPT; k += 8) {
      const int64_t r = r0 + k, c = c0 + 2 * tx;
      if (r >= h || c >= w) continue;
      const int64_t o = row * h * w + r * w + c;
      float v0 = tile[2 * tx][k], v1 = tile[2 * tx + 1][k];
      if (!FIRST) {
        const float2 a = *reinterpret_cast<const float2*>(acc + o);
        v0 += a.x;
        v1 += a.y;
      }
      if (LAST) {
        if (z) {
          const uint32_t zw = *reinterpret_cast<const uint32_t*>(z + o);
          v0 = silu_gate(v0, __uint_as_float(zw << 16));
          v1 = silu_gate(v1, __uint_as_float(zw & 0xffff0000u));
        }
        *reinterpret_cast<uint32_t*>(y + o) = bf16_pair(v0, v1);
      } else {
        *reinterpret_cast<float2*>(acc + o) = make_float2(v0, v1);
      }
    }
  }
}

// 256-thread blocks covering n elements, capped (the flat kernels stride past it).
unsigned blocks_for(int64_t n) { return unsigned(std::min<int64_t>((n + 255) / 256, int64_t(1) << 22)); }

// Element pairs of a [h][w] map and its transpose are 4-byte words when both sides
// are even and the bases are 4-byte aligned.
bool pairs_ok(const void* a, const void* b, int64_t h, int64_t w) {
  return h % 2 == 0 && w % 2 == 0 && (reinterpret_cast<uintptr_t>(a) & 3u) == 0 &&
         (reinterpret_cast<uintptr_t>(b) & 3u) == 0;
}

template <typename T>
void launch_transpose(const void* in, void* out, int64_t rows, int64_t h, int64_t w, hipStream_t s) {
  hipLaunchKernelGGL((transpose_kernel<T>), transpose_grid(rows, h, w), dim3(kTT, 8), 0, s,
                     static_cast<const T*>(in), static_cast<T*>(out), rows, h, w);
}

// Maps of at least this many tokens gather in flat order (measured: 2.2 -> 1.5 ms per
// bf16 tensor on a 512 x 512 map, while row groups were faster on 128 x 128).
constexpr int64_t kFlatGatherLen = 65536;

template <typename T>
void launch_gather(const void* in, void* out, const int32_t* index, int64_t rows, int64_t len, hipStream_t s) {
  if (len >= kFlatGatherLen) {
    hipLaunchKernelGGL((gather_kernel<T>), dim3(blocks_for(rows * len)), dim3(256), 0, s, static_cast<const T*>(in),
                       static_cast<T*>(out), index, rows, len);
  } else {
    hipLaunchKernelGGL((gather_rows_kernel<T>), index_grid(rows, len), dim3(256), 0, s, static_cast<const T*>(in),
                       static_cast<T*>(out), index, rows, len);
  }
}

// Gathers one [rows][len] tensor into a family's visiting order (forward order;
// the reverse directions scan the same sequence backwards).
void gather_family(int family, bool bf16, const void* in, void* out, const int32_t* index, int64_t rows,
                   int64_t h, int64_t w, hipStream_t s) {
  if (family == kFamilyCol) {
    if (bf16 && pairs_ok(in, out, h, w)) {
      hipLaunchKernelGGL(transpose_pairs_kernel, pairs_grid(rows, h, w), dim3(32, 8), 0, s,
                         static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), rows, h, w);
    } else if (bf16) {
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

template <typename TIO, bool FIRST, bool LAST>
void put_family_t(int family, const float* yf, float* acc, const int32_t* inv, const void* z, void* y,
                  int64_t rows, int64_t h, int64_t w, hipStream_t s) {
  const TIO* zz = static_cast<const TIO*>(z);
  TIO* yy = static_cast<TIO*>(y);
  if (family == kFamilyCol) {
    if (std::is_same<TIO, uint16_t>::value && pairs_ok(y, z ? z : y, h, w)) {
      hipLaunchKernelGGL((put_col_pairs_kernel<FIRST, LAST>), pairs_grid(rows, w, h), dim3(32, 8), 0, s, yf, acc,
                         reinterpret_cast<const uint16_t*>(zz), reinterpret_cast<uint16_t*>(yy), rows, h, w);
    } else {
      hipLaunchKernelGGL((put_col_kernel<TIO, FIRST, LAST>), transpose_grid(rows, w, h), dim3(kTT, 8), 0, s, yf,
                         acc, zz, yy, rows, w, h);
    }
  } else {
    hipLaunchKernelGGL((put_index_kernel<TIO, FIRST, LAST>), index_grid(rows, h * w), dim3(256), 0, s, yf, acc, inv,
                       zz, yy, rows, h * w);
  }
}

template <typename TIO>
void put_family(int family, const float* yf, float* acc, const int32_t* inv, const void* z, void* y, int64_t rows,
                int64_t h, int64_t w, bool first, bool last, hipStream_t s) {
  if (first && last) {
    put_family_t<TIO, true, true>(family, yf, acc, inv, z, y, rows, h, w, s);
  } else if (first) {
    put_family_t<TIO, true, false>(family, yf, acc, inv, z, y, rows, h, w, s);
  } else if (last) {
    put_family_t<TIO, false, true>(family, yf, acc, inv, z, y, rows, h, w, s);
  } else {
    put_family_t<TIO, false, false>(family, yf, acc, inv, z, y, rows, h, w, s);
  }
}

// Puts a tensor in a family's visiting order back at the token positions (the
// gather's inverse): the column order's [w][h] map is transposed back onto [h][w];
// the index order is read through its inverse (out[t] = vis[inv[t]]).
void scatter_family(int family, bool bf16, const void* vis, void* out, const int32_t* inv, int64_t rows, int64_t h,
                    int64_t w, hipStream_t s) {
  if (family == kFamilyCol) {
    gather_family(kFamilyCol, bf16, vis, out, nullptr, rows, w, h, s);
  } else {
    gather_family(kFamilyIndex, bf16, vis, out, inv, rows, h, w, s);
  }
}

// The families present among kinds[0..ndir), in the fixed order rows, columns, index.
int families_of(const int* kinds, int ndir, int* fams) {
  int nf = 0;
  for (int f = 0; f < kFamilies; ++f)
    for (int k = 0; k < ndir; ++k)
      if (kinds[k] / 2 == f) {
        fams[nf++] = f;
        break;
      }
  return nf;
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
  bool has_index = false;
  for (int k = 0; k < ndir; ++k) has_index = has_index || kinds[k] / 2 == kFamilyIndex;
  p.off_inv = off;
  off += has_index ? up(size_t(len) * 4) : 0;
  p.off_scan = off;
  off += up(scan);
  p.workspace_bytes = off;
  return p;
}

hipError_t launch_multi(const MultiArgs& a, const MultiPlan& p, char* ws, hipStream_t stream) {
  const int64_t len = a.height * a.width;
  const int64_t rows = a.batch * a.dim, bc_rows = a.batch * kDState;
  float* acc = reinterpret_cast<float*>(ws + p.off_acc);
  int fams[kFamilies];
  const int nf = families_of(a.kind, a.ndir, fams);
  for (int fi = 0; fi < nf; ++fi) {
    const int f = fams[fi];
    const bool first = fi == 0, last = fi == nf - 1;
    int idx[2] = {-1, -1};  // forward, reverse direction of this family
    for (int k = 0; k < a.ndir; ++k)
      if (a.kind[k] / 2 == f) idx[a.kind[k] % 2] = k;
    ScanArgs s;
    std::memset(&s, 0, sizeof(s));
    s.softplus = a.softplus;
    s.io_bf16 = a.io_bf16;
    s.bc_bf16 = a.bc_bf16;
    s.batch = a.batch;
    s.dim = a.dim;
    s.len = len;
    if (f == kFamilyRow) {
      s.u = a.u;
      if (last) {
        // rows alone: the plain gated scan
        s.z = a.z;
        s.y = a.y;
      } else {
        // rows come first: scan straight into the accumulator
        s.y = acc;
        s.y_f32 = 1;
      }
    } else {
      s.u = ws + p.off_u;
      s.y = ws + p.off_y;
      s.y_f32 = 1;  // summed before any rounding
      gather_family(f, a.io_bf16, a.u, ws + p.off_u, a.index, rows, a.height, a.width, stream);
    }
    int slot = 0;
    const void* gathered_delta = nullptr;  // a delta shared by the family's two directions is gathered once
    for (int j = 0; j < 2; ++j) {
      if (idx[j] < 0) continue;
      DirArgs d = a.dir[idx[j]];
      if (f != kFamilyRow) {
        if (slot == 1 && d.delta == a.dir[idx[0]].delta && gathered_delta) {
          d.delta = gathered_delta;
        } else {
          gather_family(f, a.io_bf16, d.delta, ws + p.off_delta[slot], a.index, rows, a.height, a.width, stream);
          d.delta = ws + p.off_delta[slot];
        }
        if (slot == 0) gathered_delta = d.delta;
        gather_family(f, a.bc_bf16, d.B, ws + p.off_B[slot], a.index, bc_rows, a.height, a.width, stream);
        gather_family(f, a.bc_bf16, d.C, ws + p.off_C[slot], a.index, bc_rows, a.height, a.width, stream);
        d.B = ws + p.off_B[slot];
        d.C = ws + p.off_C[slot];
      }
      s.dir[slot++] = d;
    }
    s.ndir = slot;
    s.reverse = (slot == 1 && idx[1] >= 0) ? 1 : 0;  // a lone reverse direction
    // a gathered family's inputs are in its visiting order: the scan sees a plain
    // sequence (for columns, the [width][height] transpose read row by row)
    const Plan plan = make_plan(a.batch, a.dim, len, s.ndir);
    const hipError_t e = launch_scan(s, plan, reinterpret_cast<float*>(ws + p.off_scan), stream);
    if (e != hipSuccess) return e;
    if (f != kFamilyRow) {
      const float* yf = reinterpret_cast<const float*>(ws + p.off_y);
      int32_t* inv = reinterpret_cast<int32_t*>(ws + p.off_inv);
      if (f == kFamilyIndex) {
        hipLaunchKernelGGL(fill_kernel, dim3(blocks_for(len)), dim3(256), 0, stream, inv, len, -1);
        hipLaunchKernelGGL(invert_kernel, dim3(blocks_for(len)), dim3(256), 0, stream, a.index, inv, len);
      }
      if (a.io_bf16) {
        put_family<uint16_t>(f, yf, acc, inv, a.z, a.y, rows, a.height, a.width, first, last, stream);
      } else {
        put_family<float>(f, yf, acc, inv, a.z, a.y, rows, a.height, a.width, first, last, stream);
      }
    }
  }
  return hipGetLastError();
}

}  // namespace sscan

namespace sscan {

MultiBwdPlan make_multi_bwd_plan(int64_t batch, int64_t dim, int64_t height, int64_t width, const int* kinds,
                                 int ndir, bool io_bf16, bool bc_bf16) {
  MultiBwdPlan p{};
  const int64_t len = height * width;
  const size_t io = io_bf16 ? 2 : 4, bc = bc_bf16 ? 2 : 4;
  const size_t n = size_t(batch) * size_t(dim) * size_t(len), nbc = size_t(batch) * kDState * size_t(len);
  int nfam = 0, slots = 0;  // families present; direction slots of the gathered families
  bool has_index = false;
  size_t bwd = 0;
  for (int f = 0; f < kFamilies; ++f) {
    int nd = 0;
    for (int k = 0; k < ndir; ++k) nd += kinds[k] / 2 == f;
    if (nd == 0) continue;
    ++nfam;
    bwd = std::max(bwd, make_bwd_plan(batch, dim, len, nd).workspace_bytes);
    if (f != kFamilyRow) slots = std::max(slots, nd);
    has_index = has_index || f == kFamilyIndex;
  }
  size_t off = 0;
  auto take = [&off](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const size_t acc = nfam > 1 ? n * 4 : 0;
  p.off_acc_du = take(acc);
  p.off_acc_dz = take(acc);
  const size_t gat = slots > 0 ? 1 : 0;
  p.off_vdu = take(gat * n * 4);
  p.off_vdz = take(gat * n * 4);
  p.off_u = take(gat * n * io);
  p.off_z = take(gat * n * io);
  p.off_g = take(gat * n * io);
  for (int j = 0; j < 2; ++j) {
    const size_t on = j < slots ? 1 : 0;
    p.off_delta[j] = take(on * n * io);
    p.off_B[j] = take(on * nbc * bc);
    p.off_C[j] = take(on * nbc * bc);
    p.off_dd[j] = take(on * n * io);
    p.off_dB[j] = take(on * nbc * bc);
    p.off_dC[j] = take(on * nbc * bc);
  }
  p.off_inv = take(has_index ? size_t(len) * 4 : 0);
  p.off_bwd = take(bwd);
  p.workspace_bytes = off;
  return p;
}

hipError_t launch_multi_bwd(const MultiBwdArgs& a, const MultiBwdPlan& p, char* ws, hipStream_t stream) {
  const MultiArgs& m = a.fwd;
  const int64_t len = m.height * m.width;
  const int64_t rows = m.batch * m.dim, bc_rows = m.batch * kDState;
  float* acc_du = reinterpret_cast<float*>(ws + p.off_acc_du);
  float* acc_dz = reinterpret_cast<float*>(ws + p.off_acc_dz);
  float* vdu = reinterpret_cast<float*>(ws + p.off_vdu);
  float* vdz = reinterpret_cast<float*>(ws + p.off_vdz);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + p.off_inv);
  int fams[kFamilies];
  const int nf = families_of(m.kind, m.ndir, fams);
  for (int fi = 0; fi < nf; ++fi) {
    const int f = fams[fi];
    const bool first = fi == 0, last = fi == nf - 1, gathered = f != kFamilyRow;
    int idx[2] = {-1, -1};  // forward, reverse direction of this family
    for (int k = 0; k < m.ndir; ++k)
      if (m.kind[k] / 2 == f) idx[m.kind[k] % 2] = k;
    BwdArgs b;
    std::memset(&b, 0, sizeof(b));
    ScanArgs& s = b.fwd;
    s.softplus = m.softplus;
    s.io_bf16 = m.io_bf16;
    s.bc_bf16 = m.bc_bf16;
    s.batch = m.batch;
    s.dim = m.dim;
    s.len = len;
    if (!gathered) {
      s.u = m.u;
      s.z = m.z;
      b.dout = a.dout;
      if (last) {
        // rows alone: the plain (gated) backward
        b.du = a.du;
        b.dz = a.dz;
      } else {
        // rows come first: du and dz straight into the sums
        b.du = acc_du;
        b.dz = acc_dz;
        b.du_f32 = b.dz_f32 = 1;
      }
    } else {
      gather_family(f, m.io_bf16, m.u, ws + p.off_u, m.index, rows, m.height, m.width, stream);
      gather_family(f, m.io_bf16, a.dout, ws + p.off_g, m.index, rows, m.height, m.width, stream);
      if (m.z) gather_family(f, m.io_bf16, m.z, ws + p.off_z, m.index, rows, m.height, m.width, stream);
      s.u = ws + p.off_u;
      s.z = m.z ? ws + p.off_z : nullptr;
      b.dout = ws + p.off_g;
      b.du = vdu;
      b.dz = vdz;
      b.du_f32 = b.dz_f32 = 1;  // summed with the other families' before any rounding
    }
    int slot = 0, dir_of[2] = {-1, -1};
    const void* gathered_delta = nullptr;  // a delta shared by the family's two directions is gathered once
    for (int j = 0; j < 2; ++j) {
      if (idx[j] < 0) continue;
      DirArgs d = m.dir[idx[j]];
      DirGrads g = a.grads[idx[j]];
      if (gathered) {
        if (slot == 1 && d.delta == m.dir[idx[0]].delta && gathered_delta) {
          d.delta = gathered_delta;
        } else {
          gather_family(f, m.io_bf16, d.delta, ws + p.off_delta[slot], m.index, rows, m.height, m.width, stream);
          d.delta = ws + p.off_delta[slot];
        }
        if (slot == 0) gathered_delta = d.delta;
        gather_family(f, m.bc_bf16, d.B, ws + p.off_B[slot], m.index, bc_rows, m.height, m.width, stream);
        gather_family(f, m.bc_bf16, d.C, ws + p.off_C[slot], m.index, bc_rows, m.height, m.width, stream);
        d.B = ws + p.off_B[slot];
        d.C = ws + p.off_C[slot];
        // the sequence-shaped gradients land in visit order first
        g.ddelta = ws + p.off_dd[slot];
        g.dB = ws + p.off_dB[slot];
        g.dC = ws + p.off_dC[slot];
      }
      s.dir[slot] = d;
      b.grads[slot] = g;
      dir_of[slot++] = idx[j];
    }
    s.ndir = slot;
    s.reverse = (slot == 1 && idx[1] >= 0) ? 1 : 0;  // a lone reverse direction
    const BwdPlan bp = make_bwd_plan(m.batch, m.dim, len, slot);
    hipError_t e = launch_bwd(b, bp, reinterpret_cast<float*>(ws + p.off_bwd), stream);
    if (e != hipSuccess) return e;
    if (!gathered) continue;
    if (f == kFamilyIndex) {
      hipLaunchKernelGGL(fill_kernel, dim3(blocks_for(len)), dim3(256), 0, stream, inv, len, -1);
      hipLaunchKernelGGL(invert_kernel, dim3(blocks_for(len)), dim3(256), 0, stream, m.index, inv, len);
    }
    // du, dz: summed over the families in fp32, rounded once by the last put-back
    if (m.io_bf16) {
      put_family<uint16_t>(f, vdu, acc_du, inv, nullptr, a.du, rows, m.height, m.width, first, last, stream);
      if (m.z) put_family<uint16_t>(f, vdz, acc_dz, inv, nullptr, a.dz, rows, m.height, m.width, first, last, stream);
    } else {
      put_family<float>(f, vdu, acc_du, inv, nullptr, a.du, rows, m.height, m.width, first, last, stream);
      if (m.z) put_family<float>(f, vdz, acc_dz, inv, nullptr, a.dz, rows, m.height, m.width, first, last, stream);
    }
    for (int j = 0; j < slot; ++j) {
      const DirGrads& g = a.grads[dir_of[j]];
      scatter_family(f, m.io_bf16, ws + p.off_dd[j], g.ddelta, inv, rows, m.height, m.width, stream);
      scatter_family(f, m.bc_bf16, ws + p.off_dB[j], g.dB, inv, bc_rows, m.height, m.width, stream);
      scatter_family(f, m.bc_bf16, ws + p.off_dC[j], g.dC, inv, bc_rows, m.height, m.width, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace sscan
