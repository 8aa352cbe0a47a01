// sscan_kernels.hip -- gfx950 kernels of the selective scan (Mamba S6).
//
// Recurrence (Hand-written simplified Mamba2 page, section 2.2; step size from
// section 4.2; skip and gate from section 4.4):
//     h_n <- exp(dt_t A_n) h_n + dt_t B_{n,t} u_t,   y_t = sum_n C_{n,t} h_n + D u_t,
//     out_t = (y_t [+ y_t of the reverse scan]) * silu(z_t).
//
// Mapping: lane = channel.  A wavefront owns 64 consecutive channels of one batch
// row; every lane keeps its channel's 16 fp32 states in registers and walks the
// tokens of its segment in order.  All lanes of a wave are at the same token, so
// B_t and C_t are wave-uniform: a staging kernel rewrites them token-major
// ([t][B_0..15, C_0..15], fp32) and the scan reads each token's 32 values with
// two scalar 64-byte loads straight into SGPRs, which the VALU ops take as
// operands.  u, delta and z are read per lane in 16-token register tiles with
// 16-byte vector loads (element loads when rows are not 16-byte aligned, and for
// the ragged last tile); y is written back the same way.  The state sequence
// never leaves registers.
//
// Long sequences are cut into segments so that enough wavefronts exist; the state
// entering each segment comes from a three-step chunked scan (same page, section
// 3.2: recurrence between chunks, independent work inside them; the state is
// carried across chunk boundaries, never reset):
//   1. aggregate: each segment, scanned from a zero state, yields its end state
//      and the sum of its step sizes (its decay is exp(A * sum dt));
//   2. carry: per (channel, state) the segment aggregates are chained in order,
//      h_in[s+1] = exp(A * sum_dt[s]) * h_in[s] + H[s], giving every entry state;
//   3. output: every segment is scanned again from its entry state, producing y.
// The bidirectional output kernel runs the forward and the reverse scan of one
// segment in two wavefronts that meet in the middle through LDS, so the two
// directions are summed and gated before the single store (Reproducing Vision
// Mamba page, section 3.2: the two directions' results are added).
#include "sscan_internal.h"

#include <algorithm>

namespace sscan {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBC = 2 * kDState;  // floats per token in the staged B/C buffer

// Scan kernels keep about 100 live VGPRs per lane (16 states, 16 scaled A, the
// token tiles); capping them at 128 lets four waves share each SIMD and stops the
// scheduler from hoisting many tokens' exponentials ahead at the cost of occupancy.
#define SSCAN_OCCUPANCY __attribute__((amdgpu_waves_per_eu(4, 8)))

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = max(x, 0) + log1p(exp(-|x|)).  log1p(w) is taken as
// log(1 + w) * w / ((1 + w) - 1): the quotient cancels the rounding of 1 + w, so
// the result keeps full relative accuracy for small w (step sizes near 1e-4).
__device__ __forceinline__ float softplus_f32(float x) {
  const float w = exp2_hw(-fabsf(x) * kLog2e);
  const float s = 1.0f + w;
  const float d = s - 1.0f;
  const float lp = (d == 0.0f) ? w : (log2_hw(s) * kLn2) * (w * rcp_hw(d));
  return fmaxf(x, 0.0f) + lp;
}

__device__ __forceinline__ float silu_f32(float x) { return x * rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats to two bf16 (round to nearest even, NaN kept), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// Storage-type access.  A tile holds kTile consecutive tokens of one row as
// 32-bit words (two bf16 per word, low half = earlier token).
template <bool BF16>
struct Io;
template <>
struct Io<false> {
  using T = float;
  static constexpr int kWords = kTile;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ float get(const uint32_t (&w)[kWords], int j) { return __uint_as_float(w[j]); }
  static __device__ __forceinline__ void load_elems(uint32_t (&w)[kWords], const T* row, int64_t t) {
#pragma unroll
    for (int j = 0; j < kTile; ++j) w[j] = __float_as_uint(row[t + j]);
  }
  static __device__ __forceinline__ void store_tile(T* row, int64_t t, const float (&y)[kTile], bool vec) {
    if (vec) {
      uint4* p = reinterpret_cast<uint4*>(row + t);
#pragma unroll
      for (int i = 0; i < kTile / 4; ++i)
        p[i] = make_uint4(__float_as_uint(y[4 * i]), __float_as_uint(y[4 * i + 1]), __float_as_uint(y[4 * i + 2]),
                          __float_as_uint(y[4 * i + 3]));
    } else {
#pragma unroll
      for (int j = 0; j < kTile; ++j) row[t + j] = y[j];
    }
  }
};
template <>
struct Io<true> {
  using T = uint16_t;
  static constexpr int kWords = kTile / 2;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }
  static __device__ __forceinline__ void store(T* p, int64_t i, float v) {
    p[i] = uint16_t(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
  static __device__ __forceinline__ float get(const uint32_t (&w)[kWords], int j) {
    return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
  }
  static __device__ __forceinline__ void load_elems(uint32_t (&w)[kWords], const T* row, int64_t t) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = uint32_t(row[t + 2 * i]) | (uint32_t(row[t + 2 * i + 1]) << 16);
  }
  static __device__ __forceinline__ void store_tile(T* row, int64_t t, const float (&y)[kTile], bool vec) {
    uint32_t w[kWords];
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    if (vec) {
      uint4* p = reinterpret_cast<uint4*>(row + t);
#pragma unroll
      for (int i = 0; i < kWords / 4; ++i) p[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < kWords; ++i) {
        row[t + 2 * i] = uint16_t(w[i] & 0xffffu);
        row[t + 2 * i + 1] = uint16_t(w[i] >> 16);
      }
    }
  }
};

template <bool BF16>
__device__ __forceinline__ void load_tile(uint32_t (&w)[Io<BF16>::kWords], const typename Io<BF16>::T* row,
                                          int64_t t, bool vec) {
  if (vec) {
    const uint4* p = reinterpret_cast<const uint4*>(row + t);
#pragma unroll
    for (int i = 0; i < Io<BF16>::kWords / 4; ++i) {
      const uint4 v = p[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  } else {
    Io<BF16>::load_elems(w, row, t);
  }
}

typedef __attribute__((address_space(3))) float lds_float;

// What a scan pass does with each token's output.
enum Mode : int {
  kAggregate = 0,  // no readout: advance the state, sum the step sizes
  kStore = 1,      // gate and store y
  kPark = 2,       // park y (ungated, one direction) in the LDS meeting buffer
  kMeet = 3,       // add the partner direction's parked y, gate, store
};

// One lane's view of one direction of one (batch, channel) row.  SOFTPLUS and
// HAS_Z are compile-time so that a tile's 16 tokens form one straight-line block.
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z>
struct Lane {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  const T* u;
  const T* delta;
  const T* z;     // nullable
  T* y;
  const float* __restrict__ bc;  // staged B/C of this (direction, batch): bc[t * 32 + ...]
  lds_float* part;  // LDS meeting buffer (bidirectional kernel), [t - t0][64]
  int64_t t0;     // first token of the segment (LDS buffer origin)
  float A2[kDState];  // A * log2(e)
  float h[kDState];
  float bias, Dd;
  float sum_dt;
  int lane;
  bool vec;       // 16-byte vector access is valid for full tiles
  bool active;    // lane maps to a real channel (stores enabled)

  __device__ __forceinline__ float step_size(float draw) const {
    const float x = draw + bias;
    return SOFTPLUS ? softplus_f32(x) : x;
  }

  // Advances the state by one token; returns y (before the gate) for the output
  // modes, nothing useful for kAggregate.
  template <int MODE>
  __device__ __forceinline__ float token(float uu, float draw, int64_t t) {
    const float* bct = bc + t * kBC;
    const float dt = step_size(draw);
    const float dtu = dt * uu;
    if (MODE == kAggregate) {
      sum_dt += dt;
#pragma unroll
      for (int n = 0; n < kDState; ++n) h[n] = fmaf(exp2_hw(dt * A2[n]), h[n], dtu * bct[n]);
      return 0.0f;
    }
    float s = 0.0f;
#pragma unroll
    for (int n = 0; n < kDState; ++n) {
      h[n] = fmaf(exp2_hw(dt * A2[n]), h[n], dtu * bct[n]);
      s = fmaf(bct[kDState + n], h[n], s);
    }
    return fmaf(Dd, uu, s);
  }

  __device__ __forceinline__ float gate(float yv, float zv) const { return HAS_Z ? yv * silu_f32(zv) : yv; }

  // Tokens [ta, tb) in scan order (descending when REV).  ta/tb are multiples of
  // kTile except at the end of the sequence.
  template <bool REV, int MODE>
  __device__ void scan(int64_t ta, int64_t tb) {
    if (tb <= ta) return;
    const int64_t k_first = ta / kTile, k_last = (tb - 1) / kTile;
    for (int64_t kk = 0; kk <= k_last - k_first; ++kk) {
      const int64_t k = REV ? k_last - kk : k_first + kk;
      const int64_t tlo = max64(ta, k * kTile), thi = min64(tb, (k + 1) * kTile);
      if (thi - tlo == kTile) {
        full_tile<REV, MODE>(tlo);
      } else {
        for (int64_t i = 0; i < thi - tlo; ++i) partial_token<MODE>(REV ? thi - 1 - i : tlo + i);
      }
    }
  }

  template <bool REV, int MODE>
  __device__ __forceinline__ void full_tile(int64_t t) {
    constexpr bool kNeedZ = HAS_Z && (MODE == kStore || MODE == kMeet);
    uint32_t wu[IO::kWords], wd[IO::kWords], wz[IO::kWords];
    load_tile<IO_BF16>(wu, u, t, vec);
    load_tile<IO_BF16>(wd, delta, t, vec);
    if (kNeedZ) {
      load_tile<IO_BF16>(wz, z, t, vec);
    } else {
#pragma unroll
      for (int i = 0; i < IO::kWords; ++i) wz[i] = 0;
    }
    float yt[kTile];
#pragma unroll
    for (int jj = 0; jj < kTile; ++jj) {
      const int j = REV ? kTile - 1 - jj : jj;
      float yv = token<MODE>(IO::get(wu, j), IO::get(wd, j), t + j);
      // materialise this token's readout now: otherwise it is sunk towards the
      // tile's store and all 16 tokens' states stay live
      if (MODE != kAggregate) asm volatile("" : "+v"(yv));
      if (MODE == kStore) {
        yt[j] = gate(yv, IO::get(wz, j));
      } else if (MODE == kPark) {
        part[(t + j - t0) * kLanes + lane] = yv;
      } else if (MODE == kMeet) {
        yt[j] = gate(yv + part[(t + j - t0) * kLanes + lane], IO::get(wz, j));
      }
      // keep each token's work together: the 16 state chains of one token give
      // enough independent instructions, and hoisting later tokens' exponentials
      // ahead only raises register pressure
      __builtin_amdgcn_sched_barrier(0);
    }
    if ((MODE == kStore || MODE == kMeet) && active) IO::store_tile(y, t, yt, vec);
  }

  template <int MODE>
  __device__ __forceinline__ void partial_token(int64_t t) {
    const float uu = IO::load(u, t);
    const float yv = token<MODE>(uu, IO::load(delta, t), t);
    if (MODE == kPark) {
      part[(t - t0) * kLanes + lane] = yv;
    } else if (MODE == kStore || MODE == kMeet) {
      float v = (MODE == kMeet) ? yv + part[(t - t0) * kLanes + lane] : yv;
      if (HAS_Z) v *= silu_f32(IO::load(z, t));
      if (active) IO::store(y, t, v);
    }
  }
};

struct SegIndex {
  int64_t g, seg, b;  // channel group, segment, batch
};

__device__ __forceinline__ SegIndex decode_block(int64_t blk, int64_t ngroups, int64_t nseg) {
  SegIndex s;
  s.g = blk % ngroups;
  const int64_t r = blk / ngroups;
  s.seg = r % nseg;
  s.b = r / nseg;
  return s;
}

__device__ __forceinline__ size_t agg_index(int dir, int64_t b, int64_t seg, int n, int64_t d, int64_t batch,
                                            int64_t dim, int64_t nseg) {
  return ((((size_t)dir * batch + b) * nseg + seg) * (kDState + 1) + n) * dim + d;
}

__device__ __forceinline__ size_t hin_index(int dir, int64_t b, int64_t seg, int n, int64_t d, int64_t batch,
                                            int64_t dim, int64_t nseg) {
  return ((((size_t)dir * batch + b) * nseg + seg) * kDState + n) * dim + d;
}

// Sets up a lane for direction `dir` of batch b, channel group g.
template <class LaneT>
__device__ __forceinline__ void init_lane(LaneT& L, const ScanArgs& a, int dir, int64_t b, int64_t g,
                                          const float* bc, bool vec) {
  using T = typename LaneT::T;
  const int lane = threadIdx.x % kLanes;
  const int64_t d_raw = g * kLanes + lane;
  L.active = d_raw < a.dim;
  const int64_t d = L.active ? d_raw : a.dim - 1;  // idle lanes shadow a valid row and store nothing
  const DirArgs p = dir ? a.dir[1] : a.dir[0];
  const int64_t row = (b * a.dim + d) * a.len;
  L.u = static_cast<const T*>(a.u) + row;
  L.delta = static_cast<const T*>(p.delta) + row;
  L.z = a.z ? static_cast<const T*>(a.z) + row : nullptr;
  L.y = static_cast<T*>(a.y) + row;
  L.bc = bc + ((size_t)dir * a.batch + b) * a.len * kBC;
  L.part = nullptr;
  L.t0 = 0;
#pragma unroll
  for (int n = 0; n < kDState; ++n) L.A2[n] = p.A[d * kDState + n] * kLog2e;
  L.bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
  L.Dd = p.D ? p.D[d] : 0.0f;
  L.sum_dt = 0.0f;
  L.lane = lane;
  L.vec = vec;
#pragma unroll
  for (int n = 0; n < kDState; ++n) L.h[n] = 0.0f;
}

template <class LaneT>
__device__ __forceinline__ void load_entry(LaneT& L, const ScanArgs& a, int dir, int64_t b, int64_t seg,
                                           int64_t g, int64_t nseg, const float* hin) {
  if (nseg <= 1) return;
  const int64_t d = min64(g * kLanes + threadIdx.x % kLanes, a.dim - 1);
#pragma unroll
  for (int n = 0; n < kDState; ++n) L.h[n] = hin[hin_index(dir, b, seg, n, d, a.batch, a.dim, nseg)];
}

// Stage B and C token-major in fp32: bc[dir][b][t][0..15] = B[b][:, t],
// bc[dir][b][t][16..31] = C[b][:, t].  One block per (direction, batch, 64 tokens).
template <bool BC_BF16>
__global__ __launch_bounds__(256) void stage_bc_kernel(ScanArgs a, float* __restrict__ bc) {
  __shared__ float tile[kBC][65];
  const int64_t ntiles = (a.len + 63) / 64;
  const int64_t tt = blockIdx.x % ntiles;
  const int64_t db = blockIdx.x / ntiles;  // dir * batch + b
  const int dir = int(db / a.batch);
  const int64_t b = db % a.batch;
  const DirArgs p = dir ? a.dir[1] : a.dir[0];
  const int64_t t0 = tt * 64;
  for (int i = threadIdx.x; i < kBC * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    const int64_t t = t0 + c;
    float v = 0.0f;
    if (t < a.len) {
      const size_t idx = ((size_t)b * kDState + (r % kDState)) * a.len + t;
      const void* src = r < kDState ? p.B : p.C;
      v = BC_BF16 ? Io<true>::load(static_cast<const uint16_t*>(src), idx) : static_cast<const float*>(src)[idx];
    }
    tile[r][c] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * kBC; i += 256) {
    const int c = i / kBC, r = i % kBC;
    const int64_t t = t0 + c;
    if (t < a.len) bc[((size_t)db * a.len + t) * kBC + r] = tile[r][c];
  }
}

// Step 1: end state (from zero) and sum of step sizes of every segment except the
// last one in scan order.  Grid: batch * nseg * ngroups one-wave blocks;
// blockIdx.y selects the direction.
template <bool IO_BF16, bool SOFTPLUS>
__global__ __launch_bounds__(kLanes) SSCAN_OCCUPANCY void scan_aggregate_kernel(ScanArgs a, int64_t seg_len, int64_t nseg,
                                                                const float* __restrict__ bc,
                                                                float* __restrict__ agg, int vec) {
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const SegIndex s = decode_block(blockIdx.x, ngroups, nseg);
  const int dir = blockIdx.y;
  const int reverse = a.ndir == 2 ? dir : a.reverse;
  if (reverse ? s.seg == 0 : s.seg == nseg - 1) return;
  Lane<IO_BF16, SOFTPLUS, false> L;
  init_lane(L, a, dir, s.b, s.g, bc, vec != 0);
  const int64_t t0 = s.seg * seg_len;
  const int64_t t1 = min64(a.len, t0 + seg_len);
  if (reverse) {
    L.template scan<true, kAggregate>(t0, t1);
  } else {
    L.template scan<false, kAggregate>(t0, t1);
  }
  if (!L.active) return;
  const int64_t d = s.g * kLanes + threadIdx.x;
#pragma unroll
  for (int n = 0; n < kDState; ++n) agg[agg_index(dir, s.b, s.seg, n, d, a.batch, a.dim, nseg)] = L.h[n];
  agg[agg_index(dir, s.b, s.seg, kDState, d, a.batch, a.dim, nseg)] = L.sum_dt;
}

// Step 2: one thread per (direction, batch, state, channel) chains the segment
// aggregates in scan order and writes the state entering every segment.  The
// aggregate loads do not depend on the chain, so they are issued in batches.
__global__ __launch_bounds__(256) void scan_carry_kernel(ScanArgs a, int64_t nseg, const float* __restrict__ agg,
                                                         float* __restrict__ hin) {
  constexpr int kBatch = 32;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(a.ndir) * a.batch * kDState * a.dim;
  if (idx >= total) return;
  const int64_t d = idx % a.dim;
  const int n = int((idx / a.dim) % kDState);
  const int64_t rest = idx / (a.dim * kDState);
  const int64_t b = rest % a.batch;
  const int dir = int(rest / a.batch);
  const int reverse = a.ndir == 2 ? dir : a.reverse;
  const float* Adir = dir ? a.dir[1].A : a.dir[0].A;
  const float A2 = Adir[d * kDState + n] * kLog2e;
  float h = 0.0f;
  for (int64_t k0 = 0; k0 < nseg; k0 += kBatch) {
    float H[kBatch], S[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t k = k0 + i;
      const int64_t seg = reverse ? nseg - 1 - k : k;
      const bool has = k + 1 < nseg;
      H[i] = has ? agg[agg_index(dir, b, seg, n, d, a.batch, a.dim, nseg)] : 0.0f;
      S[i] = has ? agg[agg_index(dir, b, seg, kDState, d, a.batch, a.dim, nseg)] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t k = k0 + i;
      if (k < nseg) {
        const int64_t seg = reverse ? nseg - 1 - k : k;
        hin[hin_index(dir, b, seg, n, d, a.batch, a.dim, nseg)] = h;
        h = fmaf(exp2_hw(A2 * S[i]), h, H[i]);
      }
    }
  }
}

// Step 3, one direction: every wave scans one segment of 64 channels from its entry
// state and stores the gated output.
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z>
__global__ __launch_bounds__(kLanes) SSCAN_OCCUPANCY void scan_output_dir_kernel(ScanArgs a, int64_t seg_len, int64_t nseg,
                                                                 const float* __restrict__ bc,
                                                                 const float* __restrict__ hin, int vec) {
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const SegIndex s = decode_block(blockIdx.x, ngroups, nseg);
  Lane<IO_BF16, SOFTPLUS, HAS_Z> L;
  init_lane(L, a, 0, s.b, s.g, bc, vec != 0);
  load_entry(L, a, 0, s.b, s.seg, s.g, nseg, hin);
  const int64_t t0 = s.seg * seg_len;
  const int64_t t1 = min64(a.len, t0 + seg_len);
  if (a.reverse) {
    L.template scan<true, kStore>(t0, t1);
  } else {
    L.template scan<false, kStore>(t0, t1);
  }
}

// Step 3, both directions: wave 0 scans the segment forward, wave 1 in reverse.
// Each first covers the half it meets first and parks its outputs in LDS, then
// covers the other half, adds the partner's parked outputs, gates and stores.
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z>
__global__ __launch_bounds__(2 * kLanes) SSCAN_OCCUPANCY void scan_output_bidir_kernel(ScanArgs a, int64_t seg_len, int64_t nseg,
                                                                       const float* __restrict__ bc,
                                                                       const float* __restrict__ hin, int vec) {
  extern __shared__ float part[];  // [seg_len][64]
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const SegIndex s = decode_block(blockIdx.x, ngroups, nseg);
  const int dir = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kLanes);  // wave-uniform
  Lane<IO_BF16, SOFTPLUS, HAS_Z> L;
  init_lane(L, a, dir, s.b, s.g, bc, vec != 0);
  load_entry(L, a, dir, s.b, s.seg, s.g, nseg, hin);
  const int64_t t0 = s.seg * seg_len;
  const int64_t t1 = min64(a.len, t0 + seg_len);
  const int64_t mid = t0 + ((t1 - t0) / 2) / kTile * kTile;
  L.part = (lds_float*)part;
  L.t0 = t0;
  if (dir == 0) {
    L.template scan<false, kPark>(t0, mid);
  } else {
    L.template scan<true, kPark>(mid, t1);
  }
  __syncthreads();
  if (dir == 0) {
    L.template scan<false, kMeet>(mid, t1);
  } else {
    L.template scan<true, kMeet>(t0, mid);
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z>
hipError_t launch_typed(const ScanArgs& a, const Plan& p, float* w, hipStream_t stream) {
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const int64_t nblocks = a.batch * p.nseg * ngroups;
  const size_t esz = IO_BF16 ? 2 : 4;
  bool vec = (size_t(a.len) * esz) % 16 == 0 && aligned16(a.u) && aligned16(a.y) && (!a.z || aligned16(a.z));
  for (int k = 0; k < a.ndir; ++k) vec = vec && aligned16(a.dir[k].delta);
  float* bc = w;
  float* agg = p.nseg > 1 ? w + p.bc_floats : nullptr;
  float* hin = p.nseg > 1 ? agg + p.agg_floats : nullptr;

  const int64_t bc_blocks = int64_t(a.ndir) * a.batch * ((a.len + 63) / 64);
  if (a.bc_bf16) {
    hipLaunchKernelGGL(stage_bc_kernel<true>, dim3(unsigned(bc_blocks)), dim3(256), 0, stream, a, bc);
  } else {
    hipLaunchKernelGGL(stage_bc_kernel<false>, dim3(unsigned(bc_blocks)), dim3(256), 0, stream, a, bc);
  }
  if (p.nseg > 1) {
    hipLaunchKernelGGL((scan_aggregate_kernel<IO_BF16, SOFTPLUS>), dim3(unsigned(nblocks), unsigned(a.ndir)),
                       dim3(kLanes), 0, stream, a, p.seg_len, p.nseg, static_cast<const float*>(bc), agg, int(vec));
    const int64_t threads = int64_t(a.ndir) * a.batch * kDState * a.dim;
    hipLaunchKernelGGL(scan_carry_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, a, p.nseg,
                       static_cast<const float*>(agg), hin);
  }
  if (a.ndir == 1) {
    hipLaunchKernelGGL((scan_output_dir_kernel<IO_BF16, SOFTPLUS, HAS_Z>), dim3(unsigned(nblocks)), dim3(kLanes), 0,
                       stream, a, p.seg_len, p.nseg, static_cast<const float*>(bc), static_cast<const float*>(hin),
                       int(vec));
  } else {
    const size_t lds = size_t(p.seg_len) * kLanes * sizeof(float);
    hipLaunchKernelGGL((scan_output_bidir_kernel<IO_BF16, SOFTPLUS, HAS_Z>), dim3(unsigned(nblocks)),
                       dim3(2 * kLanes), lds, stream, a, p.seg_len, p.nseg, static_cast<const float*>(bc),
                       static_cast<const float*>(hin), int(vec));
  }
  return hipGetLastError();
}

template <bool IO_BF16>
hipError_t launch_io(const ScanArgs& a, const Plan& p, float* w, hipStream_t stream) {
  if (a.softplus) {
    return a.z ? launch_typed<IO_BF16, true, true>(a, p, w, stream) : launch_typed<IO_BF16, true, false>(a, p, w, stream);
  }
  return a.z ? launch_typed<IO_BF16, false, true>(a, p, w, stream) : launch_typed<IO_BF16, false, false>(a, p, w, stream);
}

}  // namespace

Plan make_plan(int64_t batch, int64_t dim, int64_t len, int ndir) {
  Plan p{};
  const int64_t ngroups = (dim + kLanes - 1) / kLanes;
  const int64_t groups = std::max<int64_t>(1, batch * ngroups);
  p.seg_len = std::max<int64_t>(len, 1);
  p.nseg = 1;
  if (len > kShortMax) {
    // Aim for about 8 wavefronts per SIMD (256 CUs x 4 SIMDs) over the output step.
    const int64_t target_waves = 8192;
    const int64_t waves_per_seg = groups * ndir;
    int64_t nseg = std::max<int64_t>(2, (target_waves + waves_per_seg - 1) / waves_per_seg);
    int64_t seg_len = (len + nseg - 1) / nseg;
    seg_len = std::max<int64_t>(kSegAlign, (seg_len + kSegAlign - 1) / kSegAlign * kSegAlign);
    if (ndir == 2) seg_len = std::min<int64_t>(seg_len, kMaxBidirSegment);
    nseg = (len + seg_len - 1) / seg_len;
    while (nseg > 1 && batch * nseg * ngroups > (int64_t(1) << 30)) {  // keep the block count within a 1-D grid
      seg_len *= 2;
      nseg = (len + seg_len - 1) / seg_len;
    }
    p.seg_len = seg_len;
    p.nseg = nseg;
  }
  p.bc_floats = size_t(ndir) * batch * len * kBC;
  // keep the sections 256-byte aligned
  p.bc_floats = (p.bc_floats + 63) / 64 * 64;
  if (p.nseg > 1) {
    p.agg_floats = (size_t(ndir) * batch * p.nseg * (kDState + 1) * dim + 63) / 64 * 64;
    p.hin_floats = size_t(ndir) * batch * p.nseg * kDState * dim;
  }
  p.workspace_bytes = (p.bc_floats + p.agg_floats + p.hin_floats) * sizeof(float);
  return p;
}

hipError_t launch_scan(const ScanArgs& a, const Plan& p, float* ws, hipStream_t stream) {
  return a.io_bf16 ? launch_io<true>(a, p, ws, stream) : launch_io<false>(a, p, ws, stream);
}

}  // namespace sscan
