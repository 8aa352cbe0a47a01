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

// Scan kernels keep about 150 live VGPRs per lane (16 states, 16 scaled A, the
// current and next token tiles); capping them at 168 lets three waves share each
// SIMD and stops the scheduler from hoisting many tokens' exponentials ahead at the
// cost of occupancy.
#define SSCAN_OCCUPANCY __attribute__((amdgpu_waves_per_eu(3, 8)))

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = max(x, 0) + log1p(w), w = exp(-|x|) in (0, 1].  log1p(w) is
// log(s) for s = 1 + w rounded, plus the rounding error c = w - (s - 1) scaled by
// 1/s ~ 1 - w: log(s + c) = log(s) + c/s + O(c^2), and c (below 2^-24) times
// the dropped w^2 term is far below the result's last bit (log1p(w) ~ w).  This
// keeps full relative accuracy for small step sizes (1e-4 and below).
__device__ __forceinline__ float softplus_f32(float x) {
  const float w = exp2_hw(-fabsf(x) * kLog2e);
  const float s = 1.0f + w;
  const float c = w - (s - 1.0f);
  const float lp = fmaf(log2_hw(s), kLn2, c * (1.0f - w));
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

// Storage-type access.  A tile holds kTok consecutive tokens of one row as sixteen
// 32-bit words (32 bf16 tokens, two per word with the earlier token in the low
// half, or 16 f32 tokens): four 16-byte vector loads per tensor, half a 128-byte
// L2 line.  Narrower tiles touch each line more times, far enough apart that the
// line has left L2 in between and is fetched again.
constexpr int kWords = 16;

template <bool BF16>
struct Io;
template <>
struct Io<false> {
  using T = float;
  static constexpr int kTok = 16;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ float get(const uint32_t (&w)[kWords], int j) { return __uint_as_float(w[j]); }
  static __device__ __forceinline__ void load_elems(uint32_t (&w)[kWords], const T* row, int64_t t) {
#pragma unroll
    for (int j = 0; j < kTok; ++j) w[j] = __float_as_uint(row[t + j]);
  }
  static __device__ __forceinline__ void pack(uint32_t (&w)[kWords], const float (&y)[kTok]) {
#pragma unroll
    for (int j = 0; j < kTok; ++j) w[j] = __float_as_uint(y[j]);
  }
  static __device__ __forceinline__ void store_elems(T* row, int64_t t, const uint32_t (&w)[kWords]) {
#pragma unroll
    for (int j = 0; j < kTok; ++j) row[t + j] = __uint_as_float(w[j]);
  }
};
template <>
struct Io<true> {
  using T = uint16_t;
  static constexpr int kTok = 32;
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
  static __device__ __forceinline__ void pack(uint32_t (&w)[kWords], const float (&y)[kTok]) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
  }
  static __device__ __forceinline__ void store_elems(T* row, int64_t t, const uint32_t (&w)[kWords]) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) {
      row[t + 2 * i] = uint16_t(w[i] & 0xffffu);
      row[t + 2 * i + 1] = uint16_t(w[i] >> 16);
    }
  }
};

// Tiles start at multiples of kTok, so with 16-byte aligned rows ("vec") each tile
// is two aligned 16-byte words per lane.
template <bool BF16>
__device__ __forceinline__ void load_tile(uint32_t (&w)[kWords], const typename Io<BF16>::T* row, int64_t t,
                                          bool vec) {
  if (vec) {
    const uint4* p = reinterpret_cast<const uint4*>(row + t);
#pragma unroll
    for (int i = 0; i < kWords / 4; ++i) {
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

template <bool BF16>
__device__ __forceinline__ void store_tile(typename Io<BF16>::T* row, int64_t t, const float (&y)[Io<BF16>::kTok],
                                           bool vec) {
  uint32_t w[kWords];
  Io<BF16>::pack(w, y);
  if (vec) {
    uint4* p = reinterpret_cast<uint4*>(row + t);
#pragma unroll
    for (int i = 0; i < kWords / 4; ++i) p[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else {
    Io<BF16>::store_elems(row, t, w);
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
  static constexpr int kTok = IO::kTok;
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

  // The staged B/C of token t (wave-uniform: scalar loads into SGPRs).
  struct BC {
    float v[kBC];
  };
  template <int MODE>
  __device__ __forceinline__ void load_bc(BC& r, int64_t t) const {
    const float* p = bc + t * kBC;
    constexpr int kCount = MODE == kAggregate ? kDState : kBC;  // the aggregate needs no C
#pragma unroll
    for (int i = 0; i < kCount; ++i) r.v[i] = p[i];
  }

  // Advances the state by one token; returns y (before the gate) for the output
  // modes, nothing useful for kAggregate.
  template <int MODE>
  __device__ __forceinline__ float token(float uu, float draw, const BC& bct) {
    const float dt = step_size(draw);
    const float dtu = dt * uu;
    if (MODE == kAggregate) {
      sum_dt += dt;
#pragma unroll
      for (int n = 0; n < kDState; ++n) h[n] = fmaf(exp2_hw(dt * A2[n]), h[n], dtu * bct.v[n]);
      return 0.0f;
    }
    float s = 0.0f;
#pragma unroll
    for (int n = 0; n < kDState; ++n) {
      h[n] = fmaf(exp2_hw(dt * A2[n]), h[n], dtu * bct.v[n]);
      s = fmaf(bct.v[kDState + n], h[n], s);
    }
    return fmaf(Dd, uu, s);
  }

  __device__ __forceinline__ float gate(float yv, float zv) const { return HAS_Z ? yv * silu_f32(zv) : yv; }

  // Tokens [ta, tb) in scan order (descending when REV).  ta is a multiple of
  // kTok; tb too unless it is the end of the sequence, so only the top tile can be
  // partial.  Full tiles are software-pipelined: the next tile's u and delta are
  // loaded while the current one is scanned.
  template <bool REV, int MODE>
  __device__ void scan(int64_t ta, int64_t tb) {
    if (tb <= ta) return;
    const int64_t tfull = ta + (tb - ta) / kTok * kTok;
    if (REV) {
      for (int64_t t = tb - 1; t >= tfull; --t) partial_token<MODE>(t);
      full_tiles<REV, MODE>(ta, tfull);
    } else {
      full_tiles<REV, MODE>(ta, tfull);
      for (int64_t t = tfull; t < tb; ++t) partial_token<MODE>(t);
    }
  }

  template <bool REV, int MODE>
  __device__ __forceinline__ void full_tiles(int64_t ta, int64_t tb) {
    const int64_t ntiles = (tb - ta) / kTok;
    if (ntiles <= 0) return;
    uint32_t cu[kWords], cd[kWords], nu[kWords], nd[kWords];
    int64_t t = REV ? tb - kTok : ta;
    load_tile<IO_BF16>(cu, u, t, vec);
    load_tile<IO_BF16>(cd, delta, t, vec);
    for (int64_t i = 0; i < ntiles; ++i) {
      const int64_t tn = REV ? t - kTok : t + kTok;
      if (i + 1 < ntiles) {
        load_tile<IO_BF16>(nu, u, tn, vec);
        load_tile<IO_BF16>(nd, delta, tn, vec);
      }
      tile<REV, MODE>(t, cu, cd);
#pragma unroll
      for (int w = 0; w < kWords; ++w) {
        cu[w] = nu[w];
        cd[w] = nd[w];
      }
      t = tn;
    }
  }

  template <bool REV, int MODE>
  __device__ __forceinline__ void tile(int64_t t, const uint32_t (&wu)[kWords], const uint32_t (&wd)[kWords]) {
    constexpr bool kOut = (MODE == kStore || MODE == kMeet);
    uint32_t wz[kWords];
    // z is needed only for the gate at the end of the tile: its load latency hides
    // behind the tile's tokens
    if (kOut && HAS_Z) load_tile<IO_BF16>(wz, z, t, vec);
    float yt[kTok];
    BC cur, nxt;
    load_bc<MODE>(cur, t + (REV ? kTok - 1 : 0));
#pragma unroll
    for (int jj = 0; jj < kTok; ++jj) {
      const int j = REV ? kTok - 1 - jj : jj;
      // prefetch the next token's B/C: its scalar-load latency hides behind this token
      if (jj + 1 < kTok) load_bc<MODE>(nxt, t + (REV ? j - 1 : j + 1));
      float yv = token<MODE>(IO::get(wu, j), IO::get(wd, j), cur);
      // materialise this token's readout now: otherwise it is sunk towards the
      // tile's store and all tokens' states stay live
      if (MODE != kAggregate) asm volatile("" : "+v"(yv));
      if (MODE == kPark) {
        part[(t + j - t0) * kLanes + lane] = yv;
      } else if (kOut) {
        yt[j] = yv;
      }
      cur = nxt;
      // keep each token's work together: the 16 state chains of one token give
      // enough independent instructions, and hoisting later tokens' exponentials
      // ahead only raises register pressure
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kOut) {
#pragma unroll
      for (int j = 0; j < kTok; ++j) {
        float v = yt[j];
        if (MODE == kMeet) v += part[(t + j - t0) * kLanes + lane];
        yt[j] = gate(v, HAS_Z ? IO::get(wz, j) : 0.0f);
      }
      if (active) store_tile<IO_BF16>(y, t, yt, vec);
    }
  }

  template <int MODE>
  __device__ __forceinline__ void partial_token(int64_t t) {
    const float uu = IO::load(u, t);
    BC cur;
    load_bc<MODE>(cur, t);
    const float yv = token<MODE>(uu, IO::load(delta, t), cur);
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

// A lane's 16 states in the caller's [batch][dim][16] layout (64 contiguous bytes).
__device__ __forceinline__ void load_state16(float (&h)[kDState], const float* p) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < kDState / 4; ++i) {
    const float4 v = q[i];
    h[4 * i] = v.x;
    h[4 * i + 1] = v.y;
    h[4 * i + 2] = v.z;
    h[4 * i + 3] = v.w;
  }
}

__device__ __forceinline__ void store_state16(float* p, const float (&h)[kDState]) {
  float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
  for (int i = 0; i < kDState / 4; ++i) q[i] = make_float4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
}

// State entering a segment: from the carry chain when the sequence is split, else
// the caller's entry state (or zero).
template <class LaneT>
__device__ __forceinline__ void load_entry(LaneT& L, const ScanArgs& a, int dir, int64_t b, int64_t seg,
                                           int64_t g, int64_t nseg, const float* hin) {
  const int64_t d = min64(g * kLanes + threadIdx.x % kLanes, a.dim - 1);
  if (nseg <= 1) {
    if (a.h0) load_state16(L.h, a.h0 + (b * a.dim + d) * kDState);
    return;
  }
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

// Step 2: the chain of segment aggregates in scan order,
//   h_in[k+1] = exp(A sum_dt[k]) h_in[k] + H[k],   h_in[0] = h0 (or 0),
// for every (direction, batch, state, channel).  The combine is associative, so
// each chain is split into runs of consecutive segments, one wave per run (up to
// kCarryParts, each run at least kCarryMinRun segments): each run is first reduced
// on its own (its decay exponent is the sum of its sum_dt), the runs' totals are
// chained through LDS, and each run is walked again from its entry state writing
// h_in.  A block holds 64 channels (coalesced along d) x the runs.
constexpr int kCarryParts = 16;
constexpr int64_t kCarryMinRun = 8;

int carry_parts(int64_t nseg) {
  int p = 1;
  while (p < kCarryParts && nseg / (2 * p) >= kCarryMinRun) p *= 2;
  return p;
}

__global__ __launch_bounds__(kLanes * kCarryParts) void scan_carry_kernel(ScanArgs a, int64_t nseg,
                                                                       const float* __restrict__ agg,
                                                                       float* __restrict__ hin) {
  __shared__ float sh_s[kCarryParts][kLanes];
  __shared__ float sh_h[kCarryParts][kLanes];
  const int nparts = int(blockDim.x) / kLanes;
  const int lane = threadIdx.x % kLanes;
  const int part = threadIdx.x / kLanes;
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  int64_t r = blockIdx.x;
  const int64_t g = r % ngroups;
  r /= ngroups;
  const int n = int(r % kDState);
  r /= kDState;
  const int64_t b = r % a.batch;
  const int dir = int(r / a.batch);
  const int reverse = a.ndir == 2 ? dir : a.reverse;
  const int64_t d_raw = g * kLanes + lane;
  const bool active = d_raw < a.dim;
  const int64_t d = active ? d_raw : a.dim - 1;
  const float* Adir = dir ? a.dir[1].A : a.dir[0].A;
  const float A2 = Adir[d * kDState + n] * kLog2e;
  const int64_t chunk = (nseg + nparts - 1) / nparts;
  const int64_t k0 = min64(nseg, part * chunk), k1 = min64(nseg, k0 + chunk);
  auto seg_of = [&](int64_t k) { return reverse ? nseg - 1 - k : k; };
  // the last segment in scan order has no aggregate (nothing follows it)
  const int64_t kagg = min64(k1, nseg - 1);
  // a run's aggregates are loaded kBatch at a time, all loads in flight together
  // (they do not depend on the chain); runs of up to kBatch segments are loaded once
  constexpr int kBatch = 32;
  float hb[kBatch], sb[kBatch];
  auto load_batch = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t k = kb + i;
      const bool has = k < kagg;
      const int64_t seg = seg_of(has ? k : 0);  // a valid segment even when the run is empty
      hb[i] = has ? agg[agg_index(dir, b, seg, n, d, a.batch, a.dim, nseg)] : 0.0f;
      sb[i] = has ? agg[agg_index(dir, b, seg, kDState, d, a.batch, a.dim, nseg)] : 0.0f;
    }
  };
  float S = 0.0f, H = 0.0f;
  for (int64_t kb = k0; kb < kagg; kb += kBatch) {
    load_batch(kb);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (kb + i < kagg) {
        H = fmaf(exp2_hw(A2 * sb[i]), H, hb[i]);
        S += sb[i];
      }
    }
  }
  sh_s[part][lane] = S;
  sh_h[part][lane] = H;
  __syncthreads();
  float h = a.h0 ? a.h0[(b * a.dim + d) * kDState + n] : 0.0f;  // entry state of the first segment
  for (int q = 0; q < part; ++q) h = fmaf(exp2_hw(A2 * sh_s[q][lane]), h, sh_h[q][lane]);
  const bool reuse = kagg - k0 <= kBatch;  // the run's aggregates are still in registers
  for (int64_t kb = k0; kb < k1; kb += kBatch) {
    if (!reuse) load_batch(kb);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t k = kb + i;
      if (k < k1) {
        if (active) hin[hin_index(dir, b, seg_of(k), n, d, a.batch, a.dim, nseg)] = h;
        if (k < kagg) h = fmaf(exp2_hw(A2 * sb[i]), h, hb[i]);
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
  // the segment scanned last holds the final state
  if (a.h_last && L.active && (a.reverse ? s.seg == 0 : s.seg == nseg - 1))
    store_state16(a.h_last + (s.b * a.dim + s.g * kLanes + threadIdx.x) * kDState, L.h);
}

// len == 0 with a final state requested: the state passes through unchanged.
__global__ __launch_bounds__(256) void state_passthrough_kernel(const float* h0, float* h_last, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) h_last[i] = h0 ? h0[i] : 0.0f;
}

// One token from a stored state.  Four consecutive lanes share a channel and
// each owns four of its states, so the state and A are read and written as
// contiguous 16-byte pieces (a wave covers 16 channels = 1 KiB of state):
//   h_n <- exp(dt A_n) h_n + dt B_n u,  out = (sum_n C_n h_n + D u) silu(z).
// The four partial readouts are summed across the lane quad with DPP.  Grid:
// x over channels (64 per block), y = batch row, so B and C are block-uniform.
// The per-state arithmetic is the same as one token of the sequence kernels.
constexpr int kStepThreads = 256;
constexpr int kStepChannels = kStepThreads / 4;

__device__ __forceinline__ float quad_sum(float v) {
  // xor 1 then xor 2 within each group of four lanes (DPP quad permutations)
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return v;
}

template <bool IO_BF16, bool BC_BF16, bool SOFTPLUS>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepArgs a, int64_t b0) {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  const int64_t b = b0 + blockIdx.y;
  const int q = threadIdx.x & 3;  // which four states
  const int64_t d_raw = int64_t(blockIdx.x) * kStepChannels + (threadIdx.x >> 2);
  const bool active = d_raw < a.dim;
  const int64_t d = active ? d_raw : a.dim - 1;  // idle lanes shadow a valid channel and store nothing
  const int64_t i = b * a.dim + d;
  const float4 hv = reinterpret_cast<const float4*>(a.state + i * kDState)[q];
  const float4 av = reinterpret_cast<const float4*>(a.A + d * kDState)[q];
  float h[4] = {hv.x, hv.y, hv.z, hv.w};
  const float A2[4] = {av.x * kLog2e, av.y * kLog2e, av.z * kLog2e, av.w * kLog2e};
  float Bv[4], Cv[4];
  if (BC_BF16) {
    const uint2 bw = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.B) + b * kDState)[q];
    const uint2 cw = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.C) + b * kDState)[q];
    Bv[0] = bf16_lo(bw.x), Bv[1] = bf16_hi(bw.x), Bv[2] = bf16_lo(bw.y), Bv[3] = bf16_hi(bw.y);
    Cv[0] = bf16_lo(cw.x), Cv[1] = bf16_hi(cw.x), Cv[2] = bf16_lo(cw.y), Cv[3] = bf16_hi(cw.y);
  } else {
    const float4 bv = reinterpret_cast<const float4*>(static_cast<const float*>(a.B) + b * kDState)[q];
    const float4 cv = reinterpret_cast<const float4*>(static_cast<const float*>(a.C) + b * kDState)[q];
    Bv[0] = bv.x, Bv[1] = bv.y, Bv[2] = bv.z, Bv[3] = bv.w;
    Cv[0] = cv.x, Cv[1] = cv.y, Cv[2] = cv.z, Cv[3] = cv.w;
  }
  const float uu = IO::load(static_cast<const T*>(a.u), i);
  const float x = IO::load(static_cast<const T*>(a.delta), i) + (a.delta_bias ? a.delta_bias[d] : 0.0f);
  const float dt = SOFTPLUS ? softplus_f32(x) : x;
  const float dtu = dt * uu;
  float s = 0.0f;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    h[n] = fmaf(exp2_hw(dt * A2[n]), h[n], dtu * Bv[n]);
    s = fmaf(Cv[n], h[n], s);
  }
  s = quad_sum(s);
  if (!active) return;
  reinterpret_cast<float4*>(a.state + i * kDState)[q] = make_float4(h[0], h[1], h[2], h[3]);
  if (q == 0) {
    float yv = fmaf(a.D ? a.D[d] : 0.0f, uu, s);
    if (a.z) yv *= silu_f32(IO::load(static_cast<const T*>(a.z), i));
    IO::store(static_cast<T*>(a.y), i, yv);
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
  const int64_t mid = t0 + ((t1 - t0) / 2) / kTile * kTile;  // a multiple of both tile sizes
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
hipError_t launch_typed(const ScanArgs& a, const Plan& p, float* w, hipStream_t stream, hipEvent_t const* ev) {
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const int64_t nblocks = a.batch * p.nseg * ngroups;
  const size_t esz = IO_BF16 ? 2 : 4;
  bool vec = (size_t(a.len) * esz) % 16 == 0 && aligned16(a.u) && aligned16(a.y) && (!a.z || aligned16(a.z));
  for (int k = 0; k < a.ndir; ++k) vec = vec && aligned16(a.dir[k].delta);
  float* bc = w;
  float* agg = p.nseg > 1 ? w + p.bc_floats : nullptr;
  float* hin = p.nseg > 1 ? agg + p.agg_floats : nullptr;

  const int64_t bc_blocks = int64_t(a.ndir) * a.batch * ((a.len + 63) / 64);
  mark(0);
  if (a.bc_bf16) {
    hipLaunchKernelGGL(stage_bc_kernel<true>, dim3(unsigned(bc_blocks)), dim3(256), 0, stream, a, bc);
  } else {
    hipLaunchKernelGGL(stage_bc_kernel<false>, dim3(unsigned(bc_blocks)), dim3(256), 0, stream, a, bc);
  }
  mark(1);
  if (p.nseg > 1) {
    hipLaunchKernelGGL((scan_aggregate_kernel<IO_BF16, SOFTPLUS>), dim3(unsigned(nblocks), unsigned(a.ndir)),
                       dim3(kLanes), 0, stream, a, p.seg_len, p.nseg, static_cast<const float*>(bc), agg, int(vec));
    mark(2);
    const int64_t carry_blocks = int64_t(a.ndir) * a.batch * kDState * ngroups;
    hipLaunchKernelGGL(scan_carry_kernel, dim3(unsigned(carry_blocks)), dim3(kLanes * carry_parts(p.nseg)), 0, stream,
                       a, p.nseg, static_cast<const float*>(agg), hin);
  }
  if (p.nseg <= 1) mark(2);
  mark(3);
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
  mark(4);
  return hipGetLastError();
}

template <bool IO_BF16>
hipError_t launch_io(const ScanArgs& a, const Plan& p, float* w, hipStream_t stream, hipEvent_t const* ev) {
  if (a.softplus) {
    return a.z ? launch_typed<IO_BF16, true, true>(a, p, w, stream, ev) : launch_typed<IO_BF16, true, false>(a, p, w, stream, ev);
  }
  return a.z ? launch_typed<IO_BF16, false, true>(a, p, w, stream, ev) : launch_typed<IO_BF16, false, false>(a, p, w, stream, ev);
}

}  // namespace

// Resident wave slots of the scan kernels on MI355X: 256 CUs x 4 SIMDs x 3 waves
// (the scan kernels are held to <= 168 VGPRs).
constexpr int64_t kWaveSlots = 256 * 4 * 3;
// Bidirectional segments: the LDS meeting buffer (seg_len x 64 lanes x 4 B) must
// leave room for eight two-wave blocks per CU.
constexpr int64_t kBidirSegment = 64;

// Splitting along the sequence.  Sequences up to kShortMax tokens are scanned whole.
// Longer ones are cut into equal segments (multiples of kTile tokens) so that the
// output step has about two rounds of resident waves: enough waves to cover load
// latency and even out per-wave speed, without the long carry chain and large
// aggregate buffers of many short segments (measured on the long-sequence and
// Mamba-YOLO workloads).
Plan make_plan(int64_t batch, int64_t dim, int64_t len, int ndir) {
  Plan p{};
  const int64_t ngroups = (dim + kLanes - 1) / kLanes;
  const int64_t groups = std::max<int64_t>(1, batch * ngroups);
  p.seg_len = std::max<int64_t>(len, 1);
  p.nseg = 1;
  if (len > kShortMax) {
    int64_t seg_len;
    if (ndir == 2) {
      seg_len = kBidirSegment;
    } else {
      const int64_t target_segs = std::max<int64_t>(2, 2 * kWaveSlots / groups);
      seg_len = (len + target_segs - 1) / target_segs;
      seg_len = std::max<int64_t>(kSegAlign, (seg_len + kTile - 1) / kTile * kTile);
    }
    // keep the block count within a 1-D grid
    while ((len + seg_len - 1) / seg_len > 1 && batch * ((len + seg_len - 1) / seg_len) * ngroups > (int64_t(1) << 30))
      seg_len *= 2;
    p.seg_len = seg_len;
    p.nseg = (len + seg_len - 1) / seg_len;
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

hipError_t launch_scan(const ScanArgs& a, const Plan& p, float* ws, hipStream_t stream, hipEvent_t const* events) {
  return a.io_bf16 ? launch_io<true>(a, p, ws, stream, events) : launch_io<false>(a, p, ws, stream, events);
}

hipError_t launch_state_passthrough(const ScanArgs& a, hipStream_t stream) {
  const int64_t n = a.batch * a.dim * kDState;
  hipLaunchKernelGGL(state_passthrough_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, a.h0, a.h_last,
                     n);
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  constexpr int64_t kMaxRows = 65535;  // grid y limit: batch rows per launch
  const int key = (a.io_bf16 ? 4 : 0) | (a.bc_bf16 ? 2 : 0) | (a.softplus ? 1 : 0);
  for (int64_t b0 = 0; b0 < a.batch; b0 += kMaxRows) {
    const dim3 grid(unsigned((a.dim + kStepChannels - 1) / kStepChannels), unsigned(std::min(kMaxRows, a.batch - b0)));
    const dim3 block(kStepThreads);
    switch (key) {
      case 0: hipLaunchKernelGGL((step_kernel<false, false, false>), grid, block, 0, stream, a, b0); break;
      case 1: hipLaunchKernelGGL((step_kernel<false, false, true>), grid, block, 0, stream, a, b0); break;
      case 2: hipLaunchKernelGGL((step_kernel<false, true, false>), grid, block, 0, stream, a, b0); break;
      case 3: hipLaunchKernelGGL((step_kernel<false, true, true>), grid, block, 0, stream, a, b0); break;
      case 4: hipLaunchKernelGGL((step_kernel<true, false, false>), grid, block, 0, stream, a, b0); break;
      case 5: hipLaunchKernelGGL((step_kernel<true, false, true>), grid, block, 0, stream, a, b0); break;
      case 6: hipLaunchKernelGGL((step_kernel<true, true, false>), grid, block, 0, stream, a, b0); break;
      default: hipLaunchKernelGGL((step_kernel<true, true, true>), grid, block, 0, stream, a, b0); break;
    }
  }
  return hipGetLastError();
}

}  // namespace sscan
