// sscan_device.h -- device-side building blocks shared by the forward and backward
// gfx950 kernels of the selective scan: storage-type tiles, the per-lane scan of one
// channel (lane = channel, 16 fp32 states in registers), the B/C staging kernel,
// the segment-aggregate kernel and the carry chain between segments.  Included by
// sscan_kernels.hip and sscan_bwd.hip (everything here has internal linkage).
#pragma once

#include "sscan_internal.h"

#include <algorithm>
#include <type_traits>

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
// The output kernels with bf16 I/O and no convolution (one direction, and two
// directions meeting in LDS) are held to 128 VGPRs, four waves per SIMD, and load
// each tile at its start (long-sequence output pass 1.386 -> 1.328 ms).  With the
// tile prefetch kept, the bidirectional blocks ran slower at four waves (Mamba-YOLO
// rows 0.187 -> 0.194 ms); the other variants would spill several times more and
// keep three.
#define SSCAN_OUT_OCCUPANCY(FOUR) __attribute__((amdgpu_waves_per_eu((FOUR) ? 4 : 3, 8)))

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// The workgroups of a launch are dealt to the chip's eight XCDs in turn (block i
// to XCD i mod 8), each XCD with its own L2.  xcd_stretch renumbers block i to its
// place in a contiguous stretch of the launch owned by XCD i mod 8, so that
// neighbouring logical blocks run on one XCD and data they share is fetched into
// one L2.  It is a bijection on [0, n) whatever the dispatch order.
constexpr int64_t kXcds = 8;
__device__ __forceinline__ int64_t xcd_stretch(int64_t i, int64_t n) {
  const int64_t x = i % kXcds, q = i / kXcds, m = n / kXcds, r = n % kXcds;
  return x < r ? x * (m + 1) + q : r * (m + 1) + (x - r) * m + q;
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = max(x, 0) + log1p(w), w = exp(-|x|) in (0, 1].  log1p(w) is
// log(s) for s = 1 + w rounded, plus the rounding error c = w - (s - 1) (exact):
// log(s + c) = log(s) + c/s + O(c^2).  Adding c in place of c/s is off by
// c w / s <= 2^-24 w, and log1p(w) >= w ln 2 on (0, 1], so the substitution
// costs at most 0.72 units in the result's last place.  This keeps full relative
// accuracy for small step sizes (1e-4 and below), where log(s) alone loses it.
__device__ __forceinline__ float softplus_f32(float x) {
  const float w = exp2_hw(-fabsf(x) * kLog2e);
  const float s = 1.0f + w;
  const float c = w - (s - 1.0f);
  const float lp = fmaf(log2_hw(s), kLn2, c);
  return fmaxf(x, 0.0f) + lp;
}

__device__ __forceinline__ float silu_f32(float x) { return x * rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// Sum over each group of four lanes (DPP quad permutations: xor 1, then xor 2).
// (bound_ctrl set: every quad lane is a valid source, and it lets the compiler fold
// each move into the add as its DPP source)
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return v;
}

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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_uint4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// A bf16 tile is half of a 128-byte line, and by the time a lane reaches the
// line's other half it has left L2, so it would be fetched twice.  Where rows are
// 128-byte aligned the one-direction output and aggregate passes load each line of
// u and delta once: the half scanned first into registers, the other half with
// gfx950's direct-to-LDS loads (each lane's 16 bytes land at base + lane * 16) into
// a per-wave slot, read back when that tile comes up.  Slot: [u, delta][4][64
// lanes] x 16 bytes = 8 KB per wave.
constexpr int kLineSlot = 2 * 4 * 64;

// What a scan pass does with each token's output.
enum Mode : int {
  kAggregate = 0,  // no readout: advance the state, sum the step sizes
  kStore = 1,      // gate and store y
  kPark = 2,       // park y (ungated, one direction) in the LDS meeting buffer
  kMeet = 3,       // add the partner direction's parked y, gate, store
  kAdjoint = 4,    // adjoint recurrence (backward pass): u holds dLoss/dout, the lane's
                   // h holds mu and runs opposite to the direction's scan order
};

// Front-end convolution modes of the lane scan.
enum Conv : int {
  kNoConv = 0,    // u is read as is
  kConvLin = 1,   // u = bias + depthwise convolution of x
  kConvSilu = 2,  // u = silu(bias + depthwise convolution of x)
};

// The convolution reads a fixed window of five tokens, x[t-3 .. t+1]; a kernel of
// `width` taps starting `left` tokens before t sits in it with zeros elsewhere.
constexpr int kConvTaps = 5;
constexpr int kConvBack = 3;

// One lane's view of one direction of one (batch, channel) row.  SOFTPLUS, HAS_Z
// and CONV are compile-time so that a tile's tokens form one straight-line block.
// Y_F32 stores y in fp32 whatever the input dtype (partial outputs that are summed
// before rounding, in the multi-order scan).  GPARK moves the bidirectional
// kernel's meeting buffer from LDS to global memory.
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z, int CONV = kNoConv, bool Y_F32 = false, bool GPARK = false>
struct Lane {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  using TY = typename std::conditional<Y_F32, float, T>::type;
  static constexpr int kTok = IO::kTok;
  static constexpr int kConv = CONV;
  const T* u;
  const T* delta;
  const T* z;     // nullable
  TY* y;
  const float* __restrict__ bc;  // staged B/C of this (direction, batch): bc[t * 32 + ...]
  // meeting buffer of the bidirectional kernel, [t - t0][64]: LDS, or (GPARK) the
  // block's slice of a workspace buffer
  typename std::conditional<GPARK, float*, lds_float*>::type part;
  int64_t t0;     // first token of the segment (LDS buffer origin)
  float A2[kDState];  // A * log2(e)
  float h[kDState];
  float bias, Dd;
  float sum_dt;
  float cw[kConvTaps], cb;  // front-end convolution taps over x[t-3 .. t+1], bias
  int64_t len;
  int lane;
  bool vec;       // 16-byte vector access is valid for full tiles
  bool active;    // lane maps to a real channel (stores enabled)
  bool line;      // rows are 128-byte aligned and lbuf is this wave's line slot
  lds_uint4* lbuf;

  // The one-direction output and aggregate passes with bf16 I/O load whole lines.
  template <int MODE>
  static constexpr bool kLinePairs = IO_BF16 && CONV == kNoConv && !GPARK && (MODE == kStore || MODE == kAggregate);

  // Issues the direct-to-LDS loads of the tile of u and delta at t (the other half
  // of a line whose first half is being loaded into registers).
  __device__ __forceinline__ void park_half(int64_t t) const {
    const uint4* pu = reinterpret_cast<const uint4*>(u + t);
    const uint4* pd = reinterpret_cast<const uint4*>(delta + t);
#pragma unroll
    for (int i = 0; i < kWords / 4; ++i) {
      __builtin_amdgcn_global_load_lds((global_void*)(pu + i), (lds_void*)(lbuf + i * kLanes), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((global_void*)(pd + i), (lds_void*)(lbuf + (kWords / 4 + i) * kLanes), 16, 0, 0);
    }
  }

  // Reads the parked tile back (the compiler waits for the loads that wrote it).
  __device__ __forceinline__ void unpark_half(uint32_t (&wu)[kWords], uint32_t (&wd)[kWords]) const {
#pragma unroll
    for (int i = 0; i < kWords / 4; ++i) {
      const u32x4 a = lbuf[i * kLanes + lane];
      const u32x4 b = lbuf[(kWords / 4 + i) * kLanes + lane];
      wu[4 * i] = a.x;
      wu[4 * i + 1] = a.y;
      wu[4 * i + 2] = a.z;
      wu[4 * i + 3] = a.w;
      wd[4 * i] = b.x;
      wd[4 * i + 1] = b.y;
      wd[4 * i + 2] = b.z;
      wd[4 * i + 3] = b.w;
    }
  }

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
    // the aggregate needs only B, the adjoint only C
    constexpr int kFirst = MODE == kAdjoint ? kDState : 0;
    constexpr int kEnd = MODE == kAggregate ? kDState : kBC;
#pragma unroll
    for (int i = kFirst; i < kEnd; ++i) r.v[i] = p[i];
  }

  // Advances the state by one token; returns y (before the gate) for the output
  // modes, nothing useful for kAggregate.
  template <int MODE>
  __device__ __forceinline__ float token(float uu, float draw, const BC& bct, float zv = 0.0f) {
    const float dt = step_size(draw);
    if (MODE == kAdjoint) {
      // lambda = C dy + mu;  mu <- exp(dt A) lambda   (dy = dout * silu(z))
      sum_dt += dt;
      const float dy = HAS_Z ? uu * silu_f32(zv) : uu;
#pragma unroll
      for (int n = 0; n < kDState; ++n) h[n] = exp2_hw(dt * A2[n]) * fmaf(bct.v[kDState + n], dy, h[n]);
      return 0.0f;
    }
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

  // a finished tile of y: the storage dtype, or fp32 for Y_F32
  __device__ __forceinline__ void store_y(int64_t t, const float (&yt)[kTok]) {
    if (!Y_F32) {
      store_tile<IO_BF16>(reinterpret_cast<T*>(y), t, yt, vec);
    } else if (vec) {
      float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + t);
#pragma unroll
      for (int i = 0; i < kTok / 4; ++i) p[i] = make_float4(yt[4 * i], yt[4 * i + 1], yt[4 * i + 2], yt[4 * i + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < kTok; ++j) reinterpret_cast<float*>(y)[t + j] = yt[j];
    }
  }

  // u from the convolution window x[t-3 .. t+1]
  __device__ __forceinline__ float conv_out(const float (&xw)[kConvTaps]) const {
    float acc = cb;
#pragma unroll
    for (int k = 0; k < kConvTaps; ++k) acc = fmaf(cw[k], xw[k], acc);
    return CONV == kConvSilu ? silu_f32(acc) : acc;
  }

  // x at token t, zero outside the sequence (the convolution's padding)
  __device__ __forceinline__ float x_at(int64_t t) const { return (t >= 0 && t < len) ? IO::load(u, t) : 0.0f; }

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
    // The next tile is loaded while this one runs, except in the bf16 output passes
    // held to four waves per SIMD (one direction, and two directions meeting in LDS):
    // there the prefetched tile does not fit in 128 VGPRs, and spilling it waited for
    // its loads anyway, so each tile is loaded at its start (long-sequence output
    // pass 1.363 -> 1.328 ms; Mamba-YOLO rows 0.185 -> 0.181 ms).  Long single
    // bidirectional segments (meeting in global memory, Vim) ran 11% slower so and
    // keep three waves and the prefetch.
    constexpr bool kAhead =
        !(IO_BF16 && CONV == kNoConv && (MODE == kStore || ((MODE == kPark || MODE == kMeet) && !GPARK)));
    int64_t t = REV ? tb - kTok : ta;
    // Tiles in pairs that fill a 128-byte line: the first visited of a pair (even i)
    // is loaded into registers and its partner (the next tile) parked in LDS.
    const bool pairs = kLinePairs<MODE> && line && (ta % (2 * kTok)) == 0 && (tb % (2 * kTok)) == 0;
    if (kAhead) {
      load_tile<IO_BF16>(cu, u, t, vec);
      load_tile<IO_BF16>(cd, delta, t, vec);
      if (pairs) park_half(REV ? t - kTok : t + kTok);
    }
    // convolution halo of the tile: the three tokens before it and the one after.
    // Inside a run of tiles it comes from the neighbouring tiles' registers (the one
    // just scanned, the one prefetched); only the run's ends read memory.
    float xl[kConvBack] = {}, xr = 0.0f;
    if (CONV != kNoConv) {
      if (REV) {
        xr = x_at(t + kTok);
      } else {
#pragma unroll
        for (int k = 0; k < kConvBack; ++k) xl[k] = x_at(t - kConvBack + k);
      }
    }
    for (int64_t i = 0; i < ntiles; ++i) {
      const int64_t tn = REV ? t - kTok : t + kTok;
      const bool more = i + 1 < ntiles;
      if (!kAhead) {
        if (pairs && (i & 1)) {
          unpark_half(cu, cd);
        } else {
          load_tile<IO_BF16>(cu, u, t, vec);
          load_tile<IO_BF16>(cd, delta, t, vec);
          if (pairs) park_half(tn);
        }
      } else if (more) {
        if (pairs && !(i & 1)) {
          unpark_half(nu, nd);
        } else {
          load_tile<IO_BF16>(nu, u, tn, vec);
          load_tile<IO_BF16>(nd, delta, tn, vec);
          if (pairs) {
            // the slot still holds the tile read back one tile ago, whose registers
            // this tile is about to use: let that read finish before it is overwritten
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            park_half(REV ? tn - kTok : tn + kTok);
          }
        }
      }
      if (CONV != kNoConv) {
        if (REV) {
#pragma unroll
          for (int k = 0; k < kConvBack; ++k) xl[k] = more ? IO::get(nu, kTok - kConvBack + k) : x_at(t - kConvBack + k);
        } else {
          xr = more ? IO::get(nu, 0) : x_at(t + kTok);
        }
      }
      tile<REV, MODE>(t, cu, cd, xl, xr);
      if (CONV != kNoConv) {
        if (REV) {
          xr = IO::get(cu, 0);
        } else {
#pragma unroll
          for (int k = 0; k < kConvBack; ++k) xl[k] = IO::get(cu, kTok - kConvBack + k);
        }
      }
      if (kAhead) {
#pragma unroll
        for (int w = 0; w < kWords; ++w) {
          cu[w] = nu[w];
          cd[w] = nd[w];
        }
      }
      t = tn;
    }
  }

  template <bool REV, int MODE>
  __device__ __forceinline__ void tile(int64_t t, const uint32_t (&wu)[kWords], const uint32_t (&wd)[kWords],
                                      const float (&xl)[kConvBack], float xr) {
    constexpr bool kOut = (MODE == kStore || MODE == kMeet);
    uint32_t wz[kWords];
    // z is needed only for the gate at the end of the tile (the adjoint reads it at
    // every token)
    if ((kOut || MODE == kAdjoint) && HAS_Z) load_tile<IO_BF16>(wz, z, t, vec);
    float yt[kTok];
    BC cur, nxt;
    load_bc<MODE>(cur, t + (REV ? kTok - 1 : 0));
#pragma unroll
    for (int jj = 0; jj < kTok; ++jj) {
      const int j = REV ? kTok - 1 - jj : jj;
      // Scalar loads return out of order, so the wait before this token's B/C is a
      // wait for every scalar load in flight.  Take it here, before the next token's
      // loads go out: that wait then finds nothing issued less than a token ago
      // (long-sequence forward: output pass 1.435 -> 1.381 ms, aggregate 1.039 ->
      // 1.025 ms).  The adjoint chain, which also waits for z at every token, and
      // the aggregate with the convolution in front ran 5% slower with it and keep
      // the compiler's placement.
      if constexpr (MODE != kAdjoint && !(MODE == kAggregate && CONV != kNoConv)) {
        asm volatile("" ::"s"(cur.v[0]));
        __builtin_amdgcn_sched_barrier(0);
      }
      // prefetch the next token's B/C: its scalar-load latency hides behind this token
      if (jj + 1 < kTok) load_bc<MODE>(nxt, t + (REV ? j - 1 : j + 1));
      float uu = IO::get(wu, j);
      if (CONV != kNoConv) {
        float xw[kConvTaps];
#pragma unroll
        for (int k = 0; k < kConvTaps; ++k) {
          const int jk = j - kConvBack + k;  // compile-time: inside the tile or in the halo
          xw[k] = jk < 0 ? xl[jk + kConvBack < 0 ? 0 : jk + kConvBack] : (jk >= kTok ? xr : IO::get(wu, jk < kTok ? jk : 0));
        }
        uu = conv_out(xw);
      }
      float yv = token<MODE>(uu, IO::get(wd, j), cur, (MODE == kAdjoint && HAS_Z) ? IO::get(wz, j) : 0.0f);
      // materialise this token's readout now: otherwise it is sunk towards the
      // tile's store and all tokens' states stay live
      if (MODE != kAggregate && MODE != kAdjoint) asm volatile("" : "+v"(yv));
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
      if (active) store_y(t, yt);
    }
  }

  template <int MODE>
  __device__ __forceinline__ void partial_token(int64_t t) {
    float uu;
    if (CONV != kNoConv) {
      float xw[kConvTaps];
#pragma unroll
      for (int k = 0; k < kConvTaps; ++k) xw[k] = x_at(t - kConvBack + k);
      uu = conv_out(xw);
    } else {
      uu = IO::load(u, t);
    }
    BC cur;
    load_bc<MODE>(cur, t);
    const float yv = token<MODE>(uu, IO::load(delta, t), cur, (MODE == kAdjoint && HAS_Z) ? IO::load(z, t) : 0.0f);
    if (MODE == kPark) {
      part[(t - t0) * kLanes + lane] = yv;
    } else if (MODE == kStore || MODE == kMeet) {
      float v = (MODE == kMeet) ? yv + part[(t - t0) * kLanes + lane] : yv;
      if (HAS_Z) v *= silu_f32(IO::load(z, t));
      if (active) {
        if (Y_F32) {
          reinterpret_cast<float*>(y)[t] = v;
        } else {
          IO::store(reinterpret_cast<T*>(y), t, v);
        }
      }
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

// Chains walked over runs of consecutive segments (or windows): after each one, a
// (segment, channel)'s 16 values so far contiguous, and its summed step sizes.
__device__ __forceinline__ size_t chain_state_index(int dir, int64_t b, int64_t k, int64_t d, int64_t batch,
                                                    int64_t dim, int64_t nseg) {
  return ((((size_t)dir * batch + b) * nseg + k) * dim + d) * kDState;
}
__device__ __forceinline__ size_t chain_sum_index(int dir, int64_t b, int64_t k, int64_t d, int64_t batch,
                                                  int64_t dim, int64_t nseg) {
  return (((size_t)dir * batch + b) * nseg + k) * dim + d;
}

// The state chain across the segments of a split sequence.  Segments are grouped
// in runs of run_len: p and s hold, after each segment, the state reached walking
// its run from a zero state and the step sizes summed so far (not kept for a
// run's last segment, so absent when run_len is 1); r holds each run's totals in
// the layout the carry kernel reads; e the state entering each run.
struct SegChain {
  float* p;  // [ndir][batch][nseg][dim][16]
  float* s;  // [ndir][batch][nseg][dim]
  float* r;  // [ndir][batch][nrun][17][dim]
  float* e;  // [ndir][batch][nrun][16][dim]
  int64_t run_len, nrun;
};

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
  L.y = static_cast<typename LaneT::TY*>(a.y) + row;
  L.bc = bc + ((size_t)dir * a.batch + b) * a.len * kBC;
  L.part = nullptr;
  L.t0 = 0;
#pragma unroll
  for (int n = 0; n < kDState; ++n) L.A2[n] = p.A[d * kDState + n] * kLog2e;
  L.bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
  L.Dd = p.D ? p.D[d] : 0.0f;
  L.sum_dt = 0.0f;
  L.len = a.len;
  L.cb = 0.0f;
#pragma unroll
  for (int k = 0; k < kConvTaps; ++k) L.cw[k] = 0.0f;
  if (LaneT::kConv != kNoConv) {
    // tap j of the kernel multiplies x[t - conv_left + j], slot kConvBack - conv_left + j
#pragma unroll
    for (int k = 0; k < kConvTaps; ++k) {
      const int j = k - (kConvBack - a.conv_left);
      L.cw[k] = (j >= 0 && j < a.conv_width) ? a.conv_w[d * a.conv_width + j] : 0.0f;
    }
    L.cb = a.conv_b ? a.conv_b[d] : 0.0f;
  }
  L.lane = lane;
  L.vec = vec;
  L.line = false;
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

// State entering a segment: the caller's entry state (or zero) when the sequence
// is not split; else the state entering the segment's run, advanced over the
// run's segments before this one: p + exp(A s) e, the composition of two affine
// steps (e alone for the run's first segment in scan order).  Needs L.A2.
template <class LaneT>
__device__ __forceinline__ void load_entry(LaneT& L, const ScanArgs& a, int dir, int64_t b, int64_t seg,
                                           int64_t g, int64_t nseg, const SegChain& ch) {
  const int64_t d = min64(g * kLanes + threadIdx.x % kLanes, a.dim - 1);
  if (nseg <= 1) {
    if (a.h0) load_state16(L.h, a.h0 + (b * a.dim + d) * kDState);
    return;
  }
  const int64_t run = seg / ch.run_len;
#pragma unroll
  for (int n = 0; n < kDState; ++n) L.h[n] = ch.e[hin_index(dir, b, run, n, d, a.batch, a.dim, ch.nrun)];
  const bool rev = (a.ndir == 2 ? dir : a.reverse) != 0;
  const int64_t lo = run * ch.run_len, hi = min64(nseg, lo + ch.run_len) - 1;
  if (rev ? seg < hi : seg > lo) {
    const int64_t k = rev ? seg + 1 : seg - 1;
    float p[kDState];
    load_state16(p, ch.p + chain_state_index(dir, b, k, d, a.batch, a.dim, nseg));
    const float sd = ch.s[chain_sum_index(dir, b, k, d, a.batch, a.dim, nseg)];
#pragma unroll
    for (int n = 0; n < kDState; ++n) L.h[n] = fmaf(exp2_hw(L.A2[n] * sd), L.h[n], p[n]);
  }
}

// Stage B and C token-major in fp32: bc[dir][b][t][0..15] = B[b][:, t],
// bc[dir][b][t][16..31] = C[b][:, t].  One block per (direction, batch row, 64
// tokens).  Each thread reads 8 consecutive tokens of one of the 32 rows (one
// 16-byte load for bf16, two for fp32, when the rows start 16-byte aligned: vec);
// the tile turns through LDS and each thread writes two 16-byte pieces of the
// token-major rows (128 bytes per token, always aligned in the workspace).
template <bool BC_BF16>
__global__ __launch_bounds__(256) void stage_bc_kernel(ScanArgs a, float* __restrict__ bc, int vec) {
  __shared__ float tile[kBC][65];
  const int64_t ntiles = (a.len + 63) / 64;
  const int64_t tt = blockIdx.x % ntiles;
  const int64_t db = blockIdx.x / ntiles;  // dir * batch + b
  const int dir = int(db / a.batch);
  const int64_t b = db % a.batch;
  const DirArgs p = dir ? a.dir[1] : a.dir[0];
  const int64_t t0 = tt * 64;
  const int r = int(threadIdx.x) >> 3, c0 = (int(threadIdx.x) & 7) * 8;  // row r, tokens c0 .. c0 + 7
  const void* src = r < kDState ? p.B : p.C;
  const size_t at = ((size_t)b * kDState + (r % kDState)) * a.len + t0 + c0;
  float v[8];
  if (vec && t0 + c0 + 8 <= a.len) {
    if (BC_BF16) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + at);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(ws[k]);
        v[2 * k + 1] = bf16_hi(ws[k]);
      }
    } else {
      const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(src) + at);
      const float4 x0 = q[0], x1 = q[1];
      v[0] = x0.x, v[1] = x0.y, v[2] = x0.z, v[3] = x0.w;
      v[4] = x1.x, v[5] = x1.y, v[6] = x1.z, v[7] = x1.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool in = t0 + c0 + k < a.len;
      v[k] = !in ? 0.0f
                 : BC_BF16 ? Io<true>::load(static_cast<const uint16_t*>(src), at + k)
                           : static_cast<const float*>(src)[at + k];
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) tile[r][c0 + k] = v[k];
  __syncthreads();
  float* out = bc + ((size_t)db * a.len + t0) * kBC;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = int(threadIdx.x) + h * 256;
    const int t = i >> 3, q = (i & 7) * 4;  // token t, rows q .. q + 3
    if (t0 + t < a.len)
      *reinterpret_cast<float4*>(out + (size_t)t * kBC + q) =
          make_float4(tile[q][t], tile[q + 1][t], tile[q + 2][t], tile[q + 3][t]);
  }
}

// Stages B and C of every direction of a call into bc (ndir * batch * len * 32 floats).
inline void launch_stage_bc(const ScanArgs& a, float* bc, hipStream_t stream) {
  const size_t esz = a.bc_bf16 ? 2 : 4;
  bool vec = (size_t(a.len) * esz) % 16 == 0;
  for (int k = 0; k < a.ndir; ++k)
    vec = vec && (reinterpret_cast<uintptr_t>(a.dir[k].B) & 15u) == 0 &&
          (reinterpret_cast<uintptr_t>(a.dir[k].C) & 15u) == 0;
  const dim3 grid(unsigned(int64_t(a.ndir) * a.batch * ((a.len + 63) / 64)));
  if (a.bc_bf16) {
    hipLaunchKernelGGL(stage_bc_kernel<true>, grid, dim3(256), 0, stream, a, bc, int(vec));
  } else {
    hipLaunchKernelGGL(stage_bc_kernel<false>, grid, dim3(256), 0, stream, a, bc, int(vec));
  }
}

// Step 1: the segments of a run walked in scan order from a zero state, storing
// after each one (but the run's last) the state so far and the summed step sizes,
// and at the end the run's totals.  The segment scanned last in the whole row is
// skipped (nothing follows it).  Grid: batch * nrun * ngroups one-wave blocks;
// blockIdx.y selects the direction.  RUNS = false is the one-segment-per-run form
// without the loop (fewer registers: four waves per SIMD in the plain scan).
template <bool IO_BF16, bool SOFTPLUS, int CONV = kNoConv, bool RUNS = false>
__global__ __launch_bounds__(kLanes) SSCAN_OCCUPANCY void scan_aggregate_kernel(ScanArgs a, int64_t seg_len, int64_t nseg,
                                                                SegChain ch, const float* __restrict__ bc, int vec) {
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const SegIndex s = decode_block(blockIdx.x, ngroups, ch.nrun);  // s.seg: the run
  const int dir = blockIdx.y;
  const int reverse = a.ndir == 2 ? dir : a.reverse;
  const int64_t last = reverse ? 0 : nseg - 1;
  Lane<IO_BF16, SOFTPLUS, false, CONV> L;
  constexpr bool kLines = IO_BF16 && CONV == kNoConv;
  __shared__ uint4 lslot[kLines ? kLineSlot : 1];
  const int64_t d = s.g * kLanes + threadIdx.x;
  if (!RUNS) {
    if (s.seg == last) return;
    init_lane(L, a, dir, s.b, s.g, bc, (vec & 1) != 0);
    if (kLines) {
      L.line = (vec & 2) != 0;
      L.lbuf = (lds_uint4*)lslot;
    }
    const int64_t t0 = s.seg * seg_len;
    const int64_t t1 = min64(a.len, t0 + seg_len);
    if (reverse) {
      L.template scan<true, kAggregate>(t0, t1);
    } else {
      L.template scan<false, kAggregate>(t0, t1);
    }
  } else {
    const int64_t k_lo = s.seg * ch.run_len, k_hi = min64(nseg, k_lo + ch.run_len);
    if (k_hi - k_lo == 1 && k_lo == last) return;
    init_lane(L, a, dir, s.b, s.g, bc, (vec & 1) != 0);
    if (kLines) {
      L.line = (vec & 2) != 0;
      L.lbuf = (lds_uint4*)lslot;
    }
    for (int64_t i = k_lo; i < k_hi; ++i) {
      const int64_t k = reverse ? k_lo + k_hi - 1 - i : i;
      if (k == last) break;
      const int64_t t0 = k * seg_len;
      const int64_t t1 = min64(a.len, t0 + seg_len);
      if (reverse) {
        L.template scan<true, kAggregate>(t0, t1);
      } else {
        L.template scan<false, kAggregate>(t0, t1);
      }
      if (i + 1 < k_hi && L.active) {
        store_state16(ch.p + chain_state_index(dir, s.b, k, d, a.batch, a.dim, nseg), L.h);
        ch.s[chain_sum_index(dir, s.b, k, d, a.batch, a.dim, nseg)] = L.sum_dt;
      }
    }
  }
  if (!L.active) return;
#pragma unroll
  for (int n = 0; n < kDState; ++n) ch.r[agg_index(dir, s.b, s.seg, n, d, a.batch, a.dim, ch.nrun)] = L.h[n];
  ch.r[agg_index(dir, s.b, s.seg, kDState, d, a.batch, a.dim, ch.nrun)] = L.sum_dt;
}

// Step 2: the chain of run totals (segments grouped in runs; a run may be one
// segment) in scan order,
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

// kBatch: aggregates a lane keeps in flight; runs of up to kBatch elements are
// loaded once.  16 keeps the kernel near 56 VGPRs (two 16-wave blocks per CU); 32
// (about 80 VGPRs, one block per CU) serves longer runs, which 16 would read twice.
template <int kBatch>
__global__ __launch_bounds__(kLanes * kCarryParts) void scan_carry_kernel(ScanArgs a, int64_t nseg,
                                                                       const float* __restrict__ agg,
                                                                       float* __restrict__ hin, int flip) {
  __shared__ float sh_s[kCarryParts][kLanes];
  __shared__ float sh_h[kCarryParts][kLanes];
  const int nparts = int(blockDim.x) / kLanes;
  const int lane = threadIdx.x % kLanes;
  // wave-uniform: read through readfirstlane so the chain's indices stay scalar
  const int part = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kLanes);
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  int64_t r = blockIdx.x;
  const int64_t g = r % ngroups;
  r /= ngroups;
  const int n = int(r % kDState);
  r /= kDState;
  const int64_t b = r % a.batch;
  const int dir = int(r / a.batch);
  // chain order: the direction's scan order, or the opposite one (flip: the
  // adjoint of the backward pass travels against the scan)
  const int reverse = (a.ndir == 2 ? dir : a.reverse) ^ flip;
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
  // Addresses split into a wave-uniform row (scalar registers) and the lane's
  // channel offset, so the per-step loads and stores cost no vector arithmetic.
  const uint32_t dl = uint32_t(d);
  auto agg_row = [&](int64_t seg, int row) {  // row n: H of state n; row kDState: S
    return agg + ((((size_t)dir * a.batch + b) * nseg + seg) * (kDState + 1) + row) * a.dim;
  };
  auto hin_row = [&](int64_t seg) { return hin + ((((size_t)dir * a.batch + b) * nseg + seg) * kDState + n) * a.dim; };
  // a run's aggregates are loaded kBatch at a time, all loads in flight together
  // (they do not depend on the chain)
  float hb[kBatch], sb[kBatch];
  auto load_batch = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t k = kb + i;
      const bool has = k < kagg;
      const int64_t seg = seg_of(has ? k : 0);  // a valid segment even past the run's end
      hb[i] = has ? agg_row(seg, n)[dl] : 0.0f;
      sb[i] = has ? agg_row(seg, kDState)[dl] : 0.0f;
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
        if (active) hin_row(seg_of(k))[dl] = h;
        if (k < kagg) h = fmaf(exp2_hw(A2 * sb[i]), h, hb[i]);
      }
    }
  }
}

// The carry over nseg chain elements for every (direction, batch row, state,
// 64-channel group): the batch size by run length (on the long-sequence forward,
// 512 segments in runs of 32: 48 us with 16, 38 us with 32).
inline void launch_carry(const ScanArgs& a, int64_t nseg, const float* agg, float* hin, int flip,
                         hipStream_t stream) {
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const int parts = carry_parts(nseg);
  const int64_t run = (nseg + parts - 1) / parts;
  const dim3 grid(unsigned(int64_t(a.ndir) * a.batch * kDState * ngroups)), block(kLanes * parts);
  if (run <= 16) {
    hipLaunchKernelGGL((scan_carry_kernel<16>), grid, block, 0, stream, a, nseg, agg, hin, flip);
  } else {
    hipLaunchKernelGGL((scan_carry_kernel<32>), grid, block, 0, stream, a, nseg, agg, hin, flip);
  }
}

}  // namespace
}  // namespace sscan
