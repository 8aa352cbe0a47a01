// sscan_short.hip -- the selective scan of short sequences with four lanes per
// channel (gfx950).  Same operation as the lane = channel kernels of
// sscan_kernels.hip (Hand-written simplified Mamba2 page, section 2.2 recurrence,
// sections 4.2 and 4.4 step size, skip and gate; Reproducing Vision Mamba page,
// section 3.2, the two directions added before the gate), for one-segment
// sequences that would give the lane = channel kernels too few waves.
#include "sscan_device.h"

namespace sscan {
namespace {

// Short sequences that fill few wave slots with lane = channel (a Vim sequence of
// 197 tokens over 64 x 384 channels gives 768 waves for 3072 slots, each a serial
// 197-token chain): four lanes per channel, each owning four of its states, so
// four times the waves.  A wave covers 16 channels; lane l is quarter q = l & 3 of
// channel l >> 2 of the wave, row position r = (l >> 2) & 3 within its 16-lane row.
//
// Per-token work that does not depend on the state (step size, softplus, dt * u,
// D skip, gate) is done once per channel, not once per lane: in an 8-token tile,
// quarter q owns tokens 2q and 2q + 1 (it loads their u, delta and z, computes
// their step sizes and finishes their outputs), and each token's dt and dt * u
// reach the other three lanes of the quad with a quad-broadcast DPP move.
//
// B_t and C_t are shared by all channels.  Lane (r, q) loads B_t[4q + r] and
// C_t[4q + r] of the token-major staged buffer (one dword each); rotating them
// across the row by 4m lanes (row_ror DPP, fused into the multiply and the readout
// FMA) hands lane (r, q) the values of state 4q + sigma(m), where sigma(m) is the
// row position of the lane it reads from.  Each lane keeps its four states in that
// order (slot m), with A gathered to match; sigma is found at set-up by passing the
// row position itself through the same rotation.  The four partial readouts are
// summed across the quad with DPP.
//
// Two directions: wave 0 scans forward, wave 1 in reverse, meeting in LDS as the
// lane = channel kernel does (the half met first is parked, ungated, with D u).
// Measured on the Vim-tiny call (64 x 384 x 197, two directions, f32, cold inputs),
// output pass: lane = channel 113 us; here 16-token tiles loaded at their start
// 97 us, 8-token tiles 97 us, either with a scheduling barrier per token 96-101 us
// (a wave-uniform bounds check on every token, not only in the ragged tile: 99-103
// us), z loaded with the tile instead of before each store 92.5-94 us.  16-token
// tiles loaded a tile ahead spill; 8-token ones do not (78-162 VGPRs).
constexpr int kQuadTile = 8;       // tokens per tile
constexpr int kOwn = kQuadTile / 4; // tokens of a tile each quarter owns
constexpr bool kQuadPrefetch = true;  // load each tile's data while the tile before it runs
constexpr int kQuadBarrier = 0;       // tokens between scheduling barriers (0: none)
constexpr int kQuadChannels = 16;  // channels per wave

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  // bound_ctrl set (zero-fill): the controls used here always read a valid lane, and
  // it lets the compiler fold the move into the consuming VALU op as its DPP source
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int quad_bcast(int k) { return k | (k << 2) | (k << 4) | (k << 6); }
constexpr int row_ror(int n) { return 0x120 + n; }  // rotate right within a 16-lane row, n = 1..15

// quad broadcast from lane k of each quad; k is a constant once the token loop is unrolled
__device__ __forceinline__ float quad_bcast_from(int k, float v) {
  switch (k) {
    case 0: return dpp<quad_bcast(0)>(v);
    case 1: return dpp<quad_bcast(1)>(v);
    case 2: return dpp<quad_bcast(2)>(v);
    default: return dpp<quad_bcast(3)>(v);
  }
}

template <int M>
__device__ __forceinline__ float rot(float v) {
  if constexpr (M == 0) {
    return v;
  } else {
    return dpp<row_ror(4 * M)>(v);
  }
}

template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z>
struct QuadLane {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  const T* u;
  const T* delta;
  const T* z;
  T* y;
  const float* bc;   // staged B/C of this (direction, batch row)
  float* part;       // LDS meeting buffer [16 channels][len] (two directions)
  float A2[4];       // A * log2(e) of the lane's states, in slot order
  float h[4];
  float bias, Dd;
  int64_t len;
  int q;             // quarter of the channel (lane & 3)
  int ch;            // channel within the wave
  int bcidx;         // the lane's B/C index within a token: 4q + r
  bool active;

  // What a tile needs from memory: the quarter's own tokens of u and delta, and
  // every token's B/C dword of the lane.  Tokens outside [ta, tb) read as zero (B/C
  // stay inside the staged rows).
  struct Tile {
    float u[kOwn], d[kOwn], z[kOwn];
    float bv[kQuadTile], cv[kQuadTile];
  };

  // z only where the tile's outputs are finished (not for parked halves)
  template <int MODE>
  __device__ __forceinline__ void load(Tile& T_, int64_t t0, int64_t ta, int64_t tb) const {
#pragma unroll
    for (int i = 0; i < kOwn; ++i) {
      const int64_t t = t0 + kOwn * q + i;
      const bool in = t >= ta && t < tb;
      T_.u[i] = in ? IO::load(u, t) : 0.0f;
      T_.d[i] = in ? IO::load(delta, t) : 0.0f;
      T_.z[i] = (HAS_Z && MODE != kPark && in) ? IO::load(z, t) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kQuadTile; ++j) {
      const int64_t t = t0 + j;
      const int64_t tc = t < len ? t : len - 1;
      T_.bv[j] = bc[tc * kBC + bcidx];
      T_.cv[j] = bc[tc * kBC + kDState + bcidx];
    }
  }

  // One tile [t0, t0 + kQuadTile) from its loaded data, in descending order when
  // REV.  MODE: kStore, kPark or kMeet.  PARTIAL: the tile holds the end of the
  // sequence and only its tokens inside [ta, tb) are scanned (a wave-uniform check
  // per token; full tiles have none, so their tokens form one block the scheduler
  // can overlap).
  template <bool REV, int MODE, bool PARTIAL>
  __device__ __forceinline__ void tile(const Tile& T_, int64_t t0, int64_t ta, int64_t tb) {
    float dt[kOwn], dtu[kOwn], yo[kOwn];
#pragma unroll
    for (int i = 0; i < kOwn; ++i) {
      const float x = T_.d[i] + bias;
      dt[i] = SOFTPLUS ? softplus_f32(x) : x;
      dtu[i] = dt[i] * T_.u[i];
      yo[i] = 0.0f;
    }
#pragma unroll
    for (int jj = 0; jj < kQuadTile; ++jj) {
      const int tt = REV ? kQuadTile - 1 - jj : jj;
      const int k = tt / kOwn, i = tt % kOwn;  // owning quarter and its slot
      if (PARTIAL && (t0 + tt < ta || t0 + tt >= tb)) continue;
      const float dtb = quad_bcast_from(k, dt[i]);
      const float dtub = quad_bcast_from(k, dtu[i]);
      float s = 0.0f;
      step_state<0>(dtb, dtub, T_.bv[tt], T_.cv[tt], s);
      step_state<1>(dtb, dtub, T_.bv[tt], T_.cv[tt], s);
      step_state<2>(dtb, dtub, T_.bv[tt], T_.cv[tt], s);
      step_state<3>(dtb, dtub, T_.bv[tt], T_.cv[tt], s);
      s = quad_sum(s);
      yo[i] = (q == k) ? s : yo[i];
      // keep groups of tokens together: hoisting later tokens' exponentials far ahead
      // only raises register pressure
      if (kQuadBarrier > 0 && (jj + 1) % (kQuadBarrier > 0 ? kQuadBarrier : 1) == 0)
        __builtin_amdgcn_sched_barrier(0);
    }
    // the quarter's own outputs
#pragma unroll
    for (int i = 0; i < kOwn; ++i) {
      const int64_t t = t0 + kOwn * q + i;
      if (PARTIAL && (t < ta || t >= tb)) continue;
      float v = fmaf(Dd, T_.u[i], yo[i]);
      if (MODE == kPark) {
        part[ch * len + t] = v;
      } else {
        if (MODE == kMeet) v += part[ch * len + t];
        if (HAS_Z) v *= silu_f32(T_.z[i]);
        if (active) IO::store(y, t, v);
      }
    }
  }

  template <int M>
  __device__ __forceinline__ void step_state(float dtb, float dtub, float bvt, float cvt, float& s) {
    const float a = exp2_hw(dtb * A2[M]);
    h[M] = fmaf(a, h[M], rot<M>(bvt) * dtub);
    s = fmaf(rot<M>(cvt), h[M], s);
  }

  // Tokens [ta, tb) in scan order; ta is a multiple of the tile, tb too unless it
  // is the end of the sequence.  Two tile buffers alternate: each tile's data is
  // loaded while the tile before it runs.
  template <bool REV, int MODE>
  __device__ void scan(int64_t ta, int64_t tb) {
    if (tb <= ta) return;
    const int64_t ntiles = (tb - ta + kQuadTile - 1) / kQuadTile;
    const int64_t tlast = ta + (ntiles - 1) * kQuadTile;  // the only tile that may be partial
    const bool ragged = tb - tlast < kQuadTile;
    const int64_t step = REV ? -kQuadTile : kQuadTile;
    int64_t t0 = REV ? tlast : ta;
    auto run = [&](const Tile& T_, int64_t t) {
      if (ragged && t == tlast) {
        tile<REV, MODE, true>(T_, t, ta, tb);
      } else {
        tile<REV, MODE, false>(T_, t, ta, tb);
      }
    };
    Tile ta_, tb_;
    if constexpr (!kQuadPrefetch) {
      for (int64_t n = 0; n < ntiles; ++n, t0 += step) {
        load<MODE>(ta_, t0, ta, tb);
        run(ta_, t0);
      }
      return;
    }
    load<MODE>(ta_, t0, ta, tb);
    for (int64_t n = 0; n < ntiles; n += 2) {
      if (n + 1 < ntiles) load<MODE>(tb_, t0 + step, ta, tb);
      run(ta_, t0);
      if (n + 1 >= ntiles) break;
      if (n + 2 < ntiles) load<MODE>(ta_, t0 + 2 * step, ta, tb);
      run(tb_, t0 + step);
      t0 += 2 * step;
    }
  }
};

// Grid: batch * ceil(dim / 16) blocks of NDIR waves; blockIdx.x = b * groups + g.
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z, int NDIR>
__global__ __launch_bounds__(kLanes * NDIR) SSCAN_OCCUPANCY void scan_short_quad_kernel(
    ScanArgs a, const float* __restrict__ bc) {
  extern __shared__ float part[];  // [16][len] (two directions)
  using T = typename Io<IO_BF16>::T;
  const int64_t groups = (a.dim + kQuadChannels - 1) / kQuadChannels;
  const int64_t b = blockIdx.x / groups, g = blockIdx.x % groups;
  const int dir = NDIR == 2 ? __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kLanes) : 0;
  const int lane = threadIdx.x % kLanes;
  QuadLane<IO_BF16, SOFTPLUS, HAS_Z> L;
  L.q = lane & 3;
  L.ch = lane >> 2;
  const int r = (lane >> 2) & 3;
  const int64_t d_raw = g * kQuadChannels + L.ch;
  L.active = d_raw < a.dim;
  const int64_t d = L.active ? d_raw : a.dim - 1;  // idle lanes shadow a valid channel and store nothing
  const DirArgs p = dir ? a.dir[1] : a.dir[0];
  const int64_t row = (b * a.dim + d) * a.len;
  L.u = static_cast<const T*>(a.u) + row;
  L.delta = static_cast<const T*>(p.delta) + row;
  L.z = a.z ? static_cast<const T*>(a.z) + row : nullptr;
  L.y = static_cast<T*>(a.y) + row;
  L.bc = bc + ((size_t)dir * a.batch + b) * a.len * kBC;
  L.part = part;
  L.len = a.len;
  L.bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
  L.Dd = p.D ? p.D[d] : 0.0f;
  L.bcidx = 4 * L.q + r;
  // slot m holds state 4q + (row position of the lane that row_ror:4m reads from)
  const float rf = float(r);
  const int src[4] = {r, int(rot<1>(rf)), int(rot<2>(rf)), int(rot<3>(rf))};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    L.A2[m] = p.A[d * kDState + 4 * L.q + src[m]] * kLog2e;
    L.h[m] = 0.0f;
  }
  const bool rev1 = NDIR == 1 && a.reverse;
  if (NDIR == 1) {
    if (rev1) {
      L.template scan<true, kStore>(0, a.len);
    } else {
      L.template scan<false, kStore>(0, a.len);
    }
    return;
  }
  const int64_t mid = (a.len / 2) / kQuadTile * kQuadTile;  // a tile boundary
  if (dir == 0) {
    L.template scan<false, kPark>(0, mid);
  } else {
    L.template scan<true, kPark>(mid, a.len);
  }
  __syncthreads();
  if (dir == 0) {
    L.template scan<false, kMeet>(mid, a.len);
  } else {
    L.template scan<true, kMeet>(0, mid);
  }
}

}  // namespace

hipError_t launch_short_quad(const ScanArgs& a, const float* bc, hipStream_t stream) {
  const int64_t blocks = a.batch * ((a.dim + kQuadChannels - 1) / kQuadChannels);
  const int key = (a.io_bf16 ? 4 : 0) | (a.softplus ? 2 : 0) | (a.z ? 1 : 0);
#define SSCAN_QUAD_LAUNCH(BF, SP, Z)                                                                            \
  if (a.ndir == 1) {                                                                                            \
    hipLaunchKernelGGL((scan_short_quad_kernel<BF, SP, Z, 1>), dim3(unsigned(blocks)), dim3(kLanes), 0, stream, \
                       a, bc);                                                                                  \
  } else {                                                                                                      \
    hipLaunchKernelGGL((scan_short_quad_kernel<BF, SP, Z, 2>), dim3(unsigned(blocks)), dim3(2 * kLanes),        \
                       size_t(kQuadChannels) * size_t(a.len) * sizeof(float), stream, a, bc);                  \
  }
  switch (key) {
    case 0: SSCAN_QUAD_LAUNCH(false, false, false) break;
    case 1: SSCAN_QUAD_LAUNCH(false, false, true) break;
    case 2: SSCAN_QUAD_LAUNCH(false, true, false) break;
    case 3: SSCAN_QUAD_LAUNCH(false, true, true) break;
    case 4: SSCAN_QUAD_LAUNCH(true, false, false) break;
    case 5: SSCAN_QUAD_LAUNCH(true, false, true) break;
    case 6: SSCAN_QUAD_LAUNCH(true, true, false) break;
    default: SSCAN_QUAD_LAUNCH(true, true, true) break;
  }
#undef SSCAN_QUAD_LAUNCH
  return hipGetLastError();
}

}  // namespace sscan
