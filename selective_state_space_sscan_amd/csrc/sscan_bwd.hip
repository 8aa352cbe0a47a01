// sscan_bwd.hip -- gfx950 kernels of the selective scan's backward pass.
//
// Gradients of sum(dout * out) for out = (sum over directions of the scan + D u) *
// silu(z), with respect to u, z and each direction's delta, delta_bias, A, B, C, D.
// Training differentiates the scan by hand and recomputes the forward states
// rather than storing them (Reproducing Vision Mamba page, section 1.3; Hand-written
// simplified Mamba2 page, section 5.1).  Reverse-mode differentiation of
//   h_t = a_t h_{t-1} + dt_t B_t u_t,  a_t = exp(dt_t A),  y_t = C_t h_t + D u_t
// gives, with the adjoint lambda_t = dLoss/dh_t travelling against the scan,
//   lambda_t = C_t dy_t + mu_t,  mu_{t-1} = a_t lambda_t,  dy_t = dout_t silu(z_t),
// dC_t += dy_t h_t, dB_t += lambda_t dt_t u_t, du_t += D dy_t + sum_n lambda dt B,
// d(dt_t) = sum_n lambda (B u_t + A a_t h_{t-1}), dA += lambda dt a_t h_{t-1},
// ddelta = d(dt) softplus'(delta + bias), dz = dout y silu'(z).
//
// Work is cut into 32-token windows.  The state entering every window and the
// adjoint entering it from the other side are two chains across the windows, each
// found in two steps: one pass walks runs of consecutive windows in chain order
// from zero (the scan order for the state, the opposite order for the adjoint),
// storing after every window what it has so far and the summed step sizes; the
// forward pass's carry kernel then chains the runs' totals.  A window's entry value
// is the stored value of the window before it plus the run's entry value decayed
// by exp(A * summed step sizes) -- the composition of two affine steps.  The window pass then
// needs, for every token, the state before it while the adjoint walks backwards:
// one lane per (channel, state) -- four channels x 16 states per wavefront -- keeps
// the window's 32 states of its (channel, state) in registers, recomputed forward
// from the window's entry state, and walks back through them.  Sums over the 16
// states of a channel use DPP within a 16-lane row.  A wavefront holds one
// (batch, window) and loops over its share of the channel groups (a window's groups
// are split over a few blocks), so the sums over channels that dB and dC need stay
// in registers (a sum per token and state, no atomics) and the few splits' partials
// are added afterwards; sums over tokens and batch rows (dA, dD, delta_bias) go
// through per-window partials.  Every reduction runs in a fixed order, so results
// are bitwise reproducible.
#include "sscan_device.h"

#include <type_traits>

namespace sscan {
namespace {

constexpr int kWin = 32;           // tokens per backward window
constexpr int kGroup = 4;          // channels per wavefront in the window pass
// LDS floats per token of the window pass's per-token tables.  In steps 1 and 4 a
// lane handles two tokens of one channel, so with 4 floats per token the 16 lanes of
// a channel hit addresses 8 floats apart: four banks, four-way conflicts.  With 5,
// each 32-lane half of a wave reaches 32 different banks.  Window pass on the long
// sequence 7.13 -> 6.95 ms, Mamba-YOLO rows 1.12 -> 1.09 ms.
constexpr int kTokPad = kGroup + 1;
constexpr int kPartRows = kDState + 2;  // per-window partials: dA[16], dD, delta_bias
#ifndef SSCAN_BWD_SCHED_TOKENS
#define SSCAN_BWD_SCHED_TOKENS 4
#endif
// The window sweeps let the scheduler interleave this many consecutive tokens: one
// token at a time leaves the single state chain of a lane exposed, unbounded
// interleaving hoists so much that registers spill.
constexpr int kSchedTokens = SSCAN_BWD_SCHED_TOKENS;

// per-token, per-channel values shared through LDS in the window pass
enum TokQ : int { QDT, QDTU, QDY, QU, QSIG, QDZ, QDUSKIP, QYSKIP, kTokQ };
enum OutQ : int { OP, OQ, OY, kOutQ };  // sum_n lambda B, sum_n A w, y

// Output handling of the window pass.
enum BwdOut : int {
  kSingle = 0,  // one direction: du, dz final
  kFirst = 1,   // first of two directions: du and y kept in fp32 scratch
  kSecond = 2,  // second of two: adds the first direction's du and y, writes du, dz
};

__device__ __forceinline__ float sigmoid_f32(float x) { return rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// Sum over the 16 lanes of a DPP row (quad xor 1, quad xor 2, row rotate 4, 8);
// every lane of the row receives the sum.
// Every source lane of these patterns is inside the row, so bound_ctrl never takes
// effect; with it (and a zero old value) the move folds into the add as one DPP add.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x128>(v);  // row_ror:8
  return v;
}

// Sums over the 16 states of a channel for a chunk of four tokens v[0..3] (slot =
// token % 4), reduce-scattered over the row: lane n of the row receives the sum
// for slot (n >> 2) & 3.  Round one pairs lanes n and n^8 (row_ror:8): the lower
// half keeps slots 0, 1 (the sums with the lanes 8 apart), the upper half slots 2,
// 3; round two pairs n and n^7 (row_half_mirror), which keeps bit 3 and flips bit
// 2: lanes with bit 2 clear keep the first of their two slots, the others the
// second; the last two rounds add over the quad (quad_perm xor 1, xor 2), the
// lanes n..n^3 whose partial sums together cover the whole row.  Where lanes keep
// different slots, two DPP adds with complementary bank masks (bank = four lanes
// of a row) write one register, each for its own lanes, so no lane has to select
// what it sends or keeps: 8 VALU operations for four tokens, where four all-lane
// sums take 16 (and selecting operands, 11).  The DPP reads of registers written
// by the VALU just before take two wait states (s_nop 1), which the compiler does
// not insert for an asm block.
// a = (a of the lane 8 apart) + a on banks LO (lanes of the row's lower or mirror
// half as the control says), b's sum on the other banks: two DPP adds, each writing
// its own lanes of one register.  The first reads only lanes the second writes, and
// the second does not read a, so a can be updated in place.
#define SSCAN_DPP_PAIR(CTRL, LO, HI)                                                  \
  "s_nop 1\n\t"                                                                     \
  "v_add_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:" LO "\n\t"             \
  "v_add_f32_dpp %0, %1, %1 " CTRL " row_mask:0xf bank_mask:" HI
__device__ __forceinline__ float row_scatter4(const float (&v)[kGroup], bool, bool) {
  float k0 = v[0], k1 = v[1];
  asm(SSCAN_DPP_PAIR("row_ror:8", "0x3", "0xc") : "+v"(k0) : "v"(v[2]));
  asm(SSCAN_DPP_PAIR("row_ror:8", "0x3", "0xc") : "+v"(k1) : "v"(v[3]));
  asm(SSCAN_DPP_PAIR("row_half_mirror", "0x5", "0xa") : "+v"(k0) : "v"(k1));
  k0 += dpp_mov<0xB1>(k0);
  k0 += dpp_mov<0x4E>(k0);
  return k0;
}
#undef SSCAN_DPP_PAIR

// row_scatter4 of two chunks at once (the reverse sweep's P and Q terms), their
// rounds interleaved so that each DPP add reads registers written at least two
// instructions earlier (the wait states the hardware needs) with four s_nop wait
// states in all instead of about twenty.
__device__ __forceinline__ void row_scatter4x2(const float (&v)[kGroup], const float (&w)[kGroup], float& rv,
                                               float& rw) {
  float a0 = v[0], a1 = v[1], b0 = w[0], b1 = w[1];
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %2, %2 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %3, %3 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_add_f32_dpp %2, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_add_f32_dpp %2, %2, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1)
      : "v"(v[2]), "v"(v[3]), "v"(w[2]), "v"(w[3]));
  rv = a0;
  rw = b0;
}

// x + (x of the lane 32 apart) on lanes 0..31, y + (y of the lane 32 apart) on lanes
// 32..63: v_permlane32_swap exchanges x's upper half with y's lower half.
__device__ __forceinline__ float swap_add32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same between rows 2r and 2r + 1 (v_permlane16_swap): x's sum on even rows,
// y's on odd rows.
__device__ __forceinline__ float swap_add16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the four channel rows of a wavefront (lanes l, l+16, l+32, l+48 hold
// the same state) of a chunk of four tokens' values v[0..3], reduce-scattered: row
// c receives the sum for slot c.  Round one pairs rows c and c^2: rows 0, 1 keep
// slots 0, 1 and rows 2, 3 slots 2, 3; round two pairs rows c and c^1: even rows
// keep the first of their two slots, odd rows the second.
__device__ __forceinline__ float chunk_sum(const float (&v)[kGroup]) {
  return swap_add16(swap_add32(v[0], v[2]), swap_add32(v[1], v[3]));
}

__device__ __forceinline__ size_t part_index(int dir, int64_t b, int64_t k, int r, int64_t d, int64_t batch,
                                             int64_t dim, int64_t nwin) {
  return ((((size_t)dir * batch + b) * nwin + k) * kPartRows + r) * dim + d;
}

__device__ __forceinline__ size_t pbc_index(int j, int dir, int64_t b, int which, int n, int64_t t, int ndir,
                                            int64_t batch, int64_t len) {
  return (((((size_t)j * ndir + dir) * batch + b) * 2 + which) * kDState + n) * len + t;
}

// One chain across the windows, over a run of consecutive windows: walking the run
// in chain order from zero -- the scan order for the state (kAggregate), the
// opposite order for the adjoint (kAdjoint: mu, with a.u holding dout) -- the lane
// stores after every window its 16 values so far and the summed step sizes, and at
// the end the run's totals in the segment-aggregate layout the carry kernel reads.
// Grid: batch * nrun * ngroups one-wave blocks (64 channels each); blockIdx.y is the
// direction.
// CONV (state chain only): u is recomputed from x (a.u) by the front-end convolution,
// as in the fused forward.
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z, bool ADJ, int CONV = kNoConv>
__global__ __launch_bounds__(kLanes) SSCAN_OCCUPANCY void bwd_chain_kernel(
    ScanArgs a, int64_t nwin, int64_t run_len, int64_t nrun, const float* __restrict__ bc, float* __restrict__ pw,
    float* __restrict__ sw, float* __restrict__ ragg, int vec) {
  static_assert(!ADJ || CONV == kNoConv, "the adjoint chain reads dout, not x");
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const SegIndex s = decode_block(blockIdx.x, ngroups, nrun);
  const int dir = blockIdx.y;
  const bool chain_rev = (a.ndir == 2 ? dir : a.reverse) != ADJ;  // windows visited high to low
  constexpr int kMode = ADJ ? kAdjoint : kAggregate;
  Lane<IO_BF16, SOFTPLUS, ADJ && HAS_Z, CONV> L;
  init_lane(L, a, dir, s.b, s.g, bc, vec != 0);
  const int64_t k_lo = s.seg * run_len, k_hi = min64(nwin, k_lo + run_len);
  const int64_t d = s.g * kLanes + threadIdx.x;
  for (int64_t i = k_lo; i < k_hi; ++i) {
    const int64_t k = chain_rev ? k_lo + k_hi - 1 - i : i;
    const int64_t t0 = k * kWin, t1 = min64(a.len, t0 + kWin);
    if (chain_rev) {
      L.template scan<true, kMode>(t0, t1);
    } else {
      L.template scan<false, kMode>(t0, t1);
    }
    if (L.active) {
      store_state16(pw + chain_state_index(dir, s.b, k, d, a.batch, a.dim, nwin), L.h);
      sw[chain_sum_index(dir, s.b, k, d, a.batch, a.dim, nwin)] = L.sum_dt;
    }
  }
  if (!L.active) return;
#pragma unroll
  for (int n = 0; n < kDState; ++n) ragg[agg_index(dir, s.b, s.seg, n, d, a.batch, a.dim, nrun)] = L.h[n];
  ragg[agg_index(dir, s.b, s.seg, kDState, d, a.batch, a.dim, nrun)] = L.sum_dt;
}

// What the window pass reads of the two chains (0: state, 1: adjoint).
struct WinChains {
  const float* p[2];
  const float* s[2];
  const float* e[2];
  int64_t run_len, nrun;
};

// One channel group's per-token inputs for one lane: two consecutive tokens of one
// channel (lane >> 4) in the window.
template <bool IO_BF16, bool HAS_Z>
struct TokIn {
  float u[2], draw[2], z[2], g[2];
  float bias, D;
};

// What a window-pass instance compiles in beyond the plain backward (bit mask).
constexpr int kExtIO = 1;     // u read in fp32 (the convolution's output), du / dz stored in fp32
constexpr int kExtState = 2;  // the entry state, the final state's gradient, dh0

template <bool IO_BF16, bool HAS_Z, int EXT>
__device__ __forceinline__ void load_tok(TokIn<IO_BF16, HAS_Z>& r, const BwdArgs& a, const DirArgs& pd, int64_t b,
                                         int64_t g, int64_t t0, int wl) {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  const int cc = threadIdx.x >> 4, i0 = (threadIdx.x & 15) * 2;
  const int64_t d = min64(g * kGroup + cc, a.fwd.dim - 1);
  const int64_t row = (b * a.fwd.dim + d) * a.fwd.len + t0;
  r.bias = pd.delta_bias ? pd.delta_bias[d] : 0.0f;
  r.D = pd.D ? pd.D[d] : 0.0f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = i0 + e < wl ? i0 + e : wl - 1;  // a valid token for the ragged tail
    r.u[e] = ((EXT & kExtIO) && a.u32) ? a.u32[row + i] : IO::load(static_cast<const T*>(a.fwd.u), row + i);
    r.draw[e] = IO::load(static_cast<const T*>(pd.delta), row + i);
    r.g[e] = IO::load(static_cast<const T*>(a.dout), row + i);
    r.z[e] = HAS_Z ? IO::load(static_cast<const T*>(a.fwd.z), row + i) : 0.0f;
  }
}

// The window pass for one direction.  Grid: batch * nwin * csplit one-wave blocks;
// block j of a window covers channel groups [j*gps, (j+1)*gps).  EXT selects the
// extensions compiled in (kExtIO, kExtState): the plain backward keeps a kernel
// without them (their live values had spilled registers in the sweeps: window pass
// 7.09 -> 8.61 ms on the long workload), and each extension is an instance of its own.
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z, bool REV, int OUT, int EXT>
__global__ __launch_bounds__(kLanes) void bwd_window_kernel(BwdArgs a, int dir, int64_t nwin, int csplit, int64_t gps,
                                                           const float* __restrict__ bc, WinChains ch,
                                                           float* __restrict__ part, float* __restrict__ pbc,
                                                           float* __restrict__ acc_du, float* __restrict__ acc_y) {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  __shared__ float sBC[kWin][kBC];
  __shared__ float sTok[kTokQ][kWin][kTokPad];
  __shared__ float sOutF[kOutQ * kWin * kTokPad];  // [q][i][c]
  auto sOut = [&](int q, int i, int cc) -> float { return sOutF[(q * kWin + i) * kTokPad + cc]; };
  const ScanArgs& f = a.fwd;
  const int lane = threadIdx.x;
  const int c = lane >> 4, n = lane & 15;
  // A window's row of each per-token tensor is half a 128-byte line; the other half
  // is the next window's, which the same XCD then takes up soon after.
  int64_t blk = xcd_stretch(blockIdx.x, gridDim.x);
  const int j = int(blk % csplit);
  blk /= csplit;
  const int64_t k = blk % nwin;
  const int64_t b = blk / nwin;
  const int64_t t0 = k * kWin;
  const int wl = int(min64(kWin, f.len - t0));
  const DirArgs pd = dir ? f.dir[1] : f.dir[0];
  const DirGrads gd = dir ? a.grads[1] : a.grads[0];
  const int64_t ngroups = (f.dim + kGroup - 1) / kGroup;
  const int64_t g_begin = j * gps, g_end = min64(ngroups, g_begin + gps);

  const float* bcw = bc + (((size_t)dir * f.batch + b) * f.len + t0) * kBC;
  for (int e = lane; e < wl * kBC; e += kLanes) sBC[e / kBC][e % kBC] = bcw[e];

  // dB and dC of this window over the block's channels.  Every 4 tokens the four
  // channel rows' per-token terms are summed by a reduce-scatter (two shuffle
  // rounds) that leaves row c owning token 4j + c: 8 accumulators per quantity
  // per lane instead of 32.
  constexpr int kChunks = kWin / kGroup;
  float accB[kChunks], accC[kChunks];
#pragma unroll
  for (int q = 0; q < kChunks; ++q) accB[q] = accC[q] = 0.0f;

  // Each chain's entry into this window: the run's entry value alone when the window
  // opens its run in that chain's order, else also the window before it (pred).
  int64_t run = 0, pred[2] = {0, 0};
  bool has_pred[2] = {false, false};
  if (nwin > 1) {
    run = k / ch.run_len;
    const int64_t lo = run * ch.run_len, hi = min64(nwin, lo + ch.run_len) - 1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bool down = (q == 0) == REV;  // the chain visits windows high to low
      has_pred[q] = down ? k < hi : k > lo;
      pred[q] = down ? k + 1 : k - 1;
    }
  }

  // software pipeline: the next group's inputs are in flight while this one runs
  TokIn<IO_BF16, HAS_Z> nx;
  float nx_A = 0.0f, nx_e[2] = {0.0f, 0.0f}, nx_p[2] = {0.0f, 0.0f}, nx_s[2] = {0.0f, 0.0f};
  auto prefetch = [&](int64_t g) {
    load_tok<IO_BF16, HAS_Z, EXT>(nx, a, pd, b, g, t0, wl);
    const int64_t d = min64(g * kGroup + c, f.dim - 1);
    nx_A = pd.A[d * kDState + n];
    if (nwin > 1) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        nx_e[q] = ch.e[q][hin_index(dir, b, run, n, d, f.batch, f.dim, ch.nrun)];
        if (has_pred[q]) {
          nx_p[q] = ch.p[q][chain_state_index(dir, b, pred[q], d, f.batch, f.dim, nwin) + n];
          nx_s[q] = ch.s[q][chain_sum_index(dir, b, pred[q], d, f.batch, f.dim, nwin)];
        }
      }
    } else if constexpr ((EXT & kExtState) != 0) {
      // one window: the forward's entry state, and the gradient reaching its final state
      nx_e[0] = f.h0 ? f.h0[(b * f.dim + d) * kDState + n] : 0.0f;
      nx_e[1] = a.dh_last ? a.dh_last[(b * f.dim + d) * kDState + n] : 0.0f;
    }
  };
  // the window holding the first token in scan order ends its adjoint sweep with the
  // gradient of the forward's entry state
  const bool writes_dh0 = (EXT & kExtState) && a.dh0 != nullptr && k == (REV ? nwin - 1 : 0);
  if (g_begin < g_end) prefetch(g_begin);

  for (int64_t g = g_begin; g < g_end; ++g) {
    const TokIn<IO_BF16, HAS_Z> cur = nx;
    const float A = nx_A;
    const float A2 = A * kLog2e;
    // entry state and adjoint: p + exp(A s) e (e alone where p, s are zero)
    const float h_in = fmaf(exp2_hw(A2 * nx_s[0]), nx_e[0], nx_p[0]);
    const float mu_in = fmaf(exp2_hw(A2 * nx_s[1]), nx_e[1], nx_p[1]);
    __syncthreads();  // the previous group is done with the LDS buffers (and sBC is written)
    if (g + 1 < g_end) prefetch(g + 1);

    // 1. per-token values of the four channels (two tokens per lane)
    float dD_row;
    {
      const int cc = lane >> 4, i0 = (lane & 15) * 2;
      const bool act = g * kGroup + cc < f.dim;
      float dDp = 0.0f;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = i0 + e;
        const float uu = act ? cur.u[e] : 0.0f;
        const float x = cur.draw[e] + cur.bias;
        const float dt = SOFTPLUS ? softplus_f32(x) : x;
        const float sig = SOFTPLUS ? sigmoid_f32(x) : 1.0f;
        float dy = cur.g[e], qz = 0.0f;
        if (HAS_Z) {
          const float zv = cur.z[e];
          const float sz = sigmoid_f32(zv);
          dy = cur.g[e] * (zv * sz);
          qz = cur.g[e] * (sz * fmaf(zv, 1.0f - sz, 1.0f));
        }
        if (!act) dy = 0.0f;
        if (i < wl) {
          sTok[QDT][i][cc] = dt;
          sTok[QDTU][i][cc] = dt * uu;
          sTok[QDY][i][cc] = dy;
          sTok[QU][i][cc] = uu;
          sTok[QSIG][i][cc] = sig;
          sTok[QDZ][i][cc] = qz;
          sTok[QDUSKIP][i][cc] = cur.D * dy;
          sTok[QYSKIP][i][cc] = cur.D * uu;
          dDp = fmaf(dy, uu, dDp);
        }
      }
      dD_row = row_sum16(dDp);
    }
    __syncthreads();

    // 2-3. forward sweep over the window from its entry state, keeping every state,
    // then the reverse sweep: the adjoint and the gradient terms of every token.
    // Full windows take a copy without per-token conditions, so the unrolled tokens
    // form one block the scheduler can interleave (each lane carries one state, one
    // dependency chain).  The per-token sums over states (y, P, Q) and over the
    // channel rows (dB, dC) are taken a chunk of four tokens at a time,
    // reduce-scattered over the lanes; the state sums go to LDS for step 4.
    const bool hi8 = (n & 8) != 0, hi4 = (n & 4) != 0;
    const int slot_off = ((n >> 2) & 3) * kTokPad + c;
    float hist[kWin];
    float dA_acc = 0.0f;
    float mu_end = 0.0f;  // the adjoint past the window's first token in scan order
    auto sweeps = [&](auto full_tag) {
      constexpr bool kFull = decltype(full_tag)::value;
      // A chunk's row sums leave lane n holding token 4 * chunk + ((n >> 2) & 3) (the
      // four lanes of a quad store the same value to the same word).
      auto out_slot = [&](int q, int i) { return (q * kWin + (i & ~(kGroup - 1))) * kTokPad + slot_off; };
      // a chunk of four tokens is complete at its last token in sweep order
      constexpr int kFwdLast = REV ? 0 : kGroup - 1, kRevLast = REV ? kGroup - 1 : 0;
      float h = h_in;
      float tY[kGroup];  // this chunk's per-token terms of y, slot i % 4
#pragma unroll
      for (int s = 0; s < kWin; ++s) {
        const int i = REV ? kWin - 1 - s : s;
        tY[i % kGroup] = 0.0f;
        if (kFull || i < wl) {
          h = fmaf(exp2_hw(sTok[QDT][i][c] * A2), h, sTok[QDTU][i][c] * sBC[i][n]);
          hist[i] = h;
          tY[i % kGroup] = sBC[i][kDState + n] * h;
        }
        if (HAS_Z && i % kGroup == kFwdLast) sOutF[out_slot(OY, i)] = row_scatter4(tY, hi8, hi4);
        if (s % kSchedTokens == kSchedTokens - 1) __builtin_amdgcn_sched_barrier(0);
      }
      float mu = mu_in;
      // this chunk's per-token dB, dC, P and Q terms, slot i % 4
      float tB[kGroup], tC[kGroup], tP[kGroup], tQ[kGroup];
#pragma unroll
      for (int s = kWin - 1; s >= 0; --s) {
        const int i = REV ? kWin - 1 - s : s;
        tB[i % kGroup] = tC[i % kGroup] = tP[i % kGroup] = tQ[i % kGroup] = 0.0f;
        if (kFull || i < wl) {
          const float dt = sTok[QDT][i][c];
          const float dy = sTok[QDY][i][c];
          const float lam = fmaf(sBC[i][kDState + n], dy, mu);
          const float at = exp2_hw(dt * A2);
          // the state before token i in scan order (the entry state for the first)
          float hprev;
          if (!REV) {
            hprev = i == 0 ? h_in : hist[i > 0 ? i - 1 : 0];
          } else if (kFull) {
            hprev = i == kWin - 1 ? h_in : hist[i + 1 < kWin ? i + 1 : kWin - 1];
          } else {
            hprev = i == wl - 1 ? h_in : hist[i + 1 < kWin ? i + 1 : kWin - 1];
          }
          const float w = lam * at * hprev;
          dA_acc = fmaf(w, dt, dA_acc);
          tB[i % kGroup] = lam * sTok[QDTU][i][c];
          tC[i % kGroup] = dy * hist[i];
          // du = dt * P + D dy and d(dt) = u * P + Q with P = sum_n lambda B, Q = sum_n A w
          tP[i % kGroup] = lam * sBC[i][n];
          tQ[i % kGroup] = A * w;
          mu = at * lam;
        }
        if (i % kGroup == kRevLast) {
          float sP, sQ;
          row_scatter4x2(tP, tQ, sP, sQ);
          sOutF[out_slot(OP, i)] = sP;
          sOutF[out_slot(OQ, i)] = sQ;
          accB[i / kGroup] += chunk_sum(tB);
          accC[i / kGroup] += chunk_sum(tC);
        }
        if (s % kSchedTokens == 0) __builtin_amdgcn_sched_barrier(0);
      }
      mu_end = mu;
    };
    if (wl == kWin) {
      sweeps(std::integral_constant<bool, true>());
    } else {
      sweeps(std::integral_constant<bool, false>());
    }
    {
      const int64_t d = g * kGroup + c;
      if (d < f.dim) {
        part[part_index(dir, b, k, n, d, f.batch, f.dim, nwin)] = dA_acc;
        if constexpr ((EXT & kExtState) != 0) {
          if (writes_dh0) a.dh0[(b * f.dim + d) * kDState + n] = mu_end;
        }
      }
    }
    __syncthreads();

    // 4. per-token outputs (same two tokens per lane as step 1)
    {
      const int cc = lane >> 4, i0 = (lane & 15) * 2;
      const int64_t d = g * kGroup + cc;
      const bool act = d < f.dim;
      const int64_t row = (b * f.dim + (act ? d : 0)) * f.len + t0;
      float dbp = 0.0f;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = i0 + e;
        if (i < wl) {
          const float P = sOut(OP, i, cc);
          const float du = fmaf(sTok[QDT][i][cc], P, sTok[QDUSKIP][i][cc]);
          const float ddl = fmaf(sTok[QU][i][cc], P, sOut(OQ, i, cc)) * sTok[QSIG][i][cc];
          const float y = HAS_Z ? sOut(OY, i, cc) + sTok[QYSKIP][i][cc] : 0.0f;  // y before the gate
          dbp += ddl;
          if (act) {
            IO::store(static_cast<T*>(gd.ddelta), row + i, ddl);
            if (OUT == kSingle) {
              if ((EXT & kExtIO) && a.du_f32) {
                static_cast<float*>(a.du)[row + i] = du;
              } else {
                IO::store(static_cast<T*>(a.du), row + i, du);
              }
              if (HAS_Z) {
                if ((EXT & kExtIO) && a.dz_f32) {
                  static_cast<float*>(a.dz)[row + i] = sTok[QDZ][i][cc] * y;
                } else {
                  IO::store(static_cast<T*>(a.dz), row + i, sTok[QDZ][i][cc] * y);
                }
              }
            } else if (OUT == kFirst) {
              acc_du[row + i] = du;
              if (HAS_Z) acc_y[row + i] = y;
            } else {
              if ((EXT & kExtIO) && a.du_f32) {
                static_cast<float*>(a.du)[row + i] = du + acc_du[row + i];
              } else {
                IO::store(static_cast<T*>(a.du), row + i, du + acc_du[row + i]);
              }
              if (HAS_Z) {
                if ((EXT & kExtIO) && a.dz_f32) {
                  static_cast<float*>(a.dz)[row + i] = sTok[QDZ][i][cc] * (y + acc_y[row + i]);
                } else {
                  IO::store(static_cast<T*>(a.dz), row + i, sTok[QDZ][i][cc] * (y + acc_y[row + i]));
                }
              }
            }
          }
        }
      }
      dbp = row_sum16(dbp);
      if ((lane & 15) == 0 && act) {
        part[part_index(dir, b, k, kDState, d, f.batch, f.dim, nwin)] = dD_row;
        part[part_index(dir, b, k, kDState + 1, d, f.batch, f.dim, nwin)] = dbp;
      }
    }
  }

  // row c holds dB / dC of tokens 4q + c of the window
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    const int i = q * kGroup + c;
    if (i < wl) {
      pbc[pbc_index(j, dir, b, 0, n, t0 + i, f.ndir, f.batch, f.len)] = accB[q];
      pbc[pbc_index(j, dir, b, 1, n, t0 + i, f.ndir, f.batch, f.len)] = accC[q];
    }
  }
}

// dA, dD and delta_bias: the per-window partials summed over windows and batch
// rows.  A block covers 64 channels of one (direction, row of the partials) with
// kReduceWaves waves, the q-th summing every kReduceWaves-th (batch row, window)
// from q with several loads in flight; the waves' sums are added in a fixed order.  Accumulation is in double, so thousands
// of partials add no error of their own (the partials carry float32 rounding only).
#ifndef SSCAN_BWD_REDUCE_WAVES
#define SSCAN_BWD_REDUCE_WAVES 16
#endif
constexpr int kReduceWaves = SSCAN_BWD_REDUCE_WAVES;

__global__ __launch_bounds__(kLanes * kReduceWaves) void bwd_reduce_params_kernel(BwdArgs a, int64_t nwin,
                                                                                const float* __restrict__ part) {
  __shared__ double sh[kReduceWaves][kLanes];
  const ScanArgs& f = a.fwd;
  const int lane = threadIdx.x % kLanes;
  const int q = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kLanes);  // wave-uniform
  const int64_t d_raw = int64_t(blockIdx.x) * kLanes + lane;
  const int64_t d = min64(d_raw, f.dim - 1);
  const int r = int(blockIdx.y % kPartRows);
  const int dir = int(blockIdx.y / kPartRows);
  // the (batch row, window) pairs m of one direction are consecutive in the layout
  const int64_t m_total = f.batch * nwin;
  const float* base = part + ((size_t)dir * m_total * kPartRows + r) * f.dim + d;
  const size_t stride = size_t(kPartRows) * f.dim;
  constexpr int kUnroll = 8;
  double acc[kUnroll] = {};
  int64_t m = q;
  for (; m + (kUnroll - 1) * kReduceWaves < m_total; m += kUnroll * kReduceWaves) {
#pragma unroll
    for (int e = 0; e < kUnroll; ++e) acc[e] += base[(m + e * kReduceWaves) * stride];
  }
  for (; m < m_total; m += kReduceWaves) acc[0] += base[m * stride];
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < kUnroll; ++e) s += acc[e];
  sh[q][lane] = s;
  __syncthreads();
  if (q != 0 || d_raw >= f.dim) return;
  s = sh[0][lane];
#pragma unroll
  for (int w = 1; w < kReduceWaves; ++w) s += sh[w][lane];
  const DirGrads gd = dir ? a.grads[1] : a.grads[0];
  if (r < kDState) {
    gd.dA[d * kDState + r] = float(s);
  } else if (r == kDState) {
    if (gd.dD) gd.dD[d] = float(s);
  } else if (gd.ddelta_bias) {
    gd.ddelta_bias[d] = float(s);
  }
}

// dB and dC: the channel splits' partials summed in split order, stored in B/C's dtype.
// Grid: x over tokens (256 per block), y over the (direction, batch row, dB/dC,
// state) rows, striding above the grid limit; no thread divides.
template <bool BC_BF16>
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(BwdArgs a, int csplit, const float* __restrict__ pbc) {
  const ScanArgs& f = a.fwd;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= f.len) return;
  const int64_t rows = int64_t(f.ndir) * f.batch * 2 * kDState;
  for (int64_t rr = blockIdx.y; rr < rows; rr += gridDim.y) {
    const int n = int(rr & (kDState - 1));
    const int which = int((rr >> 4) & 1);
    const int64_t db = rr >> 5;  // dir * batch + b
    const int dir = db >= f.batch ? 1 : 0;
    const int64_t b = db - dir * f.batch;
    double s = 0.0;
    for (int j = 0; j < csplit; ++j) s += pbc[pbc_index(j, dir, b, which, n, t, f.ndir, f.batch, f.len)];
    const DirGrads gd = dir ? a.grads[1] : a.grads[0];
    void* out = which ? gd.dC : gd.dB;
    Io<BC_BF16>::store(static_cast<typename Io<BC_BF16>::T*>(out), (b * kDState + n) * f.len + t, float(s));
  }
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(void* p, int64_t bytes) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < bytes) static_cast<unsigned char*>(p)[i] = 0;
}

bool aligned16_b(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z>
hipError_t launch_bwd_typed(const BwdArgs& a, const BwdPlan& p, float* w, hipStream_t stream, hipEvent_t const* ev) {
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  const ScanArgs& f = a.fwd;
  const int64_t ngroups = (f.dim + kLanes - 1) / kLanes;
  float* bc = w + p.off_bc;
  WinChains ch{};
  ch.run_len = p.run_len;
  ch.nrun = p.nrun;
  for (int q = 0; q < 2; ++q) {
    ch.p[q] = w + p.off_p[q];
    ch.s[q] = w + p.off_s[q];
    ch.e[q] = w + p.off_e[q];
  }
  float* part = w + p.off_part;
  float* pbc = w + p.off_pbc;
  float* acc_du = w + p.off_acc;
  float* acc_y = acc_du + (p.off_acc ? size_t(f.batch) * f.dim * f.len : 0);

  mark(0);
  launch_stage_bc(f, bc, stream);
  mark(1);
  if (p.nwin <= 1) {
    mark(2);
    mark(3);
  } else {
    const size_t esz = IO_BF16 ? 2 : 4;
    bool vec = (size_t(f.len) * esz) % 16 == 0 && aligned16_b(f.u) && aligned16_b(a.dout) &&
               (!f.z || aligned16_b(f.z));
    for (int k = 0; k < f.ndir; ++k) vec = vec && aligned16_b(f.dir[k].delta);
    const int64_t chain_blocks = f.batch * p.nrun * ngroups;
    const dim3 cgrid(unsigned(chain_blocks), unsigned(f.ndir));
    float* pw[2] = {w + p.off_p[0], w + p.off_p[1]};
    float* sw[2] = {w + p.off_s[0], w + p.off_s[1]};
    float* rw[2] = {w + p.off_r[0], w + p.off_r[1]};
    float* ew[2] = {w + p.off_e[0], w + p.off_e[1]};
    // the state entering every window
    if (!f.conv_w) {
      hipLaunchKernelGGL((bwd_chain_kernel<IO_BF16, SOFTPLUS, false, false>), cgrid, dim3(kLanes), 0, stream, f,
                         p.nwin, p.run_len, p.nrun, static_cast<const float*>(bc), pw[0], sw[0], rw[0], int(vec));
    } else if (f.conv_silu) {
      hipLaunchKernelGGL((bwd_chain_kernel<IO_BF16, SOFTPLUS, false, false, kConvSilu>), cgrid, dim3(kLanes), 0,
                         stream, f, p.nwin, p.run_len, p.nrun, static_cast<const float*>(bc), pw[0], sw[0], rw[0],
                         int(vec));
    } else {
      hipLaunchKernelGGL((bwd_chain_kernel<IO_BF16, SOFTPLUS, false, false, kConvLin>), cgrid, dim3(kLanes), 0,
                         stream, f, p.nwin, p.run_len, p.nrun, static_cast<const float*>(bc), pw[0], sw[0], rw[0],
                         int(vec));
    }
    launch_carry(f, p.nrun, rw[0], ew[0], 0, stream);
    mark(2);
    // the adjoint entering every window from the other side
    ScanArgs adj = f;
    adj.u = a.dout;
    hipLaunchKernelGGL((bwd_chain_kernel<IO_BF16, SOFTPLUS, HAS_Z, true>), cgrid, dim3(kLanes), 0, stream, adj,
                       p.nwin, p.run_len, p.nrun, static_cast<const float*>(bc), pw[1], sw[1], rw[1], int(vec));
    // the adjoint chain enters from beyond the last token with the final state's gradient
    ScanArgs adj_carry = f;
    adj_carry.h0 = a.dh_last;
    launch_carry(adj_carry, p.nrun, rw[1], ew[1], 1, stream);
    mark(3);
  }
  const dim3 wgrid(unsigned(f.batch * p.nwin * p.csplit));
  const int64_t nw = p.nwin;
  const int ext = ((a.u32 || a.du_f32 || a.dz_f32) ? kExtIO : 0) | ((f.h0 || a.dh_last || a.dh0) ? kExtState : 0);
  auto windows = [&](auto ext_tag) {
    constexpr int E = decltype(ext_tag)::value;
    if (f.ndir == 1) {
      if (f.reverse) {
        hipLaunchKernelGGL((bwd_window_kernel<IO_BF16, SOFTPLUS, HAS_Z, true, kSingle, E>), wgrid, dim3(kLanes), 0,
                           stream, a, 0, nw, p.csplit, p.gps, bc, ch, part, pbc, acc_du, acc_y);
      } else {
        hipLaunchKernelGGL((bwd_window_kernel<IO_BF16, SOFTPLUS, HAS_Z, false, kSingle, E>), wgrid, dim3(kLanes), 0,
                           stream, a, 0, nw, p.csplit, p.gps, bc, ch, part, pbc, acc_du, acc_y);
      }
    } else {
      hipLaunchKernelGGL((bwd_window_kernel<IO_BF16, SOFTPLUS, HAS_Z, false, kFirst, E>), wgrid, dim3(kLanes), 0,
                         stream, a, 0, nw, p.csplit, p.gps, bc, ch, part, pbc, acc_du, acc_y);
      hipLaunchKernelGGL((bwd_window_kernel<IO_BF16, SOFTPLUS, HAS_Z, true, kSecond, E>), wgrid, dim3(kLanes), 0,
                         stream, a, 1, nw, p.csplit, p.gps, bc, ch, part, pbc, acc_du, acc_y);
    }
  };
  // no entry point combines state I/O with the fp32 paths of the convolution or the
  // multi-order scan, so no instance has both
  if (ext == (kExtState | kExtIO)) return hipErrorInvalidValue;
  if (ext & kExtState) {
    windows(std::integral_constant<int, kExtState>());
  } else if (ext & kExtIO) {
    windows(std::integral_constant<int, kExtIO>());
  } else {
    windows(std::integral_constant<int, 0>());
  }
  mark(4);
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3(unsigned((f.dim + kLanes - 1) / kLanes), unsigned(f.ndir * kPartRows)),
                     dim3(kLanes * kReduceWaves), 0, stream, a, p.nwin, static_cast<const float*>(part));
  const int64_t bc_rows = int64_t(f.ndir) * f.batch * 2 * kDState;
  const dim3 bc_grid(unsigned((f.len + 255) / 256), unsigned(std::min<int64_t>(bc_rows, 65535)));
  if (f.bc_bf16) {
    hipLaunchKernelGGL(bwd_reduce_bc_kernel<true>, bc_grid, dim3(256), 0, stream, a, p.csplit,
                       static_cast<const float*>(pbc));
  } else {
    hipLaunchKernelGGL(bwd_reduce_bc_kernel<false>, bc_grid, dim3(256), 0, stream, a, p.csplit,
                       static_cast<const float*>(pbc));
  }
  mark(5);
  return hipGetLastError();
}

template <bool IO_BF16>
hipError_t launch_bwd_io(const BwdArgs& a, const BwdPlan& p, float* w, hipStream_t stream, hipEvent_t const* ev) {
  const bool z = a.fwd.z != nullptr;
  if (a.fwd.softplus) {
    return z ? launch_bwd_typed<IO_BF16, true, true>(a, p, w, stream, ev)
             : launch_bwd_typed<IO_BF16, true, false>(a, p, w, stream, ev);
  }
  return z ? launch_bwd_typed<IO_BF16, false, true>(a, p, w, stream, ev)
           : launch_bwd_typed<IO_BF16, false, false>(a, p, w, stream, ev);
}

}  // namespace

// Window pass: the channel groups of a window are split over several one-wave
// blocks, aiming for about kBwdBlockTarget blocks per launch (32 per SIMD) with at
// least kMinGroupsPerBlock groups each.  Measured splits (window pass, ms):
// long sequence (8192 windows, 384 groups) 1: 7.61, 2: 7.33, 3: 7.44, 4: 7.11,
// 8: 7.24, 16: 7.48; Mamba-YOLO map rows (8 x 512 windows per direction, 48 groups)
// 1: 1.18, 2: 1.09, 3: 1.06, 4: 1.08, 8: 1.14; Vim-small (128 x 7 windows per
// direction, 192 groups) 3: 1.00, 8: 0.96, 16: 0.93.  The minimum of groups per
// block, 8 / 12 / 16 / 32 / 48: Vim-small 1.01 / 0.98 / 0.98 / 1.02 / 1.18, Vim-tiny
// 0.28 / 0.31 / 0.27 / 0.38 / 0.49, Mamba-YOLO rows 1.17 / 1.14 / 1.12 / - / -.
constexpr int64_t kBwdBlockTarget = 32768;
constexpr int64_t kMinGroupsPerBlock = 16;
// Chain passes: blocks per pass the run length aims for (about eight waves per
// SIMD), and the longest run.  A short sequence (at most kShortMax tokens) is
// walked whole (no carry between runs) when one wave per (direction, batch row, 64
// channels) still fills kWholeRunWaves slots (three waves per SIMD).  Measured
// chain passes, states + adjoints (ms): Vim-small (7 windows, 3,072 such waves)
// runs of 2 windows 0.21 + 0.23, the whole sequence 0.17 + 0.20; on the long
// sequence, 3,072 waves of 64-window runs were 13% slower than 8,192 of 24.
constexpr int64_t kChainWaveTarget = 256 * 4 * 8;
constexpr int64_t kMaxRun = 64;
constexpr int64_t kWholeRunWaves = 256 * 4 * 3;

BwdPlan make_bwd_plan(int64_t batch, int64_t dim, int64_t len, int ndir) {
  BwdPlan p{};
  p.nwin = std::max<int64_t>(1, (len + kWin - 1) / kWin);
  const int64_t ngroups = std::max<int64_t>(1, (dim + kGroup - 1) / kGroup);
  const int64_t base = std::max<int64_t>(1, int64_t(ndir) * batch * p.nwin);
  const int64_t per_launch = std::max<int64_t>(1, batch * p.nwin);  // one direction per launch
  const int64_t split = std::max<int64_t>(1, std::min<int64_t>((kBwdBlockTarget + per_launch - 1) / per_launch,
                                                               ngroups / kMinGroupsPerBlock));
  p.gps = (ngroups + split - 1) / split;
  p.csplit = int((ngroups + p.gps - 1) / p.gps);
  auto up = [](size_t n) { return (n + 63) / 64 * 64; };
  size_t off = 0;
  p.off_bc = off;
  off += up(size_t(ndir) * batch * len * kBC);
  // chain runs: about kChainWaveTarget one-wave blocks per chain pass, runs of at
  // most kMaxRun windows
  const int64_t ngroups64 = std::max<int64_t>(1, (dim + 63) / 64);
  p.run_len = std::max<int64_t>(1, std::min<int64_t>(kMaxRun, base * ngroups64 / kChainWaveTarget));
  if (len <= kShortMax && int64_t(ndir) * batch * ngroups64 >= kWholeRunWaves) p.run_len = p.nwin;
  p.nrun = (p.nwin + p.run_len - 1) / p.run_len;
  const bool chains = p.nwin > 1;
  for (int q = 0; q < 2; ++q) {
    p.off_p[q] = off;
    off += chains ? up(size_t(ndir) * batch * p.nwin * dim * kDState) : 0;
    p.off_s[q] = off;
    off += chains ? up(size_t(ndir) * batch * p.nwin * dim) : 0;
    p.off_r[q] = off;
    off += chains ? up(size_t(ndir) * batch * p.nrun * (kDState + 1) * dim) : 0;
    p.off_e[q] = off;
    off += chains ? up(size_t(ndir) * batch * p.nrun * kDState * dim) : 0;
  }
  p.off_part = off;
  off += up(size_t(ndir) * batch * p.nwin * kPartRows * dim);
  p.off_pbc = off;
  off += up(size_t(p.csplit) * ndir * batch * 2 * kDState * len);
  p.off_acc = ndir == 2 ? off : 0;
  if (ndir == 2) off += up(2 * size_t(batch) * dim * len);
  p.workspace_bytes = off * sizeof(float);
  return p;
}

bool bwd_plan_fits_grid(const BwdPlan& p, int64_t batch, int64_t dim, int64_t len, int ndir) {
  constexpr int64_t kMax = (int64_t(1) << 32) - 1;
  auto fits = [](int64_t blocks, int64_t threads) { return blocks <= kMax / threads; };
  const int64_t ngroups64 = (dim + 63) / 64;
  bool ok = fits(int64_t(ndir) * batch * ((len + 63) / 64), 256);     // B/C staging
  ok = ok && fits(batch * p.nwin * p.csplit, kLanes);                 // window pass
  if (p.nwin > 1) {
    ok = ok && fits(batch * p.nrun * ngroups64, kLanes);              // chain passes (blockIdx.y: direction)
    ok = ok && fits(int64_t(ndir) * batch * kDState * ngroups64, int64_t(kLanes) * carry_parts(p.nrun));
  }
  ok = ok && fits((len + 255) / 256, 256);                            // dB/dC sums
  return ok;
}

hipError_t launch_bwd_zero(const BwdArgs& a, hipStream_t stream) {
  const ScanArgs& f = a.fwd;
  const int64_t bc_esz = f.bc_bf16 ? 2 : 4;
  for (int k = 0; k < f.ndir; ++k) {
    const DirGrads& g = a.grads[k];
    const struct {
      void* p;
      int64_t bytes;
    } bufs[] = {{g.dA, f.dim * kDState * 4},
                {g.dD, g.dD ? f.dim * 4 : 0},
                {g.ddelta_bias, g.ddelta_bias ? f.dim * 4 : 0},
                {g.dB, f.batch * kDState * f.len * bc_esz},
                {g.dC, f.batch * kDState * f.len * bc_esz}};
    for (const auto& bf : bufs)
      if (bf.p && bf.bytes > 0)
        hipLaunchKernelGGL(bwd_zero_kernel, dim3(unsigned((bf.bytes + 255) / 256)), dim3(256), 0, stream, bf.p,
                           bf.bytes);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, float* workspace, hipStream_t stream,
                      hipEvent_t const* events) {
  return a.fwd.io_bf16 ? launch_bwd_io<true>(a, p, workspace, stream, events)
                       : launch_bwd_io<false>(a, p, workspace, stream, events);
}

}  // namespace sscan
