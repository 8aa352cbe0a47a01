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
#include "sscan_device.h"

#include <algorithm>

namespace sscan {
namespace {

// Step 3, one direction: every wave scans one segment of 64 channels from its entry
// state and stores the gated output.
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z, int CONV, bool Y_F32 = false>
__global__ __launch_bounds__(kLanes) SSCAN_OUT_OCCUPANCY(IO_BF16 && CONV == kNoConv) void scan_output_dir_kernel(ScanArgs a, int64_t seg_len, int64_t nseg,
                                                                 const float* __restrict__ bc, SegChain ch,
                                                                 int vec) {
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const SegIndex s = decode_block(blockIdx.x, ngroups, nseg);
  Lane<IO_BF16, SOFTPLUS, HAS_Z, CONV, Y_F32> L;
  constexpr bool kLines = IO_BF16 && CONV == kNoConv;
  __shared__ uint4 lslot[kLines ? kLineSlot : 1];
  init_lane(L, a, 0, s.b, s.g, bc, (vec & 1) != 0);
  if (kLines) {
    L.line = (vec & 2) != 0;
    L.lbuf = (lds_uint4*)lslot;
  }
  load_entry(L, a, 0, s.b, s.seg, s.g, nseg, ch);
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


// Each thread handles kStepReps channel quads (kStepChannels apart), all their loads
// issued before any arithmetic: more bytes in flight per wave for a kernel that is
// one round trip to memory.  Measured on 256 x 1536 bf16, cold state (rotating
// buffers): loads interleaved with the arithmetic 15.0 us; loads first with one
// quad 13.8 us, two 13.7 us, four 15.9 us.
constexpr int kStepReps = 2;

constexpr int kStepConvMax = 4;  // taps of the causal convolution in front of the step

template <bool IO_BF16, bool BC_BF16, bool SOFTPLUS, bool CONV>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepArgs a, int64_t b0) {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  const int64_t b = b0 + blockIdx.y;
  const int q = threadIdx.x & 3;  // which four states
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
  float4 hv[kStepReps], av[kStepReps];
  float uu[kStepReps], xr[kStepReps], zr[kStepReps], Dd[kStepReps];
  float win[kStepReps][kStepConvMax];  // the convolution window (CONV)
  int64_t idx[kStepReps];
  bool active[kStepReps];
#pragma unroll
  for (int r = 0; r < kStepReps; ++r) {
    const int64_t d_raw = (int64_t(blockIdx.x) * kStepReps + r) * kStepChannels + (threadIdx.x >> 2);
    active[r] = d_raw < a.dim;
    const int64_t d = active[r] ? d_raw : a.dim - 1;  // idle lanes shadow a valid channel and store nothing
    const int64_t i = b * a.dim + d;
    idx[r] = i;
    hv[r] = reinterpret_cast<const float4*>(a.state + i * kDState)[q];
    av[r] = reinterpret_cast<const float4*>(a.A + d * kDState)[q];
    uu[r] = IO::load(static_cast<const T*>(a.u), i);
    xr[r] = IO::load(static_cast<const T*>(a.delta), i) + (a.delta_bias ? a.delta_bias[d] : 0.0f);
    zr[r] = a.z ? IO::load(static_cast<const T*>(a.z), i) : 0.0f;
    Dd[r] = a.D ? a.D[d] : 0.0f;
    if (CONV) {
      // window: the stored inputs (oldest first), then x_t; every lane of the quad
      // computes u_t (four taps at most), the quad's first lane stores the shifted window
      const int W = a.conv_width;
      const T* cs = static_cast<const T*>(a.conv_state) + i * (W - 1);
      float acc = a.conv_b ? a.conv_b[d] : 0.0f;
#pragma unroll
      for (int j = 0; j < kStepConvMax - 1; ++j) {
        if (j < W - 1) {
          win[r][j] = IO::load(cs, j);
          acc = fmaf(a.conv_w[d * W + j], win[r][j], acc);
        }
      }
      acc = fmaf(a.conv_w[d * W + W - 1], uu[r], acc);
      win[r][kStepConvMax - 1] = uu[r];  // x_t, the newest input
      uu[r] = a.conv_silu ? silu_f32(acc) : acc;
    }
  }
#pragma unroll
  for (int r = 0; r < kStepReps; ++r) {
    float h[4] = {hv[r].x, hv[r].y, hv[r].z, hv[r].w};
    const float A2[4] = {av[r].x * kLog2e, av[r].y * kLog2e, av[r].z * kLog2e, av[r].w * kLog2e};
    const float dt = SOFTPLUS ? softplus_f32(xr[r]) : xr[r];
    const float dtu = dt * uu[r];
    float s = 0.0f;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      h[n] = fmaf(exp2_hw(dt * A2[n]), h[n], dtu * Bv[n]);
      s = fmaf(Cv[n], h[n], s);
    }
    s = quad_sum(s);
    if (!active[r]) continue;
    const int64_t i = idx[r];
    reinterpret_cast<float4*>(a.state + i * kDState)[q] = make_float4(h[0], h[1], h[2], h[3]);
    if (CONV && q == 0) {
      // the window without its oldest input: win[1 .. W-2], then x_t
      const int W = a.conv_width;
      T* cs = static_cast<T*>(a.conv_state) + i * (W - 1);
#pragma unroll
      for (int j = 0; j < kStepConvMax - 1; ++j)
        if (j < W - 1) IO::store(cs, j, j + 1 < W - 1 ? win[r][j + 1] : win[r][kStepConvMax - 1]);
    }
    if (q == 0) {
      float yv = fmaf(Dd[r], uu[r], s);
      if (a.z) yv *= silu_f32(zr[r]);
      IO::store(static_cast<T*>(a.y), i, yv);
    }
  }
}

// Step 3, both directions: wave 0 scans the segment forward, wave 1 in reverse.
// Each first covers the half it meets first and parks its outputs, then covers the
// other half, adds the partner's parked outputs, gates and stores.  The meeting
// buffer is LDS for segments up to kBidirSegment tokens; longer (single) segments
// park in the block's slice of a workspace buffer (GPARK), so that LDS does not
// cut the number of resident blocks (a 197-token buffer is 50 KB).
template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z, int CONV, bool Y_F32 = false, bool GPARK = false>
__global__ __launch_bounds__(2 * kLanes) SSCAN_OUT_OCCUPANCY(IO_BF16 && CONV == kNoConv && !GPARK) void scan_output_bidir_kernel(ScanArgs a, int64_t seg_len, int64_t nseg,
                                                                       const float* __restrict__ bc, SegChain ch,
                                                                       float* __restrict__ gpark, int vec) {
  extern __shared__ float part[];  // [seg_len][64]
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const SegIndex s = decode_block(blockIdx.x, ngroups, nseg);
  const int dir = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kLanes);  // wave-uniform
  Lane<IO_BF16, SOFTPLUS, HAS_Z, CONV, Y_F32, GPARK> L;
  init_lane(L, a, dir, s.b, s.g, bc, (vec & 1) != 0);
  load_entry(L, a, dir, s.b, s.seg, s.g, nseg, ch);
  const int64_t t0 = s.seg * seg_len;
  const int64_t t1 = min64(a.len, t0 + seg_len);
  const int64_t mid = t0 + ((t1 - t0) / 2) / kTile * kTile;  // a multiple of both tile sizes
  if constexpr (GPARK) {
    L.part = gpark + size_t(blockIdx.x) * size_t(seg_len) * kLanes;
  } else {
    L.part = (lds_float*)part;
  }
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
bool aligned128(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 127u) == 0; }

template <bool IO_BF16, bool SOFTPLUS, bool HAS_Z, int CONV, bool Y_F32 = false>
hipError_t launch_typed(const ScanArgs& a, const Plan& p, float* w, hipStream_t stream, hipEvent_t const* ev) {
  auto mark = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  const int64_t ngroups = (a.dim + kLanes - 1) / kLanes;
  const int64_t nblocks = a.batch * p.nseg * ngroups;
  const size_t esz = IO_BF16 ? 2 : 4;
  bool vec = (size_t(a.len) * esz) % 16 == 0 && aligned16(a.u) && aligned16(a.y) && (!a.z || aligned16(a.z));
  for (int k = 0; k < a.ndir; ++k) vec = vec && aligned16(a.dir[k].delta);
  // whole 128-byte lines of u and delta (bf16): rows and segments start on a line
  bool line = IO_BF16 && vec && (size_t(a.len) * esz) % 128 == 0 && (p.nseg <= 1 || (size_t(p.seg_len) * esz) % 128 == 0) &&
              aligned128(a.u);
  for (int k = 0; k < a.ndir; ++k) line = line && aligned128(a.dir[k].delta);
  const int flags = int(vec) | (int(line) << 1);
  float* bc = w;
  SegChain ch{};
  ch.run_len = p.run_len;
  ch.nrun = p.nrun;
  if (p.nseg > 1) {
    float* q = w + p.bc_floats;
    ch.p = p.p_floats ? q : nullptr;
    q += p.p_floats;
    ch.s = p.s_floats ? q : nullptr;
    q += p.s_floats;
    ch.r = q;
    q += p.r_floats;
    ch.e = q;
  }

  mark(0);
  launch_stage_bc(a, bc, stream);
  mark(1);
  if constexpr (CONV == kNoConv && !Y_F32) {
    if (p.quad && !a.h0 && !a.h_last) {
      mark(2);
      mark(3);
      const hipError_t e = launch_short_quad(a, bc, stream);
      mark(4);
      return e;
    }
  }
  if (p.nseg > 1) {
    const int64_t agg_blocks = a.batch * p.nrun * ngroups;
    if (p.run_len > 1) {
      hipLaunchKernelGGL((scan_aggregate_kernel<IO_BF16, SOFTPLUS, CONV, true>),
                         dim3(unsigned(agg_blocks), unsigned(a.ndir)), dim3(kLanes), 0, stream, a, p.seg_len, p.nseg,
                         ch, static_cast<const float*>(bc), flags);
    } else {
      hipLaunchKernelGGL((scan_aggregate_kernel<IO_BF16, SOFTPLUS, CONV, false>),
                         dim3(unsigned(agg_blocks), unsigned(a.ndir)), dim3(kLanes), 0, stream, a, p.seg_len, p.nseg,
                         ch, static_cast<const float*>(bc), flags);
    }
    mark(2);
    launch_carry(a, p.nrun, ch.r, ch.e, 0, stream);
  }
  if (p.nseg <= 1) mark(2);
  mark(3);
  if (a.ndir == 1) {
    hipLaunchKernelGGL((scan_output_dir_kernel<IO_BF16, SOFTPLUS, HAS_Z, CONV, Y_F32>), dim3(unsigned(nblocks)), dim3(kLanes), 0,
                       stream, a, p.seg_len, p.nseg, static_cast<const float*>(bc), ch, flags);
  } else if (p.park_floats) {
    float* gpark = w + p.bc_floats + p.p_floats + p.s_floats + p.r_floats + p.e_floats;
    hipLaunchKernelGGL((scan_output_bidir_kernel<IO_BF16, SOFTPLUS, HAS_Z, CONV, Y_F32, true>), dim3(unsigned(nblocks)),
                       dim3(2 * kLanes), 0, stream, a, p.seg_len, p.nseg, static_cast<const float*>(bc), ch, gpark,
                       int(vec));
  } else {
    const size_t lds = size_t(p.seg_len) * kLanes * sizeof(float);
    hipLaunchKernelGGL((scan_output_bidir_kernel<IO_BF16, SOFTPLUS, HAS_Z, CONV, Y_F32, false>), dim3(unsigned(nblocks)),
                       dim3(2 * kLanes), lds, stream, a, p.seg_len, p.nseg, static_cast<const float*>(bc), ch, nullptr,
                       int(vec));
  }
  mark(4);
  return hipGetLastError();
}

template <bool IO_BF16, int CONV>
hipError_t launch_conv_mode(const ScanArgs& a, const Plan& p, float* w, hipStream_t stream, hipEvent_t const* ev) {
  if (a.softplus) {
    return a.z ? launch_typed<IO_BF16, true, true, CONV>(a, p, w, stream, ev)
               : launch_typed<IO_BF16, true, false, CONV>(a, p, w, stream, ev);
  }
  return a.z ? launch_typed<IO_BF16, false, true, CONV>(a, p, w, stream, ev)
             : launch_typed<IO_BF16, false, false, CONV>(a, p, w, stream, ev);
}

template <bool IO_BF16>
hipError_t launch_io(const ScanArgs& a, const Plan& p, float* w, hipStream_t stream, hipEvent_t const* ev) {
  if (a.y_f32 && IO_BF16) {
    // fp32 partial outputs (ungated, no convolution): the multi-order scan
    if (a.z || a.conv_w) return hipErrorInvalidValue;
    return a.softplus ? launch_typed<IO_BF16, true, false, kNoConv, true>(a, p, w, stream, ev)
                      : launch_typed<IO_BF16, false, false, kNoConv, true>(a, p, w, stream, ev);
  }
  if (!a.conv_w) return launch_conv_mode<IO_BF16, kNoConv>(a, p, w, stream, ev);
  return a.conv_silu ? launch_conv_mode<IO_BF16, kConvSilu>(a, p, w, stream, ev)
                     : launch_conv_mode<IO_BF16, kConvLin>(a, p, w, stream, ev);
}

// Standalone depthwise convolution: each thread produces kConvReps runs of kConvRun
// consecutive outputs of one row, the runs 64 x kConvRun tokens apart.  A run moves
// as 16-byte vectors when rows are 16-byte aligned, and all of a thread's runs are
// loaded before any is computed, so each wave keeps kConvReps KB in flight.
// Block (64 runs, 4 channels): a wavefront holds 64 consecutive runs of one row, so
// the halo -- three tokens before the run, one after -- is the neighbouring lanes'
// data, moved across lanes; only the wave's first and last lanes read theirs from
// memory.  Grid (run chunks, channel quads, batch rows -- striding above the grid
// limit), so every thread knows its runs and channel without dividing and loads its
// channel's taps once.  Lanes past the row's end stay active (zeros) for the
// cross-lane moves.
constexpr int kConvRun = 8;
constexpr int kConvRows = 4;
constexpr int kConvReps = 4;

template <bool IO_BF16, bool SILU, bool Y_F32 = false>
__global__ __launch_bounds__(kLanes * kConvRows) void conv1d_kernel(ConvArgs a, int vec) {
  using IO = Io<IO_BF16>;
  using T = typename IO::T;
  using TY = typename std::conditional<Y_F32, float, T>::type;
  using IOY = Io<!Y_F32 && IO_BF16>;
  constexpr int kSpan = kConvBack + kConvRun + 1;
  for (int64_t d = int64_t(blockIdx.y) * kConvRows + threadIdx.y; d < a.dim; d += int64_t(gridDim.y) * kConvRows) {
    float cw[kConvTaps];
#pragma unroll
    for (int k = 0; k < kConvTaps; ++k) {
      const int j = k - (kConvBack - a.left);
      cw[k] = (j >= 0 && j < a.width) ? a.w[d * a.width + j] : 0.0f;
    }
    const float cb = a.b ? a.b[d] : 0.0f;
    for (int64_t b = blockIdx.z; b < a.batch; b += gridDim.z) {
      const int64_t row = b * a.dim + d;
      const T* x = static_cast<const T*>(a.x) + row * a.len;
      TY* y = static_cast<TY*>(a.y) + row * a.len;
      // x[t0 - 3 .. t0 + kConvRun] of each run, zero outside the row; a run may start
      // past the row's end: the lane loads and stores nothing for it.  The runs' words
      // are only loaded here (unpacked below), so no load waits for another.
      constexpr int kRaw = IO_BF16 ? 4 : 8;
      uint32_t raw[kConvReps][kRaw];
      uint32_t hraw[kConvReps][kConvBack + 1];
      // one element's bits (zero-extended for bf16), t clamped into the row
      auto raw_at = [&](int64_t t) -> uint32_t {
        t = t < 0 ? 0 : (t >= a.len ? a.len - 1 : t);
        if (IO_BF16) return uint32_t(reinterpret_cast<const uint16_t*>(x)[t]);
        return __float_as_uint(reinterpret_cast<const float*>(x)[t]);
      };
      auto widen = [](uint32_t r) -> float { return IO_BF16 ? __uint_as_float(r << 16) : __uint_as_float(r); };
      float xs[kConvReps][kSpan];
      int64_t t0[kConvReps];
#pragma unroll
      for (int q = 0; q < kConvReps; ++q) {
        t0[q] = ((int64_t(blockIdx.x) * kConvReps + q) * kLanes + threadIdx.x) * kConvRun;
        const bool full = vec && t0[q] + kConvRun <= a.len;
        if (full) {
          const uint4* p = reinterpret_cast<const uint4*>(x + t0[q]);
          const uint4 v = p[0];
          raw[q][0] = v.x;
          raw[q][1] = v.y;
          raw[q][2] = v.z;
          raw[q][3] = v.w;
          if (!IO_BF16) {
            const uint4 v1 = p[1];
            raw[q][4 % kRaw] = v1.x;
            raw[q][5 % kRaw] = v1.y;
            raw[q][6 % kRaw] = v1.z;
            raw[q][7 % kRaw] = v1.w;
          }
        } else {
#pragma unroll
          for (int k = 0; k < kConvRun; ++k) {
            const uint32_t e = t0[q] + k < a.len ? __float_as_uint(IO::load(x, t0[q] + k)) : 0u;
            if (IO_BF16) {
              // the widened value's upper half is the bf16 bit pattern
              raw[q][k / 2] = (k & 1) ? ((raw[q][k / 2] & 0xffffu) | (e & 0xffff0000u)) : (e >> 16);
            } else {
              raw[q][k % kRaw] = e;
            }
          }
        }
        // the halo tokens, raw, at indices clamped into the row (zeroed outside it below):
        // loaded by every lane, with no branch for a wait to land in, though only the
        // wave's end lanes use theirs (the others' come across lanes; all are in lines
        // the wave reads anyway)
#pragma unroll
        for (int k = 0; k < kConvBack; ++k) hraw[q][k] = raw_at(t0[q] - kConvBack + k);
        hraw[q][kConvBack] = raw_at(t0[q] + kConvRun);
      }
#pragma unroll
      for (int q = 0; q < kConvReps; ++q) {
#pragma unroll
        for (int k = 0; k < kConvRun; ++k)
          xs[q][kConvBack + k] = IO_BF16 ? ((k & 1) ? bf16_hi(raw[q][k / 2]) : bf16_lo(raw[q][k / 2]))
                                         : __uint_as_float(raw[q][k % kRaw]);
#pragma unroll
        for (int k = 0; k < kConvBack; ++k) {
          const int64_t t = t0[q] - kConvBack + k;
          xs[q][k] = (t >= 0 && t < a.len) ? widen(hraw[q][k]) : 0.0f;
        }
        xs[q][kSpan - 1] = t0[q] + kConvRun < a.len ? widen(hraw[q][kConvBack]) : 0.0f;
        // the halo: the previous lane's last three tokens, the next lane's first (the
        // wave's end lanes keep what they loaded)
#pragma unroll
        for (int k = 0; k < kConvBack; ++k) {
          const float v = __shfl_up(xs[q][kConvRun + k], 1);
          if (threadIdx.x != 0) xs[q][k] = v;
        }
        {
          const float v = __shfl_down(xs[q][kConvBack], 1);
          if (threadIdx.x != kLanes - 1) xs[q][kSpan - 1] = v;
        }
        float out[kConvRun];
#pragma unroll
        for (int j = 0; j < kConvRun; ++j) {
          float acc = cb;
#pragma unroll
          for (int k = 0; k < kConvTaps; ++k) acc = fmaf(cw[k], xs[q][j + k], acc);
          out[j] = SILU ? silu_f32(acc) : acc;
        }
        const bool full = vec && t0[q] + kConvRun <= a.len;
        if (full) {
          if (IO_BF16 && !Y_F32) {
            *reinterpret_cast<uint4*>(y + t0[q]) = make_uint4(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]),
                                                              pack_bf16x2(out[4], out[5]), pack_bf16x2(out[6], out[7]));
          } else {
            float4* p = reinterpret_cast<float4*>(y + t0[q]);
            p[0] = make_float4(out[0], out[1], out[2], out[3]);
            p[1] = make_float4(out[4], out[5], out[6], out[7]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < kConvRun; ++j)
            if (t0[q] + j < a.len) IOY::store(reinterpret_cast<typename IOY::T*>(y), t0[q] + j, out[j]);
        }
      }
    }
  }
}
}  // namespace

// Resident wave slots of the scan kernels on MI355X: 256 CUs x 4 SIMDs x 3 waves
// (the scan kernels are held to <= 168 VGPRs).
constexpr int64_t kWaveSlots = 256 * 4 * 3;
// Bidirectional segments: the LDS meeting buffer (seg_len x 64 lanes x 4 B) must
// leave room for eight two-wave blocks per CU.  (A sequence short enough to be one
// segment may be longer; its meeting buffer is in global memory.)
constexpr int64_t kBidirSegment = 64;
// Rounds of resident waves the output step of a long one-direction scan aims for.
// Measured on the long-sequence workload (1 x 1536 x 262144): 1 round (2048-token
// segments) 3.19 ms per call, 2 rounds 2.66, 3 rounds 2.67, 4 rounds (512 tokens)
// 2.59, 5 rounds 2.61, 6 rounds 2.63, 8 rounds 2.60: four rounds even out the
// waves' finishing times best before the longer carry chain costs more than it
// saves.
constexpr int64_t kSegRounds = 4;
// Segments are grouped in aggregate runs only where one wave per segment would
// give the aggregate pass more than about four rounds of resident waves (very long
// bidirectional sequences, cut into 64-token segments): the run form holds more
// registers, and a short chain costs the carry little.
constexpr int64_t kAggWaves = 4 * kWaveSlots;
// Short sequences use the four-lanes-per-channel kernel below this many rounds of
// lane = channel waves (Vim-tiny, 768 waves: output pass 108 -> 74 us; Vim-small,
// 3072 waves, one full round: 188 -> 217 us, so it keeps lane = channel).
constexpr int64_t kQuadRounds = 1;

// Splitting along the sequence.  Sequences up to kShortMax tokens are scanned whole
// (splitting a 197-token Vim sequence that fills only a quarter of the resident
// wave slots was measured slower: its 64-token aggregate waves and short carry cost
// more than the output pass gains).  Longer ones are cut into equal segments
// (multiples of kTile tokens) so that the output step has about kSegRounds rounds
// of resident waves: enough waves to cover load latency and even out per-wave
// speed, without the long carry chain and large aggregate buffers of many short
// segments.
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
      const int64_t target_segs = std::max<int64_t>(2, kSegRounds * kWaveSlots / groups);
      seg_len = (len + target_segs - 1) / target_segs;
      seg_len = std::max<int64_t>(kSegAlign, (seg_len + kTile - 1) / kTile * kTile);
    }
    // keep the output pass's grid (two-wave blocks) under 2^32 work-items
    while ((len + seg_len - 1) / seg_len > 1 &&
           batch * ((len + seg_len - 1) / seg_len) * ngroups * 2 * kLanes >= (int64_t(1) << 32))
      seg_len *= 2;
    p.seg_len = seg_len;
    p.nseg = (len + seg_len - 1) / seg_len;
  }
  // A one-segment sequence whose lane = channel waves fill less than kQuadRounds
  // rounds of the resident slots goes to the four-lanes-per-channel kernel (four
  // times the waves).
  p.quad = p.nseg == 1 && int64_t(ndir) * groups < kQuadRounds * kWaveSlots;
  // Aggregate runs: enough segments per run that the aggregate pass has about
  // kAggWaves waves and the carry chains fewer runs.
  p.run_len = std::max<int64_t>(1, int64_t(ndir) * groups * p.nseg / kAggWaves);
  p.nrun = (p.nseg + p.run_len - 1) / p.run_len;
  // keep the sections 256-byte aligned
  auto up = [](size_t n) { return (n + 63) / 64 * 64; };
  p.bc_floats = up(size_t(ndir) * batch * len * kBC);
  if (p.nseg > 1) {
    if (p.run_len > 1) {
      p.p_floats = up(size_t(ndir) * batch * p.nseg * dim * kDState);
      p.s_floats = up(size_t(ndir) * batch * p.nseg * dim);
    }
    p.r_floats = up(size_t(ndir) * batch * p.nrun * (kDState + 1) * dim);
    p.e_floats = up(size_t(ndir) * batch * p.nrun * kDState * dim);
  }
  // bidirectional segments longer than kBidirSegment park in global memory
  if (ndir == 2 && p.seg_len > kBidirSegment)
    p.park_floats = up(size_t(batch) * p.nseg * ngroups * p.seg_len * kLanes);
  p.workspace_bytes =
      (p.bc_floats + p.p_floats + p.s_floats + p.r_floats + p.e_floats + p.park_floats) * sizeof(float);
  return p;
}

namespace {
constexpr int64_t kMaxItems = (int64_t(1) << 32) - 1;  // work-items of one grid dimension
bool fits(int64_t blocks, int64_t threads) { return blocks <= kMaxItems / threads; }
}  // namespace

bool plan_fits_grid(const Plan& p, int64_t batch, int64_t dim, int64_t len, int ndir) {
  const int64_t ngroups = (dim + kLanes - 1) / kLanes;
  bool ok = fits(int64_t(ndir) * batch * ((len + 63) / 64), 256);  // B/C staging
  if (p.quad) ok = ok && fits(batch * ((dim + 15) / 16), int64_t(ndir) * kLanes);
  ok = ok && fits(batch * p.nseg * ngroups, int64_t(ndir) * kLanes);  // output pass (also the fallback for a quad plan)
  if (p.nseg > 1) {
    ok = ok && fits(batch * p.nrun * ngroups, kLanes);  // aggregate (blockIdx.y: direction)
    ok = ok && fits(int64_t(ndir) * batch * kDState * ngroups, int64_t(kLanes) * carry_parts(p.nrun));
  }
  return ok;
}

hipError_t launch_scan(const ScanArgs& a, const Plan& p, float* ws, hipStream_t stream, hipEvent_t const* events) {
  return a.io_bf16 ? launch_io<true>(a, p, ws, stream, events) : launch_io<false>(a, p, ws, stream, events);
}

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t stream) {
  constexpr int64_t kMaxGridYZ = 65535;
  const int64_t runs = (a.len + kConvRun - 1) / kConvRun;
  const int64_t quads = (a.dim + kConvRows - 1) / kConvRows;
  const int64_t per_block = int64_t(kLanes) * kConvReps;
  const dim3 grid(unsigned((runs + per_block - 1) / per_block), unsigned(std::min(quads, kMaxGridYZ)),
                  unsigned(std::min(a.batch, kMaxGridYZ)));
  const dim3 block(kLanes, kConvRows);
  // runs start at multiples of 8 tokens: 16-byte aligned when every row is
  const size_t esz = a.io_bf16 ? 2 : 4;
  const int vec = (size_t(a.len) * esz) % 16 == 0 && aligned16(a.x) && aligned16(a.y);
  if (a.io_bf16 && a.y_f32) {
    // bf16 x, float32 output (the backward's copy of u); float32 rows of 8-token
    // runs are 16-byte aligned whenever the bf16 ones are
    if (a.silu) {
      hipLaunchKernelGGL((conv1d_kernel<true, true, true>), grid, block, 0, stream, a, vec);
    } else {
      hipLaunchKernelGGL((conv1d_kernel<true, false, true>), grid, block, 0, stream, a, vec);
    }
  } else if (a.io_bf16) {
    if (a.silu) {
      hipLaunchKernelGGL((conv1d_kernel<true, true>), grid, block, 0, stream, a, vec);
    } else {
      hipLaunchKernelGGL((conv1d_kernel<true, false>), grid, block, 0, stream, a, vec);
    }
  } else {
    if (a.silu) {
      hipLaunchKernelGGL((conv1d_kernel<false, true>), grid, block, 0, stream, a, vec);
    } else {
      hipLaunchKernelGGL((conv1d_kernel<false, false>), grid, block, 0, stream, a, vec);
    }
  }
  return hipGetLastError();
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
    const int64_t per_block = int64_t(kStepChannels) * kStepReps;
    const dim3 grid(unsigned((a.dim + per_block - 1) / per_block), unsigned(std::min(kMaxRows, a.batch - b0)));
    const dim3 block(kStepThreads);
#define SSCAN_STEP_LAUNCH(CONV)                                                                            \
  switch (key) {                                                                                          \
    case 0: hipLaunchKernelGGL((step_kernel<false, false, false, CONV>), grid, block, 0, stream, a, b0); break; \
    case 1: hipLaunchKernelGGL((step_kernel<false, false, true, CONV>), grid, block, 0, stream, a, b0); break;  \
    case 2: hipLaunchKernelGGL((step_kernel<false, true, false, CONV>), grid, block, 0, stream, a, b0); break;  \
    case 3: hipLaunchKernelGGL((step_kernel<false, true, true, CONV>), grid, block, 0, stream, a, b0); break;   \
    case 4: hipLaunchKernelGGL((step_kernel<true, false, false, CONV>), grid, block, 0, stream, a, b0); break;  \
    case 5: hipLaunchKernelGGL((step_kernel<true, false, true, CONV>), grid, block, 0, stream, a, b0); break;   \
    case 6: hipLaunchKernelGGL((step_kernel<true, true, false, CONV>), grid, block, 0, stream, a, b0); break;   \
    default: hipLaunchKernelGGL((step_kernel<true, true, true, CONV>), grid, block, 0, stream, a, b0); break;  \
  }
    if (a.conv_w) {
      SSCAN_STEP_LAUNCH(true)
    } else {
      SSCAN_STEP_LAUNCH(false)
    }
#undef SSCAN_STEP_LAUNCH
  }
  return hipGetLastError();
}

}  // namespace sscan
