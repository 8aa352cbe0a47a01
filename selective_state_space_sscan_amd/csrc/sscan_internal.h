// sscan_internal.h -- launch interface between the C ABI (sscan_capi.cpp) and the
// gfx950 kernels (sscan_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace sscan {

constexpr int kDState = 16;        // states per channel held in registers
constexpr int kLanes = 64;         // channels per wavefront (lane = channel)

constexpr int kTile = 32;          // tile alignment unit (tokens; a multiple of every tile size)

// Sequences longer than kShortMax are split into segments scanned in parallel;
// the state entering each segment is produced by the aggregate and carry kernels.
constexpr int64_t kShortMax = 256;
constexpr int64_t kSegAlign = 64;          // segment lengths are multiples of this

struct DirArgs {
  const void* delta;
  const float* delta_bias;  // nullable
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // nullable
};

struct ScanArgs {
  const void* u;
  const void* z;            // nullable
  void* y;
  DirArgs dir[2];
  int ndir;                 // 1 or 2
  int reverse;              // single direction only
  int softplus;
  int io_bf16;              // u, delta, z, y are bf16 (else f32)
  int bc_bf16;              // B, C are bf16 (else f32)
  int64_t batch, dim, len;
  const float* h0;          // nullable: state before the first scanned token, [batch][dim][16]
  float* h_last;            // nullable: receives the state after the last scanned token (may equal h0)
  // Depthwise convolution in front of the scan (conv_w != nullptr): u is then
  // act(conv_b + sum_j conv_w[d][j] * x[t - conv_left + j]) of the x held in `u`.
  const float* conv_w;      // [dim][conv_width]
  const float* conv_b;      // nullable, [dim]
  int conv_width;           // taps, with conv_left <= 3 and conv_width - 1 - conv_left <= 1
  int conv_left;            // taps before the output token (causal: width - 1)
  int conv_silu;            // silu after the bias
  int y_f32;                // store y in fp32 whatever io_bf16 (no gate, no convolution)
};

// Scans of a 2-D map along several visiting orders.  A direction's kind is
// family * 2 + (1 for the reversed order); families: row-major, column-major, and
// a caller-given permutation of the tokens.
constexpr int kFamilyRow = 0, kFamilyCol = 1, kFamilyIndex = 2, kFamilies = 3;
constexpr int kMaxMultiDirs = 2 * kFamilies;

struct MultiArgs {
  const void* u;            // [batch][dim][height * width] io dtype, token t = r * width + c
  const void* z;            // nullable
  void* y;
  DirArgs dir[kMaxMultiDirs];
  int kind[kMaxMultiDirs];
  int ndir;
  const int32_t* index;     // [height * width] visiting order of the index family
  int softplus, io_bf16, bc_bf16;
  int64_t batch, dim, height, width;
};

// Workspace (byte offsets, 256-aligned): fp32 accumulator, one family's output,
// gathered u, gathered delta/B/C of a family's two directions, the scan's own.
struct MultiPlan {
  size_t off_acc, off_y, off_u, off_delta[2], off_B[2], off_C[2], off_inv, off_scan;
  size_t workspace_bytes;
};

MultiPlan make_multi_plan(int64_t batch, int64_t dim, int64_t height, int64_t width, const int* kinds, int ndir,
                          bool io_bf16, bool bc_bf16);
hipError_t launch_multi(const MultiArgs& a, const MultiPlan& p, char* workspace, hipStream_t stream);

// A standalone depthwise convolution (the same operation as the scan's front-end).
struct ConvArgs {
  const void* x;
  void* y;                  // io dtype, or float32 when y_f32
  const float* w;
  const float* b;           // nullable
  int width, left, silu, io_bf16;
  int64_t batch, dim, len;
  int y_f32;
};

// Backward of that convolution: du = dLoss/d(its output) gives dx, and the sums
// over batch rows and tokens dw [dim][width] and db [dim] (nullable).
struct ConvBwdArgs {
  const void* x;
  const float* du;          // float32 [batch][dim][len]
  void* dx;
  const float* w;
  const float* b;           // nullable
  float* dw;
  float* db;                // nullable
  int width, left, silu, io_bf16;
  int64_t batch, dim, len;
};

// Partial sums (floats) of the weight and bias gradients the backward kernel keeps.
size_t conv_bwd_partial_floats(int64_t batch, int64_t dim, int64_t len);
hipError_t launch_conv1d_bwd(const ConvBwdArgs& a, float* partials, hipStream_t stream);

// One token of the recurrence from a stored state (single-step decode).
struct StepArgs {
  float* state;             // [batch][dim][16], read and updated in place
  const void* u;            // [batch][dim] io dtype
  const void* delta;
  const void* z;            // nullable
  void* y;
  const float* delta_bias;  // nullable, [dim]
  const float* A;           // [dim][16]
  const void* B;            // [batch][16] bc dtype
  const void* C;
  const float* D;           // nullable, [dim]
  int softplus, io_bf16, bc_bf16;
  int64_t batch, dim;
  // Causal convolution in front of the step (conv_w != nullptr): `u` holds x_t, and
  // u_t = act(conv_b + sum_j conv_w[d][j] * window[j]) over the window of the
  // stored last conv_width - 1 inputs (conv_state [batch][dim][conv_width - 1], io
  // dtype, oldest first) followed by x_t; the window then drops its oldest input.
  void* conv_state;         // read and updated in place (nullable when conv_width == 1)
  const float* conv_w;      // [dim][conv_width], nullable: no convolution
  const float* conv_b;      // nullable, [dim]
  int conv_width;           // 1 .. 4
  int conv_silu;
};

// Gradients of one direction (backward pass); nullable members are not computed.
struct DirGrads {
  void* ddelta;             // [batch][dim][len] io dtype
  float* ddelta_bias;       // nullable, [dim]
  float* dA;                // [dim][16]
  void* dB;                 // [batch][16][len] bc dtype
  void* dC;
  float* dD;                // nullable, [dim]
};

struct BwdArgs {
  ScanArgs fwd;             // the forward call's inputs (y, h0 and h_last unused)
  const void* dout;         // dLoss/dout, [batch][dim][len] io dtype
  void* du;                 // io dtype, or float32 when du_f32
  void* dz;                 // written when fwd.z is set
  DirGrads grads[2];
  int du_f32;               // du stored in float32 whatever the io dtype (for the convolution's backward)
  int dz_f32;               // dz stored in float32 likewise (a partial summed with other orders' before rounding)
  // With the convolution in front (fwd.conv_w set, fwd.u holding x): u = conv(x) in
  // float32, as the fused forward computes it.  The state chain recomputes it from
  // x itself; the window pass reads it here.
  const float* u32;
  // State I/O (one direction): the forward's entry state is fwd.h0; dh_last
  // (nullable, [batch][dim][16]) is the gradient reaching its final state, and dh0
  // (nullable) receives the gradient of the entry state.
  const float* dh_last;
  float* dh0;
};

// Backward split into 32-token windows, and its workspace (float offsets):
//   bc   [ndir][batch][len][32]             staged B/C
// Two chains cross the windows: the state in scan order (chain 0) and the adjoint
// against it (chain 1).  Each is walked over runs of run_len consecutive windows
// (nwin > 1 only):
//   p    [ndir][batch][nwin][dim][16]  after each window, the chain walked from zero
//                                      at the start of its run
//   s    [ndir][batch][nwin][dim]      the step sizes summed over the same stretch
//   r    [ndir][batch][nrun][17][dim]  run totals (16 states, step-size sum)
//   e    [ndir][batch][nrun][16][dim]  the chain entering each run (carry over runs)
//   part [ndir][batch][nwin][18][dim]      per-window dA[16], dD, delta_bias
//   pbc  [csplit][ndir][batch][2][16][len] dB, dC per channel split
//   acc  [2][batch][dim][len]              first direction's du and y (two directions)
struct BwdPlan {
  int64_t nwin;             // windows per row
  int csplit;               // channel splits per window (blocks per window)
  int64_t gps;              // 4-channel groups per split
  int64_t run_len, nrun;    // windows per chain run, runs per row
  size_t off_bc, off_part, off_pbc, off_acc;
  size_t off_p[2], off_s[2], off_r[2], off_e[2];
  size_t workspace_bytes;
};

BwdPlan make_bwd_plan(int64_t batch, int64_t dim, int64_t len, int ndir);

// Step boundaries of a backward call: before staging, after staging, after the
// window entry states, after the window adjoints, after the window pass(es), after
// the reductions.
constexpr int kBwdProfileEvents = 6;

hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& p, float* workspace, hipStream_t stream,
                      hipEvent_t const* events = nullptr);

// Gradients of an empty call: the parameter gradients (dA, dD, delta_bias, dB, dC)
// that have elements are zero.
hipError_t launch_bwd_zero(const BwdArgs& a, hipStream_t stream);

// Backward of the scans along several orders: each family's backward runs on its
// gathered inputs (gated, du and dz in fp32); du and dz are put back and summed
// over the families in the fixed family order, ddelta/dB/dC put back per
// direction.  Workspace (byte offsets, 256-aligned):
//   acc_du, acc_dz  [batch][dim][len] f32   sums over the families (two or more)
//   vdu, vdz        [batch][dim][len] f32   a gathered family's du, dz (visit order)
//   u, z, dout      io dtype                gathered
//   delta[2]        io dtype, B[2], C[2]    gathered per direction slot
//   dd[2]           io dtype, dB[2], dC[2]  gradients in visit order
//   inv             [len] int32             inverse of the index order
//   bwd             the backward's own workspace (largest family)
struct MultiBwdArgs {
  MultiArgs fwd;            // fwd.y unused
  const void* dout;
  void* du;
  void* dz;                 // written when fwd.z is set
  DirGrads grads[kMaxMultiDirs];
};

struct MultiBwdPlan {
  size_t off_acc_du, off_acc_dz, off_vdu, off_vdz, off_u, off_z, off_g;
  size_t off_delta[2], off_B[2], off_C[2], off_dd[2], off_dB[2], off_dC[2];
  size_t off_inv, off_bwd;
  size_t workspace_bytes;
};

MultiBwdPlan make_multi_bwd_plan(int64_t batch, int64_t dim, int64_t height, int64_t width, const int* kinds,
                                 int ndir, bool io_bf16, bool bc_bf16);
hipError_t launch_multi_bwd(const MultiBwdArgs& a, const MultiBwdPlan& p, char* workspace, hipStream_t stream);

// How a call is split along the sequence, and the workspace it needs (floats,
// in this order):
//   bc   [ndir][batch][len][32]        B_t (16 states) then C_t (16), fp32, token-major
//   agg  [ndir][batch][nseg][17][dim]  segment end states (from zero) + sum of dt
//   hin  [ndir][batch][nseg][16][dim]  state entering every segment
// agg and hin exist only when nseg > 1.
struct Plan {
  int64_t seg_len;          // tokens per segment
  int64_t nseg;             // segments per row (1: no aggregate/carry kernels)
  int64_t run_len;          // segments per aggregate run
  int64_t nrun;             // runs per row
  size_t bc_floats;         // workspace sections, in order (floats, 64-aligned)
  size_t p_floats;          // per segment: state so far in its run (run_len > 1 only)
  size_t s_floats;          // per segment: summed step sizes so far (run_len > 1 only)
  size_t r_floats;          // per run: totals
  size_t e_floats;          // per run: entry state
  size_t park_floats;       // bidirectional meeting buffers kept in global memory
  size_t workspace_bytes;
  bool quad;                // one segment scanned by the four-lanes-per-channel kernel (when the call
                            // has no convolution, fp32 partial output or state I/O)
};

Plan make_plan(int64_t batch, int64_t dim, int64_t len, int ndir);

// A dispatch covers fewer than 2^32 work-items per grid dimension (blocks x block
// size): true when every kernel a call of this plan launches stays below that.
bool plan_fits_grid(const Plan& p, int64_t batch, int64_t dim, int64_t len, int ndir);
bool bwd_plan_fits_grid(const BwdPlan& p, int64_t batch, int64_t dim, int64_t len, int ndir);

// Boundaries of the steps of one call: before staging, after staging, after the
// segment aggregates, after the carry chain, after the output pass.
constexpr int kProfileEvents = 5;

// Enqueues the whole call on `stream`; returns the first HIP error (hipSuccess if none).
// With `events` (kProfileEvents entries, NULL entries skipped) each step boundary is
// also recorded on the stream.
hipError_t launch_scan(const ScanArgs& a, const Plan& p, float* workspace, hipStream_t stream,
                       hipEvent_t const* events = nullptr);

// The scan of one-segment sequences with four lanes per channel (Plan::quad): B/C
// already staged in bc.
hipError_t launch_short_quad(const ScanArgs& a, const float* bc, hipStream_t stream);

// A call with len == 0 and a final state requested: h_last = h0 (or 0).
hipError_t launch_state_passthrough(const ScanArgs& a, hipStream_t stream);

hipError_t launch_step(const StepArgs& a, hipStream_t stream);

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t stream);

}  // namespace sscan
