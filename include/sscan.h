/*
 * sscan.h -- C ABI of the MI355X (gfx950) selective scan (Mamba S6).
 *
 * Operation (Hand-written simplified Mamba2 page, sections 2.2, 4.2-4.4;
 * Reproducing Vision Mamba page, section 3.2 for the bidirectional sum):
 *
 *   dt_t = softplus(delta_t + delta_bias_d)   (or delta_t + delta_bias_d if softplus == 0)
 *   h_n  = 0 at the first processed token
 *   h_n <- exp(dt_t * A[d,n]) * h_n + dt_t * B[b,n,t] * u_t      (zero-order hold for A,
 *                                                                  first-order Bbar = dt*B)
 *   y_t  = sum_n C[b,n,t] * h_n + D_d * u_t
 *   out_t = y_t * silu(z_t),  silu(x) = x / (1 + exp(-x))          (z == NULL: out = y)
 *
 * sscan_fwd runs one direction: t ascending, or t descending when reverse != 0
 * (a forward scan of the time-flipped sequence, flipped back).  sscan_bidir runs
 * both directions, each with its own delta/bias/A/B/C/D, adds the two y and gates
 * the sum once.  The state is carried across the whole sequence (it is never reset
 * between internal chunks) and is never written to memory as a sequence.
 *
 * Layouts (all row-major and contiguous, element strides implied by the sizes):
 *   u, delta, z, y : [batch, dim, len]     dtype io_dtype  (SSCAN_F32 or SSCAN_BF16)
 *   B, C           : [batch, dstate, len]  dtype bc_dtype  (shared by all channels)
 *   A              : [dim, dstate]         float32 (diagonal state matrix per channel)
 *   D, delta_bias  : [dim]                 float32
 * Arithmetic and the state are float32; bf16 inputs widen exactly, bf16 outputs
 * round to nearest even.  dstate must be 16.
 *
 * Ownership: every data pointer is a DEVICE pointer owned by the caller.  The
 * library allocates no memory on these calls and keeps no state after return.
 * Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 * call returns; y is valid once the stream reaches that point, and inputs must stay
 * alive until then.  y must not overlap any input.  Calls take a caller-provided
 * device workspace of sscan_workspace_bytes(...) bytes, 16-byte aligned (B/C re-laid token-major;
 * for long sequences the segment chains; for one-segment bidirectional sequences
 * over 64 tokens the two directions' meeting buffers; NULL is allowed when that
 * size is 0); its contents on entry do not matter.
 *
 * Errors: every argument is checked before any HIP call; on error nothing is
 * enqueued and a negative status is returned (see sscan_strerror).  A failure
 * reported by the HIP runtime at launch is returned as SSCAN_ERR_HIP.  No
 * exception crosses this interface.  Calls are thread-safe (no global mutable
 * state); calls that share a workspace must be ordered on one stream.
 */
#ifndef SSCAN_H_
#define SSCAN_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define SSCAN_API __attribute__((visibility("default")))
#else
#define SSCAN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum sscan_status {
  SSCAN_OK = 0,
  SSCAN_ERR_NULL = -1,        /* a required pointer is NULL */
  SSCAN_ERR_SHAPE = -2,       /* batch, dim or len < 0, a size product overflows, or batch * len > 2^36 */
  SSCAN_ERR_UNSUPPORTED = -3, /* dstate != 16, unknown dtype code or convolution shape */
  SSCAN_ERR_ALIGN = -4,       /* a pointer is not aligned to its element size */
  SSCAN_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than sscan_workspace_bytes */
  SSCAN_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
  SSCAN_ERR_ALIAS = -7,       /* an output overlaps an input, another output or the workspace */
  SSCAN_ERR_TOO_LARGE = -8    /* a no-alloc call needs more than SSCAN_NOALLOC_SCRATCH_BYTES of workspace */
};

enum sscan_dtype { SSCAN_F32 = 0, SSCAN_BF16 = 1 };

/* Parameters of one scan direction (all device pointers). */
typedef struct sscan_dir_params {
  const void* delta;        /* [batch, dim, len] io_dtype, required (may alias the other direction's) */
  const float* delta_bias;  /* [dim], optional (NULL = 0) */
  const float* A;           /* [dim, dstate], required */
  const void* B;            /* [batch, dstate, len] bc_dtype, required */
  const void* C;            /* [batch, dstate, len] bc_dtype, required */
  const float* D;           /* [dim], optional (NULL = 0) */
} sscan_dir_params;

/* One direction.  Required: u, delta, A, B, C, y.  Optional: delta_bias, D, z.
 * A size of 0 in batch, dim or len is a valid empty call (nothing is enqueued). */
SSCAN_API int sscan_fwd(const void* u, const void* delta, const float* delta_bias, int softplus,
              const float* A, const void* B, const void* C, const float* D,
              const void* z, void* y,
              int64_t batch, int64_t dim, int64_t len, int64_t dstate,
              int reverse, void* stream,
              int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);

/* Both directions summed, gated once.  Required: u, y, fwd, rev and inside each
 * direction delta, A, B, C.  Optional: z and each direction's delta_bias and D. */
SSCAN_API int sscan_bidir(const void* u, const void* z, void* y,
                const sscan_dir_params* fwd, const sscan_dir_params* rev, int softplus,
                int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);

/* One direction with state I/O, for recurrent inference over a stream cut into
 * pieces (Hand-written simplified Mamba2 page, section 5.2: the fixed-size state is
 * all that carries from one step to the next; Mamba in the YOLO26 backbone page,
 * section 5.1: segments hand their hidden state on).  The same as sscan_fwd, and
 *   h0     [batch, dim, dstate] float32, optional: the state before the first scanned
 *          token (NULL = 0); with reverse != 0 the first scanned token is t = len-1;
 *   h_last [batch, dim, dstate] float32, optional: receives the state after the last
 *          scanned token (t = len-1 forward, t = 0 reverse).  With len == 0 it
 *          receives h0 (or zeros).
 * Calling this on consecutive pieces of a sequence, each h_last passed as the next
 * h0, gives the outputs of one call on the whole sequence (up to rounding).  Both
 * pointers must be 16-byte aligned.  h_last may be the same pointer as h0 (the
 * state is updated in place) but must not otherwise overlap h0, any input, y or
 * the workspace; y must not overlap h0.  Workspace: sscan_workspace_bytes(..., 0). */
SSCAN_API int sscan_fwd_state(const void* u, const void* delta, const float* delta_bias, int softplus,
                    const float* A, const void* B, const void* C, const float* D,
                    const void* z, void* y, const float* h0, float* h_last,
                    int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                    int reverse, void* stream,
                    int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);

/* One token of the recurrence from a stored state (single-step decode, same
 * passages as sscan_fwd_state): for every (b, d)
 *   h[b,d,:] <- exp(dt A[d,:]) * h[b,d,:] + dt * B[b,:] * u[b,d]
 *   y[b,d]    = (sum_n C[b,n] h[b,d,n] + D_d u[b,d]) * silu(z[b,d])
 * with dt as in sscan_fwd.  Layouts: state [batch, dim, dstate] float32 (read and
 * updated in place); u, delta, z, y [batch, dim] io_dtype; B, C [batch, dstate]
 * bc_dtype; A [dim, dstate], D and delta_bias [dim] float32.  state and A must be
 * 16-byte aligned, B and C aligned to four elements (16 bytes f32, 8 bytes bf16).
 * Required: state, u, delta, A, B, C, y; optional: delta_bias, D, z.  No
 * workspace.  state and y must not overlap each other or any input.  Equal to
 * sscan_fwd_state with len = 1 and h0 = h_last = state. */
SSCAN_API int sscan_step(float* state, const void* u, const void* delta, const float* delta_bias, int softplus,
               const float* A, const void* B, const void* C, const float* D,
               const void* z, void* y, int64_t batch, int64_t dim, int64_t dstate, void* stream,
               int io_dtype, int bc_dtype);

/* Depthwise convolution in front of the scan (Hand-written simplified Mamba2 page,
 * section 4.4: a per-channel Conv1d of d_conv taps padded by d_conv - 1 and cut back
 * to the sequence length, i.e. causal; Reproducing Vision Mamba page, section 3.2:
 * kernel 3 with 'same' padding).  For every (b, d, t):
 *   causal: out = bias_d + sum_{j<width} weight[d,j] * x[b,d,t - (width-1) + j]
 *   same:   out = bias_d + sum_{j<width} weight[d,j] * x[b,d,t - (width-1)/2 + j]
 * with x = 0 outside [0, len); then silu(out) when silu != 0 (the pages' layers use
 * no activation here; silu is an option). */
typedef struct sscan_conv_params {
  const float* weight;  /* [dim, width] float32, required */
  const float* bias;    /* [dim] float32, optional (NULL = 0) */
  int width;            /* taps: 1..4 causal, 1 or 3 centred */
  int same;             /* 0 causal, 1 centred ('same') */
  int silu;             /* 0 or 1 */
} sscan_conv_params;

/* The convolution alone: y = conv(x), x and y [batch, dim, len] io_dtype (device
 * pointers; y must not overlap x).  No workspace. */
SSCAN_API int sscan_conv1d(const void* x, const sscan_conv_params* conv, void* y,
                 int64_t batch, int64_t dim, int64_t len, void* stream, int io_dtype);

/* sscan_fwd / sscan_bidir on u = conv(x) computed inside the scan kernels: the
 * convolved sequence is never written to memory (both scan passes recompute it
 * from x and a 4-token halo).  Arguments as sscan_fwd / sscan_bidir with x in
 * place of u; workspace as there (sscan_workspace_bytes). */
SSCAN_API int sscan_fwd_conv(const void* x, const sscan_conv_params* conv, const void* delta, const float* delta_bias,
                   int softplus, const float* A, const void* B, const void* C, const float* D,
                   const void* z, void* y, int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                   int reverse, void* stream, int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);
SSCAN_API int sscan_bidir_conv(const void* x, const sscan_conv_params* conv, const void* z, void* y,
                     const sscan_dir_params* fwd, const sscan_dir_params* rev, int softplus,
                     int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                     int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);

/* The decode step (sscan_step) through the causal convolution in front of the
 * scan: the recurrent step of the Hand-written simplified Mamba2 page (section 5.2,
 * step(x_t, h, conv_state)), which keeps the last width - 1 inputs of the
 * convolution beside the scan state.  For every (b, d):
 *   window  = conv_state[b,d,0 .. width-2] (oldest first), then x[b,d]
 *   u       = bias_d + sum_{j<width} weight[d,j] * window[j]    (then silu(u) if conv->silu)
 *   state, y: one token of sscan_step on u
 *   conv_state[b,d,:] <- window[1 .. width-1]                    (x[b,d] appended, oldest dropped)
 * A zero conv_state is the convolution's zero padding before the first token, so
 * steps from zero states reproduce sscan_fwd_conv token by token.  conv must be
 * causal (conv->same == 0; a centred window needs the next token: SSCAN_ERR_UNSUPPORTED).
 * Layouts: conv_state [batch, dim, width - 1] io_dtype (read and updated in place;
 * NULL allowed when width == 1), x [batch, dim] io_dtype; the rest as sscan_step.
 * conv_state must not overlap any other argument.  No workspace. */
SSCAN_API int sscan_step_conv(float* state, void* conv_state, const void* x, const sscan_conv_params* conv,
                    const void* delta, const float* delta_bias, int softplus, const float* A, const void* B,
                    const void* C, const float* D, const void* z, void* y, int64_t batch, int64_t dim,
                    int64_t dstate, void* stream, int io_dtype, int bc_dtype);

/* Scans of a 2-D feature map along several visiting orders (Mamba in the YOLO26
 * backbone page, section 1.2: rows, columns or crosswise in several directions;
 * sections 2.2 and 4.4: row scans both ways, four directions; Samba page, section
 * 3.1: a centre-out spiral).  The map [height, width] is flattened row-major, token
 * t = r * width + c, so u, z, y and every direction's delta are [batch, dim,
 * height * width] and B, C [batch, dstate, height * width] in that token layout.
 * Direction k visits the tokens in the order kinds[k] names and has its own
 * parameters dirs[k]; its output is written at the tokens' own positions, the
 * directions are summed (in fp32) and gated once:
 *   out = (sum_k scan_k) * silu(z)          (z == NULL: no gate)
 * kinds: rows, columns (column by column, top to bottom), or the permutation
 * index[0 .. height*width) (a device int32 array, required when used; entries must
 * be a permutation of the tokens -- an entry outside [0, height*width) reads as 0,
 * and a token no entry names gets nothing from the index directions), each
 * forward or reversed; each kind at most once (1 to 6 directions).  Workspace:
 * sscan_multi_workspace_bytes(...) bytes, 256-byte aligned. */
enum sscan_order {
  SSCAN_ORDER_ROW = 0,
  SSCAN_ORDER_ROW_REV = 1,
  SSCAN_ORDER_COL = 2,
  SSCAN_ORDER_COL_REV = 3,
  SSCAN_ORDER_INDEX = 4,
  SSCAN_ORDER_INDEX_REV = 5
};
SSCAN_API int sscan_multi(const void* u, const void* z, void* y, const sscan_dir_params* dirs, const int* kinds,
                int ndirs, const int32_t* index, int softplus, int64_t batch, int64_t dim,
                int64_t height, int64_t width, int64_t dstate, void* stream, int io_dtype, int bc_dtype,
                void* workspace, size_t workspace_bytes);
SSCAN_API size_t sscan_multi_workspace_bytes(int64_t batch, int64_t dim, int64_t height, int64_t width,
                                   int64_t dstate, const int* kinds, int ndirs, int io_dtype, int bc_dtype);

/* The Samba page's centre-out clockwise spiral over a [height, width] map, read as
 * the square spiral right 1, down 1, left 2, up 2, right 3, ... from the centre cell
 * (the lower middle index of an even side; rows grow downwards), skipping cells
 * outside the map.  Writes height*width row-major token indices to `order` (HOST
 * memory, caller-owned) for SSCAN_ORDER_INDEX. */
SSCAN_API int sscan_spiral_order(int64_t height, int64_t width, int32_t* order);

/* Gradients of one direction's parameters (all device pointers, written by the
 * backward entry points). */
typedef struct sscan_dir_grads {
  void* ddelta;         /* [batch, dim, len] io_dtype, required (when it has elements) */
  float* ddelta_bias;   /* [dim], optional (NULL = not computed) */
  float* dA;            /* [dim, dstate], required (when it has elements) */
  void* dB;             /* [batch, dstate, len] bc_dtype, required (when it has elements) */
  void* dC;             /* [batch, dstate, len] bc_dtype, required (when it has elements) */
  float* dD;            /* [dim], optional (NULL = not computed) */
} sscan_dir_grads;

/* Backward pass of sscan_fwd (training: Reproducing Vision Mamba page, section 1.3,
 * hand-written gradients of the scan; Hand-written simplified Mamba2 page, section
 * 5.1, a custom backward that recomputes the forward states instead of storing
 * them).  Given dout = dLoss/dout [batch, dim, len] io_dtype for the output of
 * sscan_fwd with the same inputs, writes
 *   du [batch, dim, len] io_dtype (required), dz (required when z is given, else
 *   ignored), and grads->ddelta, ddelta_bias, dA, dB, dC, dD,
 * the exact gradients of sum(dout * out) up to float32 rounding (bf16 outputs
 * round to nearest even).  The forward states are recomputed in 32-token windows;
 * nothing from the forward call is needed.  Results are bitwise reproducible (no
 * atomics: every sum runs in a fixed order).  Workspace: sscan_bwd_workspace_bytes
 * (..., 0) bytes, 16-byte aligned (a few bytes per element: window entry states,
 * adjoints and partial sums).  Outputs must not overlap each other, any input or
 * the workspace; inputs may overlap each other.  An empty call (batch, dim or len
 * 0) writes zeros to the parameter gradients that have elements. */
SSCAN_API int sscan_bwd(const void* u, const void* delta, const float* delta_bias, int softplus,
              const float* A, const void* B, const void* C, const float* D,
              const void* z, const void* dout, void* du, void* dz, const sscan_dir_grads* grads,
              int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse, void* stream,
              int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);

/* Backward pass of sscan_fwd_state (one direction with state I/O): sscan_bwd's
 * arguments and outputs, and
 *   h0      [batch, dim, dstate] float32, optional: the forward call's entry state
 *           (NULL = 0);
 *   dh_last [batch, dim, dstate] float32, optional: dLoss/dh_last, the gradient
 *           reaching the forward's final state from outside (NULL = 0);
 *   dh0     [batch, dim, dstate] float32, optional output: dLoss/dh0, the gradient
 *           of the entry state (NULL = not computed).
 * The gradients are those of sum(dout * out) + sum(dh_last * h_last).  A learned
 * initial state (Samba page, section 3.2) takes dh0; a stream trained in pieces
 * (Hand-written simplified Mamba2 page, section 5.2) runs the pieces' backward in
 * reverse order, each dh0 passed on as the previous piece's dh_last.  All three
 * 16-byte aligned; dh0 overlaps nothing else, h0 and dh_last no output.  With
 * len == 0, dh0 = dh_last.  Workspace: sscan_bwd_workspace_bytes(..., 0). */
SSCAN_API int sscan_bwd_state(const void* u, const void* delta, const float* delta_bias, int softplus,
                    const float* A, const void* B, const void* C, const float* D, const void* z, const void* dout,
                    const float* h0, const float* dh_last, void* du, void* dz, const sscan_dir_grads* grads,
                    float* dh0, int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse, void* stream,
                    int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);
SSCAN_API int sscan_validate_bwd_state(const void* u, const void* delta, const float* delta_bias, int softplus,
                             const float* A, const void* B, const void* C, const float* D, const void* z,
                             const void* dout, const float* h0, const float* dh_last, const void* du,
                             const void* dz, const sscan_dir_grads* grads, const float* dh0, int64_t batch,
                             int64_t dim, int64_t len, int64_t dstate, int reverse, int io_dtype, int bc_dtype,
                             const void* workspace, size_t workspace_bytes);

/* Backward pass of sscan_bidir: du and dz of the shared u and z, and each
 * direction's parameter gradients in its own sscan_dir_grads (when both directions
 * read one delta tensor, its gradient is gfwd->ddelta + grev->ddelta).
 * Workspace: sscan_bwd_workspace_bytes(..., 1). */
SSCAN_API int sscan_bidir_bwd(const void* u, const void* z, const void* dout, void* du, void* dz,
                    const sscan_dir_params* fwd, const sscan_dir_params* rev,
                    const sscan_dir_grads* gfwd, const sscan_dir_grads* grev, int softplus,
                    int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                    int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);

/* Backward pass of sscan_multi (Mamba in the YOLO26 backbone page, sections 1.2,
 * 2.2 and 4.4, and Samba page, section 3.1, for the orders; Reproducing Vision
 * Mamba page, section 1.3: the scan block is trained with hand-written gradients).
 * Given dout [batch, dim, height*width] io_dtype for the output of sscan_multi with
 * the same inputs, writes du (required) and dz (required when z is given) in the
 * token layout, and for every direction k its own grads[k] (sscan_dir_grads;
 * ddelta, dB, dC in the token layout): the exact gradients of sum(dout * out) up to
 * float32 rounding.  Through the single gate, dout * silu(z) reaches every
 * direction's output and dz = dout * (sum_k scan_k) * silu'(z); each direction's
 * gradients are those of its own scan along its order; du sums them over the
 * directions in float32 and is rounded once.  index must be a permutation of the
 * tokens (the gradients of any other index are unspecified).  When two directions
 * read one tensor (a shared delta), its gradient is the sum of theirs.  Results
 * are bitwise reproducible.  Workspace: sscan_multi_bwd_workspace_bytes(...) bytes,
 * 256-byte aligned.  Outputs must not overlap each other, any input or the
 * workspace.  An empty call writes zeros to the parameter gradients that have
 * elements. */
SSCAN_API int sscan_multi_bwd(const void* u, const void* z, const void* dout, void* du, void* dz,
                    const sscan_dir_params* dirs, const sscan_dir_grads* grads, const int* kinds, int ndirs,
                    const int32_t* index, int softplus, int64_t batch, int64_t dim, int64_t height,
                    int64_t width, int64_t dstate, void* stream, int io_dtype, int bc_dtype, void* workspace,
                    size_t workspace_bytes);
SSCAN_API int sscan_validate_multi_bwd(const void* u, const void* z, const void* dout, const void* du,
                             const void* dz, const sscan_dir_params* dirs, const sscan_dir_grads* grads,
                             const int* kinds, int ndirs, const int32_t* index, int softplus, int64_t batch,
                             int64_t dim, int64_t height, int64_t width, int64_t dstate, int io_dtype,
                             int bc_dtype, const void* workspace, size_t workspace_bytes);
SSCAN_API size_t sscan_multi_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t height, int64_t width,
                                       int64_t dstate, const int* kinds, int ndirs, int io_dtype,
                                       int bc_dtype);

/* Backward of sscan_fwd_conv / sscan_bidir_conv: the scan's gradients taken at
 * u = conv(x), and du carried back through the convolution (Reproducing Vision
 * Mamba page, section 1.3: the block is trained with hand-written gradients;
 * Hand-written simplified Mamba2 page, sections 4.4 and 5.1: the convolution sits
 * inside the trained block).  Arguments as sscan_bwd / sscan_bidir_bwd with x in
 * place of u and dx [batch, dim, len] io_dtype in place of du, and
 *   dconv_w [dim, width] float32 (required), dconv_b [dim] float32 (required when
 *   conv->bias is given, else ignored): sums over batch rows and tokens.
 * u = conv(x) is recomputed in float32, as the fused forward computes it (never
 * rounded to the io dtype), and du reaches the convolution's backward in float32.  Results are
 * bitwise reproducible (fixed-order sums).  Workspace:
 * sscan_bwd_conv_workspace_bytes(..., bidir, io_dtype) bytes, 256-byte aligned.  An
 * empty call writes zeros to the parameter gradients that have elements. */
SSCAN_API int sscan_bwd_conv(const void* x, const sscan_conv_params* conv, const void* delta, const float* delta_bias,
                   int softplus, const float* A, const void* B, const void* C, const float* D, const void* z,
                   const void* dout, void* dx, void* dz, const sscan_dir_grads* grads, float* dconv_w,
                   float* dconv_b, int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse,
                   void* stream, int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);
SSCAN_API int sscan_bidir_bwd_conv(const void* x, const sscan_conv_params* conv, const void* z, const void* dout,
                         void* dx, void* dz, const sscan_dir_params* fwd, const sscan_dir_params* rev,
                         const sscan_dir_grads* gfwd, const sscan_dir_grads* grev, float* dconv_w, float* dconv_b,
                         int softplus, int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                         int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes);
SSCAN_API int sscan_validate_bwd_conv(const void* x, const sscan_conv_params* conv, const void* delta,
                            const float* delta_bias, int softplus, const float* A, const void* B, const void* C,
                            const float* D, const void* z, const void* dout, const void* dx, const void* dz,
                            const sscan_dir_grads* grads, const float* dconv_w, const float* dconv_b,
                            int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse, int io_dtype,
                            int bc_dtype, const void* workspace, size_t workspace_bytes);
SSCAN_API size_t sscan_bwd_conv_workspace_bytes(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir,
                                      int io_dtype);

/* Bytes of device workspace a backward call needs (0 if none or invalid sizes). */
SSCAN_API size_t sscan_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir);

/* Profiling variants (for timing the internal steps of a call, not needed for
 * results): the same work as sscan_fwd / sscan_bidir, and on the same stream
 * events[0] is recorded before the first kernel and events[k] after step k of
 * the call: 1 = B/C staging, 2 = segment aggregates, 3 = carry chain between
 * segments, 4 = output pass.  Steps a call does not need (an unsplit sequence has
 * no aggregate or carry step) get zero-length intervals.  events holds
 * SSCAN_PROFILE_EVENTS hipEvent_t handles created by the caller (NULL entries are
 * skipped; events itself may be NULL). */
#define SSCAN_PROFILE_EVENTS 5
SSCAN_API int sscan_fwd_profiled(const void* u, const void* delta, const float* delta_bias, int softplus,
                       const float* A, const void* B, const void* C, const float* D,
                       const void* z, void* y,
                       int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                       int reverse, void* stream,
                       int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes,
                       void* const* events);
SSCAN_API int sscan_bidir_profiled(const void* u, const void* z, void* y,
                         const sscan_dir_params* fwd, const sscan_dir_params* rev, int softplus,
                         int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                         int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes,
                         void* const* events);

/* Profiling variants of sscan_fwd_conv / sscan_bidir_conv: events as for
 * sscan_fwd_profiled (SSCAN_PROFILE_EVENTS handles). */
SSCAN_API int sscan_fwd_conv_profiled(const void* x, const sscan_conv_params* conv, const void* delta,
                            const float* delta_bias, int softplus, const float* A, const void* B,
                            const void* C, const float* D, const void* z, void* y,
                            int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse, void* stream,
                            int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes,
                            void* const* events);
SSCAN_API int sscan_bidir_conv_profiled(const void* x, const sscan_conv_params* conv, const void* z, void* y,
                              const sscan_dir_params* fwd, const sscan_dir_params* rev, int softplus,
                              int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                              int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes,
                              void* const* events);

/* Profiling variants of the backward entry points: the same work, and events[0]
 * is recorded before the first kernel and events[k] after step k: 1 = B/C staging,
 * 2 = states entering every window (segment aggregates and carry chain), 3 = the
 * adjoints entering every window from the other side, 4 = the window pass(es),
 * 5 = the sums of the parameter gradients.  events holds SSCAN_BWD_PROFILE_EVENTS
 * hipEvent_t handles (NULL entries skipped; events may be NULL). */
#define SSCAN_BWD_PROFILE_EVENTS 6
SSCAN_API int sscan_bwd_profiled(const void* u, const void* delta, const float* delta_bias, int softplus,
                       const float* A, const void* B, const void* C, const float* D,
                       const void* z, const void* dout, void* du, void* dz, const sscan_dir_grads* grads,
                       int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse, void* stream,
                       int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes,
                       void* const* events);
SSCAN_API int sscan_bidir_bwd_profiled(const void* u, const void* z, const void* dout, void* du, void* dz,
                             const sscan_dir_params* fwd, const sscan_dir_params* rev,
                             const sscan_dir_grads* gfwd, const sscan_dir_grads* grev, int softplus,
                             int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                             int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes,
                             void* const* events);

/* Same checks as sscan_fwd / sscan_bidir without touching the GPU: returns the
 * status the call would return before any launch.  workspace is only compared with
 * the required size (it is never dereferenced). */
SSCAN_API int sscan_validate_fwd(const void* u, const void* delta, const float* delta_bias, int softplus,
                       const float* A, const void* B, const void* C, const float* D,
                       const void* z, const void* y,
                       int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                       int reverse, int io_dtype, int bc_dtype,
                       const void* workspace, size_t workspace_bytes);
SSCAN_API int sscan_validate_bidir(const void* u, const void* z, const void* y,
                         const sscan_dir_params* fwd, const sscan_dir_params* rev, int softplus,
                         int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                         int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes);

SSCAN_API int sscan_validate_fwd_state(const void* u, const void* delta, const float* delta_bias, int softplus,
                             const float* A, const void* B, const void* C, const float* D,
                             const void* z, const void* y, const float* h0, const float* h_last,
                             int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                             int reverse, int io_dtype, int bc_dtype,
                             const void* workspace, size_t workspace_bytes);
SSCAN_API int sscan_validate_step(const float* state, const void* u, const void* delta, const float* delta_bias,
                        int softplus, const float* A, const void* B, const void* C, const float* D,
                        const void* z, const void* y, int64_t batch, int64_t dim, int64_t dstate,
                        int io_dtype, int bc_dtype);

SSCAN_API int sscan_validate_step_conv(const float* state, const void* conv_state, const void* x,
                             const sscan_conv_params* conv, const void* delta, const float* delta_bias, int softplus,
                             const float* A, const void* B, const void* C, const float* D, const void* z,
                             const void* y, int64_t batch, int64_t dim, int64_t dstate, int io_dtype, int bc_dtype);

SSCAN_API int sscan_validate_bwd(const void* u, const void* delta, const float* delta_bias, int softplus,
                       const float* A, const void* B, const void* C, const float* D,
                       const void* z, const void* dout, const void* du, const void* dz,
                       const sscan_dir_grads* grads, int64_t batch, int64_t dim, int64_t len,
                       int64_t dstate, int reverse, int io_dtype, int bc_dtype,
                       const void* workspace, size_t workspace_bytes);
SSCAN_API int sscan_validate_bidir_bwd(const void* u, const void* z, const void* dout, const void* du,
                             const void* dz, const sscan_dir_params* fwd, const sscan_dir_params* rev,
                             const sscan_dir_grads* gfwd, const sscan_dir_grads* grev, int softplus,
                             int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                             int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes);

SSCAN_API int sscan_validate_conv1d(const void* x, const sscan_conv_params* conv, const void* y,
                          int64_t batch, int64_t dim, int64_t len, int io_dtype);

SSCAN_API int sscan_validate_multi(const void* u, const void* z, const void* y, const sscan_dir_params* dirs,
                         const int* kinds, int ndirs, const int32_t* index, int softplus, int64_t batch,
                         int64_t dim, int64_t height, int64_t width, int64_t dstate, int io_dtype, int bc_dtype,
                         const void* workspace, size_t workspace_bytes);

/* sscan_fwd for callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same operation,
 * arguments, layouts and checks as sscan_fwd, without the workspace arguments.  The
 * workspace comes from a fixed device array of the library, SSCAN_NOALLOC_SCRATCH_BYTES
 * bytes on every GPU the library runs on, held until the process ends.  A call that
 * needs more (sscan_workspace_bytes(batch, dim, len, dstate, 0) above that) returns
 * SSCAN_ERR_TOO_LARGE before any HIP call.  The array of the CURRENT device is used,
 * so `stream` must belong to the current device.  The call allocates no memory (no
 * hipMalloc, no allocating library routine); the first call on a device looks up
 * that device's copy of the array once.  Every call on one GPU shares that GPU's
 * array: calls that may overlap in time on one GPU (different streams, different
 * host threads) race and must be ordered by the caller.  The array's contents on
 * entry do not matter. */
#define SSCAN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
SSCAN_API int sscan_fwd_noalloc(const void* u, const void* delta, const float* delta_bias, int softplus,
                      const float* A, const void* B, const void* C, const float* D,
                      const void* z, void* y,
                      int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                      int reverse, void* stream, int io_dtype, int bc_dtype);

/* Bytes of device workspace a call with these sizes needs (0 if none); bidir != 0
 * for sscan_bidir.  Returns 0 for invalid sizes (the call itself reports them). */
SSCAN_API size_t sscan_workspace_bytes(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir);

/* How sscan_fwd / sscan_bidir (and the scans inside sscan_multi) split a sequence
 * of these sizes, for tools and tests: out[0] tokens per segment, out[1] segments
 * per row (1: scanned whole, no aggregate or carry kernels), out[2] segments per
 * aggregate run (runs > 1 segment: the aggregate pass walks a run from a zero state
 * and the carry chains only the runs' totals), out[3] runs per row.  out is HOST
 * memory (4 entries).  Returns SSCAN_OK, SSCAN_ERR_NULL, SSCAN_ERR_SHAPE or
 * SSCAN_ERR_UNSUPPORTED (dstate != 16). */
SSCAN_API int sscan_scan_plan(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir, int64_t* out);

/* How sscan_bwd / sscan_bidir_bwd split a call of these sizes, for tools and
 * tests: out[0] 32-token windows per row, out[1] blocks each window's channel
 * groups (four channels each) are split over, out[2] channel groups per block,
 * out[3] windows per chain run (the window entry states and adjoints are walked
 * over runs of consecutive windows), out[4] runs per row.  out is HOST memory
 * (5 entries).  Returns SSCAN_OK, SSCAN_ERR_NULL, SSCAN_ERR_SHAPE or
 * SSCAN_ERR_UNSUPPORTED (dstate != 16). */
SSCAN_API int sscan_bwd_plan(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir, int64_t* out);

/* Static description of a status code; never NULL. */
SSCAN_API const char* sscan_strerror(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
SSCAN_API int sscan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSCAN_H_ */
