// sscan_capi.cpp -- C ABI of the selective scan: argument checks, then one call
// into the kernel launcher.  Every check happens before any HIP call, so the
// validate entry points work on a machine without a GPU.
#include "sscan.h"

#include <cstdint>
#include <cstring>

#include "sscan_internal.h"

namespace {

constexpr int kVersion = 200;  // 0.2.0
static_assert(SSCAN_PROFILE_EVENTS == sscan::kProfileEvents, "event count mismatch");
static_assert(SSCAN_BWD_PROFILE_EVENTS == sscan::kBwdProfileEvents, "event count mismatch");

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

struct Sizes {
  size_t io_elems;   // batch * dim * len
  size_t bc_elems;   // batch * 16 * len
  size_t io_esz, bc_esz;
};

// Checks sizes and dtype codes; fills Sizes.  Returns SSCAN_OK or an error.
int check_sizes(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int io_dtype, int bc_dtype,
                Sizes* sz) {
  if (batch < 0 || dim < 0 || len < 0) return SSCAN_ERR_SHAPE;
  if (dstate != sscan::kDState) return SSCAN_ERR_UNSUPPORTED;
  if ((io_dtype != SSCAN_F32 && io_dtype != SSCAN_BF16) || (bc_dtype != SSCAN_F32 && bc_dtype != SSCAN_BF16))
    return SSCAN_ERR_UNSUPPORTED;
  int64_t bd = 0, n_io = 0, n_bc = 0, b16 = 0, bl = 0;
  // batch * len <= 2^36 keeps every one-dimensional grid of the kernels below 2^32
  // blocks (the B/C staging launches one block per 64 tokens of each row); inputs
  // that large would not fit in device memory anyway.
  if (__builtin_mul_overflow(batch, dim, &bd) || __builtin_mul_overflow(bd, len, &n_io) ||
      __builtin_mul_overflow(batch, int64_t(sscan::kDState), &b16) || __builtin_mul_overflow(b16, len, &n_bc) ||
      __builtin_mul_overflow(batch, len, &bl) || bl > (int64_t(1) << 36) ||
      n_io > (int64_t(1) << 50) || n_bc > (int64_t(1) << 50) || dim > (int64_t(1) << 40))
    return SSCAN_ERR_SHAPE;
  sz->io_elems = size_t(n_io);
  sz->bc_elems = size_t(n_bc);
  sz->io_esz = io_dtype == SSCAN_BF16 ? 2 : 4;
  sz->bc_esz = bc_dtype == SSCAN_BF16 ? 2 : 4;
  return SSCAN_OK;
}

struct DirView {
  const void* delta;
  const float* delta_bias;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
};

int check_dir(const DirView& p, const Sizes& sz, int64_t dim, const Range& y) {
  if (!p.delta || !p.A || !p.B || !p.C) return SSCAN_ERR_NULL;
  if (!aligned(p.delta, sz.io_esz) || !aligned(p.B, sz.bc_esz) || !aligned(p.C, sz.bc_esz) ||
      !aligned(p.A, 4) || !aligned(p.delta_bias, 4) || !aligned(p.D, 4))
    return SSCAN_ERR_ALIGN;
  const size_t vec = size_t(dim) * 4;
  if (overlap(y, range_of(p.delta, sz.io_elems * sz.io_esz)) || overlap(y, range_of(p.B, sz.bc_elems * sz.bc_esz)) ||
      overlap(y, range_of(p.C, sz.bc_elems * sz.bc_esz)) || overlap(y, range_of(p.A, vec * sscan::kDState)) ||
      (p.delta_bias && overlap(y, range_of(p.delta_bias, vec))) || (p.D && overlap(y, range_of(p.D, vec))))
    return SSCAN_ERR_ALIAS;
  return SSCAN_OK;
}

// The front-end convolution: causal kernels of 1..4 taps, or centred ('same') ones
// of 1 or 3 taps; fp32 weights [dim][width] and optional bias [dim].
int check_conv(const sscan_conv_params* c, int64_t dim, const Range& y) {
  if (!c) return SSCAN_OK;
  if (!c->weight) return SSCAN_ERR_NULL;
  if (c->width < 1 || (c->same ? (c->width % 2 == 0 || c->width > 3) : c->width > 4) ||
      (c->same != 0 && c->same != 1) || (c->silu != 0 && c->silu != 1))
    return SSCAN_ERR_UNSUPPORTED;
  if (!aligned(c->weight, 4) || !aligned(c->bias, 4)) return SSCAN_ERR_ALIGN;
  if (overlap(y, range_of(c->weight, size_t(dim) * size_t(c->width) * 4)) ||
      (c->bias && overlap(y, range_of(c->bias, size_t(dim) * 4))))
    return SSCAN_ERR_ALIAS;
  return SSCAN_OK;
}

int conv_left(const sscan_conv_params* c) { return c->same ? (c->width - 1) / 2 : c->width - 1; }

// Shared by the run and validate entry points.  On success *plan is filled and
// *empty tells whether there is nothing to do.
int validate(const void* u, const void* z, const void* y, const DirView* dirs, int ndir, int64_t batch, int64_t dim,
             int64_t len, int64_t dstate, int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes,
             sscan::Plan* plan, bool* empty, const sscan_conv_params* conv = nullptr) {
  Sizes sz{};
  int st = check_sizes(batch, dim, len, dstate, io_dtype, bc_dtype, &sz);
  if (st != SSCAN_OK) return st;
  *empty = (batch == 0 || dim == 0 || len == 0);
  if (*empty) return SSCAN_OK;
  if (!u || !y) return SSCAN_ERR_NULL;
  for (int k = 0; k < ndir; ++k)
    if (!dirs[k].delta || !dirs[k].A || !dirs[k].B || !dirs[k].C) return SSCAN_ERR_NULL;
  if (!aligned(u, sz.io_esz) || !aligned(y, sz.io_esz) || !aligned(z, sz.io_esz)) return SSCAN_ERR_ALIGN;
  const Range yr = range_of(y, sz.io_elems * sz.io_esz);
  if (overlap(yr, range_of(u, sz.io_elems * sz.io_esz)) || (z && overlap(yr, range_of(z, sz.io_elems * sz.io_esz))))
    return SSCAN_ERR_ALIAS;
  for (int k = 0; k < ndir; ++k) {
    st = check_dir(dirs[k], sz, dim, yr);
    if (st != SSCAN_OK) return st;
  }
  st = check_conv(conv, dim, yr);
  if (st != SSCAN_OK) return st;
  *plan = sscan::make_plan(batch, dim, len, ndir);
  if (!sscan::plan_fits_grid(*plan, batch, dim, len, ndir)) return SSCAN_ERR_SHAPE;
  if (plan->workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan->workspace_bytes) return SSCAN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return SSCAN_ERR_ALIGN;
    if (overlap(yr, range_of(workspace, plan->workspace_bytes))) return SSCAN_ERR_ALIAS;
  }
  return SSCAN_OK;
}

// Entry and final state of a single-direction call: 16-byte aligned [batch][dim][16]
// fp32; h_last may be h0 itself but must not overlap anything else the call reads
// or writes, and y must not overlap h0.
int check_state(const float* h0, float* h_last, const void* u, const void* z, const void* y, const DirView& p,
                int64_t batch, int64_t dim, int64_t len, int io_dtype, int bc_dtype, const void* workspace,
                size_t workspace_bytes) {
  if (!aligned(h0, 16) || !aligned(h_last, 16)) return SSCAN_ERR_ALIGN;
  Sizes sz{};
  const int st = check_sizes(batch, dim, len, sscan::kDState, io_dtype, bc_dtype, &sz);
  if (st != SSCAN_OK) return st;
  const size_t sbytes = size_t(batch) * size_t(dim) * sscan::kDState * 4;
  const Range h0r = h0 ? range_of(h0, sbytes) : Range{0, 0};
  const Range hlr = h_last ? range_of(h_last, sbytes) : Range{0, 0};
  const size_t io = sz.io_elems * sz.io_esz, bcb = sz.bc_elems * sz.bc_esz, vec = size_t(dim) * 4;
  const Range others[] = {range_of(u, io),       range_of(z, z ? io : 0),       range_of(y, io),
                          range_of(p.delta, io), range_of(p.B, bcb),            range_of(p.C, bcb),
                          range_of(p.A, vec * sscan::kDState), range_of(p.delta_bias, p.delta_bias ? vec : 0),
                          range_of(p.D, p.D ? vec : 0), range_of(workspace, workspace ? workspace_bytes : 0)};
  for (const Range& r : others)
    if (overlap(hlr, r)) return SSCAN_ERR_ALIAS;
  if (overlap(h0r, range_of(y, io)) || overlap(h0r, range_of(workspace, workspace ? workspace_bytes : 0)))
    return SSCAN_ERR_ALIAS;
  if (h0 && h_last && overlap(h0r, hlr) && h0r.lo != hlr.lo) return SSCAN_ERR_ALIAS;
  return SSCAN_OK;
}

sscan::ScanArgs make_args(const void* u, const void* z, void* y, const DirView* dirs, int ndir, int reverse,
                          int softplus, int64_t batch, int64_t dim, int64_t len, int io_dtype, int bc_dtype) {
  sscan::ScanArgs a;
  std::memset(&a, 0, sizeof(a));
  a.u = u;
  a.z = z;
  a.y = y;
  for (int k = 0; k < ndir; ++k)
    a.dir[k] = sscan::DirArgs{dirs[k].delta, dirs[k].delta_bias, dirs[k].A, dirs[k].B, dirs[k].C, dirs[k].D};
  a.ndir = ndir;
  a.reverse = reverse ? 1 : 0;
  a.softplus = softplus ? 1 : 0;
  a.io_bf16 = io_dtype == SSCAN_BF16;
  a.bc_bf16 = bc_dtype == SSCAN_BF16;
  a.batch = batch;
  a.dim = dim;
  a.len = len;
  return a;
}

int validate_state_call(const void* u, const void* z, const void* y, const DirView& d, const float* h0,
                        float* h_last, int64_t batch, int64_t dim, int64_t len, int64_t dstate, int io_dtype,
                        int bc_dtype, const void* workspace, size_t workspace_bytes, sscan::Plan* plan,
                        bool* empty) {
  int st = validate(u, z, y, &d, 1, batch, dim, len, dstate, io_dtype, bc_dtype, workspace, workspace_bytes, plan,
                    empty);
  if (st != SSCAN_OK) return st;
  if (batch == 0 || dim == 0) return SSCAN_OK;  // no state at all
  return check_state(h0, h_last, u, z, y, d, batch, dim, len, io_dtype, bc_dtype, workspace, workspace_bytes);
}

int run(const void* u, const void* z, void* y, const DirView* dirs, int ndir, int reverse, int softplus,
        int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream, int io_dtype, int bc_dtype,
        void* workspace, size_t workspace_bytes, void* const* events = nullptr, const float* h0 = nullptr,
        float* h_last = nullptr, const sscan_conv_params* conv = nullptr) {
  sscan::Plan plan{};
  bool empty = false;
  const bool state = h0 || h_last;
  const int st = state ? validate_state_call(u, z, y, dirs[0], h0, h_last, batch, dim, len, dstate, io_dtype,
                                             bc_dtype, workspace, workspace_bytes, &plan, &empty)
                       : validate(u, z, y, dirs, ndir, batch, dim, len, dstate, io_dtype, bc_dtype, workspace,
                                  workspace_bytes, &plan, &empty, conv);
  if (st != SSCAN_OK) return st;
  sscan::ScanArgs a = make_args(u, z, y, dirs, ndir, reverse, softplus, batch, dim, len, io_dtype, bc_dtype);
  a.h0 = h0;
  a.h_last = h_last;
  if (conv) {
    a.conv_w = conv->weight;
    a.conv_b = conv->bias;
    a.conv_width = conv->width;
    a.conv_left = conv_left(conv);
    a.conv_silu = conv->silu;
  }
  if (empty) {
    // no tokens: the final state is the entry state
    if (len == 0 && h_last && h_last != h0 && batch > 0 && dim > 0) {
      const hipError_t e = sscan::launch_state_passthrough(a, static_cast<hipStream_t>(stream));
      return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
    }
    return SSCAN_OK;
  }
  hipEvent_t ev[sscan::kProfileEvents] = {};
  if (events)
    for (int i = 0; i < sscan::kProfileEvents; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  const hipError_t e = sscan::launch_scan(a, plan, static_cast<float*>(workspace), static_cast<hipStream_t>(stream),
                                          events ? ev : nullptr);
  return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
}

DirView view_of(const sscan_dir_params* p) {
  return DirView{p->delta, p->delta_bias, p->A, p->B, p->C, p->D};
}

// ---- backward ----------------------------------------------------------------------

constexpr int kMaxRanges = 64;

struct RangeSet {
  Range r[kMaxRanges];
  int n = 0;
  void add(const void* p, size_t bytes) {
    if (p && bytes && n < kMaxRanges) r[n++] = range_of(p, bytes);
  }
};

// One direction of a backward call: alignment of its parameters and gradients,
// and their ranges (gradients as outputs, parameters as inputs when not empty).
int add_bwd_dir(const DirView& p, const sscan_dir_grads& g, const Sizes& sz, int64_t dim, bool empty, RangeSet* in,
                RangeSet* out) {
  const size_t io = sz.io_elems * sz.io_esz, bcb = sz.bc_elems * sz.bc_esz, vec = size_t(dim) * 4;
  if (!aligned(p.A, 4) || !aligned(p.delta_bias, 4) || !aligned(p.D, 4) || !aligned(g.dA, 4) ||
      !aligned(g.ddelta_bias, 4) || !aligned(g.dD, 4) || !aligned(g.dB, sz.bc_esz) || !aligned(g.dC, sz.bc_esz))
    return SSCAN_ERR_ALIGN;
  out->add(g.dA, vec * sscan::kDState);
  out->add(g.ddelta_bias, vec);
  out->add(g.dD, vec);
  out->add(g.dB, bcb);
  out->add(g.dC, bcb);
  if (!empty) {
    if (!aligned(p.delta, sz.io_esz) || !aligned(p.B, sz.bc_esz) || !aligned(p.C, sz.bc_esz) ||
        !aligned(g.ddelta, sz.io_esz))
      return SSCAN_ERR_ALIGN;
    in->add(p.delta, io);
    in->add(p.B, bcb);
    in->add(p.C, bcb);
    in->add(p.A, vec * sscan::kDState);
    in->add(p.delta_bias, vec);
    in->add(p.D, vec);
    out->add(g.ddelta, io);
  }
  return SSCAN_OK;
}

// Outputs overlap neither each other nor any input.
int disjoint(const RangeSet& in, const RangeSet& out) {
  for (int i = 0; i < out.n; ++i) {
    for (int j = 0; j < in.n; ++j)
      if (overlap(out.r[i], in.r[j])) return SSCAN_ERR_ALIAS;
    for (int j = i + 1; j < out.n; ++j)
      if (overlap(out.r[i], out.r[j])) return SSCAN_ERR_ALIAS;
  }
  return SSCAN_OK;
}

// Checks a backward call; on success fills *plan and *empty.
int validate_bwd(const void* u, const void* z, const void* dout, const void* du, const void* dz, const DirView* dirs,
                 const sscan_dir_grads* grads, int ndir, int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                 int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes, sscan::BwdPlan* plan,
                 bool* empty) {
  Sizes sz{};
  int st = check_sizes(batch, dim, len, dstate, io_dtype, bc_dtype, &sz);
  if (st != SSCAN_OK) return st;
  // a gradient buffer is required whenever it has elements
  for (int k = 0; k < ndir; ++k)
    if ((dim > 0 && !grads[k].dA) || (sz.bc_elems > 0 && (!grads[k].dB || !grads[k].dC))) return SSCAN_ERR_NULL;
  *empty = (batch == 0 || dim == 0 || len == 0);
  const size_t io = sz.io_elems * sz.io_esz;
  RangeSet in, out;
  if (!*empty) {
    if (!u || !dout || !du || (z && !dz)) return SSCAN_ERR_NULL;
    for (int k = 0; k < ndir; ++k)
      if (!dirs[k].delta || !dirs[k].A || !dirs[k].B || !dirs[k].C || !grads[k].ddelta) return SSCAN_ERR_NULL;
    const void* io_ptrs[] = {u, z, dout, du, dz};
    for (const void* q : io_ptrs)
      if (!aligned(q, sz.io_esz)) return SSCAN_ERR_ALIGN;
    in.add(u, io);
    in.add(z, io);
    in.add(dout, io);
    out.add(du, io);
    if (z) out.add(dz, io);
  }
  for (int k = 0; k < ndir; ++k) {
    st = add_bwd_dir(dirs[k], grads[k], sz, dim, *empty, &in, &out);
    if (st != SSCAN_OK) return st;
  }
  if (!*empty) {
    *plan = sscan::make_bwd_plan(batch, dim, len, ndir);
    if (!sscan::bwd_plan_fits_grid(*plan, batch, dim, len, ndir)) return SSCAN_ERR_SHAPE;
    if (!workspace || workspace_bytes < plan->workspace_bytes) return SSCAN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return SSCAN_ERR_ALIGN;
    out.add(workspace, plan->workspace_bytes);
  }
  return disjoint(in, out);
}

// State I/O of a one-direction backward: h0 and dh_last (inputs) and dh0 (output),
// [batch][dim][16] float32, 16-byte aligned; dh0 overlaps nothing else of the call.
int check_bwd_state(const float* h0, const float* dh_last, const float* dh0, const void* u, const void* z,
                    const void* dout, const void* du, const void* dz, const DirView& p, const sscan_dir_grads& g,
                    int64_t batch, int64_t dim, int64_t len, int io_dtype, int bc_dtype, const void* workspace,
                    size_t workspace_bytes) {
  if (!aligned(h0, 16) || !aligned(dh_last, 16) || !aligned(dh0, 16)) return SSCAN_ERR_ALIGN;
  Sizes sz{};
  const int st = check_sizes(batch, dim, len, sscan::kDState, io_dtype, bc_dtype, &sz);
  if (st != SSCAN_OK) return st;
  const size_t sbytes = size_t(batch) * size_t(dim) * sscan::kDState * 4;
  const size_t io = sz.io_elems * sz.io_esz, bcb = sz.bc_elems * sz.bc_esz, vec = size_t(dim) * 4;
  const Range outr = range_of(dh0, dh0 ? sbytes : 0);
  const Range others[] = {range_of(h0, h0 ? sbytes : 0), range_of(dh_last, dh_last ? sbytes : 0),
                          range_of(u, io), range_of(z, z ? io : 0), range_of(dout, io), range_of(du, io),
                          range_of(dz, dz ? io : 0), range_of(p.delta, io), range_of(p.B, bcb), range_of(p.C, bcb),
                          range_of(p.A, vec * sscan::kDState), range_of(p.delta_bias, p.delta_bias ? vec : 0),
                          range_of(p.D, p.D ? vec : 0), range_of(g.ddelta, io), range_of(g.dA, vec * sscan::kDState),
                          range_of(g.dB, bcb), range_of(g.dC, bcb), range_of(g.ddelta_bias, g.ddelta_bias ? vec : 0),
                          range_of(g.dD, g.dD ? vec : 0), range_of(workspace, workspace ? workspace_bytes : 0)};
  for (const Range& r : others)
    if (overlap(outr, r)) return SSCAN_ERR_ALIAS;
  // the state inputs are read while the gradients are written
  const Range outs[] = {range_of(du, io), range_of(dz, dz ? io : 0), range_of(g.ddelta, io),
                        range_of(g.dA, vec * sscan::kDState), range_of(g.dB, bcb), range_of(g.dC, bcb),
                        range_of(g.ddelta_bias, g.ddelta_bias ? vec : 0), range_of(g.dD, g.dD ? vec : 0),
                        range_of(workspace, workspace ? workspace_bytes : 0)};
  for (const Range& r : outs)
    if (overlap(range_of(h0, h0 ? sbytes : 0), r) || overlap(range_of(dh_last, dh_last ? sbytes : 0), r))
      return SSCAN_ERR_ALIAS;
  return SSCAN_OK;
}

int run_bwd(const void* u, const void* z, const void* dout, void* du, void* dz, const DirView* dirs,
            const sscan_dir_grads* grads, int ndir, int reverse, int softplus, int64_t batch, int64_t dim,
            int64_t len, int64_t dstate, void* stream, int io_dtype, int bc_dtype, void* workspace,
            size_t workspace_bytes, void* const* events = nullptr, const float* h0 = nullptr,
            const float* dh_last = nullptr, float* dh0 = nullptr) {
  sscan::BwdPlan plan{};
  bool empty = false;
  int st = validate_bwd(u, z, dout, du, dz, dirs, grads, ndir, batch, dim, len, dstate, io_dtype, bc_dtype,
                        workspace, workspace_bytes, &plan, &empty);
  if (st != SSCAN_OK) return st;
  if (h0 || dh_last || dh0) {
    st = check_bwd_state(h0, dh_last, dh0, u, z, dout, du, dz, dirs[0], grads[0], batch, dim, len, io_dtype,
                         bc_dtype, workspace, workspace_bytes);
    if (st != SSCAN_OK) return st;
  }
  sscan::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.fwd = make_args(u, z, nullptr, dirs, ndir, reverse, softplus, batch, dim, len, io_dtype, bc_dtype);
  a.fwd.h0 = h0;
  a.dh_last = dh_last;
  a.dh0 = dh0;
  a.dout = dout;
  a.du = du;
  a.dz = dz;
  for (int k = 0; k < ndir; ++k)
    a.grads[k] = sscan::DirGrads{grads[k].ddelta, grads[k].ddelta_bias, grads[k].dA, grads[k].dB, grads[k].dC,
                                 grads[k].dD};
  hipEvent_t ev[sscan::kBwdProfileEvents] = {};
  if (events)
    for (int i = 0; i < sscan::kBwdProfileEvents; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  hipError_t e = empty ? sscan::launch_bwd_zero(a, static_cast<hipStream_t>(stream))
                       : sscan::launch_bwd(a, plan, static_cast<float*>(workspace), static_cast<hipStream_t>(stream),
                                           events ? ev : nullptr);
  if (e == hipSuccess && empty && dh0 && batch > 0 && dim > 0) {
    // no tokens: the final state is the entry state, so dh0 = dh_last (or zeros)
    sscan::ScanArgs pass = a.fwd;
    pass.h0 = dh_last;
    pass.h_last = dh0;
    e = sscan::launch_state_passthrough(pass, static_cast<hipStream_t>(stream));
  }
  return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
}

// ---- backward through the front-end convolution ------------------------------------

// Workspace of a backward call through the convolution: the scan backward's own,
// then u = conv(x) and its gradient du (both float32: u as the fused forward
// computes it, du unrounded for the convolution's gradients), then the
// convolution's partial sums (floats); sections 256-byte aligned.
struct ConvBwdLayout {
  sscan::BwdPlan plan;
  size_t off_u, off_du, off_part, bytes;
};

ConvBwdLayout conv_bwd_layout(int64_t batch, int64_t dim, int64_t len, int ndir, size_t io_esz) {
  ConvBwdLayout l{};
  auto up = [](size_t n) { return (n + 255) / 256 * 256; };
  l.plan = sscan::make_bwd_plan(batch, dim, len, ndir);
  (void)io_esz;
  const size_t n32 = size_t(batch) * size_t(dim) * size_t(len) * sizeof(float);
  l.off_u = up(l.plan.workspace_bytes);
  l.off_du = l.off_u + up(n32);
  l.off_part = l.off_du + up(n32);
  l.bytes = l.off_part + up(sscan::conv_bwd_partial_floats(batch, dim, len) * sizeof(float));
  return l;
}

// The scan backward's checks with x in u's place and dx in du's, the convolution's,
// and its weight and bias gradients (fp32 [dim][width] and [dim], dbias required
// when conv->bias is given) overlapping nothing the call reads or writes.
int validate_bwd_conv(const void* x, const sscan_conv_params* conv, const void* z, const void* dout, const void* dx,
                      const void* dz, const DirView* dirs, const sscan_dir_grads* grads, float* dconv_w,
                      float* dconv_b, int ndir, int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                      int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes,
                      ConvBwdLayout* layout, bool* empty) {
  if (!conv) return SSCAN_ERR_NULL;
  Sizes sz{};
  int st = check_sizes(batch, dim, len, dstate, io_dtype, bc_dtype, &sz);
  if (st != SSCAN_OK) return st;
  *layout = conv_bwd_layout(batch, dim, len, ndir, sz.io_esz);
  const bool nonempty = batch > 0 && dim > 0 && len > 0;
  // the scan backward's own checks, its workspace being the front of ours
  st = validate_bwd(x, z, dout, dx, dz, dirs, grads, ndir, batch, dim, len, dstate, io_dtype, bc_dtype, workspace,
                    nonempty ? layout->plan.workspace_bytes : workspace_bytes, &layout->plan, empty);
  if (st != SSCAN_OK) return st;
  const size_t io = sz.io_elems * sz.io_esz;
  st = check_conv(conv, dim, range_of(dx, nonempty ? io : 0));
  if (st != SSCAN_OK) return st;
  if (dim > 0 && (!dconv_w || (conv->bias && !dconv_b))) return SSCAN_ERR_NULL;
  if (!aligned(dconv_w, 4) || !aligned(dconv_b, 4)) return SSCAN_ERR_ALIGN;
  if (nonempty) {
    if (!workspace || workspace_bytes < layout->bytes) return SSCAN_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SSCAN_ERR_ALIGN;
  }
  // the convolution's gradients against every other buffer of the call
  const size_t vec = size_t(dim) * 4, bcb = sz.bc_elems * sz.bc_esz;
  RangeSet all;
  all.add(x, nonempty ? io : 0);
  all.add(z, nonempty && z ? io : 0);
  all.add(dout, nonempty ? io : 0);
  all.add(dx, nonempty ? io : 0);
  all.add(dz, nonempty && dz ? io : 0);
  all.add(conv->weight, vec * size_t(conv->width));
  all.add(conv->bias, conv->bias ? vec : 0);
  all.add(workspace, nonempty ? layout->bytes : 0);
  for (int k = 0; k < ndir; ++k) {
    all.add(dirs[k].delta, nonempty ? io : 0);
    all.add(dirs[k].B, bcb);
    all.add(dirs[k].C, bcb);
    all.add(dirs[k].A, vec * sscan::kDState);
    all.add(dirs[k].delta_bias, dirs[k].delta_bias ? vec : 0);
    all.add(dirs[k].D, dirs[k].D ? vec : 0);
    all.add(grads[k].ddelta, nonempty ? io : 0);
    all.add(grads[k].dA, vec * sscan::kDState);
    all.add(grads[k].dB, bcb);
    all.add(grads[k].dC, bcb);
    all.add(grads[k].ddelta_bias, grads[k].ddelta_bias ? vec : 0);
    all.add(grads[k].dD, grads[k].dD ? vec : 0);
  }
  const Range wr = range_of(dconv_w, vec * size_t(conv->width)), br = range_of(dconv_b, dconv_b ? vec : 0);
  if (overlap(wr, br)) return SSCAN_ERR_ALIAS;
  for (int i = 0; i < all.n; ++i)
    if (overlap(wr, all.r[i]) || overlap(br, all.r[i])) return SSCAN_ERR_ALIAS;
  // the whole workspace (the scan backward checked only its own front part)
  const Range wsr = range_of(workspace, nonempty ? layout->bytes : 0);
  for (int i = 0; i < all.n; ++i)
    if (all.r[i].lo != wsr.lo && overlap(wsr, all.r[i])) return SSCAN_ERR_ALIAS;
  return SSCAN_OK;
}

int run_bwd_conv(const void* x, const sscan_conv_params* conv, const void* z, const void* dout, void* dx, void* dz,
                 const DirView* dirs, const sscan_dir_grads* grads, float* dconv_w, float* dconv_b, int ndir,
                 int reverse, int softplus, int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                 int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes) {
  ConvBwdLayout l{};
  bool empty = false;
  const int st = validate_bwd_conv(x, conv, z, dout, dx, dz, dirs, grads, dconv_w, dconv_b, ndir, batch, dim, len,
                                   dstate, io_dtype, bc_dtype, workspace, workspace_bytes, &l, &empty);
  if (st != SSCAN_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  sscan::ConvBwdArgs c{x, nullptr, dx, conv->weight, conv->bias, dconv_w, dconv_b, conv->width, conv_left(conv),
                       conv->silu, io_dtype == SSCAN_BF16, batch, dim, len};
  sscan::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int k = 0; k < ndir; ++k)
    a.grads[k] = sscan::DirGrads{grads[k].ddelta, grads[k].ddelta_bias, grads[k].dA, grads[k].dB, grads[k].dC,
                                 grads[k].dD};
  if (empty) {
    a.fwd = make_args(x, z, nullptr, dirs, ndir, reverse, softplus, batch, dim, len, io_dtype, bc_dtype);
    hipError_t e = sscan::launch_bwd_zero(a, s);
    if (e == hipSuccess && dim > 0) e = sscan::launch_conv1d_bwd(c, nullptr, s);
    return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
  }
  float* u = reinterpret_cast<float*>(ws + l.off_u);
  void* du = ws + l.off_du;
  // u = conv(x) in float32 (the window pass reads it; the state chain recomputes it
  // from x, as the fused forward does), the scan's backward at u, then du back
  // through the convolution
  const sscan::ConvArgs fa{x, u, conv->weight, conv->bias, conv->width, conv_left(conv), conv->silu,
                           io_dtype == SSCAN_BF16, batch, dim, len, 1};
  hipError_t e = sscan::launch_conv1d(fa, s);
  if (e != hipSuccess) return SSCAN_ERR_HIP;
  a.fwd = make_args(x, z, nullptr, dirs, ndir, reverse, softplus, batch, dim, len, io_dtype, bc_dtype);
  a.fwd.conv_w = conv->weight;
  a.fwd.conv_b = conv->bias;
  a.fwd.conv_width = conv->width;
  a.fwd.conv_left = conv_left(conv);
  a.fwd.conv_silu = conv->silu;
  a.u32 = u;
  a.dout = dout;
  a.du = du;
  a.dz = dz;
  a.du_f32 = 1;
  e = sscan::launch_bwd(a, l.plan, reinterpret_cast<float*>(ws), s);
  if (e != hipSuccess) return SSCAN_ERR_HIP;
  c.du = static_cast<const float*>(du);
  e = sscan::launch_conv1d_bwd(c, reinterpret_cast<float*>(ws + l.off_part), s);
  return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
}

}  // namespace

extern "C" {

int sscan_bwd_conv(const void* x, const sscan_conv_params* conv, const void* delta, const float* delta_bias,
                   int softplus, const float* A, const void* B, const void* C, const float* D, const void* z,
                   const void* dout, void* dx, void* dz, const sscan_dir_grads* grads, float* dconv_w,
                   float* dconv_b, int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse,
                   void* stream, int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes) {
  if (!grads) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  return run_bwd_conv(x, conv, z, dout, dx, dz, &d, grads, dconv_w, dconv_b, 1, reverse, softplus, batch, dim, len,
                      dstate, stream, io_dtype, bc_dtype, workspace, workspace_bytes);
}

int sscan_bidir_bwd_conv(const void* x, const sscan_conv_params* conv, const void* z, const void* dout, void* dx,
                         void* dz, const sscan_dir_params* fwd, const sscan_dir_params* rev,
                         const sscan_dir_grads* gfwd, const sscan_dir_grads* grev, float* dconv_w, float* dconv_b,
                         int softplus, int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                         int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes) {
  if (!fwd || !rev || !gfwd || !grev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  const sscan_dir_grads g[2] = {*gfwd, *grev};
  return run_bwd_conv(x, conv, z, dout, dx, dz, d, g, dconv_w, dconv_b, 2, 0, softplus, batch, dim, len, dstate,
                      stream, io_dtype, bc_dtype, workspace, workspace_bytes);
}

int sscan_validate_bwd_conv(const void* x, const sscan_conv_params* conv, const void* delta, const float* delta_bias,
                            int softplus, const float* A, const void* B, const void* C, const float* D,
                            const void* z, const void* dout, const void* dx, const void* dz,
                            const sscan_dir_grads* grads, const float* dconv_w, const float* dconv_b, int64_t batch,
                            int64_t dim, int64_t len, int64_t dstate, int reverse, int io_dtype, int bc_dtype,
                            const void* workspace, size_t workspace_bytes) {
  (void)softplus;
  (void)reverse;
  if (!grads) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  ConvBwdLayout l{};
  bool empty = false;
  return validate_bwd_conv(x, conv, z, dout, dx, dz, &d, grads, const_cast<float*>(dconv_w),
                           const_cast<float*>(dconv_b), 1, batch, dim, len, dstate, io_dtype, bc_dtype, workspace,
                           workspace_bytes, &l, &empty);
}

size_t sscan_bwd_conv_workspace_bytes(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir,
                                      int io_dtype) {
  Sizes sz{};
  if (check_sizes(batch, dim, len, dstate, io_dtype, SSCAN_F32, &sz) != SSCAN_OK) return 0;
  if (batch == 0 || dim == 0 || len == 0) return 0;
  return conv_bwd_layout(batch, dim, len, bidir ? 2 : 1, sz.io_esz).bytes;
}

int sscan_fwd(const void* u, const void* delta, const float* delta_bias, int softplus, const float* A,
              const void* B, const void* C, const float* D, const void* z, void* y, int64_t batch, int64_t dim,
              int64_t len, int64_t dstate, int reverse, void* stream, int io_dtype, int bc_dtype, void* workspace,
              size_t workspace_bytes) {
  const DirView d{delta, delta_bias, A, B, C, D};
  return run(u, z, y, &d, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes);
}

int sscan_bidir(const void* u, const void* z, void* y, const sscan_dir_params* fwd, const sscan_dir_params* rev,
                int softplus, int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream, int io_dtype,
                int bc_dtype, void* workspace, size_t workspace_bytes) {
  if (!fwd || !rev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  return run(u, z, y, d, 2, 0, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes);
}

int sscan_fwd_profiled(const void* u, const void* delta, const float* delta_bias, int softplus, const float* A,
                       const void* B, const void* C, const float* D, const void* z, void* y, int64_t batch,
                       int64_t dim, int64_t len, int64_t dstate, int reverse, void* stream, int io_dtype,
                       int bc_dtype, void* workspace, size_t workspace_bytes, void* const* events) {
  const DirView d{delta, delta_bias, A, B, C, D};
  return run(u, z, y, &d, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes, events);
}

int sscan_bidir_profiled(const void* u, const void* z, void* y, const sscan_dir_params* fwd,
                         const sscan_dir_params* rev, int softplus, int64_t batch, int64_t dim, int64_t len,
                         int64_t dstate, void* stream, int io_dtype, int bc_dtype, void* workspace,
                         size_t workspace_bytes, void* const* events) {
  if (!fwd || !rev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  return run(u, z, y, d, 2, 0, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes, events);
}

int sscan_validate_fwd(const void* u, const void* delta, const float* delta_bias, int softplus, const float* A,
                       const void* B, const void* C, const float* D, const void* z, const void* y, int64_t batch,
                       int64_t dim, int64_t len, int64_t dstate, int reverse, int io_dtype, int bc_dtype,
                       const void* workspace, size_t workspace_bytes) {
  (void)softplus;
  (void)reverse;
  const DirView d{delta, delta_bias, A, B, C, D};
  sscan::Plan plan{};
  bool empty = false;
  return validate(u, z, y, &d, 1, batch, dim, len, dstate, io_dtype, bc_dtype, workspace, workspace_bytes, &plan,
                  &empty);
}

int sscan_validate_bidir(const void* u, const void* z, const void* y, const sscan_dir_params* fwd,
                         const sscan_dir_params* rev, int softplus, int64_t batch, int64_t dim, int64_t len,
                         int64_t dstate, int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes) {
  (void)softplus;
  if (!fwd || !rev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  sscan::Plan plan{};
  bool empty = false;
  return validate(u, z, y, d, 2, batch, dim, len, dstate, io_dtype, bc_dtype, workspace, workspace_bytes, &plan,
                  &empty);
}

int sscan_fwd_state(const void* u, const void* delta, const float* delta_bias, int softplus, const float* A,
                    const void* B, const void* C, const float* D, const void* z, void* y, const float* h0,
                    float* h_last, int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse,
                    void* stream, int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes) {
  const DirView d{delta, delta_bias, A, B, C, D};
  if (!h0 && !h_last)
    return run(u, z, y, &d, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
               workspace_bytes);
  return run(u, z, y, &d, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes, nullptr, h0, h_last);
}

int sscan_validate_fwd_state(const void* u, const void* delta, const float* delta_bias, int softplus,
                             const float* A, const void* B, const void* C, const float* D, const void* z,
                             const void* y, const float* h0, const float* h_last, int64_t batch, int64_t dim,
                             int64_t len, int64_t dstate, int reverse, int io_dtype, int bc_dtype,
                             const void* workspace, size_t workspace_bytes) {
  (void)softplus;
  (void)reverse;
  const DirView d{delta, delta_bias, A, B, C, D};
  sscan::Plan plan{};
  bool empty = false;
  return validate_state_call(u, z, y, d, h0, const_cast<float*>(h_last), batch, dim, len, dstate, io_dtype,
                             bc_dtype, workspace, workspace_bytes, &plan, &empty);
}

int sscan_validate_step(const float* state, const void* u, const void* delta, const float* delta_bias,
                        int softplus, const float* A, const void* B, const void* C, const float* D, const void* z,
                        const void* y, int64_t batch, int64_t dim, int64_t dstate, int io_dtype, int bc_dtype) {
  (void)softplus;
  Sizes sz{};
  // one token: the sequence checks with len = 1 cover sizes and dtypes
  int st = check_sizes(batch, dim, 1, dstate, io_dtype, bc_dtype, &sz);
  if (st != SSCAN_OK) return st;
  if (batch == 0 || dim == 0) return SSCAN_OK;
  if (!state || !u || !delta || !A || !B || !C || !y) return SSCAN_ERR_NULL;
  // state and A are read as 16-byte pieces, B and C as 4 states at a time
  const size_t bc_align = 4 * sz.bc_esz;
  if (!aligned(state, 16) || !aligned(u, sz.io_esz) || !aligned(delta, sz.io_esz) || !aligned(z, sz.io_esz) ||
      !aligned(y, sz.io_esz) || !aligned(B, bc_align) || !aligned(C, bc_align) || !aligned(A, 16) ||
      !aligned(D, 4) || !aligned(delta_bias, 4))
    return SSCAN_ERR_ALIGN;
  const size_t io = sz.io_elems * sz.io_esz, bcb = sz.bc_elems * sz.bc_esz, vec = size_t(dim) * 4;
  const Range sr = range_of(state, sz.io_elems * sscan::kDState * 4), yr = range_of(y, io);
  const Range ins[] = {range_of(u, io), range_of(delta, io), range_of(z, z ? io : 0), range_of(B, bcb),
                       range_of(C, bcb), range_of(A, vec * sscan::kDState),
                       range_of(delta_bias, delta_bias ? vec : 0), range_of(D, D ? vec : 0)};
  if (overlap(sr, yr)) return SSCAN_ERR_ALIAS;
  for (const Range& r : ins)
    if (overlap(sr, r) || overlap(yr, r)) return SSCAN_ERR_ALIAS;
  return SSCAN_OK;
}

int sscan_validate_step_conv(const float* state, const void* conv_state, const void* x, const sscan_conv_params* conv,
                             const void* delta, const float* delta_bias, int softplus, const float* A, const void* B,
                             const void* C, const float* D, const void* z, const void* y, int64_t batch, int64_t dim,
                             int64_t dstate, int io_dtype, int bc_dtype) {
  int st = sscan_validate_step(state, x, delta, delta_bias, softplus, A, B, C, D, z, y, batch, dim, dstate, io_dtype,
                               bc_dtype);
  if (st != SSCAN_OK) return st;
  if (!conv) return SSCAN_ERR_NULL;
  if (conv->same != 0) return SSCAN_ERR_UNSUPPORTED;  // a centred window needs the next token
  Sizes sz{};
  check_sizes(batch, dim, 1, dstate, io_dtype, bc_dtype, &sz);
  const Range yr = range_of(y, batch * dim > 0 ? sz.io_elems * sz.io_esz : 0);
  st = check_conv(conv, dim, yr);
  if (st != SSCAN_OK || batch == 0 || dim == 0) return st;
  const size_t cs_bytes = sz.io_elems * size_t(conv->width - 1) * sz.io_esz;
  if (cs_bytes > 0 && !conv_state) return SSCAN_ERR_NULL;
  if (!aligned(conv_state, sz.io_esz)) return SSCAN_ERR_ALIGN;
  // the window is updated in place: it overlaps nothing else the call reads or writes
  const size_t io = sz.io_elems * sz.io_esz, bcb = sz.bc_elems * sz.bc_esz, vec = size_t(dim) * 4;
  const Range cr = range_of(conv_state, cs_bytes);
  const Range others[] = {range_of(state, sz.io_elems * sscan::kDState * 4), yr, range_of(x, io),
                          range_of(delta, io), range_of(z, z ? io : 0), range_of(B, bcb), range_of(C, bcb),
                          range_of(A, vec * sscan::kDState), range_of(delta_bias, delta_bias ? vec : 0),
                          range_of(D, D ? vec : 0), range_of(conv->weight, vec * size_t(conv->width)),
                          range_of(conv->bias, conv->bias ? vec : 0)};
  for (const Range& r : others)
    if (overlap(cr, r)) return SSCAN_ERR_ALIAS;
  if (overlap(range_of(state, sz.io_elems * sscan::kDState * 4), range_of(conv->weight, vec * size_t(conv->width))) ||
      (conv->bias && overlap(range_of(state, sz.io_elems * sscan::kDState * 4), range_of(conv->bias, vec))))
    return SSCAN_ERR_ALIAS;
  return SSCAN_OK;
}

int sscan_step_conv(float* state, void* conv_state, const void* x, const sscan_conv_params* conv, const void* delta,
                    const float* delta_bias, int softplus, const float* A, const void* B, const void* C,
                    const float* D, const void* z, void* y, int64_t batch, int64_t dim, int64_t dstate, void* stream,
                    int io_dtype, int bc_dtype) {
  const int st = sscan_validate_step_conv(state, conv_state, x, conv, delta, delta_bias, softplus, A, B, C, D, z, y,
                                          batch, dim, dstate, io_dtype, bc_dtype);
  if (st != SSCAN_OK || batch == 0 || dim == 0) return st;
  sscan::StepArgs a{state, x, delta, z, y, delta_bias, A, B, C, D, softplus ? 1 : 0, io_dtype == SSCAN_BF16,
                    bc_dtype == SSCAN_BF16, batch, dim, conv_state, conv->weight, conv->bias, conv->width,
                    conv->silu};
  const hipError_t e = sscan::launch_step(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
}

int sscan_step(float* state, const void* u, const void* delta, const float* delta_bias, int softplus,
               const float* A, const void* B, const void* C, const float* D, const void* z, void* y, int64_t batch,
               int64_t dim, int64_t dstate, void* stream, int io_dtype, int bc_dtype) {
  const int st = sscan_validate_step(state, u, delta, delta_bias, softplus, A, B, C, D, z, y, batch, dim, dstate,
                                     io_dtype, bc_dtype);
  if (st != SSCAN_OK || batch == 0 || dim == 0) return st;
  sscan::StepArgs a{state, u, delta, z, y, delta_bias, A, B, C, D, softplus ? 1 : 0, io_dtype == SSCAN_BF16,
                    bc_dtype == SSCAN_BF16, batch, dim, nullptr, nullptr, nullptr, 0, 0};
  const hipError_t e = sscan::launch_step(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
}

int sscan_bwd(const void* u, const void* delta, const float* delta_bias, int softplus, const float* A, const void* B,
              const void* C, const float* D, const void* z, const void* dout, void* du, void* dz,
              const sscan_dir_grads* grads, int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse,
              void* stream, int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes) {
  if (!grads) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  return run_bwd(u, z, dout, du, dz, &d, grads, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype,
                 bc_dtype, workspace, workspace_bytes);
}

int sscan_bwd_state(const void* u, const void* delta, const float* delta_bias, int softplus, const float* A,
                    const void* B, const void* C, const float* D, const void* z, const void* dout, const float* h0,
                    const float* dh_last, void* du, void* dz, const sscan_dir_grads* grads, float* dh0,
                    int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse, void* stream, int io_dtype,
                    int bc_dtype, void* workspace, size_t workspace_bytes) {
  if (!grads) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  return run_bwd(u, z, dout, du, dz, &d, grads, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype,
                 bc_dtype, workspace, workspace_bytes, nullptr, h0, dh_last, dh0);
}

int sscan_validate_bwd_state(const void* u, const void* delta, const float* delta_bias, int softplus,
                             const float* A, const void* B, const void* C, const float* D, const void* z,
                             const void* dout, const float* h0, const float* dh_last, const void* du, const void* dz,
                             const sscan_dir_grads* grads, const float* dh0, int64_t batch, int64_t dim, int64_t len,
                             int64_t dstate, int reverse, int io_dtype, int bc_dtype, const void* workspace,
                             size_t workspace_bytes) {
  (void)softplus;
  (void)reverse;
  if (!grads) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  sscan::BwdPlan plan{};
  bool empty = false;
  const int st = validate_bwd(u, z, dout, du, dz, &d, grads, 1, batch, dim, len, dstate, io_dtype, bc_dtype,
                              workspace, workspace_bytes, &plan, &empty);
  if (st != SSCAN_OK) return st;
  return check_bwd_state(h0, dh_last, dh0, u, z, dout, du, dz, d, *grads, batch, dim, len, io_dtype, bc_dtype,
                         workspace, workspace_bytes);
}

int sscan_bidir_bwd(const void* u, const void* z, const void* dout, void* du, void* dz, const sscan_dir_params* fwd,
                    const sscan_dir_params* rev, const sscan_dir_grads* gfwd, const sscan_dir_grads* grev,
                    int softplus, int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream,
                    int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes) {
  if (!fwd || !rev || !gfwd || !grev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  const sscan_dir_grads g[2] = {*gfwd, *grev};
  return run_bwd(u, z, dout, du, dz, d, g, 2, 0, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype,
                 workspace, workspace_bytes);
}

int sscan_bwd_profiled(const void* u, const void* delta, const float* delta_bias, int softplus, const float* A,
                       const void* B, const void* C, const float* D, const void* z, const void* dout, void* du,
                       void* dz, const sscan_dir_grads* grads, int64_t batch, int64_t dim, int64_t len,
                       int64_t dstate, int reverse, void* stream, int io_dtype, int bc_dtype, void* workspace,
                       size_t workspace_bytes, void* const* events) {
  if (!grads) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  return run_bwd(u, z, dout, du, dz, &d, grads, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype,
                 bc_dtype, workspace, workspace_bytes, events);
}

int sscan_bidir_bwd_profiled(const void* u, const void* z, const void* dout, void* du, void* dz,
                             const sscan_dir_params* fwd, const sscan_dir_params* rev, const sscan_dir_grads* gfwd,
                             const sscan_dir_grads* grev, int softplus, int64_t batch, int64_t dim, int64_t len,
                             int64_t dstate, void* stream, int io_dtype, int bc_dtype, void* workspace,
                             size_t workspace_bytes, void* const* events) {
  if (!fwd || !rev || !gfwd || !grev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  const sscan_dir_grads g[2] = {*gfwd, *grev};
  return run_bwd(u, z, dout, du, dz, d, g, 2, 0, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype,
                 workspace, workspace_bytes, events);
}

int sscan_validate_bwd(const void* u, const void* delta, const float* delta_bias, int softplus, const float* A,
                       const void* B, const void* C, const float* D, const void* z, const void* dout,
                       const void* du, const void* dz, const sscan_dir_grads* grads, int64_t batch, int64_t dim,
                       int64_t len, int64_t dstate, int reverse, int io_dtype, int bc_dtype, const void* workspace,
                       size_t workspace_bytes) {
  (void)softplus;
  (void)reverse;
  if (!grads) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  sscan::BwdPlan plan{};
  bool empty = false;
  return validate_bwd(u, z, dout, du, dz, &d, grads, 1, batch, dim, len, dstate, io_dtype, bc_dtype, workspace,
                      workspace_bytes, &plan, &empty);
}

int sscan_validate_bidir_bwd(const void* u, const void* z, const void* dout, const void* du, const void* dz,
                             const sscan_dir_params* fwd, const sscan_dir_params* rev, const sscan_dir_grads* gfwd,
                             const sscan_dir_grads* grev, int softplus, int64_t batch, int64_t dim, int64_t len,
                             int64_t dstate, int io_dtype, int bc_dtype, const void* workspace,
                             size_t workspace_bytes) {
  (void)softplus;
  if (!fwd || !rev || !gfwd || !grev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  const sscan_dir_grads g[2] = {*gfwd, *grev};
  sscan::BwdPlan plan{};
  bool empty = false;
  return validate_bwd(u, z, dout, du, dz, d, g, 2, batch, dim, len, dstate, io_dtype, bc_dtype, workspace,
                      workspace_bytes, &plan, &empty);
}

size_t sscan_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir) {
  Sizes sz{};
  if (check_sizes(batch, dim, len, dstate, SSCAN_F32, SSCAN_F32, &sz) != SSCAN_OK) return 0;
  if (batch == 0 || dim == 0 || len == 0) return 0;
  return sscan::make_bwd_plan(batch, dim, len, bidir ? 2 : 1).workspace_bytes;
}

int sscan_validate_conv1d(const void* x, const sscan_conv_params* conv, const void* y, int64_t batch, int64_t dim,
                          int64_t len, int io_dtype) {
  Sizes sz{};
  int st = check_sizes(batch, dim, len, sscan::kDState, io_dtype, SSCAN_F32, &sz);
  if (st != SSCAN_OK) return st;
  if (!conv) return SSCAN_ERR_NULL;
  if (batch == 0 || dim == 0 || len == 0) return SSCAN_OK;
  if (!x || !y) return SSCAN_ERR_NULL;
  if (!aligned(x, sz.io_esz) || !aligned(y, sz.io_esz)) return SSCAN_ERR_ALIGN;
  const Range yr = range_of(y, sz.io_elems * sz.io_esz);
  if (overlap(yr, range_of(x, sz.io_elems * sz.io_esz))) return SSCAN_ERR_ALIAS;
  return check_conv(conv, dim, yr);
}

int sscan_conv1d(const void* x, const sscan_conv_params* conv, void* y, int64_t batch, int64_t dim, int64_t len,
                 void* stream, int io_dtype) {
  const int st = sscan_validate_conv1d(x, conv, y, batch, dim, len, io_dtype);
  if (st != SSCAN_OK || batch == 0 || dim == 0 || len == 0) return st;
  const sscan::ConvArgs a{x, y, conv->weight, conv->bias, conv->width, conv_left(conv), conv->silu,
                          io_dtype == SSCAN_BF16, batch, dim, len};
  const hipError_t e = sscan::launch_conv1d(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
}

int sscan_fwd_conv(const void* x, const sscan_conv_params* conv, const void* delta, const float* delta_bias,
                   int softplus, const float* A, const void* B, const void* C, const float* D, const void* z, void* y,
                   int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse, void* stream, int io_dtype,
                   int bc_dtype, void* workspace, size_t workspace_bytes) {
  if (!conv) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  return run(x, z, y, &d, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes, nullptr, nullptr, nullptr, conv);
}

int sscan_bidir_conv(const void* x, const sscan_conv_params* conv, const void* z, void* y, const sscan_dir_params* fwd,
                     const sscan_dir_params* rev, int softplus, int64_t batch, int64_t dim, int64_t len,
                     int64_t dstate, void* stream, int io_dtype, int bc_dtype, void* workspace,
                     size_t workspace_bytes) {
  if (!conv || !fwd || !rev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  return run(x, z, y, d, 2, 0, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes, nullptr, nullptr, nullptr, conv);
}

int sscan_fwd_conv_profiled(const void* x, const sscan_conv_params* conv, const void* delta, const float* delta_bias,
                            int softplus, const float* A, const void* B, const void* C, const float* D, const void* z,
                            void* y, int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse,
                            void* stream, int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes,
                            void* const* events) {
  if (!conv) return SSCAN_ERR_NULL;
  const DirView d{delta, delta_bias, A, B, C, D};
  return run(x, z, y, &d, 1, reverse, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes, events, nullptr, nullptr, conv);
}

int sscan_bidir_conv_profiled(const void* x, const sscan_conv_params* conv, const void* z, void* y,
                              const sscan_dir_params* fwd, const sscan_dir_params* rev, int softplus, int64_t batch,
                              int64_t dim, int64_t len, int64_t dstate, void* stream, int io_dtype, int bc_dtype,
                              void* workspace, size_t workspace_bytes, void* const* events) {
  if (!conv || !fwd || !rev) return SSCAN_ERR_NULL;
  const DirView d[2] = {view_of(fwd), view_of(rev)};
  return run(x, z, y, d, 2, 0, softplus, batch, dim, len, dstate, stream, io_dtype, bc_dtype, workspace,
             workspace_bytes, events, nullptr, nullptr, conv);
}

// ---- several visiting orders of a 2-D map ------------------------------------------

}  // extern "C"

namespace {

int check_kinds(const int* kinds, int ndirs, const int32_t* index) {
  if (!kinds) return SSCAN_ERR_NULL;
  if (ndirs < 1 || ndirs > sscan::kMaxMultiDirs) return SSCAN_ERR_UNSUPPORTED;
  bool seen[sscan::kMaxMultiDirs] = {};
  bool uses_index = false;
  for (int k = 0; k < ndirs; ++k) {
    if (kinds[k] < 0 || kinds[k] >= sscan::kMaxMultiDirs || seen[kinds[k]]) return SSCAN_ERR_UNSUPPORTED;
    seen[kinds[k]] = true;
    uses_index = uses_index || kinds[k] / 2 == sscan::kFamilyIndex;
  }
  if (uses_index && !index) return SSCAN_ERR_NULL;
  return SSCAN_OK;
}

int validate_multi(const void* u, const void* z, const void* y, const sscan_dir_params* dirs, const int* kinds,
                   int ndirs, const int32_t* index, int64_t batch, int64_t dim, int64_t height, int64_t width,
                   int64_t dstate, int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes,
                   sscan::MultiPlan* plan, bool* empty) {
  if (height < 0 || width < 0) return SSCAN_ERR_SHAPE;
  if (height > 0 && width > (int64_t(1) << 40) / height) return SSCAN_ERR_SHAPE;
  const int64_t len = height * width;
  Sizes sz{};
  int st = check_sizes(batch, dim, len, dstate, io_dtype, bc_dtype, &sz);
  if (st != SSCAN_OK) return st;
  st = check_kinds(kinds, ndirs, index);
  if (st != SSCAN_OK) return st;
  if (!dirs) return SSCAN_ERR_NULL;
  *empty = (batch == 0 || dim == 0 || len == 0);
  if (*empty) return SSCAN_OK;
  if (!u || !y) return SSCAN_ERR_NULL;
  if (!aligned(u, sz.io_esz) || !aligned(y, sz.io_esz) || !aligned(z, sz.io_esz) || !aligned(index, 4))
    return SSCAN_ERR_ALIGN;
  const Range yr = range_of(y, sz.io_elems * sz.io_esz);
  if (overlap(yr, range_of(u, sz.io_elems * sz.io_esz)) || (z && overlap(yr, range_of(z, sz.io_elems * sz.io_esz))) ||
      (index && overlap(yr, range_of(index, size_t(len) * 4))))
    return SSCAN_ERR_ALIAS;
  for (int k = 0; k < ndirs; ++k) {
    st = check_dir(view_of(&dirs[k]), sz, dim, yr);
    if (st != SSCAN_OK) return st;
  }
  *plan = sscan::make_multi_plan(batch, dim, height, width, kinds, ndirs, io_dtype == SSCAN_BF16,
                                 bc_dtype == SSCAN_BF16);
  // each family's scan runs one or two directions over the whole map
  for (int n = 1; n <= 2; ++n)
    if (!sscan::plan_fits_grid(sscan::make_plan(batch, dim, height * width, n), batch, dim, height * width, n))
      return SSCAN_ERR_SHAPE;
  if (!workspace || workspace_bytes < plan->workspace_bytes) return SSCAN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return SSCAN_ERR_ALIGN;
  if (overlap(yr, range_of(workspace, plan->workspace_bytes))) return SSCAN_ERR_ALIAS;
  return SSCAN_OK;
}

}  // namespace

extern "C" {

int sscan_validate_multi(const void* u, const void* z, const void* y, const sscan_dir_params* dirs, const int* kinds,
                         int ndirs, const int32_t* index, int softplus, int64_t batch, int64_t dim, int64_t height,
                         int64_t width, int64_t dstate, int io_dtype, int bc_dtype, const void* workspace,
                         size_t workspace_bytes) {
  (void)softplus;
  sscan::MultiPlan plan{};
  bool empty = false;
  return validate_multi(u, z, y, dirs, kinds, ndirs, index, batch, dim, height, width, dstate, io_dtype, bc_dtype,
                        workspace, workspace_bytes, &plan, &empty);
}

int sscan_multi(const void* u, const void* z, void* y, const sscan_dir_params* dirs, const int* kinds, int ndirs,
                const int32_t* index, int softplus, int64_t batch, int64_t dim, int64_t height, int64_t width,
                int64_t dstate, void* stream, int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes) {
  sscan::MultiPlan plan{};
  bool empty = false;
  const int st = validate_multi(u, z, y, dirs, kinds, ndirs, index, batch, dim, height, width, dstate, io_dtype,
                                bc_dtype, workspace, workspace_bytes, &plan, &empty);
  if (st != SSCAN_OK || empty) return st;
  sscan::MultiArgs a;
  std::memset(&a, 0, sizeof(a));
  a.u = u;
  a.z = z;
  a.y = y;
  for (int k = 0; k < ndirs; ++k) {
    const sscan_dir_params& p = dirs[k];
    a.dir[k] = sscan::DirArgs{p.delta, p.delta_bias, p.A, p.B, p.C, p.D};
    a.kind[k] = kinds[k];
  }
  a.ndir = ndirs;
  a.index = index;
  a.softplus = softplus ? 1 : 0;
  a.io_bf16 = io_dtype == SSCAN_BF16;
  a.bc_bf16 = bc_dtype == SSCAN_BF16;
  a.batch = batch;
  a.dim = dim;
  a.height = height;
  a.width = width;
  const hipError_t e = sscan::launch_multi(a, plan, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
}

size_t sscan_multi_workspace_bytes(int64_t batch, int64_t dim, int64_t height, int64_t width, int64_t dstate,
                                   const int* kinds, int ndirs, int io_dtype, int bc_dtype) {
  if (height < 0 || width < 0 || (height > 0 && width > (int64_t(1) << 40) / height)) return 0;
  Sizes sz{};
  if (check_sizes(batch, dim, height * width, dstate, io_dtype, bc_dtype, &sz) != SSCAN_OK) return 0;
  if (check_kinds(kinds, ndirs, reinterpret_cast<const int32_t*>(1)) != SSCAN_OK) return 0;
  if (batch == 0 || dim == 0 || height * width == 0) return 0;
  return sscan::make_multi_plan(batch, dim, height, width, kinds, ndirs, io_dtype == SSCAN_BF16,
                                bc_dtype == SSCAN_BF16)
      .workspace_bytes;
}

}  // extern "C"

namespace {

// A multi-order backward call: the forward's sizes, kinds and parameters, the
// backward's gradient buffers (every direction's, per direction), and the
// workspace.  Outputs overlap nothing else; inputs may overlap each other.
int validate_multi_bwd(const void* u, const void* z, const void* dout, const void* du, const void* dz,
                       const sscan_dir_params* dirs, const sscan_dir_grads* grads, const int* kinds, int ndirs,
                       const int32_t* index, int64_t batch, int64_t dim, int64_t height, int64_t width,
                       int64_t dstate, int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes,
                       sscan::MultiBwdPlan* plan, bool* empty) {
  if (height < 0 || width < 0) return SSCAN_ERR_SHAPE;
  if (height > 0 && width > (int64_t(1) << 40) / height) return SSCAN_ERR_SHAPE;
  const int64_t len = height * width;
  Sizes sz{};
  int st = check_sizes(batch, dim, len, dstate, io_dtype, bc_dtype, &sz);
  if (st != SSCAN_OK) return st;
  st = check_kinds(kinds, ndirs, index);
  if (st != SSCAN_OK) return st;
  if (!dirs || !grads) return SSCAN_ERR_NULL;
  for (int k = 0; k < ndirs; ++k)
    if ((dim > 0 && !grads[k].dA) || (sz.bc_elems > 0 && (!grads[k].dB || !grads[k].dC))) return SSCAN_ERR_NULL;
  *empty = (batch == 0 || dim == 0 || len == 0);
  const size_t io = sz.io_elems * sz.io_esz;
  RangeSet in, out;
  if (!*empty) {
    if (!u || !dout || !du || (z && !dz)) return SSCAN_ERR_NULL;
    for (int k = 0; k < ndirs; ++k)
      if (!dirs[k].delta || !dirs[k].A || !dirs[k].B || !dirs[k].C || !grads[k].ddelta) return SSCAN_ERR_NULL;
    const void* io_ptrs[] = {u, z, dout, du, dz};
    for (const void* q : io_ptrs)
      if (!aligned(q, sz.io_esz)) return SSCAN_ERR_ALIGN;
    if (!aligned(index, 4)) return SSCAN_ERR_ALIGN;
    in.add(u, io);
    in.add(z, io);
    in.add(dout, io);
    in.add(index, size_t(len) * 4);
    out.add(du, io);
    if (z) out.add(dz, io);
  }
  for (int k = 0; k < ndirs; ++k) {
    st = add_bwd_dir(view_of(&dirs[k]), grads[k], sz, dim, *empty, &in, &out);
    if (st != SSCAN_OK) return st;
  }
  if (!*empty) {
    // each family's backward runs one or two directions over the whole map
    for (int n = 1; n <= 2; ++n)
      if (!sscan::bwd_plan_fits_grid(sscan::make_bwd_plan(batch, dim, len, n), batch, dim, len, n))
        return SSCAN_ERR_SHAPE;
    *plan = sscan::make_multi_bwd_plan(batch, dim, height, width, kinds, ndirs, io_dtype == SSCAN_BF16,
                                       bc_dtype == SSCAN_BF16);
    if (!workspace || workspace_bytes < plan->workspace_bytes) return SSCAN_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SSCAN_ERR_ALIGN;
    out.add(workspace, plan->workspace_bytes);
  }
  return disjoint(in, out);
}

}  // namespace

extern "C" {

int sscan_validate_multi_bwd(const void* u, const void* z, const void* dout, const void* du, const void* dz,
                             const sscan_dir_params* dirs, const sscan_dir_grads* grads, const int* kinds, int ndirs,
                             const int32_t* index, int softplus, int64_t batch, int64_t dim, int64_t height,
                             int64_t width, int64_t dstate, int io_dtype, int bc_dtype, const void* workspace,
                             size_t workspace_bytes) {
  (void)softplus;
  sscan::MultiBwdPlan plan{};
  bool empty = false;
  return validate_multi_bwd(u, z, dout, du, dz, dirs, grads, kinds, ndirs, index, batch, dim, height, width, dstate,
                            io_dtype, bc_dtype, workspace, workspace_bytes, &plan, &empty);
}

int sscan_multi_bwd(const void* u, const void* z, const void* dout, void* du, void* dz, const sscan_dir_params* dirs,
                    const sscan_dir_grads* grads, const int* kinds, int ndirs, const int32_t* index, int softplus,
                    int64_t batch, int64_t dim, int64_t height, int64_t width, int64_t dstate, void* stream,
                    int io_dtype, int bc_dtype, void* workspace, size_t workspace_bytes) {
  sscan::MultiBwdPlan plan{};
  bool empty = false;
  const int st = validate_multi_bwd(u, z, dout, du, dz, dirs, grads, kinds, ndirs, index, batch, dim, height, width,
                                    dstate, io_dtype, bc_dtype, workspace, workspace_bytes, &plan, &empty);
  if (st != SSCAN_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (empty) {
    // no tokens or no channels: the parameter gradients that have elements are zero
    for (int k = 0; k < ndirs; ++k) {
      sscan::BwdArgs b;
      std::memset(&b, 0, sizeof(b));
      b.fwd = make_args(u, z, nullptr, nullptr, 0, 0, softplus, batch, dim, height * width, io_dtype, bc_dtype);
      b.fwd.ndir = 1;
      b.grads[0] = sscan::DirGrads{grads[k].ddelta, grads[k].ddelta_bias, grads[k].dA, grads[k].dB, grads[k].dC,
                                   grads[k].dD};
      if (sscan::launch_bwd_zero(b, s) != hipSuccess) return SSCAN_ERR_HIP;
    }
    return SSCAN_OK;
  }
  sscan::MultiBwdArgs a;
  std::memset(&a, 0, sizeof(a));
  sscan::MultiArgs& m = a.fwd;
  m.u = u;
  m.z = z;
  for (int k = 0; k < ndirs; ++k) {
    const sscan_dir_params& p = dirs[k];
    m.dir[k] = sscan::DirArgs{p.delta, p.delta_bias, p.A, p.B, p.C, p.D};
    m.kind[k] = kinds[k];
    a.grads[k] = sscan::DirGrads{grads[k].ddelta, grads[k].ddelta_bias, grads[k].dA, grads[k].dB, grads[k].dC,
                                 grads[k].dD};
  }
  m.ndir = ndirs;
  m.index = index;
  m.softplus = softplus ? 1 : 0;
  m.io_bf16 = io_dtype == SSCAN_BF16;
  m.bc_bf16 = bc_dtype == SSCAN_BF16;
  m.batch = batch;
  m.dim = dim;
  m.height = height;
  m.width = width;
  a.dout = dout;
  a.du = du;
  a.dz = dz;
  const hipError_t e = sscan::launch_multi_bwd(a, plan, static_cast<char*>(workspace), s);
  return e == hipSuccess ? SSCAN_OK : SSCAN_ERR_HIP;
}

size_t sscan_multi_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t height, int64_t width, int64_t dstate,
                                       const int* kinds, int ndirs, int io_dtype, int bc_dtype) {
  if (height < 0 || width < 0 || (height > 0 && width > (int64_t(1) << 40) / height)) return 0;
  Sizes sz{};
  if (check_sizes(batch, dim, height * width, dstate, io_dtype, bc_dtype, &sz) != SSCAN_OK) return 0;
  if (check_kinds(kinds, ndirs, reinterpret_cast<const int32_t*>(1)) != SSCAN_OK) return 0;
  if (batch == 0 || dim == 0 || height * width == 0) return 0;
  return sscan::make_multi_bwd_plan(batch, dim, height, width, kinds, ndirs, io_dtype == SSCAN_BF16,
                                    bc_dtype == SSCAN_BF16)
      .workspace_bytes;
}

// The centre-out clockwise spiral: from the centre cell (the lower middle index of
// an even side) walk right 1, down 1, left 2, up 2, right 3, down 3, ... (rows grow
// downwards), listing the cells that fall inside the map.
int sscan_spiral_order(int64_t height, int64_t width, int32_t* order) {
  if (height < 0 || width < 0 || (height > 0 && width > (int64_t(1) << 31) / height)) return SSCAN_ERR_SHAPE;
  const int64_t n = height * width;
  if (n == 0) return SSCAN_OK;
  if (!order) return SSCAN_ERR_NULL;
  int64_t r = (height - 1) / 2, c = (width - 1) / 2, k = 0;
  order[k++] = int32_t(r * width + c);
  static const int dr[4] = {0, 1, 0, -1}, dc[4] = {1, 0, -1, 0};
  for (int64_t leg = 0; k < n; ++leg) {
    const int64_t steps = leg / 2 + 1;
    for (int64_t i = 0; i < steps; ++i) {
      r += dr[leg % 4];
      c += dc[leg % 4];
      if (r >= 0 && r < height && c >= 0 && c < width) order[k++] = int32_t(r * width + c);
    }
  }
  return SSCAN_OK;
}

size_t sscan_workspace_bytes(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir) {
  Sizes sz{};
  if (check_sizes(batch, dim, len, dstate, SSCAN_F32, SSCAN_F32, &sz) != SSCAN_OK) return 0;
  if (batch == 0 || dim == 0 || len == 0) return 0;
  return sscan::make_plan(batch, dim, len, bidir ? 2 : 1).workspace_bytes;
}

int sscan_scan_plan(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir, int64_t* out) {
  if (!out) return SSCAN_ERR_NULL;
  Sizes sz{};
  const int st = check_sizes(batch, dim, len, dstate, SSCAN_F32, SSCAN_F32, &sz);
  if (st != SSCAN_OK) return st;
  const sscan::Plan p = sscan::make_plan(batch, dim, len, bidir ? 2 : 1);
  out[0] = p.seg_len;
  out[1] = p.nseg;
  out[2] = p.run_len;
  out[3] = p.nrun;
  return SSCAN_OK;
}

int sscan_bwd_plan(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir, int64_t* out) {
  if (!out) return SSCAN_ERR_NULL;
  Sizes sz{};
  const int st = check_sizes(batch, dim, len, dstate, SSCAN_F32, SSCAN_F32, &sz);
  if (st != SSCAN_OK) return st;
  const sscan::BwdPlan p = sscan::make_bwd_plan(batch, dim, len, bidir ? 2 : 1);
  out[0] = p.nwin;
  out[1] = p.csplit;
  out[2] = p.gps;
  out[3] = p.run_len;
  out[4] = p.nrun;
  return SSCAN_OK;
}

const char* sscan_strerror(int status) {
  switch (status) {
    case SSCAN_OK: return "ok";
    case SSCAN_ERR_NULL: return "a required pointer is NULL";
    case SSCAN_ERR_SHAPE: return "invalid sizes (negative, or too large)";
    case SSCAN_ERR_UNSUPPORTED: return "unsupported dstate (must be 16), dtype code or convolution shape";
    case SSCAN_ERR_ALIGN: return "a pointer is not aligned to its element size (workspace: 16 bytes)";
    case SSCAN_ERR_WORKSPACE: return "workspace missing or smaller than sscan_workspace_bytes()";
    case SSCAN_ERR_HIP: return "HIP runtime error at launch";
    case SSCAN_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
    case SSCAN_ERR_TOO_LARGE: return "the call needs more workspace than the no-alloc scratch array holds";
    default: return "unknown status";
  }
}

int sscan_version(void) { return kVersion; }

}  // extern "C"
