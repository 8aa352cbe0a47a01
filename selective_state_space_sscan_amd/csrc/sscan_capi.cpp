// sscan_capi.cpp -- C ABI of the selective scan: argument checks, then one call
// into the kernel launcher.  Every check happens before any HIP call, so the
// validate entry points work on a machine without a GPU.
#include "sscan.h"

#include <cstdint>
#include <cstring>

#include "sscan_internal.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
static_assert(SSCAN_PROFILE_EVENTS == sscan::kProfileEvents, "event count mismatch");

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
  int64_t bd = 0, n_io = 0, n_bc = 0, b16 = 0;
  if (__builtin_mul_overflow(batch, dim, &bd) || __builtin_mul_overflow(bd, len, &n_io) ||
      __builtin_mul_overflow(batch, int64_t(sscan::kDState), &b16) || __builtin_mul_overflow(b16, len, &n_bc) ||
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

// Shared by the run and validate entry points.  On success *plan is filled and
// *empty tells whether there is nothing to do.
int validate(const void* u, const void* z, const void* y, const DirView* dirs, int ndir, int64_t batch, int64_t dim,
             int64_t len, int64_t dstate, int io_dtype, int bc_dtype, const void* workspace, size_t workspace_bytes,
             sscan::Plan* plan, bool* empty) {
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
  *plan = sscan::make_plan(batch, dim, len, ndir);
  if (plan->workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan->workspace_bytes) return SSCAN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return SSCAN_ERR_ALIGN;
    if (overlap(yr, range_of(workspace, plan->workspace_bytes))) return SSCAN_ERR_ALIAS;
  }
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

int run(const void* u, const void* z, void* y, const DirView* dirs, int ndir, int reverse, int softplus,
        int64_t batch, int64_t dim, int64_t len, int64_t dstate, void* stream, int io_dtype, int bc_dtype,
        void* workspace, size_t workspace_bytes, void* const* events = nullptr) {
  sscan::Plan plan{};
  bool empty = false;
  const int st = validate(u, z, y, dirs, ndir, batch, dim, len, dstate, io_dtype, bc_dtype, workspace,
                          workspace_bytes, &plan, &empty);
  if (st != SSCAN_OK || empty) return st;
  const sscan::ScanArgs a = make_args(u, z, y, dirs, ndir, reverse, softplus, batch, dim, len, io_dtype, bc_dtype);
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

}  // namespace

extern "C" {

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

size_t sscan_workspace_bytes(int64_t batch, int64_t dim, int64_t len, int64_t dstate, int bidir) {
  Sizes sz{};
  if (check_sizes(batch, dim, len, dstate, SSCAN_F32, SSCAN_F32, &sz) != SSCAN_OK) return 0;
  if (batch == 0 || dim == 0 || len == 0) return 0;
  return sscan::make_plan(batch, dim, len, bidir ? 2 : 1).workspace_bytes;
}

const char* sscan_strerror(int status) {
  switch (status) {
    case SSCAN_OK: return "ok";
    case SSCAN_ERR_NULL: return "a required pointer is NULL";
    case SSCAN_ERR_SHAPE: return "invalid sizes (negative, or too large)";
    case SSCAN_ERR_UNSUPPORTED: return "unsupported dstate (must be 16) or dtype code";
    case SSCAN_ERR_ALIGN: return "a pointer is not aligned to its element size (workspace: 16 bytes)";
    case SSCAN_ERR_WORKSPACE: return "workspace missing or smaller than sscan_workspace_bytes()";
    case SSCAN_ERR_HIP: return "HIP runtime error at launch";
    case SSCAN_ERR_ALIAS: return "the output overlaps an input or the workspace";
    default: return "unknown status";
  }
}

int sscan_version(void) { return kVersion; }

}  // extern "C"
