// C-ABI front end of libssmscan.so (include/ssm_scan.h).
//
// Every check here is plain host arithmetic on the parameter struct; nothing
// touches the HIP runtime until all checks have passed, so invalid calls
// return their status with no device-side effect (and can be exercised on a
// machine without a GPU). The launches themselves live in scan_fwd.hip,
// scan_bwd.hip and state_update.hip.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

ssm_status fail(ssm_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

ssm_status ok() {
  g_last_error[0] = '\0';
  return SSM_OK;
}

bool valid_dtype(int32_t t) { return t == SSM_F32 || t == SSM_BF16; }
bool valid_disc(int32_t t) { return t == SSM_DISC_DELTA_B || t == SSM_DISC_ZOH; }
bool valid_kind(int32_t k) { return k == SSM_STATE_REAL || k == SSM_STATE_COMPLEX; }

ssm_status check_kind(int32_t kind) {
  if (!valid_kind(kind)) return fail(SSM_ERR_UNSUPPORTED, "unknown state_kind %d", kind);
  return SSM_OK;
}
size_t dtype_size(int32_t t) { return t == SSM_BF16 ? 2 : 4; }

// a * b without overflow for non-negative operands.
bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
  *r = a * b;
  return true;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A byte range [p, p + n) of one tensor; empty when p is null.
struct Range {
  const char* p;
  size_t n;
  const char* name;
};

bool overlaps(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  return a.p < b.p + b.n && b.p < a.p + a.n;
}

Range range(const void* p, int64_t count, size_t esize, const char* name) {
  return Range{static_cast<const char*>(p), p ? static_cast<size_t>(count) * esize : 0, name};
}

// Sizes of a scan, checked for range and overflow.
struct ScanSizes {
  int64_t bdl, bln, dn, bdn, bl;
  bool empty() const { return bdl == 0; }  // no (b, d, t): nothing is scanned
};

ssm_status check_scan_sizes(const ssm_scan_params* p, ScanSizes* sz) {
  if (p->batch < 0 || p->dim < 0 || p->seqlen < 0)
    return fail(SSM_ERR_BAD_SHAPE, "batch, dim and seqlen must be >= 0 (got %lld, %lld, %lld)",
                (long long)p->batch, (long long)p->dim, (long long)p->seqlen);
  if (p->dstate < 1 || p->dstate > SSM_MAX_DSTATE)
    return fail(SSM_ERR_BAD_SHAPE, "dstate must be in [1, %d] (got %lld)", SSM_MAX_DSTATE,
                (long long)p->dstate);
  if (p->seqlen >= (int64_t{1} << 27))
    return fail(SSM_ERR_BAD_SHAPE, "seqlen must be below 2^27 (got %lld)", (long long)p->seqlen);
  int64_t bd;
  const int64_t lim = std::numeric_limits<int64_t>::max() / 8;
  if (!mul_ok(p->batch, p->dim, &bd) || !mul_ok(bd, p->seqlen, &sz->bdl) ||
      !mul_ok(p->batch, p->seqlen, &sz->bl) || !mul_ok(sz->bl, p->dstate, &sz->bln) ||
      !mul_ok(p->dim, p->dstate, &sz->dn) || !mul_ok(bd, p->dstate, &sz->bdn) || sz->bdl > lim ||
      sz->bln > lim || sz->bdn > lim)
    return fail(SSM_ERR_BAD_SHAPE, "element count overflows");
  return SSM_OK;
}

ssm_status plan_scan(const ssm_scan_params* p, int* nseg, int64_t* seg_len, size_t* ws) {
  if (p->num_segments < 0) return fail(SSM_ERR_BAD_SHAPE, "num_segments must be >= 0");
  if (p->batch == 0 || p->dim == 0 || p->seqlen == 0) {  // empty: no launch, no workspace
    *nseg = 1;
    *seg_len = p->seqlen;
    *ws = 0;
    return SSM_OK;
  }
  if (p->state_kind == SSM_STATE_COMPLEX) {
    ssm::plan_cplx_segments(p->batch, p->dim, p->seqlen, p->dstate, p->num_segments, nseg, seg_len);
    if (ssm::cplx_scan_grid_blocks(p->batch, p->dim, *nseg) > std::numeric_limits<int32_t>::max())
      return fail(SSM_ERR_BAD_SHAPE, "problem needs more workgroups than one launch allows");
    *ws = ssm::cplx_workspace_bytes(p->batch, p->dim, p->dstate, *nseg);
    return SSM_OK;
  }
  const bool plain = !p->conv_w && p->discretization != SSM_DISC_ZOH;
  ssm::plan_segments(p->batch, p->dim, p->seqlen, p->dstate, p->num_segments, nseg, seg_len, plain);
  if (ssm::scan_grid_blocks(p->batch, p->dim, p->dstate, *nseg) > std::numeric_limits<int32_t>::max())
    return fail(SSM_ERR_BAD_SHAPE, "problem needs more workgroups than one launch allows");
  *ws = ssm::scan_workspace_bytes(p->batch, p->dim, p->dstate, *nseg);
  return SSM_OK;
}

// Checks of a scan call's inputs shared by ssm_scan_fwd (aggregate = false)
// and ssm_scan_aggregate (aggregate = true: C, z, D, h0 and the outputs of
// the forward are not read). With pointers = false only sizes, types and
// flags are checked (the workspace-size queries).
constexpr int kScanInputs = 13;

struct ScanCheck {
  ScanSizes sz;
  int64_t K = 0, cw = 1, bdk = 0;
  size_t si = 4, so = 4;
  bool cplx = false;
};

ssm_status check_scan_inputs(const ssm_scan_params* p, bool aggregate, ScanCheck* c, Range (&inputs)[kScanInputs],
                             bool pointers = true) {
  ssm_status s = check_scan_sizes(p, &c->sz);
  if (s != SSM_OK) return s;
  const ScanSizes& sz = c->sz;
  if (!valid_dtype(p->in_dtype) || (!aggregate && !valid_dtype(p->out_dtype)))
    return fail(SSM_ERR_BAD_DTYPE, "in_dtype/out_dtype must be SSM_F32 or SSM_BF16");
  if (!valid_disc(p->discretization))
    return fail(SSM_ERR_UNSUPPORTED, "unknown discretization %d", p->discretization);
  if ((s = check_kind(p->state_kind)) != SSM_OK) return s;
  c->cplx = p->state_kind == SSM_STATE_COMPLEX;
  c->cw = c->cplx ? 2 : 1;
  c->K = p->conv_w ? p->conv_width : 0;
  if (p->conv_w && (c->K < 1 || c->K > 4))
    return fail(SSM_ERR_BAD_SHAPE, "conv_width must be in [1, 4] (got %d)", p->conv_width);
  if (!pointers) return SSM_OK;
  // A pointer to an empty tensor may be NULL.
  const struct {
    const void* ptr;
    int64_t count;
    const char* name;
  } required[] = {{p->u, sz.bdl, "u"}, {p->dt_raw, sz.bdl, "dt_raw"}, {p->A, sz.dn, "A"}, {p->Bm, sz.bln, "Bm"},
                  {p->Cm, aggregate ? 0 : sz.bln, "Cm"}, {p->out, aggregate ? 0 : sz.bdl, "out"}};
  for (const auto& r : required)
    if (!r.ptr && r.count > 0) return fail(SSM_ERR_NULL_POINTER, "%s is NULL", r.name);
  c->si = dtype_size(p->in_dtype);
  c->so = aggregate ? 4 : dtype_size(p->out_dtype);
  if (!p->conv_w && (p->conv_b || p->conv_state_in || p->conv_state_out))
    return fail(SSM_ERR_NULL_POINTER, "conv_b / conv_state given without conv_w");
  const int64_t K = c->K, cw = c->cw;
  const size_t si = c->si;
  c->bdk = sz.bdn / p->dstate * (K > 0 ? K - 1 : 0);  // B*D*(K-1)
  const void* z = aggregate ? nullptr : p->z;
  const void* Cm = aggregate ? nullptr : p->Cm;
  const void* Dskip = aggregate ? nullptr : p->Dskip;
  const void* h0 = aggregate ? nullptr : p->h0;
  const Range in[kScanInputs] = {
      range(p->u, sz.bdl, si, "u"),          range(p->dt_raw, sz.bdl, si, "dt_raw"),
      range(z, sz.bdl, si, "z"),             range(p->Bm, sz.bln * cw, si, "Bm"),
      range(Cm, sz.bln * cw, si, "Cm"),      range(p->A, sz.dn * cw, 4, "A"),
      range(p->dt_bias, p->dim, 4, "dt_bias"), range(Dskip, p->dim, 4, "Dskip"),
      range(p->reset, sz.bl, 1, "reset"),    range(h0, sz.bdn * cw, 4, "h0"),
      range(p->conv_w, p->dim * K, 4, "conv_w"), range(p->conv_b, p->dim, 4, "conv_b"),
      range(p->conv_state_in, c->bdk, 4, "conv_state_in"),
  };
  for (int i = 0; i < kScanInputs; ++i) inputs[i] = in[i];
  const struct {
    const void* ptr;
    size_t align;
    const char* name;
  } aligns[] = {{p->u, si, "u"},           {p->dt_raw, si, "dt_raw"}, {z, si, "z"},
                {p->Bm, si, "Bm"},         {Cm, si, "Cm"},            {p->A, 4, "A"},
                {p->dt_bias, 4, "dt_bias"}, {Dskip, 4, "Dskip"},      {h0, 4, "h0"},
                {aggregate ? nullptr : p->out, c->so, "out"},
                {aggregate ? nullptr : p->h_last, 4, "h_last"},       {p->workspace, 4, "workspace"},
                {p->conv_w, 4, "conv_w"},  {p->conv_b, 4, "conv_b"},  {p->conv_state_in, 4, "conv_state_in"},
                {aggregate ? nullptr : p->conv_state_out, 4, "conv_state_out"}};
  for (const auto& a : aligns)
    if (a.ptr && !aligned(a.ptr, a.align))
      return fail(SSM_ERR_MISALIGNED, "%s is not aligned to %zu bytes", a.name, a.align);
  return SSM_OK;
}

// The caller's workspace: large enough and clear of the inputs and outputs.
ssm_status check_workspace(const ssm_scan_params* p, size_t ws, const Range (&inputs)[kScanInputs],
                           const Range* outs, int n_outs) {
  if (ws == 0) return SSM_OK;
  if (!p->workspace || p->workspace_bytes < ws)
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws,
                p->workspace ? p->workspace_bytes : static_cast<size_t>(0));
  const Range w{static_cast<const char*>(p->workspace), ws, "workspace"};
  for (const Range& r : inputs)
    if (overlaps(w, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps %s", r.name);
  for (int i = 0; i < n_outs; ++i)
    if (overlaps(w, outs[i])) return fail(SSM_ERR_ALIAS, "workspace overlaps an output");
  return SSM_OK;
}

// The aggregate pass: every piece's aggregate goes to the workspace (then one
// fold into P and H) unless the sequence stays in one piece.
ssm_status plan_aggregate(const ssm_scan_params* p, int* nseg, int64_t* seg_len, size_t* ws) {
  if (p->num_segments < 0) return fail(SSM_ERR_BAD_SHAPE, "num_segments must be >= 0");
  if (p->batch == 0 || p->dim == 0 || p->seqlen == 0) {  // empty: no launch, no workspace
    *nseg = 1;
    *seg_len = p->seqlen;
    *ws = 0;
    return SSM_OK;
  }
  const bool cplx = p->state_kind == SSM_STATE_COMPLEX;
  if (cplx)
    ssm::plan_cplx_segments(p->batch, p->dim, p->seqlen, p->dstate, p->num_segments, nseg, seg_len);
  else
    ssm::plan_segments(p->batch, p->dim, p->seqlen, p->dstate, p->num_segments, nseg, seg_len, true, 512);
  const int64_t blocks = cplx ? ssm::cplx_scan_grid_blocks(p->batch, p->dim, *nseg)
                              : ssm::scan_grid_blocks(p->batch, p->dim, p->dstate, *nseg);
  if (blocks > std::numeric_limits<int32_t>::max())
    return fail(SSM_ERR_BAD_SHAPE, "problem needs more workgroups than one launch allows");
  *ws = *nseg > 1 ? static_cast<size_t>(2) * static_cast<size_t>(*nseg) * static_cast<size_t>(p->batch) *
                        static_cast<size_t>(p->dim) * static_cast<size_t>(p->dstate) * (cplx ? 2 : 1) *
                        sizeof(float)
                  : 0;
  return SSM_OK;
}

// The launch description common to the forward and the aggregate pass.
ssm::ScanPlan scan_plan(const ssm_scan_params* p, const ScanCheck& c, int nseg, int64_t seg_len, size_t ws) {
  ssm::ScanPlan plan{};
  plan.B = p->batch;
  plan.D = p->dim;
  plan.L = p->seqlen;
  plan.N = p->dstate;
  plan.in_bf16 = p->in_dtype == SSM_BF16;
  plan.out_bf16 = p->out_dtype == SSM_BF16;
  plan.u = p->u;
  plan.dt = p->dt_raw;
  plan.Bm = p->Bm;
  plan.dt_bias = p->dt_bias;
  plan.A = p->A;
  plan.reset = p->reset;
  plan.ws = ws > 0 ? static_cast<float*>(p->workspace) : nullptr;
  plan.nseg = nseg;
  plan.seg_len = seg_len;
  plan.zoh = p->discretization == SSM_DISC_ZOH;
  plan.conv_w = p->conv_w;
  plan.conv_b = p->conv_b;
  plan.conv_state_in = p->conv_state_in;
  plan.conv_k = static_cast<int>(c.K);
  return plan;
}

// Workspace layout of the backward pass (byte offsets, each 256-aligned).
struct BwdLayout {
  int nseg;           // pieces of the checkpoint sweep (forward split)
  int64_t seg_len;
  int nsegb;          // segments of the reverse sweep
  int64_t seg_steps;
  int64_t n_ck;       // 16-step checkpoints
  size_t off_agg, off_ckpt, off_segP, off_segG, off_part, off_uconv, off_duconv, off_convpart, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

ssm_status check_bwd_sizes(const ssm_scan_bwd_params* p, ScanSizes* sz) {
  ssm_scan_params f{};
  f.batch = p->batch;
  f.dim = p->dim;
  f.seqlen = p->seqlen;
  f.dstate = p->dstate;
  return check_scan_sizes(&f, sz);
}

ssm_status check_bwd_kind(const ssm_scan_bwd_params* p) { return check_kind(p->state_kind); }

// Complex state: checkpoints every 16 / NPL steps and complex aggregates,
// checkpoints and partials (two floats per value).
ssm_status plan_bwd_cplx(const ssm_scan_bwd_params* p, const ScanSizes& sz, BwdLayout* lay) {
  const int64_t B = p->batch, D = p->dim, L = p->seqlen, N = p->dstate;
  ssm::plan_cplx_bwd(B, D, L, N, &lay->nsegb, &lay->seg_steps, &lay->nseg, &lay->seg_len, &lay->n_ck);
  if (ssm::cplx_scan_grid_blocks(B, D, lay->nseg) > std::numeric_limits<int32_t>::max() ||
      ssm::cplx_bwd_grid_blocks(B, D, lay->nsegb) > std::numeric_limits<int32_t>::max())
    return fail(SSM_ERR_BAD_SHAPE, "problem needs more workgroups than one launch allows");
  int64_t ck, seg, part;
  const int64_t groups = (D + 15) / 16;
  if (!mul_ok(2 * sz.bdn, lay->n_ck, &ck) || !mul_ok(2 * sz.bdn, lay->nsegb, &seg) ||
      !mul_ok(2 * sz.bln, 2 * groups, &part) || ck > (int64_t{1} << 58) || seg > (int64_t{1} << 58) ||
      part > (int64_t{1} << 58))
    return fail(SSM_ERR_BAD_SHAPE, "backward workspace size overflows");
  size_t off = 0;
  lay->off_agg = off;
  off += align256(ssm::cplx_workspace_bytes(B, D, N, lay->nseg));
  lay->off_ckpt = off;
  off += align256(static_cast<size_t>(ck) * 4);
  lay->off_segP = off;
  off += align256(static_cast<size_t>(seg) * 4);
  lay->off_segG = off;
  off += align256(static_cast<size_t>(seg) * 4);
  lay->off_part = off;
  off += align256(ssm::cplx_bwd_partial_floats(B, D, L, N, lay->nsegb) * 4);
  lay->off_uconv = lay->off_duconv = lay->off_convpart = off;
  if (p->conv_w) {  // the conv stage's u' and its gradient, and the conv parameter partials
    lay->off_uconv = off;
    off += align256(static_cast<size_t>(sz.bdl) * 4);
    lay->off_duconv = off;
    off += align256(static_cast<size_t>(sz.bdl) * 4);
    lay->off_convpart = off;
    off += align256(ssm::bwd_conv_partial_floats(B, D, L) * 4);
  }
  lay->total = off;
  return SSM_OK;
}

ssm_status plan_bwd(const ssm_scan_bwd_params* p, const ScanSizes& sz, BwdLayout* lay) {
  if (sz.empty()) {  // nothing to sweep: no launch plan, no workspace
    *lay = BwdLayout{};
    lay->nseg = lay->nsegb = 1;
    return SSM_OK;
  }
  if (p->state_kind == SSM_STATE_COMPLEX) return plan_bwd_cplx(p, sz, lay);
  const int64_t B = p->batch, D = p->dim, L = p->seqlen, N = p->dstate;
  ssm::plan_bwd_segments(B, D, L, N, p->discretization == SSM_DISC_ZOH, &lay->nsegb, &lay->seg_steps);
  int nseg;
  int64_t seg_len;
  ssm::plan_segments(B, D, L, N, 0, &nseg, &seg_len);
  seg_len = (seg_len + lay->seg_steps - 1) / lay->seg_steps * lay->seg_steps;
  lay->seg_len = seg_len;
  lay->nseg = static_cast<int>((L + seg_len - 1) / seg_len);
  lay->n_ck = (L + 15) / 16;
  if (ssm::scan_grid_blocks(B, D, N, lay->nseg) > std::numeric_limits<int32_t>::max() ||
      ssm::bwd_grid_blocks(B, D, N, lay->nsegb) > std::numeric_limits<int32_t>::max())
    return fail(SSM_ERR_BAD_SHAPE, "problem needs more workgroups than one launch allows");
  int64_t ck, seg, part;
  const int64_t groups = (D + ssm::bwd_channels_per_block(N) - 1) / ssm::bwd_channels_per_block(N);
  if (!mul_ok(sz.bdn, lay->n_ck, &ck) || !mul_ok(sz.bdn, lay->nsegb, &seg) || !mul_ok(sz.bln, 2 * groups, &part) ||
      ck > (int64_t{1} << 58) || seg > (int64_t{1} << 58) || part > (int64_t{1} << 58))
    return fail(SSM_ERR_BAD_SHAPE, "backward workspace size overflows");
  size_t off = 0;
  lay->off_agg = off;
  off += align256(ssm::scan_workspace_bytes(B, D, N, lay->nseg));
  lay->off_ckpt = off;
  off += align256(static_cast<size_t>(ck) * 4);
  lay->off_segP = off;
  off += align256(static_cast<size_t>(seg) * 4);
  lay->off_segG = off;
  off += align256(static_cast<size_t>(seg) * 4);
  lay->off_part = off;
  off += align256(ssm::bwd_partial_floats(B, D, L, N, lay->nsegb) * 4);
  lay->off_uconv = lay->off_duconv = lay->off_convpart = off;
  if (p->conv_w) {  // the conv stage's u' and its gradient, and the conv parameter partials
    lay->off_uconv = off;
    off += align256(static_cast<size_t>(sz.bdl) * 4);
    lay->off_duconv = off;
    off += align256(static_cast<size_t>(sz.bdl) * 4);
    lay->off_convpart = off;
    off += align256(ssm::bwd_conv_partial_floats(B, D, L) * 4);
  }
  lay->total = off;
  return SSM_OK;
}

// The forward scan. With noalloc the split-scan buffer is the library's
// scratch on the current device instead of the caller's workspace (whose
// fields are then ignored); a split larger than the scratch is refused.
// With wavefront the scan runs as the chunked associative scan of
// scan_fwd_wavefront.hip (16 real states, delta B, no conv stage; never split).
ssm_status scan_fwd(const ssm_scan_params* p, void* hip_stream, bool noalloc, bool wavefront = false) {
  if (!p) return fail(SSM_ERR_NULL_POINTER, "params is NULL");
  ScanCheck c;
  Range inputs[kScanInputs];
  ssm_status s = check_scan_inputs(p, false, &c, inputs);
  if (s != SSM_OK) return s;
  if (wavefront && (p->dstate != 16 || c.cplx || p->discretization != SSM_DISC_DELTA_B || p->conv_w))
    return fail(SSM_ERR_UNSUPPORTED,
                "ssm_scan_fwd_wavefront supports dstate 16, real states, the delta B coefficient and no conv stage");
  if (wavefront && (!aligned(p->Bm, 16) || !aligned(p->Cm, 16)))  // its lanes load whole 16-state rows
    return fail(SSM_ERR_MISALIGNED, "ssm_scan_fwd_wavefront needs Bm and Cm aligned to 16 bytes");
  const ScanSizes& sz = c.sz;
  const Range out = range(p->out, sz.bdl, c.so, "out");
  const Range hl = range(p->h_last, sz.bdn * c.cw, 4, "h_last");
  const Range cso = range(p->conv_state_out, c.bdk, 4, "conv_state_out");
  for (const Range& r : inputs) {
    if (overlaps(out, r)) return fail(SSM_ERR_ALIAS, "out overlaps %s", r.name);
    if (overlaps(hl, r)) return fail(SSM_ERR_ALIAS, "h_last overlaps %s", r.name);
    if (overlaps(cso, r)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps %s", r.name);
  }
  if (overlaps(out, hl)) return fail(SSM_ERR_ALIAS, "out overlaps h_last");
  if (overlaps(out, cso) || overlaps(hl, cso)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps an output");

  int nseg;
  int64_t seg_len;
  size_t ws;
  if ((s = plan_scan(p, &nseg, &seg_len, &ws)) != SSM_OK) return s;
  if (wavefront) {  // one wave per (b, d) over the whole sequence
    nseg = 1;
    seg_len = p->seqlen;
    ws = 0;
    if ((p->batch * p->dim + 3) / 4 > std::numeric_limits<int32_t>::max())
      return fail(SSM_ERR_BAD_SHAPE, "problem needs more workgroups than one launch allows");
  }
  const Range outs[] = {out, hl, cso};
  if (noalloc) {
    if (ws > ssm::noalloc_scratch_bytes())
      return fail(SSM_ERR_WORKSPACE,
                  "this split needs %zu bytes of scratch; the allocation-free entry point holds %zu per device",
                  ws, ssm::noalloc_scratch_bytes());
  } else if ((s = check_workspace(p, ws, inputs, outs, 3)) != SSM_OK) {
    return s;
  }
  SSM_LOG("%s: B %lld D %lld L %lld N %lld, %s state, %s in, %s out, %s, conv width %lld, resets %d; %d pieces of "
          "%lld steps, workspace %zu bytes%s",
          noalloc ? "ssm_scan_fwd_noalloc" : wavefront ? "ssm_scan_fwd_wavefront" : "ssm_scan_fwd",
          (long long)p->batch, (long long)p->dim,
          (long long)p->seqlen, (long long)p->dstate, c.cplx ? "complex" : "real",
          p->in_dtype == SSM_BF16 ? "bf16" : "f32", p->out_dtype == SSM_BF16 ? "bf16" : "f32",
          p->discretization == SSM_DISC_ZOH ? "zoh" : "delta B", (long long)c.K, p->reset != nullptr, nseg,
          (long long)seg_len, ws, noalloc ? " (library scratch)" : "");
  if (sz.empty()) {  // the states pass through an empty sequence
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    hipError_t e = ssm::launch_fill(p->h_last, p->h0, 0.0f, 0.0f, sz.bdn * c.cw, st);
    if (e == hipSuccess) e = ssm::launch_fill(p->conv_state_out, p->conv_state_in, 0.0f, 0.0f, c.bdk, st);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "fill launch failed: %s", hipGetErrorString(e));
    return ok();
  }

  ssm::ScanPlan plan = scan_plan(p, c, nseg, seg_len, ws);
  if (noalloc && ws > 0) {
    void* scratch = nullptr;
    const hipError_t e = ssm::noalloc_scratch(&scratch);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
    plan.ws = static_cast<float*>(scratch);
  }
  plan.out = p->out;
  plan.h_last = p->h_last;
  plan.conv_state_out = p->conv_state_out;
  plan.Cm = p->Cm;
  plan.z = p->z;
  plan.Dskip = p->Dskip;
  plan.h0 = p->h0;
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = wavefront ? ssm::launch_scan_wavefront(plan, st)
                       : c.cplx  ? ssm::launch_scan_cplx(plan, st)
                                 : ssm::launch_scan(plan, st);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "scan launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

ssm_status ssm_scan_bwd_workspace_size(const ssm_scan_bwd_params* p, size_t* bytes) {
  if (!p || !bytes) return fail(SSM_ERR_NULL_POINTER, "params or bytes is NULL");
  ScanSizes sz;
  ssm_status s = check_bwd_sizes(p, &sz);
  if (s != SSM_OK) return s;
  if (!valid_dtype(p->in_dtype) || !valid_dtype(p->grad_dtype))
    return fail(SSM_ERR_BAD_DTYPE, "in_dtype/grad_dtype must be SSM_F32 or SSM_BF16");
  if (!valid_disc(p->discretization))
    return fail(SSM_ERR_UNSUPPORTED, "unknown discretization %d", p->discretization);
  if ((s = check_bwd_kind(p)) != SSM_OK) return s;
  BwdLayout lay;
  if ((s = plan_bwd(p, sz, &lay)) != SSM_OK) return s;
  *bytes = lay.total;
  return ok();
}

ssm_status ssm_scan_bwd(const ssm_scan_bwd_params* p, void* hip_stream) {
  if (!p) return fail(SSM_ERR_NULL_POINTER, "params is NULL");
  ScanSizes sz;
  ssm_status s = check_bwd_sizes(p, &sz);
  if (s != SSM_OK) return s;
  if (!valid_dtype(p->in_dtype) || !valid_dtype(p->grad_dtype))
    return fail(SSM_ERR_BAD_DTYPE, "in_dtype/grad_dtype must be SSM_F32 or SSM_BF16");
  const struct {  // a pointer to an empty tensor may be NULL; the workspace is checked below
    const void* ptr;
    int64_t count;
    const char* name;
  } required[] = {{p->u, sz.bdl, "u"},   {p->dt_raw, sz.bdl, "dt_raw"}, {p->A, sz.dn, "A"},
                  {p->Bm, sz.bln, "Bm"}, {p->Cm, sz.bln, "Cm"},         {p->dout, sz.bdl, "dout"},
                  {p->du, sz.bdl, "du"}, {p->d_dt_raw, sz.bdl, "d_dt_raw"}, {p->dA, sz.dn, "dA"},
                  {p->dBm, sz.bln, "dBm"}, {p->dCm, sz.bln, "dCm"}};
  for (const auto& r : required)
    if (!r.ptr && r.count > 0) return fail(SSM_ERR_NULL_POINTER, "%s is NULL", r.name);
  if (p->z && !p->dz && sz.bdl > 0) return fail(SSM_ERR_NULL_POINTER, "dz is NULL although z is given");
  if (!p->z && p->dz) return fail(SSM_ERR_BAD_SHAPE, "dz is given although z is NULL");
  if (!valid_disc(p->discretization))
    return fail(SSM_ERR_UNSUPPORTED, "unknown discretization %d", p->discretization);
  if ((s = check_bwd_kind(p)) != SSM_OK) return s;
  const bool cplx = p->state_kind == SSM_STATE_COMPLEX;
  const int64_t cw = cplx ? 2 : 1;  // scalars per A, B, C and state entry
  const int64_t K = p->conv_w ? p->conv_width : 0;
  if (p->conv_w && (K < 1 || K > 4)) return fail(SSM_ERR_BAD_SHAPE, "conv_width must be in [1, 4] (got %d)", p->conv_width);
  if (!p->conv_w && (p->conv_b || p->conv_state_in || p->dconv_w || p->dconv_b || p->dconv_state_in))
    return fail(SSM_ERR_NULL_POINTER, "conv arguments given without conv_w");
  const int64_t bdk = sz.bdn / p->dstate * (K > 0 ? K - 1 : 0);

  const size_t si = dtype_size(p->in_dtype), sg = dtype_size(p->grad_dtype);
  const struct {
    const void* ptr;
    size_t align;
    const char* name;
  } aligns[] = {{p->u, si, "u"},           {p->dt_raw, si, "dt_raw"},   {p->z, si, "z"},
                {p->Bm, si, "Bm"},         {p->Cm, si, "Cm"},           {p->dout, si, "dout"},
                {p->A, 4, "A"},            {p->dt_bias, 4, "dt_bias"},  {p->Dskip, 4, "Dskip"},
                {p->h0, 4, "h0"},          {p->dh_last, 4, "dh_last"},  {p->du, sg, "du"},
                {p->d_dt_raw, sg, "d_dt_raw"}, {p->dz, sg, "dz"},       {p->dA, 4, "dA"},
                {p->dBm, 4, "dBm"},        {p->dCm, 4, "dCm"},          {p->dDskip, 4, "dDskip"},
                {p->d_dt_bias, 4, "d_dt_bias"}, {p->dh0, 4, "dh0"},     {p->workspace, 16, "workspace"},
                {p->conv_w, 4, "conv_w"},  {p->conv_b, 4, "conv_b"},    {p->conv_state_in, 4, "conv_state_in"},
                {p->dconv_w, 4, "dconv_w"}, {p->dconv_b, 4, "dconv_b"}, {p->dconv_state_in, 4, "dconv_state_in"}};
  for (const auto& a : aligns)
    if (a.ptr && !aligned(a.ptr, a.align))
      return fail(SSM_ERR_MISALIGNED, "%s is not aligned to %zu bytes", a.name, a.align);

  BwdLayout lay;
  if ((s = plan_bwd(p, sz, &lay)) != SSM_OK) return s;
  if (lay.total > 0 && !p->workspace) return fail(SSM_ERR_NULL_POINTER, "workspace is NULL");
  if (p->workspace_bytes < lay.total)
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total, p->workspace_bytes);

  const Range inputs[] = {
      range(p->u, sz.bdl, si, "u"),          range(p->dt_raw, sz.bdl, si, "dt_raw"),
      range(p->z, sz.bdl, si, "z"),          range(p->Bm, cw * sz.bln, si, "Bm"),
      range(p->Cm, cw * sz.bln, si, "Cm"),   range(p->A, cw * sz.dn, 4, "A"),
      range(p->dt_bias, p->dim, 4, "dt_bias"), range(p->Dskip, p->dim, 4, "Dskip"),
      range(p->reset, sz.bl, 1, "reset"),    range(p->h0, cw * sz.bdn, 4, "h0"),
      range(p->dout, sz.bdl, si, "dout"),    range(p->dh_last, cw * sz.bdn, 4, "dh_last"),
      range(p->conv_w, p->dim * K, 4, "conv_w"), range(p->conv_b, p->dim, 4, "conv_b"),
      range(p->conv_state_in, bdk, 4, "conv_state_in"),
  };
  const Range outputs[] = {
      range(p->du, sz.bdl, sg, "du"),        range(p->d_dt_raw, sz.bdl, sg, "d_dt_raw"),
      range(p->dz, sz.bdl, sg, "dz"),        range(p->dA, cw * sz.dn, 4, "dA"),
      range(p->dBm, cw * sz.bln, 4, "dBm"),  range(p->dCm, cw * sz.bln, 4, "dCm"),
      range(p->dDskip, p->dim, 4, "dDskip"), range(p->d_dt_bias, p->dim, 4, "d_dt_bias"),
      range(p->dh0, cw * sz.bdn, 4, "dh0"),
      range(p->dconv_w, p->dim * K, 4, "dconv_w"), range(p->dconv_b, p->dim, 4, "dconv_b"),
      range(p->dconv_state_in, bdk, 4, "dconv_state_in"),
      Range{lay.total ? static_cast<const char*>(p->workspace) : nullptr, lay.total, "workspace"},
  };
  constexpr int n_out = sizeof(outputs) / sizeof(outputs[0]);
  for (int i = 0; i < n_out; ++i) {
    for (const Range& r : inputs)
      if (overlaps(outputs[i], r)) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outputs[i].name, r.name);
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outputs[i], outputs[j]))
        return fail(SSM_ERR_ALIAS, "%s overlaps %s", outputs[i].name, outputs[j].name);
  }

  char* ws = static_cast<char*>(p->workspace);
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (sz.empty()) {
    // Sums over no (b, t) or no channel are 0; the adjoint passes through an
    // empty sequence (h_last = h0); the outputs do not depend on the initial
    // conv state.
    hipError_t e = ssm::launch_fill(p->dA, nullptr, 0.0f, 0.0f, cw * sz.dn, stream);
    if (e == hipSuccess) e = ssm::launch_fill(p->dBm, nullptr, 0.0f, 0.0f, cw * sz.bln, stream);
    if (e == hipSuccess) e = ssm::launch_fill(p->dCm, nullptr, 0.0f, 0.0f, cw * sz.bln, stream);
    const struct {
      float* dst;
      const float* src;
      int64_t n;
    } fills[] = {{p->dDskip, nullptr, p->dim}, {p->d_dt_bias, nullptr, p->dim}, {p->dconv_w, nullptr, p->dim * K},
                 {p->dconv_b, nullptr, p->dim}, {p->dconv_state_in, nullptr, bdk}, {p->dh0, p->dh_last, cw * sz.bdn}};
    for (const auto& f : fills)
      if (e == hipSuccess) e = ssm::launch_fill(f.dst, f.src, 0.0f, 0.0f, f.n, stream);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "fill launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  ssm::ScanPlan sp{};
  sp.B = p->batch;
  sp.D = p->dim;
  sp.L = p->seqlen;
  sp.N = p->dstate;
  sp.in_bf16 = p->in_dtype == SSM_BF16;
  sp.u = p->u;
  sp.dt = p->dt_raw;
  sp.z = p->z;
  sp.Bm = p->Bm;
  sp.Cm = p->Cm;
  sp.dt_bias = p->dt_bias;
  sp.A = p->A;
  sp.Dskip = p->Dskip;
  sp.h0 = p->h0;
  sp.reset = p->reset;
  sp.ws = lay.nseg > 1 ? reinterpret_cast<float*>(ws + lay.off_agg) : nullptr;
  sp.nseg = lay.nseg;
  sp.seg_len = lay.seg_len;
  sp.checkpoint = 1;
  sp.dout = p->dout;
  sp.ckpt = reinterpret_cast<float*>(ws + lay.off_ckpt);
  sp.seg_P = reinterpret_cast<float*>(ws + lay.off_segP);
  sp.seg_G = reinterpret_cast<float*>(ws + lay.off_segG);
  sp.seg_steps = lay.seg_steps;
  sp.n_ck = lay.n_ck;
  sp.nsegb = lay.nsegb;
  sp.conv_w = p->conv_w;
  sp.conv_b = p->conv_b;
  sp.conv_state_in = p->conv_state_in;
  sp.conv_k = static_cast<int>(K);
  sp.uconv_out = p->conv_w ? reinterpret_cast<float*>(ws + lay.off_uconv) : nullptr;
  sp.zoh = p->discretization == SSM_DISC_ZOH;
  SSM_LOG("ssm_scan_bwd: B %lld D %lld L %lld N %lld, %s state; checkpoint sweep in %d pieces of %lld steps, "
          "reverse sweep in %d segments of %lld steps, workspace %zu bytes",
          (long long)p->batch, (long long)p->dim, (long long)p->seqlen, (long long)p->dstate,
          cplx ? "complex" : "real", lay.nseg, (long long)lay.seg_len, lay.nsegb, (long long)lay.seg_steps,
          lay.total);
  hipError_t e = hipSuccess;
  if (!cplx) {
    e = ssm::launch_scan(sp, stream);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "checkpoint sweep launch failed: %s", hipGetErrorString(e));
  }

  ssm::BwdPlan bp{};
  bp.B = p->batch;
  bp.D = p->dim;
  bp.L = p->seqlen;
  bp.N = p->dstate;
  bp.in_bf16 = p->in_dtype == SSM_BF16;
  bp.grad_bf16 = p->grad_dtype == SSM_BF16;
  bp.u = p->u;
  bp.dt = p->dt_raw;
  bp.z = p->z;
  bp.Bm = p->Bm;
  bp.Cm = p->Cm;
  bp.dout = p->dout;
  bp.dt_bias = p->dt_bias;
  bp.A = p->A;
  bp.Dskip = p->Dskip;
  bp.reset = p->reset;
  bp.dh_last = p->dh_last;
  bp.ckpt = sp.ckpt;
  bp.seg_P = sp.seg_P;
  bp.seg_G = sp.seg_G;
  bp.du = p->du;
  bp.ddt = p->d_dt_raw;
  bp.dz = p->dz;
  bp.dA = p->dA;
  bp.dB = p->dBm;
  bp.dC = p->dCm;
  bp.dD = p->dDskip;
  bp.dbias = p->d_dt_bias;
  bp.dh0 = p->dh0;
  bp.part = reinterpret_cast<float*>(ws + lay.off_part);
  bp.seg_steps = lay.seg_steps;
  bp.n_ck = lay.n_ck;
  bp.nsegb = lay.nsegb;
  bp.conv_w = p->conv_w;
  bp.conv_b = p->conv_b;
  bp.conv_state_in = p->conv_state_in;
  bp.conv_k = static_cast<int>(K);
  bp.uconv = sp.uconv_out;
  bp.du_conv = p->conv_w ? reinterpret_cast<float*>(ws + lay.off_duconv) : nullptr;
  bp.conv_part = p->conv_w ? reinterpret_cast<float*>(ws + lay.off_convpart) : nullptr;
  bp.dconv_w = p->dconv_w;
  bp.dconv_b = p->dconv_b;
  bp.dconv_state = K > 1 ? p->dconv_state_in : nullptr;
  bp.zoh = p->discretization == SSM_DISC_ZOH;
  if (cplx) {
    e = ssm::launch_scan_cplx_bwd(sp, bp, stream);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "complex backward launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  e = ssm::launch_scan_bwd(bp, stream);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "reverse sweep launch failed: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_scan_workspace_size(const ssm_scan_params* p, size_t* bytes) {
  if (!p || !bytes) return fail(SSM_ERR_NULL_POINTER, "params or bytes is NULL");
  ScanSizes sz;
  ssm_status s = check_scan_sizes(p, &sz);
  if (s != SSM_OK) return s;
  if (!valid_dtype(p->in_dtype) || !valid_dtype(p->out_dtype))
    return fail(SSM_ERR_BAD_DTYPE, "in_dtype/out_dtype must be SSM_F32 or SSM_BF16");
  if (!valid_kind(p->state_kind)) return fail(SSM_ERR_UNSUPPORTED, "unknown state_kind %d", p->state_kind);
  int nseg;
  int64_t seg_len;
  size_t ws;
  if ((s = plan_scan(p, &nseg, &seg_len, &ws)) != SSM_OK) return s;
  *bytes = ws;
  return ok();
}

ssm_status ssm_scan_fwd(const ssm_scan_params* p, void* hip_stream) { return scan_fwd(p, hip_stream, false); }

ssm_status ssm_scan_fwd_noalloc(const ssm_scan_params* p, void* hip_stream) { return scan_fwd(p, hip_stream, true); }

ssm_status ssm_scan_fwd_wavefront(const ssm_scan_params* p, void* hip_stream) {
  return scan_fwd(p, hip_stream, false, true);
}

ssm_status ssm_scan_aggregate_workspace_size(const ssm_scan_params* p, size_t* bytes) {
  if (!p || !bytes) return fail(SSM_ERR_NULL_POINTER, "params or bytes is NULL");
  ScanCheck c;
  Range inputs[kScanInputs];
  ssm_status s = check_scan_inputs(p, true, &c, inputs, false);
  if (s != SSM_OK) return s;
  int nseg;
  int64_t seg_len;
  size_t ws;
  if ((s = plan_aggregate(p, &nseg, &seg_len, &ws)) != SSM_OK) return s;
  *bytes = ws;
  return ok();
}

ssm_status ssm_scan_aggregate(const ssm_scan_params* p, float* P, float* H, void* hip_stream) {
  if (!p) return fail(SSM_ERR_NULL_POINTER, "params is NULL");
  ScanCheck c;
  Range inputs[kScanInputs];
  ssm_status s = check_scan_inputs(p, true, &c, inputs);
  if (s != SSM_OK) return s;
  if ((!P || !H) && c.sz.bdn > 0) return fail(SSM_ERR_NULL_POINTER, "P or H is NULL");
  if (!aligned(P, 4) || !aligned(H, 4)) return fail(SSM_ERR_MISALIGNED, "P and H must be 4-byte aligned");
  const Range rp = range(P, c.sz.bdn * c.cw, 4, "P"), rh = range(H, c.sz.bdn * c.cw, 4, "H");
  for (const Range& r : inputs) {
    if (overlaps(rp, r)) return fail(SSM_ERR_ALIAS, "P overlaps %s", r.name);
    if (overlaps(rh, r)) return fail(SSM_ERR_ALIAS, "H overlaps %s", r.name);
  }
  if (overlaps(rp, rh)) return fail(SSM_ERR_ALIAS, "P overlaps H");
  int nseg;
  int64_t seg_len;
  size_t ws;
  if ((s = plan_aggregate(p, &nseg, &seg_len, &ws)) != SSM_OK) return s;
  const Range outs[] = {rp, rh};
  if ((s = check_workspace(p, ws, inputs, outs, 2)) != SSM_OK) return s;
  SSM_LOG("ssm_scan_aggregate: B %lld D %lld L %lld N %lld, %s state; %d pieces of %lld steps, workspace %zu bytes",
          (long long)p->batch, (long long)p->dim, (long long)p->seqlen, (long long)p->dstate,
          c.cplx ? "complex" : "real", nseg, (long long)seg_len, ws);
  if (c.sz.empty()) {  // an empty sequence is the identity map: P = 1, H = 0
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    hipError_t e = ssm::launch_fill(P, nullptr, 1.0f, c.cplx ? 0.0f : 1.0f, c.sz.bdn * c.cw, st);
    if (e == hipSuccess) e = ssm::launch_fill(H, nullptr, 0.0f, 0.0f, c.sz.bdn * c.cw, st);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "fill launch failed: %s", hipGetErrorString(e));
    return ok();
  }

  ssm::ScanPlan plan = scan_plan(p, c, nseg, seg_len, ws);
  const hipError_t e = c.cplx ? ssm::launch_aggregate_cplx(plan, P, H, static_cast<hipStream_t>(hip_stream))
                              : ssm::launch_aggregate(plan, P, H, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "aggregate launch failed: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_state_update(const ssm_update_params* p, void* hip_stream) {
  if (!p) return fail(SSM_ERR_NULL_POINTER, "params is NULL");
  if (p->batch < 0 || p->dim < 0)
    return fail(SSM_ERR_BAD_SHAPE, "batch and dim must be >= 0 (got %lld, %lld)", (long long)p->batch,
                (long long)p->dim);
  if (p->dstate < 1 || p->dstate > SSM_MAX_DSTATE)
    return fail(SSM_ERR_BAD_SHAPE, "dstate must be in [1, %d] (got %lld)", SSM_MAX_DSTATE,
                (long long)p->dstate);
  int64_t bd, bdn, bn, dn;
  if (!mul_ok(p->batch, p->dim, &bd) || !mul_ok(bd, p->dstate, &bdn) || !mul_ok(p->batch, p->dstate, &bn) ||
      !mul_ok(p->dim, p->dstate, &dn) || bdn > std::numeric_limits<int64_t>::max() / 8)
    return fail(SSM_ERR_BAD_SHAPE, "element count overflows");
  if ((bd + 3) / 4 > std::numeric_limits<int32_t>::max())
    return fail(SSM_ERR_BAD_SHAPE, "problem needs more workgroups than one launch allows");
  if (!valid_dtype(p->in_dtype) || !valid_dtype(p->out_dtype))
    return fail(SSM_ERR_BAD_DTYPE, "in_dtype/out_dtype must be SSM_F32 or SSM_BF16");
  const struct {  // a pointer to an empty tensor may be NULL
    const void* ptr;
    int64_t count;
    const char* name;
  } required[] = {{p->h, bdn, "h"}, {p->u, bd, "u"}, {p->dt_raw, bd, "dt_raw"}, {p->A, dn, "A"},
                  {p->Bm, bn, "Bm"}, {p->Cm, bn, "Cm"}, {p->out, bd, "out"}};
  for (const auto& r : required)
    if (!r.ptr && r.count > 0) return fail(SSM_ERR_NULL_POINTER, "%s is NULL", r.name);
  const size_t si = dtype_size(p->in_dtype), so = dtype_size(p->out_dtype);
  const struct {
    const void* ptr;
    size_t align;
    const char* name;
  } aligns[] = {{p->h, 4, "h"},   {p->u, si, "u"},   {p->dt_raw, si, "dt_raw"}, {p->z, si, "z"},
                {p->dt_bias, 4, "dt_bias"}, {p->A, 4, "A"}, {p->Dskip, 4, "Dskip"}, {p->Bm, si, "Bm"},
                {p->Cm, si, "Cm"}, {p->out, so, "out"}};
  for (const auto& a : aligns)
    if (a.ptr && !aligned(a.ptr, a.align))
      return fail(SSM_ERR_MISALIGNED, "%s is not aligned to %zu bytes", a.name, a.align);
  if (!valid_disc(p->discretization))
    return fail(SSM_ERR_UNSUPPORTED, "unknown discretization %d", p->discretization);
  ssm_status s = check_kind(p->state_kind);
  if (s != SSM_OK) return s;
  const bool cplx = p->state_kind == SSM_STATE_COMPLEX;
  const int64_t ce = cplx ? 2 : 1;  // scalars per A, B, C and state entry
  const Range inputs[] = {range(p->u, bd, si, "u"),         range(p->dt_raw, bd, si, "dt_raw"),
                          range(p->z, bd, si, "z"),         range(p->dt_bias, p->dim, 4, "dt_bias"),
                          range(p->A, dn * ce, 4, "A"),     range(p->Dskip, p->dim, 4, "Dskip"),
                          range(p->Bm, bn * ce, si, "Bm"),  range(p->Cm, bn * ce, si, "Cm")};
  const int64_t K = p->conv_w ? p->conv_width : 0;
  if (p->conv_w && (K < 1 || K > 4)) return fail(SSM_ERR_BAD_SHAPE, "conv_width must be in [1, 4] (got %d)", p->conv_width);
  if (!p->conv_w && (p->conv_b || p->conv_state))
    return fail(SSM_ERR_NULL_POINTER, "conv_b / conv_state given without conv_w");
  if (K > 1 && !p->conv_state && bd > 0)
    return fail(SSM_ERR_NULL_POINTER, "conv_state is NULL although conv_width > 1");
  for (const void* q : {static_cast<const void*>(p->conv_state), static_cast<const void*>(p->conv_w),
                        static_cast<const void*>(p->conv_b)})
    if (q && !aligned(q, 4)) return fail(SSM_ERR_MISALIGNED, "a conv pointer is not aligned to 4 bytes");
  const Range cw = range(p->conv_w, p->dim * K, 4, "conv_w"), cb = range(p->conv_b, p->dim, 4, "conv_b");
  const Range cs = range(K > 1 ? p->conv_state : nullptr, bd * (K - 1), 4, "conv_state");
  const Range h = range(p->h, bdn * ce, 4, "h");
  const Range out = range(p->out, bd, so, "out");
  for (const Range& r : inputs) {
    if (overlaps(h, r)) return fail(SSM_ERR_ALIAS, "h overlaps %s", r.name);
    if (overlaps(out, r)) return fail(SSM_ERR_ALIAS, "out overlaps %s", r.name);
    if (overlaps(cs, r)) return fail(SSM_ERR_ALIAS, "conv_state overlaps %s", r.name);
  }
  if (overlaps(out, h)) return fail(SSM_ERR_ALIAS, "out overlaps h");
  for (const Range& r : {h, out, cw, cb})
    if (overlaps(cs, r)) return fail(SSM_ERR_ALIAS, "conv_state overlaps %s", r.name);
  if (overlaps(h, cw) || overlaps(h, cb) || overlaps(out, cw) || overlaps(out, cb))
    return fail(SSM_ERR_ALIAS, "h or out overlaps a conv parameter");

  if (bd == 0) return ok();  // no rows: nothing to update

  ssm::UpdatePlan plan{};
  plan.B = p->batch;
  plan.D = p->dim;
  plan.N = p->dstate;
  plan.in_bf16 = p->in_dtype == SSM_BF16;
  plan.out_bf16 = p->out_dtype == SSM_BF16;
  plan.h = p->h;
  plan.u = p->u;
  plan.dt = p->dt_raw;
  plan.z = p->z;
  plan.dt_bias = p->dt_bias;
  plan.A = p->A;
  plan.Dskip = p->Dskip;
  plan.Bm = p->Bm;
  plan.Cm = p->Cm;
  plan.out = p->out;
  plan.conv_state = K > 1 ? p->conv_state : nullptr;
  plan.conv_w = p->conv_w;
  plan.conv_b = p->conv_b;
  plan.conv_k = static_cast<int>(K);
  plan.zoh = p->discretization == SSM_DISC_ZOH;
  SSM_LOG("ssm_state_update: B %lld D %lld N %lld, %s state, %s in, conv width %lld", (long long)p->batch,
          (long long)p->dim, (long long)p->dstate, cplx ? "complex" : "real", plan.in_bf16 ? "bf16" : "f32",
          (long long)K);
  hipError_t e = cplx ? ssm::launch_state_update_cplx(plan, static_cast<hipStream_t>(hip_stream))
                      : ssm::launch_state_update(plan, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "state update launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* ssm_status_string(int32_t status) {
  switch (status) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_NULL_POINTER: return "SSM_ERR_NULL_POINTER";
    case SSM_ERR_BAD_SHAPE: return "SSM_ERR_BAD_SHAPE";
    case SSM_ERR_BAD_DTYPE: return "SSM_ERR_BAD_DTYPE";
    case SSM_ERR_MISALIGNED: return "SSM_ERR_MISALIGNED";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE";
    case SSM_ERR_ALIAS: return "SSM_ERR_ALIAS";
    case SSM_ERR_HIP: return "SSM_ERR_HIP";
    default: return "unknown status";
  }
}

const char* ssm_last_error(void) { return g_last_error; }

int32_t ssm_version(void) { return SSM_SCAN_VERSION; }

size_t ssm_abi_struct_size(int32_t which) {
  if (which == 0) return sizeof(ssm_scan_params);
  if (which == 1) return sizeof(ssm_update_params);
  if (which == 2) return sizeof(ssm_scan_bwd_params);
  return 0;
}

}  // extern "C"
