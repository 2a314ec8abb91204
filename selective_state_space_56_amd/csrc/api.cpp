// C ABI of the selective scan library: argument validation, planning and
// dispatch to the HIP kernels. See include/mamba_scan.h for the contract.
#include "mamba_scan.h"
#include "mamba_scan_bwd.h"
#include "mamba_ssd.h"
#include "mamba_conv.h"

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>

#include "conv.h"
#include "kernels.h"
#include "scan_split.h"

namespace {

thread_local std::string g_last_error;

mamba_status fail(mamba_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mamba_status ok() {
  g_last_error.clear();
  return MAMBA_OK;
}

bool supported_dstate(int64_t n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

size_t io_bytes(int32_t io) { return io == MAMBA_BF16 ? 2 : 4; }

struct Span {
  const char* name;
  const void* p;
  size_t bytes;
};

bool overlaps(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const auto a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Checks the descriptor fields common to both entry points.
mamba_status check_desc(const mamba_scan_desc* d, const char* who) {
  if (!d) return fail(MAMBA_ERR_INVALID_ARG, "%s: desc is NULL", who);
  if (d->batch < 0 || d->seqlen < 0 || d->dim < 0)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: negative size (batch=%lld seqlen=%lld dim=%lld)", who,
                (long long)d->batch, (long long)d->seqlen, (long long)d->dim);
  if (d->io_dtype != MAMBA_F32 && d->io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: io_dtype %d is not MAMBA_F32 or MAMBA_BF16", who,
                (int)d->io_dtype);
  if (d->dstate < 1) return fail(MAMBA_ERR_INVALID_ARG, "%s: dstate %lld < 1", who, (long long)d->dstate);
  if (!supported_dstate(d->dstate))
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: dstate %lld not supported (1, 2, 4, 8 or 16)", who,
                (long long)d->dstate);
  // Keep every element index and grid size well inside 63 and 32 bits.
  const int64_t lim = int64_t(1) << 40;
  // one time step of one tensor (dim * 4 bytes) must stay far below 2^31
  if (d->dim > (int64_t(1) << 26))
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: dim %lld too large", who, (long long)d->dim);
  if (d->batch > lim || d->seqlen > lim || d->dim > lim ||
      (d->batch && d->dim && d->batch > (int64_t(1) << 31) / d->dim) ||
      (d->batch * d->dim && d->seqlen > lim / (d->batch * d->dim)))
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: problem too large", who);
  return MAMBA_OK;
}

int forced_segments(const mamba_scan_desc* d) { return static_cast<int>(d->flags & 0xffffu); }

constexpr uint32_t kFwdFlags = 0xffffu | MAMBA_SCAN_ZOH | MAMBA_SCAN_SPLIT_STATES;

// MAMBA_SCAN_SPLIT_STATES: 0 not asked for, 1 asked for and applicable, -1
// asked for what the state-split kernel does not do.
int split_mode(const mamba_scan_desc* d, int64_t row_elems) {
  if (!(d->flags & MAMBA_SCAN_SPLIT_STATES)) return 0;
  const bool fits = !(d->flags & MAMBA_SCAN_ZOH) && forced_segments(d) == 0 &&
                    mscan::scan_split_fits(d->dstate, row_elems, d->io_dtype);
  return fits ? 1 : -1;
}

int64_t groups_of(const mamba_scan_desc* d) { return d->ngroups > 1 ? d->ngroups : 1; }

// Channel groups: G must divide dim; the full-sequence kernels stage one
// group's B and C per 256-channel tile, so there each group must be a whole
// number of tiles.
mamba_status check_groups(const mamba_scan_desc* d, const char* who, bool tiles) {
  if (d->ngroups < 0)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: ngroups %lld < 0", who, (long long)d->ngroups);
  const int64_t G = groups_of(d);
  if (G > 1 && (d->dim % G) != 0)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: dim %lld is not a multiple of ngroups %lld", who,
                (long long)d->dim, (long long)G);
  if (G > 1 && tiles && (d->dim / G) % 256 != 0)
    return fail(MAMBA_ERR_UNSUPPORTED,
                "%s: with %lld groups each group must be a multiple of 256 channels", who,
                (long long)G);
  return MAMBA_OK;
}

// Row strides of the token tensors, resolved: 0 in the caller's struct (or no
// struct) means contiguous rows.
struct Rows {
  int64_t x, d, z, o, bc;
};

mamba_status resolve_rows(const mamba_scan_strides* s, const mamba_scan_desc* d, const char* who,
                          Rows& r) {
  const int64_t G = groups_of(d);
  const int64_t bc_min = G * d->dstate;
  r = Rows{d->dim, d->dim, d->dim, d->dim, bc_min};
  if (!s) return MAMBA_OK;
  const struct {
    const char* name;
    int64_t given, min;
    int64_t* dst;
  } f[] = {{"x", s->x, d->dim, &r.x}, {"delta", s->delta, d->dim, &r.d}, {"z", s->z, d->dim, &r.z},
           {"out", s->out, d->dim, &r.o}, {"bc", s->bc, bc_min, &r.bc}};
  for (const auto& e : f) {
    if (e.given == 0) continue;
    if (e.given < e.min)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: %s stride %lld is below its row length %lld", who,
                  e.name, (long long)e.given, (long long)e.min);
    // one row of one tensor (stride * 4 bytes) must stay far below 2^31
    if (e.given > (int64_t(1) << 26))
      return fail(MAMBA_ERR_UNSUPPORTED, "%s: %s stride %lld too large", who, e.name,
                  (long long)e.given);
    *e.dst = e.given;
  }
  return MAMBA_OK;
}

int64_t widest(const Rows& r) {
  int64_t w = r.x;
  for (int64_t v : {r.d, r.z, r.o, r.bc}) w = v > w ? v : w;
  return w;
}

// Bytes spanned by `rows` rows of `len` elements `stride` elements apart.
size_t span_bytes(int64_t rows, int64_t stride, int64_t len, size_t eb) {
  return rows > 0 ? static_cast<size_t>((rows - 1) * stride + len) * eb : 0;
}

}  // namespace

extern "C" {

const char* mamba_status_string(int s) {
  switch (s) {
    case MAMBA_OK: return "MAMBA_OK";
    case MAMBA_ERR_INVALID_ARG: return "MAMBA_ERR_INVALID_ARG";
    case MAMBA_ERR_UNSUPPORTED: return "MAMBA_ERR_UNSUPPORTED";
    case MAMBA_ERR_HIP: return "MAMBA_ERR_HIP";
    default: return "MAMBA_ERR_UNKNOWN";
  }
}

const char* mamba_last_error(void) { return g_last_error.c_str(); }

size_t mamba_scan_workspace_size_strided(const mamba_scan_desc* d, const mamba_scan_strides* s) {
  const char* who = "mamba_scan_workspace_size";
  if (check_desc(d, who) != MAMBA_OK) return 0;
  if (d->flags & ~kFwdFlags) return 0;
  if (check_groups(d, who, true) != MAMBA_OK) return 0;
  Rows r;
  if (resolve_rows(s, d, who, r) != MAMBA_OK) return 0;
  const int split = split_mode(d, widest(r));
  if (split != 0) return 0;  // the state-split kernel needs none
  return mscan::plan_scan(d->batch, d->seqlen, d->dim, static_cast<int>(d->dstate),
                          forced_segments(d), widest(r))
      .workspace_bytes;
}

size_t mamba_scan_workspace_size(const mamba_scan_desc* d) {
  return mamba_scan_workspace_size_strided(d, nullptr);
}

}  // extern "C"

namespace {

static_assert(MAMBA_SCAN_NOALLOC_SCRATCH_BYTES == mscan::kScanScratchBytes,
              "the header states the scratch array's size");

// use_scratch: the allocation-free entry point (the workspace is the
// library's fixed device array, not an argument).
mamba_status scan_fwd_impl(const char* who, const mamba_scan_desc* d,
                           const mamba_scan_strides* strides, const void* x, const void* delta,
                           const float* A, const void* B, const void* C, const float* D,
                           const void* z, const float* delta_bias, const float* h0, void* out,
                           float* last_state, void* workspace, size_t workspace_bytes,
                           void* stream, bool use_scratch = false) {
  mamba_status st = check_desc(d, who);
  if (st != MAMBA_OK) return st;
  if (d->flags & ~kFwdFlags)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: unknown flag bits 0x%x", who, d->flags & ~kFwdFlags);
  if ((st = check_groups(d, who, true)) != MAMBA_OK) return st;
  Rows rs;
  if ((st = resolve_rows(strides, d, who, rs)) != MAMBA_OK) return st;
  // every element offset of a strided tensor stays within 2^40 elements
  if (d->batch * d->seqlen > 0 && widest(rs) > (int64_t(1) << 40) / (d->batch * d->seqlen))
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: problem too large", who);
  const int64_t G = groups_of(d);
  const int64_t rows = d->batch * d->dim;
  const int64_t tokens = d->batch * d->seqlen;
  const int64_t elems = tokens * d->dim;
  if (elems > 0) {
    if (!x) return fail(MAMBA_ERR_INVALID_ARG, "%s: x is NULL", who);
    if (!delta) return fail(MAMBA_ERR_INVALID_ARG, "%s: delta is NULL", who);
    if (!A) return fail(MAMBA_ERR_INVALID_ARG, "%s: A is NULL", who);
    if (!B) return fail(MAMBA_ERR_INVALID_ARG, "%s: B is NULL", who);
    if (!C) return fail(MAMBA_ERR_INVALID_ARG, "%s: C is NULL", who);
    if (!out) return fail(MAMBA_ERR_INVALID_ARG, "%s: out is NULL", who);
  }
  if ((d->flags & MAMBA_SCAN_SPLIT_STATES) && forced_segments(d) > 0)
    return fail(MAMBA_ERR_INVALID_ARG,
                "%s: MAMBA_SCAN_SPLIT_STATES and a forced number of segments exclude each other", who);
  const int split = split_mode(d, widest(rs));
  if (split < 0)
    return fail(MAMBA_ERR_UNSUPPORTED,
                "%s: MAMBA_SCAN_SPLIT_STATES needs dstate 16, the first-order input weight and "
                "rows of at most %lld bytes",
                who, (long long)((int64_t(1) << 31) / 9 - 1));
  mscan::ScanPlan plan{d->seqlen, 1, 0};
  if (split == 0)
    plan = mscan::plan_scan(d->batch, d->seqlen, d->dim, static_cast<int>(d->dstate),
                            forced_segments(d), widest(rs));
  if (use_scratch && elems > 0 && plan.workspace_bytes > mscan::kScanScratchBytes)
    return fail(MAMBA_ERR_UNSUPPORTED,
                "%s: this problem's segment plan needs %zu bytes of scratch, the library's fixed "
                "device array holds %zu (force fewer time segments with flags bits 0-15, or call "
                "mamba_scan_fwd_init with a workspace)",
                who, plan.workspace_bytes, static_cast<size_t>(mscan::kScanScratchBytes));
  if (!use_scratch && elems > 0 && plan.workspace_bytes > 0) {
    if (!workspace)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace is NULL but %zu bytes are needed", who,
                  plan.workspace_bytes);
    if (workspace_bytes < plan.workspace_bytes)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace has %zu bytes, %zu needed", who,
                  workspace_bytes, plan.workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", who);
  }
  const size_t eb = io_bytes(d->io_dtype);
  const size_t N = static_cast<size_t>(d->dstate);
  const int64_t rowsteps = elems > 0 ? tokens : 0;  // rows of each token tensor
  const Span in[] = {
      {"x", x, span_bytes(rowsteps, rs.x, d->dim, eb)},
      {"delta", delta, span_bytes(rowsteps, rs.d, d->dim, eb)},
      {"z", z, span_bytes(rowsteps, rs.z, d->dim, eb)},
      {"B", B, span_bytes(tokens, rs.bc, G * d->dstate, eb)},
      {"C", C, span_bytes(tokens, rs.bc, G * d->dstate, eb)},
      {"A", A, static_cast<size_t>(d->dim) * N * 4},
      {"D", D, static_cast<size_t>(d->dim) * 4},
      {"delta_bias", delta_bias, static_cast<size_t>(d->dim) * 4},
  };
  const Span o_out{"out", out, span_bytes(rowsteps, rs.o, d->dim, eb)};
  const Span o_last{"last_state", last_state, static_cast<size_t>(rows) * N * 4};
  // (the fixed scratch array is the library's own: no caller buffer can overlap it)
  const Span o_ws{"workspace", elems > 0 && !use_scratch ? workspace : nullptr,
                  plan.workspace_bytes};
  for (const Span& s : in) {
    if (overlaps(o_out, s)) return fail(MAMBA_ERR_INVALID_ARG, "%s: out overlaps %s", who, s.name);
    if (overlaps(o_last, s))
      return fail(MAMBA_ERR_INVALID_ARG, "%s: last_state overlaps %s", who, s.name);
    if (overlaps(o_ws, s)) return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace overlaps %s", who, s.name);
  }
  if (overlaps(o_out, o_last)) return fail(MAMBA_ERR_INVALID_ARG, "%s: out overlaps last_state", who);
  const Span i_h0{"h0", h0, static_cast<size_t>(rows) * N * 4};
  if (overlaps(i_h0, o_out) || overlaps(i_h0, o_last) || overlaps(i_h0, o_ws))
    return fail(MAMBA_ERR_INVALID_ARG, "%s: h0 overlaps out, last_state or the workspace", who);
  if (overlaps(o_ws, o_out) || overlaps(o_ws, o_last))
    return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace overlaps an output", who);
  const size_t align = eb;
  for (const Span& s : {in[0], in[1], in[2], o_out})
    if (s.p && reinterpret_cast<uintptr_t>(s.p) % align)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: %s is not %zu-byte aligned", who, s.name, align);
  // B and C rows are read as 32-bit words (unless one bf16 state per step)
  const size_t bc_align = (eb == 2 && N == 1) ? 2 : 4;
  for (const Span& s : {in[3], in[4]})
    if (s.p && reinterpret_cast<uintptr_t>(s.p) % bc_align)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: %s is not %zu-byte aligned", who, s.name, bc_align);
  if ((static_cast<size_t>(rs.bc) * eb) % bc_align)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: B/C rows (stride %lld) are not %zu-byte aligned", who,
                (long long)rs.bc, bc_align);
  for (const void* p : {static_cast<const void*>(A), static_cast<const void*>(D),
                        static_cast<const void*>(delta_bias), static_cast<const void*>(last_state),
                        static_cast<const void*>(h0)})
    if (p && reinterpret_cast<uintptr_t>(p) % 4)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: an fp32 argument is not 4-byte aligned", who);

  if (rows == 0 || (elems == 0 && !last_state)) return ok();
  if (use_scratch && elems > 0 && plan.workspace_bytes > 0) {
    void* sp = nullptr;
    const hipError_t se = mscan::scan_scratch(&sp);
    if (se != hipSuccess)
      return fail(MAMBA_ERR_HIP, "%s: the scratch array's device address: %s", who,
                  hipGetErrorString(se));
    workspace = sp;
  }

  mscan::ScanProblem p;
  p.x = x;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.h0 = h0;
  p.out = out;
  p.last_state = last_state;
  p.batch = d->batch;
  p.seqlen = d->seqlen;
  p.dim = d->dim;
  p.dstate = static_cast<int>(d->dstate);
  p.io = d->io_dtype;
  p.zoh = (d->flags & MAMBA_SCAN_ZOH) != 0;
  p.ngroups = G;
  p.sx = rs.x;
  p.sd = rs.d;
  p.sz = rs.z;
  p.so = rs.o;
  p.sbc = rs.bc;
  const hipError_t e =
      split == 1 && p.seqlen > 0
          ? mscan::launch_scan_split(p, static_cast<hipStream_t>(stream))
          : mscan::launch_scan_fwd(p, plan, plan.workspace_bytes > 0 ? workspace : nullptr,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MAMBA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

mamba_status mamba_scan_fwd(const mamba_scan_desc* d, const void* x, const void* delta,
                            const float* A, const void* B, const void* C, const float* D,
                            const void* z, const float* delta_bias, void* out, float* last_state,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return scan_fwd_impl("mamba_scan_fwd", d, nullptr, x, delta, A, B, C, D, z, delta_bias, nullptr,
                       out, last_state, workspace, workspace_bytes, stream);
}

mamba_status mamba_scan_fwd_init(const mamba_scan_desc* d, const void* x, const void* delta,
                                 const float* A, const void* B, const void* C, const float* D,
                                 const void* z, const float* delta_bias, const float* h0,
                                 void* out, float* last_state, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return scan_fwd_impl("mamba_scan_fwd_init", d, nullptr, x, delta, A, B, C, D, z, delta_bias, h0,
                       out, last_state, workspace, workspace_bytes, stream);
}

mamba_status mamba_scan_fwd_strided(const mamba_scan_desc* d, const mamba_scan_strides* strides,
                                    const void* x, const void* delta, const float* A, const void* B,
                                    const void* C, const float* D, const void* z,
                                    const float* delta_bias, const float* h0, void* out,
                                    float* last_state, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return scan_fwd_impl("mamba_scan_fwd_strided", d, strides, x, delta, A, B, C, D, z, delta_bias, h0,
                       out, last_state, workspace, workspace_bytes, stream);
}

mamba_status mamba_scan_fwd_noalloc(const mamba_scan_desc* d, const void* x, const void* delta,
                                    const float* A, const void* B, const void* C, const float* D,
                                    const void* z, const float* delta_bias, const float* h0,
                                    void* out, float* last_state, void* stream) {
  return scan_fwd_impl("mamba_scan_fwd_noalloc", d, nullptr, x, delta, A, B, C, D, z, delta_bias,
                       h0, out, last_state, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {

mamba_status state_update_impl(const char* who, const mamba_scan_desc* d,
                               const mamba_scan_strides* strides, float* state, const void* x,
                               const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, void* out,
                               void* stream) {
  mamba_status st = check_desc(d, who);
  if (st != MAMBA_OK) return st;
  if (d->flags & ~MAMBA_SCAN_ZOH)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: flags must be 0 or MAMBA_SCAN_ZOH", who);
  if ((st = check_groups(d, who, false)) != MAMBA_OK) return st;
  const int64_t G = groups_of(d);
  if (d->seqlen != 1)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: seqlen must be 1 (got %lld)", who, (long long)d->seqlen);
  if ((d->batch + 3) / 4 > 65535)   // grid rows of four batch rows
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: batch %lld too large", who, (long long)d->batch);
  Rows rs;
  if ((st = resolve_rows(strides, d, who, rs)) != MAMBA_OK) return st;
  const int64_t rows = d->batch * d->dim;
  if (rows == 0) return ok();
  if (!state) return fail(MAMBA_ERR_INVALID_ARG, "%s: state is NULL", who);
  if (!x) return fail(MAMBA_ERR_INVALID_ARG, "%s: x is NULL", who);
  if (!delta) return fail(MAMBA_ERR_INVALID_ARG, "%s: delta is NULL", who);
  if (!A) return fail(MAMBA_ERR_INVALID_ARG, "%s: A is NULL", who);
  if (!B) return fail(MAMBA_ERR_INVALID_ARG, "%s: B is NULL", who);
  if (!C) return fail(MAMBA_ERR_INVALID_ARG, "%s: C is NULL", who);
  if (!out) return fail(MAMBA_ERR_INVALID_ARG, "%s: out is NULL", who);
  const size_t eb = io_bytes(d->io_dtype);
  const size_t N = static_cast<size_t>(d->dstate);
  const Span in[] = {
      {"x", x, span_bytes(d->batch, rs.x, d->dim, eb)},
      {"delta", delta, span_bytes(d->batch, rs.d, d->dim, eb)},
      {"z", z, span_bytes(d->batch, rs.z, d->dim, eb)},
      {"B", B, span_bytes(d->batch, rs.bc, G * d->dstate, eb)},
      {"C", C, span_bytes(d->batch, rs.bc, G * d->dstate, eb)},
      {"A", A, static_cast<size_t>(d->dim) * N * 4},
      {"D", D, static_cast<size_t>(d->dim) * 4},
      {"delta_bias", delta_bias, static_cast<size_t>(d->dim) * 4},
  };
  const Span o_state{"state", state, static_cast<size_t>(rows) * N * 4};
  const Span o_out{"out", out, span_bytes(d->batch, rs.o, d->dim, eb)};
  for (const Span& s : in) {
    if (overlaps(o_state, s)) return fail(MAMBA_ERR_INVALID_ARG, "%s: state overlaps %s", who, s.name);
    if (overlaps(o_out, s)) return fail(MAMBA_ERR_INVALID_ARG, "%s: out overlaps %s", who, s.name);
  }
  if (overlaps(o_out, o_state)) return fail(MAMBA_ERR_INVALID_ARG, "%s: out overlaps state", who);
  const size_t state_align = N >= 4 ? 16 : 4;
  if (reinterpret_cast<uintptr_t>(state) % state_align)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: state is not %zu-byte aligned", who, state_align);
  for (const Span& s : {in[0], in[1], in[2], in[3], in[4], o_out})
    if (s.p && reinterpret_cast<uintptr_t>(s.p) % eb)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: %s is not %zu-byte aligned", who, s.name, eb);
  for (const void* p : {static_cast<const void*>(A), static_cast<const void*>(D),
                        static_cast<const void*>(delta_bias)})
    if (p && reinterpret_cast<uintptr_t>(p) % 4)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: an fp32 argument is not 4-byte aligned", who);

  mscan::DecodeProblem p;
  p.state = state;
  p.x = x;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.out = out;
  p.batch = d->batch;
  p.dim = d->dim;
  p.dstate = static_cast<int>(d->dstate);
  p.io = d->io_dtype;
  p.zoh = (d->flags & MAMBA_SCAN_ZOH) != 0;
  p.ngroups = G;
  p.sx = rs.x;
  p.sd = rs.d;
  p.sz = rs.z;
  p.so = rs.o;
  p.sbc = rs.bc;
  const hipError_t e = mscan::launch_state_update(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MAMBA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

mamba_status mamba_state_update(const mamba_scan_desc* d, float* state, const void* x,
                                const void* delta, const float* A, const void* B, const void* C,
                                const float* D, const void* z, const float* delta_bias, void* out,
                                void* stream) {
  return state_update_impl("mamba_state_update", d, nullptr, state, x, delta, A, B, C, D, z,
                           delta_bias, out, stream);
}

mamba_status mamba_state_update_strided(const mamba_scan_desc* d, const mamba_scan_strides* strides,
                                        float* state, const void* x, const void* delta,
                                        const float* A, const void* B, const void* C,
                                        const float* D, const void* z, const float* delta_bias,
                                        void* out, void* stream) {
  return state_update_impl("mamba_state_update_strided", d, strides, state, x, delta, A, B, C, D, z,
                           delta_bias, out, stream);
}


}  // extern "C"

namespace {

// Descriptor fields common to both convolution entry points.
mamba_status check_conv_desc(const mamba_conv_desc* d, const char* who) {
  if (!d) return fail(MAMBA_ERR_INVALID_ARG, "%s: desc is NULL", who);
  if (d->batch < 0 || d->seqlen < 0 || d->dim < 0)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: negative size (batch=%lld seqlen=%lld dim=%lld)", who,
                (long long)d->batch, (long long)d->seqlen, (long long)d->dim);
  if (d->io_dtype != MAMBA_F32 && d->io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: io_dtype %d is not MAMBA_F32 or MAMBA_BF16", who,
                (int)d->io_dtype);
  if (d->width < 1) return fail(MAMBA_ERR_INVALID_ARG, "%s: width %lld < 1", who, (long long)d->width);
  if (d->width > 4)
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: width %lld not supported (1 to 4)", who,
                (long long)d->width);
  if (d->flags != 0) return fail(MAMBA_ERR_INVALID_ARG, "%s: flags must be 0", who);
  const int64_t lim = int64_t(1) << 40;
  if (d->batch > 65535 || d->seqlen > lim || d->dim > (int64_t(1) << 31) ||
      (d->batch && d->dim > (int64_t(1) << 31) / d->batch) ||
      (d->batch * d->dim && d->seqlen > lim / (d->batch * d->dim)) ||
      (d->seqlen + 63) / 64 > 65535)
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: problem too large", who);
  return MAMBA_OK;
}

mamba_status check_align(const char* who, std::initializer_list<Span> spans, size_t align) {
  for (const Span& s : spans)
    if (s.p && reinterpret_cast<uintptr_t>(s.p) % align)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: %s is not %zu-byte aligned", who, s.name, align);
  return MAMBA_OK;
}

}  // namespace

extern "C" {

mamba_status mamba_conv1d_fwd(const mamba_conv_desc* d, const void* xin, const float* weight,
                              const float* bias, const void* state_in, void* out,
                              void* state_out, void* stream) {
  const char* who = "mamba_conv1d_fwd";
  mamba_status st = check_conv_desc(d, who);
  if (st != MAMBA_OK) return st;
  const int64_t rows = d->batch * d->dim;
  const int64_t elems = rows * d->seqlen;
  if (rows == 0) return ok();
  if (elems > 0) {
    if (!xin) return fail(MAMBA_ERR_INVALID_ARG, "%s: xin is NULL", who);
    if (!out) return fail(MAMBA_ERR_INVALID_ARG, "%s: out is NULL", who);
  }
  if (!weight) return fail(MAMBA_ERR_INVALID_ARG, "%s: weight is NULL", who);
  const size_t eb = io_bytes(d->io_dtype);
  const size_t W = static_cast<size_t>(d->width);
  const size_t state_bytes = static_cast<size_t>(rows) * (W - 1) * eb;
  const Span in[] = {
      {"xin", xin, static_cast<size_t>(elems) * eb},
      {"weight", weight, static_cast<size_t>(d->dim) * W * 4},
      {"bias", bias, static_cast<size_t>(d->dim) * 4},
      {"state_in", W > 1 ? state_in : nullptr, state_bytes},
  };
  const Span o_out{"out", out, static_cast<size_t>(elems) * eb};
  const Span o_st{"state_out", W > 1 ? state_out : nullptr, state_bytes};
  for (const Span& s : in) {
    if (overlaps(o_out, s)) return fail(MAMBA_ERR_INVALID_ARG, "%s: out overlaps %s", who, s.name);
    if (overlaps(o_st, s))
      return fail(MAMBA_ERR_INVALID_ARG, "%s: state_out overlaps %s", who, s.name);
  }
  if (overlaps(o_out, o_st)) return fail(MAMBA_ERR_INVALID_ARG, "%s: out overlaps state_out", who);
  if ((st = check_align(who, {in[0], in[3], o_out, o_st}, eb)) != MAMBA_OK) return st;
  if ((st = check_align(who, {in[1], in[2]}, 4)) != MAMBA_OK) return st;

  mscan::ConvProblem p{};
  p.xin = xin;
  p.weight = weight;
  p.bias = bias;
  p.state_in = W > 1 ? state_in : nullptr;
  p.out = out;
  p.state_out = W > 1 ? state_out : nullptr;
  p.batch = d->batch;
  p.seqlen = d->seqlen;
  p.dim = d->dim;
  p.width = static_cast<int>(W);
  p.io = d->io_dtype;
  const hipError_t e = mscan::launch_conv1d(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MAMBA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

mamba_status mamba_conv1d_update(const mamba_conv_desc* d, void* state, const void* xin,
                                 const float* weight, const float* bias, void* out, void* stream) {
  const char* who = "mamba_conv1d_update";
  mamba_status st = check_conv_desc(d, who);
  if (st != MAMBA_OK) return st;
  if (d->seqlen != 1)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: seqlen must be 1 (got %lld)", who, (long long)d->seqlen);
  const int64_t rows = d->batch * d->dim;
  if (rows == 0) return ok();
  const size_t W = static_cast<size_t>(d->width);
  if (W > 1 && !state) return fail(MAMBA_ERR_INVALID_ARG, "%s: state is NULL", who);
  if (!xin) return fail(MAMBA_ERR_INVALID_ARG, "%s: xin is NULL", who);
  if (!weight) return fail(MAMBA_ERR_INVALID_ARG, "%s: weight is NULL", who);
  if (!out) return fail(MAMBA_ERR_INVALID_ARG, "%s: out is NULL", who);
  const size_t eb = io_bytes(d->io_dtype);
  const Span in[] = {
      {"xin", xin, static_cast<size_t>(rows) * eb},
      {"weight", weight, static_cast<size_t>(d->dim) * W * 4},
      {"bias", bias, static_cast<size_t>(d->dim) * 4},
  };
  const Span o_state{"state", W > 1 ? state : nullptr, static_cast<size_t>(rows) * (W - 1) * eb};
  const Span o_out{"out", out, static_cast<size_t>(rows) * eb};
  for (const Span& s : in) {
    if (overlaps(o_state, s)) return fail(MAMBA_ERR_INVALID_ARG, "%s: state overlaps %s", who, s.name);
    if (overlaps(o_out, s)) return fail(MAMBA_ERR_INVALID_ARG, "%s: out overlaps %s", who, s.name);
  }
  if (overlaps(o_out, o_state)) return fail(MAMBA_ERR_INVALID_ARG, "%s: out overlaps state", who);
  if ((st = check_align(who, {in[0], o_state, o_out}, eb)) != MAMBA_OK) return st;
  if ((st = check_align(who, {in[1], in[2]}, 4)) != MAMBA_OK) return st;

  mscan::ConvProblem p{};
  p.xin = xin;
  p.weight = weight;
  p.bias = bias;
  p.out = out;
  p.state = W > 1 ? state : nullptr;
  p.batch = d->batch;
  p.seqlen = 1;
  p.dim = d->dim;
  p.width = static_cast<int>(W);
  p.io = d->io_dtype;
  const hipError_t e = mscan::launch_conv1d_update(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MAMBA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

mamba_status scan_bwd_check(const char* who, const mamba_scan_desc* d) {
  mamba_status st = check_desc(d, who);
  if (st != MAMBA_OK) return st;
  if (d->flags & MAMBA_SCAN_ZOH)
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: the backward of the MAMBA_SCAN_ZOH mode is not provided",
                who);
  if (d->flags & ~0xffffu)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: unknown flag bits 0x%x", who, d->flags & ~0xffffu);
  // one state checkpoint (every row's N fp32 states) is addressed with 32-bit offsets
  if (d->dim > 0 && d->batch > ((int64_t(1) << 31) - 1) / (4 * d->dstate) / d->dim)
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: batch * dim * dstate * 4 bytes must stay below 2^31",
                who);
  return check_groups(d, who, true);
}

mscan::ScanBwdPlan bwd_plan(const mamba_scan_desc* d) {
  return mscan::plan_scan_bwd(d->batch, d->seqlen, d->dim, static_cast<int>(d->dstate),
                              forced_segments(d));
}

}  // namespace

extern "C" {

size_t mamba_scan_bwd_workspace_size(const mamba_scan_desc* d) {
  if (!d || scan_bwd_check("mamba_scan_bwd_workspace_size", d) != MAMBA_OK) return 0;
  return bwd_plan(d).workspace_bytes;
}

mamba_status mamba_scan_bwd(const mamba_scan_desc* d, const void* x, const void* delta,
                            const float* A, const void* B, const void* C, const float* D,
                            const void* z, const float* delta_bias, const float* h0,
                            const void* dout, const float* dlast, void* dx, void* ddelta,
                            float* dA, float* dB, float* dC, float* dD, void* dz,
                            float* ddelta_bias, float* dh0, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const char* who = "mamba_scan_bwd";
  mamba_status st = scan_bwd_check(who, d);
  if (st != MAMBA_OK) return st;
  const int64_t rows = d->batch * d->dim;
  const int64_t tokens = d->batch * d->seqlen;
  const int64_t elems = tokens * d->dim;
  const int64_t G = groups_of(d);
  if (d->dim == 0) return ok();
  if (!dA) return fail(MAMBA_ERR_INVALID_ARG, "%s: dA is NULL", who);
  if (elems > 0) {
    const struct {
      const char* name;
      const void* p;
    } req[] = {{"x", x},       {"delta", delta},   {"A", A},   {"B", B},   {"C", C},
               {"dout", dout}, {"dx", dx},         {"ddelta", ddelta},     {"dB", dB},
               {"dC", dC}};
    for (const auto& r : req)
      if (!r.p) return fail(MAMBA_ERR_INVALID_ARG, "%s: %s is NULL", who, r.name);
  }
  const mscan::ScanBwdPlan plan = bwd_plan(d);
  if (elems > 0) {
    if (!workspace)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace is NULL but %zu bytes are needed", who,
                  plan.workspace_bytes);
    if (workspace_bytes < plan.workspace_bytes)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace has %zu bytes, %zu needed", who,
                  workspace_bytes, plan.workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", who);
  }
  const size_t eb = io_bytes(d->io_dtype);
  const size_t N = static_cast<size_t>(d->dstate);
  const size_t E = static_cast<size_t>(elems) * eb;
  const Span in[] = {
      {"x", x, E},
      {"delta", delta, E},
      {"z", z, E},
      {"dout", dout, E},
      {"B", B, static_cast<size_t>(tokens * G) * N * eb},
      {"C", C, static_cast<size_t>(tokens * G) * N * eb},
      {"A", A, static_cast<size_t>(d->dim) * N * 4},
      {"D", D, static_cast<size_t>(d->dim) * 4},
      {"delta_bias", delta_bias, static_cast<size_t>(d->dim) * 4},
      {"h0", h0, static_cast<size_t>(rows) * N * 4},
      {"dlast", dlast, static_cast<size_t>(rows) * N * 4},
  };
  const Span out[] = {
      {"dx", dx, E},
      {"ddelta", ddelta, E},
      {"dz", z ? dz : nullptr, E},
      {"dA", dA, static_cast<size_t>(d->dim) * N * 4},
      {"dB", dB, static_cast<size_t>(tokens * G) * N * 4},
      {"dC", dC, static_cast<size_t>(tokens * G) * N * 4},
      {"dD", dD, static_cast<size_t>(d->dim) * 4},
      {"ddelta_bias", ddelta_bias, static_cast<size_t>(d->dim) * 4},
      {"dh0", dh0, static_cast<size_t>(rows) * N * 4},
      {"workspace", elems > 0 ? workspace : nullptr, plan.workspace_bytes},
  };
  const size_t n_out = sizeof(out) / sizeof(out[0]);
  for (size_t i = 0; i < n_out; ++i) {
    for (const Span& s : in)
      if (overlaps(out[i], s))
        return fail(MAMBA_ERR_INVALID_ARG, "%s: %s overlaps %s", who, out[i].name, s.name);
    for (size_t j = i + 1; j < n_out; ++j)
      if (overlaps(out[i], out[j]))
        return fail(MAMBA_ERR_INVALID_ARG, "%s: %s overlaps %s", who, out[i].name, out[j].name);
  }
  if ((st = check_align(who, {in[0], in[1], in[2], in[3], out[0], out[1], out[2]}, eb)) != MAMBA_OK)
    return st;
  const size_t bc_align = (eb == 2 && N == 1) ? 2 : 4;
  if ((st = check_align(who, {in[4], in[5]}, bc_align)) != MAMBA_OK) return st;
  if ((st = check_align(who, {in[6], in[7], in[8], in[9], in[10], out[3], out[4], out[5], out[6],
                              out[7], out[8]},
                        4)) != MAMBA_OK)
    return st;

  mscan::ScanBwdProblem p;
  p.x = x;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.bias = delta_bias;
  p.h0 = h0;
  p.dout = dout;
  p.dlast = dlast;
  p.dx = dx;
  p.ddelta = ddelta;
  p.dA = dA;
  p.dB = dB;
  p.dC = dC;
  p.dD = dD;
  p.dz = z ? dz : nullptr;
  p.dbias = ddelta_bias;
  p.dh0 = dh0;
  p.batch = d->batch;
  p.seqlen = d->seqlen;
  p.dim = d->dim;
  p.dstate = static_cast<int>(d->dstate);
  p.io = d->io_dtype;
  p.ngroups = G;
  const hipError_t e = mscan::launch_scan_bwd(p, plan, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MAMBA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

mamba_status check_ssd_desc(const mamba_ssd_desc* d, const char* who) {
  if (!d) return fail(MAMBA_ERR_INVALID_ARG, "%s: desc is NULL", who);
  if (d->batch < 0 || d->seqlen < 0 || d->nheads < 0)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: negative size", who);
  if (d->ngroups < 1 || (d->nheads > 0 && d->nheads % d->ngroups != 0))
    return fail(MAMBA_ERR_INVALID_ARG, "%s: ngroups %lld must be >= 1 and divide nheads %lld", who,
                (long long)d->ngroups, (long long)d->nheads);
  if (d->flags != 0) return fail(MAMBA_ERR_INVALID_ARG, "%s: flags must be 0", who);
  if (d->io_dtype != MAMBA_BF16 && d->io_dtype != MAMBA_F32)
    return fail(MAMBA_ERR_INVALID_ARG, "%s: io_dtype %d is not a mamba_dtype", who, (int)d->io_dtype);
  if (d->io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: only MAMBA_BF16 io is supported", who);
  if (d->headdim != 64 || d->dstate != 128)
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: headdim %lld, dstate %lld not supported (64, 128)", who,
                (long long)d->headdim, (long long)d->dstate);
  const int64_t lim = int64_t(1) << 40;
  if (d->batch > 65535 || d->nheads > 65535 || d->seqlen > lim ||
      (d->batch * d->nheads && d->seqlen > lim / (d->batch * d->nheads * 64)) ||
      (d->seqlen + 255) / 256 > (int64_t(1) << 30))
    return fail(MAMBA_ERR_UNSUPPORTED, "%s: problem too large", who);
  return MAMBA_OK;
}

}  // namespace

extern "C" {

size_t mamba_ssd_workspace_size(const mamba_ssd_desc* d) {
  if (check_ssd_desc(d, "mamba_ssd_workspace_size") != MAMBA_OK) return 0;
  if (d->batch == 0 || d->nheads == 0 || d->seqlen == 0) return 0;
  return mscan::ssd_workspace_bytes(d->batch, d->seqlen, d->nheads, d->ngroups);
}

mamba_status mamba_ssd_fwd(const mamba_ssd_desc* d, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const float* dt_bias,
                           const float* h0, void* out, float* last_state, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const char* who = "mamba_ssd_fwd";
  mamba_status st = check_ssd_desc(d, who);
  if (st != MAMBA_OK) return st;
  const int64_t H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
  const int64_t tokens = d->batch * d->seqlen;
  const int64_t elems = tokens * H * P;
  if (d->batch == 0 || H == 0) return ok();
  if (elems > 0) {
    const struct {
      const char* name;
      const void* p;
    } req[] = {{"x", x}, {"dt", dt}, {"A", A}, {"B", B}, {"C", C}, {"out", out}};
    for (const auto& r : req)
      if (!r.p) return fail(MAMBA_ERR_INVALID_ARG, "%s: %s is NULL", who, r.name);
  }
  const size_t need = mamba_ssd_workspace_size(d);
  if (elems > 0) {
    if (!workspace)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace is NULL but %zu bytes are needed", who, need);
    if (workspace_bytes < need)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace has %zu bytes, %zu needed", who,
                  workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(MAMBA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", who);
  }
  const Span in[] = {
      {"x", x, static_cast<size_t>(elems) * 2},
      {"dt", dt, static_cast<size_t>(tokens * H) * 2},
      {"B", B, static_cast<size_t>(tokens * G * N) * 2},
      {"C", C, static_cast<size_t>(tokens * G * N) * 2},
      {"A", A, static_cast<size_t>(H) * 4},
      {"D", D, static_cast<size_t>(H) * 4},
      {"dt_bias", dt_bias, static_cast<size_t>(H) * 4},
      {"h0", h0, static_cast<size_t>(d->batch * H * N * P) * 4},
  };
  const Span outs[] = {
      {"out", out, static_cast<size_t>(elems) * 2},
      {"last_state", last_state, static_cast<size_t>(d->batch * H * N * P) * 4},
      {"workspace", elems > 0 ? workspace : nullptr, need},
  };
  for (size_t i = 0; i < 3; ++i) {
    for (const Span& s : in)
      if (overlaps(outs[i], s))
        return fail(MAMBA_ERR_INVALID_ARG, "%s: %s overlaps %s", who, outs[i].name, s.name);
    for (size_t j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j]))
        return fail(MAMBA_ERR_INVALID_ARG, "%s: %s overlaps %s", who, outs[i].name, outs[j].name);
  }
  if ((st = check_align(who, {in[0], in[2], in[3]}, 16)) != MAMBA_OK) return st;
  if ((st = check_align(who, {in[1], outs[0]}, 2)) != MAMBA_OK) return st;
  if ((st = check_align(who, {in[4], in[5], in[6], in[7], outs[1]}, 4)) != MAMBA_OK) return st;

  mscan::SsdProblem p;
  p.x = x;
  p.dt = dt;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.dt_bias = dt_bias;
  p.h0 = h0;
  p.out = out;
  p.last_state = last_state;
  p.batch = d->batch;
  p.seqlen = d->seqlen;
  p.nheads = H;
  p.ngroups = G;
  const hipError_t e = mscan::launch_ssd_fwd(p, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MAMBA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // extern "C"
