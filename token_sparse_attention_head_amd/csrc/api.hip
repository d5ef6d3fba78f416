// C ABI of libtsa.so: argument validation, workspace layout and stage orchestration.
// Every entry point validates on the host before enqueuing anything; on error nothing
// is launched and nothing is written.  All work goes to the caller's stream.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.h"
#include "kernels.h"

// The scratch array of tsa_forward_noalloc (see device_scratch below).
static __device__ __align__(256) char scratch[TSA_NOALLOC_SCRATCH_BYTES];

namespace {

using tsa::launch_attn_compact;

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t elem_bytes(const tsa_desc& d) { return d.dtype == TSA_BF16 ? 2 : 4; }

int window(const tsa_desc& d) { return d.W < d.L ? d.W : d.L; }

int64_t forced_count(const tsa_desc& d) {
  const int Wp = window(d);
  const int c1 = d.L - Wp;
  const int c0 = d.n_sink < c1 ? d.n_sink : c1;
  return (int64_t)c0 + Wp;
}

bool empty_problem(const tsa_desc& d) { return d.B == 0 || d.L == 0; }

bool fused_forward(const tsa_desc& d) { return d.dtype == TSA_BF16; }

// Sizes, dtype and scale; keep/W/n_sink are checked separately (dense attention ignores them).
tsa_status check_shape(const tsa_desc* d) {
  if (!d) return TSA_ERR_NULL;
  if (d->dtype != TSA_F32 && d->dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (d->B < 0 || d->L < 0 || d->H <= 0 || d->Hkv <= 0 || d->d <= 0) return TSA_ERR_SHAPE;
  if (d->H % d->Hkv != 0) return TSA_ERR_SHAPE;
  if (d->d != 64 && d->d != 128) return TSA_ERR_SHAPE;
  if (!std::isfinite(d->scale) || d->scale < 0.f) return TSA_ERR_ARG;
  if (!(d->tau >= 0.f && d->tau <= 1.f)) return TSA_ERR_ARG;   // also rejects NaN
  if (d->subsets != TSA_SUBSETS_PER_HEAD && d->subsets != TSA_SUBSETS_PER_KV_HEAD) return TSA_ERR_ARG;
  // Index limits of the launch grids (grid.y = B*H, 32-bit thread indices per batch entry).
  if ((int64_t)d->B * d->H > 65535) return TSA_ERR_SHAPE;
  const int64_t chunks_per_row = (int64_t)d->d * elem_bytes(*d) / 16;
  if ((int64_t)d->L * d->H * chunks_per_row >= (int64_t)1 << 31) return TSA_ERR_SHAPE;
  // The attention kernels address K and V rows by 32-bit byte offsets within one batch entry.
  if ((int64_t)d->L * d->Hkv * d->d * elem_bytes(*d) >= (int64_t)1 << 32) return TSA_ERR_SHAPE;
  return TSA_OK;
}

tsa_status check_budget(const tsa_desc& d) {
  if (d.W < 1 || d.W > TSA_MAX_W || d.n_sink < 0 || d.keep < 0) return TSA_ERR_BUDGET;
  if (d.L == 0) return d.keep == 0 ? TSA_OK : TSA_ERR_BUDGET;
  if (d.keep < forced_count(d) || d.keep > d.L) return TSA_ERR_BUDGET;
  return TSA_OK;
}

tsa_status check_full(const tsa_desc* d) {
  tsa_status st = check_shape(d);
  if (st != TSA_OK) return st;
  return check_budget(*d);
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t n;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

tsa_status status_of(hipError_t e) { return e == hipSuccess ? TSA_OK : TSA_ERR_LAUNCH; }

// With TSA_DEBUG_SYNC=1 every stage is synchronised and checked, so an asynchronous
// fault is reported by the call that caused it.
tsa_status after_launch(hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return TSA_ERR_LAUNCH;
  const char* dbg = std::getenv("TSA_DEBUG_SYNC");
  if (dbg && dbg[0] == '1') {
    if (hipStreamSynchronize(s) != hipSuccess) return TSA_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return TSA_ERR_LAUNCH;
  }
  return TSA_OK;
}

#define TSA_TRY(expr)                    \
  do {                                   \
    const tsa_status st_ = (expr);       \
    if (st_ != TSA_OK) return st_;       \
  } while (0)

// Byte sizes of the tensors of a descriptor (idx, inv and the compact K/V have one row
// per subset: H of them per head, Hkv per KV head; sel is the workspace of the select).
struct Sizes {
  size_t q, kv, scores, idx, compact, kvc, inv, sel, part, stat, counts;
};

Sizes sizes_of(const tsa_desc& d) {
  Sizes z;
  const int64_t e = elem_bytes(d);
  z.q = (size_t)d.B * d.L * d.H * d.d * e;
  z.kv = (size_t)d.B * d.L * d.Hkv * d.d * e;
  z.scores = (size_t)d.B * d.H * d.L * 4;
  const int R = tsa::subset_rows(d);
  z.idx = (size_t)d.B * R * d.keep * 4;
  z.compact = (size_t)d.B * d.H * d.keep * d.d * e;
  z.kvc = (size_t)d.B * R * d.keep * d.d * e;
  z.inv = (size_t)d.B * R * d.L * 4;
  z.sel = tsa::select_layout(d).total;
  z.counts = (size_t)d.B * R * 4;
  int chunk = 32, nchunk = 1;
  if (d.L > 0) tsa::score_chunking(d, chunk, nchunk);
  z.part = (size_t)d.B * d.H * nchunk * window(d) * 8;
  z.stat = (size_t)d.B * d.H * window(d) * 8;
  return z;
}

// Workspace carve-up of tsa_forward (regions in this order, each 256-byte aligned).  The
// bf16 forward is fused (attention reads the rows through idx and writes residual + O), so
// it needs no compact tensors; the fp32 forward runs the stages one after the other.
struct FwdLayout {
  size_t scores, idx, inv, sel, part, stat, counts, plan, qh, kh, vh, oh, total;
};

// hold_outputs = false leaves out the scores and idx regions (the caller passes both).
FwdLayout fwd_layout(const tsa_desc& d, bool hold_outputs = true) {
  const Sizes z = sizes_of(d);
  const size_t comp = fused_forward(d) ? 0 : round_up(z.compact);
  const size_t kvc = fused_forward(d) ? 0 : round_up(z.kvc);
  FwdLayout f;
  size_t o = 0;
  f.scores = o; o += hold_outputs ? round_up(z.scores) : 0;
  f.idx = o; o += hold_outputs ? round_up(z.idx) : 0;
  f.inv = o; o += round_up(z.inv);
  f.sel = o; o += round_up(z.sel);
  f.part = o; o += round_up(z.part);
  f.stat = o; o += round_up(z.stat);
  f.counts = o; o += d.tau > 0.f ? round_up(z.counts) : 0;
  f.plan = o; o += d.tau > 0.f && fused_forward(d) ? round_up(tsa::attn_plan_bytes(d)) : 0;
  f.qh = o; o += comp;
  f.kh = o; o += kvc;
  f.vh = o; o += kvc;
  f.oh = o; o += comp;
  f.total = o;
  return f;
}

// Workspace of tsa_sparse_attn: the inverse map (out-of-place output), the row counts and
// per-XCD plan of adaptive budgets, and for fp32 the compact tensors of the staged path.
struct SparseLayout {
  size_t inv, counts, plan, qh, kh, vh, oh, total;
};

SparseLayout sparse_layout(const tsa_desc& d) {
  const Sizes z = sizes_of(d);
  const size_t comp = fused_forward(d) ? 0 : round_up(z.compact);
  const size_t kvc = fused_forward(d) ? 0 : round_up(z.kvc);
  SparseLayout y;
  size_t o = 0;
  y.inv = o; o += round_up(z.inv);
  y.counts = o; o += d.tau > 0.f ? round_up(z.counts) : 0;
  y.plan = o; o += d.tau > 0.f && fused_forward(d) ? round_up(tsa::attn_plan_bytes(d)) : 0;
  y.qh = o; o += comp;
  y.kh = o; o += kvc;
  y.vh = o; o += kvc;
  y.oh = o; o += comp;
  y.total = o;
  return y;
}

template <typename P>
P* at(void* base, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}

// Pointer and alignment checks of the forward's tensors (scores / idx may be NULL).
tsa_status forward_args(const void* q, const void* k, const void* v, const void* residual, const void* out,
                        const float* scores, const int32_t* idx) {
  if (!q || !k || !v || !residual || !out) return TSA_ERR_NULL;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(residual) || !aligned(out) || !aligned(scores) ||
      !aligned(idx))
    return TSA_ERR_ALIGN;
  return TSA_OK;
}

// The forward on a workspace laid out by f: overlap checks, then the stages on stream s.
// scores_opt / idx_opt NULL: they live in the workspace (f holds their regions).
tsa_status forward_run(const tsa_desc& d, const void* q, const void* k, const void* v, const void* residual,
                       void* out, float* scores_opt, int32_t* idx_opt, void* ws, const FwdLayout& f, hipStream_t s) {
  const Sizes z = sizes_of(d);
  const Range ro{out, z.q}, rw{ws, f.total}, rs{scores_opt, z.scores}, ri{idx_opt, z.idx};
  const Range ins[4] = {{q, z.q}, {k, z.kv}, {v, z.kv}, {residual, z.q}};
  for (int i = 0; i < 4; ++i) {
    if (overlap(rw, ins[i]) || overlap(rs, ins[i]) || overlap(ri, ins[i])) return TSA_ERR_ALIAS;
    if (i < 3 && overlap(ro, ins[i])) return TSA_ERR_ALIAS;
  }
  if (out != residual && overlap(ro, ins[3])) return TSA_ERR_ALIAS;
  if (overlap(ro, rw) || overlap(ro, rs) || overlap(ro, ri) || overlap(rs, rw) || overlap(ri, rw) || overlap(rs, ri))
    return TSA_ERR_ALIAS;

  float* scores = scores_opt ? scores_opt : at<float>(ws, f.scores);
  int32_t* idx = idx_opt ? idx_opt : at<int32_t>(ws, f.idx);
  int32_t* inv = at<int32_t>(ws, f.inv);
  void* qh = at<char>(ws, f.qh);
  void* kh = at<char>(ws, f.kh);
  void* vh = at<char>(ws, f.vh);
  void* oh = at<char>(ws, f.oh);
  const bool in_place = out == residual;
  TSA_TRY(after_launch(tsa::launch_score(d, q, k, scores, at<float2>(ws, f.part), at<float2>(ws, f.stat), s), s));
  int32_t* counts = d.tau > 0.f ? at<int32_t>(ws, f.counts) : nullptr;
  TSA_TRY(after_launch(tsa::launch_select(d, scores, idx, in_place ? nullptr : inv, counts, at<char>(ws, f.sel), s), s));
  if (fused_forward(d)) {
    // Rows a head does not keep are the residual (copied out of place, untouched in place);
    // the attention epilogue writes residual + O into the kept rows.
    // Out of place the attention launch also copies the unkept rows (on its first
    // workgroups, overlapping the attention).
    if (d.keep == 0) {
      if (!in_place) return after_launch(tsa::launch_copy_unselected(d, inv, residual, out, s), s);
      return TSA_OK;
    }
    return after_launch(tsa::launch_attn_fused(d, q, k, v, idx, counts, at<int32_t>(ws, f.plan), residual, out,
                                               in_place ? nullptr : inv, s),
                        s);
  }
  if (d.keep > 0) {
    TSA_TRY(after_launch(tsa::launch_gather_qkv(d, q, k, v, idx, qh, kh, vh, s), s));
    TSA_TRY(after_launch(launch_attn_compact(d, qh, kh, vh, oh, s), s));
  }
  if (in_place) return after_launch(tsa::launch_scatter_inplace(d, oh, idx, out, s), s);
  return after_launch(tsa::launch_scatter_residual(d, oh, inv, residual, out, s), s);
}

// Scratch of tsa_forward_noalloc: a device array in the library's code object, one copy per
// GPU, held until the process ends.  Host code never uses the array's name as an address:
// the first call on each device (with that device current) looks the device address up
// with hipGetSymbolAddress and keeps it; every later use goes through that address.  No
// region of it has to start at zero: every kernel of the forward writes what it later reads
// (the select clears its own histograms).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

tsa_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TSA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TSA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TSA_OK;
}

}  // namespace

extern "C" {

int tsa_abi_version(void) { return TSA_ABI_VERSION; }

const char* tsa_status_str(int status) {
  switch (status) {
    case TSA_OK: return "ok";
    case TSA_ERR_NULL: return "a required pointer is NULL";
    case TSA_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case TSA_ERR_BUDGET: return "keep/W/n_sink out of range (need |forced| <= keep <= L, 1 <= W <= 64, n_sink >= 0)";
    case TSA_ERR_DTYPE: return "unsupported dtype";
    case TSA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case TSA_ERR_WORKSPACE: return "workspace missing or too small";
    case TSA_ERR_ALIAS: return "an output overlaps an input";
    case TSA_ERR_LAUNCH: return "kernel launch failed";
    case TSA_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

tsa_status tsa_check(const tsa_desc* desc) { return check_full(desc); }

tsa_status tsa_workspace_size(const tsa_desc* desc, int op, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  if (op == TSA_OP_DRIFT) {   // uses the sizes only
    TSA_TRY(check_shape(desc));
    *bytes = round_up(tsa::drift_workspace_bytes(*desc));
    return TSA_OK;
  }
  TSA_TRY(check_full(desc));
  const Sizes z = sizes_of(*desc);
  switch (op) {
    case TSA_OP_SCORE: *bytes = round_up(z.part) + round_up(z.stat); break;
    case TSA_OP_SELECT: *bytes = round_up(z.sel); break;
    case TSA_OP_SCATTER: *bytes = round_up(z.inv); break;
    case TSA_OP_FORWARD: *bytes = fwd_layout(*desc).total; break;
    case TSA_OP_SPARSE_ATTN: *bytes = sparse_layout(*desc).total; break;
    default: return TSA_ERR_ARG;
  }
  return TSA_OK;
}

tsa_status tsa_score(const tsa_desc* desc, const void* q, const void* k, float* scores, void* ws, size_t ws_bytes,
                     void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  if (!q || !k || !scores) return TSA_ERR_NULL;
  if (!aligned(q) || !aligned(k) || !aligned(scores) || !aligned(ws)) return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  const size_t need = round_up(z.part) + round_up(z.stat);
  if (!ws || ws_bytes < need) return TSA_ERR_WORKSPACE;
  const Range rs{scores, z.scores}, rw{ws, need};
  if (overlap(rs, {q, z.q}) || overlap(rs, {k, z.kv}) || overlap(rw, {q, z.q}) || overlap(rw, {k, z.kv}) ||
      overlap(rs, rw))
    return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(
      tsa::launch_score(d, q, k, scores, at<float2>(ws, 0), at<float2>(ws, round_up(z.part)), s), s);
}

tsa_status tsa_select(const tsa_desc* desc, const float* scores, int32_t* idx, void* ws, size_t ws_bytes,
                      void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  if (!scores || !idx) return TSA_ERR_NULL;
  if (!aligned(scores) || !aligned(idx) || !aligned(ws)) return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  if (overlap({scores, z.scores}, {idx, z.idx})) return TSA_ERR_ALIAS;
  const size_t need = round_up(z.sel);
  if (!ws || ws_bytes < need) return TSA_ERR_WORKSPACE;
  if (overlap({ws, need}, {scores, z.scores}) || overlap({ws, need}, {idx, z.idx})) return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(tsa::launch_select(d, scores, idx, nullptr, nullptr, ws, s), s);
}

tsa_status tsa_budget(const tsa_desc* desc, const float* scores, int32_t* counts, void* ws, size_t ws_bytes,
                      void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  if (!scores || !counts) return TSA_ERR_NULL;
  if (!aligned(scores) || !aligned(counts) || !aligned(ws)) return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  if (overlap({scores, z.scores}, {counts, z.counts})) return TSA_ERR_ALIAS;
  const size_t need = round_up(z.sel);
  if (!ws || ws_bytes < need) return TSA_ERR_WORKSPACE;
  if (overlap({ws, need}, {scores, z.scores}) || overlap({ws, need}, {counts, z.counts})) return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(tsa::launch_budget(d, scores, counts, ws, s), s);
}

tsa_status tsa_gather_qkv(const tsa_desc* desc, const void* q, const void* k, const void* v, const int32_t* idx,
                          void* qh, void* kh, void* vh, void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d) || d.keep == 0) return TSA_OK;
  if (!q || !k || !v || !idx || !qh || !kh || !vh) return TSA_ERR_NULL;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(idx) || !aligned(qh) || !aligned(kh) || !aligned(vh))
    return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  const Range outs[3] = {{qh, z.compact}, {kh, z.kvc}, {vh, z.kvc}};
  const Range ins[4] = {{q, z.q}, {k, z.kv}, {v, z.kv}, {idx, z.idx}};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return TSA_ERR_ALIAS;
  if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2])) return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(tsa::launch_gather_qkv(d, q, k, v, idx, qh, kh, vh, s), s);
}

tsa_status tsa_attn(const tsa_desc* desc, const void* qh, const void* kh, const void* vh, void* oh, void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d) || d.keep == 0) return TSA_OK;
  if (!qh || !kh || !vh || !oh) return TSA_ERR_NULL;
  if (!aligned(qh) || !aligned(kh) || !aligned(vh) || !aligned(oh)) return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  const Range ro{oh, z.compact};
  if (overlap(ro, {qh, z.compact}) || overlap(ro, {kh, z.kvc}) || overlap(ro, {vh, z.kvc}))
    return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_attn_compact(d, qh, kh, vh, oh, s), s);
}

tsa_status tsa_scatter_residual(const tsa_desc* desc, const void* oh, const int32_t* idx, const void* residual,
                                void* out, void* ws, size_t ws_bytes, void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  if (!oh || !idx || !residual || !out) return TSA_ERR_NULL;
  if (!aligned(oh) || !aligned(idx) || !aligned(residual) || !aligned(out)) return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  const Range ro{out, z.q};
  if (overlap(ro, {oh, z.compact}) || overlap(ro, {idx, z.idx})) return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (out == residual) return after_launch(tsa::launch_scatter_inplace(d, oh, idx, out, s), s);
  if (overlap(ro, {residual, z.q})) return TSA_ERR_ALIAS;
  const size_t need = round_up(z.inv);
  if (!ws || ws_bytes < need) return TSA_ERR_WORKSPACE;
  if (!aligned(ws)) return TSA_ERR_ALIGN;
  const Range rw{ws, need};
  if (overlap(rw, ro) || overlap(rw, {oh, z.compact}) || overlap(rw, {idx, z.idx}) || overlap(rw, {residual, z.q}))
    return TSA_ERR_ALIAS;
  int32_t* inv = static_cast<int32_t*>(ws);
  TSA_TRY(after_launch(tsa::launch_build_inverse(d, idx, inv, s), s));
  return after_launch(tsa::launch_scatter_residual(d, oh, inv, residual, out, s), s);
}

tsa_status tsa_forward(const tsa_desc* desc, const void* q, const void* k, const void* v, const void* residual,
                       void* out, float* scores_opt, int32_t* idx_opt, void* ws, size_t ws_bytes, void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  TSA_TRY(forward_args(q, k, v, residual, out, scores_opt, idx_opt));
  if (!aligned(ws)) return TSA_ERR_ALIGN;
  const FwdLayout f = fwd_layout(d);
  if (!ws || ws_bytes < f.total) return TSA_ERR_WORKSPACE;
  return forward_run(d, q, k, v, residual, out, scores_opt, idx_opt, ws, f, static_cast<hipStream_t>(stream));
}

tsa_status tsa_forward_noalloc(const tsa_desc* desc, const void* q, const void* k, const void* v,
                               const void* residual, void* out, float* scores, int32_t* idx, void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  if (!scores || !idx) return TSA_ERR_NULL;
  TSA_TRY(forward_args(q, k, v, residual, out, scores, idx));
  const FwdLayout f = fwd_layout(d, false);
  if (f.total > TSA_NOALLOC_SCRATCH_BYTES) return TSA_ERR_WORKSPACE;
  void* ws = nullptr;
  TSA_TRY(device_scratch(&ws));
  return forward_run(d, q, k, v, residual, out, scores, idx, ws, f, static_cast<hipStream_t>(stream));
}

tsa_status tsa_sparse_attn(const tsa_desc* desc, const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* residual, void* out, void* ws, size_t ws_bytes, void* stream) {
  TSA_TRY(check_full(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  if (!q || !k || !v || !idx || !residual || !out) return TSA_ERR_NULL;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(idx) || !aligned(residual) || !aligned(out) ||
      !aligned(ws))
    return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  const SparseLayout y = sparse_layout(d);
  if (!ws || ws_bytes < y.total) return TSA_ERR_WORKSPACE;
  const Range ro{out, z.q}, rw{ws, y.total};
  const Range ins[5] = {{q, z.q}, {k, z.kv}, {v, z.kv}, {idx, z.idx}, {residual, z.q}};
  for (int i = 0; i < 5; ++i) {
    if (overlap(rw, ins[i])) return TSA_ERR_ALIAS;
    if (i < 4 && overlap(ro, ins[i])) return TSA_ERR_ALIAS;
  }
  const bool in_place = out == residual;
  if (!in_place && overlap(ro, ins[4])) return TSA_ERR_ALIAS;
  if (overlap(ro, rw)) return TSA_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* counts = nullptr;
  if (d.tau > 0.f) {
    counts = at<int32_t>(ws, y.counts);
    TSA_TRY(after_launch(tsa::launch_row_counts(d, idx, counts, s), s));
  }
  int32_t* inv = at<int32_t>(ws, y.inv);
  if (fused_forward(d)) {
    if (!in_place) TSA_TRY(after_launch(tsa::launch_build_inverse(d, idx, inv, s), s));
    if (d.keep == 0) {
      if (!in_place) return after_launch(tsa::launch_copy_unselected(d, inv, residual, out, s), s);
      return TSA_OK;
    }
    return after_launch(tsa::launch_attn_fused(d, q, k, v, idx, counts, at<int32_t>(ws, y.plan), residual, out,
                                               in_place ? nullptr : inv, s),
                        s);
  }
  void* qh = at<char>(ws, y.qh);
  void* kh = at<char>(ws, y.kh);
  void* vh = at<char>(ws, y.vh);
  void* oh = at<char>(ws, y.oh);
  if (d.keep > 0) {
    TSA_TRY(after_launch(tsa::launch_gather_qkv(d, q, k, v, idx, qh, kh, vh, s), s));
    TSA_TRY(after_launch(launch_attn_compact(d, qh, kh, vh, oh, s), s));
  }
  if (in_place) return after_launch(tsa::launch_scatter_inplace(d, oh, idx, out, s), s);
  TSA_TRY(after_launch(tsa::launch_build_inverse(d, idx, inv, s), s));
  return after_launch(tsa::launch_scatter_residual(d, oh, inv, residual, out, s), s);
}

tsa_status tsa_dense_attn(const tsa_desc* desc, const void* q, const void* k, const void* v, void* o, void* stream) {
  TSA_TRY(check_shape(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  if (!q || !k || !v || !o) return TSA_ERR_NULL;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o)) return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  const Range ro{o, z.q};
  if (overlap(ro, {q, z.q}) || overlap(ro, {k, z.kv}) || overlap(ro, {v, z.kv})) return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(tsa::launch_attn_dense(d, q, k, v, o, s), s);
}

tsa_status tsa_drift(const tsa_desc* desc, const void* a, const void* b, double* drift, void* ws, size_t ws_bytes,
                     void* stream) {
  TSA_TRY(check_shape(desc));
  const tsa_desc& d = *desc;
  if (empty_problem(d)) return TSA_OK;
  if (!a || !b || !drift) return TSA_ERR_NULL;
  if (!aligned(a) || !aligned(b) || !aligned(ws) || reinterpret_cast<uintptr_t>(drift) % 8 != 0) return TSA_ERR_ALIGN;
  const Sizes z = sizes_of(d);
  const size_t need = round_up(tsa::drift_workspace_bytes(d));
  if (!ws || ws_bytes < need) return TSA_ERR_WORKSPACE;
  const Range rw{ws, need}, rd{drift, sizeof(double)};
  if (overlap(rw, {a, z.q}) || overlap(rw, {b, z.q}) || overlap(rd, {a, z.q}) || overlap(rd, {b, z.q}) ||
      overlap(rd, rw))
    return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(tsa::launch_drift(d, a, b, drift, static_cast<double*>(ws), s), s);
}

tsa_status tsa_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0) return TSA_OK;
  if (!dst || !src) return TSA_ERR_NULL;
  if (!aligned(dst) || !aligned(src) || bytes % 16 != 0) return TSA_ERR_ALIGN;
  if (overlap({dst, bytes}, {src, bytes})) return TSA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(tsa::launch_stream_copy(dst, src, bytes, s), s);
}

}  // extern "C"
