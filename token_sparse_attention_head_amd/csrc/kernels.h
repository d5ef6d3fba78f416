// Host-side launchers of the token-sparse attention kernels (internal to libtsa.so).
#pragma once

#include <hip/hip_runtime.h>

#include "tsa.h"

namespace tsa {

// Token subsets: R rows of idx (H per query head, Hkv per KV head) and the number of
// query heads sharing one subset; query head h uses subset h / heads_per_subset.
inline int subset_rows(const tsa_desc& d) { return d.subsets == TSA_SUBSETS_PER_KV_HEAD ? d.Hkv : d.H; }
inline int heads_per_subset(const tsa_desc& d) { return d.H / subset_rows(d); }

// Key chunking of the scoring passes (shared by the launcher and workspace sizing).
void score_chunking(const tsa_desc& d, int& chunk, int& nchunk);

hipError_t launch_score(const tsa_desc& d, const void* q, const void* k, float* scores, float2* part, float2* stat,
                        hipStream_t s);
// Workspace of the select (each region 256-byte aligned): the summed score rows of a
// KV group (subsets per KV head only), the per-row state of the radix select, the
// per-row global histograms and the per-wave counts of the compaction; with adaptive
// budgets (tau > 0) also the per-row mass histograms, the budget state and the row
// budgets.  S position slices of seg positions per row.
struct SelectLayout {
  size_t gsum, state, hist, counts, mhist, bstate, budgets, total;
  int S, seg;
};
SelectLayout select_layout(const tsa_desc& d);
// Representation drift of [B][L][H*d] hidden states: partial sums in a workspace of
// drift_workspace_bytes(d) bytes, the result as one double.
size_t drift_workspace_bytes(const tsa_desc& d);
hipError_t launch_drift(const tsa_desc& d, const void* a, const void* b, double* out, double* partial,
                        hipStream_t s);
// Row budgets [B][R]: keep for every row, or the token-coverage budget when tau > 0.
hipError_t launch_budget(const tsa_desc& d, const float* scores, int32_t* counts, void* ws, hipStream_t s);
// Subsets into idx (rows padded with -1 below keep when tau > 0) and optionally the inverse
// map; with tau > 0 the row budgets go to `budgets` (NULL: the workspace).
hipError_t launch_select(const tsa_desc& d, const float* scores, int32_t* idx, int32_t* inv, int32_t* budgets,
                         void* ws, hipStream_t s);
hipError_t launch_gather_qkv(const tsa_desc& d, const void* q, const void* k, const void* v, const int32_t* idx,
                             void* qh, void* kh, void* vh, hipStream_t s);
hipError_t launch_attn_compact(const tsa_desc& d, const void* qh, const void* kh, const void* vh, void* oh,
                               hipStream_t s);
// Fused forward attention (bf16): compact rows read through idx, out rows = residual + O.
// counts (NULL: keep rows everywhere) gives each subset's row count under adaptive budgets;
// plan is a workspace of attn_plan_bytes(d) bytes for the per-XCD head lists (0 bytes: too
// many heads for a plan, heads are then interleaved over the XCDs).  inv (out of place; NULL
// in place) is the kept-row map: the same launch then also copies residual to out at the
// rows no subset keeps (inv < 0), on its first workgroups, overlapping the attention.
size_t attn_plan_bytes(const tsa_desc& d);
hipError_t launch_attn_fused(const tsa_desc& d, const void* q, const void* k, const void* v, const int32_t* idx,
                             const int32_t* counts, int32_t* plan, const void* res, void* out, const int32_t* inv,
                             hipStream_t s);
// Copies residual to out at the positions a head does not keep (inverse map < 0).
hipError_t launch_copy_unselected(const tsa_desc& d, const int32_t* inv, const void* res, void* out, hipStream_t s);
// Rows of every subset from an index list (first -1 entry, keep when there is none) into counts [B][R].
hipError_t launch_row_counts(const tsa_desc& d, const int32_t* idx, int32_t* counts, hipStream_t s);
// Plain device copy of bytes (a multiple of 16) from src to dst.
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_attn_dense(const tsa_desc& d, const void* q, const void* k, const void* v, void* o,
                             hipStream_t s);
hipError_t launch_build_inverse(const tsa_desc& d, const int32_t* idx, int32_t* inv, hipStream_t s);
hipError_t launch_scatter_residual(const tsa_desc& d, const void* oh, const int32_t* inv, const void* res, void* out,
                                   hipStream_t s);
hipError_t launch_scatter_inplace(const tsa_desc& d, const void* oh, const int32_t* idx, void* out, hipStream_t s);

}  // namespace tsa
