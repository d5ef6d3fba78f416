/*
 * tsa.h -- C ABI of the token-sparse attention library (libtsa.so), gfx950 only.
 *
 * The library runs one attention layer of Token Sparse Attention: every query head
 * scores the keys, keeps a subset S_h of them, runs dense causal attention on the
 * compact subset and scatters the result back to full length with the residual added.
 * Sources: the skill page "Token Sparse Attention Long Context" (Core Concept,
 * Architecture Overview, Steps 1-3) and the paper page "Token Sparse Attention:
 * Efficient Long-Context Inference with Interleaved Token Selection" (Abstract,
 * Figure 3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Sizes (tsa_desc):  B batch, H query heads, Hkv KV heads (H % Hkv == 0, G = H / Hkv),
 *   L sequence length, d head dim (64 or 128), keep = |S| positions per subset, W score
 *   window, n_sink sink tokens, dtype of q/k/v/residual/out and of the compact
 *   tensors, scale of the logits (0 means 1/sqrt(d)).
 * Grouped-query map: query head h reads KV head g(h) = h / G.
 * Subsets (tsa_desc.subsets): TSA_SUBSETS_PER_HEAD (the pages' method: every query head
 *   keeps its own subset S_h, R = H subsets) or TSA_SUBSETS_PER_KV_HEAD (an extension of
 *   this library, not from the pages: the G query heads of KV head g share one subset
 *   S_g, chosen by the same rule on the sum of their G score rows, R = Hkv subsets).  Query
 *   head h uses subset r(h) = h / (H / R).
 * Adaptive budgets (tsa_desc.tau > 0): the paper page lets per-head budgets adapt through
 *   a token coverage tau (TL;DR; Figures 1 and 5: higher is sparser) and gives no formula.
 *   This library's rule, per subset row: non-forced positions leave in the reverse of the
 *   keep order (lower score first, equal scores from the higher position) while the scores
 *   that left add up to at most floor(tau * T), T the row's total score; every score
 *   counts as a whole number of 2^-40 units, rounded down, so the sums are exact.  The
 *   row keeps K_r = min(L - leavers, keep) positions (keep is the cap; K_r >= |F|).  idx
 *   rows then hold K_r ascending positions followed by -1 padding up to keep.  tau = 0
 *   disables the rule (every row keeps exactly keep positions).
 * Layouts (contiguous, row-major, element strides implied by the sizes):
 *   q, residual, out, o        [B][L][H][d]      (dtype)
 *   k, v                        [B][L][Hkv][d]    (dtype)
 *   scores                      [B][H][L]         (fp32, always per query head)
 *   idx                         [B][R][keep]      (int32, strictly ascending per subset;
 *                                                  -1 padding past K_r when tau > 0)
 *   counts                      [B][R]            (int32, K_r of every subset row)
 *   qh, oh                      [B][H][keep][d]   (dtype; compact per-query-head tensors)
 *   kh, vh                      [B][R][keep][d]   (dtype; compact K/V rows of each subset,
 *                                                  read from KV head g(h) of its heads)
 * Memory and ownership: every pointer is a device pointer allocated by the caller and
 *   aligned to 16 bytes; the library allocates and frees nothing, keeps no pointer
 *   after a call returns, and holds no mutable global state.  Scratch space comes from
 *   the caller's workspace (ws, ws_bytes), sized by tsa_workspace_size.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *   call only enqueues work on it and returns; nothing synchronises, nothing copies
 *   between host and device.  Results are deterministic (no floating-point atomics).
 * Errors: arguments are validated on the host before anything is enqueued; on a
 *   validation error the call returns the status and writes nothing.  TSA_ERR_LAUNCH
 *   reports a failed kernel launch.  Faults inside kernels surface at the caller's
 *   next synchronisation.  Inputs must be finite; non-finite values give unspecified
 *   (but memory-safe) results.
 */
#ifndef TSA_H_
#define TSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TSA_ABI_VERSION 4
#define TSA_MAX_W 64 /* largest score window the scoring kernel holds in registers */
/* Scratch bytes tsa_forward_noalloc may use per GPU (its largest workspace). */
#define TSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

typedef enum {
  TSA_OK = 0,
  TSA_ERR_NULL = 1,      /* a required pointer is NULL */
  TSA_ERR_SHAPE = 2,     /* a size <= 0, H % Hkv != 0, d not 64/128, or sizes past index limits */
  TSA_ERR_BUDGET = 3,    /* keep < |forced set| or keep > L, W < 1 or W > TSA_MAX_W, n_sink < 0 */
  TSA_ERR_DTYPE = 4,     /* dtype not TSA_F32 / TSA_BF16 */
  TSA_ERR_ALIGN = 5,     /* a pointer not 16-byte aligned */
  TSA_ERR_WORKSPACE = 6, /* ws_bytes smaller than tsa_workspace_size, or ws NULL when needed */
  TSA_ERR_ALIAS = 7,     /* an output overlaps an input it must not overlap */
  TSA_ERR_LAUNCH = 8,    /* a kernel launch failed */
  TSA_ERR_ARG = 9        /* an enum argument (op, subsets) out of range, scale not finite / negative, or
                            tau outside [0, 1] */
} tsa_status;

typedef enum { TSA_F32 = 0, TSA_BF16 = 1 } tsa_dtype;

/* Who shares a token subset (see "Subsets" above). */
typedef enum { TSA_SUBSETS_PER_HEAD = 0, TSA_SUBSETS_PER_KV_HEAD = 1 } tsa_subsets;

/* Which call a workspace is sized for. */
typedef enum {
  TSA_OP_SCORE = 0,
  TSA_OP_SELECT = 1,
  TSA_OP_SCATTER = 2,
  TSA_OP_FORWARD = 3,
  TSA_OP_DRIFT = 4,
  TSA_OP_SPARSE_ATTN = 5
} tsa_op;

typedef struct {
  int32_t B, H, Hkv, L, d;
  int32_t keep;   /* |S|, the number of positions each subset keeps */
  int32_t W;      /* score window: the last min(W, L) query positions score the keys */
  int32_t n_sink; /* positions [0, n_sink) are always kept */
  int32_t dtype;  /* tsa_dtype */
  float scale;    /* logit scale; 0 selects 1/sqrt(d) */
  int32_t subsets; /* tsa_subsets */
  float tau;       /* token coverage in [0, 1]: 0 = every subset keeps `keep` positions, > 0 = adaptive
                      budgets capped at `keep` (see "Adaptive budgets") */
} tsa_desc;

/* Returns TSA_ABI_VERSION. */
int tsa_abi_version(void);

/* Static text for a status code (never NULL). */
const char* tsa_status_str(int status);

/* Host-only validation of a descriptor (no HIP call).  Forced set
 * F = [0, min(n_sink, L)) U [L - min(W, L), L); keep must satisfy |F| <= keep <= L;
 * subsets must be a tsa_subsets value (else TSA_ERR_ARG).  Index limits (else
 * TSA_ERR_SHAPE): B * H <= 65535, L * H * d * e < 2^35 and one batch entry's K (and V),
 * L * Hkv * d * e bytes, below 4 GiB (e = bytes per element). */
tsa_status tsa_check(const tsa_desc* desc);

/* Host-only: bytes of workspace the call `op` needs for `desc` (written to *bytes). */
tsa_status tsa_workspace_size(const tsa_desc* desc, int op, size_t* bytes);

/* Token scoring (skill page, Step 1: query-key alignment scores, softmax over keys
 * summed over queries; restricted here to the last W' = min(W, L) query rows, causal).
 * For every (b, h) and key j:
 *   scores[b][h][j] = sum over rows i in [L-W', L), i >= j, of
 *                     softmax_j'( scale * <q[b][i][h], k[b][j'][g(h)]> ), j' <= i,
 * evaluated at j.  Products accumulate in fp32, probabilities and sums are fp32.
 * In: q, k.  Out: scores.  Workspace: tsa_workspace_size(TSA_OP_SCORE). */
tsa_status tsa_score(const tsa_desc* desc, const void* q, const void* k, float* scores,
                     void* ws, size_t ws_bytes, void* stream);

/* Top-K selection (skill page, Step 1, selection of the top-scoring tokens; the paper
 * page's Figure 3 per-head subset S_h).  Per (b, r): S = F plus the keep - |F|
 * non-forced positions with the largest subset scores, equal scores going to the lower
 * position; written ascending to idx[b][r][0..keep).  The subset score is the head's
 * score row (per head) or, per KV head, the fp32 sum of the G rows of its query heads
 * taken in ascending head order.  Scores must be >= 0 (as tsa_score produces).  In:
 * scores [B][H][L].  Out: idx [B][R][keep].  Workspace: TSA_OP_SELECT (never 0: the
 * radix-select histograms and counts, about 8 KiB per (b, r) row, plus B*Hkv*L*4 bytes of
 * summed scores per KV head); its contents need no initialisation and are not kept. */
tsa_status tsa_select(const tsa_desc* desc, const float* scores, int32_t* idx,
                      void* ws, size_t ws_bytes, void* stream);

/* Adaptive budgets alone (paper page: TL;DR and Figures 1 and 5, token coverage; the rule
 * is the library's reading, see "Adaptive budgets").  In: scores [B][H][L] (>= 0).  Out:
 * counts [B][R], K_r of every subset row (keep everywhere when tau = 0), exactly the row
 * lengths tsa_select produces.  Workspace: TSA_OP_SELECT. */
tsa_status tsa_budget(const tsa_desc* desc, const float* scores, int32_t* counts,
                      void* ws, size_t ws_bytes, void* stream);

/* Gather-compression (skill page, Step 2, gathering the selected tokens; Figure 3,
 * stage 1):  qh[b][h][t] = q[b][idx[b][r(h)][t]][h]; for each subset r, with g the KV
 * head of its query heads, kh[b][r][t] = k[b][idx[b][r][t]][g] and vh likewise.
 * Bit-exact copies.  An idx entry outside [0, L) (the -1 padding of adaptive budgets)
 * gives zero rows at t.  The outputs must not overlap the inputs or one another. */
tsa_status tsa_gather_qkv(const tsa_desc* desc, const void* q, const void* k, const void* v,
                          const int32_t* idx, void* qh, void* kh, void* vh, void* stream);

/* Dense causal attention on the compact rows (skill page, Step 3; Figure 3, stage 2):
 *   oh[b][h][t] = sum over u <= t of
 *                 softmax_u( scale * <qh[b][h][t], kh[b][r(h)][u]> ) vh[b][r(h)][u],
 * fp32 accumulation and online softmax, result rounded once to dtype.  Because every
 * subset is ascending, the causal mask on compact rows equals the mask on original
 * positions, and rows t < K_r never see the zero rows gathered for padding entries.  oh
 * must not overlap qh, kh or vh. */
tsa_status tsa_attn(const tsa_desc* desc, const void* qh, const void* kh, const void* vh,
                    void* oh, void* stream);

/* Scatter-decompression plus residual (skill page, Step 2, scattering back to the full
 * sequence; Figure 3: scatter into the full layout, then add the residual):
 *   out[b][p][h] = residual[b][p][h] + oh[b][h][t]   if p = idx[b][r(h)][t],
 *   out[b][p][h] = residual[b][p][h]                 (bit-exact) otherwise;
 * idx entries outside [0, L) (padding) are skipped.
 * The sum is formed in fp32 and rounded once (round to nearest even).  out == residual
 * (exactly the same pointer) updates in place and touches only the kept rows; any other
 * overlap of out with residual, oh or idx is TSA_ERR_ALIAS.  Workspace: TSA_OP_SCATTER
 * (an inverse position map for the out-of-place pass; 0 bytes in place). */
tsa_status tsa_scatter_residual(const tsa_desc* desc, const void* oh, const int32_t* idx,
                                const void* residual, void* out, void* ws, size_t ws_bytes,
                                void* stream);

/* The whole layer in one call on one stream: score -> select -> gather -> attention ->
 * scatter + residual (the skill page's Core Concept compress/decompress sequence;
 * Figure 3, both stages).  scores_opt / idx_opt, when not NULL, receive the scores and
 * the subsets; otherwise they live in the workspace.  out may equal residual (in place).
 * With tau > 0 the row budgets are taken first and the attention runs only the K_r rows
 * of each subset.  Workspace: TSA_OP_FORWARD. */
tsa_status tsa_forward(const tsa_desc* desc, const void* q, const void* k, const void* v,
                       const void* residual, void* out, float* scores_opt, int32_t* idx_opt,
                       void* ws, size_t ws_bytes, void* stream);

/* tsa_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments and
 * results as tsa_forward (bit for bit), except that scores and idx are required outputs
 * and there is no workspace argument: the rest of the workspace (inverse map, select
 * histograms, score partials; for fp32 also the compact tensors) lives in a static device
 * array of TSA_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held until the process
 * ends.  A problem needing more (tsa_workspace_size(TSA_OP_FORWARD) minus the scores and
 * idx bytes, rounded up per region) returns TSA_ERR_WORKSPACE before anything runs; 32 MiB
 * cover a bf16 layer of B = 1, 32 query heads and L up to about 240K, per head.  The first
 * call on a device looks the array up on the current device (TSA_ERR_LAUNCH if that
 * fails).  Nothing is allocated or freed, no library routine that allocates is called.
 * Calls that overlap on one GPU share the array and race: the caller serialises them (one
 * stream, or events between streams).  Nothing in the array needs to start at zero. */
tsa_status tsa_forward_noalloc(const tsa_desc* desc, const void* q, const void* k, const void* v,
                               const void* residual, void* out, float* scores, int32_t* idx, void* stream);

/* Compress, attend and decompress on given subsets (the paper page's Figure 3, stages 1
 * and 2; skill page, Steps 2 and 3): for every query head h with subset r(h) and its
 * K_r kept rows,
 *   out[b][p][h] = residual[b][p][h] + O[b][h][t]   if p = idx[b][r(h)][t], t < K_r,
 *   out[b][p][h] = residual[b][p][h]                (bit-exact) otherwise,
 * with O the causal attention of tsa_attn over the rows q, k, v hold at the subset's
 * positions, rounded to dtype, and residual + O summed in fp32 and rounded once: exactly
 * what tsa_gather_qkv -> tsa_attn -> tsa_scatter_residual produce.  idx [B][R][keep] as
 * tsa_select writes it: ascending positions in [0, L), then (tau > 0 only) -1 padding;
 * the row counts K_r are read off the padding.  bf16 runs one attention kernel that
 * reads the rows through idx and writes residual + O into the kept rows (no compact
 * tensors); out of place, the same launch copies the residual to the rows no head keeps
 * (on workgroups of its own, while the others run the attention).  fp32 runs the three
 * stages through compact tensors in the workspace.  out ==
 * residual (the same pointer) updates in place; any other overlap of out with an input
 * is TSA_ERR_ALIAS.  Positions outside [0, L) in a kept row give unspecified results but
 * no access outside the tensors.  Workspace: TSA_OP_SPARSE_ATTN. */
tsa_status tsa_sparse_attn(const tsa_desc* desc, const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* residual, void* out, void* ws, size_t ws_bytes, void* stream);

/* Dense causal attention over all L positions with grouped-query heads, the library's
 * own full-attention reference (the paper page's Abstract: the method composes with
 * dense attention kernels).  o[b][i][h] = sum over j <= i of
 * softmax_j(scale * <q[b][i][h], k[b][j][g(h)]>) v[b][j][g(h)].  keep, W and n_sink
 * are ignored.  o must not overlap q, k or v. */
tsa_status tsa_dense_attn(const tsa_desc* desc, const void* q, const void* k, const void* v,
                          void* o, void* stream);

/* Representation drift between a layer's input and output hidden states (skill page,
 * Step 4, the layer-stability analysis; paper page, Figure 4):
 *   drift = 1 - (1/T) sum over tokens t of <a_t, b_t> / (max(|a_t|, 1e-12) max(|b_t|, 1e-12)),
 * over the T = B*L token rows of a, b [B][L][H][d] (dtype; each row is one hidden vector of
 * H*d values, e.g. the layer's residual input and its output).  Per token the dot product
 * and the squared norms accumulate in fp32 and the cosine is formed in fp32; the mean
 * accumulates in fp64 in a fixed order (deterministic).  Out: drift[0], one double in
 * device memory (8-byte aligned), not written for an empty problem.  Only the sizes and
 * dtype of desc are used (keep, W, n_sink, subsets, tau are ignored).  Workspace:
 * TSA_OP_DRIFT (partial sums).  A layer counts as stable once the mean of its last three
 * drifts is below 0.1 (host logic, not part of the library). */
tsa_status tsa_drift(const tsa_desc* desc, const void* a, const void* b, double* drift,
                     void* ws, size_t ws_bytes, void* stream);

/* Plain device copy of `bytes` bytes (a multiple of 16; src and dst 16-byte aligned and
 * not overlapping), streamed with non-temporal 16-byte loads and stores.  Not a step of
 * the method: it is the measured bandwidth reference that the library's data-movement
 * kernels (gather, scatter, the copy of unkept rows, drift) are compared with, and the
 * calibration kernel of hardware byte counters. */
tsa_status tsa_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSA_H_ */
