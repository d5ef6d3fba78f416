// Top-K token selection per (batch, subset row): the subset S, ascending.
//
// The skill page "Token Sparse Attention Long Context", Step 1, keeps the top-scoring
// tokens of each head; the paper page "Token Sparse Attention: Efficient Long-Context
// Inference with Interleaved Token Selection", Figure 3, calls the result the per-head
// token subset.  This library fixes what the pages leave open: the sink positions
// [0, n_sink) and the window [L-W', L) are always kept, the remaining budget goes to
// the highest scores with ties to the lower position, and S_h is written in ascending
// position order.
//
// Scores are >= 0, so their fp32 bit patterns order like the values.  The threshold T
// (the score of the last candidate taken) is found by a three-pass radix select
// (11 + 11 + 10 bits) whose histograms are built by many workgroups per row; then every
// wave compacts its own contiguous range of positions with wave ballots and mbcnt prefix
// counts, ties at T going to the lowest positions.
#include "common.h"
#include "kernels.h"

namespace tsa {

namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / TSA_WAVE;
constexpr int SEL_MAX_BINS = 2048;
constexpr int SEL_UNROLL = 8;      // loads in flight per thread in the streaming passes
constexpr int SEL_MAX_SLICES = 64; // position slices (workgroups) per row

// Inclusive scan of one value per thread over the whole workgroup.
__device__ uint32_t block_inclusive_scan(uint32_t x, uint32_t* wave_tot) {
  const int lane = lane_id();
  const int wave = threadIdx.x / TSA_WAVE;
#pragma unroll
  for (int o = 1; o < TSA_WAVE; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, TSA_WAVE);
    if (lane >= o) x += y;
  }
  if (lane == TSA_WAVE - 1) wave_tot[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  __syncthreads();
  return x + before;
}

// Per-KV-head subsets: the score row of KV head g is the fp32 sum, in ascending head
// order, of the score rows of its G query heads (rows (b*R + g)*G + h' of [B][H][L]).
__global__ __launch_bounds__(256) void group_sum_kernel(const float* __restrict__ scores, float* __restrict__ out,
                                                        int G, int L, int64_t n) {
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t row = e / L;
    const int64_t j = e - row * L;
    const float* src = scores + row * G * L + j;
    float acc = src[0];
    for (int h = 1; h < G; ++h) acc += src[(int64_t)h * L];
    out[e] = acc;
  }
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ out, int32_t v, int64_t n) {
  const int64_t i = blockIdx.x * 256ll + threadIdx.x;
  if (i < n) out[i] = v;
}

// ---- multi-workgroup radix select --------------------------------------------------
//
// A row is split into S position slices of seg positions (seg a multiple of 256), one
// 256-thread workgroup each, so every CU helps even when there are few rows.  Per-row
// state in the workspace: need (candidates still to take), prefix and pmask of the
// threshold key found so far, and mode (0: threshold needed, 1: take every candidate,
// 2: take none).  Each pass: every slice builds an LDS histogram of the candidates that
// match the prefix and adds it to the row's global histogram; one workgroup per row then
// scans it from the top, narrows the prefix and clears the histogram.  After three
// passes the prefix is the threshold key T and need is the number of candidates equal
// to T to take (lowest positions first).  Compaction: every wave of every slice counts
// its strict and equal positions; then every wave writes its positions at the offset the
// counts of all earlier waves give, in position order.
constexpr int SEL_WG = 256;
constexpr int SEL_WG_WAVES = SEL_WG / TSA_WAVE;

struct SelGeom {
  int L, keep, c0, c1, S, seg;
};

__device__ __forceinline__ int sel_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ int sel_bins(int pass) { return pass == 2 ? 1024 : SEL_MAX_BINS; }

// Subset size of a row: keep, or the row's adaptive budget.
__device__ __forceinline__ int row_keep(const int32_t* counts, int row, const SelGeom& g) {
  return counts ? counts[row] : g.keep;
}

__global__ __launch_bounds__(SEL_WG) void sel_init_kernel(uint32_t* __restrict__ state, uint32_t* __restrict__ hist,
                                                          const int32_t* __restrict__ counts, SelGeom g) {
  const int row = blockIdx.x;
  for (int i = threadIdx.x; i < SEL_MAX_BINS; i += SEL_WG) hist[(int64_t)row * SEL_MAX_BINS + i] = 0;
  if (threadIdx.x == 0) {
    const int n_cand = g.c1 - g.c0;
    const int need = row_keep(counts, row, g) - (g.L - n_cand);
    uint32_t* st = state + (int64_t)row * 4;
    st[0] = (uint32_t)need;
    st[1] = 0;
    st[2] = 0;
    st[3] = need >= n_cand ? 1u : (need == 0 ? 2u : 0u);
  }
}

__global__ __launch_bounds__(SEL_WG) void sel_hist_kernel(const float* __restrict__ scores,
                                                          const uint32_t* __restrict__ state,
                                                          uint32_t* __restrict__ hist, SelGeom g, int pass) {
  __shared__ uint32_t lh[SEL_MAX_BINS];
  const int row = blockIdx.y;
  const uint32_t* st = state + (int64_t)row * 4;
  if (st[3] != 0) return;
  const uint32_t prefix = st[1], pmask = st[2];
  const int shift = sel_shift(pass), nb = sel_bins(pass);
  const int tid = threadIdx.x;
  for (int i = tid; i < nb; i += SEL_WG) lh[i] = 0;
  __syncthreads();
  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores + (int64_t)row * g.L);
  const int beg = max(g.c0, blockIdx.x * g.seg);
  const int end = min(g.c1, (blockIdx.x + 1) * g.seg);
  for (int j0 = beg + tid; j0 < end; j0 += SEL_UNROLL * SEL_WG) {
    uint32_t u[SEL_UNROLL];
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = j0 + k * SEL_WG;
      u[k] = j < end ? key[j] : 0u;
    }
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = j0 + k * SEL_WG;
      if (j < end && (u[k] & pmask) == prefix) atomicAdd(&lh[(u[k] >> shift) & (nb - 1)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)row * SEL_MAX_BINS;
  for (int i = tid; i < nb; i += SEL_WG)
    if (lh[i] != 0) atomicAdd(&gh[i], lh[i]);
}

__global__ __launch_bounds__(SEL_THREADS) void sel_find_kernel(uint32_t* __restrict__ state, uint32_t* __restrict__ hist,
                                                               int pass) {
  __shared__ uint32_t wave_tot[SEL_WAVES];
  const int row = blockIdx.x;
  uint32_t* st = state + (int64_t)row * 4;
  if (st[3] != 0) return;
  const uint32_t need = st[0];
  const int shift = sel_shift(pass), nb = sel_bins(pass);
  const int tid = threadIdx.x;
  uint32_t* gh = hist + (int64_t)row * SEL_MAX_BINS;
  // Bins in descending order; thread t owns ranks [t*per, (t+1)*per).
  const int per = nb / SEL_THREADS;
  uint32_t cnt[SEL_MAX_BINS / SEL_THREADS];
  uint32_t local = 0;
  for (int q = 0; q < per; ++q) {
    cnt[q] = gh[nb - 1 - (tid * per + q)];
    local += cnt[q];
  }
  const uint32_t incl = block_inclusive_scan(local, wave_tot);
  const uint32_t excl = incl - local;
  if (excl < need && need <= incl) {
    uint32_t cum = excl;
    for (int q = 0; q < per; ++q) {
      if (cum + cnt[q] >= need) {
        const uint32_t bin = (uint32_t)(nb - 1 - (tid * per + q));
        st[0] = need - cum;
        st[1] |= bin << shift;
        st[2] |= (uint32_t)(nb - 1) << shift;
        break;
      }
      cum += cnt[q];
    }
  }
  __syncthreads();
  for (int i = tid; i < nb; i += SEL_THREADS) gh[i] = 0;   // clear for the next pass
}

// Whether position j (of a wave's range) is a forced or above-threshold position (strict)
// or a candidate equal to the threshold (eq).
struct SelRule {
  int c0, c1;
  uint32_t T;
  bool take_all, take_none;
  __device__ __forceinline__ void classify(int j, bool valid, uint32_t u, bool& strict, bool& eq) const {
    const bool cand = valid && j >= c0 && j < c1;
    strict = (valid && !cand) || (cand && (take_all || (!take_none && u > T)));
    eq = cand && !take_all && !take_none && u == T;
  }
};

__device__ __forceinline__ SelRule sel_rule(const uint32_t* st, const SelGeom& g) {
  SelRule r;
  r.c0 = g.c0;
  r.c1 = g.c1;
  r.take_all = st[3] == 1;
  r.take_none = st[3] == 2;
  r.T = st[1];
  return r;
}

__global__ __launch_bounds__(SEL_WG) void sel_count_kernel(const float* __restrict__ scores,
                                                           const uint32_t* __restrict__ state,
                                                           uint32_t* __restrict__ counts, SelGeom g) {
  const int row = blockIdx.y, s = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x / TSA_WAVE;
  const SelRule rule = sel_rule(state + (int64_t)row * 4, g);
  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores + (int64_t)row * g.L);
  const int wseg = g.seg / SEL_WG_WAVES;
  const int beg = s * g.seg + wave * wseg;
  const int end = min(g.L, beg + wseg);
  uint32_t n_strict = 0, n_eq = 0;
  for (int base = beg; base < end; base += SEL_UNROLL * TSA_WAVE) {
    uint32_t u[SEL_UNROLL];
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = base + k * TSA_WAVE + lane;
      u[k] = (j < end && j >= rule.c0 && j < rule.c1) ? key[j] : 0u;
    }
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = base + k * TSA_WAVE + lane;
      bool st, eq;
      rule.classify(j, j < end, u[k], st, eq);
      n_strict += __popcll(__ballot(st));
      n_eq += __popcll(__ballot(eq));
    }
  }
  if (lane == 0) {
    uint32_t* c = counts + (((int64_t)row * g.S + s) * SEL_WG_WAVES + wave) * 2;
    c[0] = n_strict;
    c[1] = n_eq;
  }
}

__global__ __launch_bounds__(SEL_WG) void sel_write_kernel(const float* __restrict__ scores,
                                                           const uint32_t* __restrict__ state,
                                                           const uint32_t* __restrict__ counts,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ inv,
                                                           const int32_t* __restrict__ budgets, SelGeom g) {
  const int row = blockIdx.y, s = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x / TSA_WAVE;
  const uint32_t keep = (uint32_t)row_keep(budgets, row, g);
  const uint32_t* st = state + (int64_t)row * 4;
  const SelRule rule = sel_rule(st, g);
  const uint32_t need_eq = (rule.take_all || rule.take_none) ? 0u : st[0];
  // This wave's offset: the strict positions of every earlier wave of the row plus the
  // equal ones they take, min(need_eq, equal positions before this wave).
  const int my_w = s * SEL_WG_WAVES + wave;
  const uint32_t* crow = counts + (int64_t)row * g.S * SEL_WG_WAVES * 2;
  uint32_t n_st = 0, n_eq = 0;
  for (int w = lane; w < my_w; w += TSA_WAVE) {
    n_st += crow[2 * w];
    n_eq += crow[2 * w + 1];
  }
#pragma unroll
  for (int o = TSA_WAVE / 2; o > 0; o >>= 1) {
    n_st += __shfl_xor(n_st, o, TSA_WAVE);
    n_eq += __shfl_xor(n_eq, o, TSA_WAVE);
  }
  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores + (int64_t)row * g.L);
  int32_t* row_idx = idx + (int64_t)row * g.keep;
  int32_t* row_inv = inv ? inv + (int64_t)row * g.L : nullptr;
  // A row with an adaptive budget below keep is padded with -1.
  for (int t = (int)keep + s * SEL_WG + (int)threadIdx.x; t < g.keep; t += g.S * SEL_WG) row_idx[t] = -1;
  const int wseg = g.seg / SEL_WG_WAVES;
  const int beg = s * g.seg + wave * wseg;
  const int end = min(g.L, beg + wseg);
  uint32_t pos = n_st + min(need_eq, n_eq);
  uint32_t eq_rank = n_eq;
  for (int base = beg; base < end; base += SEL_UNROLL * TSA_WAVE) {
    uint32_t u[SEL_UNROLL];
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = base + k * TSA_WAVE + lane;
      u[k] = (j < end && j >= rule.c0 && j < rule.c1) ? key[j] : 0u;
    }
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = base + k * TSA_WAVE + lane;
      bool strict, e;
      rule.classify(j, j < end, u[k], strict, e);
      const uint64_t emask = __ballot(e);
      const uint32_t my_eq = eq_rank + __builtin_amdgcn_mbcnt_hi((uint32_t)(emask >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)emask, 0u));
      const bool take = strict || (e && my_eq < need_eq);
      const uint64_t tmask = __ballot(take);
      const uint32_t my_pos = pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(tmask >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)tmask, 0u));
      if (take && my_pos < keep) row_idx[my_pos] = j;
      if (row_inv && j < end) row_inv[j] = (take && my_pos < keep) ? (int32_t)my_pos : -1;
      pos += __popcll(tmask);
      eq_rank += __popcll(emask);
    }
  }
}


__device__ unsigned long long block_inclusive_scan64(unsigned long long x, unsigned long long* wave_tot);

// ---- one-workgroup select for rows of at most 16384 positions ------------------------
//
// The same rule and the same three radix passes, in one launch: a 1024-thread workgroup per
// row holds the row's scores in registers (thread t owns the PER consecutive positions
// [t*PER, (t+1)*PER)), builds each pass's histogram in LDS and scans it itself, then counts
// its strict and equal positions; one block-wide scan of the (strict, equal) counts gives
// every thread the offset of its positions, which it writes in ascending order, ties at T
// to the lowest positions.  For short rows the nine launches of the multi-workgroup path
// cost more than the work: 32 rows, L = 8192: 34 us, here 14 us; at L = 32768 one workgroup
// per row is slower (45 us against 31: 32 workgroups on 256 CUs each do a whole row's passes
// serially; four histogram copies per workgroup, a quarter of the threads each, made no
// difference, so it is not the atomics).
constexpr int SEL_ROW_MAX_L = 16384;

template <int PER>
__global__ __launch_bounds__(SEL_THREADS) void sel_row_kernel(const float* __restrict__ scores,
                                                              int32_t* __restrict__ idx, int32_t* __restrict__ inv,
                                                              const int32_t* __restrict__ budgets, SelGeom g) {
  __shared__ uint32_t hist[SEL_MAX_BINS];
  __shared__ uint32_t wave_tot[SEL_WAVES];
  __shared__ unsigned long long wave_tot64[SEL_WAVES];
  __shared__ uint32_t found[2];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores + (int64_t)row * g.L);
  const int j0 = tid * PER;
  uint32_t u[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) u[p] = j0 + p < g.L ? key[j0 + p] : 0u;
  const int keep = row_keep(budgets, row, g);
  const int n_cand = g.c1 - g.c0;
  uint32_t need = (uint32_t)(keep - (g.L - n_cand));
  const bool take_all = (int)need >= n_cand, take_none = need == 0;
  uint32_t prefix = 0, pmask = 0;
  if (!take_all && !take_none) {
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = sel_shift(pass), nb = sel_bins(pass);
      for (int i = tid; i < nb; i += SEL_THREADS) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int j = j0 + p;
        if (j >= g.c0 && j < g.c1 && (u[p] & pmask) == prefix) atomicAdd(&hist[(u[p] >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      // Bins in descending order; thread t owns ranks [t*per, (t+1)*per).
      const int per = nb / SEL_THREADS;
      uint32_t cnt[SEL_MAX_BINS / SEL_THREADS];
      uint32_t local = 0;
      for (int q = 0; q < per; ++q) {
        cnt[q] = hist[nb - 1 - (tid * per + q)];
        local += cnt[q];
      }
      const uint32_t incl = block_inclusive_scan(local, wave_tot);
      const uint32_t excl = incl - local;
      if (excl < need && need <= incl) {
        uint32_t cum = excl;
        for (int q = 0; q < per; ++q) {
          if (cum + cnt[q] >= need) {
            found[0] = need - cum;
            found[1] = (uint32_t)(nb - 1 - (tid * per + q));
            break;
          }
          cum += cnt[q];
        }
      }
      __syncthreads();
      need = found[0];
      prefix |= found[1] << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      __syncthreads();                             // found and hist are rewritten next pass
    }
  }
  SelRule rule;
  rule.c0 = g.c0;
  rule.c1 = g.c1;
  rule.T = prefix;
  rule.take_all = take_all;
  rule.take_none = take_none;
  const uint32_t need_eq = (take_all || take_none) ? 0u : need;
  uint32_t n_st = 0, n_eq = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    bool st, eq;
    rule.classify(j0 + p, j0 + p < g.L, u[p], st, eq);
    n_st += st;
    n_eq += eq;
  }
  const unsigned long long mine = ((unsigned long long)n_st << 32) | n_eq;
  const unsigned long long before = block_inclusive_scan64(mine, wave_tot64) - mine;
  uint32_t pos = (uint32_t)(before >> 32) + min(need_eq, (uint32_t)before);
  uint32_t eq_rank = (uint32_t)before;
  int32_t* row_idx = idx + (int64_t)row * g.keep;
  int32_t* row_inv = inv ? inv + (int64_t)row * g.L : nullptr;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int j = j0 + p;
    bool st, eq;
    rule.classify(j, j < g.L, u[p], st, eq);
    const bool take = st || (eq && eq_rank < need_eq);
    eq_rank += eq;
    if (take && pos < (uint32_t)keep) row_idx[pos] = j;
    if (row_inv && j < g.L) row_inv[j] = (take && pos < (uint32_t)keep) ? (int32_t)pos : -1;
    pos += take;
  }
  for (int t = keep + tid; t < g.keep; t += SEL_THREADS) row_idx[t] = -1;   // adaptive budget below keep
}

// ---- adaptive budgets (token coverage tau) ------------------------------------------
//
// The paper page "Token Sparse Attention: Efficient Long-Context Inference with
// Interleaved Token Selection" lets per-head budgets adapt through a token coverage tau
// (TL;DR; Figures 1 and 5: higher is sparser) without a formula.  This library's rule:
// non-forced positions leave in the reverse of the keep order (lower score first, equal
// scores from the higher position) while the scores that left sum to at most
// floor(tau * total), all masses in whole units of 2^-40 (each score rounded down, so the
// sums are exact integers); K = L - (positions that left), capped at keep.
//
// The same radix passes as the select, walking the bins upwards: each slice adds the
// count and the 64-bit mass of its candidates to the row's global histograms (pass 0
// also sums the units of all L positions into the row total); one workgroup per row then
// finds the first bin whose cumulative mass exceeds the remaining budget, counts every
// candidate below it as leaving and narrows the prefix.  If no bin exceeds it, every
// candidate still in play leaves.  After the last pass the prefix is one key T with unit
// mass u_T > 0, of which floor(remaining / u_T) leave (at most all of them).
struct BudState {
  unsigned long long rem;     // budget still to spend (units)
  unsigned long long total;   // units of all L positions (pass 0)
  uint32_t left;              // candidates known to leave
  uint32_t prefix, pmask;     // key bits fixed so far
  uint32_t done;              // 1 once the row's count is final
};

__device__ __forceinline__ unsigned long long mass_units(uint32_t key) {
  return (unsigned long long)((double)__uint_as_float(key) * 1099511627776.0);   // x 2^40, rounded down
}

__global__ __launch_bounds__(SEL_WG) void bud_init_kernel(BudState* __restrict__ st, uint32_t* __restrict__ hist,
                                                          unsigned long long* __restrict__ mhist, int32_t* __restrict__ counts,
                                                          SelGeom g) {
  const int row = blockIdx.x;
  for (int i = threadIdx.x; i < SEL_MAX_BINS; i += SEL_WG) {
    hist[(int64_t)row * SEL_MAX_BINS + i] = 0;
    mhist[(int64_t)row * SEL_MAX_BINS + i] = 0;
  }
  if (threadIdx.x == 0) {
    BudState b;
    b.rem = 0;
    b.total = 0;
    b.left = 0;
    b.prefix = 0;
    b.pmask = 0;
    b.done = g.c1 > g.c0 ? 0u : 1u;             // no candidates: nothing can leave
    st[row] = b;
    if (b.done) counts[row] = min(g.L, g.keep);
  }
}

__global__ __launch_bounds__(SEL_WG) void bud_hist_kernel(const float* __restrict__ scores, BudState* __restrict__ st,
                                                          uint32_t* __restrict__ hist,
                                                          unsigned long long* __restrict__ mhist, SelGeom g, int pass) {
  __shared__ uint32_t lc[SEL_MAX_BINS];
  __shared__ unsigned long long lm[SEL_MAX_BINS];
  __shared__ unsigned long long ltot[SEL_WG_WAVES];
  const int row = blockIdx.y;
  const BudState b = st[row];
  if (b.done) return;
  const int shift = sel_shift(pass), nb = sel_bins(pass);
  const int tid = threadIdx.x;
  for (int i = tid; i < nb; i += SEL_WG) {
    lc[i] = 0;
    lm[i] = 0;
  }
  __syncthreads();
  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores + (int64_t)row * g.L);
  // Pass 0 reads the whole slice (forced positions count towards the total).
  const int lo = pass == 0 ? blockIdx.x * g.seg : max(g.c0, blockIdx.x * g.seg);
  const int hi = pass == 0 ? min(g.L, (blockIdx.x + 1) * g.seg) : min(g.c1, (blockIdx.x + 1) * g.seg);
  unsigned long long tot = 0;
  for (int j0 = lo + tid; j0 < hi; j0 += SEL_UNROLL * SEL_WG) {
    uint32_t u[SEL_UNROLL];
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = j0 + k * SEL_WG;
      u[k] = j < hi ? key[j] : 0u;
    }
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = j0 + k * SEL_WG;
      if (j >= hi) continue;
      const unsigned long long m = mass_units(u[k]);
      tot += m;
      if (j >= g.c0 && j < g.c1 && (u[k] & b.pmask) == b.prefix) {
        const int bin = (u[k] >> shift) & (nb - 1);
        atomicAdd(&lc[bin], 1u);
        if (m) atomicAdd(&lm[bin], m);
      }
    }
  }
  if (pass == 0) {
#pragma unroll
    for (int o = TSA_WAVE / 2; o > 0; o >>= 1) tot += __shfl_xor(tot, o, TSA_WAVE);
    if (lane_id() == 0) ltot[tid / TSA_WAVE] = tot;
  }
  __syncthreads();
  const int64_t base = (int64_t)row * SEL_MAX_BINS;
  for (int i = tid; i < nb; i += SEL_WG) {
    if (lc[i] != 0) atomicAdd(&hist[base + i], lc[i]);
    if (lm[i] != 0) atomicAdd(&mhist[base + i], lm[i]);
  }
  if (pass == 0 && tid == 0) {
    unsigned long long t = 0;
    for (int w = 0; w < SEL_WG_WAVES; ++w) t += ltot[w];
    if (t) atomicAdd(&st[row].total, t);
  }
}

// Inclusive scan of one 64-bit value per thread over the workgroup.
__device__ unsigned long long block_inclusive_scan64(unsigned long long x, unsigned long long* wave_tot) {
  const int lane = lane_id();
  const int wave = threadIdx.x / TSA_WAVE;
#pragma unroll
  for (int o = 1; o < TSA_WAVE; o <<= 1) {
    const unsigned long long y = __shfl_up(x, o, TSA_WAVE);
    if (lane >= o) x += y;
  }
  if (lane == TSA_WAVE - 1) wave_tot[wave] = x;
  __syncthreads();
  unsigned long long before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  __syncthreads();
  return x + before;
}

__global__ __launch_bounds__(SEL_THREADS) void bud_find_kernel(BudState* __restrict__ st, uint32_t* __restrict__ hist,
                                                               unsigned long long* __restrict__ mhist,
                                                               int32_t* __restrict__ counts, SelGeom g, float tau,
                                                               int pass) {
  __shared__ uint32_t wave_cnt[SEL_WAVES];
  __shared__ unsigned long long wave_mass[SEL_WAVES];
  __shared__ int found;
  const int row = blockIdx.x;
  BudState* bs = st + row;
  if (bs->done) return;
  const int shift = sel_shift(pass), nb = sel_bins(pass);
  const int tid = threadIdx.x;
  if (tid == 0) found = 0;
  unsigned long long rem = bs->rem;
  if (pass == 0) rem = (unsigned long long)((double)tau * (double)bs->total);   // floor(tau * total)
  const int64_t base = (int64_t)row * SEL_MAX_BINS;
  // Bins in ascending order; thread t owns bins [t*per, (t+1)*per).
  const int per = nb / SEL_THREADS;
  uint32_t cnt[SEL_MAX_BINS / SEL_THREADS];
  unsigned long long ms[SEL_MAX_BINS / SEL_THREADS];
  uint32_t c_loc = 0;
  unsigned long long m_loc = 0;
  for (int q = 0; q < per; ++q) {
    cnt[q] = hist[base + tid * per + q];
    ms[q] = mhist[base + tid * per + q];
    c_loc += cnt[q];
    m_loc += ms[q];
  }
  const uint32_t c_incl = block_inclusive_scan(c_loc, wave_cnt);
  const unsigned long long m_incl = block_inclusive_scan64(m_loc, wave_mass);
  const uint32_t c_excl = c_incl - c_loc;
  const unsigned long long m_excl = m_incl - m_loc;
  if (m_excl <= rem && rem < m_incl) {
    // The first bin whose cumulative mass exceeds the budget is one of this thread's.
    uint32_t c_cum = c_excl;
    unsigned long long m_cum = m_excl;
    for (int q = 0; q < per; ++q) {
      if (m_cum + ms[q] > rem) {
        const uint32_t bin = (uint32_t)(tid * per + q);
        const unsigned long long r = rem - m_cum;
        uint32_t left = bs->left + c_cum;
        if (pass == 2) {
          // One key T: floor(r / u_T) of its cnt[q] positions leave (u_T > 0 here).
          const unsigned long long uT = mass_units(bs->prefix | bin);
          const unsigned long long n = r / uT;
          left += (uint32_t)(n < cnt[q] ? n : cnt[q]);
          counts[row] = min(g.L - (int)left, g.keep);
          bs->done = 1;
        } else {
          bs->rem = r;
          bs->prefix |= bin << shift;
          bs->pmask |= (uint32_t)(nb - 1) << shift;
        }
        bs->left = left;
        found = 1;
        break;
      }
      c_cum += cnt[q];
      m_cum += ms[q];
    }
  }
  __syncthreads();
  if (tid == SEL_THREADS - 1 && !found) {
    // No bin exceeds the budget: every candidate still in play leaves.
    const uint32_t left = bs->left + c_incl;
    counts[row] = min(g.L - (int)left, g.keep);
    bs->done = 1;
  }
  for (int i = tid; i < nb; i += SEL_THREADS) {   // clear for the next pass
    hist[base + i] = 0;
    mhist[base + i] = 0;
  }
}
}  // namespace

SelectLayout select_layout(const tsa_desc& d) {
  const int64_t rows = (int64_t)d.B * subset_rows(d);
  SelectLayout y;
  // About 512 workgroups per pass, at least 256 positions per slice.
  int S = (int)std::min<int64_t>(std::max<int64_t>((512 + rows - 1) / std::max<int64_t>(rows, 1), 1), SEL_MAX_SLICES);
  const int L = d.L > 0 ? d.L : 1;
  y.seg = ((L + S - 1) / S + SEL_WG - 1) / SEL_WG * SEL_WG;
  y.S = (L + y.seg - 1) / y.seg;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const bool adaptive = d.tau > 0.f;
  size_t o = 0;
  y.gsum = o; o += heads_per_subset(d) > 1 ? up((size_t)rows * d.L * 4) : 0;
  y.state = o; o += up((size_t)rows * 4 * 4);
  y.hist = o; o += up((size_t)rows * SEL_MAX_BINS * 4);
  y.counts = o; o += up((size_t)rows * y.S * SEL_WG_WAVES * 2 * 4);
  y.mhist = o; o += adaptive ? up((size_t)rows * SEL_MAX_BINS * 8) : 0;
  y.bstate = o; o += adaptive ? up((size_t)rows * sizeof(BudState)) : 0;
  y.budgets = o; o += adaptive ? up((size_t)rows * 4) : 0;
  y.total = o;
  return y;
}

namespace {

// The score rows the subsets are chosen on: the head's own row, or the fp32 group sums.
const float* subset_scores(const tsa_desc& d, const float* scores, const SelectLayout& y, char* base,
                           hipStream_t s) {
  const int G = heads_per_subset(d);
  if (G == 1) return scores;
  float* gsum = reinterpret_cast<float*>(base + y.gsum);
  const int64_t n = (int64_t)d.B * subset_rows(d) * d.L;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
  group_sum_kernel<<<blocks, 256, 0, s>>>(scores, gsum, G, d.L, n);
  return gsum;
}

SelGeom sel_geom(const tsa_desc& d, const SelectLayout& y) {
  const int Wp = d.W < d.L ? d.W : d.L;
  const int c1 = d.L - Wp;
  const int c0 = d.n_sink < c1 ? d.n_sink : c1;
  return SelGeom{d.L, d.keep, c0, c1, y.S, y.seg};
}

// Row budgets under token coverage d.tau (> 0) into counts [B][R].
void budget_rows(const tsa_desc& d, const float* src, int32_t* counts, const SelectLayout& y, char* base,
                 hipStream_t s) {
  const int rows = d.B * subset_rows(d);
  const SelGeom g = sel_geom(d, y);
  BudState* st = reinterpret_cast<BudState*>(base + y.bstate);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + y.hist);
  unsigned long long* mhist = reinterpret_cast<unsigned long long*>(base + y.mhist);
  bud_init_kernel<<<rows, SEL_WG, 0, s>>>(st, hist, mhist, counts, g);
  for (int pass = 0; pass < 3; ++pass) {
    bud_hist_kernel<<<dim3(y.S, rows), SEL_WG, 0, s>>>(src, st, hist, mhist, g, pass);
    bud_find_kernel<<<rows, SEL_THREADS, 0, s>>>(st, hist, mhist, counts, g, d.tau, pass);
  }
}

}  // namespace

hipError_t launch_budget(const tsa_desc& d, const float* scores, int32_t* counts, void* ws, hipStream_t s) {
  const SelectLayout y = select_layout(d);
  char* base = static_cast<char*>(ws);
  if (d.tau > 0.f) {
    budget_rows(d, subset_scores(d, scores, y, base, s), counts, y, base, s);
  } else {
    const int64_t rows = (int64_t)d.B * subset_rows(d);
    fill_i32_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(counts, d.keep, rows);
  }
  return hipGetLastError();
}

hipError_t launch_select(const tsa_desc& d, const float* scores, int32_t* idx, int32_t* inv, int32_t* budgets,
                         void* ws, hipStream_t s) {
  const int rows = d.B * subset_rows(d);
  const SelectLayout y = select_layout(d);
  char* base = static_cast<char*>(ws);
  const float* src = subset_scores(d, scores, y, base, s);
  const SelGeom g = sel_geom(d, y);
  const int32_t* counts_in = nullptr;
  if (d.tau > 0.f) {
    int32_t* out = budgets ? budgets : reinterpret_cast<int32_t*>(base + y.budgets);
    budget_rows(d, src, out, y, base, s);
    counts_in = out;
  }
  if (d.L <= SEL_ROW_MAX_L) {
    // Short rows: the whole select in one launch, one workgroup per row.
    const int per = (d.L + SEL_THREADS - 1) / SEL_THREADS;
    if (per <= 1) sel_row_kernel<1><<<rows, SEL_THREADS, 0, s>>>(src, idx, inv, counts_in, g);
    else if (per <= 2) sel_row_kernel<2><<<rows, SEL_THREADS, 0, s>>>(src, idx, inv, counts_in, g);
    else if (per <= 4) sel_row_kernel<4><<<rows, SEL_THREADS, 0, s>>>(src, idx, inv, counts_in, g);
    else if (per <= 8) sel_row_kernel<8><<<rows, SEL_THREADS, 0, s>>>(src, idx, inv, counts_in, g);
    else sel_row_kernel<16><<<rows, SEL_THREADS, 0, s>>>(src, idx, inv, counts_in, g);
    return hipGetLastError();
  }
  uint32_t* state = reinterpret_cast<uint32_t*>(base + y.state);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + y.hist);
  uint32_t* counts = reinterpret_cast<uint32_t*>(base + y.counts);
  sel_init_kernel<<<rows, SEL_WG, 0, s>>>(state, hist, counts_in, g);
  for (int pass = 0; pass < 3; ++pass) {
    sel_hist_kernel<<<dim3(y.S, rows), SEL_WG, 0, s>>>(src, state, hist, g, pass);
    sel_find_kernel<<<rows, SEL_THREADS, 0, s>>>(state, hist, pass);
  }
  sel_count_kernel<<<dim3(y.S, rows), SEL_WG, 0, s>>>(src, state, counts, g);
  sel_write_kernel<<<dim3(y.S, rows), SEL_WG, 0, s>>>(src, state, counts, idx, inv, counts_in, g);
  return hipGetLastError();
}

}  // namespace tsa
