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
// One 1024-thread workgroup per (b, subset) row.  Scores are >= 0, so their fp32 bit
// patterns order like the values.  The threshold T (the score of the last candidate
// taken) is found by a three-pass radix select (11 + 11 + 10 bits) with LDS
// histograms; then every wave compacts a contiguous segment of the row with wave
// ballots and mbcnt prefix counts, ties at T going to the lowest positions.
#include "common.h"
#include "kernels.h"

namespace tsa {

namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / TSA_WAVE;
constexpr int SEL_MAX_BINS = 2048;
constexpr int SEL_UNROLL = 8;      // loads in flight per thread in the streaming passes

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

__global__ __launch_bounds__(SEL_THREADS) void select_kernel(const float* __restrict__ scores,
                                                             int32_t* __restrict__ idx, int32_t* __restrict__ inv,
                                                             int L, int keep, int c0, int c1) {
  // Candidates are the positions [c0, c1); [0, c0) and [c1, L) are forced.
  __shared__ uint32_t hist[SEL_MAX_BINS];
  __shared__ uint32_t wave_tot[SEL_WAVES];
  __shared__ uint32_t found_bin, found_above;
  __shared__ uint32_t seg_strict[SEL_WAVES], seg_eq[SEL_WAVES];
  __shared__ uint32_t seg_out[SEL_WAVES], seg_eq_before[SEL_WAVES];

  const int bh = blockIdx.x;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(scores + (int64_t)bh * L);
  const int tid = threadIdx.x;
  const int n_cand = c1 - c0;
  const int n_forced = L - n_cand;
  uint32_t need = (uint32_t)(keep - n_forced);   // candidates still to take
  const bool take_all = (int)need >= n_cand;
  const bool take_none = need == 0;

  uint32_t T = 0xFFFFFFFFu;   // threshold key
  uint32_t need_eq = 0;       // how many candidates equal to T are taken (lowest positions first)
  if (!take_all && !take_none) {
    uint32_t prefix = 0, pmask = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nb = pass == 2 ? 1024 : 2048;
      for (int i = tid; i < nb; i += SEL_THREADS) hist[i] = 0;
      __syncthreads();
      // SEL_UNROLL loads in flight per thread before any of them is used.
      for (int j0 = c0 + tid; j0 < c1; j0 += SEL_UNROLL * SEL_THREADS) {
        uint32_t u[SEL_UNROLL];
#pragma unroll
        for (int k = 0; k < SEL_UNROLL; ++k) {
          const int j = j0 + k * SEL_THREADS;
          u[k] = j < c1 ? key[j] : 0u;
        }
#pragma unroll
        for (int k = 0; k < SEL_UNROLL; ++k) {
          const int j = j0 + k * SEL_THREADS;
          if (j < c1 && (u[k] & pmask) == prefix) atomicAdd(&hist[(u[k] >> shift) & (nb - 1)], 1u);
        }
      }
      __syncthreads();
      // Bins in descending order; thread t owns ranks [t*per, (t+1)*per).
      const int per = nb / SEL_THREADS;
      uint32_t local = 0;
      for (int q = 0; q < per; ++q) local += hist[nb - 1 - (tid * per + q)];
      const uint32_t incl = block_inclusive_scan(local, wave_tot);
      const uint32_t excl = incl - local;
      if (excl < need && need <= incl) {
        uint32_t cum = excl;
        for (int q = 0; q < per; ++q) {
          const int bin = nb - 1 - (tid * per + q);
          if (cum + hist[bin] >= need) {
            found_bin = bin;
            found_above = cum;
            break;
          }
          cum += hist[bin];
        }
      }
      __syncthreads();
      need -= found_above;
      prefix |= found_bin << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      __syncthreads();
    }
    T = prefix;
    need_eq = need;
  }

  // Compaction: wave w owns positions [w*seg, (w+1)*seg).
  const int lane = lane_id();
  const int wave = tid / TSA_WAVE;
  const int seg = ((L + SEL_WAVES - 1) / SEL_WAVES + TSA_WAVE - 1) / TSA_WAVE * TSA_WAVE;
  const int beg = wave * seg;
  const int end = min(L, beg + seg);

  auto load_key = [&](int j) -> uint32_t { return (j < end && j >= c0 && j < c1) ? key[j] : 0u; };
  auto classify = [&](int j, uint32_t u, bool& strict, bool& eq) {
    const bool valid = j < end;
    const bool cand = valid && j >= c0 && j < c1;
    strict = (valid && !cand) || (cand && (take_all || (!take_none && u > T)));
    eq = cand && !take_all && !take_none && u == T;
  };

  uint32_t n_strict = 0, n_eq = 0;
  for (int base = beg; base < end; base += SEL_UNROLL * TSA_WAVE) {
    uint32_t u[SEL_UNROLL];
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) u[k] = load_key(base + k * TSA_WAVE + lane);
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      bool s, e;
      classify(base + k * TSA_WAVE + lane, u[k], s, e);
      n_strict += __popcll(__ballot(s));
      n_eq += __popcll(__ballot(e));
    }
  }
  if (lane == 0) {
    seg_strict[wave] = n_strict;
    seg_eq[wave] = n_eq;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t eq_before = 0, out = 0;
    for (int w = 0; w < SEL_WAVES; ++w) {
      const uint32_t rem = need_eq > eq_before ? need_eq - eq_before : 0;
      const uint32_t take_eq = min(rem, seg_eq[w]);
      seg_eq_before[w] = eq_before;
      seg_out[w] = out;
      out += seg_strict[w] + take_eq;
      eq_before += seg_eq[w];
    }
  }
  __syncthreads();

  int32_t* row_idx = idx + (int64_t)bh * keep;
  int32_t* row_inv = inv ? inv + (int64_t)bh * L : nullptr;
  uint32_t pos = seg_out[wave];
  uint32_t eq_rank = seg_eq_before[wave];
  for (int base = beg; base < end; base += SEL_UNROLL * TSA_WAVE) {
    uint32_t u[SEL_UNROLL];
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) u[k] = load_key(base + k * TSA_WAVE + lane);
#pragma unroll
    for (int k = 0; k < SEL_UNROLL; ++k) {
      const int j = base + k * TSA_WAVE + lane;
      bool s, e;
      classify(j, u[k], s, e);
      const uint64_t emask = __ballot(e);
      const uint32_t my_eq = eq_rank + __builtin_amdgcn_mbcnt_hi((uint32_t)(emask >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)emask, 0u));
      const bool take = s || (e && my_eq < need_eq);
      const uint64_t tmask = __ballot(take);
      const uint32_t my_pos = pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(tmask >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)tmask, 0u));
      if (take && my_pos < (uint32_t)keep) row_idx[my_pos] = j;
      if (row_inv && j < end) row_inv[j] = (take && my_pos < (uint32_t)keep) ? (int32_t)my_pos : -1;
      pos += __popcll(tmask);
      eq_rank += __popcll(emask);
    }
  }
}

}  // namespace

hipError_t launch_select(const tsa_desc& d, const float* scores, int32_t* idx, int32_t* inv, float* gsum,
                         hipStream_t s) {
  const int Wp = d.W < d.L ? d.W : d.L;
  const int c1 = d.L - Wp;
  const int c0 = d.n_sink < c1 ? d.n_sink : c1;
  const int R = subset_rows(d), G = heads_per_subset(d);
  const float* rows = scores;
  if (G > 1) {
    const int64_t n = (int64_t)d.B * R * d.L;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
    group_sum_kernel<<<blocks, 256, 0, s>>>(scores, gsum, G, d.L, n);
    rows = gsum;
  }
  select_kernel<<<d.B * R, SEL_THREADS, 0, s>>>(rows, idx, inv, d.L, d.keep, c0, c1);
  return hipGetLastError();
}

}  // namespace tsa
