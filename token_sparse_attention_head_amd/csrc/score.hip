// Per-head token scoring on MFMA.
//
// The skill page "Token Sparse Attention Long Context", Step 1, scores a key by the
// softmax(q k^T / sqrt(d)) weight it receives, summed over queries; the paper page
// "Token Sparse Attention: Efficient Long-Context Inference with Interleaved Token
// Selection" asks for a lightweight score (TL;DR, Abstract).  This library restricts
// the sum to the last W' = min(W, L) query rows of each query head, with the causal
// mask, so scoring costs O(W' L d) instead of O(L^2 d):
//
//   s[b,h,j] = sum_{i in [L-W', L), i >= j} exp(z_ij - m_i) / l_i,
//   z_ij = scale <q_i, k_j>,  m_i = max_{j<=i} z_ij,  l_i = sum_{j<=i} exp(z_ij - m_i).
//
// Pass 1 (one wave per (b, h, key chunk)): z on MFMA with keys as rows and window
// queries as columns, so each lane owns one query and a running (max, sum) over its
// keys.  A merge kernel folds the chunks into (m_i, 1/l_i).  Pass 2 recomputes z with
// window queries as rows and keys as columns, so each lane owns one key and sums its
// probabilities over the window rows in a fixed order (the same order for every key,
// so equal inputs give bit-equal scores).  Probabilities and sums stay fp32.
//
// bf16: a workgroup is four query heads of one KV group (one wave each) on one key
// chunk.  64-key tiles of the shared K rows are loaded once per workgroup (each lane a few
// 16-byte chunks, two tiles in flight in registers) into padded LDS rows, and every wave
// reads its MFMA operands from there, so the K bytes cross HBM once and enough of them are
// in flight to hide its latency.  fp32: every wave reads its operands straight from global
// memory (a lane reads one contiguous half of a head-dim row).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tsa {

namespace {

constexpr float NEG_BIG = -3.0e38f;

struct ScoreGeom {
  int B, H, G, Hkv, L, Wp, chunk, nchunk;
  int64_t q_row, k_row;  // element strides between consecutive positions
};

// Wave unit -> (b, h, chunk); heads of one KV group are consecutive units.
__device__ __forceinline__ bool unit_of(const ScoreGeom& g, int unit, int& b, int& h, int& ch) {
  const int hh = unit % g.G;
  int rest = unit / g.G;
  ch = rest % g.nchunk;
  rest /= g.nchunk;
  if (rest >= g.B * g.Hkv) return false;
  const int kvh = rest % g.Hkv;
  b = rest / g.Hkv;
  h = kvh * g.G + hh;
  return true;
}

template <typename T, int D, int RB>
__device__ __forceinline__ void load_window_q(const T* q, const ScoreGeom& g, int b, int h, int lane,
                                              HalfRow<T, D> (&qf)[RB]) {
  const int hf = lane >> 5;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rb * 32 + (lane & 31);
    if (row < g.Wp) {
      const int64_t i = g.L - g.Wp + row;
      qf[rb].load(q + ((int64_t)b * g.L + i) * g.q_row + (int64_t)h * D + hf * (D / 2));
    } else {
      qf[rb].zero();
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void load_key(const T* k, const ScoreGeom& g, int b, int kvh, int j, int lane,
                                         HalfRow<T, D>& kf) {
  if (j < g.L)
    kf.load(k + ((int64_t)b * g.L + j) * g.k_row + (int64_t)kvh * D + (lane >> 5) * (D / 2));
  else
    kf.zero();
}

template <typename T, int D, int RB>
__global__ __launch_bounds__(256) void score_pass1_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          float2* __restrict__ part, ScoreGeom g, float c) {
  const int lane = lane_id();
  const int hf = lane >> 5;
  int b, h, ch;
  if (!unit_of(g, blockIdx.x * 4 + threadIdx.x / TSA_WAVE, b, h, ch)) return;
  const int kvh = h / g.G;

  HalfRow<T, D> qf[RB];
  load_window_q<T, D, RB>(q, g, b, h, lane, qf);

  float m[RB], s[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) { m[rb] = NEG_BIG; s[rb] = 0.f; }

  const int j_beg = ch * g.chunk;
  const int j_end = min(g.L, j_beg + g.chunk);
  const int first_row_pos = g.L - g.Wp;
  HalfRow<T, D> kf, kn;                        // current and prefetched key tile
  load_key<T, D>(k, g, b, kvh, j_beg + (lane & 31), lane, kf);
  for (int j0 = j_beg; j0 < j_end; j0 += 32) {
    if (j0 + 32 < j_end) load_key<T, D>(k, g, b, kvh, j0 + 32 + (lane & 31), lane, kn);
    const bool need_mask = j0 + 31 > first_row_pos;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x16 acc = {};
      acc = dot_tile<T, D>(acc, kf, qf[rb]);     // rows: keys, columns: window queries
      const int i = first_row_pos + rb * 32 + (lane & 31);
      float tmax = -__builtin_huge_valf();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + acc_row(r, hf);
        if (need_mask && j > i) acc[r] = -__builtin_huge_valf();   // masked: contributes exp2(-inf) = 0
        tmax = fmaxf(tmax, acc[r]);
      }
      // m stays finite (starts at NEG_BIG), so a fully masked tile leaves (m, s) unchanged.
      const float mn = fmaxf(m[rb], tmax * c);
      float add = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) add += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], c, -mn));
      s[rb] = s[rb] * __builtin_amdgcn_exp2f(m[rb] - mn) + add;
      m[rb] = mn;
    }
    kf = kn;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float mo = xor32(m[rb]);
    const float so = xor32(s[rb]);
    const float M = fmaxf(m[rb], mo);
    const float S = s[rb] * __builtin_amdgcn_exp2f(m[rb] - M) + so * __builtin_amdgcn_exp2f(mo - M);
    const int row = rb * 32 + (lane & 31);
    if (hf == 0 && row < g.Wp)
      part[(((int64_t)b * g.H + h) * g.nchunk + ch) * g.Wp + row] = make_float2(M, S);
  }
}

// Folds the per-chunk (max, sum) of every window row into (m_i, 1 / l_i).  Four threads
// per row each fold a strided quarter of the chunks, then the first folds the four
// partials; the order is fixed, so the result is deterministic.
constexpr int MERGE_PARTS = 4;
__global__ __launch_bounds__(64 * MERGE_PARTS) void score_merge_kernel(const float2* __restrict__ part,
                                                                       float2* __restrict__ stat, int nchunk,
                                                                       int Wp) {
  __shared__ float2 partial[MERGE_PARTS][64];
  const int bh = blockIdx.x;
  const int row = threadIdx.x % 64;
  const int q = threadIdx.x / 64;
  const float2* p = part + (int64_t)bh * nchunk * Wp + row;
  float M = NEG_BIG, S = 0.f;
  if (row < Wp) {
    for (int c = q; c < nchunk; c += MERGE_PARTS) M = fmaxf(M, p[(int64_t)c * Wp].x);
    for (int c = q; c < nchunk; c += MERGE_PARTS) {
      const float2 v = p[(int64_t)c * Wp];
      S += v.y * __builtin_amdgcn_exp2f(v.x - M);
    }
  }
  partial[q][row] = make_float2(M, S);
  __syncthreads();
  if (q == 0 && row < Wp) {
    float Mt = NEG_BIG;
    for (int i = 0; i < MERGE_PARTS; ++i) Mt = fmaxf(Mt, partial[i][row].x);
    float St = 0.f;
    for (int i = 0; i < MERGE_PARTS; ++i) St += partial[i][row].y * __builtin_amdgcn_exp2f(partial[i][row].x - Mt);
    stat[(int64_t)bh * Wp + row] = make_float2(Mt, 1.0f / St);
  }
}

template <typename T, int D, int RB>
__global__ __launch_bounds__(256) void score_pass2_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const float2* __restrict__ stat, float* __restrict__ scores,
                                                          ScoreGeom g, float c) {
  const int lane = lane_id();
  const int hf = lane >> 5;
  int b, h, ch;
  if (!unit_of(g, blockIdx.x * 4 + threadIdx.x / TSA_WAVE, b, h, ch)) return;
  const int kvh = h / g.G;

  HalfRow<T, D> qf[RB];
  load_window_q<T, D, RB>(q, g, b, h, lane, qf);

  // Row statistics of the 16 window rows this lane holds in each 32-row block.
  float mrow[RB][16], il[RB][16];
  const float2* st = stat + ((int64_t)b * g.H + h) * g.Wp;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rb * 32 + acc_row(r, hf);
      if (row < g.Wp) {
        const float2 v = st[row];
        mrow[rb][r] = v.x;
        il[rb][r] = v.y;
      } else {
        mrow[rb][r] = __builtin_huge_valf();   // exp2(z - inf) = 0
        il[rb][r] = 0.f;
      }
    }

  const int j_beg = ch * g.chunk;
  const int j_end = min(g.L, j_beg + g.chunk);
  const int first_row_pos = g.L - g.Wp;
  float* out = scores + ((int64_t)b * g.H + h) * g.L;
  HalfRow<T, D> kf, kn;                        // current and prefetched key tile
  load_key<T, D>(k, g, b, kvh, j_beg + (lane & 31), lane, kf);
  for (int j0 = j_beg; j0 < j_end; j0 += 32) {
    const int j = j0 + (lane & 31);
    if (j0 + 32 < j_end) load_key<T, D>(k, g, b, kvh, j + 32, lane, kn);
    const bool need_mask = j0 + 31 > first_row_pos;
    float col = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x16 acc = {};
      acc = dot_tile<T, D>(acc, qf[rb], kf);     // rows: window queries, columns: keys
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = first_row_pos + rb * 32 + acc_row(r, hf);
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], c, -mrow[rb][r])) * il[rb][r];
        if (need_mask && j > i) p = 0.f;
        col += p;
      }
    }
    col += xor32(col);
    if (hf == 0 && j < g.L) out[j] = col;
    kf = kn;
  }
}

// ---- bf16 kernels with the K tile staged once per workgroup ------------------------------

constexpr int SBN = 64;       // keys per staged tile
constexpr int SPF = 2;        // tiles in flight in registers

// Cooperative staging of 64-key K tiles of one (b, KV head) into padded LDS rows
// (2D + 16 bytes apart: the 16-byte operand reads of 16 consecutive keys hit every bank once).
template <int D>
struct KStage {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int LPT = SBN * CPR / 256;        // chunks per thread per tile
  static constexpr int KP = 2 * D + 16;
  const char* base;          // K row of position 0 for this (b, KV head), bytes
  int64_t row_bytes;         // bytes between positions
  int L, lrow[LPT], lch[LPT], soff[LPT];
  u32x4 st[SPF][LPT];
  __device__ __forceinline__ void init(const __bf16* k, const ScoreGeom& g, int b, int kvh) {
    base = reinterpret_cast<const char*>(k + ((int64_t)b * g.L * g.Hkv + kvh) * D);
    row_bytes = (int64_t)g.Hkv * D * 2;
    L = g.L;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = threadIdx.x + 256 * i;
      lrow[i] = e / CPR;
      lch[i] = e % CPR;
      soff[i] = lrow[i] * KP + lch[i] * 16;
    }
  }
  // Rows past the sequence repeat its last row (their keys are masked by the callers).
  __device__ __forceinline__ void load(int set, int j0) {
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      st[set][i] = ld16(base + (int64_t)min(j0 + lrow[i], L - 1) * row_bytes + lch[i] * 16);
  }
  __device__ __forceinline__ void store(int set, char* lds) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) *reinterpret_cast<u32x4*>(lds + soff[i]) = st[set][i];
  }
};

// The K operand of one 32-key block for this lane (key kb * 32 + lane % 32, d half lane / 32).
template <int D>
__device__ __forceinline__ void lds_key(const char* tile, int kb, int lane, HalfRow<__bf16, D>& kf) {
  const char* a = tile + (kb * 32 + (lane & 31)) * KStage<D>::KP + (lane >> 5) * D;
#pragma unroll
  for (int s2 = 0; s2 < D / 16; ++s2) kf.f[s2] = *reinterpret_cast<const bf16x8*>(a + s2 * 16);
}

// Workgroup unit -> (b, KV head, head quad, chunk); wave w takes query head kvh*G + 4*quad + w.
__device__ __forceinline__ void unit_of4(const ScoreGeom& g, int& b, int& kvh, int& quad, int& ch) {
  const int nq = (g.G + 3) / 4;
  int u = blockIdx.x;
  ch = u % g.nchunk;
  u /= g.nchunk;
  quad = u % nq;
  u /= nq;
  kvh = u % g.Hkv;
  b = u / g.Hkv;
}

template <int D, int RB>
__global__ __launch_bounds__(256) void score_pass1_lds_kernel(const __bf16* __restrict__ q,
                                                              const __bf16* __restrict__ k,
                                                              float2* __restrict__ part, ScoreGeom g, float c) {
  __shared__ __attribute__((aligned(16))) char lds[2][SBN * KStage<D>::KP];
  const int lane = lane_id(), wave = threadIdx.x / TSA_WAVE;
  const int hf = lane >> 5;
  int b, kvh, quad, ch;
  unit_of4(g, b, kvh, quad, ch);
  const int hg = 4 * quad + wave;                    // head within the group
  const bool active = hg < g.G;
  const int h = kvh * g.G + (active ? hg : 0);
  HalfRow<__bf16, D> qf[RB];
  load_window_q<__bf16, D, RB>(q, g, b, h, lane, qf);
  float m[RB], sacc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) { m[rb] = NEG_BIG; sacc[rb] = 0.f; }

  const int j_beg = ch * g.chunk;
  const int j_end = min(g.L, j_beg + g.chunk);
  const int nt = (j_end - j_beg + SBN - 1) / SBN;
  const int first_row_pos = g.L - g.Wp;
  KStage<D> ks;
  ks.init(k, g, b, kvh);
  ks.load(0, j_beg);
  ks.load(1, j_beg + SBN);
  auto step = [&](int t, char* tile, int set) __attribute__((always_inline)) {
    ks.store(set, tile);
    __syncthreads();
    ks.load(set, j_beg + (t + SPF) * SBN);
    const int j0t = j_beg + t * SBN;
    if (!active || t >= nt) return;
#pragma unroll
    for (int kb = 0; kb < SBN / 32; ++kb) {
      // Chunks are whole tiles except the last, which ends at L: keys at or past L come
      // after every window row, so the causal mask also removes the ragged tail.
      const int j0 = j0t + kb * 32;
      __builtin_amdgcn_sched_barrier(0);
      HalfRow<__bf16, D> kf;
      lds_key<D>(tile, kb, lane, kf);
      // The causal mask only touches the blocks that reach the window rows: those take a
      // separate copy of the code so the others run without per-element selects.
      auto rows = [&](auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          f32x16 acc = {};
          acc = dot_tile<__bf16, D>(acc, kf, qf[rb]);   // rows: keys, columns: window queries
          const int i = first_row_pos + rb * 32 + (lane & 31);
          float tmax = -__builtin_huge_valf();
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (MASK && j0 + acc_row(r, hf) > i) acc[r] = -__builtin_huge_valf();
            tmax = fmaxf(tmax, acc[r]);
          }
          const float mn = fmaxf(m[rb], tmax * c);
          float add = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) add += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], c, -mn));
          sacc[rb] = sacc[rb] * __builtin_amdgcn_exp2f(m[rb] - mn) + add;
          m[rb] = mn;
        }
      };
      if (j0 + 31 > first_row_pos) rows(std::true_type{});
      else rows(std::false_type{});
    }
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, lds[0], 0);
    step(t + 1, lds[1], 1);
  }
  if (!active) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float mo = xor32(m[rb]);
    const float so = xor32(sacc[rb]);
    const float M = fmaxf(m[rb], mo);
    const float S = sacc[rb] * __builtin_amdgcn_exp2f(m[rb] - M) + so * __builtin_amdgcn_exp2f(mo - M);
    const int row = rb * 32 + (lane & 31);
    if (hf == 0 && row < g.Wp)
      part[(((int64_t)b * g.H + h) * g.nchunk + ch) * g.Wp + row] = make_float2(M, S);
  }
}

template <int D, int RB>
__global__ __launch_bounds__(256, 2) void score_pass2_lds_kernel(const __bf16* __restrict__ q,
                                                              const __bf16* __restrict__ k,
                                                              const float2* __restrict__ stat,
                                                              float* __restrict__ scores, ScoreGeom g, float c) {
  __shared__ __attribute__((aligned(16))) char lds[2][SBN * KStage<D>::KP];
  const int lane = lane_id(), wave = threadIdx.x / TSA_WAVE;
  const int hf = lane >> 5;
  int b, kvh, quad, ch;
  unit_of4(g, b, kvh, quad, ch);
  const int hg = 4 * quad + wave;
  const bool active = hg < g.G;
  const int h = kvh * g.G + (active ? hg : 0);
  HalfRow<__bf16, D> qf[RB];
  load_window_q<__bf16, D, RB>(q, g, b, h, lane, qf);
  float mrow[RB][16], il[RB][16];
  const float2* st = stat + ((int64_t)b * g.H + h) * g.Wp;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rb * 32 + acc_row(r, hf);
      if (row < g.Wp) {
        const float2 v = st[row];
        mrow[rb][r] = v.x;
        il[rb][r] = v.y;
      } else {
        mrow[rb][r] = __builtin_huge_valf();   // exp2(z - inf) = 0
        il[rb][r] = 0.f;
      }
    }

  const int j_beg = ch * g.chunk;
  const int j_end = min(g.L, j_beg + g.chunk);
  const int nt = (j_end - j_beg + SBN - 1) / SBN;
  const int first_row_pos = g.L - g.Wp;
  float* out = scores + ((int64_t)b * g.H + h) * g.L;
  KStage<D> ks;
  ks.init(k, g, b, kvh);
  ks.load(0, j_beg);
  ks.load(1, j_beg + SBN);
  auto step = [&](int t, char* tile, int set) __attribute__((always_inline)) {
    ks.store(set, tile);
    __syncthreads();
    ks.load(set, j_beg + (t + SPF) * SBN);
    const int j0t = j_beg + t * SBN;
    if (!active || t >= nt) return;
#pragma unroll
    for (int kb = 0; kb < SBN / 32; ++kb) {
      const int j0 = j0t + kb * 32;
      __builtin_amdgcn_sched_barrier(0);
      HalfRow<__bf16, D> kf;
      lds_key<D>(tile, kb, lane, kf);
      const int j = j0 + (lane & 31);
      auto cols = [&](auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        float col = 0.f;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          f32x16 acc = {};
          acc = dot_tile<__bf16, D>(acc, qf[rb], kf);   // rows: window queries, columns: keys
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], c, -mrow[rb][r])) * il[rb][r];
            if (MASK && j > first_row_pos + rb * 32 + acc_row(r, hf)) p = 0.f;
            col += p;
          }
        }
        return col;
      };
      float col = j0 + 31 > first_row_pos ? cols(std::true_type{}) : cols(std::false_type{});
      col += xor32(col);
      if (hf == 0 && j < j_end) out[j] = col;
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, lds[0], 0);
    step(t + 1, lds[1], 1);
  }
}

template <typename T, int D>
hipError_t launch_score_t(const tsa_desc& d, const void* q, const void* k, float* scores, float2* part,
                          float2* stat, hipStream_t s) {
  ScoreGeom g;
  g.B = d.B; g.H = d.H; g.Hkv = d.Hkv; g.G = d.H / d.Hkv; g.L = d.L;
  g.Wp = d.W < d.L ? d.W : d.L;
  score_chunking(d, g.chunk, g.nchunk);
  g.q_row = (int64_t)d.H * D;
  g.k_row = (int64_t)d.Hkv * D;
  const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)D);
  const float c = scale * TSA_LOG2E;
  if constexpr (sizeof(T) == 2) {
    const unsigned blocks = (unsigned)(d.B * d.Hkv * ((g.G + 3) / 4) * g.nchunk);
    if (g.Wp > 32)
      score_pass1_lds_kernel<D, 2><<<blocks, 256, 0, s>>>((const __bf16*)q, (const __bf16*)k, part, g, c);
    else
      score_pass1_lds_kernel<D, 1><<<blocks, 256, 0, s>>>((const __bf16*)q, (const __bf16*)k, part, g, c);
    score_merge_kernel<<<d.B * d.H, 64 * MERGE_PARTS, 0, s>>>(part, stat, g.nchunk, g.Wp);
    if (g.Wp > 32)
      score_pass2_lds_kernel<D, 2><<<blocks, 256, 0, s>>>((const __bf16*)q, (const __bf16*)k, stat, scores, g, c);
    else
      score_pass2_lds_kernel<D, 1><<<blocks, 256, 0, s>>>((const __bf16*)q, (const __bf16*)k, stat, scores, g, c);
    return hipGetLastError();
  }
  const int units = d.B * d.H * g.nchunk;
  const unsigned blocks = (unsigned)((units + 3) / 4);
  if (g.Wp > 32) {
    score_pass1_kernel<T, D, 2><<<blocks, 256, 0, s>>>((const T*)q, (const T*)k, part, g, c);
  } else {
    score_pass1_kernel<T, D, 1><<<blocks, 256, 0, s>>>((const T*)q, (const T*)k, part, g, c);
  }
  score_merge_kernel<<<d.B * d.H, 64 * MERGE_PARTS, 0, s>>>(part, stat, g.nchunk, g.Wp);
  if (g.Wp > 32) {
    score_pass2_kernel<T, D, 2><<<blocks, 256, 0, s>>>((const T*)q, (const T*)k, stat, scores, g, c);
  } else {
    score_pass2_kernel<T, D, 1><<<blocks, 256, 0, s>>>((const T*)q, (const T*)k, stat, scores, g, c);
  }
  return hipGetLastError();
}

}  // namespace

void score_chunking(const tsa_desc& d, int& chunk, int& nchunk) {
  if (d.dtype == TSA_BF16) {
    // About 512 workgroups (four query heads of one KV group each), 64-key tiles.
    const int64_t groups = (int64_t)d.B * d.Hkv * ((d.H / d.Hkv + 3) / 4);
    const int64_t want = std::max<int64_t>(1, (512 + groups - 1) / groups);
    int64_t ck = ((d.L + want - 1) / want + 63) / 64 * 64;
    if (ck < 64) ck = 64;
    chunk = (int)ck;
    nchunk = (int)((d.L + ck - 1) / ck);
    return;
  }
  // About 4096 waves in flight over the whole problem, at least 32 keys per wave.
  const int64_t keys_per_wave = ((int64_t)d.B * d.H * d.L + 4095) / 4096;
  int64_t ck = (keys_per_wave + 31) / 32 * 32;
  if (ck < 32) ck = 32;
  if (ck > d.L) ck = (d.L + 31) / 32 * 32;
  chunk = (int)ck;
  nchunk = (int)((d.L + ck - 1) / ck);
}

hipError_t launch_score(const tsa_desc& d, const void* q, const void* k, float* scores, float2* part, float2* stat,
                        hipStream_t s) {
  if (d.dtype == TSA_BF16) {
    if (d.d == 128) return launch_score_t<__bf16, 128>(d, q, k, scores, part, stat, s);
    if (d.d == 64) return launch_score_t<__bf16, 64>(d, q, k, scores, part, stat, s);
  } else {
    if (d.d == 128) return launch_score_t<float, 128>(d, q, k, scores, part, stat, s);
    if (d.d == 64) return launch_score_t<float, 64>(d, q, k, scores, part, stat, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tsa
