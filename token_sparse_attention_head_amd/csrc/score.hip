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
// Pass 1 computes z with keys as rows and window queries as columns, so each lane owns a
// query and a running sum of exp2 over its keys against a reference; a merge kernel folds the
// key chunks into (m_i, 1/l_i).  Pass 2 recomputes z with window queries as rows and keys as
// columns, so each lane owns one key and sums its probabilities over the window rows in a
// fixed order (the same order for every key, so equal inputs give bit-equal scores).
// Probabilities and sums stay fp32.
//
// bf16: a workgroup is four query heads of one KV group (one wave each) on one key chunk,
// on the 16x16x32 MFMA (details at the kernels).  64-key tiles of the shared K rows are
// loaded once per workgroup into padded LDS rows that all four waves read their operands
// from, so the K bytes cross HBM once.  fp32: every wave reads its operands straight from
// global memory (a lane reads one contiguous half of a head-dim row) on the 32x32x2 fp32
// MFMA, with an exact running max in pass 1.
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

// Folds the per-chunk (max, sum) of every window row into (m_i, 1 / l_i).  A workgroup takes
// 16 rows of one (b, h): lane r + 16 s of wave w folds the chunks c = 4 w + s (mod 16) of row r
// (the 16 rows of a chunk are adjacent in memory), then the four lanes of a row in a wave and
// the four waves are folded, always in the same order, so the result is deterministic.
constexpr int MERGE_ROWS = 16;
constexpr int MERGE_SLICES = 16;

__device__ __forceinline__ void fold_ms(float& M, float& S, float mo, float so) {
  const float mm = fmaxf(M, mo);
  S = S * __builtin_amdgcn_exp2f(M - mm) + so * __builtin_amdgcn_exp2f(mo - mm);
  M = mm;
}

__global__ __launch_bounds__(MERGE_ROWS * MERGE_SLICES) void score_merge_kernel(const float2* __restrict__ part,
                                                                               float2* __restrict__ stat,
                                                                               int nchunk, int Wp) {
  __shared__ float2 wpart[MERGE_SLICES / 4][MERGE_ROWS];
  const int groups = (Wp + MERGE_ROWS - 1) / MERGE_ROWS;
  const int bh = blockIdx.x / groups;
  const int row = (blockIdx.x % groups) * MERGE_ROWS + threadIdx.x % MERGE_ROWS;
  const int slice = threadIdx.x / MERGE_ROWS;
  const float2* p = part + (int64_t)bh * nchunk * Wp + row;
  float M = NEG_BIG, S = 0.f;
  if (row < Wp) {
    int c = slice;
    for (; c + 3 * MERGE_SLICES < nchunk; c += 4 * MERGE_SLICES) {   // four chunks in flight
      float2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = p[(int64_t)(c + u * MERGE_SLICES) * Wp];
#pragma unroll
      for (int u = 0; u < 4; ++u) fold_ms(M, S, v[u].x, v[u].y);
    }
    for (; c < nchunk; c += MERGE_SLICES) {
      const float2 v = p[(int64_t)c * Wp];
      fold_ms(M, S, v.x, v.y);
    }
  }
  // The four slices of a row in this wave: lanes r, r + 16, r + 32, r + 48.
  fold_ms(M, S, __shfl_xor(M, 16, TSA_WAVE), __shfl_xor(S, 16, TSA_WAVE));
  fold_ms(M, S, __shfl_xor(M, 32, TSA_WAVE), __shfl_xor(S, 32, TSA_WAVE));
  const int wave = threadIdx.x / TSA_WAVE, lane = threadIdx.x % TSA_WAVE;
  if (lane < MERGE_ROWS) wpart[wave][lane] = make_float2(M, S);
  __syncthreads();
  if (wave == 0 && lane < MERGE_ROWS && row < Wp) {
    float Mt = wpart[0][lane].x, St = wpart[0][lane].y;
#pragma unroll
    for (int w = 1; w < MERGE_SLICES / 4; ++w) fold_ms(Mt, St, wpart[w][lane].x, wpart[w][lane].y);
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
constexpr int SCORE_BUF_FLAGS = 0x00020000;   // buffer resource word 3: 32-bit data format, raw access
constexpr int SPF = 2;        // tiles in flight in registers

// Cooperative staging of the 64-key K tiles of one (b, KV head) chunk into padded LDS rows
// KP_ bytes apart, NSETS tiles in flight in registers.  The rows come through a buffer view
// of the chunk: a lane's byte offset within a tile is fixed, a tile adds a wave-uniform
// offset, and rows past the sequence fall outside the view and read as zero (their keys
// are masked by the callers).  So a load costs one add, not a 64-bit address computation.
template <int D, int KP_, int NSETS = SPF>
struct KStage {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int LPT = SBN * CPR / 256;        // chunks per thread per tile
  static constexpr int KP = KP_;
  __amdgpu_buffer_rsrc_t rows;
  uint32_t tile_bytes;       // bytes between consecutive tiles
  int last_tile;             // the chunk's last tile; prefetches past it re-read it
  uint32_t loff[LPT];
  int soff[LPT];
  u32x4 st[NSETS][LPT];
  // The chunk's rows [j_beg, j_end) of batch entry b, KV head kvh.
  __device__ __forceinline__ void init(const __bf16* k, const ScoreGeom& g, int b, int kvh, int j_beg, int j_end) {
    const uint32_t row_bytes = (uint32_t)g.Hkv * D * 2;
    // The view is wave-uniform; pinning its parts to scalar registers keeps the compiler
    // from wrapping every load in a loop over distinct views.
    const uint64_t addr = reinterpret_cast<uint64_t>(k + (((int64_t)b * g.L + j_beg) * g.Hkv + kvh) * D);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    char* base = reinterpret_cast<char*>(((uint64_t)hi << 32) | lo);
    // Up to the end of the chunk's last row's own D values.
    const uint32_t bytes = __builtin_amdgcn_readfirstlane((j_end - j_beg - 1) * row_bytes + 2 * D);
    rows = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, SCORE_BUF_FLAGS);
    tile_bytes = SBN * row_bytes;
    last_tile = (j_end - j_beg - 1) / SBN;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int lrow = e / CPR, lch = e % CPR;
      loff[i] = (uint32_t)lrow * row_bytes + lch * 16;
      soff[i] = lrow * KP + lch * 16;
    }
  }
  // Tile t of the chunk (keys j_beg + 64 t ...).
  __device__ __forceinline__ void load(int set, int t) {
    const uint32_t toff = (uint32_t)min(t, last_tile) * tile_bytes;
#pragma unroll
    for (int i = 0; i < LPT; ++i) st[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rows, loff[i] + toff, 0, 0);
  }
  __device__ __forceinline__ void store(int set, char* lds) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) *reinterpret_cast<u32x4*>(lds + soff[i]) = st[set][i];
  }
};

// Consecutive workgroups take the head quads and KV heads of one key chunk, so the
// workgroups in flight read whole K rows of consecutive positions together (a position's
// KV heads are adjacent in memory; one head's rows alone are a 2 D-byte piece of every
// Hkv * 2 D bytes).
__device__ __forceinline__ void unit_of4(const ScoreGeom& g, int& b, int& kvh, int& quad, int& ch) {
  const int nq = (g.G + 3) / 4;
  int u = blockIdx.x;
  quad = u % nq;
  u /= nq;
  kvh = u % g.Hkv;
  u /= g.Hkv;
  ch = u % g.nchunk;
  b = u / g.nchunk;
}

// ---- bf16 kernels on the 16x16x32 MFMA ------------------------------------------------
//
// v_mfma_f32_16x16x32_bf16: operand lanes l supply row (or column) l % 16 and the
// contraction slice 8 (l / 16) .. +7 of each 32-wide step; the 16x16 result gives lane l
// column l % 16 and rows 4 (l / 16) + i, i = 0..3.  The window rows form RB blocks of 16
// (block qb, row r = window row 16 qb + r).  A lane's Q fragment of block qb and step s is
// row 16 qb + l % 16 at d = 32 s + 8 (l / 16); its K fragment of a 16-key block is key
// l % 16 at the same d, read from LDS rows 2D + 32 bytes apart (the four lane groups of a
// key read its 64 contiguous bytes of the step, and the 16 keys fall on distinct banks).
// Every K fragment feeds RB independent products (one per query block), so no product
// waits for the one before it.
//
// Pass 1 forms S^T = K Q^T (lane: one query of each block, four keys of each 16-key block)
// and keeps, per lane and query, a sum of exp2 against a lazily moved reference m: the
// block's probabilities are taken against m as it is and their sum (below 2^32: nothing near
// overflow) decides whether that was safe; only otherwise (the first block, or a jump of the
// logits by 32 in log2 units) the lane's max moves m and rescales the sum.  The four lanes of
// a query are merged at the end (max, then the rescaled sums), so no row max is taken per
// element.  Pass 2 forms S = Q K^T (lane: one key, four queries of each block) and sums the
// normalised probabilities of its key over its 4 RB queries in a fixed order, then over the
// four lane groups (xor 16, then xor 32): the same order for every key.

constexpr int KP16_PAD = 32;
constexpr int SPF16 = 2;      // K tiles in flight in registers

template <int D, int RB>
__device__ __forceinline__ void load_window_q16(const __bf16* q, const ScoreGeom& g, int b, int h, int lane,
                                                bf16x8 (&qf)[RB][D / 32]) {
  const int lq = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) {
    const int row = 16 * qb + lq;
    if (row < g.Wp) {
      const __bf16* src = q + ((int64_t)b * g.L + g.L - g.Wp + row) * g.q_row + (int64_t)h * D + 8 * gq;
#pragma unroll
      for (int st = 0; st < D / 32; ++st) qf[qb][st] = *reinterpret_cast<const bf16x8*>(src + 32 * st);
    } else {
#pragma unroll
      for (int st = 0; st < D / 32; ++st) qf[qb][st] = bf16x8{};
    }
  }
}

__device__ __forceinline__ f32x4 mfma16s(f32x4 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Both passes are software-pipelined over 16-key blocks: the products of block kb are
// issued with the softmax arithmetic of block kb - 1, at a raised wave priority, so that of
// the two waves of a SIMD the one with matrix work ready issues first and the other's
// vector work fills in behind it.  Pass 1 issues the 16 products as one burst at the raised
// priority and the softmax after it; pass 2 interleaves them (one matrix instruction, then
// three vector instructions, as scheduling groups) and raises the priority over the whole
// group.  Of the four arrangements (interleaved or not, with or without the priority) these
// measured fastest: L = 131072, pass 1 79.2 -> 75.5 us, pass 2 81.6 -> 79.2 us.  The causal
// mask is evaluated only in steps whose blocks reach the window rows (a step processes
// block 3 of the previous tile and blocks 0-2 of its own).

// Sixteen groups of one matrix instruction followed by three vector instructions.
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);   // vector ALU, transcendental included
  }
}

template <int D, int RB>
__global__ __launch_bounds__(256, 2) void score_pass1_k16_kernel(const __bf16* __restrict__ q,
                                                                 const __bf16* __restrict__ k,
                                                                 float2* __restrict__ part, ScoreGeom g, float c) {
  constexpr int ST = D / 32, KP = 2 * D + KP16_PAD, NS = SPF16;
  __shared__ __attribute__((aligned(16))) char lds[2][SBN * KP];
  const int lane = lane_id(), wave = threadIdx.x / TSA_WAVE;
  const int lq = lane & 15, gq = lane >> 4;
  int b, kvh, quad, ch;
  unit_of4(g, b, kvh, quad, ch);
  const int hg = 4 * quad + wave;
  const bool active = hg < g.G;
  const int h = kvh * g.G + (active ? hg : 0);
  bf16x8 qf[RB][ST];
  load_window_q16<D, RB>(q, g, b, h, lane, qf);
  float m[RB], l[RB];
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) { m[qb] = NEG_BIG; l[qb] = 0.f; }

  const int j_beg = ch * g.chunk;
  const int j_end = min(g.L, j_beg + g.chunk);
  const int nt = (j_end - j_beg + SBN - 1) / SBN;
  const int first_row_pos = g.L - g.Wp;
  const int koff = lq * KP + 16 * gq;
  // The block in flight: its products (keys jp + 4 gq + i, query 16 qb + lq).  Before the
  // first block it holds -inf everywhere, which adds nothing.
  f32x4 pacc[RB];
  int jp = j_beg;
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) pacc[qb] = f32x4{-__builtin_huge_valf(), -__builtin_huge_valf(), -__builtin_huge_valf(), -__builtin_huge_valf()};

  // Softmax sums of the block in pacc (keys from jp) into ls; MASK applies the causal mask.
  float ls[RB];
  auto softmax_prev = [&](auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (MASK) {
#pragma unroll
      for (int qb = 0; qb < RB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (jp + 4 * gq + i > first_row_pos + 16 * qb + lq) pacc[qb][i] = -__builtin_huge_valf();
    }
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(pacc[qb][0], c, -m[qb]));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(pacc[qb][1], c, -m[qb]));
      const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(pacc[qb][2], c, -m[qb]));
      const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(pacc[qb][3], c, -m[qb]));
      ls[qb] = (e0 + e1) + (e2 + e3);
    }
  };
  // Guard of those sums (after the next block's products are issued): a sum of 2^32 or more
  // (or the first block, against the initial reference) moves the reference to the lane's
  // max and the sums are taken again; then they join the running sums.
  auto guard_prev = [&]() __attribute__((always_inline)) {
    bool unsafe = false;
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) unsafe |= !(ls[qb] < 4294967296.0f);
    if (__ballot(unsafe) != 0) {
#pragma unroll
      for (int qb = 0; qb < RB; ++qb) {
        const float tmax = fmaxf(fmaxf(pacc[qb][0], pacc[qb][1]), fmaxf(pacc[qb][2], pacc[qb][3]));
        const float mn = fmaxf(m[qb], tmax * c);   // m stays finite (starts at NEG_BIG)
        l[qb] *= __builtin_amdgcn_exp2f(m[qb] - mn);
        m[qb] = mn;
      }
      softmax_prev(std::false_type{});   // pacc is already masked
    }
#pragma unroll
    for (int qb = 0; qb < RB; ++qb) l[qb] += ls[qb];
  };

  KStage<D, KP, NS> ks;
  ks.init(k, g, b, kvh, j_beg, j_end);
  // Tiles in order (the loop waits for the oldest set only if the sets were issued in order).
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    ks.load(i, i);
    __builtin_amdgcn_sched_barrier(0);
  }
  auto step = [&](int t, char* tile, int set) __attribute__((always_inline)) {
    ks.store(set, tile);
    __syncthreads();
    ks.load(set, t + NS);
    if (!active || t >= nt) return;
    const int j0t = j_beg + t * SBN;
    auto blocks = [&](auto mask_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < SBN / 16; ++kb) {
        bf16x8 kf[ST];
#pragma unroll
        for (int st = 0; st < ST; ++st)
          kf[st] = *reinterpret_cast<const bf16x8*>(tile + 16 * kb * KP + koff + 64 * st);
        f32x4 acc[RB];
#pragma unroll
        for (int qb = 0; qb < RB; ++qb) acc[qb] = f32x4{};
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < ST; ++st)
#pragma unroll
          for (int qb = 0; qb < RB; ++qb) acc[qb] = mfma16s(acc[qb], kf[st], qf[qb][st]);   // rows: keys, cols: queries
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        softmax_prev(mask_tag);
        guard_prev();
#pragma unroll
        for (int qb = 0; qb < RB; ++qb) pacc[qb] = acc[qb];
        jp = j0t + 16 * kb;
      }
    };
    if (j0t + SBN - 17 > first_row_pos) blocks(std::true_type{});
    else blocks(std::false_type{});
  };
  for (int t = 0; t < nt; t += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) step(t + u, lds[u & 1], u);
  }
  if (!active) return;
  softmax_prev(std::true_type{});    // the last block
  guard_prev();
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) {
    float M = m[qb], S = l[qb];
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {     // merge the four lanes of the query
      const float mo = __shfl_xor(M, x, TSA_WAVE);
      const float so = __shfl_xor(S, x, TSA_WAVE);
      const float mm = fmaxf(M, mo);
      S = S * __builtin_amdgcn_exp2f(M - mm) + so * __builtin_amdgcn_exp2f(mo - mm);
      M = mm;
    }
    const int row = 16 * qb + lq;
    if (gq == 0 && row < g.Wp) part[(((int64_t)b * g.H + h) * g.nchunk + ch) * g.Wp + row] = make_float2(M, S);
  }
}

template <int D, int RB>
__global__ __launch_bounds__(256, 2) void score_pass2_k16_kernel(const __bf16* __restrict__ q,
                                                                 const __bf16* __restrict__ k,
                                                                 const float2* __restrict__ stat,
                                                                 float* __restrict__ scores, ScoreGeom g, float c) {
  constexpr int ST = D / 32, KP = 2 * D + KP16_PAD, NS = 2;
  __shared__ __attribute__((aligned(16))) char lds[2][SBN * KP];
  const int lane = lane_id(), wave = threadIdx.x / TSA_WAVE;
  const int lq = lane & 15, gq = lane >> 4;
  int b, kvh, quad, ch;
  unit_of4(g, b, kvh, quad, ch);
  const int hg = 4 * quad + wave;
  const bool active = hg < g.G;
  const int h = kvh * g.G + (active ? hg : 0);
  bf16x8 qf[RB][ST];
  load_window_q16<D, RB>(q, g, b, h, lane, qf);
  // Statistics of the four window rows this lane holds in each block (rows 16 qb + 4 gq + i).
  float mrow[RB][4], il[RB][4];
  const float2* stp = stat + ((int64_t)b * g.H + h) * g.Wp;
#pragma unroll
  for (int qb = 0; qb < RB; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * qb + 4 * gq + i;
      if (row < g.Wp) {
        const float2 v = stp[row];
        mrow[qb][i] = v.x;
        il[qb][i] = v.y;
      } else {
        mrow[qb][i] = __builtin_huge_valf();   // exp2(z - inf) = 0
        il[qb][i] = 0.f;
      }
    }

  const int j_beg = ch * g.chunk;
  const int j_end = min(g.L, j_beg + g.chunk);
  const int nt = (j_end - j_beg + SBN - 1) / SBN;
  const int first_row_pos = g.L - g.Wp;
  const int koff = lq * KP + 16 * gq;
  float* out = scores + ((int64_t)b * g.H + h) * g.L;
  // The block in flight (key jp + lq, queries 16 qb + 4 gq + i); before the first block it
  // holds zeros for a key at j_end, which is not written.
  f32x4 pacc[RB];
  int jp = j_end;
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) pacc[qb] = f32x4{};

  // Column sum of the key this lane holds in the block in pacc, over its 4 RB queries in a
  // fixed order, then over the four lane groups; returns the write of the result.
  auto colsum_prev = [&](auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int j = jp + lq;
    float col = 0.f;
#pragma unroll
    for (int qb = 0; qb < RB; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(pacc[qb][i], c, -mrow[qb][i])) * il[qb][i];
        if (MASK && j > first_row_pos + 16 * qb + 4 * gq + i) p = 0.f;
        col += p;
      }
    return [=]() __attribute__((always_inline)) {
      float cs = col;
      cs += __shfl_xor(cs, 16, TSA_WAVE);
      cs += __shfl_xor(cs, 32, TSA_WAVE);
      if (gq == 0 && j < j_end) out[j] = cs;
    };
  };

  KStage<D, KP, NS> ks;
  ks.init(k, g, b, kvh, j_beg, j_end);
  // Tiles in order (the loop waits for the oldest set only if the sets were issued in order).
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    ks.load(i, i);
    __builtin_amdgcn_sched_barrier(0);
  }
  auto step = [&](int t, char* tile, int set) __attribute__((always_inline)) {
    ks.store(set, tile);
    __syncthreads();
    ks.load(set, t + NS);
    if (!active || t >= nt) return;
    const int j0t = j_beg + t * SBN;
    auto blocks = [&](auto mask_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < SBN / 16; ++kb) {
        bf16x8 kf[ST];
#pragma unroll
        for (int st = 0; st < ST; ++st)
          kf[st] = *reinterpret_cast<const bf16x8*>(tile + 16 * kb * KP + koff + 64 * st);
        f32x4 acc[RB];
#pragma unroll
        for (int qb = 0; qb < RB; ++qb) acc[qb] = f32x4{};
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < ST; ++st)
#pragma unroll
          for (int qb = 0; qb < RB; ++qb) acc[qb] = mfma16s(acc[qb], qf[qb][st], kf[st]);   // rows: queries, cols: keys
        auto finish = colsum_prev(mask_tag);
        interleave_mfma_valu();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        finish();
#pragma unroll
        for (int qb = 0; qb < RB; ++qb) pacc[qb] = acc[qb];
        jp = j0t + 16 * kb;
      }
    };
    if (j0t + SBN - 17 > first_row_pos) blocks(std::true_type{});
    else blocks(std::false_type{});
  };
  for (int t = 0; t < nt; t += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) step(t + u, lds[u & 1], u);
  }
  if (!active) return;
  colsum_prev(std::true_type{})();    // the last block
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
    const __bf16* qb = static_cast<const __bf16*>(q);
    const __bf16* kb = static_cast<const __bf16*>(k);
    // RB = 16-row blocks of window queries (W' <= 64).
    switch ((g.Wp + 15) / 16) {
      case 1: score_pass1_k16_kernel<D, 1><<<blocks, 256, 0, s>>>(qb, kb, part, g, c); break;
      case 2: score_pass1_k16_kernel<D, 2><<<blocks, 256, 0, s>>>(qb, kb, part, g, c); break;
      case 3: score_pass1_k16_kernel<D, 3><<<blocks, 256, 0, s>>>(qb, kb, part, g, c); break;
      default: score_pass1_k16_kernel<D, 4><<<blocks, 256, 0, s>>>(qb, kb, part, g, c); break;
    }
    score_merge_kernel<<<d.B * d.H * ((g.Wp + MERGE_ROWS - 1) / MERGE_ROWS), MERGE_ROWS * MERGE_SLICES, 0, s>>>(
        part, stat, g.nchunk, g.Wp);
    switch ((g.Wp + 15) / 16) {
      case 1: score_pass2_k16_kernel<D, 1><<<blocks, 256, 0, s>>>(qb, kb, stat, scores, g, c); break;
      case 2: score_pass2_k16_kernel<D, 2><<<blocks, 256, 0, s>>>(qb, kb, stat, scores, g, c); break;
      case 3: score_pass2_k16_kernel<D, 3><<<blocks, 256, 0, s>>>(qb, kb, stat, scores, g, c); break;
      default: score_pass2_k16_kernel<D, 4><<<blocks, 256, 0, s>>>(qb, kb, stat, scores, g, c); break;
    }
    return hipGetLastError();
  }
  const int units = d.B * d.H * g.nchunk;
  const unsigned blocks = (unsigned)((units + 3) / 4);
  if (g.Wp > 32) {
    score_pass1_kernel<T, D, 2><<<blocks, 256, 0, s>>>((const T*)q, (const T*)k, part, g, c);
  } else {
    score_pass1_kernel<T, D, 1><<<blocks, 256, 0, s>>>((const T*)q, (const T*)k, part, g, c);
  }
  score_merge_kernel<<<d.B * d.H * ((g.Wp + MERGE_ROWS - 1) / MERGE_ROWS), MERGE_ROWS * MERGE_SLICES, 0, s>>>(
        part, stat, g.nchunk, g.Wp);
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
    // About 512 workgroups (four query heads of one KV group each), 64-key tiles, at least
    // 256 keys per workgroup: every workgroup first loads its four heads' window queries
    // (64 KB), so short chunks pay mostly for that (L = 8192, 32 heads: 128-key chunks 0.032
    // ms, 256-key chunks 0.028, 512-key chunks 0.038).
    const int64_t groups = (int64_t)d.B * d.Hkv * ((d.H / d.Hkv + 3) / 4);
    const int64_t want = std::max<int64_t>(1, (512 + groups - 1) / groups);
    int64_t ck = ((d.L + want - 1) / want + 63) / 64 * 64;
    if (ck < 256) ck = 256;
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
