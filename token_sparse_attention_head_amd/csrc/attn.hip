// Causal flash-style attention on MFMA, used for the compact per-head rows and for the
// library's own dense reference.
//
// The skill page "Token Sparse Attention Long Context", Step 3, runs plain softmax
// attention on the gathered tokens; the paper page "Token Sparse Attention: Efficient
// Long-Context Inference with Interleaved Token Selection", Figure 3, stage 2, runs a
// standard attention kernel on the compact tensors (the Abstract: compatible with dense
// attention kernels).  Causality on compact rows equals causality on positions because
// each subset is ascending.
//
//   o_t = sum_{u <= t} softmax_u(scale <q_t, k_u>) v_u,   fp32 accumulation, one rounding.
//
// Design for gfx950 (CDNA4):
// * bf16: a workgroup is 8 waves (2 per SIMD, within 256 registers each, so one wave's
//   softmax arithmetic issues while the other wave's matrix instructions run) over 384
//   query rows of one (batch, head), or 192 rows of each of two query heads that read the
//   same K/V rows (GQA with one subset per KV head, and the dense reference), which then
//   share every staged K/V tile.  Each wave keeps 48 query rows in registers as the
//   operands of three 16-row blocks on the 16x16x32 bf16 MFMA, so each K or V operand it
//   reads from LDS feeds three blocks: LDS operand traffic, the kernel's main cost, per
//   unit of matrix work is two thirds of what 32-row blocks on the 32x32x16 MFMA need.
//   fp32: 4 waves of 32 query rows on the 32x32x2 fp32 MFMA.
// * Key/value tiles of 64 rows stream through LDS, double buffered, with the global loads
//   of the next tile in flight in registers while the current tile is on the matrix
//   cores.
// * Scores are formed transposed, S^T = K Q^T, so a lane owns one query of each block and
//   its row sums stay lane-local (a row's keys are split over four lanes in the bf16
//   kernel, two in the fp32 one; they are combined once, at the end).
// * O^T = V^T P^T: the probabilities a lane already holds are the B operand as they
//   are; the bf16 kernel reads V^T from V's natural [key][d] rows with the transposing
//   LDS read ds_read_b64_tr_b16.  LDS rows are padded so no operand read has bank
//   conflicts.
// * Online softmax in exp2 units against a lazily moved reference: a key block's
//   probabilities (32 keys in the bf16 kernel, a 64-key tile in the fp32 one) are taken
//   against the current reference without a row max, and their sum tells whether that
//   was safe (below 2^32 nothing is near overflow).  Only when it is not (the first
//   block, or a row max that jumped) does the exact max move the reference and rescale
//   O and l.
// * Query tiles are issued longest first; all tiles of a head go to one XCD (workgroup
//   IDs are dealt to the 8 XCDs round-robin) and an XCD runs one head's tiles before the
//   next head's, so its concurrent workgroups stream the same K/V tiles through its L2.
//   With adaptive budgets (rows differ per head) attn_plan_kernel first deals the heads,
//   sorted by attention work, to the XCDs in snake order, keeping that locality while
//   the XCDs get equal work.
// * Out of place, the fused launch also copies the residual rows no head keeps: its first
//   workgroups (64, eight per XCD) stream those rows with buffer accesses, two steps in
//   flight per wave, while the other CUs run the attention, so the copy's memory latency
//   hides behind the attention's arithmetic (a separate copy kernel would occupy every CU
//   for its whole run).
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace tsa {

namespace {

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_b, q_h, q_r;   // element strides of q: batch, head, row
  int64_t k_b, k_h, k_r;   // of k and v (same layout)
  int64_t o_b, o_h, o_r;   // of o
  int n;                   // rows of every head (queries = keys)
  int H;                   // query heads
  int kv_div;              // KV head of query head h is h / kv_div
  int BH, ntiles;
  float c;                 // logit scale * log2(e)
  const int32_t* idx;      // fused forward: [B][H / idx_div][n] positions of each subset's rows
  int idx_div;             // query heads per subset: head h reads idx row b * (H / idx_div) + h / idx_div
  const void* res;         // fused forward: residual, same layout as o
  const int32_t* counts;   // fused forward with adaptive budgets: rows of each subset [B][H / idx_div], or NULL
  const int32_t* plan;     // with counts: the per-XCD head lists of attn_plan_kernel, or NULL
  int plan_cap;            // heads per XCD list in the plan
  int L;                   // fused forward: sequence length (index-list entries are clamped below it)
  int interleave;          // 1: an XCD deals the tiles of its heads in turn (longest first over all of them)
  const int32_t* inv;      // fused forward out of place: [B][H / idx_div][L] kept-row map, < 0 at rows to copy
  int copy_wgs;            // with inv: the first copy_wgs workgroups copy those rows of res to o
  int B;                   // batch entries
};

// Plan of the fused attention under adaptive budgets (rows differ per head).  A head's
// workgroups read that head's own rows, so they should share an XCD's L2 (one XCD, one
// head at a time); the XCDs should get equal work.  Heads are sorted by attention work
// (tiles * (tiles + 1) / 2, longest first; ties by head) and dealt to the 8 XCDs in
// snake order (0..7, 7..0, ...).  Plan layout (int32): [0, 8) tiles per XCD, then per XCD
// `cap` head entries (bh, first slot).  Slot s of XCD x runs tile (tiles - 1 - (s - first))
// of the entry whose range holds s.
constexpr int PLAN_MAX_HEADS = 4096;
constexpr int PLAN_THREADS = 1024;

__global__ __launch_bounds__(PLAN_THREADS) void attn_plan_kernel(const int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ plan, int BH, int H,
                                                                 int idx_div, int BM, int cap) {
  __shared__ unsigned long long key[PLAN_MAX_HEADS];
  int n2 = 1;
  while (n2 < BH) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += PLAN_THREADS) {
    unsigned long long k = 0;
    if (i < BH) {
      const int n = counts[(i / H) * (H / idx_div) + (i % H) / idx_div];
      const unsigned long long t = (unsigned long long)((n + BM - 1) / BM);
      k = ((t * (t + 1) / 2) << 32) | (0xFFFFFFFFu - (unsigned)i);   // work, then lower head first
    }
    key[i] = k;
  }
  __syncthreads();
  // Bitonic sort, descending.
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n2; i += PLAN_THREADS) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const unsigned long long a = key[i], b = key[j];
          if (desc ? a < b : a > b) {
            key[i] = b;
            key[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x < 8) {
    const int x = threadIdx.x;
    int32_t* list = plan + 8 + x * cap * 2;
    int first = 0, e = 0;
    for (int round = 0; round * 8 < BH; ++round) {
      const int pos = (round & 1) ? 7 - x : x;
      const int rank = round * 8 + pos;
      if (rank >= BH) continue;
      const int bh = (int)(0xFFFFFFFFu - (unsigned)(key[rank] & 0xFFFFFFFFu));
      const int n = counts[(bh / H) * (H / idx_div) + (bh % H) / idx_div];
      list[2 * e] = bh;
      list[2 * e + 1] = first;
      first += (n + BM - 1) / BM;
      ++e;
    }
    for (; e < cap; ++e) {            // unused entries start past the end
      list[2 * e] = 0;
      list[2 * e + 1] = first;
    }
    plan[x] = first;
  }
}

constexpr int ATT_COMPACT = 0, ATT_DENSE = 1, ATT_FUSED = 2;
constexpr int BN = 64;          // keys per tile
constexpr int KB = BN / 32;     // 32-key blocks per tile
constexpr float NEG_BIG = -3.0e38f;
constexpr float RESCALE_SLACK = 8.0f;   // log2 units

template <typename T, int D> struct AttnLds;
template <int D> struct AttnLds<float, D> {
  float k[2][BN * D];     // [key][d], 16-byte chunks swizzled by key
  float v[2][BN * D];     // [key][d]
};

template <typename T, int D>
__device__ __forceinline__ void lds_k_frag(const T* ks, int key, int hf, HalfRow<T, D>& f);

template <int D>
__device__ __forceinline__ void lds_k_frag_f32(const float* ks, int key, int hf, HalfRow<float, D>& f) {
#pragma unroll
  for (int s4 = 0; s4 < D / 8; ++s4) {
    const int c = hf * (D / 8) + s4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(ks + key * D + ((c ^ (key & 7)) << 2));
    f.f[4 * s4 + 0] = v[0]; f.f[4 * s4 + 1] = v[1]; f.f[4 * s4 + 2] = v[2]; f.f[4 * s4 + 3] = v[3];
  }
}
template <>
__device__ __forceinline__ void lds_k_frag<float, 64>(const float* ks, int key, int hf, HalfRow<float, 64>& f) {
  lds_k_frag_f32<64>(ks, key, hf, f);
}
template <>
__device__ __forceinline__ void lds_k_frag<float, 128>(const float* ks, int key, int hf, HalfRow<float, 128>& f) {
  lds_k_frag_f32<128>(ks, key, hf, f);
}

// ---- global -> register -> LDS staging of one key/value tile --------------------------
// Rows past the end of the sequence are loaded as copies of the last row: they only
// meet queries that mask them (probability exactly 0), so any finite value will do.

template <typename T, int D, int NT> struct Stage;

template <int D, int NT> struct Stage<float, D, NT> {
  static constexpr int CPR = D / 4;
  static constexpr int CH = BN * CPR / NT;
  u32x4 kr[CH];
  u32x4 vr[CH];

  __device__ __forceinline__ void load(const float* kbase, const float* vbase, int64_t rstride, int k0, int n,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int e = tid + NT * i;
      const int key = e / CPR, c = e % CPR;
      const int j = min(k0 + key, n - 1);
      kr[i] = ld16(kbase + (int64_t)j * rstride + c * 4);
      vr[i] = ld16(vbase + (int64_t)j * rstride + c * 4);
    }
  }

  __device__ __forceinline__ void store(AttnLds<float, D>& L, int buf, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int e = tid + NT * i;
      const int key = e / CPR, c = e % CPR;
      *reinterpret_cast<u32x4*>(&L.k[buf][key * D + ((c ^ (key & 7)) << 2)]) = kr[i];
      *reinterpret_cast<u32x4*>(&L.v[buf][key * D + c * 4]) = vr[i];
    }
  }
};

// ---- P.V for one tile -----------------------------------------------------------------

template <int D, int QB>
__device__ __forceinline__ void pv_tile(const AttnLds<float, D>& L, int buf, int lane,
                                        const f32x16 (&s)[KB][QB], f32x16 (&o)[QB][D / 32]) {
  const int hf = lane >> 5, lc = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + acc_row(r, hf);
        const float va = L.v[buf][key * D + db * 32 + lc];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma(o[qb][db], va, s[kb][qb][r]);
      }
}

// Online softmax of one tile for the wave's query blocks: masks keys above the diagonal
// (only on tiles that reach it), moves the running max lazily, turns scores into
// probabilities in place and accumulates the lane's share of the row sums.
template <bool MASK, int QB, int ND>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[KB][QB], float (&m)[QB], float (&l)[QB],
                                             f32x16 (&o)[QB][ND], int k0, int wrow0, int hf, int lc, float c) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // key k0 + kb*32 + acc_row(r, hf) is above the diagonal iff acc_row(r, 0) > lim - 32*kb
    const int lim = wrow0 + qb * 32 + lc - k0 - 4 * hf;
    float tmax = -__builtin_huge_valf();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (MASK && acc_row(r, 0) > lim - 32 * kb) s[kb][qb][r] = -__builtin_huge_valf();
        tmax = fmaxf(tmax, s[kb][qb][r]);
      }
    tmax = fmaxf(tmax, xor32(tmax));
    const float mt = tmax * c;
    if (__ballot(mt > m[qb] + RESCALE_SLACK) != 0) {
      const float mn = fmaxf(m[qb], mt);
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) o[qb][db] *= alpha;
      m[qb] = mn;
    }
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], c, -m[qb]));
        s[kb][qb][r] = pr;
        lsum += pr;
      }
    l[qb] += lsum;
  }
}

template <typename T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// DENSE selects the strided [B][L][H][d] layout with grouped KV heads (the library's dense
// reference); otherwise rows are the contiguous compact [B][H][keep][d] tensors and the
// row strides are compile-time constants.
template <typename T, int D, int QB, int NW, bool DENSE>
__global__ __launch_bounds__(NW * TSA_WAVE) void attn_kernel(AttnParams p) {
  if (!DENSE) p.q_r = p.k_r = p.o_r = D;
  __shared__ AttnLds<T, D> lds;
  constexpr int BM = NW * QB * 32;
  const int tid = threadIdx.x;
  const int wave = tid / TSA_WAVE;
  const int lane = lane_id();
  const int hf = lane >> 5, lc = lane & 31;

  int bh, tile;
  {
    const int bid = blockIdx.x;
    if (p.BH % 8 == 0) {
      const int hpx = p.BH / 8;
      const int x = bid % 8, sl = bid / 8;
      bh = x * hpx + sl / p.ntiles;
      tile = p.ntiles - 1 - sl % p.ntiles;
    } else {
      bh = bid % p.BH;
      tile = p.ntiles - 1 - bid / p.BH;
    }
  }
  const int64_t b = bh / p.H;
  const int h = bh % p.H;
  const int kvh = h / p.kv_div;
  const T* qbase = reinterpret_cast<const T*>(p.q) + b * p.q_b + h * p.q_h;
  const T* kbase = reinterpret_cast<const T*>(p.k) + b * p.k_b + kvh * p.k_h;
  const T* vbase = reinterpret_cast<const T*>(p.v) + b * p.k_b + kvh * p.k_h;
  T* obase = reinterpret_cast<T*>(p.o) + b * p.o_b + h * p.o_h;

  const int q0 = tile * BM;
  const int wrow0 = q0 + wave * QB * 32;
  const int wave_last = min(p.n - 1, wrow0 + QB * 32 - 1);
  const int nkt = (min(p.n, q0 + BM) - 1) / BN + 1;

  HalfRow<T, D> qf[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + qb * 32 + lc;
    if (row < p.n)
      qf[qb].load(qbase + (int64_t)row * p.q_r + hf * (D / 2));
    else
      qf[qb].zero();
  }

  f32x16 o[QB][D / 32];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = NEG_BIG;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[qb][db] = f32x16{};
  }

  Stage<T, D, NW * TSA_WAVE> st;
  st.load(kbase, vbase, p.k_r, 0, p.n, tid);
  for (int t = 0; t < nkt; ++t) {
    const int buf = t & 1;
    st.store(lds, buf, tid);
    __syncthreads();
    if (t + 1 < nkt) st.load(kbase, vbase, p.k_r, (t + 1) * BN, p.n, tid);
    const int k0 = t * BN;
    if (wrow0 > wave_last || k0 > wave_last) continue;   // no visible key for this wave's rows

    // S^T = K Q^T for the tile.
    f32x16 s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      HalfRow<T, D> kf;
      lds_k_frag<T, D>(lds.k[buf], kb * 32 + lc, hf, kf);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[kb][qb] = f32x16{};
        s[kb][qb] = dot_tile<T, D>(s[kb][qb], kf, qf[qb]);
      }
    }

    if (k0 + BN - 1 > wrow0)
      softmax_tile<true, QB>(s, m, l, o, k0, wrow0, hf, lc, p.c);
    else
      softmax_tile<false, QB>(s, m, l, o, k0, wrow0, hf, lc, p.c);

    pv_tile<D, QB>(lds, buf, lane, s, o);
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + xor32(l[qb]);
    const float inv = 1.0f / lt;
    const int i = wrow0 + qb * 32 + lc;
    if (i < p.n) {
      T* orow = obase + (int64_t)i * p.o_r;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = db * 32 + 8 * r4 + 4 * hf;
          store4<T>(orow + d0, o[qb][db][4 * r4] * inv, o[qb][db][4 * r4 + 1] * inv, o[qb][db][4 * r4 + 2] * inv,
                    o[qb][db][4 * r4 + 3] * inv);
        }
    }
  }
}

// ---- bf16 kernel ------------------------------------------------------------------------
//
// 48 query rows per wave as three 16-row blocks on v_mfma_f32_16x16x32_bf16.  16x16 output
// tiles: lane l holds column (l % 16) and rows 4*(l/16) + i, i = 0..3; operand A: lane l
// supplies row (l % 16) and the contraction slice 8*(l/16) .. +7; operand B: column
// (l % 16) and the same slice.  Every K and V operand a wave reads from LDS feeds its three
// query blocks, so a 64-key tile's LDS operand bytes serve 48 query rows per wave.
//
// Scores: S^T (16 keys x 16 queries) = K Q^T over D/32 steps of 32 d.  In step s lane
// group g = l/16 supplies d = 32 s + 8 g .. +7 (K and Q use the same split), so the four
// lane groups of one key row read its 64 contiguous bytes of the step.  The lane then owns
// query (l % 16) of each block and keys 4g .. 4g+3 of each 16-key block.
//
// P.V: O^T (16 d x 16 queries) += V^T (16 d x 32 keys) P^T.  A lane's P^T operand is its
// own 8 probabilities of the 32-key half, keys {4g .. 4g+3} and {16+4g .. 16+4g+3}; the V^T
// operand must cover the same keys, which the transposing LDS read ds_read_b64_tr_b16
// gives from V's natural [key][d] rows: it hands lane i of each 16-lane block element
// i % 4 of the 8 bytes that lanes 4j + i/4 (j = 0..3) address, so pointing lane s at
// V[k0 + s/4][d0 + 4 (s%4) .. +3] gives lane i the values V[k0 + j][d0 + i].  Two such
// reads (k0 = 4g and 16 + 4g) make the operand.
//
// LDS rows are padded, not swizzled, so every operand address is one register plus an
// immediate.  K and V rows are both 2d+32 bytes apart (8 banks between rows).  For V: one
// transposing read cycle serves 32 lanes, eight key rows of 8 banks each, which this pitch
// keeps disjoint (2d+64, the pitch for a 32x32 operand layout, puts rows four apart on the
// same banks).  For K the pitch was chosen by the bank-conflict counter: with the 64-byte
// row segments above it reads without conflicts, while 2d+16 and 2d+64 (and every pitch
// tried, 2d+16 to 2d+80, with K split into contiguous quarters of d per lane group) conflict.  The tile loop is
// unrolled by two so the buffer offsets are immediates too.

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 tr_read2(const char* a, const char* b) {
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a);
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)b);
  const i16x8 z = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ f32x4 mfma16(f32x4 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Copy of the residual rows no subset keeps, run by the first workgroups of the fused
// attention launch so that it overlaps the attention on the other CUs: the copy is bound by
// memory latency and needs few CUs, the attention by the matrix and vector units.  Rows are
// (position, head) rows of d elements in memory order.  Every wave of a copy workgroup
// streams a contiguous run of rows on its own (no barriers: a workgroup barrier waits for
// every load in flight).  A step is CP_UNROLL wave-wide 16-byte accesses, each covering
// 64 / (row vectors) rows; the rows whose kept-row map entry is negative are read and
// written.  Two steps of data are in flight: the next step's reads are issued before this
// step's writes, and the map entries (one load per lane for a step's rows, handed to the
// lanes that copy each row by cross-lane reads) two steps ahead.
#ifndef TSA_COPY_WGS
#define TSA_COPY_WGS 64
#endif
#ifndef TSA_COPY_UNROLL
#define TSA_COPY_UNROLL 16
#endif
constexpr int kCopyWgs = TSA_COPY_WGS;     // copy workgroups (a multiple of 8: one share per XCD)
constexpr int CP_UNROLL = TSA_COPY_UNROLL;

template <int ROWB>
constexpr int copy_rows_per_step() { return TSA_WAVE / (ROWB / 16) * CP_UNROLL; }

// A step covers whole positions (the host launches the in-attention copy only when the
// heads H divide the step's rows, L >= the step's positions and the rows fit 32 bits), so a
// lane's head and position offset within a step are fixed; the position (b, pos) of the
// next step to fetch advances by the step's positions.
template <int ROWB, int NT>
__device__ __forceinline__ void copy_unkept_rows(const AttnParams& p, int wg) {
  constexpr int VPR = ROWB / 16;                   // 16-byte vectors per row
  constexpr int RPI = TSA_WAVE / VPR;              // rows per wave-wide access
  constexpr int U = CP_UNROLL;
  constexpr int RPS = copy_rows_per_step<ROWB>();  // rows per step
  constexpr int EPL = RPS / TSA_WAVE;              // map entries per lane per step
  static_assert(RPS % TSA_WAVE == 0 && TSA_WAVE % RPI == 0, "step shape");
  const int lane = lane_id();
  // Wave-uniform (the buffer views below must live in scalar registers).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / TSA_WAVE);
  const int sub = lane / VPR, vec = lane % VPR;
  const int H = p.H, L = p.L, R = p.H / p.idx_div;
  const int PPS = RPS / H;                         // positions per step
  const uint32_t npos = (uint32_t)p.B * (uint32_t)L;
  const uint32_t nw = (uint32_t)p.copy_wgs * (NT / TSA_WAVE);
  const uint32_t seg = ((npos + nw - 1) / nw + PPS - 1) / PPS * PPS;   // positions per wave
  const uint32_t g0 = ((uint32_t)wg * (NT / TSA_WAVE) + wave) * seg;
  if (g0 >= npos) return;
  const uint32_t g1 = g0 + seg < npos ? g0 + seg : npos;
  const uint32_t row_end = g1 * (uint32_t)H;
  int po[EPL], hs[EPL];                            // position offset and subset of the lane's map entries
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int t = i * TSA_WAVE + lane;
    po[i] = t / H;
    hs[i] = (t % H) / p.idx_div;
  }
  // Buffer views of the wave's run of rows: a lane whose row is kept (or past the run)
  // gets an offset beyond the range, so its read returns 0 and its write is dropped, with
  // no branch (branches around the accesses would make the compiler wait for every access
  // in flight where they join).
  const uint32_t row0 = g0 * (uint32_t)H;
  const uint32_t run_bytes = (row_end - row0) * (uint32_t)ROWB;
  constexpr uint32_t OUTSIDE = 0x80000000u;
  constexpr int BUF_FLAGS = 0x00020000;            // buffer resource word 3: 32-bit data format, raw access
  constexpr int NT_POLICY = 2;                     // non-temporal
  const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(p.res)) + (int64_t)row0 * ROWB, 0, (int)run_bytes, BUF_FLAGS);
  const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<char*>(p.o) + (int64_t)row0 * ROWB, 0, (int)run_bytes, BUF_FLAGS);
  int b = (int)(g0 / (uint32_t)L), pos = (int)(g0 % (uint32_t)L);
  // Map entries of the step at (b, pos) whose first row is r0 (0, i.e. kept, past the run);
  // then (b, pos) moves to the next step.  The read index is always in range.
  auto fetch = [&](int (&ent)[EPL], uint32_t r0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      int pj = pos + po[i], bj = b;
      if (pj >= L) { pj -= L; ++bj; }
      bj = bj < p.B ? bj : p.B - 1;
      const int e = p.inv[((int64_t)bj * R + hs[i]) * L + pj];
      ent[i] = r0 + i * TSA_WAVE + lane < row_end ? e : 0;
    }
    pos += PPS;
    if (pos >= L) { pos -= L; ++b; }
  };
  // Access j of a step copies row j * RPI + sub of the step: its byte offset in the run,
  // or OUTSIDE.
  auto offsets = [&](uint32_t (&o)[U], const int (&ent)[EPL], uint32_t r0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int e = __shfl(ent[j * RPI / TSA_WAVE], (j * RPI) % TSA_WAVE + sub, TSA_WAVE);
      o[j] = e < 0 ? (r0 - row0 + j * RPI + sub) * (uint32_t)ROWB + vec * 16 : OUTSIDE;
    }
  };
  auto load = [&](u32x4 (&v)[U], const uint32_t (&o)[U]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(src, o[j], 0, NT_POLICY);
  };
  auto store = [&](const u32x4 (&v)[U], const uint32_t (&o)[U]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < U; ++j) __builtin_amdgcn_raw_buffer_store_b128(v[j], dst, o[j], 0, NT_POLICY);
  };
  uint32_t r = row0;
  int entA[EPL], entB[EPL];
  uint32_t oA[U], oB[U];
  u32x4 vA[U], vB[U];
  fetch(entA, r);                                  // entries of steps 0 and 1
  fetch(entB, r + RPS);
  offsets(oA, entA, r);
  load(vA, oA);                                    // step 0 in flight
  fetch(entA, r + 2 * RPS);                        // entries of step 2
  // Steps past the run have no negative entries, so the pairs need no tail.
  for (; r < row_end; r += 2 * RPS) {
    offsets(oB, entB, r + RPS);
    load(vB, oB);                                  // step k + 1 in flight
    store(vA, oA);                                 // step k written
    fetch(entB, r + 3 * RPS);
    offsets(oA, entA, r + 2 * RPS);
    load(vA, oA);                                  // step k + 2 in flight
    store(vB, oB);                                 // step k + 1 written
    fetch(entA, r + 4 * RPS);
  }
}

// Whether the fused launch can carry the copy (else the forward launches it on its own).
template <int ROWB>
bool copy_fits(int B, int L, int H) {
  constexpr int RPS = copy_rows_per_step<ROWB>();
  // Rows, and the rows of the steps fetched up to four past a run's end, fit 32 bits; a copy
  // wave's run (at least 512 waves) stays below 2^31 bytes.
  const int64_t rows = (int64_t)B * L * H;
  return H > 0 && RPS % H == 0 && L >= RPS / H && rows < ((int64_t)1 << 32) - 8 * RPS &&
         rows / (8 * (kCopyWgs < 64 ? kCopyWgs : 64)) * ROWB < ((int64_t)1 << 30);
}

constexpr int BF16_QB = 3;                 // 16-row query blocks per wave
constexpr int BF16_WQ = 16 * BF16_QB;      // query rows per wave

// MODE selects where rows live: ATT_COMPACT (contiguous [B][H][n][d] compact tensors),
// ATT_DENSE ([B][L][H][d] and [B][L][Hkv][d], all L rows: the dense reference) or
// ATT_FUSED (the compact rows are read through each head's index list straight from
// [B][L][H][d] / [B][L][Hkv][d], and the epilogue writes residual + O into those rows of
// the output: the fused forward, which never materialises Q^, K^, V^ or O^).
//
// HPW = 2: the workgroup runs two query heads that read the same K/V rows (a GQA group with
// one subset per KV head, or the dense reference), four waves each, so each staged K/V tile
// serves both heads.
template <int D, int NW, int MODE, int HPW>
__global__ __launch_bounds__(NW * TSA_WAVE, 2) void attn_bf16_kernel(AttnParams p) {
  constexpr bool FUSED = MODE == ATT_FUSED, STRIDED = MODE != ATT_COMPACT;
  constexpr int NT = NW * TSA_WAVE;
  constexpr int QB = BF16_QB, WQ = BF16_WQ;
  constexpr int WPH = NW / HPW;                   // waves per query head
  constexpr int BM = WPH * WQ;                    // query rows per head in the tile
  constexpr int ST = D / 32;                      // MFMA steps over d
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  constexpr int LOADS = BN * CPR / NT;            // chunks per lane per tensor per tile
  static_assert(LOADS >= 1 && BN * CPR % NT == 0, "a tile splits evenly over the lanes");
  constexpr int RSTEP = NT / CPR;                 // rows between a lane's chunks
  constexpr int KP = 2 * D + 32, VP = 2 * D + 32; // padded row pitches, bytes
  struct Buf {
    char k[BN * KP];
    char v[BN * VP];
  };
  __shared__ __attribute__((aligned(16))) Buf lds[2];

  // Arguments in registers (lambdas capture by reference; a captured argument struct
  // would be placed in scratch memory).
  const int64_t q_r = STRIDED ? p.q_r : D, k_r = STRIDED ? p.k_r : D, o_r = STRIDED ? p.o_r : D;
  const int kv_div = p.kv_div;
  const float c = p.c;

  const int tid = threadIdx.x;
  const int wave = tid / TSA_WAVE;
  const int lane = lane_id();
  const int g = lane >> 4, lq = lane & 15;

  int bh, tile, n = p.n;
  {
    int bid = blockIdx.x;
    if (FUSED && p.copy_wgs > 0) {
      if (bid < p.copy_wgs) {
        copy_unkept_rows<2 * D, NT>(p, bid);
        return;
      }
      bid -= p.copy_wgs;
    }
    if (FUSED && p.counts && p.plan) {
      // Rows differ per subset: the XCD's head list from attn_plan_kernel, one head after
      // another, longest tiles first.
      const int x = bid % 8, sl = bid / 8;
      if (sl >= p.plan[x]) return;
      const int32_t* list = p.plan + 8 + x * p.plan_cap * 2;
      int lo = 0, hi = p.plan_cap - 1;             // last entry whose first slot <= sl
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (list[2 * mid + 1] <= sl) lo = mid; else hi = mid - 1;
      }
      bh = list[2 * lo];
      n = p.counts[(bh / p.H) * (p.H / p.idx_div) + (bh % p.H) / p.idx_div];
      tile = (n + BM - 1) / BM - 1 - (sl - list[2 * lo + 1]);
    } else if (FUSED && p.counts) {
      // Too many heads for a plan: rank r of every head in turn (longest tiles first),
      // heads rotated so that one head's tiles spread over all XCDs.
      const int r = bid / p.BH;
      bh = (bid % p.BH + r) % p.BH;
      n = p.counts[(bh / p.H) * (p.H / p.idx_div) + (bh % p.H) / p.idx_div];
      tile = (n + BM - 1) / BM - 1 - r;
      if (tile < 0) return;
    } else if (p.BH % 8 == 0) {
      // Heads are dealt to XCDs in blocks of BH / 8.  Long rows: one head at a time per XCD,
      // so its workgroups share the head's K/V tiles in that XCD's L2.  Few tiles per head:
      // the tiles of the XCD's heads in turn, longest first over all of them, so no head's
      // longest tile starts late (the grid is short and the tail would dominate).
      const int hpx = p.BH / 8;
      const int x = bid % 8, sl = bid / 8;
      if (p.interleave) {
        bh = x * hpx + sl % hpx;
        tile = p.ntiles - 1 - sl / hpx;
      } else {
        bh = x * hpx + sl / p.ntiles;
        tile = p.ntiles - 1 - sl % p.ntiles;
      }
    } else {
      bh = bid % p.BH;
      tile = p.ntiles - 1 - bid / p.BH;
    }
  }
  // bh counts groups of HPW query heads that read the same K/V rows; this wave's head:
  const int64_t b = bh / (p.H / HPW);
  const int h = HPW == 1 ? (int)(bh % p.H) : (int)(bh % (p.H / HPW)) * HPW + wave / WPH;
  const int kvh = h / kv_div;
  const __bf16* qbase = reinterpret_cast<const __bf16*>(p.q) + b * p.q_b + h * p.q_h;
  const char* kb8 = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(p.k) + b * p.k_b + kvh * p.k_h);
  const char* vb8 = reinterpret_cast<const char*>(reinterpret_cast<const __bf16*>(p.v) + b * p.k_b + kvh * p.k_h);
  __bf16* obase = reinterpret_cast<__bf16*>(p.o) + b * p.o_b + h * p.o_h;
  const int32_t* idx_bh = FUSED ? p.idx + (b * (p.H / p.idx_div) + h / p.idx_div) * (int64_t)p.n : nullptr;
  // Index-list entries are clamped to the sequence, so a corrupt list stays in bounds.
  const uint32_t lmax = FUSED ? (uint32_t)(p.L - 1) : 0u;

  const int q0 = tile * BM;
  const int wrow0 = q0 + (HPW == 1 ? wave : wave % WPH) * WQ;
  const int wave_last = min(n - 1, wrow0 + WQ - 1);
  const int nkt = (min(n, q0 + BM) - 1) / BN + 1;

  // Staging: chunk i of this lane is row lrow + i * RSTEP, 16-byte chunk lch of the tile.
  // Global offsets are 32-bit bytes from the head's K / V base (the host keeps one batch
  // entry's K and V below 4 GiB).
  const int lrow = tid / CPR, lch = tid % CPR;
  const int soff_k = lrow * KP + lch * 16, soff_v = lrow * VP + lch * 16;
  const uint32_t rbytes = (uint32_t)(k_r * 2);
  uint32_t goff = lrow * rbytes + lch * 16;       // chunk 0 of the next tile
  int pnext[LOADS];                               // fused: positions of the next tile's rows
  if (FUSED) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) pnext[i] = idx_bh[min(lrow + i * RSTEP, n - 1)];
  }
  u32x4 kst[LOADS], vst[LOADS];                   // the next tile, in flight in registers
  int next_k0 = 0;
  // Loads the next tile into registers; rows past the end repeat the last row (they
  // only meet queries that mask them).  Fused: the rows' positions were fetched one tile
  // earlier, and this fetches the positions of the tile after.
  auto load_next = [&]() __attribute__((always_inline)) {
    if (FUSED) {
      // The next tile's positions are requested before this tile's rows: loads complete
      // in order, so waiting for the positions later does not wait for the rows.
      int pcur[LOADS];
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        pcur[i] = pnext[i];
        pnext[i] = idx_bh[min(next_k0 + BN + lrow + i * RSTEP, n - 1)];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t off = min((uint32_t)pcur[i], lmax) * rbytes + lch * 16;
        kst[i] = ld16(kb8 + off);
        vst[i] = ld16(vb8 + off);
      }
    } else if (next_k0 + BN <= n) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        kst[i] = ld16(kb8 + (goff + i * RSTEP * rbytes));
        vst[i] = ld16(vb8 + (goff + i * RSTEP * rbytes));
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t off = (uint32_t)min(next_k0 + lrow + i * RSTEP, n - 1) * rbytes + lch * 16;
        kst[i] = ld16(kb8 + off);
        vst[i] = ld16(vb8 + off);
      }
    }
    goff += BN * rbytes;
    next_k0 += BN;
  };

  // Q operands: block qb, step s = 8 values of row wrow0 + 16 qb + lq from d = 32 s + 8 g.
  bf16x8 qf[QB][ST];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 16 * qb + lq;
    if (row < n) {
      const __bf16* src = qbase + (int64_t)(FUSED ? min((uint32_t)idx_bh[row], lmax) : (uint32_t)row) * q_r + 8 * g;
#pragma unroll
      for (int s = 0; s < ST; ++s) qf[qb][s] = *reinterpret_cast<const bf16x8*>(src + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < ST; ++s) qf[qb][s] = bf16x8{};
    }
  }
  const int koff = lq * KP + g * 16;                               // K operand: key lq, d 8g + 32 s
  const int voff = (4 * g + (lq >> 2)) * VP + 4 * (lq & 3) * 2;   // V^T operand, see above

  f32x4 o[D / 16][QB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = NEG_BIG;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db][qb] = f32x4{};
  }

  auto step = [&](int t, Buf& cur) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      *reinterpret_cast<u32x4*>(cur.k + soff_k + i * RSTEP * KP) = kst[i];
      *reinterpret_cast<u32x4*>(cur.v + soff_v + i * RSTEP * VP) = vst[i];
    }
    __syncthreads();
    // Unconditional (past the end it re-reads the clamped last rows): every step then
    // issues the same loads, so the wait before a store only waits for that tile.
    load_next();
    const int k0 = t * BN;
    if (wrow0 > wave_last || k0 > wave_last) return;   // no key of this tile is visible
#pragma unroll
    for (int hh = 0; hh < BN / 32; ++hh) {
      const int kh = k0 + 32 * hh;
      if (kh > wave_last) break;
      // S^T blocks: keys kh + 16 kk + 4 g + i, query 16 qb + lq.  Each 16-key block's K
      // operands are read before its MFMAs so the reads overlap one another.
      f32x4 s[2][QB];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 kf[ST];
#pragma unroll
        for (int st = 0; st < ST; ++st)
          kf[st] = *reinterpret_cast<const bf16x8*>(cur.k + (32 * hh + 16 * kk) * KP + koff + st * 64);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kk][qb] = f32x4{};
        // The score products issue at a raised wave priority: when both waves of a SIMD
        // are ready, the one starting its burst of products goes first and the other's
        // softmax arithmetic fills in behind it (about 1% faster at L = 131072 and 32768;
        // the same over the PV products as well, or over the softmax, was slower).
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < ST; ++st)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kk][qb] = mfma16(s[kk][qb], kf[st], qf[qb][st]);
        __builtin_amdgcn_s_setprio(0);
      }
      if (kh + 31 > wrow0) {                       // the half reaches the diagonal
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (kh + 16 * kk + 4 * g + i > wrow0 + 16 * qb + lq) s[kk][qb][i] = -__builtin_huge_valf();
      }
      // Online softmax of the half: probabilities against the running reference m; the
      // probability sums guard it (below 2^32 nothing is near overflow), else the exact
      // row max (over the four lane groups) moves m and rescales O and l.
      bf16x8 pf[QB];
      float ls[QB];
      auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float pr[8];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pr[4 * kk + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kk][qb][i], c, -m[qb]));
              pf[qb][4 * kk + i] = static_cast<__bf16>(pr[4 * kk + i]);
            }
          // The lane's 8 probabilities summed as a tree (7 additions, no chain through zero).
          ls[qb] = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
        }
      };
      probs();
      bool unsafe = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) unsafe |= !(ls[qb] < 4294967296.0f);
      if (__ballot(unsafe) != 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float tmax = -__builtin_huge_valf();
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[kk][qb][i]);
          tmax = fmaxf(tmax, __shfl_xor(tmax, 16, TSA_WAVE));
          tmax = fmaxf(tmax, __shfl_xor(tmax, 32, TSA_WAVE));
          const float mn = fmaxf(m[qb], tmax * c);
          const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 16; ++db) o[db][qb] *= alpha;
          m[qb] = mn;
        }
        probs();
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l[qb] += ls[qb];
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const char* a = cur.v + (32 * hh) * VP + voff + db * 32;
        const bf16x8 va = tr_read2(a, a + 16 * VP);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma16(o[db][qb], va, pf[qb]);
      }
    }
  };

  load_next();
  // Steps run in pairs; a step past the last tile only stages and meets the barrier
  // (no wave sees its keys), which keeps the loop body free of conditions.
  for (int t = 0; t < nkt; t += 2) {
    step(t, lds[0]);
    step(t + 1, lds[1]);
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float lt = l[qb];                              // row sum over the four lane groups
    lt += __shfl_xor(lt, 16, TSA_WAVE);
    lt += __shfl_xor(lt, 32, TSA_WAVE);
    const float inv = 1.0f / lt;
    const int i = wrow0 + 16 * qb + lq;
    if (i >= n) continue;
    if (FUSED) {
      // out = residual + O, with O first rounded to bf16 as the staged path stores it.
      const int64_t roff = (int64_t)min((uint32_t)idx_bh[i], lmax) * o_r;
      const __bf16* rrow = reinterpret_cast<const __bf16*>(p.res) + b * p.o_b + h * p.o_h + roff;
      __bf16* orow = obase + roff;
      u32x2 rvs[D / 16];                           // all residual reads in flight at once
#pragma unroll
      for (int db = 0; db < D / 16; ++db) rvs[db] = *reinterpret_cast<const u32x2*>(rrow + 16 * db + 4 * g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ob = bf16_to_f32(f32_to_bf16(o[db][qb][e] * inv));
          const uint32_t rb = (rvs[db][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          v[e] = bf16_to_f32(rb) + ob;
        }
        store4<__bf16>(orow + 16 * db + 4 * g, v[0], v[1], v[2], v[3]);
      }
    } else {
      __bf16* orow = obase + (int64_t)i * o_r;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        store4<__bf16>(orow + 16 * db + 4 * g, o[db][qb][0] * inv, o[db][qb][1] * inv, o[db][qb][2] * inv,
                       o[db][qb][3] * inv);
    }
  }
}

// Tile order of an XCD (see the kernel): the heads' tiles in turn below this many query
// tiles per head, one head at a time above.  Measured on one MI355X (fused attention):
// L = 8192 keep 0.5 (11 tiles) 0.212 -> 0.177 ms, the planted L = 65536 keep 0.1 layer (18)
// 0.875 -> 0.832, L = 32768 keep 0.25 (22) 0.660 -> 0.638, L = 131072 keep 0.1 (35) 1.479 ->
// 1.425; at keep 0.25 (86 tiles) interleaving lost 1% (compact kernel 6%): long rows need the
// one-head-per-XCD L2 reuse.
constexpr int kInterleaveBelowTiles = 48;
int attn_interleave(int ntiles) { return ntiles < kInterleaveBelowTiles ? 1 : 0; }

template <int D, int NW, int MODE, int HPW = 1>
hipError_t launch_attn_bf16(AttnParams p, int B, int H, hipStream_t s) {
  constexpr int BM = NW / HPW * BF16_WQ;
  p.B = B;
  p.BH = B * H / HPW;                             // head groups (the adaptive paths run HPW = 1)
  p.ntiles = (p.n + BM - 1) / BM;
  p.interleave = attn_interleave(p.ntiles);
  int64_t blocks = (int64_t)p.BH * p.ntiles;
  if (MODE == ATT_FUSED && p.counts && p.plan) {
    p.plan_cap = (p.BH + 7) / 8;
    attn_plan_kernel<<<1, PLAN_THREADS, 0, s>>>(p.counts, const_cast<int32_t*>(p.plan), p.BH, p.H, p.idx_div, BM,
                                                p.plan_cap);
    blocks = 8ll * p.plan_cap * p.ntiles;
  }
  p.copy_wgs = 0;
  if (MODE == ATT_FUSED && p.inv) {
    if (!copy_fits<2 * D>(B, p.L, H)) return hipErrorInvalidValue;
    // Copy workgroups first (dispatched first, one per CU), a multiple of 8 so that the
    // attention workgroups keep their XCD (workgroup IDs are dealt to the XCDs in turn).
    const int64_t rows = (int64_t)B * p.L * H;    // at least 4096 rows per copy workgroup
    p.copy_wgs = (int)std::min<int64_t>(kCopyWgs, (rows + 8 * 4096 - 1) / (8 * 4096) * 8);
    blocks += p.copy_wgs;
  }
  attn_bf16_kernel<D, NW, MODE, HPW><<<(unsigned)blocks, NW * TSA_WAVE, 0, s>>>(p);
  return hipGetLastError();
}

template <typename T, int D, int QB, int NW, bool DENSE>
hipError_t launch_attn_t(AttnParams p, int B, int H, hipStream_t s) {
  constexpr int BM = NW * QB * 32;
  p.BH = B * H;
  p.ntiles = (p.n + BM - 1) / BM;
  const int64_t blocks = (int64_t)p.BH * p.ntiles;
  attn_kernel<T, D, QB, NW, DENSE><<<(unsigned)blocks, NW * TSA_WAVE, 0, s>>>(p);
  return hipGetLastError();
}

template <bool DENSE>
hipError_t dispatch_attn(const tsa_desc& d, AttnParams p, hipStream_t s) {
  if (d.dtype == TSA_BF16) {
    constexpr int M = DENSE ? ATT_DENSE : ATT_COMPACT;
    const bool pairs = p.kv_div % 2 == 0;         // two query heads per K/V head and workgroup
    if (d.d == 128) return pairs ? launch_attn_bf16<128, 8, M, 2>(p, d.B, d.H, s) : launch_attn_bf16<128, 8, M>(p, d.B, d.H, s);
    if (d.d == 64) return pairs ? launch_attn_bf16<64, 8, M, 2>(p, d.B, d.H, s) : launch_attn_bf16<64, 8, M>(p, d.B, d.H, s);
  } else {
    if (d.d == 128) return launch_attn_t<float, 128, 1, 4, DENSE>(p, d.B, d.H, s);
    if (d.d == 64) return launch_attn_t<float, 64, 1, 4, DENSE>(p, d.B, d.H, s);
  }
  return hipErrorInvalidValue;
}

float attn_c(const tsa_desc& d) {
  const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.d);
  return scale * TSA_LOG2E;
}

}  // namespace

hipError_t launch_attn_compact(const tsa_desc& d, const void* qh, const void* kh, const void* vh, void* oh,
                               hipStream_t s) {
  AttnParams p{};
  p.q = qh; p.k = kh; p.v = vh; p.o = oh;
  p.n = d.keep;
  p.H = d.H;
  p.kv_div = heads_per_subset(d);               // compact K/V rows are per subset
  p.q_r = d.d; p.q_h = (int64_t)d.keep * d.d; p.q_b = (int64_t)d.H * d.keep * d.d;
  p.k_r = p.q_r; p.k_h = p.q_h; p.k_b = (int64_t)subset_rows(d) * d.keep * d.d;
  p.o_r = p.q_r; p.o_h = p.q_h; p.o_b = p.q_b;
  p.c = attn_c(d);
  return dispatch_attn<false>(d, p, s);
}

size_t attn_plan_bytes(const tsa_desc& d) {
  const int64_t BH = (int64_t)d.B * d.H;
  return BH <= PLAN_MAX_HEADS ? (size_t)(8 + 8 * ((BH + 7) / 8) * 2) * 4 : 0;
}

hipError_t launch_attn_fused(const tsa_desc& d, const void* q, const void* k, const void* v, const int32_t* idx,
                             const int32_t* counts, int32_t* plan, const void* res, void* out, const int32_t* inv,
                             hipStream_t s) {
  if (d.dtype != TSA_BF16) return hipErrorInvalidValue;
  if (inv && !(d.d == 128 ? copy_fits<256>(d.B, d.L, d.H) : copy_fits<128>(d.B, d.L, d.H))) {
    // Shapes the in-launch copy does not cover: the copy runs as its own kernel first.
    const hipError_t e = launch_copy_unselected(d, inv, res, out, s);
    if (e != hipSuccess) return e;
    inv = nullptr;
  }
  AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.idx = idx; p.res = res; p.counts = counts; p.inv = inv;
  p.plan = attn_plan_bytes(d) ? plan : nullptr;
  p.idx_div = heads_per_subset(d);
  p.n = d.keep;
  p.L = d.L;
  p.H = d.H;
  p.kv_div = d.H / d.Hkv;
  p.q_r = (int64_t)d.H * d.d; p.q_h = d.d; p.q_b = (int64_t)d.L * d.H * d.d;
  p.k_r = (int64_t)d.Hkv * d.d; p.k_h = d.d; p.k_b = (int64_t)d.L * d.Hkv * d.d;
  p.o_r = p.q_r; p.o_h = p.q_h; p.o_b = p.q_b;
  p.c = attn_c(d);
  // Two query heads per workgroup when they share a subset (and so K/V rows); adaptive
  // budgets keep one head per workgroup (the per-XCD plan deals heads).
  const bool pairs = !counts && p.idx_div % 2 == 0 && p.kv_div % 2 == 0;
  if (d.d == 128)
    return pairs ? launch_attn_bf16<128, 8, ATT_FUSED, 2>(p, d.B, d.H, s) : launch_attn_bf16<128, 8, ATT_FUSED>(p, d.B, d.H, s);
  if (d.d == 64)
    return pairs ? launch_attn_bf16<64, 8, ATT_FUSED, 2>(p, d.B, d.H, s) : launch_attn_bf16<64, 8, ATT_FUSED>(p, d.B, d.H, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_dense(const tsa_desc& d, const void* q, const void* k, const void* v, void* o,
                             hipStream_t s) {
  AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o;
  p.n = d.L;
  p.H = d.H;
  p.kv_div = d.H / d.Hkv;
  p.q_r = (int64_t)d.H * d.d; p.q_h = d.d; p.q_b = (int64_t)d.L * d.H * d.d;
  p.k_r = (int64_t)d.Hkv * d.d; p.k_h = d.d; p.k_b = (int64_t)d.L * d.Hkv * d.d;
  p.o_r = p.q_r; p.o_h = p.q_h; p.o_b = p.q_b;
  p.c = attn_c(d);
  return dispatch_attn<true>(d, p, s);
}

}  // namespace tsa
