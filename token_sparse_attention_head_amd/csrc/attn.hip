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
// * A workgroup is NW waves over BM = NW * QB * 32 query rows of one (batch, head); each
//   wave keeps its QB blocks of 32 query rows in registers as MFMA operands.  The bf16
//   kernel runs 8 waves (2 per SIMD) within 256 registers each, so one wave's softmax
//   arithmetic issues while the other wave's matrix instructions run.
// * Key/value tiles of 64 rows stream through LDS, double buffered, with the next
//   tile's global loads in flight while the current tile is on the matrix cores.
// * Scores are formed transposed, S^T = K Q^T (32x32x16 bf16 MFMA), so a lane owns one
//   query and 16 keys per 32-key block: the softmax row max needs one cross-half
//   exchange per tile and the row sum stays lane-local.
// * O^T = V^T P^T: the probabilities a lane already holds are the B operand as they
//   are; V is written to LDS transposed, with keys permuted inside each 16-key group
//   to match, so every operand read is one 16-byte LDS read.  16-byte chunks are
//   XOR-swizzled so the 32 rows a wave reads at once fall in different banks.
// * Online softmax in exp2 units with lazy rescaling: the running max moves (and O, l
//   are rescaled) only when a row's max grows by more than 2^8, which keeps every
//   probability below 256 and skips almost all rescales on long rows.
// * Query tiles are issued longest first; all tiles of a head go to one XCD (workgroup
//   IDs are dealt to the 8 XCDs round-robin) so the K/V tiles they share hit in that
//   XCD's L2.
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
};

constexpr int BN = 64;          // keys per tile
constexpr int KB = BN / 32;     // 32-key blocks per tile
constexpr float NEG_BIG = -3.0e38f;
constexpr float RESCALE_SLACK = 8.0f;   // log2 units

template <typename T, int D> struct AttnLds;
template <int D> struct AttnLds<__bf16, D> {
  __bf16 k[2][BN * D];    // [key][d], 16-byte chunks swizzled by key
  __bf16 vt[2][D * BN];   // [d][permuted key], 16-byte chunks swizzled by d
};
template <int D> struct AttnLds<float, D> {
  float k[2][BN * D];     // [key][d], 16-byte chunks swizzled by key
  float v[2][BN * D];     // [key][d]
};

__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Position of tile key w in the transposed V layout: inside each 16-key group, keys
// {0-3, 8-11} take slots 0-7 and keys {4-7, 12-15} take slots 8-15, which is the order
// in which the two lane halves hold probabilities of that group.
__device__ __forceinline__ int vt_pos(int w) {
  const int w16 = w & 15;
  return (w & ~15) + 8 * ((w16 & 7) >> 2) + 4 * (w16 >> 3) + (w16 & 3);
}

template <typename T, int D>
__device__ __forceinline__ void lds_k_frag(const T* ks, int key, int hf, HalfRow<T, D>& f);

template <>
__device__ __forceinline__ void lds_k_frag<__bf16, 128>(const __bf16* ks, int key, int hf, HalfRow<__bf16, 128>& f) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c = hf * 8 + s;
    f.f[s] = *reinterpret_cast<const bf16x8*>(ks + key * 128 + ((c ^ (key & 7)) << 3));
  }
}
template <>
__device__ __forceinline__ void lds_k_frag<__bf16, 64>(const __bf16* ks, int key, int hf, HalfRow<__bf16, 64>& f) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = hf * 4 + s;
    f.f[s] = *reinterpret_cast<const bf16x8*>(ks + key * 64 + ((c ^ (key & 7)) << 3));
  }
}
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

template <int D, int NT> struct Stage<__bf16, D, NT> {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int KCH = BN * CPR / NT;          // K chunks per thread
  static constexpr int VUNITS = (BN / 2) * CPR;      // (2-key pair, chunk) units of V
  static constexpr int VPT = (VUNITS + NT - 1) / NT; // V units per thread
  u32x4 kr[KCH];
  u32x4 vr[VPT][2];

  __device__ __forceinline__ void load(const __bf16* kbase, const __bf16* vbase, int64_t rstride, int k0, int n,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int e = tid + NT * i;
      const int key = e / CPR, c = e % CPR;
      const int j = min(k0 + key, n - 1);
      kr[i] = ld16(kbase + (int64_t)j * rstride + c * 8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int un = tid + NT * i;
      if (VUNITS % NT == 0 || un < VUNITS) {
        const int a = un / CPR, c = un % CPR;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = min(k0 + 2 * a + u, n - 1);
          vr[i][u] = ld16(vbase + (int64_t)j * rstride + c * 8);
        }
      }
    }
  }

  __device__ __forceinline__ void store(AttnLds<__bf16, D>& L, int buf, int tid) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int e = tid + NT * i;
      const int key = e / CPR, c = e % CPR;
      *reinterpret_cast<u32x4*>(&L.k[buf][key * D + ((c ^ (key & 7)) << 3)]) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int un = tid + NT * i;
      if (VUNITS % NT == 0 || un < VUNITS) {
        const int a = un / CPR, c = un % CPR;
        const int pos = vt_pos(2 * a);                 // keys 2a, 2a+1 occupy pos, pos+1
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int d = c * 8 + dd;
          const uint32_t w0 = vr[i][0][dd >> 1], w1 = vr[i][1][dd >> 1];
          // low halves (even dd) or high halves (odd dd) of the two keys, packed
          const uint32_t packed = (dd & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                                           : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
          const int off = d * BN + ((((pos >> 3) ^ vt_swz(d))) << 3) + (pos & 7);
          *reinterpret_cast<uint32_t*>(&L.vt[buf][off]) = packed;
        }
      }
    }
  }
};

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
__device__ __forceinline__ void pv_tile(const AttnLds<__bf16, D>& L, int buf, int lane,
                                        const f32x16 (&s)[KB][QB], f32x16 (&o)[QB][D / 32]) {
  const int hf = lane >> 5, lc = lane & 31;
  // Probabilities as bf16 B operands: k-step (kb, jj) uses accumulator slots 8jj..8jj+7.
  bf16x8 pf[QB][KB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int u = 0; u < 8; ++u) pf[qb][kb][jj][u] = static_cast<__bf16>(s[kb][qb][8 * jj + u]);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int d = db * 32 + lc;
    const __bf16* row = &L.vt[buf][d * BN];
    const int sw = vt_swz(d);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int chunk = 2 * (2 * kb + jj) + hf;
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(row + ((chunk ^ sw) << 3));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma(o[qb][db], vf, pf[qb][kb][jj]);
      }
  }
}

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
  if (!DENSE) {
    p.q_r = p.k_r = p.o_r = D;
    p.kv_div = 1;
  }
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
      bh = x * hpx + sl % hpx;
      tile = p.ntiles - 1 - sl / hpx;
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
    if (d.d == 128) return launch_attn_t<__bf16, 128, 1, 8, DENSE>(p, d.B, d.H, s);
    if (d.d == 64) return launch_attn_t<__bf16, 64, 1, 8, DENSE>(p, d.B, d.H, s);
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
  p.kv_div = 1;
  p.q_r = d.d; p.q_h = (int64_t)d.keep * d.d; p.q_b = (int64_t)d.H * d.keep * d.d;
  p.k_r = p.q_r; p.k_h = p.q_h; p.k_b = p.q_b;
  p.o_r = p.q_r; p.o_h = p.q_h; p.o_b = p.q_b;
  p.c = attn_c(d);
  return dispatch_attn<false>(d, p, s);
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
