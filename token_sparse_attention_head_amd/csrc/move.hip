// Data-movement kernels: gather-compression of Q/K/V into the compact per-head tensors
// and scatter-decompression of the attention output with the residual added.
//
// Gather follows the skill page "Token Sparse Attention Long Context", Step 2 (rows of
// the selected tokens copied into a dense block), and the paper page "Token Sparse
// Attention: Efficient Long-Context Inference with Interleaved Token Selection",
// Figure 3, stage 1 (per-head compact Q, K, V).  Scatter follows the same Step 2
// (outputs put back at their original positions, zeros elsewhere) and Figure 3,
// stage 2 (scatter into the full layout, then add the residual).
//
// Every thread moves 16-byte vectors; one row of d elements is 128-512 bytes, so a
// wave reads and writes whole 128-byte lines.  Kept rows are read once per query head;
// the out-of-place scatter streams residual and out once in memory order.  An index
// entry outside [0, L) (the -1 padding of rows below an adaptive budget) moves nothing:
// gather writes zero rows for it and scatter skips it.
#include "common.h"
#include "kernels.h"

namespace tsa {

namespace {

// SG query heads share a subset (1 per head, G per KV head): head h reads idx row
// b * (H / SG) + h / SG; the first head of each subset also writes the subset's K/V rows.
template <int ROWB>
__global__ __launch_bounds__(256) void gather_qkv_kernel(const char* __restrict__ q, const char* __restrict__ k,
                                                         const char* __restrict__ v, const int32_t* __restrict__ idx,
                                                         char* __restrict__ qh, char* __restrict__ kh,
                                                         char* __restrict__ vh, int H, int G, int SG, int L,
                                                         int keep) {
  constexpr int CH = ROWB / 16;
  const int bh = blockIdx.y;                  // b * H + h
  const uint32_t e = blockIdx.x * 256u + threadIdx.x;
  const int t = e / CH;
  const int c = e % CH;
  if (t >= keep) return;
  const int h = bh % H;
  const int64_t b = bh / H;
  const int Hkv = H / G;
  const int64_t srow = (b * (H / SG) + h / SG) * keep + t;   // row of the subset
  const int p = idx[srow];
  if ((unsigned)p >= (unsigned)L) {
    // Padding entry (-1 past a row's adaptive budget): zero rows.
    const u32x4 z = {0u, 0u, 0u, 0u};
    st16(qh + ((int64_t)bh * keep + t) * ROWB + c * 16, z);
    if (h % SG != 0) return;
    st16(kh + srow * ROWB + c * 16, z);
    st16(vh + srow * ROWB + c * 16, z);
    return;
  }
  const int64_t qoff = ((b * L + p) * H + h) * ROWB + c * 16;
  st16(qh + ((int64_t)bh * keep + t) * ROWB + c * 16, ld16(q + qoff));
  if (h % SG != 0) return;
  const int64_t kvoff = ((b * L + p) * Hkv + h / G) * ROWB + c * 16;
  const u32x4 kk = ld16(k + kvoff);
  const u32x4 vv = ld16(v + kvoff);
  st16(kh + srow * ROWB + c * 16, kk);
  st16(vh + srow * ROWB + c * 16, vv);
}

// 16 bytes of residual plus 16 bytes of attention output, summed in fp32, rounded once.
__device__ __forceinline__ u32x4 add_rows(u32x4 r, u32x4 o, tsa_dtype dt) {
  u32x4 out;
  if (dt == TSA_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = bf16_to_f32(r[i] & 0xFFFFu) + bf16_to_f32(o[i] & 0xFFFFu);
      const float hi = bf16_to_f32(r[i] >> 16) + bf16_to_f32(o[i] >> 16);
      out[i] = pack_bf16x2(lo, hi);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __float_as_uint(__uint_as_float(r[i]) + __uint_as_float(o[i]));
  }
  return out;
}

// Out-of-place: one pass over [B][L][H] rows in memory order.  inv[b][r][p] is the
// compact row of position p in subset r, or -1; head h uses subset h / SG.
template <int ROWB, tsa_dtype DT>
__global__ __launch_bounds__(256) void scatter_residual_kernel(const char* __restrict__ oh,
                                                               const int32_t* __restrict__ inv,
                                                               const char* __restrict__ res, char* __restrict__ out,
                                                               int H, int SG, int L, int keep) {
  constexpr int CH = ROWB / 16;
  const int64_t b = blockIdx.y;
  const uint32_t e = blockIdx.x * 256u + threadIdx.x;
  const uint32_t row = e / CH;                // p * H + h
  const int c = e % CH;
  if (row >= (uint32_t)L * (uint32_t)H) return;
  const int p = row / H;
  const int h = row % H;
  const int64_t off = ((b * L + p) * H + h) * ROWB + c * 16;
  const int t = inv[(b * (H / SG) + h / SG) * L + p];
  const u32x4 r = ld16_nt(res + off);
  u32x4 o = r;
  if (t >= 0) o = add_rows(r, ld16(oh + (((b * H + h) * keep + t) * ROWB + c * 16)), DT);
  st16_nt(out + off, o);
}

// In place (out == residual): only the kept rows are read and rewritten.
template <int ROWB, tsa_dtype DT>
__global__ __launch_bounds__(256) void scatter_add_inplace_kernel(const char* __restrict__ oh,
                                                                  const int32_t* __restrict__ idx, char* out, int H,
                                                                  int SG, int L, int keep) {
  constexpr int CH = ROWB / 16;
  const int bh = blockIdx.y;
  const uint32_t e = blockIdx.x * 256u + threadIdx.x;
  const int t = e / CH;
  const int c = e % CH;
  if (t >= keep) return;
  const int h = bh % H;
  const int64_t b = bh / H;
  const int64_t crow = (int64_t)bh * keep + t;
  const int p = idx[(b * (H / SG) + h / SG) * keep + t];
  if ((unsigned)p >= (unsigned)L) return;       // padding entry
  char* dst = out + ((b * L + p) * H + h) * ROWB + c * 16;
  st16(dst, add_rows(ld16(dst), ld16(oh + crow * ROWB + c * 16), DT));
}

// Out of place, fused forward: the residual rows no head keeps, copied to out (the kept
// rows are written by the attention epilogue).  A workgroup takes CU_ROWS consecutive
// rows of one batch entry in memory order (row = p * H + h), reads their inverse-map
// entries, lists the unkept rows in LDS in memory order, then copies the listed rows
// 16 bytes per lane with CU_UNROLL loads in flight per lane: every lane has work whatever
// the keep ratio.  (Measured on one MI355X for half of 4M random 256-byte rows: 5.1-5.3
// TB/s for 4 to 16 loads in flight, 4.4 TB/s with one masked lane per vector.)
constexpr int CU_THREADS = 256;
constexpr int CU_ROWS = 1024;
constexpr int CU_UNROLL = 16;

template <int ROWB>
__global__ __launch_bounds__(CU_THREADS) void copy_unkept_kernel(const int32_t* __restrict__ inv,
                                                                 const char* __restrict__ res,
                                                                 char* __restrict__ out, int H, int SG, int L) {
  constexpr int CH = ROWB / 16;
  constexpr int WAVES = CU_THREADS / TSA_WAVE;
  __shared__ uint16_t list[CU_ROWS];
  __shared__ uint32_t wave_n[CU_ROWS / TSA_WAVE];
  const int64_t b = blockIdx.y;
  const uint32_t nrows = (uint32_t)L * (uint32_t)H;
  const uint32_t r0 = blockIdx.x * (uint32_t)CU_ROWS;
  const int lane = lane_id(), wave = threadIdx.x / TSA_WAVE;
  const int32_t* inv_b = inv + b * (H / SG) * (int64_t)L;
  bool unkept[CU_ROWS / CU_THREADS];
#pragma unroll
  for (int k = 0; k < CU_ROWS / CU_THREADS; ++k) {
    const uint32_t row = r0 + k * CU_THREADS + threadIdx.x;
    bool u = false;
    if (row < nrows) {
      const uint32_t p = row / H, h = row % H;
      u = inv_b[(int64_t)(h / SG) * L + p] < 0;
    }
    unkept[k] = u;
    const uint64_t m = __ballot(u);
    if (lane == 0) wave_n[k * WAVES + wave] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  // Exclusive prefix over the groups (k, wave) in memory order; every lane sums the few
  // group counts before its own.
  uint32_t total = 0;
#pragma unroll
  for (int k = 0; k < CU_ROWS / CU_THREADS; ++k) {
    const int grp = k * WAVES + wave;
    uint32_t before = 0;
    for (int q = 0; q < grp; ++q) before += wave_n[q];
    const uint64_t m = __ballot(unkept[k]);
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (unkept[k]) list[before + rank] = (uint16_t)(k * CU_THREADS + threadIdx.x);
  }
  for (int q = 0; q < CU_ROWS / TSA_WAVE; ++q) total += wave_n[q];
  __syncthreads();
  const uint32_t nchunks = total * CH;
  const int64_t base = ((int64_t)b * nrows + r0) * ROWB;
  for (uint32_t e0 = 0; e0 < nchunks; e0 += CU_THREADS * CU_UNROLL) {
    u32x4 v[CU_UNROLL];
    int64_t off[CU_UNROLL];
#pragma unroll
    for (int i = 0; i < CU_UNROLL; ++i) {
      const uint32_t e = e0 + i * CU_THREADS + threadIdx.x;
      off[i] = e < nchunks ? base + (int64_t)list[e / CH] * ROWB + (e % CH) * 16 : -1;
      if (off[i] >= 0) v[i] = ld16_nt(res + off[i]);
    }
#pragma unroll
    for (int i = 0; i < CU_UNROLL; ++i)
      if (off[i] >= 0) st16_nt(out + off[i], v[i]);
  }
}

// Plain device copy of n16 16-byte vectors, one vector per lane, consecutive lanes on
// consecutive vectors, non-temporal: the bandwidth reference the data-movement kernels are
// measured against.  (Measured on one MI355X for 1 GiB: 6.5 TB/s; the same copy with 2, 4, 8
// or 16 vectors in flight per lane, strided or blocked, ran 4.3-6.2 TB/s.)
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          int64_t n16) {
  const int64_t e = blockIdx.x * 256ll + threadIdx.x;
  if (e < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + e), dst + e);
}

// Rows of each subset from an index list written by the select: idx rows hold the kept
// positions (>= 0) and then -1 padding, so the count is the first negative entry
// (binary search), keep when there is none.
__global__ __launch_bounds__(256) void row_count_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ counts,
                                                        int rows, int keep) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int32_t* row = idx + (int64_t)r * keep;
  int lo = 0, hi = keep;            // first t in [lo, hi] with row[t] < 0 (hi = keep: none)
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] < 0) hi = mid; else lo = mid + 1;
  }
  counts[r] = lo;
}

__global__ __launch_bounds__(256) void fill_kernel(int32_t* __restrict__ p, int64_t n, int32_t value) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = value;
}

__global__ __launch_bounds__(256) void invert_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ inv,
                                                     int L, int keep) {
  const int bh = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= keep) return;
  const int p = idx[(int64_t)bh * keep + t];
  if ((unsigned)p < (unsigned)L) inv[(int64_t)bh * L + p] = t;   // padding entries map nothing
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

#define TSA_ROWB_DISPATCH(ROWB_VAL, ...)            \
  switch (ROWB_VAL) {                               \
    case 128: { constexpr int RB = 128; __VA_ARGS__; break; } \
    case 256: { constexpr int RB = 256; __VA_ARGS__; break; } \
    case 512: { constexpr int RB = 512; __VA_ARGS__; break; } \
    default: return hipErrorInvalidValue;           \
  }

hipError_t launch_gather_qkv(const tsa_desc& d, const void* q, const void* k, const void* v, const int32_t* idx,
                             void* qh, void* kh, void* vh, hipStream_t s) {
  const int rowb = d.d * (d.dtype == TSA_BF16 ? 2 : 4);
  const dim3 grid(blocks_for((int64_t)d.keep * (rowb / 16)), d.B * d.H);
  TSA_ROWB_DISPATCH(rowb, gather_qkv_kernel<RB><<<grid, 256, 0, s>>>(
                              (const char*)q, (const char*)k, (const char*)v, idx, (char*)qh, (char*)kh, (char*)vh,
                              d.H, d.H / d.Hkv, heads_per_subset(d), d.L, d.keep));
  return hipGetLastError();
}

hipError_t launch_build_inverse(const tsa_desc& d, const int32_t* idx, int32_t* inv, hipStream_t s) {
  const int64_t n = (int64_t)d.B * subset_rows(d) * d.L;
  const unsigned fb = (unsigned)std::min<int64_t>(blocks_for(n), 4096);
  fill_kernel<<<fb, 256, 0, s>>>(inv, n, -1);
  invert_kernel<<<dim3(blocks_for(d.keep), d.B * subset_rows(d)), 256, 0, s>>>(idx, inv, d.L, d.keep);
  return hipGetLastError();
}

hipError_t launch_scatter_residual(const tsa_desc& d, const void* oh, const int32_t* inv, const void* res, void* out,
                                   hipStream_t s) {
  const int rowb = d.d * (d.dtype == TSA_BF16 ? 2 : 4);
  const dim3 grid(blocks_for((int64_t)d.L * d.H * (rowb / 16)), d.B);
  if (d.dtype == TSA_BF16) {
    TSA_ROWB_DISPATCH(rowb, scatter_residual_kernel<RB, TSA_BF16><<<grid, 256, 0, s>>>(
                                (const char*)oh, inv, (const char*)res, (char*)out, d.H, heads_per_subset(d), d.L,
                                d.keep));
  } else {
    TSA_ROWB_DISPATCH(rowb, scatter_residual_kernel<RB, TSA_F32><<<grid, 256, 0, s>>>(
                                (const char*)oh, inv, (const char*)res, (char*)out, d.H, heads_per_subset(d), d.L,
                                d.keep));
  }
  return hipGetLastError();
}

hipError_t launch_copy_unselected(const tsa_desc& d, const int32_t* inv, const void* res, void* out, hipStream_t s) {
  const int rowb = d.d * (d.dtype == TSA_BF16 ? 2 : 4);
  const dim3 grid((unsigned)(((int64_t)d.L * d.H + CU_ROWS - 1) / CU_ROWS), d.B);
  TSA_ROWB_DISPATCH(rowb, copy_unkept_kernel<RB><<<grid, CU_THREADS, 0, s>>>(
                              inv, (const char*)res, (char*)out, d.H, heads_per_subset(d), d.L));
  return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  constexpr int64_t kPiece = (int64_t)1 << 30;      // vectors per launch (keeps the grid below 2^22 blocks)
  for (int64_t o = 0; o < n16; o += kPiece) {
    const int64_t n = std::min(kPiece, n16 - o);
    stream_copy_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<const u32x4*>(src) + o,
                                                                  static_cast<u32x4*>(dst) + o, n);
  }
  return hipGetLastError();
}

hipError_t launch_row_counts(const tsa_desc& d, const int32_t* idx, int32_t* counts, hipStream_t s) {
  const int rows = d.B * subset_rows(d);
  row_count_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(idx, counts, rows, d.keep);
  return hipGetLastError();
}

hipError_t launch_scatter_inplace(const tsa_desc& d, const void* oh, const int32_t* idx, void* out, hipStream_t s) {
  const int rowb = d.d * (d.dtype == TSA_BF16 ? 2 : 4);
  const dim3 grid(blocks_for((int64_t)d.keep * (rowb / 16)), d.B * d.H);
  if (d.dtype == TSA_BF16) {
    TSA_ROWB_DISPATCH(rowb, scatter_add_inplace_kernel<RB, TSA_BF16><<<grid, 256, 0, s>>>(
                                (const char*)oh, idx, (char*)out, d.H, heads_per_subset(d), d.L, d.keep));
  } else {
    TSA_ROWB_DISPATCH(rowb, scatter_add_inplace_kernel<RB, TSA_F32><<<grid, 256, 0, s>>>(
                                (const char*)oh, idx, (char*)out, d.H, heads_per_subset(d), d.L, d.keep));
  }
  return hipGetLastError();
}

}  // namespace tsa
