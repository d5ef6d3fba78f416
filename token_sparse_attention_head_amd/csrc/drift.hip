// Representation drift between a layer's input and output hidden states.
//
// The skill page "Token Sparse Attention Long Context", Step 4, scores how much a layer
// changes its hidden states as one minus the mean, over tokens, of the cosine between
// each token's normalised vector before and after the layer (a vector is divided by the
// larger of its norm and 1e-12); stable layers are where token selection can be
// aggressive.  The paper page's Figure 4 plots this drift per layer.
//
//   drift = 1 - (1/T) sum_t <a_t, b_t> / (max(|a_t|, eps) max(|b_t|, eps))
//
// Bandwidth bound: both tensors are read once (2 T D e bytes).  One wave per token row at
// a time: every lane loads strided 16-byte chunks of both rows (several in flight), sums
// a.b, a.a and b.b in fp32, and a butterfly over the wave completes the sums; the cosine
// is formed in fp32 and added in fp64 to the wave's running sum, tokens in a fixed order.
// The grid depends only on T, and the partial sums are folded in a fixed order, so the
// result is deterministic.
#include "common.h"
#include "kernels.h"

namespace tsa {

namespace {

constexpr int DR_WG = 256;
constexpr int DR_WAVES = DR_WG / TSA_WAVE;
constexpr int DR_UNROLL = 4;        // chunks per lane per tensor in flight
constexpr int DR_MAX_BLOCKS = 2048;
constexpr float DR_EPS = 1e-12f;

template <tsa_dtype DT>
__device__ __forceinline__ void dot3(const u32x4& x, const u32x4& y, float& xy, float& xx, float& yy) {
  if (DT == TSA_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = bf16_to_f32(x[i] & 0xFFFFu), x1 = bf16_to_f32(x[i] >> 16);
      const float y0 = bf16_to_f32(y[i] & 0xFFFFu), y1 = bf16_to_f32(y[i] >> 16);
      xy = __builtin_fmaf(x0, y0, xy);
      xy = __builtin_fmaf(x1, y1, xy);
      xx = __builtin_fmaf(x0, x0, xx);
      xx = __builtin_fmaf(x1, x1, xx);
      yy = __builtin_fmaf(y0, y0, yy);
      yy = __builtin_fmaf(y1, y1, yy);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = __uint_as_float(x[i]), y0 = __uint_as_float(y[i]);
      xy = __builtin_fmaf(x0, y0, xy);
      xx = __builtin_fmaf(x0, x0, xx);
      yy = __builtin_fmaf(y0, y0, yy);
    }
  }
}

template <tsa_dtype DT>
__global__ __launch_bounds__(DR_WG) void drift_partial_kernel(const char* __restrict__ a, const char* __restrict__ b,
                                                              int64_t tokens, int chunks, double* __restrict__ partial) {
  __shared__ double wave_sum[DR_WAVES];
  const int lane = lane_id();
  const int wave = threadIdx.x / TSA_WAVE;
  const int64_t stride = (int64_t)gridDim.x * DR_WAVES;
  const int64_t row_bytes = (int64_t)chunks * 16;
  double acc = 0.0;
  for (int64_t t = (int64_t)blockIdx.x * DR_WAVES + wave; t < tokens; t += stride) {
    const char* ra = a + t * row_bytes;
    const char* rb = b + t * row_bytes;
    float xy = 0.f, xx = 0.f, yy = 0.f;
    for (int c0 = lane; c0 < chunks; c0 += DR_UNROLL * TSA_WAVE) {
      u32x4 va[DR_UNROLL], vb[DR_UNROLL];
#pragma unroll
      for (int k = 0; k < DR_UNROLL; ++k) {
        const int c = c0 + k * TSA_WAVE;
        const bool in = c < chunks;
        va[k] = in ? ld16_nt(ra + (int64_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
        vb[k] = in ? ld16_nt(rb + (int64_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int k = 0; k < DR_UNROLL; ++k) dot3<DT>(va[k], vb[k], xy, xx, yy);
    }
#pragma unroll
    for (int o = TSA_WAVE / 2; o > 0; o >>= 1) {
      xy += __shfl_xor(xy, o, TSA_WAVE);
      xx += __shfl_xor(xx, o, TSA_WAVE);
      yy += __shfl_xor(yy, o, TSA_WAVE);
    }
    const float cosv = xy / (fmaxf(__builtin_sqrtf(xx), DR_EPS) * fmaxf(__builtin_sqrtf(yy), DR_EPS));
    acc += (double)cosv;
  }
  if (lane == 0) wave_sum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int w = 0; w < DR_WAVES; ++w) s += wave_sum[w];
    partial[blockIdx.x] = s;
  }
}

__global__ __launch_bounds__(DR_WG) void drift_final_kernel(const double* __restrict__ partial, int n,
                                                            int64_t tokens, double* __restrict__ out) {
  __shared__ double part[DR_WG];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += DR_WG) s += partial[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = DR_WG / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = 1.0 - part[0] / (double)tokens;
}

int drift_blocks(int64_t tokens) {
  const int64_t want = (tokens + DR_WAVES - 1) / DR_WAVES;
  return (int)(want < DR_MAX_BLOCKS ? want : DR_MAX_BLOCKS);
}

}  // namespace

size_t drift_workspace_bytes(const tsa_desc& d) {
  const int64_t tokens = (int64_t)d.B * d.L;
  return tokens > 0 ? (size_t)drift_blocks(tokens) * sizeof(double) : 0;
}

hipError_t launch_drift(const tsa_desc& d, const void* a, const void* b, double* out, double* partial,
                        hipStream_t s) {
  const int64_t tokens = (int64_t)d.B * d.L;
  const int chunks = (int)((int64_t)d.H * d.d * (d.dtype == TSA_BF16 ? 2 : 4) / 16);
  const int blocks = drift_blocks(tokens);
  if (d.dtype == TSA_BF16)
    drift_partial_kernel<TSA_BF16><<<blocks, DR_WG, 0, s>>>((const char*)a, (const char*)b, tokens, chunks, partial);
  else
    drift_partial_kernel<TSA_F32><<<blocks, DR_WG, 0, s>>>((const char*)a, (const char*)b, tokens, chunks, partial);
  drift_final_kernel<<<1, DR_WG, 0, s>>>(partial, blocks, tokens, out);
  return hipGetLastError();
}

}  // namespace tsa
