// Small memory-bound kernels around the GEMMs: folding the RMSNorm gain into
// the down weights, recomputing the bottleneck activation from the saved
// fp32 H, and the fixed-order reductions of per-tile partials.
#pragma once

#include "gemm.hpp"
#include "epilogues.hpp"

namespace rbo {

// out[k][n] = g[k] * A[k][n], rounded once to the storage dtype. The gain of
// RMSNorm multiplies the reduction index of the down product, so scaling
// the weight rows is the same product as scaling the input columns.
template <typename T>
__global__ __launch_bounds__(256) void gain_fold_kernel(const T* __restrict__ A, const T* __restrict__ g,
                                                        T* __restrict__ out, int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = i / cols;
    Elem<T>::store(out, i, Elem<T>::load(g, k) * Elem<T>::load(A, i));
  }
}

// Vectorised bf16 variant: 8 elements per thread per step (cols % 8 == 0).
__global__ __launch_bounds__(256) void gain_fold_bf16x8_kernel(const u32x4* __restrict__ A,
                                                               const uint16_t* __restrict__ g,
                                                               u32x4* __restrict__ out, int64_t rows,
                                                               int64_t cols) {
  const int64_t n8 = rows * cols / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = (i * 8) / cols;
    const float gk = Elem<bf16>::to_f32(g[k]);
    const u32x4 v = A[i];
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = gk * __uint_as_float(v[w] << 16);
      const float hi = gk * __uint_as_float(v[w] & 0xffff0000u);
      bf16x2 p;
      p[0] = static_cast<bf16>(lo);
      p[1] = static_cast<bf16>(hi);
      o[w] = __builtin_bit_cast(uint32_t, p);
    }
    out[i] = o;
  }
}

// S = act(H) in the storage dtype (bottleneck activation recompute).
template <typename T>
__global__ __launch_bounds__(256) void act_quant_kernel(const float* __restrict__ H, T* __restrict__ S,
                                                        int64_t n, int act) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    Elem<T>::store(S, i, act_f(H[i], act));
}

__global__ __launch_bounds__(256) void act_quant_bf16x8_kernel(const float4* __restrict__ H,
                                                               u32x4* __restrict__ S, int64_t n8,
                                                               int act) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float4 a = H[2 * i], b = H[2 * i + 1];
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      bf16x2 p;
      p[0] = static_cast<bf16>(act_f(f[2 * w], act));
      p[1] = static_cast<bf16>(act_f(f[2 * w + 1], act));
      o[w] = __builtin_bit_cast(uint32_t, p);
    }
    S[i] = o;
  }
}

// out[n] = sum_{p < P} part[p * stride + n], in order p = 0, 1, ...
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ part, int P, int64_t stride,
                                                     int64_t N, float* __restrict__ out) {
  for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < N;
       n += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int p = 0; p < P; ++p) s += part[(int64_t)p * stride + n];
    out[n] = s;
  }
}

// Split-K reduction: part is [batch][S][MN]; out[b][e] = rowscale[e / cols] *
// sum_s part[b][s][e] (sum in order s = 0, 1, ...), fp32.
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float4* __restrict__ part, int S,
                                                            int64_t mn4, int batch, const T* rowscale,
                                                            int64_t cols, float4* __restrict__ out) {
  const int64_t total = mn4 * batch;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / mn4, e = i - b * mn4;
    const float4* p = part + b * S * mn4 + e;
    float4 s = p[0];
    for (int k = 1; k < S; ++k) {
      const float4 q = p[(int64_t)k * mn4];
      s.x += q.x; s.y += q.y; s.z += q.z; s.w += q.w;
    }
    if (rowscale) {
      const float rs = Elem<T>::load(rowscale, (e * 4) / cols);
      s.x *= rs; s.y *= rs; s.z *= rs; s.w *= rs;
    }
    out[i] = s;
  }
}

}  // namespace rbo
