// Small memory-bound kernels around the GEMMs: transposing weights into the
// K-contiguous operand layout (folding the RMSNorm gain into the down
// weights on the way), recomputing the bottleneck activation from the saved
// fp32 H, and the fixed-order reductions of per-tile partials.
#pragma once

#include "gemm.hpp"
#include "epilogues.hpp"

namespace rbo {

// out[b][c][r] = scale[r] * in[b][r][c], rounded once to the storage dtype
// (scale may be null). Turns a weight kept in [in, out] layout into the
// K-contiguous [out, in] operand of the products; with the RMSNorm gain as
// the scale it also folds the gain into the down weights. 64 x 64 tiles
// through LDS, 16-byte global accesses on both sides. R, C multiples of 64.
template <typename T>
__global__ __launch_bounds__(256) void transpose_scale_kernel(const T* __restrict__ in, const T* __restrict__ scale,
                                                              T* __restrict__ out, int R, int C) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float tile[64][65];
  const int tr = blockIdx.y * 64, tc = blockIdx.x * 64, b = blockIdx.z;
  const T* src = in + (int64_t)b * R * C;
  T* dst = out + (int64_t)b * R * C;
  const int t = threadIdx.x;
  for (int q = t; q < 64 * 64 / VEC; q += 256) {
    const int r = q / (64 / VEC), c = (q % (64 / VEC)) * VEC;
    float v[8];
    if constexpr (VEC == 8) {
      Vec8<bf16>::load(src, (int64_t)(tr + r) * C + tc + c, v);
    } else {
      const float4 f = *reinterpret_cast<const float4*>(src + (int64_t)(tr + r) * C + tc + c);
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
    const float sc = scale ? Elem<T>::load(scale, tr + r) : 1.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) tile[r][c + e] = sc * v[e];
  }
  __syncthreads();
  for (int q = t; q < 64 * 64 / VEC; q += 256) {
    const int c = q / (64 / VEC), r = (q % (64 / VEC)) * VEC;
    float v[8];
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = tile[r + e][c];
    if constexpr (VEC == 8) {
      Vec8<bf16>::store(dst, (int64_t)(tc + c) * R + tr + r, v);
    } else {
      *reinterpret_cast<float4*>(dst + (int64_t)(tc + c) * R + tr + r) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Several bf16 weight transposes in one launch: job j turns in[b][r][c]
// (R x C per batch) into out[b][c][r] = round(scale[r] * in[b][r][c]) (no
// rounding when scale is null: the values are copied). Each workgroup
// transposes a 128 x 64 block of one job: every thread loads two pairs of
// vertically adjacent 16-byte row segments (four loads in flight), packs
// the two rows of each column into one 32-bit word (the two neighbouring
// elements of an output row) and writes the words to an LDS tile indexed
// [column][row pair]; each thread then reads four consecutive words (eight
// output elements) and stores them as one 16-byte vector. The tile row
// stride of 65 words keeps both the word writes and reads free of bank
// conflicts. R and C are multiples of 64; rows of a block past R are
// skipped.
struct TransposeJob {
  const bf16* in;
  const bf16* scale;  // per input row, or null
  bf16* out;
  int R, C;
  int tiles_r, tiles_c;  // blocks per batch: ceil(R / 128) x C / 64
  int first;             // first block index of this job
};
constexpr int kMaxTransposeJobs = 4;
struct TransposeJobs {
  TransposeJob j[kMaxTransposeJobs];
  int n;
};

__global__ __launch_bounds__(256) void transpose_bf16_kernel(TransposeJobs jobs) {
  constexpr int TS = 65;  // words per tile row
  __shared__ uint32_t tile[64 * TS];
  // The job is picked field by field with compile-time indices (a runtime
  // index into the argument array would copy it to scratch memory).
  TransposeJob J = jobs.j[0];
#pragma unroll
  for (int q = 1; q < kMaxTransposeJobs; ++q)
    if (q < jobs.n && (int)blockIdx.x >= jobs.j[q].first) J = jobs.j[q];
  const int local = (int)blockIdx.x - J.first;
  const int per_batch = J.tiles_r * J.tiles_c;
  const int b = local / per_batch, rem = local - b * per_batch;
  const int tr = (rem / J.tiles_c) * 128, tc = (rem % J.tiles_c) * 64;
  const bf16* src = J.in + (int64_t)b * J.R * J.C;
  bf16* dst = J.out + (int64_t)b * J.R * J.C;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  // Load: item (pair p, column chunk c8) covers input rows 2p, 2p+1 and
  // columns c8 .. c8+7 of the block; a wave's 64 lanes take 8 pairs x 8
  // chunks, so each input row segment read is a full 128-byte line.
  float v[2][2][8];
  int pr[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int p = 8 * (wave + 4 * q) + (lane >> 3), c8 = (lane & 7) * 8;
    pr[q] = p;
    const int r0 = tr + 2 * p;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (r0 < J.R) {
        Vec8<bf16>::load(src, (int64_t)(r0 + h) * J.C + tc + c8, v[q][h]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q][h][e] = 0.f;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int p = pr[q], c8 = (lane & 7) * 8, r0 = tr + 2 * p;
    float sc0 = 1.f, sc1 = 1.f;
    if (J.scale && r0 < J.R) {
      sc0 = Elem<bf16>::load(J.scale, r0);
      sc1 = Elem<bf16>::load(J.scale, r0 + 1);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x2 w;
      w[0] = static_cast<bf16>(sc0 * v[q][0][e]);
      w[1] = static_cast<bf16>(sc1 * v[q][1][e]);
      tile[(c8 + e) * TS + p] = __builtin_bit_cast(uint32_t, w);
    }
  }
  __syncthreads();
  // Store: vector (column oc, pair group p4) = output row tc + oc, output
  // columns tr + 8 p4 .. +7; 16 lanes cover one 256-byte output row segment.
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = t + 256 * q;
    const int oc = i >> 4, p4 = i & 15;
    const int col = tr + 8 * p4;
    if (col < J.R) {
      u32x4 o;
      const uint32_t* w = tile + oc * TS + 4 * p4;
      o.x = w[0]; o.y = w[1]; o.z = w[2]; o.w = w[3];
      *reinterpret_cast<u32x4*>(dst + (int64_t)(tc + oc) * J.R + col) = o;
    }
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

// out[n] = sum_{p < P} part[p * stride + n] in a fixed order: each of four
// threads of a column sums a contiguous quarter of the partials in order,
// and the four quarter sums are added in order 0, 1, 2, 3. A workgroup
// covers 64 columns, so the grid spans N / 64 workgroups and each thread
// has about P / 4 independent loads in flight.
constexpr int kColsumCols = 64;
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ part, int P, int64_t stride,
                                                     int64_t N, float* __restrict__ out) {
  __shared__ float q[4][kColsumCols];
  const int c = threadIdx.x & (kColsumCols - 1), h = threadIdx.x / kColsumCols;
  const int64_t n = (int64_t)blockIdx.x * kColsumCols + c;
  const int p0 = (h * P) / 4, p1 = ((h + 1) * P) / 4;
  float s = 0.f;
  if (n < N)
    for (int p = p0; p < p1; ++p) s += part[(int64_t)p * stride + n];
  q[h][c] = s;
  __syncthreads();
  if (h == 0 && n < N) out[n] = ((q[0][c] + q[1][c]) + q[2][c]) + q[3][c];
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

// Attention stand-in (the attention core is not part of the block): a =
// q + k + v elementwise over qkv[3][n], and its gradient, dq = dk = dv = da.
// The sum is taken in fp64, where it is exact for any three bf16 values
// within 2^43 of each other (an fp32 sum of two of them first is not: it
// rounds when their exponents differ by more than 16), then rounded to fp32
// and stored like every other fp32 result (bf16: round to nearest even from
// that fp32 value). The bf16 rounding is done on the fp32 bits: a plain
// conversion chain double -> float -> bf16 is compiled into one rounding
// straight from the double, which differs where the fp32 value is a bf16
// tie. Finite values. n is a multiple of 8; 16-byte accesses.
template <typename T>
__global__ __launch_bounds__(256) void standin_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ a, int64_t n) {
  constexpr int VEC = 16 / sizeof(T);
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * VEC; i < n;
       i += (int64_t)gridDim.x * blockDim.x * VEC) {
    float q[8], k[8], v[8];
    if constexpr (VEC == 8) {
      Vec8<bf16>::load(qkv, i, q);
      Vec8<bf16>::load(qkv, n + i, k);
      Vec8<bf16>::load(qkv, 2 * n + i, v);
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)((double)q[e] + (double)k[e] + (double)v[e]);
        const uint32_t b = __builtin_bit_cast(uint32_t, f);
        h[e] = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
      }
      *reinterpret_cast<u32x4*>(a + i) =
          u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    } else {
      const float4 x = *reinterpret_cast<const float4*>(qkv + i);
      const float4 y = *reinterpret_cast<const float4*>(qkv + n + i);
      const float4 z = *reinterpret_cast<const float4*>(qkv + 2 * n + i);
      auto sum3 = [](float p, float q, float r) { return (float)((double)p + (double)q + (double)r); };
      *reinterpret_cast<float4*>(a + i) =
          make_float4(sum3(x.x, y.x, z.x), sum3(x.y, y.y, z.y), sum3(x.z, y.z, z.z), sum3(x.w, y.w, z.w));
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void standin_bwd_kernel(const T* __restrict__ da, T* __restrict__ dqkv, int64_t n) {
  constexpr int VEC = 16 / sizeof(T);
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * VEC; i < n;
       i += (int64_t)gridDim.x * blockDim.x * VEC) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(da + i);
    *reinterpret_cast<u32x4*>(dqkv + i) = w;
    *reinterpret_cast<u32x4*>(dqkv + n + i) = w;
    *reinterpret_cast<u32x4*>(dqkv + 2 * n + i) = w;
  }
}

}  // namespace rbo
