// Fused GEMM epilogues of the low-rank bottleneck block.
//
// Each epilogue consumes the fp32 accumulators of one output tile (layout in
// gemm.hpp) and applies the elementwise and reduction work of the block on
// them, so that no d-wide or ffn-wide intermediate makes an extra trip to
// HBM and the only roundings to the storage dtype are of GEMM operands and
// of dtype outputs. Per-row and per-column partial sums are combined in a
// fixed order (no atomics), so results are run-to-run bit-identical.
#pragma once

#include "gemm.hpp"

namespace rbo {

// sigmoid(z) = 1 / (1 + e^-z) = 1 / (1 + 2^(-z log2 e)), on the hardware
// base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32; about 1 ulp each,
// far below the bf16 rounding every activation output goes through). The
// libm-accurate exp and the IEEE division cost about 25 instructions per
// element, which the epilogue of every tile pays with the matrix cores idle.
// Limits: z -> -inf gives 2^+inf = inf and rcp(inf) = 0; z -> +inf gives 1.
__device__ __forceinline__ float sigmoid_f(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return __builtin_amdgcn_rcpf(1.f + e);
}
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }
// d/dz SiLU(z) = s (1 + z (1 - s)), s = sigmoid(z)
__device__ __forceinline__ float silu_grad_f(float z) {
  const float s = sigmoid_f(z);
  return s * (1.f + z * (1.f - s));
}
// Bottleneck activation: 0 identity (SVD-style), 1 SiLU (CoLA).
__device__ __forceinline__ float act_f(float z, int act) { return act ? silu_f(z) : z; }
__device__ __forceinline__ float act_grad_f(float z, int act) { return act ? silu_grad_f(z) : 1.f; }
__device__ __forceinline__ float rms_scale(float sumsq, float inv_dnorm, float eps) {
  return 1.f / sqrtf(sumsq * inv_dnorm + eps);
}

// ---------------------------------------------------------------------------
// 8-wide vector access to global tensors (16 bytes of bf16, 32 of fp32).
// Every column offset handed to an epilogue is a multiple of 8 and every
// row length is a multiple of 64, so these are always aligned.
// ---------------------------------------------------------------------------
template <typename T> struct Vec8;
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const void* base, int64_t i, float (&o)[8]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
    const float4 a = p[0], b = p[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
  static __device__ __forceinline__ void store(void* base, int64_t i, const float (&v)[8]) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + i);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const void* base, int64_t i, float (&o)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + i);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = __uint_as_float(ws[q] << 16);
      o[2 * q + 1] = __uint_as_float(ws[q] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(void* base, int64_t i, const float (&v)[8]) {
    uint32_t ws[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x2 h;
      h[0] = static_cast<bf16>(v[2 * q]);      // round to nearest even
      h[1] = static_cast<bf16>(v[2 * q + 1]);
      ws[q] = __builtin_bit_cast(uint32_t, h);
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + i) = u32x4{ws[0], ws[1], ws[2], ws[3]};
  }
};

// Defaults for functors that need no preparation or reductions.
struct EpiBase {
  static constexpr bool kRowSumsq = false, kRowSum = false, kColSum = false;
  // Global inputs of one apply() call, loaded by pre() ahead of time (the
  // driver issues every pre() of a 32-row chunk before staging it).
  struct Pre {};
  template <class C, class A>
  static __device__ __forceinline__ void pre(const TileCtx&, const A&, int, int, Pre&) {}
  template <class C, class A>
  static __device__ __forceinline__ void begin(const TileCtx&, const A&) {}
  template <class C, class A>
  static __device__ __forceinline__ void rows_done(const TileCtx&, const A&, const float*) {}
  template <class C, class A>
  static __device__ __forceinline__ void cols_done(const TileCtx&, const A&, const float*) {}
};

// ---------------------------------------------------------------------------
// out = acc (optionally row-scaled), dtype or fp32. Also the split-K partial
// writer (out then points at the partial buffer, indexed by prob).
// ---------------------------------------------------------------------------
template <bool F32>
struct EpiStore : EpiBase {
  struct Args {
    void* out;
    int64_t ldo;
    int64_t pstride;          // elements between consecutive probs
    const void* rowscale;     // dtype [M] or null
  };
  template <class C>
  static __device__ __forceinline__ void begin(const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    if (a.rowscale)
      for (int r = c.t; r < C::BM; r += C::NT)
        c.rowv[r] = c.m0 + r < c.M ? Elem<T>::load(a.rowscale, c.m0 + r) : 0.f;
  }
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float&, float (&)[8]) {
    typedef typename C::T T;
    typedef typename std::conditional<F32, float, T>::type O;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    const float rs = a.rowscale ? c.rowv[lr] : 1.f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = rs * v[0][e];
    Vec8<O>::store(a.out, (int64_t)c.prob * a.pstride + (int64_t)row * a.ldo + col, o);
  }
};

// ---------------------------------------------------------------------------
// Grouped down projection with the deferred Online-RMSNorm scale:
// H = rho * acc (fp32, saved), S = act(H) (dtype, operand of the up
// products), sumsq from the A loader's row statistics (tile column 0 writes).
// ---------------------------------------------------------------------------
template <bool NORM, bool GIVEN = false>
struct EpiDown : EpiBase {
  // GIVEN: the row sums of squares come from the producer of x (sumsq_in)
  // instead of being taken from the A fragments here.
  static constexpr bool kRowSumsq = NORM && !GIVEN;
  struct Args {
    float* H;
    void* S;
    float* sumsq;           // out (may be null when GIVEN)
    int64_t ld;             // columns of H and S
    float inv_dnorm, eps;
    int act;
    const float* sumsq_in;  // GIVEN only
  };
  template <class C>
  static __device__ __forceinline__ void begin(const TileCtx& c, const Args& a) {
    if constexpr (NORM) {
      // rowv holds (or receives) the row sums of squares; publish them and
      // turn them into rho.
      for (int r = c.t; r < C::BM; r += C::NT) {
        const bool in = c.m0 + r < c.M;
        float ss;
        if constexpr (GIVEN) ss = in ? a.sumsq_in[c.m0 + r] : 0.f;
        else ss = c.rowv[r];
        if (a.sumsq && c.tn == 0 && c.split == 0 && in) a.sumsq[c.m0 + r] = ss;
        c.rowv[r] = rms_scale(ss, a.inv_dnorm, a.eps);
      }
    }
  }
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float&, float (&)[8]) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    const float rho = NORM ? c.rowv[lr] : 1.f;
    float h[8], sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = rho * v[0][e];
      sv[e] = act_f(h[e], a.act);
    }
    const int64_t o = (int64_t)row * a.ld + col;
    Vec8<float>::store(a.H, o, h);
    Vec8<T>::store(a.S, o, sv);
  }
};

// ---------------------------------------------------------------------------
// Up projection into a residual stream: out = res + acc (dtype), and per-row
// partial sums over this tile's columns of out^2, taken from the stored
// (rounded) values: the statistic the next block's Online-RMSNorm needs,
// emitted by the kernel that produces its input. One row of partials per
// tile column (part[tn][row]); null part skips them.
// ---------------------------------------------------------------------------
struct EpiUpRes : EpiBase {
  static constexpr bool kRowSum = true;
  struct Pre {
    float r[8];
  };
  struct Args {
    void* out;
    int64_t ldo;
    const void* res;  // [M, ldo] dtype, or null (no residual)
    float* part;      // [tiles_n][M] fp32 or null
  };
  template <class C>
  static __device__ __forceinline__ void pre(const TileCtx& c, const Args& a, int lr, int lc, Pre& pf) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    if (a.res) {
      Vec8<T>::load(a.res, (int64_t)row * a.ldo + col, pf.r);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf.r[e] = 0.f;
    }
  }
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float& rowc,
                                               float (&)[8]) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = Elem<T>::round(pf.r[e] + v[0][e]);
      rowc += o[e] * o[e];
    }
    Vec8<T>::store(a.out, (int64_t)row * a.ldo + col, o);
  }
  template <class C>
  static __device__ __forceinline__ void rows_done(const TileCtx& c, const Args& a, const float* sums) {
    if (!a.part) return;
    for (int r = c.t; r < C::BM; r += C::NT)
      if (c.m0 + r < c.M) a.part[(int64_t)c.tn * c.M + c.m0 + r] = sums[r];
  }
};

// ---------------------------------------------------------------------------
// SwiGLU on two accumulators of the same tile: M = SiLU(gate) * up.
// ---------------------------------------------------------------------------
struct EpiSwiglu : EpiBase {
  struct Args {
    void* M;
    int64_t ld;
  };
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float&, float (&)[8]) {
    typedef typename C::T T;
    static_assert(C::NACC == 2, "SwiGLU needs two accumulators");
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = silu_f(v[0][e]) * v[1][e];
    Vec8<T>::store(a.M, (int64_t)row * a.ld + col, m);
  }
};

// ---------------------------------------------------------------------------
// Backward through the bottleneck of group j (batch index): acc = dS_j.
// dH = dS * act'(H), dU = rho * dH (dtype), S = act(H) recomputed (dtype,
// optional), and per-row partials q = sum_k dH * H over this tile's columns
// (the rho-gradient, dRho = q / rho), one row of partials per (j, tile col).
// ---------------------------------------------------------------------------
template <bool NORM>
struct EpiDS : EpiBase {
  static constexpr bool kRowSum = NORM;
  struct Pre {
    float h[8];
  };
  struct Args {
    const float* H;
    int64_t ld;        // columns of H, dU, S (= G*r)
    int64_t r;         // group width (column offset of group j is j*r)
    void* dU;
    void* S;           // may be null
    float* qpart;      // [G*tiles_n][qstride] (NORM only)
    int64_t qstride;
    const float* sumsq;
    float inv_dnorm, eps;
    int act;
  };
  template <class C>
  static __device__ __forceinline__ void begin(const TileCtx& c, const Args& a) {
    if constexpr (NORM)
      for (int r = c.t; r < C::BM; r += C::NT)
        c.rowv[r] = c.m0 + r < c.M ? rms_scale(a.sumsq[c.m0 + r], a.inv_dnorm, a.eps) : 0.f;
  }
  template <class C>
  static __device__ __forceinline__ void pre(const TileCtx& c, const Args& a, int lr, int lc, Pre& pf) {
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    Vec8<float>::load(a.H, (int64_t)row * a.ld + (int64_t)c.bidx * a.r + col, pf.h);
  }
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float& rowc, float (&)[8]) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    const int64_t o = (int64_t)row * a.ld + (int64_t)c.bidx * a.r + col;
    const float rho = NORM ? c.rowv[lr] : 1.f;
    float du[8], sv[8];
    const float (&h)[8] = pf.h;
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dh = v[0][e] * act_grad_f(h[e], a.act);
      du[e] = rho * dh;
      sv[e] = act_f(h[e], a.act);
      q += dh * h[e];
    }
    Vec8<T>::store(a.dU, o, du);
    if (a.S) Vec8<T>::store(a.S, o, sv);
    rowc = q;
  }
  template <class C>
  static __device__ __forceinline__ void rows_done(const TileCtx& c, const Args& a, const float* sums) {
    if constexpr (NORM) {
      float* qp = a.qpart + ((int64_t)c.bidx * cdiv(c.N, C::BN) + c.tn) * a.qstride;
      for (int r = c.t; r < C::BM; r += C::NT)
        if (c.m0 + r < c.M) qp[c.m0 + r] = sums[r];
    }
  }
};

// ---------------------------------------------------------------------------
// Input gradient with the RMSNorm backward: acc = dx~ = dU @ A_cat^T.
// dx = g * dx~ - (rho^2 q / d_norm) * x   (rho^3 dRho / d_norm, dRho = q/rho)
// and per-column partials of dg = sum_t x * dx~ over this tile's rows.
// ---------------------------------------------------------------------------
struct EpiDX : EpiBase {
  static constexpr bool kColSum = true;
  struct Pre {
    float x[8], g[8], add[8];
  };
  struct Args {
    const void* x;
    const void* g;
    const float* sumsq;
    const float* qpart;
    int nq;
    int64_t qstride;
    float inv_dnorm, eps;
    void* dx;
    float* dgpart;     // [tiles_m][ld]
    int64_t ld;        // d
    const void* dadd;  // [T, d] dtype gradient added to dx (residual path), or null
  };
  template <class C>
  static __device__ __forceinline__ void begin(const TileCtx& c, const Args& a) {
    for (int r = c.t; r < C::BM; r += C::NT) {
      const int row = c.m0 + r;
      float coef = 0.f;
      if (row < c.M) {
        float q = 0.f;
        for (int p = 0; p < a.nq; ++p) q += a.qpart[(int64_t)p * a.qstride + row];
        const float rho = rms_scale(a.sumsq[row], a.inv_dnorm, a.eps);
        coef = rho * rho * q * a.inv_dnorm;
      }
      c.rowv[r] = coef;
    }
  }
  template <class C>
  static __device__ __forceinline__ void pre(const TileCtx& c, const Args& a, int lr, int lc, Pre& pf) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    Vec8<T>::load(a.x, (int64_t)row * a.ld + col, pf.x);
    Vec8<T>::load(a.g, col, pf.g);
    if (a.dadd) Vec8<T>::load(a.dadd, (int64_t)row * a.ld + col, pf.add);
  }
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float&, float (&colc)[8]) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    const int64_t o = (int64_t)row * a.ld + col;
    const float coef = c.rowv[lr];
    float dx[8];
    const float (&xv)[8] = pf.x;
    const float (&gv)[8] = pf.g;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dx[e] = gv[e] * v[0][e] - coef * xv[e] + (a.dadd ? pf.add[e] : 0.f);
      colc[e] += xv[e] * v[0][e];
    }
    Vec8<T>::store(a.dx, o, dx);
  }
  template <class C>
  static __device__ __forceinline__ void cols_done(const TileCtx& c, const Args& a, const float* sums) {
    for (int n = c.t; n < C::BN; n += C::NT)
      if (c.n0 + n < c.N) a.dgpart[(int64_t)c.tm * a.ld + c.n0 + n] = sums[n];
  }
};

// ---------------------------------------------------------------------------
// SwiGLU backward with the gate/up recompute, three accumulators over the
// same [T-tile, ffn-tile]: Yg = S1_0 B1_0, Yu = S1_1 B1_1 and dM = dU2 A2^T
// (all K = r). Writes M = SiLU(Yg) Yu (operand of dA2), and
// dYg = dM Yu SiLU'(Yg), dYu = dM SiLU(Yg) into a [2,T,ffn] buffer; dM never
// leaves the registers, unrounded.
// ---------------------------------------------------------------------------
struct EpiSwigluBwd : EpiBase {
  struct Args {
    void* M;
    void* dYgu;
    int64_t ld;      // ffn
    int64_t ystride; // T * ffn
  };
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre&, float&, float (&)[8]) {
    typedef typename C::T T;
    static_assert(C::NACC == 3, "SwiGLU backward takes gate, up and dM accumulators");
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    const int64_t o = (int64_t)row * a.ld + col;
    float m[8], dg[8], du[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float yg = v[0][e], yu = v[1][e], dm = v[2][e];
      const float s = sigmoid_f(yg);
      const float sl = yg * s;
      m[e] = sl * yu;
      dg[e] = dm * yu * (s * (1.f + yg * (1.f - s)));
      du[e] = dm * sl;
    }
    Vec8<T>::store(a.M, o, m);
    Vec8<T>::store(a.dYgu, o, dg);
    Vec8<T>::store(a.dYgu, a.ystride + o, du);
  }
};

// ---------------------------------------------------------------------------
// Tensor-parallel share, forward, first product: acc = u = z @ B_s.
// a = SiLU(u); writes (a * g_s) (dtype, operand of the row-slice product) and
// per-row partial sums of a^2 over this tile's columns.
// ---------------------------------------------------------------------------
struct EpiBtpU : EpiBase {
  static constexpr bool kRowSum = true;
  struct Args {
    const void* g;
    void* ag;
    float* spart;  // [tiles_n][sstride]
    int64_t sstride;
    int64_t ld;    // d_shard
  };
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float& rowc, float (&)[8]) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    float gv[8], ag[8];
    Vec8<T>::load(a.g, col, gv);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float av = silu_f(v[0][e]);
      ag[e] = av * gv[e];
      s += av * av;
    }
    Vec8<T>::store(a.ag, (int64_t)row * a.ld + col, ag);
    rowc = s;
  }
  template <class C>
  static __device__ __forceinline__ void rows_done(const TileCtx& c, const Args& a, const float* sums) {
    for (int r = c.t; r < C::BM; r += C::NT)
      if (c.m0 + r < c.M) a.spart[(int64_t)c.tn * a.sstride + c.m0 + r] = sums[r];
  }
};

// ---------------------------------------------------------------------------
// Tensor-parallel share, forward, second product: acc = p (partial over
// shares). Tile column 0 also sums the row partials of a^2 into s.
// ---------------------------------------------------------------------------
struct EpiBtpP : EpiBase {
  struct Args {
    void* p;
    int64_t ld;  // r
    const float* spart;
    int nsp;
    int64_t sstride;
    float* s;
  };
  template <class C>
  static __device__ __forceinline__ void begin(const TileCtx& c, const Args& a) {
    if (c.tn == 0) {
      for (int r = c.t; r < C::BM; r += C::NT) {
        const int row = c.m0 + r;
        if (row >= c.M) continue;
        float s = 0.f;
        for (int q = 0; q < a.nsp; ++q) s += a.spart[(int64_t)q * a.sstride + row];
        a.s[row] = s;
      }
    }
  }
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float&, float (&)[8]) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = v[0][e];
    Vec8<T>::store(a.p, (int64_t)row * a.ld + col, o);
  }
};

// ---------------------------------------------------------------------------
// BTP share backward through the bottleneck: acc = e = dp @ A_s^T, with
// u = z @ B_s recomputed by the launch before it and stored in fp32 (the
// value its accumulator held). a = SiLU(u), da = g_s * e + 2 ds a (the
// statistic's gradient), du = da * SiLU'(u), ag = a * g_s (the operand of
// dA_s), and column partials of a * e (dg_s) per tile row.
// ---------------------------------------------------------------------------
struct EpiBtpEBwd : EpiBase {
  static constexpr bool kColSum = true;
  struct Pre {
    float g[8], u[8];
  };
  struct Args {
    const float* ds;
    const void* g;
    const float* U;   // [T][ld] fp32
    void* du;
    void* ag;
    float* dgpart;    // [tiles_m][ld]
    int64_t ld;       // d_shard
  };
  template <class C>
  static __device__ __forceinline__ void begin(const TileCtx& c, const Args& a) {
    for (int r = c.t; r < C::BM; r += C::NT) c.rowv[r] = c.m0 + r < c.M ? a.ds[c.m0 + r] : 0.f;
  }
  template <class C>
  static __device__ __forceinline__ void pre(const TileCtx& c, const Args& a, int lr, int lc, Pre& pf) {
    typedef typename C::T T;
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    Vec8<T>::load(a.g, col, pf.g);
    Vec8<float>::load(a.U, (int64_t)row * a.ld + col, pf.u);
  }
  template <class C>
  static __device__ __forceinline__ void apply(const TileCtx& c, const Args& a, int lr, int lc,
                                               const float (&v)[C::NACC][8], const Pre& pf, float&, float (&colc)[8]) {
    typedef typename C::T T;
    static_assert(C::NACC == 1, "one accumulator: e");
    const int row = c.m0 + lr, col = c.n0 + lc;
    if (row >= c.M || col >= c.N) return;
    const int64_t o = (int64_t)row * a.ld + col;
    const float dsv = c.rowv[lr];
    float du[8], ag[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = pf.u[e], ev = v[0][e];
      const float s = sigmoid_f(u);
      const float av = u * s;
      const float da = pf.g[e] * ev + 2.f * dsv * av;
      du[e] = da * (s * (1.f + u * (1.f - s)));
      ag[e] = av * pf.g[e];
      colc[e] += av * ev;
    }
    Vec8<T>::store(a.du, o, du);
    Vec8<T>::store(a.ag, o, ag);
  }
  template <class C>
  static __device__ __forceinline__ void cols_done(const TileCtx& c, const Args& a, const float* sums) {
    for (int n = c.t; n < C::BN; n += C::NT)
      if (c.n0 + n < c.N) a.dgpart[(int64_t)c.tm * a.ld + c.n0 + n] = sums[n];
  }
};

}  // namespace rbo
