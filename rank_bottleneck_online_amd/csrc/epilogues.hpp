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

__device__ __forceinline__ float sigmoid_f(float z) { return 1.f / (1.f + expf(-z)); }
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

template <class C>
using AccT = floatx16[C::NACC][C::FM][C::FN];

// Visit the rows of this lane's accumulators: f(i, v, local_row) with
// compile-time i (row block) and v (element). Accumulator columns are then
// visited with for_cols; indices stay compile-time throughout.
template <class C, class F>
__device__ __forceinline__ void for_rows(const TileCtx& c, F&& f) {
  static_for<0, C::FM>([&](auto i) { static_for<0, 16>([&](auto v) { f(i, v, acc_row<C>(c, i, v)); }); });
}
template <class C, class F>
__device__ __forceinline__ void for_cols(const TileCtx& c, F&& f) {
  static_for<0, C::FN>([&](auto j) { f(j, acc_col<C>(c, j)); });
}

// ---------------------------------------------------------------------------
// out = acc (optionally row-scaled), dtype or fp32. Also the split-K partial
// writer (out then points at the partial buffer, indexed by prob).
// ---------------------------------------------------------------------------
template <bool F32>
struct EpiStore {
  static constexpr bool kRowSumsq = false;
  struct Args {
    void* out;
    int64_t ldo;
    int64_t pstride;          // elements between consecutive probs
    const void* rowscale;     // dtype [M] or null
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    typedef typename std::conditional<F32, float, T>::type O;
    const int64_t base = (int64_t)c.prob * a.pstride;
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      const float rs = a.rowscale ? Elem<T>::load(a.rowscale, row) : 1.f;
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col < c.N) Elem<O>::store(a.out, base + (int64_t)row * a.ldo + col, rs * acc[0][i][j][v()]);
      });
    });
  }
};

// ---------------------------------------------------------------------------
// Grouped down projection with the deferred Online-RMSNorm scale:
// H = rho * acc (fp32, saved), S = act(H) (dtype, operand of the up
// products), sumsq from the A loader's row statistics (tile column 0 writes).
// ---------------------------------------------------------------------------
template <bool NORM>
struct EpiDown {
  static constexpr bool kRowSumsq = NORM;
  struct Args {
    float* H;
    void* S;
    float* sumsq;
    int64_t ld;  // columns of H and S
    float inv_dnorm, eps;
    int act;
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    if constexpr (NORM) {
      if (c.tn == 0 && c.split == 0)
        for (int r = c.t; r < C::BM; r += C::NT)
          if (c.m0 + r < c.M) a.sumsq[c.m0 + r] = c.rowv[r];
    }
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      const float rho = NORM ? rms_scale(c.rowv[lr], a.inv_dnorm, a.eps) : 1.f;
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col >= c.N) return;
        const float h = rho * acc[0][i][j][v()];
        const int64_t o = (int64_t)row * a.ld + col;
        a.H[o] = h;
        Elem<T>::store(a.S, o, act_f(h, a.act));
      });
    });
  }
};

// ---------------------------------------------------------------------------
// SwiGLU on two accumulators of the same tile: M = SiLU(gate) * up.
// ---------------------------------------------------------------------------
struct EpiSwiglu {
  static constexpr bool kRowSumsq = false;
  struct Args {
    void* M;
    int64_t ld;
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    static_assert(C::NACC == 2, "SwiGLU needs two accumulators");
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col < c.N)
          Elem<T>::store(a.M, (int64_t)row * a.ld + col, silu_f(acc[0][i][j][v()]) * acc[1][i][j][v()]);
      });
    });
  }
};

// ---------------------------------------------------------------------------
// Backward through the bottleneck of group j (batch index): acc = dS_j.
// dH = dS * act'(H), dU = rho * dH (dtype), S = act(H) recomputed (dtype,
// optional), and per-row partials q = sum_k dH * H over this tile's columns
// (the rho-gradient, dRho = q / rho), one row of partials per (j, tile col).
// ---------------------------------------------------------------------------
template <bool NORM>
struct EpiDS {
  static constexpr bool kRowSumsq = false;
  struct Args {
    const float* H;
    int64_t ld;        // columns of H, dU, S (= G*r)
    int64_t r;         // group width (column offset of group j is j*r)
    void* dU;
    void* S;           // may be null
    float* qpart;      // [G*tiles_n][qstride] or null
    int64_t qstride;
    const float* sumsq;
    float inv_dnorm, eps;
    int act;
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    const int64_t goff = (int64_t)c.bidx * a.r;
    float part[C::FM][16];
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      part[i][v] = 0.f;
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      const float rho = NORM ? rms_scale(a.sumsq[row], a.inv_dnorm, a.eps) : 1.f;
      float q = 0.f;
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col >= c.N) return;
        const int64_t o = (int64_t)row * a.ld + goff + col;
        const float h = a.H[o];
        const float dh = acc[0][i][j][v()] * act_grad_f(h, a.act);
        Elem<T>::store(a.dU, o, rho * dh);
        if (a.S) Elem<T>::store(a.S, o, act_f(h, a.act));
        q += dh * h;
      });
      part[i][v] = q;
    });
    if (a.qpart) {
      tile_row_sum<C>(c, part, c.rowv);
      const int64_t slot = (int64_t)c.bidx * cdiv(c.N, C::BN) + c.tn;
      float* qp = a.qpart + slot * a.qstride;
      for (int r = c.t; r < C::BM; r += C::NT)
        if (c.m0 + r < c.M) qp[c.m0 + r] = c.rowv[r];
    }
  }
};

// ---------------------------------------------------------------------------
// Input gradient with the RMSNorm backward: acc = dx~ = dU @ A_cat^T.
// dx = g * dx~ - (rho^2 q / d_norm) * x   (rho^3 dRho / d_norm, dRho = q/rho)
// and per-column partials of dg = sum_t x * dx~ over this tile's rows.
// ---------------------------------------------------------------------------
struct EpiDX {
  static constexpr bool kRowSumsq = false;
  struct Args {
    const void* x;
    const void* g;
    const float* sumsq;
    const float* qpart;
    int nq;
    int64_t qstride;
    float inv_dnorm, eps;
    void* dx;
    float* dgpart;  // [tiles_m][ld]
    int64_t ld;     // d
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
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
    __syncthreads();
    float part[C::FN], gv[C::FN];
    for_cols<C>(c, [&](auto j, int lc) {
      const int col = c.n0 + lc;
      gv[j] = col < c.N ? Elem<T>::load(a.g, col) : 0.f;
      part[j] = 0.f;
    });
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      const float coef = c.rowv[lr];
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col >= c.N) return;
        const int64_t o = (int64_t)row * a.ld + col;
        const float xv = Elem<T>::load(a.x, o);
        const float d = acc[0][i][j][v()];
        Elem<T>::store(a.dx, o, gv[j] * d - coef * xv);
        part[j] += xv * d;
      });
    });
    tile_col_sum<C>(c, part, c.colv);
    for (int n = c.t; n < C::BN; n += C::NT)
      if (c.n0 + n < c.N) a.dgpart[(int64_t)c.tm * a.ld + c.n0 + n] = c.colv[n];
  }
};

// ---------------------------------------------------------------------------
// SwiGLU backward with the gate/up recompute (two accumulators: Yg, Yu).
// Reads dM (fp32); writes M = SiLU(Yg) Yu (operand of dA2), and
// dYg = dM Yu SiLU'(Yg), dYu = dM SiLU(Yg) into a [2,T,ffn] buffer.
// ---------------------------------------------------------------------------
struct EpiSwigluBwd {
  static constexpr bool kRowSumsq = false;
  struct Args {
    const float* dM;
    void* M;
    void* dYgu;
    int64_t ld;      // ffn
    int64_t ystride; // T * ffn
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    static_assert(C::NACC == 2, "SwiGLU backward needs two accumulators");
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col >= c.N) return;
        const int64_t o = (int64_t)row * a.ld + col;
        const float yg = acc[0][i][j][v()], yu = acc[1][i][j][v()];
        const float dm = a.dM[o];
        const float s = sigmoid_f(yg);
        const float sl = yg * s;
        Elem<T>::store(a.M, o, sl * yu);
        Elem<T>::store(a.dYgu, o, dm * yu * (s * (1.f + yg * (1.f - s))));
        Elem<T>::store(a.dYgu, a.ystride + o, dm * sl);
      });
    });
  }
};

// ---------------------------------------------------------------------------
// Tensor-parallel share, forward, first product: acc = u = z @ B_s.
// a = SiLU(u); writes (a * g_s) (dtype, operand of the row-slice product) and
// per-row partial sums of a^2 over this tile's columns.
// ---------------------------------------------------------------------------
struct EpiBtpU {
  static constexpr bool kRowSumsq = false;
  struct Args {
    const void* g;
    void* ag;
    float* spart;  // [tiles_n][sstride]
    int64_t sstride;
    int64_t ld;    // d_shard
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    float gv[C::FN];
    for_cols<C>(c, [&](auto j, int lc) {
      const int col = c.n0 + lc;
      gv[j] = col < c.N ? Elem<T>::load(a.g, col) : 0.f;
    });
    float part[C::FM][16];
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      part[i][v] = 0.f;
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      float s = 0.f;
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col >= c.N) return;
        const float av = silu_f(acc[0][i][j][v()]);
        Elem<T>::store(a.ag, (int64_t)row * a.ld + col, av * gv[j]);
        s += av * av;
      });
      part[i][v] = s;
    });
    tile_row_sum<C>(c, part, c.rowv);
    for (int r = c.t; r < C::BM; r += C::NT)
      if (c.m0 + r < c.M) a.spart[(int64_t)c.tn * a.sstride + c.m0 + r] = c.rowv[r];
  }
};

// ---------------------------------------------------------------------------
// Tensor-parallel share, forward, second product: acc = p (partial over
// shares). Tile column 0 also sums the row partials of a^2 into s.
// ---------------------------------------------------------------------------
struct EpiBtpP {
  static constexpr bool kRowSumsq = false;
  struct Args {
    void* p;
    int64_t ld;  // r
    const float* spart;
    int nsp;
    int64_t sstride;
    float* s;
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    if (c.tn == 0) {
      for (int r = c.t; r < C::BM; r += C::NT) {
        const int row = c.m0 + r;
        if (row >= c.M) continue;
        float s = 0.f;
        for (int q = 0; q < a.nsp; ++q) s += a.spart[(int64_t)q * a.sstride + row];
        a.s[row] = s;
      }
    }
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col < c.N) Elem<T>::store(a.p, (int64_t)row * a.ld + col, acc[0][i][j][v()]);
      });
    });
  }
};

// ---------------------------------------------------------------------------
// Tensor-parallel share, backward, recompute of u = z @ B_s (acc) fused with
// the backward of SiLU, the gain and the local statistic:
//   a = SiLU(u); da = g_s e + 2 ds a; du = da SiLU'(u)   (e = dp @ A_s^T, fp32)
// writes du (dtype), a * g_s (dtype, operand of dA_s) and per-column
// partials of dg_s = sum_t a e over this tile's rows.
// ---------------------------------------------------------------------------
struct EpiBtpUBwd {
  static constexpr bool kRowSumsq = false;
  struct Args {
    const float* e;
    const float* ds;
    const void* g;
    void* du;
    void* ag;
    float* dgpart;  // [tiles_m][ld]
    int64_t ld;     // d_shard
  };
  template <class C>
  static __device__ __forceinline__ void run(AccT<C>& acc, const TileCtx& c, const Args& a) {
    typedef typename C::T T;
    float gv[C::FN], part[C::FN];
    for_cols<C>(c, [&](auto j, int lc) {
      const int col = c.n0 + lc;
      gv[j] = col < c.N ? Elem<T>::load(a.g, col) : 0.f;
      part[j] = 0.f;
    });
    for_rows<C>(c, [&](auto i, auto v, int lr) {
      const int row = c.m0 + lr;
      if (row >= c.M) return;
      const float dsv = a.ds[row];
      for_cols<C>(c, [&](auto j, int lc) {
        const int col = c.n0 + lc;
        if (col >= c.N) return;
        const int64_t o = (int64_t)row * a.ld + col;
        const float u = acc[0][i][j][v()];
        const float s = sigmoid_f(u);
        const float av = u * s;
        const float ev = a.e[o];
        const float da = gv[j] * ev + 2.f * dsv * av;
        Elem<T>::store(a.du, o, da * (s * (1.f + u * (1.f - s))));
        Elem<T>::store(a.ag, o, av * gv[j]);
        part[j] += av * ev;
      });
    });
    tile_col_sum<C>(c, part, c.colv);
    for (int n = c.t; n < C::BN; n += C::NT)
      if (c.n0 + n < c.N) a.dgpart[(int64_t)c.tm * a.ld + c.n0 + n] = c.colv[n];
  }
};

}  // namespace rbo
