// GEMM core for gfx950 (CDNA4): MFMA tiles staged through LDS.
//
// C[M,N] (+)= A[M,K] @ B[K,N] with fp32 accumulation, for the products of
// the low-rank bottleneck block (down projections, batched up projections,
// their backward products and the weight gradients with K = tokens).
//
// Element types: bfloat16 (v_mfma_f32_32x32x16_bf16) and fp32
// (v_mfma_f32_32x32x2_f32). Both use the 32x32 accumulator layout: lane l
// holds C[8*(v/4) + 4*(l/32) + v%4][l%32] for v = 0..15.
//
// Operand layouts. The MFMA wants both operands with K contiguous per lane.
//   A "KC": element (m,k) at m*ld + k  (activations x, dY, S, ...)
//   A "MC": element (m,k) at k*ld + m  (transposed activations, K = tokens)
//   B "KC": element (k,n) at n*ld + k  (a weight used transposed)
//   B "NC": element (k,n) at k*ld + n  (a weight in [in,out] layout, or an
//           activation when K = tokens)
// KC operands are copied to LDS in 16-byte chunks. MC/NC operands are loaded
// as VEC x VEC blocks (VEC elements per 16 bytes), transposed in registers,
// and written K-contiguous, so the MFMA loop only ever sees one LDS layout.
//
// LDS layout: each staged tile row holds 128 bytes of K (BK = 64 bf16 or
// 32 fp32). 16-byte chunk c of row m lives at chunk c ^ ((m ^ (m>>3)) & 7):
// MFMA fragment reads (8 consecutive rows, same chunk) and transposed
// writes (rows 8 apart, same chunk) both hit 8 distinct chunks. Rows of 128
// bytes also keep every global request one full cache line: with 64-byte
// rows the same slab streams measurably slower.
//
// Global loads use buffer instructions with a per-operand byte range, so
// every read past the end of a tensor returns zero: rows past T and the
// K tail of K = tokens products need no branches. Reads past M or N inside
// the tensor only feed accumulator rows/columns that the epilogue masks.
//
// Pipelining. When both operands are K-contiguous, each K slab goes from
// global memory straight into LDS (buffer loads with the LDS flag), with as
// many LDS stages as fit (two for 256 x 256 tiles, three or four for smaller
// ones): while the MFMAs read stage kt, the slabs of the next NSTAGE-1 steps
// are in flight, and each step waits only for the oldest. The load
// instructions of the next slab are interleaved one by one with the MFMAs of
// the first two k sub-steps, so that a stalled load issue never leaves the
// matrix cores idle (with one wave per SIMD there is no other wave to fill
// the gap). Otherwise operands pass through registers (to be transposed)
// with two LDS stages: during step kt the slab of step kt+1, already in
// registers, is written to the other stage and the slab of step kt+2 is
// fetched. MFMA fragments are double-buffered across the 16-wide k
// sub-steps; one barrier per K step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rbo {

typedef __bf16 bf16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Compile-time loop: f(std::integral_constant<int, i>) for i = B..E-1. Used
// wherever accumulator registers are indexed, so that no index is ever a
// runtime value (a runtime index would move the accumulators to scratch).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int kRowBytes = 128;  // bytes of K per staged tile row

__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ lds_swz(row)) << 4);
}

// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<bf16> {
  static __device__ __forceinline__ float to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    bf16 h = static_cast<bf16>(v);  // round to nearest even
    static_cast<bf16*>(p)[i] = h;
  }
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return to_f32(static_cast<const uint16_t*>(p)[i]);
  }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
};

// ---------------------------------------------------------------------------
// MFMA traits
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  static constexpr int KI = 16;  // K per instruction
  static constexpr int KL = 8;   // contiguous K per lane
  typedef bf16x8 Frag;
  static __device__ __forceinline__ Frag read(const char* tile, int row, int k) {
    return *reinterpret_cast<const bf16x8*>(tile + lds_off(row, k >> 3));
  }
  static __device__ __forceinline__ floatx16 mma(Frag a, Frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KI = 2;
  static constexpr int KL = 1;
  typedef float Frag;
  static __device__ __forceinline__ Frag read(const char* tile, int row, int k) {
    return *reinterpret_cast<const float*>(tile + lds_off(row, k >> 2) + ((k & 3) << 2));
  }
  static __device__ __forceinline__ floatx16 mma(Frag a, Frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Sum of squares of one MFMA A fragment, accumulated into acc.
__device__ __forceinline__ float frag_sumsq(bf16x8 f, float acc) {
  const u32x4 v = __builtin_bit_cast(u32x4, f);
  // Words are copied to scalars first: bit-casting a vector element selected
  // by a loop index straight into the dot2 builtin makes this compiler read
  // word 0 every time.
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2 p = __builtin_bit_cast(bf16x2, w[q]);
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float frag_sumsq(float f, float acc) { return __builtin_fmaf(f, f, acc); }

// ---------------------------------------------------------------------------
// Tile configuration
// ---------------------------------------------------------------------------
template <typename T_, int BM_, int BN_, int WM_, int WN_, bool AKC_, bool BKC_, int NACC_>
struct Cfg {
  typedef T_ T;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NACC = NACC_;
  static constexpr bool AKC = AKC_, BKC = BKC_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int ES = sizeof(T);
  static constexpr int VEC = 16 / ES;
  // Operands that are K-contiguous on both sides are loaded straight into
  // LDS; the others pass through registers.
  static constexpr bool DIRECT = AKC_ && BKC_;
  static constexpr int RB = kRowBytes;
  static constexpr int CH = RB / 16;  // 16-byte chunks per row
  static constexpr int BK = RB / ES;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  // The direct path takes as many stages (up to four) as fit next to the
  // epilogue vectors in the 160 KB of a CU; the register path uses two.
  static constexpr int VEC_BYTES_ = (BM + BN + WN * BM + WM * BN) * 4;
  static constexpr int FIT_ = (160 * 1024 - VEC_BYTES_) / STAGE_BYTES;
  static constexpr int NSTAGE = DIRECT ? (FIT_ < 4 ? FIT_ : 4) : 2;
  static_assert(NSTAGE >= 2, "two pipeline stages must fit in LDS");
  static constexpr int PIPE_BYTES = NSTAGE * STAGE_BYTES;
  // Epilogue staging: each wave writes 32 accumulator rows at a time (per
  // accumulator) into a private fp32 buffer with a row stride padded by 8
  // floats (the two half-waves of the MFMA layout then hit disjoint banks),
  // reusing the pipeline LDS.
  static constexpr int EPI_STR = WTN + 8;
  static constexpr int EPI_SUB = 32 * EPI_STR;
  static constexpr int EPI_BYTES = WM * WN * NACC * EPI_SUB * 4;
  static constexpr int SCR_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
  // After that: per-row / per-column fp32 vectors and reduction partials.
  static constexpr int VEC_BYTES = VEC_BYTES_;
  static constexpr int LDS_BYTES = SCR_BYTES + VEC_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "tile does not fit the LDS of a CU");
  static_assert(FM >= 1 && FN >= 1, "wave tile smaller than one MFMA block");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
};

// ---------------------------------------------------------------------------
// Operands and problem geometry (passed by value to kernels)
// ---------------------------------------------------------------------------
struct Operand {
  const void* ptr;        // batch-0 base
  int64_t ld;             // elements between consecutive memory rows
  int64_t batch_stride;   // elements between consecutive batches
  int64_t extent;         // bytes from a batch base to the end of its valid data
};

struct GemmGeom {
  int M, N, K;
  int batch;     // independent problems
  int splits;    // K splits (partial results go to separate outputs)
  int k_split;   // K range per split, a multiple of BK
  int tiles_m, tiles_n;
};

struct GemmOps {
  Operand a[2], b[2];  // one pair per accumulator (NACC <= 2)
};

// Per-tile context handed to the epilogue.
struct TileCtx {
  int m0, n0;        // tile origin in the output
  int tm, tn;        // tile indices
  int bidx, split;   // batch index, K-split index
  int prob;          // bidx * splits + split
  int M, N;
  int t, lane, wave, wm, wn;
  char* smem;        // pipeline LDS, free for epilogue scratch
  float* rowv;       // BM fp32 in LDS (row statistics from the A loader)
  float* colv;       // BN fp32 in LDS
  float* rowpart;    // [WN][BM] fp32 in LDS (row-sum partials per wave column)
  float* colpart;    // [WM][BN] fp32 in LDS (column-sum partials per wave row)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  int64_t n = bytes < 0 ? 0 : bytes;
  if (n > 0x7fffffffLL) n = 0x7fffffffLL;
  // dword3 0x00020000: raw (untyped) buffer, 32-bit data format, as used for
  // gfx9-family buffer resources.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// ---------------------------------------------------------------------------
// Operand loader: one K slab (ROWS x BK) of one operand per call.
// ---------------------------------------------------------------------------
template <class C, int ROWS, bool KC, bool FROM_TOP, bool ROWSUMSQ>
struct Loader {
  static constexpr int VEC = C::VEC;
  // KC: ROWS*CH chunks; thread t takes chunk t%CH of rows t/CH + u*(NT/CH).
  static constexpr int CH = C::CH;
  static constexpr int KC_UNITS = (ROWS * CH) / C::NT;
  // transposed: (BK/VEC) x (ROWS/VEC) blocks of VEC x VEC elements.
  static constexpr int BLOCKS = (C::BK / VEC) * (ROWS / VEC);
  static constexpr int T_UNITS = cdiv(BLOCKS, C::NT);
  static constexpr int NREG = KC ? KC_UNITS : T_UNITS * VEC;
  static_assert(!KC || (ROWS * CH) % C::NT == 0, "KC loader: ROWS*CH must divide by NT");
  static_assert(!KC || KC_UNITS >= 1, "KC loader: too few rows");

  u32x4 r[NREG];
  float ss[KC ? KC_UNITS : 1];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int u = 0; u < (KC ? KC_UNITS : 1); ++u) ss[u] = 0.f;
  }

  // Issue the global reads of the slab starting at column/row k0.
  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rs, int64_t ld_bytes, int k0, int t) {
    if constexpr (KC) {
      const int c = t % CH;
#pragma unroll
      for (int u = 0; u < KC_UNITS; ++u) {
        const int row = t / CH + u * (C::NT / CH);
        const uint32_t off = (uint32_t)(row * ld_bytes) + (uint32_t)((k0 + c * VEC) * C::ES);
        r[u] = buf_load16(rs, off);
      }
    } else {
      const int tt = FROM_TOP ? (C::NT - 1 - t) : t;
#pragma unroll
      for (int u = 0; u < T_UNITS; ++u) {
        const int b = u * C::NT + tt;
        if (BLOCKS % C::NT == 0 || b < BLOCKS) {
          const int mb = b % (ROWS / VEC), kb = b / (ROWS / VEC);
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            const int k = k0 + kb * VEC + j;
            const uint32_t off = (uint32_t)((int64_t)k * ld_bytes) + (uint32_t)(mb * 16);
            r[u * VEC + j] = buf_load16(rs, off);
          }
        }
      }
    }
  }

  // Write the fetched slab into an LDS tile (K-contiguous rows).
  // `count` says whether this slab lies inside the K range (the pipeline
  // runs one slab past the end; that slab is never read, and its values must
  // not enter the row statistics).
  __device__ __forceinline__ void store(char* tile, int t, bool count = true) {
    if constexpr (KC) {
      const int c = t % CH;
#pragma unroll
      for (int u = 0; u < KC_UNITS; ++u) {
        const int row = t / CH + u * (C::NT / CH);
        *reinterpret_cast<u32x4*>(tile + lds_off(row, c)) = r[u];
        if constexpr (ROWSUMSQ) {
          const float add = sumsq16(r[u], 0.f);
          ss[u] += count ? add : 0.f;
        }
      }
    } else {
      const int tt = FROM_TOP ? (C::NT - 1 - t) : t;
#pragma unroll
      for (int u = 0; u < T_UNITS; ++u) {
        const int b = u * C::NT + tt;
        if (BLOCKS % C::NT == 0 || b < BLOCKS) {
          const int mb = b % (ROWS / VEC), kb = b / (ROWS / VEC);
          u32x4 o[VEC];
          transpose(&r[u * VEC], o);
#pragma unroll
          for (int i = 0; i < VEC; ++i)
            *reinterpret_cast<u32x4*>(tile + lds_off(mb * VEC + i, kb)) = o[i];
        }
      }
    }
  }

  // Sum of squares of the 16 bytes of one chunk, accumulated into acc.
  static __device__ __forceinline__ float sumsq16(u32x4 v, float acc) {
    if constexpr (C::ES == 2) {
      // The words are copied to scalars first: bit-casting a vector element
      // selected by the loop index straight into the dot2 builtin makes this
      // compiler read word 0 four times.
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const bf16x2 p = __builtin_bit_cast(bf16x2, wv[w]);
        acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __uint_as_float(v[w]);
        acc = __builtin_fmaf(f, f, acc);
      }
    }
    return acc;
  }

  // in[j] holds VEC elements (m = 0..VEC-1) of K row j; out[i] gets the VEC
  // K values of m = i.
  static __device__ __forceinline__ void transpose(const u32x4* in, u32x4* out) {
    if constexpr (C::ES == 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t x = in[2 * p][i >> 1], y = in[2 * p + 1][i >> 1];
          out[i][p] = (i & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int p = 0; p < 4; ++p) out[i][p] = in[p][i];
    }
  }
};

// ---------------------------------------------------------------------------
// Direct-to-LDS loader for a K-contiguous operand. One buffer_load_dwordx4
// with the LDS flag writes 64 lanes x 16 bytes to LDS at a wave-uniform base
// (lane l at base + 16 l), i.e. 1024/RB consecutive tile rows. Lane l
// therefore fetches the global chunk that the XOR swizzle places at position
// l % CH of row l / CH. The data never passes through registers.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

template <class C, int ROWS>
struct DirectLoader {
  static constexpr int RPI = 1024 / C::RB;          // tile rows per instruction
  static constexpr int INSTR = ROWS / RPI / C::NW;  // per wave per K slab
  static_assert(ROWS % (RPI * C::NW) == 0, "direct loader: rows must split evenly over the waves");
  // oob = 0 loads the slab; oob = 0x80000000 pushes every offset past the
  // buffer range, so the instructions still issue (keeping the loop free of
  // branches) but fetch nothing.
  __device__ __forceinline__ static void issue(__amdgpu_buffer_rsrc_t rs, int64_t ld_bytes, int k0, char* tile,
                                               int wave, int lane, uint32_t oob = 0) {
#pragma unroll
    for (int q = 0; q < INSTR; ++q) {
      const int row0 = RPI * (q * C::NW + wave);
      const int row = row0 + lane / C::CH;
      const int chunk = (lane % C::CH) ^ lds_swz(row);
      const uint32_t off = ((uint32_t)(row * ld_bytes) + (uint32_t)((k0 + chunk * C::VEC) * C::ES)) | oob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + row0 * C::RB), 16, off, 0, 0, 0);
    }
  }
};

// s_waitcnt vmcnt(n) with the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Load instructions a K step interleaves with the MFMAs of sub-steps 0 and 1.
template <int V0, int V1>
struct SlabPlan {
  static constexpr int at(int kk) { return kk == 0 ? V0 : (kk == 1 ? V1 : 0); }
};

// ---------------------------------------------------------------------------
// Block -> tile mapping. Workgroups are handed to the 8 XCDs round-robin;
// the remap gives each XCD a contiguous range of logical tiles, and tiles are
// walked in groups of 8 tile rows so neighbours share A rows and B columns in
// that XCD's L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb >> 3, rem = nb & 7, x = b & 7;
  return x * q + (x < rem ? x : rem) + (b >> 3);
}

__device__ __forceinline__ void group_tile(int tile, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int gid = tile / per_group;
  const int first = gid * GROUP;
  const int gsz = (tiles_m - first) < GROUP ? (tiles_m - first) : GROUP;
  const int in = tile - gid * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

// ---------------------------------------------------------------------------
// Epilogue driver.
//
// The accumulators are handed to the epilogue through LDS, 32 rows of each
// wave's tile at a time: the wave writes them in the MFMA layout into its
// private padded buffer, then reads them back row-contiguously, 8 columns
// per lane (a row of the wave tile is WTN/8 consecutive lanes). The
// epilogue functor E sees (tile row, tile column, 8 values per accumulator)
// and does all of its global traffic as 16-byte vectors. E may return a
// per-row contribution (summed over the tile's columns) and 8 per-column
// contributions (summed over the tile's rows); both sums are formed here in
// a fixed order (lane butterflies, then waves in index order), so results
// are bit-reproducible.
//
// Functor interface:
//   kRowSumsq           the A loader accumulates row sums of squares into rowv
//   kRowSum / kColSum   the reductions above are wanted
//   begin(c, a)         per-tile preparation (all threads; a barrier follows)
//   apply(c, a, lr, lc, v, rowc, colc)   lr/lc tile-local row / first column
//   rows_done(c, a, sums) / cols_done(c, a, sums)   sums in LDS, BM / BN long
// ---------------------------------------------------------------------------
template <class C, class E>
__device__ __forceinline__ void epilogue(floatx16 (&acc)[C::NACC][C::FM][C::FN], const TileCtx& c,
                                         const typename E::Args& ea) {
  constexpr int STR = C::EPI_STR, SUB = C::EPI_SUB;
  constexpr int V8 = C::WTN / 8;        // lanes per row in the read-back
  constexpr int RPS = 64 / V8;          // rows per read-back step
  constexpr int STEPS = 32 / RPS;
  static_assert(64 % V8 == 0 && 32 % RPS == 0, "wave tile width must be 32, 64 or 128");
  float* scr = reinterpret_cast<float*>(c.smem) + c.wave * (C::NACC * SUB);
  const int c8 = c.lane % V8, rsub = c.lane / V8;

  E::template begin<C>(c, ea);
  __syncthreads();

  float colc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) colc[e] = 0.f;

  static_for<0, C::FM>([&](auto i) {
    static_for<0, C::NACC>([&](auto p) {
      static_for<0, C::FN>([&](auto j) {
        static_for<0, 16>([&](auto v) {
          constexpr int r0 = (v >> 2) * 8 + (v & 3);
          scr[p * SUB + (r0 + (c.lane >> 5) * 4) * STR + j * 32 + (c.lane & 31)] = acc[p][i][j][v()];
        });
      });
    });
    __syncthreads();
    for (int s = 0; s < STEPS; ++s) {
      const int r = s * RPS + rsub;
      const int lr = c.wm * C::WTM + i * 32 + r;
      const int lc = c.wn * C::WTN + c8 * 8;
      float vals[C::NACC][8];
      static_for<0, C::NACC>([&](auto p) {
        const float* src = scr + p * SUB + r * STR + c8 * 8;
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        vals[p][0] = a.x; vals[p][1] = a.y; vals[p][2] = a.z; vals[p][3] = a.w;
        vals[p][4] = b.x; vals[p][5] = b.y; vals[p][6] = b.z; vals[p][7] = b.w;
      });
      float rowc = 0.f;
      E::template apply<C>(c, ea, lr, lc, vals, rowc, colc);
      if constexpr (E::kRowSum) {
#pragma unroll
        for (int m = 1; m < V8; m <<= 1) rowc += __shfl_xor(rowc, m);
        if (c8 == 0) c.rowpart[c.wn * C::BM + lr] = rowc;
      }
    }
    __syncthreads();
  });

  if constexpr (E::kColSum) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int m = V8; m < 64; m <<= 1) colc[e] += __shfl_xor(colc[e], m);
    if (c.lane < V8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) c.colpart[c.wm * C::BN + c.wn * C::WTN + c.lane * 8 + e] = colc[e];
    }
  }
  if constexpr (E::kRowSum || E::kColSum) {
    __syncthreads();
    if constexpr (E::kRowSum) {
      for (int r = c.t; r < C::BM; r += C::NT) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < C::WN; ++w) s += c.rowpart[w * C::BM + r];
        c.rowv[r] = s;
      }
    }
    if constexpr (E::kColSum) {
      for (int n = c.t; n < C::BN; n += C::NT) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < C::WM; ++w) s += c.colpart[w * C::BN + n];
        c.colv[n] = s;
      }
    }
    __syncthreads();
    if constexpr (E::kRowSum) E::template rows_done<C>(c, ea, c.rowv);
    if constexpr (E::kColSum) E::template cols_done<C>(c, ea, c.colv);
  }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <class C, class E>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmGeom g, GemmOps ops, typename E::Args ea) {
  typedef typename C::T T;
  typedef Mfma<T> MF;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool RSS = E::kRowSumsq;
  static_assert(!RSS || C::NACC == 1, "row statistics are taken in single-accumulator products");

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles = g.tiles_m * g.tiles_n;
  const int prob = bid / tiles;
  int tm, tn;
  group_tile(bid - prob * tiles, g.tiles_m, g.tiles_n, tm, tn);
  const int split = prob % g.splits, bidx = prob / g.splits;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int kbeg = split * g.k_split;
  const int kend = (g.K - kbeg) < g.k_split ? g.K : kbeg + g.k_split;
  const int KT = cdiv(kend - kbeg, C::BK);

  floatx16 acc[C::NACC][C::FM][C::FN];
#pragma unroll
  for (int p = 0; p < C::NACC; ++p)
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[p][i][j][v] = 0.f;

  Loader<C, C::BM, C::AKC, false, false> la;
  Loader<C, C::BN, C::BKC, true, false> lb;
  constexpr int KK = C::BK / MF::KI;
  // Online-RMSNorm statistic: sums of squares of the A rows, taken from the
  // MFMA A fragments (each lane holds 8 k-values of one row per sub-step).
  float ss[C::FM];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) ss[i] = 0.f;

  static_for<0, C::NACC>([&](auto p) {
    const Operand& A = ops.a[p];
    const Operand& B = ops.b[p];
    // Rebase each operand on this tile so 32-bit buffer offsets suffice.
    const int64_t a_off = (int64_t)bidx * A.batch_stride * C::ES +
                          (C::AKC ? (int64_t)m0 * A.ld * C::ES : (int64_t)m0 * C::ES);
    const int64_t b_off = (int64_t)bidx * B.batch_stride * C::ES +
                          (C::BKC ? (int64_t)n0 * B.ld * C::ES : (int64_t)n0 * C::ES);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(static_cast<const char*>(A.ptr) + a_off, A.extent - ((int64_t)m0 * (C::AKC ? A.ld : 1) * C::ES));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(static_cast<const char*>(B.ptr) + b_off, B.extent - ((int64_t)n0 * (C::BKC ? B.ld : 1) * C::ES));
    const int64_t lda_b = A.ld * C::ES, ldb_b = B.ld * C::ES;
    const int kl = (lane >> 5) * MF::KL;

    // MFMAs of one LDS stage. With NV = 0, `stage_work(kk)` runs after
    // sub-step kk's MFMAs have been issued (staging of the register path).
    // With NV > 0, stage_work(kk) issues NV(kk) global->LDS load
    // instructions (the first two sub-steps), which are interleaved one by
    // one with that sub-step's MFMAs.
    auto compute = [&](const char* As, const char* Bs, auto nv_tag, auto&& stage_work) {
      typedef decltype(nv_tag) NV;
      typename MF::Frag fa[2][C::FM], fb[2][C::FN];
      static_for<0, C::FM>([&](auto i) { fa[0][i] = MF::read(As, wm * C::WTM + i * 32 + (lane & 31), kl); });
      static_for<0, C::FN>([&](auto j) { fb[0][j] = MF::read(Bs, wn * C::WTN + j * 32 + (lane & 31), kl); });
      __builtin_amdgcn_sched_group_barrier(0x100, C::FM + C::FN, 0);  // sub-step 0's reads lead
      static_for<0, KK>([&](auto kk) {
        constexpr int cur = kk & 1, nxt = cur ^ 1;
        constexpr int nv = NV::at(kk);
        if constexpr (kk + 1 < KK) {
          const int k = (kk + 1) * MF::KI + kl;
          static_for<0, C::FM>([&](auto i) { fa[nxt][i] = MF::read(As, wm * C::WTM + i * 32 + (lane & 31), k); });
          static_for<0, C::FN>([&](auto j) { fb[nxt][j] = MF::read(Bs, wn * C::WTN + j * 32 + (lane & 31), k); });
        }
        static_for<0, C::FM>([&](auto i) {
          static_for<0, C::FN>([&](auto j) { acc[p][i][j] = MF::mma(fa[cur][i], fb[cur][j], acc[p][i][j]); });
        });
        if constexpr (nv > 0) stage_work(kk);
        // Issue order: every fragment read of sub-step kk+1, then the MFMAs of
        // sub-step kk (with the slab loads, if any, one after every few
        // MFMAs), so the reads have a whole sub-step of MFMAs to land (left
        // alone, the scheduler issues each read just before its use).
        if constexpr (kk + 1 < KK) __builtin_amdgcn_sched_group_barrier(0x100, C::FM + C::FN, 0);
        if constexpr (nv > 0) {
          constexpr int NM = C::FM * C::FN;
          static_for<0, nv>([&](auto v) {
            constexpr int m = (NM * (v + 1)) / nv - (NM * v) / nv;  // MFMAs after load v
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
          });
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, C::FM * C::FN, 0);
        }
        if constexpr (RSS) static_for<0, C::FM>([&](auto i) { ss[i] = frag_sumsq(fa[cur][i], ss[i]); });
        if constexpr (nv == 0) stage_work(kk);
      });
    };

    if constexpr (C::DIRECT) {
      typedef DirectLoader<C, C::BM> DA;
      typedef DirectLoader<C, C::BN> DB;
      constexpr int L = DA::INSTR + DB::INSTR;  // loads per wave per K slab
      constexpr int NS = C::NSTAGE;
      // Every step issues exactly one slab (past the end of K, out of range),
      // so L * (NS-2) loads still outstanding means slab kt has landed.
      static_for<0, NS - 1>([&](auto s) {
        const uint32_t oob = s() < KT ? 0u : 0x80000000u;
        char* st = smem + s() * C::STAGE_BYTES;
        DA::issue(ra, lda_b, kbeg + s() * C::BK, st, wave, lane, oob);
        DB::issue(rb, ldb_b, kbeg + s() * C::BK, st + C::A_BYTES, wave, lane, oob);
      });
      int cur = 0;       // stage read in this step
      int nxt = NS - 1;  // stage refilled in this step
      for (int kt = 0; kt < KT; ++kt) {
        // Slabs kt .. kt+NS-2 are in flight; wait for slab kt only.
        wait_vmcnt<L * (NS - 2)>();
        // A plain s_barrier: __syncthreads() would add a release fence that
        // waits for every outstanding load, including the slabs still
        // allowed in flight. The empty asm statements keep the compiler from
        // moving LDS accesses across the barrier.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // Slab kt+NS-1 goes to the stage last read in step kt-1, which every
        // wave has finished once past the barrier. Past the end of K the
        // loads are issued out of range and fetch nothing.
        const int ks = kt + NS - 1;
        const uint32_t oob = ks < KT ? 0u : 0x80000000u;
        char* st = smem + nxt * C::STAGE_BYTES;
        const char* As = smem + cur * C::STAGE_BYTES;
        compute(As, As + C::A_BYTES, SlabPlan<DA::INSTR, DB::INSTR>{}, [&](auto kk) {
          if constexpr (kk == 0) DA::issue(ra, lda_b, kbeg + ks * C::BK, st, wave, lane, oob);
          if constexpr (kk == 1) DB::issue(rb, ldb_b, kbeg + ks * C::BK, st + C::A_BYTES, wave, lane, oob);
        });
        cur = cur + 1 == NS ? 0 : cur + 1;
        nxt = nxt + 1 == NS ? 0 : nxt + 1;
      }
      // Out-of-range loads still count; none may land after the epilogue
      // starts reusing this LDS.
      wait_vmcnt<0>();
      __syncthreads();
    } else {
      la.fetch(ra, lda_b, kbeg, t);
      lb.fetch(rb, ldb_b, kbeg, t);
      la.store(smem, t);
      lb.store(smem + C::A_BYTES, t);
      la.fetch(ra, lda_b, kbeg + C::BK, t);
      lb.fetch(rb, ldb_b, kbeg + C::BK, t);
      for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();
        const char* As = smem + (kt & 1) * C::STAGE_BYTES;
        char* Ns = smem + ((kt & 1) ^ 1) * C::STAGE_BYTES;
        // Staging work after the first two sub-steps' MFMAs have been issued:
        // each operand's slab for step kt+1 goes to the other LDS stage and
        // its registers are refilled at once with step kt+2, so every global
        // load has a whole K step to land. The scheduling barriers keep the
        // compiler from sinking the loads to the end of the step.
        compute(As, As + C::A_BYTES, SlabPlan<0, 0>{}, [&](auto kk) {
          if constexpr (kk == 0 || kk == 1) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kk == 0) {
              la.store(Ns, t);
              la.fetch(ra, lda_b, kbeg + (kt + 2) * C::BK, t);
            } else {
              lb.store(Ns + C::A_BYTES, t);
              lb.fetch(rb, ldb_b, kbeg + (kt + 2) * C::BK, t);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        });
      }
      __syncthreads();
    }
  });

  float* rowv = reinterpret_cast<float*>(smem + C::SCR_BYTES);
  float* colv = rowv + C::BM;
  if constexpr (RSS) {
    // Lanes l and l+32 hold the two k halves of the same row; waves in the
    // same wave row saw the same A rows, so wave column 0 publishes.
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const float s = ss[i] + __shfl_xor(ss[i], 32);
      if (wn == 0 && lane < 32) rowv[wm * C::WTM + i * 32 + lane] = s;
    }
    __syncthreads();
  }

  TileCtx c;
  c.m0 = m0; c.n0 = n0; c.tm = tm; c.tn = tn; c.bidx = bidx; c.split = split; c.prob = prob;
  c.M = g.M; c.N = g.N; c.t = t; c.lane = lane; c.wave = wave; c.wm = wm; c.wn = wn;
  c.smem = smem; c.rowv = rowv; c.colv = colv;
  c.rowpart = colv + C::BN;
  c.colpart = c.rowpart + C::WN * C::BM;
  epilogue<C, E>(acc, c, ea);
}

}  // namespace rbo
