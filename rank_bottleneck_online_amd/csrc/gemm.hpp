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
//   B "NC": element (k,n) at k*ld + n  (an activation when K = tokens)
// Every operand is copied from global memory straight into LDS (buffer
// loads with the LDS flag, 16 bytes per lane) in its own layout; the MFMA
// fragments are formed by the LDS reads.
//
// LDS layouts (16-byte chunks, XOR-swizzled so that both the fragment reads
// and the global requests stay conflict-free and full-line):
//   KC: one 128-byte row of K per tile row (BK = 64 bf16 / 32 fp32); chunk
//       c of row m at c ^ ((m ^ (m>>3)) & 7). A fragment read (8 rows, one
//       chunk) hits 8 distinct chunks.
//   MC/NC: one row of the tile's M (or N) extent per k; chunk c of row k at
//       c ^ (4 (k & 3)) for bf16 and c ^ (8 (k & 1)) for fp32. bf16
//       fragments come from the gfx950 transposing LDS read
//       (ds_read_b64_tr_b16), which in each group of 16 lanes gathers four k
//       rows of 16 values and hands every lane four consecutive k of its own
//       column; two such reads give the 8 k of an MFMA fragment. The four k
//       rows of a read then sit in four different bank quarters. fp32
//       fragments (one k per lane) are plain reads along a row.
// Rows of at least 128 bytes keep every global request a full cache line:
// with 64-byte rows the same slab streams measurably slower.
//
// Global loads use buffer instructions with a per-operand byte range, so
// every read past the end of a tensor returns zero: rows past T and the
// K tail of K = tokens products need no branches. Reads past M or N inside
// the tensor only feed accumulator rows/columns that the epilogue masks.
//
// Pipelining. As many LDS stages as fit (three or four for tiles smaller
// than 256 x 256): while the MFMAs read stage kt, the slabs of the next
// NSTAGE-1 steps are in flight, and each step waits only for the oldest.
// Single-accumulator tiles where only two whole slabs fit (256 x 256,
// 192 x 256, 256 x 192) stage each operand's K-step panels in a ring of
// its own instead, which keeps one and a half slabs or more in flight. The load instructions of the next slab are interleaved one by one
// with the MFMAs of the first two k sub-steps, so that a stalled load issue
// never leaves the matrix cores idle (with one wave per SIMD there is no
// other wave to fill the gap). MFMA fragments are double-buffered across
// the 16-wide k sub-steps; one barrier per K step.
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
// Single-accumulator tiles whose whole-slab stages fit only twice (256 x 256,
// 192 x 256, 256 x 192) stage each operand's K-step panels in a ring of its
// own instead (see the kernel's main loop).
constexpr bool kPanelRings = true;

// Ring depths (A slots, B slots) for panels of a and b bytes in `cap`
// bytes: the most panels in flight (all but the one being read of each
// ring), at least two slots per ring; {0, 0} if none fits. On a tie the B
// ring gets the extra slot (measured on the 256 x 256 tiles, 2 + 3 against
// 3 + 2 slots: the 7B MLP step 0.8-1.1% faster, the 40B layer 0.4-0.5%).
struct RingDepth {
  int na, nb;
};
constexpr RingDepth ring_depth(int a, int b, int cap) {
  RingDepth best{0, 0};
  int best_fl = -1;
  for (int na = 2; na <= 8; ++na)
    for (int nb = 2; nb <= 8; ++nb)
      if (na * a + nb * b <= cap) {
        const int fl = (na - 1) * a + (nb - 1) * b;
        if (fl > best_fl || (fl == best_fl && nb > best.nb)) {
          best = RingDepth{na, nb};
          best_fl = fl;
        }
      }
  return best;
}

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
  // The value a store of v would leave in memory (round to nearest even).
  static __device__ __forceinline__ float round(float v) { return static_cast<float>(static_cast<bf16>(v)); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ float round(float v) { return v; }
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
  static constexpr int RB = kRowBytes;
  static constexpr int CH = RB / 16;  // 16-byte chunks per row
  static constexpr int BK = RB / ES;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  // As many stages (up to four) as fit next to the epilogue vectors in the
  // 160 KB of a CU. A K slab of either layout is 128 bytes of K per tile row
  // or column.
  static constexpr int VEC_BYTES_ = (BM + BN + WN * BM + WM * BN) * 4;
  static constexpr int FIT_ = (160 * 1024 - VEC_BYTES_) / STAGE_BYTES;
  static constexpr int NSTAGE = FIT_ < 4 ? FIT_ : 4;
  static_assert(NSTAGE >= 2, "two pipeline stages must fit in LDS");
  // Panel rings: RA panels of A (A_BYTES each) and RB panels of B fill the
  // 160 KB, against two whole slabs plus the vectors.
  static constexpr RingDepth RD_ = ring_depth(A_BYTES, B_BYTES, 160 * 1024);
  static constexpr bool RING = kPanelRings && NACC == 1 && NSTAGE == 2 && RD_.na > 0;
  static constexpr int RA = RING ? RD_.na : 0, RBN = RING ? RD_.nb : 0;
  static constexpr int PIPE_BYTES = RING ? RA * A_BYTES + RBN * B_BYTES : NSTAGE * STAGE_BYTES;
  // Epilogue staging: each wave writes 32 accumulator rows at a time (per
  // accumulator) into a private fp32 buffer with a row stride padded by 8
  // floats (the two half-waves of the MFMA layout then hit disjoint banks;
  // odd rows are column-swizzled for the read-back), reusing the pipeline LDS.
  static constexpr int EPI_STR = WTN + 8;
  // Accumulator rows staged per round: 32 (one MFMA block row), or 16 with
  // three accumulators so the staging still fits next to the pipeline.
  static constexpr int EPI_ROWS = NACC > 2 ? 16 : 32;
  static constexpr int EPI_SUB = EPI_ROWS * EPI_STR;
  static constexpr int EPI_BYTES = WM * WN * NACC * EPI_SUB * 4;
  static constexpr int SCR_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
  // After that: per-row / per-column fp32 vectors and reduction partials.
  // They are used only after the main loop, so with the ring they sit in
  // the pipeline space, past the epilogue staging.
  static constexpr int VEC_BYTES = VEC_BYTES_;
  static constexpr int VEC_OFF = RING ? EPI_BYTES : SCR_BYTES;
  static_assert(!RING || EPI_BYTES + VEC_BYTES <= PIPE_BYTES, "ring: vectors must fit past the staging");
  static constexpr int LDS_BYTES = RING ? PIPE_BYTES : SCR_BYTES + VEC_BYTES;
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
  int krot;      // the workgroups of XCD x start their K loops krot * x / 16 of the way in
  int group;     // tile rows per group of the tile walk
};

struct GemmOps {
  Operand a[3], b[3];  // one pair per accumulator (NACC <= 3)
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
  // The same loads with less per-load work, for loops that keep per-lane
  // state: prepare() computes each instruction's lane offset once (row and
  // swizzled chunk); issue_fast() adds the slab's K offset (one add per
  // load, still range-checked), takes the LDS destination from a
  // wave-uniform index (scalar), and sends a slab that is out of range
  // through a resource of zero records instead of offsetting every lane.
  __device__ __forceinline__ static void prepare(int64_t ld_bytes, int wave, int lane, uint32_t (&vo)[INSTR]) {
#pragma unroll
    for (int q = 0; q < INSTR; ++q) {
      const int row = RPI * (q * C::NW + wave) + lane / C::CH;
      vo[q] = (uint32_t)(row * ld_bytes) + (uint32_t)(((lane % C::CH) ^ lds_swz(row)) * 16);
    }
  }
  __device__ __forceinline__ static void issue_fast(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t none, bool live,
                                                    const uint32_t (&vo)[INSTR], int k0, char* tile, int wave_s) {
    const __amdgpu_buffer_rsrc_t r = live ? rs : none;
    const uint32_t koff = (uint32_t)(k0 * C::ES);
#pragma unroll
    for (int q = 0; q < INSTR; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(tile + RPI * (q * C::NW + wave_s) * C::RB), 16,
                                               vo[q] + koff, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Direct-to-LDS loader for an M- (or N-) contiguous operand: a K slab is BK
// rows of k, each COLS values (RS bytes) wide. One instruction fills 1024
// contiguous LDS bytes, i.e. 1024/RS k rows; lane l writes slot l % CHR of
// row l / CHR and fetches the chunk that the swizzle of that row places
// there.
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ int mn_swz(int k) {
  if constexpr (C::ES == 2) return 4 * (k & 3);
  else return 8 * (k & 1);
}

template <class C, int COLS>
struct DirectLoaderMN {
  static constexpr int RS = COLS * C::ES;  // LDS bytes per k row
  static constexpr int CHR = RS / 16;      // chunks per row
  static constexpr int RPI = 1024 / RS;    // k rows per instruction
  static constexpr int INSTR = C::BK / RPI / C::NW;
  static_assert(CHR >= 16 && 1024 % RS == 0, "MN tile rows must be 256 to 1024 bytes");
  static_assert(C::BK % (RPI * C::NW) == 0, "direct loader: rows must split evenly over the waves");
  // k0: first k row of the slab (relative to the operand base); oob as for
  // the K-contiguous loader.
  __device__ __forceinline__ static void issue(__amdgpu_buffer_rsrc_t rs, int64_t ld_bytes, int k0,
                                               char* __restrict__ tile, int wave, int lane, uint32_t oob = 0) {
#pragma unroll
    for (int q = 0; q < INSTR; ++q) {
      const int row0 = RPI * (q * C::NW + wave);
      const int row = row0 + lane / CHR;
      const int chunk = (lane % CHR) ^ mn_swz<C>(row);
      const uint32_t off = ((uint32_t)((k0 + row) * ld_bytes) + (uint32_t)(chunk * 16)) | oob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + row0 * RS), 16, off, 0, 0, 0);
    }
  }
  // As for the K-contiguous loader: lane offsets once, then one add of the
  // slab's k-row offset per load.
  __device__ __forceinline__ static void prepare(int64_t ld_bytes, int wave, int lane, uint32_t (&vo)[INSTR]) {
#pragma unroll
    for (int q = 0; q < INSTR; ++q) {
      const int row = RPI * (q * C::NW + wave) + lane / CHR;
      vo[q] = (uint32_t)(row * ld_bytes) + (uint32_t)(((lane % CHR) ^ mn_swz<C>(row)) * 16);
    }
  }
  __device__ __forceinline__ static void issue_fast(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t none, bool live,
                                                    const uint32_t (&vo)[INSTR], int k0, int64_t ld_bytes,
                                                    char* __restrict__ tile, int wave_s) {
    const __amdgpu_buffer_rsrc_t r = live ? rs : none;
    const uint32_t koff = (uint32_t)(k0 * ld_bytes);
#pragma unroll
    for (int q = 0; q < INSTR; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(tile + RPI * (q * C::NW + wave_s) * RS), 16,
                                               vo[q] + koff, 0, 0, 0);
  }
};

// Whole-slab loads with the loaders' prepared lane offsets: the offsets of
// every operand pair, computed once per lane, and the slab issue that adds
// the K offset.
template <class C, class DA, class DB>
struct SlabLoads {
  uint32_t va[C::NACC][DA::INSTR], vb[C::NACC][DB::INSTR];
  __device__ __forceinline__ void prepare(const int64_t (&lda)[C::NACC], const int64_t (&ldb)[C::NACC], int wave,
                                          int lane) {
#pragma unroll
    for (int p = 0; p < C::NACC; ++p) {
      DA::prepare(lda[p], wave, lane, va[p]);
      DB::prepare(ldb[p], wave, lane, vb[p]);
    }
  }
  template <int Q, bool LA, bool LB>
  __device__ __forceinline__ void issue(const __amdgpu_buffer_rsrc_t (&ra)[C::NACC],
                                        const __amdgpu_buffer_rsrc_t (&rb)[C::NACC], __amdgpu_buffer_rsrc_t none,
                                        const int64_t (&lda)[C::NACC], const int64_t (&ldb)[C::NACC], bool live,
                                        int k0, char* st, int wave_s) const {
    if constexpr (LA) {
      if constexpr (C::AKC) DA::issue_fast(ra[Q], none, live, va[Q], k0, st, wave_s);
      else DA::issue_fast(ra[Q], none, live, va[Q], k0, lda[Q], st, wave_s);
    }
    if constexpr (LB) {
      if constexpr (C::BKC) DB::issue_fast(rb[Q], none, live, vb[Q], k0, st + C::A_BYTES, wave_s);
      else DB::issue_fast(rb[Q], none, live, vb[Q], k0, ldb[Q], st + C::A_BYTES, wave_s);
    }
  }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// MFMA fragment of an operand stored MN-major in LDS (RS bytes per k row):
// lane l gets the KL values k = k0 + KL*(l/32) + 0..KL-1 of column
// c0 + l%32 (c0 = first column of the 32-wide fragment block).
template <class C, int RS>
struct MnFrag {
  typedef typename Mfma<typename C::T>::Frag Frag;
  // `tile` is restrict-qualified, as is the destination of the direct-to-LDS
  // loads: the stage read here is never the one being filled (the slab
  // pipeline waits for a stage's loads before its first read), and without
  // that promise the compiler waits for every LDS-bound load in flight
  // before each transposing read.
  __device__ __forceinline__ static Frag read(const char* __restrict__ tile, int c0, int k0, int lane) {
    if constexpr (C::ES == 2) {
      // ds_read_b64_tr_b16: in each group g of 16 lanes, source lane j reads
      // 4 consecutive columns at one k row, and lane i receives component
      // (i & 3) of source lanes 4e + (i >> 2), e = 0..3. Source lane j of
      // group g therefore points at k row k0 + 8 (g >> 1) + (j >> 2) (+4 for
      // the second read) and columns c0 + 16 (g & 1) + 4 (j & 3).
      const int g = lane >> 4, j = lane & 15;
      const int col = c0 + 16 * (g & 1) + 4 * (j & 3);  // 4 columns = 8 bytes
      const int chunk = col >> 3, half = (col >> 2) & 1;
      const int k = k0 + 8 * (g >> 1) + (j >> 2);
      const int a0 = k * RS + ((chunk ^ mn_swz<C>(k)) << 4) + 8 * half;
      const int a1 = (k + 4) * RS + ((chunk ^ mn_swz<C>(k + 4)) << 4) + 8 * half;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + a0));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + a1));
      const v8i16 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(Frag, w);
    } else {
      const int k = k0 + (lane >> 5), col = c0 + (lane & 31);
      return *reinterpret_cast<const float*>(tile + k * RS + ((((col * 4) >> 4) ^ mn_swz<C>(k)) << 4) +
                                             ((col * 4) & 15));
    }
  }
};

// s_waitcnt vmcnt(n) with the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Where a K step issues the next slab's loads: VA instructions for A in
// sub-step PA and VB for B in sub-step PB, each interleaved with the MFMAs
// of its sub-step.
template <int VA, int PA, int VB, int PB>
struct SlabPlan {
  static constexpr int A_AT = PA, B_AT = PB;
  static constexpr int at(int kk) { return (kk == PA ? VA : 0) + (kk == PB ? VB : 0); }
};

// ---------------------------------------------------------------------------
// Block -> tile mapping. Workgroups are handed to the 8 XCDs round-robin;
// the remap gives each XCD a contiguous range of logical tiles, and tiles are
// walked in groups of GROUP tile rows (chosen per launch) so neighbours share
// A rows and B columns in that XCD's L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb >> 3, rem = nb & 7, x = b & 7;
  return x * q + (x < rem ? x : rem) + (b >> 3);
}

__device__ __forceinline__ void group_tile(int tile, int tiles_m, int tiles_n, int GROUP, int& tm, int& tn) {
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
// The accumulators are handed to the epilogue through LDS, 32 rows (16 with
// three accumulators) of each wave's tile at a time: the wave writes them in the MFMA layout into its
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
//   Pre, pre(c, a, lr, lc, pf)   global inputs of one apply, loaded early
//   apply(c, a, lr, lc, v, pf, rowc, colc)   lr/lc tile-local row / first column
//   rows_done(c, a, sums) / cols_done(c, a, sums)   sums in LDS, BM / BN long
// ---------------------------------------------------------------------------
template <class C, class E>
__device__ __forceinline__ void epilogue(floatx16 (&acc)[C::NACC][C::FM][C::FN], const TileCtx& c,
                                         const typename E::Args& ea) {
  constexpr int STR = C::EPI_STR, SUB = C::EPI_SUB;
  constexpr int ER = C::EPI_ROWS, ROUNDS = 32 / ER;
  constexpr int V8 = C::WTN / 8;        // lanes per row in the read-back
  constexpr int RPS = 64 / V8;          // rows per read-back step
  constexpr int STEPS = (ER + RPS - 1) / RPS;  // read-back steps per staging round
  // With a wave tile 32, 64 or 128 wide every lane reads back a row in
  // every step. With 96 (12 lanes per row, 5 rows per step) lanes 60-63
  // idle and the last step's rows past the round are skipped; the row and
  // column sums use lane butterflies, so reducing epilogues need the former.
  constexpr bool kFull = 64 % V8 == 0 && ER % RPS == 0;
  static_assert(kFull || !(E::kRowSum || E::kColSum), "row/column sums need a wave tile 32, 64 or 128 wide");
  static_assert(V8 <= 64 && C::WTN % 8 == 0, "wave tile width");
  float* scr = reinterpret_cast<float*>(c.smem) + c.wave * (C::NACC * SUB);
  const int c8 = c.lane % V8, rsub = c.lane / V8;

  E::template begin<C>(c, ea);
  __syncthreads();

  float colc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) colc[e] = 0.f;

  static_for<0, C::FM>([&](auto i) {
    static_for<0, ROUNDS>([&](auto h) {
      // The chunk's global inputs are requested first, so their latency
      // overlaps the staging, the barrier and each other.
      typename E::Pre pf[STEPS];
      static_for<0, STEPS>([&](auto s) {
        if (kFull || (rsub < RPS && s * RPS + rsub < ER))
          E::template pre<C>(c, ea, c.wm * C::WTM + i * 32 + h * ER + s * RPS + rsub, c.wn * C::WTN + c8 * 8,
                             pf[s]);
      });
      // MFMA register v holds row 8 (v/4) + 4 (lane/32) + v%4 of the block;
      // registers [16h/ROUNDS, 16(h+1)/ROUNDS) cover rows [h ER, (h+1) ER).
      static_for<0, C::NACC>([&](auto p) {
        static_for<0, C::FN>([&](auto j) {
          static_for<h * (16 / ROUNDS), (h + 1) * (16 / ROUNDS)>([&](auto v) {
            constexpr int r0 = (v >> 2) * 8 + (v & 3) - h * ER;
            // Odd rows hold their 4-column groups swapped in pairs (column
            // ^ 4), so the read-back of two neighbouring rows hits disjoint
            // banks; the row parity is that of v.
            scr[p * SUB + (r0 + (c.lane >> 5) * 4) * STR + ((j * 32 + (c.lane & 31)) ^ (4 * (v & 1)))] =
                acc[p][i][j][v()];
          });
        });
      });
      // Each wave stages into and reads back from its own LDS region, and
      // a wave's LDS accesses complete in order, so no workgroup barrier is
      // needed around a staging round (a barrier's release fence would also
      // wait for the output stores already issued); the empty asm keeps the
      // compiler from moving the accesses across each other.
      asm volatile("" ::: "memory");
      static_for<0, STEPS>([&](auto s) {
        const int r = s * RPS + rsub;
        if (!kFull && (rsub >= RPS || r >= ER)) return;
        const int lr = c.wm * C::WTM + i * 32 + h * ER + r;
        const int lc = c.wn * C::WTN + c8 * 8;
        float vals[C::NACC][8];
        const int swz = 4 * (r & 1);
        static_for<0, C::NACC>([&](auto p) {
          const float* src = scr + p * SUB + r * STR + c8 * 8;
          const float4 a = *reinterpret_cast<const float4*>(src + swz);
          const float4 b = *reinterpret_cast<const float4*>(src + (swz ^ 4));
          vals[p][0] = a.x; vals[p][1] = a.y; vals[p][2] = a.z; vals[p][3] = a.w;
          vals[p][4] = b.x; vals[p][5] = b.y; vals[p][6] = b.z; vals[p][7] = b.w;
        });
        float rowc = 0.f;
        E::template apply<C>(c, ea, lr, lc, vals, pf[s], rowc, colc);
        if constexpr (E::kRowSum) {
#pragma unroll
          for (int m = 1; m < V8; m <<= 1) rowc += __shfl_xor(rowc, m);
          if (c8 == 0) c.rowpart[c.wn * C::BM + lr] = rowc;
        }
      });
      asm volatile("" ::: "memory");
    });
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
// TAG only names the instantiation: launches that would otherwise share a
// kernel (the weight-gradient products) get distinct symbols, so a profiler
// can attribute each one.
template <class C, class E, int TAG = 0>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmGeom g, GemmOps ops, typename E::Args ea) {
  typedef typename C::T T;
  typedef Mfma<T> MF;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool RSS = E::kRowSumsq;
  static_assert(!RSS || C::NACC == 1, "row statistics are taken in single-accumulator products");
  static_assert(!RSS || C::AKC, "row statistics are taken from K-contiguous A fragments");

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles = g.tiles_m * g.tiles_n;
  const int prob = bid / tiles;
  int tm, tn;
  group_tile(bid - prob * tiles, g.tiles_m, g.tiles_n, g.group, tm, tn);
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

  constexpr int KK = C::BK / MF::KI;
  // Online-RMSNorm statistic: sums of squares of the A rows, taken from the
  // MFMA A fragments (each lane holds 8 k-values of one row per sub-step).
  float ss[C::FM];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) ss[i] = 0.f;

  // Buffer resources of every operand pair, rebased on this tile so 32-bit
  // buffer offsets suffice.
  __amdgpu_buffer_rsrc_t ra[C::NACC], rb[C::NACC];
  int64_t lda_b[C::NACC], ldb_b[C::NACC];
  static_for<0, C::NACC>([&](auto p) {
    const Operand& A = ops.a[p];
    const Operand& B = ops.b[p];
    const int64_t a_off = (int64_t)bidx * A.batch_stride * C::ES +
                          (C::AKC ? (int64_t)m0 * A.ld * C::ES : (int64_t)m0 * C::ES);
    const int64_t b_off = (int64_t)bidx * B.batch_stride * C::ES +
                          (C::BKC ? (int64_t)n0 * B.ld * C::ES : (int64_t)n0 * C::ES);
    ra[p] = make_rsrc(static_cast<const char*>(A.ptr) + a_off,
                      A.extent - ((int64_t)m0 * (C::AKC ? A.ld : 1) * C::ES));
    rb[p] = make_rsrc(static_cast<const char*>(B.ptr) + b_off,
                      B.extent - ((int64_t)n0 * (C::BKC ? B.ld : 1) * C::ES));
    lda_b[p] = A.ld * C::ES;
    ldb_b[p] = B.ld * C::ES;
  });
  const int kl = (lane >> 5) * MF::KL;

  // Loaders and fragment readers of this operand layout pair.
  typedef std::conditional_t<C::AKC, DirectLoader<C, C::BM>, DirectLoaderMN<C, C::BM>> DA;
  typedef std::conditional_t<C::BKC, DirectLoader<C, C::BN>, DirectLoaderMN<C, C::BN>> DB;
  auto frag_a = [&](const char* As, int i, int k) {
    if constexpr (C::AKC) return MF::read(As, wm * C::WTM + i * 32 + (lane & 31), k + kl);
    else return MnFrag<C, C::BM * C::ES>::read(As, wm * C::WTM + i * 32, k, lane);
  };
  auto frag_b = [&](const char* Bs, int j, int k) {
    if constexpr (C::BKC) return MF::read(Bs, wn * C::WTN + j * 32 + (lane & 31), k + kl);
    else return MnFrag<C, C::BN * C::ES>::read(Bs, wn * C::WTN + j * 32, k, lane);
  };

  // MFMAs of one LDS stage into accumulator p. stage_work(kk) issues the
  // NV(kk) global->LDS load instructions of a later slab, interleaved one by
  // one with that sub-step's MFMAs.
  auto compute = [&](auto p, const char* As, const char* Bs, auto nv_tag, auto&& stage_work) {
    typedef decltype(nv_tag) NV;
    typename MF::Frag fa[2][C::FM], fb[2][C::FN];
    static_for<0, C::FM>([&](auto i) { fa[0][i] = frag_a(As, i, 0); });
    static_for<0, C::FN>([&](auto j) { fb[0][j] = frag_b(Bs, j, 0); });
    // LDS read instructions per sub-step (a bf16 MN-major fragment takes two)
    constexpr int NR = C::FM * (C::AKC || C::ES == 4 ? 1 : 2) + C::FN * (C::BKC || C::ES == 4 ? 1 : 2);
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // sub-step 0's reads lead
    static_for<0, KK>([&](auto kk) {
      constexpr int cur = kk & 1, nxt = cur ^ 1;
      constexpr int nv = NV::at(kk);
      if constexpr (kk + 1 < KK) {
        const int k = (kk + 1) * MF::KI;
        static_for<0, C::FM>([&](auto i) { fa[nxt][i] = frag_a(As, i, k); });
        static_for<0, C::FN>([&](auto j) { fb[nxt][j] = frag_b(Bs, j, k); });
      }
      static_for<0, C::FM>([&](auto i) {
        static_for<0, C::FN>([&](auto j) { acc[p][i][j] = MF::mma(fa[cur][i], fb[cur][j], acc[p][i][j]); });
      });
      if constexpr (nv > 0) stage_work(kk);
      // Issue order: every fragment read of sub-step kk+1, then the MFMAs of
      // sub-step kk (with the slab loads, if any, one after every few
      // MFMAs), so the reads have a whole sub-step of MFMAs to land (left
      // alone, the scheduler issues each read just before its use).
      if constexpr (kk + 1 < KK) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
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
      // The WN waves of a wave row hold the same A fragments; each takes
      // every WN-th sub-step (a wave-uniform branch), so the sums cost each
      // wave 1/WN of the dot products.
      if constexpr (RSS) {
        if (wn == kk % C::WN) static_for<0, C::FM>([&](auto i) { ss[i] = frag_sumsq(fa[cur][i], ss[i]); });
      }
    });
  };

  constexpr int L = DA::INSTR + DB::INSTR;  // loads per wave per K slab
  // The next slab's loads go out during the first two sub-steps (the
  // restrict-qualified LDS pointers of the M/N-major loader and fragment
  // reader let the transposing reads run while those loads are in flight).
  // Measured exception: the three-stage 256 x 128 tile with M/N-major
  // operands runs faster with the loads in its last sub-step (its deeper
  // pipeline already hides the latency, and the early loads contend with
  // the transposing reads).
  static constexpr bool kLateMN = !(C::AKC && C::BKC) && C::NSTAGE == 3;
  typedef std::conditional_t<kLateMN, SlabPlan<DA::INSTR, KK - 1, DB::INSTR, KK - 1>,
                             SlabPlan<DA::INSTR, 0, DB::INSTR, 1>> Plan;
  constexpr int NS = C::NSTAGE;

  // The slabs of all accumulators form one sequence (operand pair 0's
  // slabs, then pair 1's, ...) streamed through one pipeline, so the loads
  // of the next pair overlap the last steps of the current one. Each pair
  // takes KTe = max(KT, NS-1) steps (steps past KT read zeros), so the NS-1
  // slabs in flight always belong to the current pair or the next one: the
  // K loop of pair p runs in two parts, the second of which issues the first
  // slabs of pair p+1. The pair of every load is thus a compile-time
  // constant (no runtime operand selection in the loop). Past the last pair
  // the loads are still issued, out of range (they fetch nothing), so every
  // step issues exactly one slab and L * (NS-2) loads still outstanding
  // means the slab to be read has landed.
  const int KTe = KT > NS - 1 ? KT : NS - 1;
  // K rotation by XCD. All workgroups of an XCD share its L2 and keep one K
  // order; different XCDs start at different slabs, so at any moment their
  // L2 misses go to different memory addresses instead of all asking for
  // the same K columns of rows a power of two apart (measured: long-K
  // 256 x 256 products 12-20% faster). Sums over K are then taken in a
  // rotated order; the order is fixed for a given problem, so results stay
  // bit-reproducible.
  const int krot = KT > 0 ? (int)((((blockIdx.x & 7u) * (unsigned)KT * (unsigned)g.krot) >> 4) % (unsigned)KT) : 0;
  // Loads with per-lane offsets computed once (the loaders' prepare() and
  // issue_fast()): a wave-uniform copy of the wave index for the LDS
  // destinations, and a resource of zero records for panels past K. The
  // panel rings and the whole-slab pipeline of tiles with one or two
  // accumulators use them; the three-accumulator tile, at the edge of the
  // register file, computes its offsets per load.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const __amdgpu_buffer_rsrc_t none_s = make_rsrc(ops.a[0].ptr, 0);
  constexpr bool kFastSlab = !C::RING && C::NACC <= 2 && C::ES == 2;
  SlabLoads<C, DA, DB> fast;
  if constexpr (kFastSlab) fast.prepare(lda_b, ldb_b, wave, lane);
  auto issue = [&](auto q_tag, int k, char* st, auto a_tag, auto b_tag) {
    constexpr int Q = decltype(q_tag)::value < C::NACC ? decltype(q_tag)::value : 0;
    constexpr bool past = decltype(q_tag)::value >= C::NACC;
    const bool live = !past && k < KT;
    int kr = k + krot;
    kr = kr >= KT ? kr - KT : kr;
    const int k0 = kbeg + (live ? kr : 0) * C::BK;
    if constexpr (kFastSlab) {
      fast.template issue<Q, decltype(a_tag)::value, decltype(b_tag)::value>(ra, rb, none_s, lda_b, ldb_b, live, k0, st,
                                                                             wave_u);
    } else {
      const uint32_t oob = live ? 0u : 0x80000000u;
      if constexpr (decltype(a_tag)::value) DA::issue(ra[Q], lda_b[Q], k0, st, wave, lane, oob);
      if constexpr (decltype(b_tag)::value) DB::issue(rb[Q], ldb_b[Q], k0, st + C::A_BYTES, wave, lane, oob);
    }
  };
  if constexpr (C::RING) {
    // Panel rings. K step k's panels are A_k and B_k; A_k lives in slot
    // k mod RA of the A ring and B_k in slot k mod RBN of the B ring. Step k
    // reads A_k, B_k and issues A_{k+dA} and B_{k+dB} (dA = RA-1, dB =
    // RBN-1) into the slots of A_{k-1} and B_{k-1}, which every wave has
    // finished once past the step's barrier: all panels but the ones being
    // read are in flight (one and a half to two slabs, against one with two
    // whole-slab stages). Of the two loads of a step, the one due sooner
    // goes first (first sub-step) and the other in the second. The prologue
    // issues the same sequence for steps -max(dA,dB)..-1, skipping panels
    // before index 0 (they all precede the later of A_0 and B_0), so with
    // in-order completion, at the top of step k at most W loads issued
    // after the later of A_k and B_k may be outstanding.
    constexpr int NA = C::RA, NB = C::RBN, dA = NA - 1, dB = NB - 1;
    constexpr bool aFirst = dA <= dB;
    constexpr int W = dA == dB ? (dA - 1) * L
                      : aFirst ? DB::INSTR + (dA - 1) * L : DA::INSTR + (dB - 1) * L;
    constexpr int D = dA > dB ? dA : dB;
    char* const ringA = smem;
    char* const ringB = smem + NA * C::A_BYTES;
    uint32_t voA[DA::INSTR], voB[DB::INSTR];
    DA::prepare(lda_b[0], wave, lane, voA);
    DB::prepare(ldb_b[0], wave, lane, voB);
    auto panel = [&](auto is_a, int k, char* dst) {
      const bool live = k < KT;
      int kr = k + krot;
      kr = kr >= KT ? kr - KT : kr;
      const int k0 = kbeg + (live ? kr : 0) * C::BK;
      if constexpr (decltype(is_a)::value) {
        if constexpr (C::AKC) DA::issue_fast(ra[0], none_s, live, voA, k0, dst, wave_u);
        else DA::issue_fast(ra[0], none_s, live, voA, k0, lda_b[0], dst, wave_u);
      } else {
        if constexpr (C::BKC) DB::issue_fast(rb[0], none_s, live, voB, k0, dst, wave_u);
        else DB::issue_fast(rb[0], none_s, live, voB, k0, ldb_b[0], dst, wave_u);
      }
    };
    static_for<0, D>([&](auto jj) {
      constexpr int j = (int)jj - D;  // virtual step
      constexpr int ka = j + dA, kb = j + dB;
      if constexpr (aFirst) {
        if constexpr (ka >= 0) panel(std::true_type{}, ka, ringA + ka * C::A_BYTES);
        if constexpr (kb >= 0) panel(std::false_type{}, kb, ringB + kb * C::B_BYTES);
      } else {
        if constexpr (kb >= 0) panel(std::false_type{}, kb, ringB + kb * C::B_BYTES);
        if constexpr (ka >= 0) panel(std::true_type{}, ka, ringA + ka * C::A_BYTES);
      }
    });
    int sa = 0, sb = 0;  // slots of A_k, B_k
    const int KTr = KT > 1 ? KT : 1;
    for (int k = 0; k < KTr; ++k) {
      wait_vmcnt<W>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int fa = sa == 0 ? NA - 1 : sa - 1;  // slot of A_{k-1}, refilled with A_{k+dA}
      const int fb = sb == 0 ? NB - 1 : sb - 1;
      char* const dstA = ringA + fa * C::A_BYTES;
      char* const dstB = ringB + fb * C::B_BYTES;
      typedef std::conditional_t<aFirst, SlabPlan<DA::INSTR, 0, DB::INSTR, 1>, SlabPlan<DA::INSTR, 1, DB::INSTR, 0>>
          RPlan;
      compute(std::integral_constant<int, 0>{}, ringA + sa * C::A_BYTES, ringB + sb * C::B_BYTES, RPlan{},
              [&](auto kk) {
                if constexpr (kk == RPlan::A_AT) panel(std::true_type{}, k + dA, dstA);
                else panel(std::false_type{}, k + dB, dstB);
              });
      sa = sa + 1 == NA ? 0 : sa + 1;
      sb = sb + 1 == NB ? 0 : sb + 1;
    }
  } else {
    static_for<0, NS - 1>([&](auto s) {
      issue(std::integral_constant<int, 0>{}, s(), smem + s() * C::STAGE_BYTES, std::true_type{}, std::true_type{});
    });
    int cur = 0;       // stage read in this step
    int nxt = NS - 1;  // stage refilled in this step
    // One K step on pair p whose loads fetch slab k of pair Q.
    auto step = [&](auto p, auto q_tag, int k) {
      // Slabs of the next NS-1 steps are in flight; wait for this one only.
      wait_vmcnt<L * (NS - 2)>();
      // A plain s_barrier: __syncthreads() would add a release fence that
      // waits for every outstanding load, including the slabs still allowed
      // in flight. The empty asm statements keep the compiler from moving
      // LDS accesses across the barrier.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // The slab NS-1 steps ahead goes to the stage last read in the
      // previous step, which every wave has finished once past the barrier.
      char* st = smem + nxt * C::STAGE_BYTES;
      const char* As = smem + cur * C::STAGE_BYTES;
      compute(p, As, As + C::A_BYTES, Plan{}, [&](auto kk) {
        issue(q_tag, k, st, std::bool_constant<kk == Plan::A_AT>{}, std::bool_constant<kk == Plan::B_AT>{});
      });
      cur = cur + 1 == NS ? 0 : cur + 1;
      nxt = nxt + 1 == NS ? 0 : nxt + 1;
    };
    static_for<0, C::NACC>([&](auto p) {
      constexpr int P = decltype(p)::value;
      for (int kt = 0; kt < KTe - (NS - 1); ++kt) step(p, std::integral_constant<int, P>{}, kt + NS - 1);
      for (int kt = KTe - (NS - 1); kt < KTe; ++kt)
        step(p, std::integral_constant<int, P + 1>{}, kt + NS - 1 - KTe);
    });
  }
  // Out-of-range loads still count; none may land after the epilogue
  // starts reusing this LDS.
  wait_vmcnt<0>();
  __syncthreads();

  float* rowv = reinterpret_cast<float*>(smem + C::VEC_OFF);
  float* colv = rowv + C::BM;
  float* rowpart = colv + C::BN;  // [WN][BM]
  if constexpr (RSS) {
    // Lanes l and l+32 hold the two k halves of the same row; each wave of a
    // wave row holds the sums over its share of the sub-steps. They are
    // added in wave-column order, so the result is reproducible.
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const float s = ss[i] + __shfl_xor(ss[i], 32);
      if (lane < 32) rowpart[wn * C::BM + wm * C::WTM + i * 32 + lane] = s;
    }
    __syncthreads();
    for (int r = t; r < C::BM; r += C::NT) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < C::WN; ++w) s += rowpart[w * C::BM + r];
      rowv[r] = s;
    }
    __syncthreads();
  }

  TileCtx c;
  c.m0 = m0; c.n0 = n0; c.tm = tm; c.tn = tn; c.bidx = bidx; c.split = split; c.prob = prob;
  c.M = g.M; c.N = g.N; c.t = t; c.lane = lane; c.wave = wave; c.wm = wm; c.wn = wn;
  c.smem = smem; c.rowv = rowv; c.colv = colv;
  c.rowpart = rowpart;
  c.colpart = c.rowpart + C::WN * C::BM;
  epilogue<C, E>(acc, c, ea);
}

}  // namespace rbo
