// Host side of the low-rank bottleneck block library: argument validation,
// launch planning (tile shape and K split per product, workspace layout),
// kernel launches in stream order, and optional kernel timing.
//
// The library allocates no device memory and never synchronises a stream
// (except inside boost_profiler_report, which waits on its own events).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "../../include/boost_lrblock.h"
#include "aux_kernels.hpp"
#include "epilogues.hpp"
#include "gemm.hpp"

namespace rbo {
namespace {

// ---------------------------------------------------------------------------
// Errors
// ---------------------------------------------------------------------------
thread_local std::string g_detail;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return code;
}

#define RBO_TRY(expr)            \
  do {                           \
    const int _st = (expr);      \
    if (_st != BOOST_OK) return _st; \
  } while (0)

// ---------------------------------------------------------------------------
// Kernel timing
// ---------------------------------------------------------------------------
struct ProfRec {
  const char* label;
  hipEvent_t start, stop;
};
// The timer itself is single-threaded (enabled, used and reported from one
// host thread); with it off, launches from any thread touch only their own
// thread-local slot.
struct Profiler {
  bool on = false;
  std::string filter;
  std::vector<ProfRec> recs;
  size_t used = 0;
} g_prof;
thread_local int t_prof_pending = -1;
// Measurement switch: while set, backward passes enqueue their weight
// gradients on the caller's stream (see SideFork), so every launch runs
// alone and its timed duration is its own.
bool g_serial_side = false;

void prof_begin(const char* label, hipStream_t s) {
  t_prof_pending = -1;
  if (!g_prof.on || g_prof.used >= g_prof.recs.size()) return;
  if (!g_prof.filter.empty() && !strstr(label, g_prof.filter.c_str())) return;
  ProfRec& r = g_prof.recs[g_prof.used];
  r.label = label;
  if (hipEventRecord(r.start, s) == hipSuccess) t_prof_pending = (int)g_prof.used;
}
void prof_end(hipStream_t s) {
  if (t_prof_pending < 0) return;
  if (hipEventRecord(g_prof.recs[t_prof_pending].stop, s) == hipSuccess) ++g_prof.used;
  t_prof_pending = -1;
}
// A single-kernel launch that the timer covers takes the record's events on
// the dispatch itself (the extended launch stamps them with the kernel's own
// start and end): the timed duration is the kernel's alone, as a kernel
// trace reports it, and no marker packet enters the stream.
ProfRec* prof_claim(const char* label) {
  if (!g_prof.on || g_prof.used >= g_prof.recs.size()) return nullptr;
  if (!g_prof.filter.empty() && !strstr(label, g_prof.filter.c_str())) return nullptr;
  ProfRec& r = g_prof.recs[g_prof.used];
  r.label = label;
  return &r;
}

// ---------------------------------------------------------------------------
// Tile configurations
// ---------------------------------------------------------------------------
enum CfgId { CFG_256x256 = 0, CFG_256x128 = 1, CFG_128x128 = 2, CFG_F32 = 3, CFG_192x256 = 4, CFG_256x192 = 5 };
struct CfgInfo {
  int bm, bn;
  double eff;  // relative MFMA efficiency used by the planner
};
constexpr CfgInfo kCfg[] = {{256, 256, 1.00}, {256, 128, 0.88}, {128, 128, 0.70}, {64, 64, 1.0}, {192, 256, 0.95},
                            {256, 192, 0.95}};

// bf16 tiles run 8 waves (two per SIMD): while one wave waits on a barrier,
// an LDS read or a load issue, the other keeps the matrix core busy.
template <bool AKC, bool BKC, int NACC> using C256 = Cfg<bf16, 256, 256, 2, 4, AKC, BKC, NACC>;
template <bool AKC, bool BKC, int NACC> using C256x128 = Cfg<bf16, 256, 128, 4, 2, AKC, BKC, NACC>;
template <bool AKC, bool BKC, int NACC> using C128 = Cfg<bf16, 128, 128, 2, 4, AKC, BKC, NACC>;
// 192 x 256 (96 x 64 wave tiles): for products whose 256 x 256 tiles would
// fill well under the 256 CUs in one round (8192 x 1280 outputs: 160 tiles
// of 256 x 256, 215 of 192 x 256). A must be K-contiguous (the M/N-major
// loader takes rows of 256 to 1024 bytes).
template <bool AKC, bool BKC, int NACC> using C192 = Cfg<bf16, 192, 256, 2, 4, AKC, BKC, NACC>;
// 256 x 192 (64 x 96 wave tiles): N a multiple of 192 where 256 x 256 tiles
// would leave half a round (the grouped QKV down products: 512 tiles in two
// rounds against 768 of 256 x 128 in three). B must be K-contiguous, and
// the epilogue without row or column sums (96 columns are 12 lanes).
template <bool AKC, bool BKC, int NACC> using C256N192 = Cfg<bf16, 256, 192, 4, 2, AKC, BKC, NACC>;
template <bool AKC, bool BKC, int NACC> using CF32 = Cfg<float, 64, 64, 2, 2, AKC, BKC, NACC>;

struct Choice {
  CfgId id;
  int bm, bn;
  int splits;
  int k_split;
  int tiles_m, tiles_n;
  int krot;  // K rotation by XCD, in sixteenths of the K loop per XCD index
};

// K rotation by XCD (eighths of the loop per XCD index) for loops of at
// least 1024. Measured: isolated long-K 256 x 256 products 12-20% faster;
// on the whole workloads, rotating loops of 4096 or more made the 7B MLP
// step 0.9% and the 1B QKV forward 2% faster (the 40B layer and 13B share
// unchanged) against no rotation; extending it to loops of 1024 (the K = r
// products) took another 0.3-0.7% off the 7B step, the others unchanged.
int krot_rule(CfgId, int64_t k_split) { return k_split >= 1024 ? 2 : 0; }

// Pick the tile shape (and, where a product writes fp32 partials that a
// reduction can sum, the number of K splits) minimising a simple model:
// full waves of 256 workgroups, each tile costing 2*BM*BN*Ksplit flops at a
// shape-dependent efficiency, plus the HBM traffic of split partials. kc:
// the operands are K-contiguous where the 192-wide tiles need it (A for
// 192 x 256, B for 256 x 192); narrow: the epilogue has no row or column
// sums and B is K-contiguous (the 256 x 192 tile).
Choice choose(int dtype, int64_t M, int64_t N, int64_t K, int64_t batch, bool allow_split, bool dual,
              bool kc = false, bool narrow = false) {
  Choice best{};
  double best_t = 1e300;
  const int bk = dtype == BOOST_DT_F32 ? 32 : 64;
  const CfgId ids_bf16[] = {CFG_256x256, CFG_256x128, CFG_128x128, CFG_192x256, CFG_256x192};
  const CfgId ids_dual[] = {CFG_256x128};
  const CfgId ids_f32[] = {CFG_F32};
  const CfgId* ids = dtype == BOOST_DT_F32 ? ids_f32 : (dual ? ids_dual : ids_bf16);
  const int nids = dtype == BOOST_DT_F32 ? 1 : (dual ? 1 : (kc ? (narrow ? 5 : 4) : 3));
  const int split_opts[] = {1, 2, 4, 8};
  for (int ii = 0; ii < nids; ++ii) {
    const CfgInfo& ci = kCfg[ids[ii]];
    const int64_t tm = (M + ci.bm - 1) / ci.bm, tn = (N + ci.bn - 1) / ci.bn;
    for (int s : split_opts) {
      if (s > 1 && !allow_split) break;
      int64_t ks = (K + s - 1) / s;
      ks = (ks + bk - 1) / bk * bk;
      const int64_t s_eff = (K + ks - 1) / ks;
      if (s > 1 && s_eff != s) continue;
      const double tiles = (double)tm * tn * batch * s_eff;
      const double waves = std::ceil(tiles / 256.0);
      double t = waves * (2.0 * ci.bm * ci.bn * (double)ks) / (9.8e12 * ci.eff);
      if (s_eff > 1) t += ((double)s_eff * 2.0 + 1.0) * (double)M * N * batch * 4.0 / 5.0e12 + 4e-6;
      if (t < best_t * 0.999) {
        best_t = t;
        best = Choice{ids[ii], ci.bm, ci.bn, (int)s_eff, (int)ks, (int)tm, (int)tn, krot_rule(ids[ii], ks)};
      }
    }
  }
  return best;
}

// Names of the weight-gradient launches (see gemm_kernel's TAG).
enum LaunchTag {
  TAG_NONE = 0,
  TAG_BLOCK_DB = 1,  // dB of a grouped block (mlp1_dB, lrblock_dB)
  TAG_BLOCK_DA = 2,  // dA_cat of a grouped block (mlp1_dA, lrblock_dA)
  TAG_MLP_DB2 = 3,
  TAG_MLP_DA2 = 4,
  TAG_BTP_DA = 5,
  TAG_BTP_DB = 6,
};

template <class C, class E, int TAG>
int launch_cfg(const char* label, const Choice& ch, int M, int N, int K, int batch, const GemmOps& ops,
               const typename E::Args& ea, hipStream_t s) {
  GemmGeom g;
  g.M = M; g.N = N; g.K = K; g.batch = batch; g.splits = ch.splits; g.k_split = ch.k_split; g.krot = ch.krot;
  // Tile rows per group of the tile walk: 4 (an XCD's 32 concurrent tiles
  // then cover 4 tile rows by 8 tile columns, for a 256 x 128 tile the
  // fewest operand bytes per round) except on the 192-wide tiles and short
  // K loops, which measured faster with 8 (the 1B QKV down product 7%).
  // Against 8 everywhere: the 7B MLP step 0.6-0.8% and the 40B layer
  // 0.8-1.2% faster; 16 everywhere was 3% slower.
  g.group = (C::BN != 192 && ch.k_split >= 1024) ? 4 : 8;
  g.tiles_m = cdiv(M, C::BM); g.tiles_n = cdiv(N, C::BN);
  const int64_t grid = (int64_t)g.tiles_m * g.tiles_n * batch * ch.splits;
  if (grid <= 0) return BOOST_OK;
  if (grid > 0x7fffffff) return fail(BOOST_ERR_UNSUPPORTED, "%s: grid too large", label);
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<C, E, TAG>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  (void)attr;
  ProfRec* pr = prof_claim(label);
  if (pr)
    hipExtLaunchKernelGGL((gemm_kernel<C, E, TAG>), dim3((unsigned)grid), dim3(C::NT), C::LDS_BYTES, s, pr->start,
                          pr->stop, 0, g, ops, ea);
  else
    hipLaunchKernelGGL((gemm_kernel<C, E, TAG>), dim3((unsigned)grid), dim3(C::NT), C::LDS_BYTES, s, g, ops, ea);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BOOST_ERR_LAUNCH, "%s: %s", label, hipGetErrorString(e));
  if (pr) ++g_prof.used;
  return BOOST_OK;
}

template <class E, bool AKC, bool BKC, int NACC, int TAG = TAG_NONE>
int gemm(const char* label, int dtype, const Choice& ch, int64_t M, int64_t N, int64_t K, int64_t batch,
         const GemmOps& ops, const typename E::Args& ea, hipStream_t s) {
  const int m = (int)M, n = (int)N, k = (int)K, b = (int)batch;
  if (dtype == BOOST_DT_F32) return launch_cfg<CF32<AKC, BKC, NACC>, E, TAG>(label, ch, m, n, k, b, ops, ea, s);
  if constexpr (NACC >= 2) {
    return launch_cfg<C256x128<AKC, BKC, NACC>, E, TAG>(label, ch, m, n, k, b, ops, ea, s);
  } else {
    switch (ch.id) {
      case CFG_256x256: return launch_cfg<C256<AKC, BKC, NACC>, E, TAG>(label, ch, m, n, k, b, ops, ea, s);
      case CFG_256x128: return launch_cfg<C256x128<AKC, BKC, NACC>, E, TAG>(label, ch, m, n, k, b, ops, ea, s);
      case CFG_192x256:
        if constexpr (AKC) {
          return launch_cfg<C192<AKC, BKC, NACC>, E, TAG>(label, ch, m, n, k, b, ops, ea, s);
        } else {
          return fail(BOOST_ERR_UNSUPPORTED, "%s: 192 x 256 tiles need a K-contiguous A", label);
        }
      case CFG_256x192:
        if constexpr (BKC && !E::kRowSum && !E::kColSum) {
          return launch_cfg<C256N192<AKC, BKC, NACC>, E, TAG>(label, ch, m, n, k, b, ops, ea, s);
        } else {
          return fail(BOOST_ERR_UNSUPPORTED, "%s: 256 x 192 tiles need a K-contiguous B and no row sums", label);
        }
      default: return launch_cfg<C128<AKC, BKC, NACC>, E, TAG>(label, ch, m, n, k, b, ops, ea, s);
    }
  }
}

// ---------------------------------------------------------------------------
// Operand helpers. extent = bytes from a batch base to the end of its data.
// ---------------------------------------------------------------------------
Operand opnd(const void* p, int64_t ld, int64_t rows, int64_t cols, int64_t es, int64_t bstride = 0) {
  Operand o;
  o.ptr = p;
  o.ld = ld;
  o.batch_stride = bstride;
  o.extent = ((rows - 1) * ld + cols) * es;
  return o;
}

int check_launch(const char* label) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BOOST_ERR_LAUNCH, "%s: %s", label, hipGetErrorString(e));
  return BOOST_OK;
}

int grid_for(int64_t n, int per_thread = 1) {
  const int64_t blocks = (n / per_thread + 255) / 256;
  return (int)std::max<int64_t>(1, std::min<int64_t>(blocks, 4096));
}

// One weight transpose: out[b][c][r] = scale[r] * in[b][r][c] (scale may be
// null), R x C per batch, R and C multiples of 64.
struct TJob {
  const void* in;
  const void* scale;
  void* out;
  int64_t R, C, batch;
};

// Runs up to kMaxTransposeJobs transposes: bf16 ones in a single launch,
// fp32 ones (small test shapes) one launch each.
int launch_transposes(int dtype, std::initializer_list<TJob> list, hipStream_t s) {
  if (list.size() > (size_t)kMaxTransposeJobs) return fail(BOOST_ERR_INVALID_VALUE, "too many transposes");
  prof_begin("weight_transpose", s);
  if (dtype == BOOST_DT_BF16) {
    TransposeJobs jobs{};
    int64_t blocks = 0;
    for (const TJob& t : list) {
      TransposeJob& J = jobs.j[jobs.n++];
      J.in = static_cast<const bf16*>(t.in);
      J.scale = static_cast<const bf16*>(t.scale);
      J.out = static_cast<bf16*>(t.out);
      J.R = (int)t.R;
      J.C = (int)t.C;
      J.tiles_r = (int)cdiv((int)t.R, 128);
      J.tiles_c = (int)(t.C / 64);
      J.first = (int)blocks;
      blocks += (int64_t)J.tiles_r * J.tiles_c * t.batch;
    }
    if (blocks > 0) hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, jobs);
  } else {
    for (const TJob& t : list) {
      const dim3 grid((unsigned)(t.C / 64), (unsigned)(t.R / 64), (unsigned)t.batch);
      hipLaunchKernelGGL(transpose_scale_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(t.in),
                         static_cast<const float*>(t.scale), static_cast<float*>(t.out), (int)t.R, (int)t.C);
    }
  }
  prof_end(s);
  return check_launch("weight_transpose");
}

int launch_act_quant(int dtype, const float* H, void* S, int64_t n, int act, hipStream_t s) {
  prof_begin("act_quant", s);
  if (dtype == BOOST_DT_BF16)
    hipLaunchKernelGGL(act_quant_bf16x8_kernel, dim3(grid_for(n, 8)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(H), static_cast<u32x4*>(S), n / 8, act);
  else
    hipLaunchKernelGGL(act_quant_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, H, static_cast<float*>(S),
                       n, act);
  prof_end(s);
  return check_launch("act_quant");
}

int launch_colsum(const float* part, int P, int64_t stride, int64_t N, float* out, hipStream_t s) {
  // N <= 2^26 (validated dims), so the grid fits.
  const int64_t blocks = (N + kColsumCols - 1) / kColsumCols;
  prof_begin("colsum", s);
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part, P, stride, N, out);
  prof_end(s);
  return check_launch("colsum");
}

int launch_splitk(int dtype, const float* part, int S, int64_t M, int64_t N, int64_t batch,
                  const void* rowscale, float* out, hipStream_t s) {
  const int64_t mn4 = M * N / 4;
  prof_begin("splitk_reduce", s);
  if (dtype == BOOST_DT_BF16)
    hipLaunchKernelGGL(splitk_reduce_kernel<bf16>, dim3(grid_for(mn4 * batch)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(part), S, mn4, (int)batch,
                       static_cast<const bf16*>(rowscale), N, reinterpret_cast<float4*>(out));
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3(grid_for(mn4 * batch)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(part), S, mn4, (int)batch,
                       static_cast<const float*>(rowscale), N, reinterpret_cast<float4*>(out));
  prof_end(s);
  return check_launch("splitk_reduce");
}

// A weight-gradient product out[batch][M][N] (fp32) = rowscale * (A^T-ish @ B)
// with K = tokens, through split-K partials when the plan asks for them.
template <int TAG>
int wgrad(const char* label, int dtype, const Choice& ch, int64_t M, int64_t N, int64_t K, int64_t batch,
          const GemmOps& ops, const void* rowscale, float* out, float* partial, hipStream_t s) {
  EpiStore<true>::Args ea;
  if (ch.splits > 1) {
    ea.out = partial;
    ea.ldo = N;
    ea.pstride = M * N;
    ea.rowscale = nullptr;
    RBO_TRY((gemm<EpiStore<true>, false, false, 1, TAG>(label, dtype, ch, M, N, K, batch, ops, ea, s)));
    return launch_splitk(dtype, partial, ch.splits, M, N, batch, rowscale, out, s);
  }
  ea.out = out;
  ea.ldo = N;
  ea.pstride = M * N;
  ea.rowscale = rowscale;
  return gemm<EpiStore<true>, false, false, 1, TAG>(label, dtype, ch, M, N, K, batch, ops, ea, s);
}

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
// Sub-buffers are carved at 256-byte offsets. Each sub-buffer is addressed
// on its own (a buffer resource of at most 2 GiB per GEMM operand), so the
// 2 GiB limit applies to the largest sub-buffer, not to the workspace.
struct WsLayout {
  size_t total = 0;
  size_t largest = 0;
  size_t take(size_t bytes) {
    const size_t off = total;
    total += (bytes + 255) / 256 * 256;
    largest = std::max(largest, bytes);
    return off;
  }
};

constexpr size_t kMaxTensorBytes = 0x7fffffff;  // per tensor and per workspace sub-buffer

int check_ws_parts(size_t largest, const char* what) {
  if (largest >= kMaxTensorBytes)
    return fail(BOOST_ERR_UNSUPPORTED, "%s workspace needs a %zu-byte buffer; buffers must be smaller than 2 GiB", what,
                largest);
  return BOOST_OK;
}

inline char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------
struct Range {
  const void* p;
  size_t bytes;
  const char* name;
  bool out;
  bool whole = false;  // the workspace: its sub-buffers are checked against the size limit instead
};

int check_dim64(int64_t v, const char* name) {
  if (v <= 0) return fail(BOOST_ERR_INVALID_VALUE, "%s = %lld must be positive", name, (long long)v);
  if (v % 64) return fail(BOOST_ERR_UNSUPPORTED, "%s = %lld must be a multiple of 64", name, (long long)v);
  if (v > (1 << 24)) return fail(BOOST_ERR_UNSUPPORTED, "%s = %lld too large", name, (long long)v);
  return BOOST_OK;
}
int check_T(int64_t T) {
  if (T <= 0) return fail(BOOST_ERR_INVALID_VALUE, "T = %lld must be positive", (long long)T);
  if (T > (1 << 26)) return fail(BOOST_ERR_UNSUPPORTED, "T = %lld too large", (long long)T);
  return BOOST_OK;
}
int check_dtype(int32_t dt) {
  if (dt != BOOST_DT_F32 && dt != BOOST_DT_BF16)
    return fail(BOOST_ERR_INVALID_VALUE, "dtype = %d is not BOOST_DT_F32 or BOOST_DT_BF16", dt);
  return BOOST_OK;
}
int check_act(int32_t act) {
  if (act != BOOST_ACT_IDENTITY && act != BOOST_ACT_SILU)
    return fail(BOOST_ERR_INVALID_VALUE, "act = %d is not BOOST_ACT_IDENTITY or BOOST_ACT_SILU", act);
  return BOOST_OK;
}
int check_eps(float eps) {
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(BOOST_ERR_INVALID_VALUE, "eps must be finite and >= 0");
  return BOOST_OK;
}

int check_ranges(std::vector<Range>& rs) {
  for (auto& r : rs) {
    if (r.bytes == 0) continue;
    if (!r.p) return fail(BOOST_ERR_INVALID_VALUE, "%s is NULL", r.name);
    if (!r.whole && r.bytes >= kMaxTensorBytes)
      return fail(BOOST_ERR_UNSUPPORTED, "%s is %zu bytes; tensors must be smaller than 2 GiB", r.name, r.bytes);
  }
  for (auto& r : rs)
    if (r.bytes && (reinterpret_cast<uintptr_t>(r.p) & 15))
      return fail(BOOST_ERR_MISALIGNED, "%s is not 16-byte aligned", r.name);
  for (size_t i = 0; i < rs.size(); ++i) {
    if (!rs[i].out || !rs[i].bytes) continue;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(rs[i].p), a1 = a0 + rs[i].bytes;
    for (size_t j = 0; j < rs.size(); ++j) {
      if (j == i || !rs[j].bytes) continue;
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(rs[j].p), b1 = b0 + rs[j].bytes;
      if (a0 < b1 && b0 < a1) return fail(BOOST_ERR_ALIASING, "%s overlaps %s", rs[i].name, rs[j].name);
    }
  }
  return BOOST_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need && (!ws || ws_bytes < need))
    return fail(BOOST_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0, need);
  return BOOST_OK;
}

inline size_t esize(int dtype) { return dtype == BOOST_DT_F32 ? 4 : 2; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------
// Side stream. The weight-gradient products of a backward pass depend on the
// input-gradient chain but nothing on that chain depends on them, so they run
// on a second stream that forks from the caller's stream (event record +
// wait) and joins it before the call returns: they fill the CUs that the
// chain's kernels leave idle (partial last waves, the 172-tile dA2 product,
// HBM-bound epilogues). One side stream and a few events per host thread and
// device, created on first use with the default priority and never
// destroyed; the library still allocates no device memory. Stream capture
// follows the fork and the join, so a captured backward stays one graph.
// ---------------------------------------------------------------------------
struct Side {
  hipStream_t s = nullptr;
  hipEvent_t ev[4] = {};
  int next = 0;
};

int side_for_device(Side** out) {
  constexpr int kMaxDev = 64;
  thread_local Side sides[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BOOST_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDev) return fail(BOOST_ERR_UNSUPPORTED, "device index %d", dev);
  Side& sd = sides[dev];
  if (!sd.s) {
    e = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking);
    if (e != hipSuccess) {
      sd.s = nullptr;
      return fail(BOOST_ERR_LAUNCH, "hipStreamCreateWithFlags: %s", hipGetErrorString(e));
    }
    for (hipEvent_t& ev : sd.ev) {
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) return fail(BOOST_ERR_LAUNCH, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
    }
  }
  *out = &sd;
  return BOOST_OK;
}

// `to` waits for everything enqueued on `from` so far.
int stream_after(hipStream_t to, hipStream_t from, Side* sd) {
  hipEvent_t ev = sd->ev[sd->next];
  sd->next = (sd->next + 1) % 4;
  hipError_t e = hipEventRecord(ev, from);
  if (e == hipSuccess) e = hipStreamWaitEvent(to, ev, 0);
  if (e != hipSuccess) return fail(BOOST_ERR_LAUNCH, "stream fork/join: %s", hipGetErrorString(e));
  return BOOST_OK;
}

// Fork of the side stream off the caller's stream with a guaranteed join:
// once a fork has been enqueued, the caller's stream is made to wait for the
// side stream before the entry point returns, on the success path (join(),
// whose status is reported) and on every error path (the destructor, which
// keeps the first error). So whatever a backward returns, work it enqueued
// on the side stream is ordered before later work on the caller's stream,
// and a stream capture never ends with the side stream unjoined.
// With the measurement switch g_serial_side set (read once, at
// construction), side() is the caller's stream and fork/join do nothing.
class SideFork {
 public:
  SideFork(Side* sd, hipStream_t main) : sd_(sd), main_(main), serial_(g_serial_side) {}
  ~SideFork() {
    if (forked_) {
      const std::string keep = g_detail;
      (void)stream_after(main_, sd_->s, sd_);
      g_detail = keep;
    }
  }
  SideFork(const SideFork&) = delete;
  SideFork& operator=(const SideFork&) = delete;
  hipStream_t side() const { return serial_ ? main_ : sd_->s; }
  // The side stream waits for everything enqueued on the caller's so far.
  int fork() {
    if (serial_) return BOOST_OK;
    RBO_TRY(stream_after(sd_->s, main_, sd_));
    forked_ = true;
    return BOOST_OK;
  }
  // The caller's stream waits for the side stream.
  int join() {
    if (!forked_) return BOOST_OK;
    forked_ = false;
    return stream_after(main_, sd_->s, sd_);
  }

 private:
  Side* sd_;
  hipStream_t main_;
  bool serial_;
  bool forked_ = false;
};

// ===========================================================================
// Grouped block
// ===========================================================================
int lrblock_check_desc(const boost_lrblock_desc* d) {
  if (!d) return fail(BOOST_ERR_INVALID_VALUE, "desc is NULL");
  if (d->abi_version != BOOST_ABI_VERSION)
    return fail(BOOST_ERR_VERSION, "desc->abi_version = %d, library is %d", d->abi_version, BOOST_ABI_VERSION);
  RBO_TRY(check_dtype(d->dtype));
  RBO_TRY(check_act(d->act));
  if (d->norm != 0 && d->norm != 1) return fail(BOOST_ERR_INVALID_VALUE, "norm = %d must be 0 or 1", d->norm);
  RBO_TRY(check_T(d->T));
  RBO_TRY(check_dim64(d->d, "d"));
  RBO_TRY(check_dim64(d->r, "r"));
  RBO_TRY(check_dim64(d->d_out, "d_out"));
  if (d->G < 1 || d->G > 16) return fail(BOOST_ERR_INVALID_VALUE, "G = %lld must be in [1, 16]", (long long)d->G);
  if (d->norm && d->d_norm < d->d)
    return fail(BOOST_ERR_INVALID_VALUE, "d_norm = %lld must be >= d = %lld", (long long)d->d_norm, (long long)d->d);
  RBO_TRY(check_eps(d->eps));
  return BOOST_OK;
}

struct LrblockPlan {
  Choice down, up, ds, dB, dA, dx;
  size_t f_AT, f_S, f_part, fwd_bytes;
  size_t b_S, b_dU, b_q, b_dg, b_part, bwd_bytes;
  size_t fwd_largest, bwd_largest;
};

LrblockPlan lrblock_plan(const boost_lrblock_desc* d) {
  LrblockPlan p{};
  const int dt = d->dtype;
  const int64_t T = d->T, D = d->d, r = d->r, G = d->G, n = d->d_out, es = esize(dt);
  p.down = choose(dt, T, G * r, D, 1, false, false, true, true);
  p.up = choose(dt, T, n, r, G, false, false, true);
  p.ds = choose(dt, T, r, n, G, false, false, true);
  p.dB = choose(dt, r, n, T, G, true, false);
  p.dA = choose(dt, D, G * r, T, 1, true, false);
  p.dx = choose(dt, T, D, G * r, 1, false, false, true);
  WsLayout f;
  p.f_AT = f.take((size_t)(D * G * r * es));
  p.f_S = f.take((size_t)(T * G * r * es));
  // per-tile-column partial row sums of Y^2 (next block's statistic, G = 1)
  p.f_part = G == 1 ? f.take((size_t)(p.up.tiles_n * T * 4)) : 0;
  p.fwd_bytes = f.total;
  p.fwd_largest = f.largest;
  WsLayout b;
  p.b_S = b.take((size_t)(T * G * r * es));
  p.b_dU = b.take((size_t)(T * G * r * es));
  p.b_q = d->norm ? b.take((size_t)(G * p.ds.tiles_n * T * 4)) : 0;
  p.b_dg = d->norm ? b.take((size_t)(p.dx.tiles_m * D * 4)) : 0;
  size_t part = 0;
  if (p.dB.splits > 1) part = std::max(part, (size_t)(p.dB.splits * G * r * n * 4));
  if (p.dA.splits > 1) part = std::max(part, (size_t)(p.dA.splits * D * G * r * 4));
  p.b_part = part ? b.take(part) : 0;
  p.bwd_bytes = b.total;
  p.bwd_largest = b.largest;
  return p;
}

int lrblock_fwd_impl(const boost_lrblock_desc* d, const void* x, const void* g, const void* A_cat, const void* B,
                     const void* residual, const float* sumsq_in, void* Y, float* H, float* sumsq,
                     float* sumsq_next, void* ws, hipStream_t s) {
  const int dt = d->dtype;
  const int64_t T = d->T, D = d->d, r = d->r, G = d->G, n = d->d_out, es = esize(dt);
  const LrblockPlan p = lrblock_plan(d);
  void* S = at(ws, p.f_S);
  void* AT = at(ws, p.f_AT);
  // The down product's weight K-contiguous, (g * A_cat)^T [G*r, d] (the gain
  // folded in). The up product reads B_j as stored, N-contiguous: measured
  // on one box each way, the 40B-shaped layer 8.57-8.59 -> 8.51-8.52 ms and
  // the 1B QKV forward 0.278-0.281 -> 0.269-0.271 ms, the up product within
  // noise of its K-contiguous time and the B transpose gone.
  RBO_TRY(launch_transposes(dt, {{A_cat, d->norm ? g : nullptr, AT, D, G * r, 1}}, s));
  // Down: H = rho * (x @ (g * A_cat)), S = act(H), sumsq.
  {
    GemmOps ops{};
    ops.a[0] = opnd(x, D, T, D, es);
    ops.b[0] = opnd(AT, D, G * r, D, es);
    if (d->norm && sumsq_in) {
      EpiDown<true, true>::Args ea{H, S, sumsq, G * r, 1.f / (float)d->d_norm, d->eps, d->act, sumsq_in};
      RBO_TRY((gemm<EpiDown<true, true>, true, true, 1>("lrblock_down", dt, p.down, T, G * r, D, 1, ops, ea, s)));
    } else if (d->norm) {
      EpiDown<true>::Args ea{H, S, sumsq, G * r, 1.f / (float)d->d_norm, d->eps, d->act, nullptr};
      RBO_TRY((gemm<EpiDown<true>, true, true, 1>("lrblock_down", dt, p.down, T, G * r, D, 1, ops, ea, s)));
    } else {
      EpiDown<false>::Args ea{H, S, nullptr, G * r, 0.f, 0.f, d->act, nullptr};
      RBO_TRY((gemm<EpiDown<false>, true, true, 1>("lrblock_down", dt, p.down, T, G * r, D, 1, ops, ea, s)));
    }
  }
  // Up, batched over groups: Y_j = S_j @ B_j (+ the residual, and the next
  // block's row sums of squares, when G = 1).
  {
    GemmOps ops{};
    ops.a[0] = opnd(S, G * r, T, r, es, r);
    ops.b[0] = opnd(B, n, r, n, es, r * n);
    if (residual || sumsq_next) {
      float* part = sumsq_next ? reinterpret_cast<float*>(at(ws, p.f_part)) : nullptr;
      EpiUpRes::Args ea{Y, n, residual, part};
      RBO_TRY((gemm<EpiUpRes, true, false, 1>("lrblock_up", dt, p.up, T, n, r, 1, ops, ea, s)));
      if (sumsq_next) RBO_TRY(launch_colsum(part, p.up.tiles_n, T, T, sumsq_next, s));
    } else {
      EpiStore<false>::Args ea{Y, n, T * n, nullptr};
      RBO_TRY((gemm<EpiStore<false>, true, false, 1>("lrblock_up", dt, p.up, T, n, r, G, ops, ea, s)));
    }
  }
  return BOOST_OK;
}

// Kernel labels (static strings: the profiler keeps the pointers).
struct BwdLabels {
  const char *ds, *dB, *dA, *dx;
};
constexpr BwdLabels kLrblockLabels{"lrblock_ds", "lrblock_dB", "lrblock_dA", "lrblock_dx"};
constexpr BwdLabels kMlp1Labels{"mlp1_ds", "mlp1_dB", "mlp1_dA", "mlp1_dx"};

// Backward of one grouped block given the recomputed-or-available S.
// If S_ready is false, the dS epilogue recomputes S = act(H) into ws.
int lrblock_bwd_core(int dt, int act, int norm, int64_t T, int64_t D, int64_t r, int64_t G, int64_t n,
                     float eps, int64_t d_norm, const void* x, const void* g, const void* A_cat, const void* B,
                     const float* H, const float* sumsq, const void* dY, void* dx, float* dg, float* dA_cat,
                     float* dB, void* S, bool S_ready, void* dU, float* qpart, float* dgpart, float* partial,
                     const Choice& c_ds, const Choice& c_dB, const Choice& c_dA, const Choice& c_dx,
                     hipStream_t s, const BwdLabels& L, SideFork* side, const void* dadd = nullptr) {
  const int64_t es = esize(dt);
  const float inv = norm ? 1.f / (float)d_norm : 0.f;
  // dS_j = dY_j @ B_j^T, fused: dH, dU = rho dH, S = act(H), row partials q.
  {
    GemmOps ops{};
    ops.a[0] = opnd(dY, n, T, n, es, T * n);
    ops.b[0] = opnd(B, n, r, n, es, r * n);
    if (norm) {
      EpiDS<true>::Args ea{H, G * r, r, dU, S_ready ? nullptr : S, qpart, T, sumsq, inv, eps, act};
      RBO_TRY((gemm<EpiDS<true>, true, true, 1>(L.ds, dt, c_ds, T, r, n, G, ops, ea, s)));
    } else {
      EpiDS<false>::Args ea{H, G * r, r, dU, S_ready ? nullptr : S, nullptr, T, nullptr, 0.f, 0.f, act};
      RBO_TRY((gemm<EpiDS<false>, true, true, 1>(L.ds, dt, c_ds, T, r, n, G, ops, ea, s)));
    }
  }
  // The weight gradients go to the side stream (it waits for dS, which
  // produces dU and, here, S); dx stays on the caller's stream.
  const hipStream_t sw = side ? side->side() : s;
  if (side) RBO_TRY(side->fork());
  // dB_j = S_j^T @ dY_j  (K = T).
  {
    GemmOps ops{};
    ops.a[0] = opnd(S, G * r, T, r, es, r);
    ops.b[0] = opnd(dY, n, T, n, es, T * n);
    RBO_TRY(wgrad<TAG_BLOCK_DB>(L.dB, dt, c_dB, r, n, T, G, ops, nullptr, dB, partial, sw));
  }
  // dA_cat = diag(g) (x^T @ dU)  (K = T); the gain row scale is exact in fp32.
  {
    GemmOps ops{};
    ops.a[0] = opnd(x, D, T, D, es);
    ops.b[0] = opnd(dU, G * r, T, G * r, es);
    RBO_TRY(wgrad<TAG_BLOCK_DA>(L.dA, dt, c_dA, D, G * r, T, 1, ops, norm ? g : nullptr, dA_cat, partial, sw));
  }
  // dx~ = dU @ A_cat^T, fused with the RMSNorm backward and dg partials.
  {
    GemmOps ops{};
    ops.a[0] = opnd(dU, G * r, T, G * r, es);
    ops.b[0] = opnd(A_cat, G * r, D, G * r, es);
    if (norm) {
      EpiDX::Args ea{x, g, sumsq, qpart, (int)(G * c_ds.tiles_n), T, inv, eps, dx, dgpart, D, dadd};
      RBO_TRY((gemm<EpiDX, true, true, 1>(L.dx, dt, c_dx, T, D, G * r, 1, ops, ea, s)));
      RBO_TRY(launch_colsum(dgpart, c_dx.tiles_m, D, D, dg, s));
    } else {
      EpiStore<false>::Args ea{dx, D, 0, nullptr};
      RBO_TRY((gemm<EpiStore<false>, true, true, 1>(L.dx, dt, c_dx, T, D, G * r, 1, ops, ea, s)));
    }
  }
  // Join: the caller's stream waits for the weight gradients.
  if (side) RBO_TRY(side->join());
  return BOOST_OK;
}

// ===========================================================================
// MLP
// ===========================================================================
int lrmlp_check_desc(const boost_lrmlp_desc* d) {
  if (!d) return fail(BOOST_ERR_INVALID_VALUE, "desc is NULL");
  if (d->abi_version != BOOST_ABI_VERSION)
    return fail(BOOST_ERR_VERSION, "desc->abi_version = %d, library is %d", d->abi_version, BOOST_ABI_VERSION);
  RBO_TRY(check_dtype(d->dtype));
  RBO_TRY(check_act(d->act));
  if (d->reserved != 0) return fail(BOOST_ERR_INVALID_VALUE, "reserved must be 0");
  RBO_TRY(check_T(d->T));
  RBO_TRY(check_dim64(d->d, "d"));
  RBO_TRY(check_dim64(d->r, "r"));
  RBO_TRY(check_dim64(d->ffn, "ffn"));
  RBO_TRY(check_eps(d->eps));
  return BOOST_OK;
}

struct LrmlpPlan {
  Choice down1, dual, down2, up2;                       // forward
  Choice ds2, dB2, rec, dA2, ds1, dB1, dA1, dx1;        // backward
  size_t f_A1T, f_B2T, f_S1, f_M, f_S2, f_part, fwd_bytes;
  size_t b_B1T, b_S2, b_dU2, b_S1, b_M, b_dY, b_dU1, b_q, b_dg, b_part, bwd_bytes;
  size_t fwd_largest, bwd_largest;
};

LrmlpPlan lrmlp_plan(const boost_lrmlp_desc* d) {
  LrmlpPlan p{};
  const int dt = d->dtype;
  const int64_t T = d->T, D = d->d, r = d->r, F = d->ffn, es = esize(dt);
  p.down1 = choose(dt, T, 2 * r, D, 1, false, false, true, true);
  p.dual = choose(dt, T, F, r, 1, false, true);
  p.down2 = choose(dt, T, r, F, 1, false, false);
  p.up2 = choose(dt, T, D, r, 1, false, false, true);
  p.ds2 = choose(dt, T, r, D, 1, false, false, true);
  p.dB2 = choose(dt, r, D, T, 1, true, false);
  p.rec = p.dual;
  p.dA2 = choose(dt, F, r, T, 1, true, false);
  p.ds1 = choose(dt, T, r, F, 2, false, false, true);
  p.dB1 = choose(dt, r, F, T, 2, true, false);
  p.dA1 = choose(dt, D, 2 * r, T, 1, true, false);
  p.dx1 = choose(dt, T, D, 2 * r, 1, false, false, true);
  WsLayout f;
  p.f_A1T = f.take((size_t)(D * 2 * r * es));
  p.f_B2T = f.take((size_t)(r * D * es));
  p.f_S1 = f.take((size_t)(T * 2 * r * es));
  p.f_M = f.take((size_t)(T * F * es));
  p.f_S2 = f.take((size_t)(T * r * es));
  p.f_part = f.take((size_t)(p.up2.tiles_n * T * 4));  // next block's statistic partials
  p.fwd_bytes = f.total;
  p.fwd_largest = f.largest;
  WsLayout b;
  p.b_B1T = b.take((size_t)(2 * r * F * es));
  p.b_S2 = b.take((size_t)(T * r * es));
  p.b_dU2 = b.take((size_t)(T * r * es));
  p.b_S1 = b.take((size_t)(T * 2 * r * es));
  p.b_M = b.take((size_t)(T * F * es));
  p.b_dY = b.take((size_t)(2 * T * F * es));
  p.b_dU1 = b.take((size_t)(T * 2 * r * es));
  p.b_q = b.take((size_t)(2 * p.ds1.tiles_n * T * 4));
  p.b_dg = b.take((size_t)(p.dx1.tiles_m * D * 4));
  size_t part = 0;
  if (p.dB2.splits > 1) part = std::max(part, (size_t)(p.dB2.splits * r * D * 4));
  if (p.dA2.splits > 1) part = std::max(part, (size_t)(p.dA2.splits * F * r * 4));
  if (p.dB1.splits > 1) part = std::max(part, (size_t)(p.dB1.splits * 2 * r * F * 4));
  if (p.dA1.splits > 1) part = std::max(part, (size_t)(p.dA1.splits * D * 2 * r * 4));
  p.b_part = part ? b.take(part) : 0;
  p.bwd_bytes = b.total;
  p.bwd_largest = b.largest;
  return p;
}

// ===========================================================================
// Tensor-parallel share
// ===========================================================================
int btp_check_desc(const boost_btp_share_desc* d) {
  if (!d) return fail(BOOST_ERR_INVALID_VALUE, "desc is NULL");
  if (d->abi_version != BOOST_ABI_VERSION)
    return fail(BOOST_ERR_VERSION, "desc->abi_version = %d, library is %d", d->abi_version, BOOST_ABI_VERSION);
  RBO_TRY(check_dtype(d->dtype));
  RBO_TRY(check_T(d->T));
  RBO_TRY(check_dim64(d->r, "r"));
  RBO_TRY(check_dim64(d->d_shard, "d_shard"));
  return BOOST_OK;
}

struct BtpPlan {
  Choice u, p, e, dA, dB, dz;
  size_t f_ag, f_sp, fwd_bytes;
  // dA_s and dB_s run one after the other and share the split-K partials.
  size_t b_U, b_du, b_ag, b_dg, b_part, bwd_bytes;
  size_t fwd_largest, bwd_largest;
};

BtpPlan btp_plan(const boost_btp_share_desc* d) {
  BtpPlan p{};
  const int dt = d->dtype;
  const int64_t T = d->T, r = d->r, S = d->d_shard, es = esize(dt);
  p.u = choose(dt, T, S, r, 1, false, false, true);
  p.p = choose(dt, T, r, S, 1, false, false, true);
  p.e = choose(dt, T, S, r, 1, false, false, true);
  p.dA = choose(dt, S, r, T, 1, true, false);
  p.dB = choose(dt, r, S, T, 1, true, false);
  p.dz = choose(dt, T, r, S, 1, false, false, true, true);
  WsLayout f;
  p.f_ag = f.take((size_t)(T * S * es));
  p.f_sp = f.take((size_t)(p.u.tiles_n * T * 4));
  p.fwd_bytes = f.total;
  p.fwd_largest = f.largest;
  WsLayout b;
  p.b_U = b.take((size_t)(T * S * 4));
  p.b_du = b.take((size_t)(T * S * es));
  p.b_ag = b.take((size_t)(T * S * es));
  p.b_dg = b.take((size_t)(p.e.tiles_m * S * 4));
  const size_t part = std::max(p.dA.splits > 1 ? (size_t)(p.dA.splits * S * r * 4) : (size_t)0,
                               p.dB.splits > 1 ? (size_t)(p.dB.splits * r * S * 4) : (size_t)0);
  p.b_part = part ? b.take(part) : 0;
  p.bwd_bytes = b.total;
  p.bwd_largest = b.largest;
  return p;
}

// ---------------------------------------------------------------------------
// Fixed scratch for the forward that allocates nothing. Each device that
// loads the library holds one copy of this array until the process ends; a
// host-side reference to `scratch` is only a stand-in, so its device address
// is looked up once per device (with that device current) and kept.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

int noalloc_scratch(void** out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BOOST_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDev) return fail(BOOST_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(BOOST_ERR_LAUNCH, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return BOOST_OK;
}

}  // namespace
}  // namespace rbo

using namespace rbo;

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int boost_abi_version(void) { return BOOST_ABI_VERSION; }

const char* boost_status_string(int st) {
  switch (st) {
    case BOOST_OK: return "BOOST_OK";
    case BOOST_ERR_INVALID_VALUE: return "BOOST_ERR_INVALID_VALUE";
    case BOOST_ERR_UNSUPPORTED: return "BOOST_ERR_UNSUPPORTED";
    case BOOST_ERR_MISALIGNED: return "BOOST_ERR_MISALIGNED";
    case BOOST_ERR_ALIASING: return "BOOST_ERR_ALIASING";
    case BOOST_ERR_WORKSPACE: return "BOOST_ERR_WORKSPACE";
    case BOOST_ERR_VERSION: return "BOOST_ERR_VERSION";
    case BOOST_ERR_LAUNCH: return "BOOST_ERR_LAUNCH";
    default: return "BOOST_ERR_UNKNOWN";
  }
}

const char* boost_last_error_detail(void) { return g_detail.c_str(); }

// ----------------------------- grouped block ------------------------------
int boost_lrblock_workspace_size(const boost_lrblock_desc* d, int is_bwd, size_t* bytes) {
  g_detail.clear();
  RBO_TRY(lrblock_check_desc(d));
  if (!bytes) return fail(BOOST_ERR_INVALID_VALUE, "bytes is NULL");
  const LrblockPlan p = lrblock_plan(d);
  RBO_TRY(check_ws_parts(is_bwd ? p.bwd_largest : p.fwd_largest, is_bwd ? "backward" : "forward"));
  *bytes = is_bwd ? p.bwd_bytes : p.fwd_bytes;
  return BOOST_OK;
}

int boost_lrblock_fwd_chained(const boost_lrblock_desc* d, const void* x, const void* g, const void* A_cat,
                              const void* B, const void* residual, const float* sumsq_in, void* Y, float* H,
                              float* sumsq, float* sumsq_next, void* ws, size_t ws_bytes, void* stream) {
  g_detail.clear();
  RBO_TRY(lrblock_check_desc(d));
  const size_t es = esize(d->dtype);
  const size_t T = d->T, D = d->d, r = d->r, G = d->G, n = d->d_out;
  if ((residual || sumsq_next) && G != 1)
    return fail(BOOST_ERR_UNSUPPORTED, "residual / sumsq_next need G = 1 (G = %lld)", (long long)G);
  if (sumsq_in && !d->norm) return fail(BOOST_ERR_INVALID_VALUE, "sumsq_in given but norm = 0");
  const LrblockPlan p = lrblock_plan(d);
  std::vector<Range> rs = {
      {x, T * D * es, "x", false},
      {g, d->norm ? D * es : 0, "g", false},
      {A_cat, D * G * r * es, "A_cat", false},
      {B, G * r * n * es, "B", false},
      {residual, residual ? T * n * es : 0, "residual", false},
      {sumsq_in, sumsq_in ? T * 4 : 0, "sumsq_in", false},
      {Y, G * T * n * es, "Y", true},
      {H, T * G * r * 4, "H", true},
      {sumsq, d->norm && (!sumsq_in || sumsq) ? T * 4 : 0, "sumsq", true},
      {sumsq_next, sumsq_next ? T * 4 : 0, "sumsq_next", true},
      {ws, (ws && p.fwd_bytes <= ws_bytes) ? p.fwd_bytes : 0, "ws", true, true},
  };
  RBO_TRY(check_ranges(rs));
  RBO_TRY(check_ws_parts(p.fwd_largest, "forward"));
  RBO_TRY(check_ws(ws, ws_bytes, p.fwd_bytes));
  return lrblock_fwd_impl(d, x, g, A_cat, B, residual, sumsq_in, Y, H, sumsq, sumsq_next, ws, as_stream(stream));
}

int boost_lrblock_fwd(const boost_lrblock_desc* d, const void* x, const void* g, const void* A_cat, const void* B,
                      void* Y, float* H, float* sumsq, void* ws, size_t ws_bytes, void* stream) {
  return boost_lrblock_fwd_chained(d, x, g, A_cat, B, nullptr, nullptr, Y, H, sumsq, nullptr, ws, ws_bytes, stream);
}

int boost_lrblock_fwd_noalloc(const boost_lrblock_desc* d, const void* x, const void* g, const void* A_cat,
                              const void* B, void* Y, float* H, float* sumsq, void* stream) {
  g_detail.clear();
  RBO_TRY(lrblock_check_desc(d));
  const size_t es = esize(d->dtype);
  const size_t T = d->T, D = d->d, r = d->r, G = d->G, n = d->d_out;
  const LrblockPlan p = lrblock_plan(d);
  std::vector<Range> rs = {
      {x, T * D * es, "x", false},
      {g, d->norm ? D * es : 0, "g", false},
      {A_cat, D * G * r * es, "A_cat", false},
      {B, G * r * n * es, "B", false},
      {Y, G * T * n * es, "Y", true},
      {H, T * G * r * 4, "H", true},
      {sumsq, d->norm ? T * 4 : 0, "sumsq", true},
  };
  RBO_TRY(check_ranges(rs));
  if (p.fwd_bytes > kNoAllocScratchBytes)
    return fail(BOOST_ERR_UNSUPPORTED, "needs %zu bytes of scratch; the fixed scratch holds %zu", p.fwd_bytes,
                kNoAllocScratchBytes);
  void* ws = nullptr;
  RBO_TRY(noalloc_scratch(&ws));
  // The scratch is the library's own memory; no caller tensor may lie in it.
  rs.push_back({ws, p.fwd_bytes, "scratch", true});
  RBO_TRY(check_ranges(rs));
  return lrblock_fwd_impl(d, x, g, A_cat, B, nullptr, nullptr, Y, H, sumsq, nullptr, ws, as_stream(stream));
}

int boost_lrblock_bwd_chained(const boost_lrblock_desc* d, const void* x, const void* g, const void* A_cat,
                              const void* B, const float* H, const float* sumsq, const void* dY, const void* dx_add,
                              void* dx, float* dg, float* dA_cat, float* dB, void* ws, size_t ws_bytes,
                              void* stream) {
  g_detail.clear();
  RBO_TRY(lrblock_check_desc(d));
  const size_t es = esize(d->dtype);
  const size_t T = d->T, D = d->d, r = d->r, G = d->G, n = d->d_out;
  if (dx_add && !d->norm) return fail(BOOST_ERR_UNSUPPORTED, "dx_add needs norm = 1");
  const LrblockPlan p = lrblock_plan(d);
  std::vector<Range> rs = {
      {x, T * D * es, "x", false},
      {g, d->norm ? D * es : 0, "g", false},
      {A_cat, D * G * r * es, "A_cat", false},
      {B, G * r * n * es, "B", false},
      {H, T * G * r * 4, "H", false},
      {sumsq, d->norm ? T * 4 : 0, "sumsq", false},
      {dY, G * T * n * es, "dY", false},
      {dx_add, dx_add ? T * D * es : 0, "dx_add", false},
      {dx, T * D * es, "dx", true},
      {dg, d->norm ? D * 4 : 0, "dg", true},
      {dA_cat, D * G * r * 4, "dA_cat", true},
      {dB, G * r * n * 4, "dB", true},
      {ws, (ws && p.bwd_bytes <= ws_bytes) ? p.bwd_bytes : 0, "ws", true, true},
  };
  RBO_TRY(check_ranges(rs));
  RBO_TRY(check_ws_parts(p.bwd_largest, "backward"));
  RBO_TRY(check_ws(ws, ws_bytes, p.bwd_bytes));
  Side* sd = nullptr;
  RBO_TRY(side_for_device(&sd));
  SideFork side(sd, as_stream(stream));
  return lrblock_bwd_core(d->dtype, d->act, d->norm, d->T, d->d, d->r, d->G, d->d_out, d->eps, d->d_norm, x, g,
                          A_cat, B, H, sumsq, dY, dx, dg, dA_cat, dB, at(ws, p.b_S), false, at(ws, p.b_dU),
                          d->norm ? reinterpret_cast<float*>(at(ws, p.b_q)) : nullptr,
                          d->norm ? reinterpret_cast<float*>(at(ws, p.b_dg)) : nullptr,
                          p.b_part ? reinterpret_cast<float*>(at(ws, p.b_part)) : nullptr, p.ds, p.dB, p.dA, p.dx,
                          as_stream(stream), kLrblockLabels, &side, dx_add);
}

int boost_lrblock_bwd(const boost_lrblock_desc* d, const void* x, const void* g, const void* A_cat, const void* B,
                      const float* H, const float* sumsq, const void* dY, void* dx, float* dg, float* dA_cat,
                      float* dB, void* ws, size_t ws_bytes, void* stream) {
  return boost_lrblock_bwd_chained(d, x, g, A_cat, B, H, sumsq, dY, nullptr, dx, dg, dA_cat, dB, ws, ws_bytes,
                                   stream);
}

// ---------------------------------- MLP -----------------------------------
int boost_lrmlp_workspace_size(const boost_lrmlp_desc* d, int is_bwd, size_t* bytes) {
  g_detail.clear();
  RBO_TRY(lrmlp_check_desc(d));
  if (!bytes) return fail(BOOST_ERR_INVALID_VALUE, "bytes is NULL");
  const LrmlpPlan p = lrmlp_plan(d);
  RBO_TRY(check_ws_parts(is_bwd ? p.bwd_largest : p.fwd_largest, is_bwd ? "backward" : "forward"));
  *bytes = is_bwd ? p.bwd_bytes : p.fwd_bytes;
  return BOOST_OK;
}

int boost_lrmlp_fwd_chained(const boost_lrmlp_desc* d, const void* x, const void* g, const void* A1_cat,
                            const void* B1, const void* A2, const void* B2, const void* residual,
                            const float* sumsq_in, void* Y, float* H1, float* H2, float* sumsq, float* sumsq_next,
                            void* ws, size_t ws_bytes, void* stream) {
  g_detail.clear();
  RBO_TRY(lrmlp_check_desc(d));
  const int dt = d->dtype;
  const size_t es = esize(dt);
  const int64_t T = d->T, D = d->d, r = d->r, F = d->ffn;
  const LrmlpPlan p = lrmlp_plan(d);
  std::vector<Range> rs = {
      {x, (size_t)(T * D) * es, "x", false},
      {g, (size_t)D * es, "g", false},
      {A1_cat, (size_t)(D * 2 * r) * es, "A1_cat", false},
      {B1, (size_t)(2 * r * F) * es, "B1", false},
      {A2, (size_t)(F * r) * es, "A2", false},
      {B2, (size_t)(r * D) * es, "B2", false},
      {residual, residual ? (size_t)(T * D) * es : 0, "residual", false},
      {sumsq_in, sumsq_in ? (size_t)T * 4 : 0, "sumsq_in", false},
      {Y, (size_t)(T * D) * es, "Y", true},
      {H1, (size_t)(T * 2 * r) * 4, "H1", true},
      {H2, (size_t)(T * r) * 4, "H2", true},
      {sumsq, (!sumsq_in || sumsq) ? (size_t)T * 4 : 0, "sumsq", true},
      {sumsq_next, sumsq_next ? (size_t)T * 4 : 0, "sumsq_next", true},
      {ws, (ws && p.fwd_bytes <= ws_bytes) ? p.fwd_bytes : 0, "ws", true, true},
  };
  RBO_TRY(check_ranges(rs));
  RBO_TRY(check_ws_parts(p.fwd_largest, "forward"));
  RBO_TRY(check_ws(ws, ws_bytes, p.fwd_bytes));
  hipStream_t s = as_stream(stream);
  void* A1T = at(ws, p.f_A1T);
  void* B2T = at(ws, p.f_B2T);
  void* S1 = at(ws, p.f_S1);
  void* M = at(ws, p.f_M);
  void* S2 = at(ws, p.f_S2);
  const float inv = 1.f / (float)D;
  // K-contiguous copies of the first down weights (with the gain folded
  // in) and of the last up weights. B1 and A2 are read as they are stored,
  // N-contiguous: for those two products the M/N-major operand path costs
  // less than the transposes it avoids (measured at the 7B MLP shape: each
  // within 2% of its K-contiguous time, against about 50 us of transposes
  // saved), while the first down and last up products run 24% and 26%
  // slower M/N-major, more than their transposes cost.
  RBO_TRY(launch_transposes(dt, {{A1_cat, g, A1T, D, 2 * r, 1}, {B2, nullptr, B2T, r, D, 1}}, s));
  {  // H1 = rho * (x @ (g * A1_cat)), S1 = act(H1), sumsq
    GemmOps ops{};
    ops.a[0] = opnd(x, D, T, D, es);
    ops.b[0] = opnd(A1T, D, 2 * r, D, es);
    if (sumsq_in) {
      EpiDown<true, true>::Args ea{H1, S1, sumsq, 2 * r, inv, d->eps, d->act, sumsq_in};
      RBO_TRY((gemm<EpiDown<true, true>, true, true, 1>("mlp_down1", dt, p.down1, T, 2 * r, D, 1, ops, ea, s)));
    } else {
      EpiDown<true>::Args ea{H1, S1, sumsq, 2 * r, inv, d->eps, d->act, nullptr};
      RBO_TRY((gemm<EpiDown<true>, true, true, 1>("mlp_down1", dt, p.down1, T, 2 * r, D, 1, ops, ea, s)));
    }
  }
  {  // M = SiLU(S1_0 @ B1_0) * (S1_1 @ B1_1)
    GemmOps ops{};
    ops.a[0] = opnd(S1, 2 * r, T, r, es);
    ops.a[1] = opnd(static_cast<const char*>(S1) + r * es, 2 * r, T, r, es);
    ops.b[0] = opnd(B1, F, r, F, es);
    ops.b[1] = opnd(static_cast<const char*>(B1) + r * F * es, F, r, F, es);
    EpiSwiglu::Args ea{M, F};
    RBO_TRY((gemm<EpiSwiglu, true, false, 2>("mlp_up1_swiglu", dt, p.dual, T, F, r, 1, ops, ea, s)));
  }
  {  // H2 = M @ A2, S2 = act(H2)
    GemmOps ops{};
    ops.a[0] = opnd(M, F, T, F, es);
    ops.b[0] = opnd(A2, r, F, r, es);
    EpiDown<false>::Args ea{H2, S2, nullptr, r, 0.f, 0.f, d->act, nullptr};
    RBO_TRY((gemm<EpiDown<false>, true, false, 1>("mlp_down2", dt, p.down2, T, r, F, 1, ops, ea, s)));
  }
  {  // Y = S2 @ B2
    GemmOps ops{};
    ops.a[0] = opnd(S2, r, T, r, es);
    ops.b[0] = opnd(B2T, r, D, r, es);
    if (residual || sumsq_next) {
      float* part = sumsq_next ? reinterpret_cast<float*>(at(ws, p.f_part)) : nullptr;
      EpiUpRes::Args ea{Y, D, residual, part};
      RBO_TRY((gemm<EpiUpRes, true, true, 1>("mlp_up2", dt, p.up2, T, D, r, 1, ops, ea, s)));
      if (sumsq_next) RBO_TRY(launch_colsum(part, p.up2.tiles_n, T, T, sumsq_next, s));
    } else {
      EpiStore<false>::Args ea{Y, D, 0, nullptr};
      RBO_TRY((gemm<EpiStore<false>, true, true, 1>("mlp_up2", dt, p.up2, T, D, r, 1, ops, ea, s)));
    }
  }
  return BOOST_OK;
}

int boost_lrmlp_fwd(const boost_lrmlp_desc* d, const void* x, const void* g, const void* A1_cat, const void* B1,
                    const void* A2, const void* B2, void* Y, float* H1, float* H2, float* sumsq, void* ws,
                    size_t ws_bytes, void* stream) {
  return boost_lrmlp_fwd_chained(d, x, g, A1_cat, B1, A2, B2, nullptr, nullptr, Y, H1, H2, sumsq, nullptr, ws,
                                 ws_bytes, stream);
}

int boost_lrmlp_bwd_chained(const boost_lrmlp_desc* d, const void* x, const void* g, const void* A1_cat,
                            const void* B1, const void* A2, const void* B2, const float* H1, const float* H2,
                            const float* sumsq, const void* dY, const void* dx_add, void* dx, float* dg,
                            float* dA1_cat, float* dB1, float* dA2, float* dB2, void* ws, size_t ws_bytes,
                            void* stream) {
  g_detail.clear();
  RBO_TRY(lrmlp_check_desc(d));
  const int dt = d->dtype;
  const size_t es = esize(dt);
  const int64_t T = d->T, D = d->d, r = d->r, F = d->ffn;
  const LrmlpPlan p = lrmlp_plan(d);
  std::vector<Range> rs = {
      {x, (size_t)(T * D) * es, "x", false},
      {g, (size_t)D * es, "g", false},
      {A1_cat, (size_t)(D * 2 * r) * es, "A1_cat", false},
      {B1, (size_t)(2 * r * F) * es, "B1", false},
      {A2, (size_t)(F * r) * es, "A2", false},
      {B2, (size_t)(r * D) * es, "B2", false},
      {H1, (size_t)(T * 2 * r) * 4, "H1", false},
      {H2, (size_t)(T * r) * 4, "H2", false},
      {sumsq, (size_t)T * 4, "sumsq", false},
      {dY, (size_t)(T * D) * es, "dY", false},
      {dx_add, dx_add ? (size_t)(T * D) * es : 0, "dx_add", false},
      {dx, (size_t)(T * D) * es, "dx", true},
      {dg, (size_t)D * 4, "dg", true},
      {dA1_cat, (size_t)(D * 2 * r) * 4, "dA1_cat", true},
      {dB1, (size_t)(2 * r * F) * 4, "dB1", true},
      {dA2, (size_t)(F * r) * 4, "dA2", true},
      {dB2, (size_t)(r * D) * 4, "dB2", true},
      {ws, (ws && p.bwd_bytes <= ws_bytes) ? p.bwd_bytes : 0, "ws", true, true},
  };
  RBO_TRY(check_ranges(rs));
  RBO_TRY(check_ws_parts(p.bwd_largest, "backward"));
  RBO_TRY(check_ws(ws, ws_bytes, p.bwd_bytes));
  hipStream_t s = as_stream(stream);
  void* S2 = at(ws, p.b_S2);
  void* dU2 = at(ws, p.b_dU2);
  void* S1 = at(ws, p.b_S1);
  void* Mr = at(ws, p.b_M);
  void* dYgu = at(ws, p.b_dY);
  void* dU1 = at(ws, p.b_dU1);
  float* q = reinterpret_cast<float*>(at(ws, p.b_q));
  float* dgp = reinterpret_cast<float*>(at(ws, p.b_dg));
  float* part = p.b_part ? reinterpret_cast<float*>(at(ws, p.b_part)) : nullptr;
  Side* sd = nullptr;
  RBO_TRY(side_for_device(&sd));
  SideFork side(sd, s);
  {  // dS2 = dY @ B2^T; dU2 = dS2 * act'(H2); S2 = act(H2)
    GemmOps ops{};
    ops.a[0] = opnd(dY, D, T, D, es);
    ops.b[0] = opnd(B2, D, r, D, es);
    EpiDS<false>::Args ea{H2, r, r, dU2, S2, nullptr, T, nullptr, 0.f, 0.f, d->act};
    RBO_TRY((gemm<EpiDS<false>, true, true, 1>("mlp_ds2", dt, p.ds2, T, r, D, 1, ops, ea, s)));
  }
  // Weight gradients on the side stream, each after what it reads is ready.
  RBO_TRY(side.fork());
  {  // dB2 = S2^T @ dY
    GemmOps ops{};
    ops.a[0] = opnd(S2, r, T, r, es);
    ops.b[0] = opnd(dY, D, T, D, es);
    RBO_TRY(wgrad<TAG_MLP_DB2>("mlp_dB2", dt, p.dB2, r, D, T, 1, ops, nullptr, dB2, part, side.side()));
  }
  // S1 = act(H1) recomputed from the saved bottleneck.
  RBO_TRY(launch_act_quant(dt, H1, S1, T * 2 * r, d->act, s));
  // The three products of the recompute share one operand layout, K
  // contiguous: A2 already is, B1 gets a transposed copy (measured: with
  // all three M/N-major instead, B1 read as stored and A2 copied, the
  // recompute at the 7B MLP shape ran 15% slower, 100 us, against 17 us
  // of transpose saved).
  void* B1T = at(ws, p.b_B1T);
  RBO_TRY(launch_transposes(dt, {{B1, nullptr, B1T, r, F, 2}}, s));
  {  // recompute Yg, Yu and dM = dU2 @ A2^T in the same tile; M, dYg, dYu
    GemmOps ops{};
    ops.a[0] = opnd(S1, 2 * r, T, r, es);
    ops.a[1] = opnd(static_cast<const char*>(S1) + r * es, 2 * r, T, r, es);
    ops.a[2] = opnd(dU2, r, T, r, es);
    ops.b[0] = opnd(B1T, r, F, r, es);
    ops.b[1] = opnd(static_cast<const char*>(B1T) + F * r * es, r, F, r, es);
    ops.b[2] = opnd(A2, r, F, r, es);
    EpiSwigluBwd::Args ea{Mr, dYgu, F, T * F};
    RBO_TRY((gemm<EpiSwigluBwd, true, true, 3>("mlp_recompute_swiglu_bwd", dt, p.rec, T, F, r, 1, ops, ea, s)));
  }
  RBO_TRY(side.fork());
  {  // dA2 = M^T @ dU2
    GemmOps ops{};
    ops.a[0] = opnd(Mr, F, T, F, es);
    ops.b[0] = opnd(dU2, r, T, r, es);
    RBO_TRY(wgrad<TAG_MLP_DA2>("mlp_dA2", dt, p.dA2, F, r, T, 1, ops, nullptr, dA2, part, side.side()));
  }
  // Block 1 backward with dY = (dYg, dYu); S1 already recomputed. It joins
  // the side stream back into the caller's before returning.
  return lrblock_bwd_core(dt, d->act, 1, T, D, r, 2, F, d->eps, D, x, g, A1_cat, B1, H1, sumsq, dYgu, dx, dg,
                          dA1_cat, dB1, S1, true, dU1, q, dgp, part, p.ds1, p.dB1, p.dA1, p.dx1, s, kMlp1Labels,
                          &side, dx_add);
}

int boost_lrmlp_bwd(const boost_lrmlp_desc* d, const void* x, const void* g, const void* A1_cat, const void* B1,
                    const void* A2, const void* B2, const float* H1, const float* H2, const float* sumsq,
                    const void* dY, void* dx, float* dg, float* dA1_cat, float* dB1, float* dA2, float* dB2,
                    void* ws, size_t ws_bytes, void* stream) {
  return boost_lrmlp_bwd_chained(d, x, g, A1_cat, B1, A2, B2, H1, H2, sumsq, dY, nullptr, dx, dg, dA1_cat, dB1,
                                 dA2, dB2, ws, ws_bytes, stream);
}

// --------------------------- tensor-parallel share -------------------------
int boost_btp_share_workspace_size(const boost_btp_share_desc* d, int is_bwd, size_t* bytes) {
  g_detail.clear();
  RBO_TRY(btp_check_desc(d));
  if (!bytes) return fail(BOOST_ERR_INVALID_VALUE, "bytes is NULL");
  const BtpPlan p = btp_plan(d);
  RBO_TRY(check_ws_parts(is_bwd ? p.bwd_largest : p.fwd_largest, is_bwd ? "backward" : "forward"));
  *bytes = is_bwd ? p.bwd_bytes : p.fwd_bytes;
  return BOOST_OK;
}

int boost_btp_share_fwd(const boost_btp_share_desc* d, const void* z, const void* B_s, const void* g_s,
                        const void* A_s, void* pout, float* s_out, void* ws, size_t ws_bytes, void* stream) {
  g_detail.clear();
  RBO_TRY(btp_check_desc(d));
  const int dt = d->dtype;
  const size_t es = esize(dt);
  const int64_t T = d->T, r = d->r, S = d->d_shard;
  const BtpPlan p = btp_plan(d);
  std::vector<Range> rs = {
      {z, (size_t)(T * r) * es, "z", false},
      {B_s, (size_t)(r * S) * es, "B_s", false},
      {g_s, (size_t)S * es, "g_s", false},
      {A_s, (size_t)(S * r) * es, "A_s", false},
      {pout, (size_t)(T * r) * es, "p", true},
      {s_out, (size_t)T * 4, "s", true},
      {ws, (ws && p.fwd_bytes <= ws_bytes) ? p.fwd_bytes : 0, "ws", true, true},
  };
  RBO_TRY(check_ranges(rs));
  RBO_TRY(check_ws_parts(p.fwd_largest, "forward"));
  RBO_TRY(check_ws(ws, ws_bytes, p.fwd_bytes));
  hipStream_t st = as_stream(stream);
  void* ag = at(ws, p.f_ag);
  float* sp = reinterpret_cast<float*>(at(ws, p.f_sp));
  // B_s and A_s are read as stored, N-contiguous (measured on the 13B share:
  // the forward 0.077-0.079 -> 0.074-0.075 ms without the two transposes).
  {  // u = z @ B_s; a = SiLU(u); ag = a * g_s; row partials of a^2
    GemmOps ops{};
    ops.a[0] = opnd(z, r, T, r, es);
    ops.b[0] = opnd(B_s, S, r, S, es);
    EpiBtpU::Args ea{g_s, ag, sp, T, S};
    RBO_TRY((gemm<EpiBtpU, true, false, 1>("btp_u", dt, p.u, T, S, r, 1, ops, ea, st)));
  }
  {  // p = ag @ A_s; s = sum of the partials
    GemmOps ops{};
    ops.a[0] = opnd(ag, S, T, S, es);
    ops.b[0] = opnd(A_s, r, S, r, es);
    EpiBtpP::Args ea{pout, r, sp, p.u.tiles_n, T, s_out};
    RBO_TRY((gemm<EpiBtpP, true, false, 1>("btp_p", dt, p.p, T, r, S, 1, ops, ea, st)));
  }
  return BOOST_OK;
}

int boost_btp_share_bwd(const boost_btp_share_desc* d, const void* z, const void* B_s, const void* g_s,
                        const void* A_s, const void* dp, const float* ds, void* dz, float* dB_s, float* dg_s,
                        float* dA_s, void* ws, size_t ws_bytes, void* stream) {
  g_detail.clear();
  RBO_TRY(btp_check_desc(d));
  const int dt = d->dtype;
  const size_t es = esize(dt);
  const int64_t T = d->T, r = d->r, S = d->d_shard;
  const BtpPlan p = btp_plan(d);
  std::vector<Range> rs = {
      {z, (size_t)(T * r) * es, "z", false},
      {B_s, (size_t)(r * S) * es, "B_s", false},
      {g_s, (size_t)S * es, "g_s", false},
      {A_s, (size_t)(S * r) * es, "A_s", false},
      {dp, (size_t)(T * r) * es, "dp", false},
      {ds, (size_t)T * 4, "ds", false},
      {dz, (size_t)(T * r) * es, "dz", true},
      {dB_s, (size_t)(r * S) * 4, "dB_s", true},
      {dg_s, (size_t)S * 4, "dg_s", true},
      {dA_s, (size_t)(S * r) * 4, "dA_s", true},
      {ws, (ws && p.bwd_bytes <= ws_bytes) ? p.bwd_bytes : 0, "ws", true, true},
  };
  RBO_TRY(check_ranges(rs));
  RBO_TRY(check_ws_parts(p.bwd_largest, "backward"));
  RBO_TRY(check_ws(ws, ws_bytes, p.bwd_bytes));
  hipStream_t st = as_stream(stream);
  void* du = at(ws, p.b_du);
  void* ag = at(ws, p.b_ag);
  float* dgp = reinterpret_cast<float*>(at(ws, p.b_dg));
  float* U = reinterpret_cast<float*>(at(ws, p.b_U));
  float* part = p.b_part ? reinterpret_cast<float*>(at(ws, p.b_part)) : nullptr;
  // u and e = dp @ A_s^T in two launches of one-round tiles (192 x 256: 215
  // tiles each, against 320 two-accumulator tiles of 256 x 128 in 1.25
  // rounds), u handed over in fp32 so the results are those of one tile
  // holding both accumulators; B_s is read as stored.
  {  // u = z @ B_s recomputed, kept in fp32
    GemmOps ops{};
    ops.a[0] = opnd(z, r, T, r, es);
    ops.b[0] = opnd(B_s, S, r, S, es);
    EpiStore<true>::Args ea{U, S, 0, nullptr};
    RBO_TRY((gemm<EpiStore<true>, true, false, 1>("btp_u_re", dt, p.u, T, S, r, 1, ops, ea, st)));
  }
  {  // e = dp @ A_s^T; du, ag, dg partials
    GemmOps ops{};
    ops.a[0] = opnd(dp, r, T, r, es);
    ops.b[0] = opnd(A_s, r, S, r, es);
    EpiBtpEBwd::Args ea{ds, g_s, U, du, ag, dgp, S};
    RBO_TRY((gemm<EpiBtpEBwd, true, true, 1>("btp_u_bwd", dt, p.e, T, S, r, 1, ops, ea, st)));
  }
  RBO_TRY(launch_colsum(dgp, p.e.tiles_m, S, S, dg_s, st));
  // dz, dA_s and dB_s in a row on the caller's stream. Measured on the 13B
  // share (three products of 8192 x 1280 x 1280 that each fill most of the
  // GPU): 0.305-0.310 ms per step this way, against 0.314-0.318 ms with dA_s
  // on the side stream beside dz and dB_s, and 0.318-0.321 ms with both
  // weight gradients on the side stream beside dz.
  {  // dz = du @ B_s^T
    GemmOps ops{};
    ops.a[0] = opnd(du, S, T, S, es);
    ops.b[0] = opnd(B_s, S, r, S, es);
    EpiStore<false>::Args ea{dz, r, 0, nullptr};
    RBO_TRY((gemm<EpiStore<false>, true, true, 1>("btp_dz", dt, p.dz, T, r, S, 1, ops, ea, st)));
  }
  {  // dA_s = ag^T @ dp
    GemmOps ops{};
    ops.a[0] = opnd(ag, S, T, S, es);
    ops.b[0] = opnd(dp, r, T, r, es);
    RBO_TRY(wgrad<TAG_BTP_DA>("btp_dA", dt, p.dA, S, r, T, 1, ops, nullptr, dA_s, part, st));
  }
  {  // dB_s = z^T @ du
    GemmOps ops{};
    ops.a[0] = opnd(z, r, T, r, es);
    ops.b[0] = opnd(du, S, T, S, es);
    RBO_TRY(wgrad<TAG_BTP_DB>("btp_dB", dt, p.dB, r, S, T, 1, ops, nullptr, dB_s, part, st));
  }
  return BOOST_OK;
}

// ------------------------------- profiler ---------------------------------
// ---------------------------- attention stand-in ---------------------------
static int standin_check(int dtype, int64_t T, int64_t d) {
  RBO_TRY(check_dtype(dtype));
  RBO_TRY(check_T(T));
  RBO_TRY(check_dim64(d, "d"));
  return BOOST_OK;
}

int boost_attn_standin_fwd(int dtype, int64_t T, int64_t d, const void* qkv, void* a, void* stream) {
  g_detail.clear();
  RBO_TRY(standin_check(dtype, T, d));
  const size_t n = (size_t)(T * d), es = esize(dtype);
  std::vector<Range> rs = {{qkv, 3 * n * es, "qkv", false}, {a, n * es, "a", true}};
  RBO_TRY(check_ranges(rs));
  hipStream_t s = as_stream(stream);
  const int grid = grid_for((int64_t)n, 8);
  prof_begin("attn_standin", s);
  if (dtype == BOOST_DT_BF16)
    hipLaunchKernelGGL(standin_fwd_kernel<bf16>, dim3(grid), dim3(256), 0, s, static_cast<const bf16*>(qkv),
                       static_cast<bf16*>(a), (int64_t)n);
  else
    hipLaunchKernelGGL(standin_fwd_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(qkv),
                       static_cast<float*>(a), (int64_t)n);
  prof_end(s);
  return check_launch("attn_standin");
}

int boost_attn_standin_bwd(int dtype, int64_t T, int64_t d, const void* da, void* dqkv, void* stream) {
  g_detail.clear();
  RBO_TRY(standin_check(dtype, T, d));
  const size_t n = (size_t)(T * d), es = esize(dtype);
  std::vector<Range> rs = {{da, n * es, "da", false}, {dqkv, 3 * n * es, "dqkv", true}};
  RBO_TRY(check_ranges(rs));
  hipStream_t s = as_stream(stream);
  const int grid = grid_for((int64_t)n, 16 / (int)es);
  prof_begin("attn_standin_bwd", s);
  if (dtype == BOOST_DT_BF16)
    hipLaunchKernelGGL(standin_bwd_kernel<bf16>, dim3(grid), dim3(256), 0, s, static_cast<const bf16*>(da),
                       static_cast<bf16*>(dqkv), (int64_t)n);
  else
    hipLaunchKernelGGL(standin_bwd_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(da),
                       static_cast<float*>(dqkv), (int64_t)n);
  prof_end(s);
  return check_launch("attn_standin_bwd");
}

int boost_profiler_serialize(int on) {
  g_detail.clear();
  if (on != 0 && on != 1) return fail(BOOST_ERR_INVALID_VALUE, "on = %d must be 0 or 1", on);
  g_serial_side = on != 0;
  return BOOST_OK;
}

int boost_profiler_enable(const char* name_filter, int max_records) {
  g_detail.clear();
  boost_profiler_disable();
  if (max_records <= 0 || max_records > (1 << 20))
    return fail(BOOST_ERR_INVALID_VALUE, "max_records = %d out of range", max_records);
  g_prof.filter = name_filter ? name_filter : "";
  g_prof.recs.reserve((size_t)max_records);
  for (int i = 0; i < max_records; ++i) {
    ProfRec r{"", nullptr, nullptr};
    // Timing-only events: without the system-scope fence a record does not
    // write back and invalidate the caches, so the events barely perturb the
    // stream they time.
    if (hipEventCreateWithFlags(&r.start, hipEventDisableSystemFence) != hipSuccess) {
      boost_profiler_disable();
      return fail(BOOST_ERR_LAUNCH, "hipEventCreate failed");
    }
    if (hipEventCreateWithFlags(&r.stop, hipEventDisableSystemFence) != hipSuccess) {
      hipEventDestroy(r.start);
      boost_profiler_disable();
      return fail(BOOST_ERR_LAUNCH, "hipEventCreate failed");
    }
    g_prof.recs.push_back(r);
  }
  g_prof.used = 0;
  g_prof.on = true;
  return BOOST_OK;
}

int boost_profiler_report(char* buf, size_t len) {
  g_detail.clear();
  if (!buf || !len) return fail(BOOST_ERR_INVALID_VALUE, "buf is NULL or empty");
  std::vector<std::pair<std::string, std::pair<int, double>>> agg;
  for (size_t i = 0; i < g_prof.used; ++i) {
    ProfRec& r = g_prof.recs[i];
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return fail(BOOST_ERR_LAUNCH, "event timing failed for %s", r.label);
    bool found = false;
    for (auto& a : agg)
      if (a.first == r.label) {
        a.second.first += 1;
        a.second.second += ms;
        found = true;
      }
    if (!found) agg.push_back({r.label, {1, (double)ms}});
  }
  std::string out;
  for (auto& a : agg) {
    char line[256];
    snprintf(line, sizeof line, "%s %d %.6f\n", a.first.c_str(), a.second.first, a.second.second);
    out += line;
  }
  const size_t n = std::min(out.size(), len - 1);
  memcpy(buf, out.data(), n);
  buf[n] = 0;
  g_prof.used = 0;
  return BOOST_OK;
}

int boost_profiler_disable(void) {
  for (auto& r : g_prof.recs) {
    hipEventDestroy(r.start);
    hipEventDestroy(r.stop);
  }
  g_prof.recs.clear();
  g_prof.used = 0;
  g_prof.on = false;
  return BOOST_OK;
}

}  // extern "C"
