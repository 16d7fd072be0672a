/*
 * boost_lrblock.h -- C ABI of the MI355X (gfx950) low-rank bottleneck block.
 *
 * The block is the one described by the BOOST summary pages ("BOOST:
 * BOttleneck-Optimized Scalable Training Framework for Low-Rank Large
 * Language Models", gist.science, paper 2512.12131, technical summary):
 *
 *   - a dense d x d_out weight replaced by a down factor (d x r) and an up
 *     factor (r x d_out)                                     (sections 1, 2.1);
 *   - CoLA (SiLU between the factors) or SVD (identity between them)
 *                                                                 (section 4);
 *   - Online-RMSNorm: per-row local statistics (the sum of squares), with the
 *     1/rms scale deferred and applied as a row scale of the down product,
 *     equal to plain RMSNorm                                    (section 2.2);
 *   - linear-layer grouping: down projections that share an input run as one
 *     product over concatenated weights; up projections run as one batched
 *     product                                                   (section 2.2);
 *   - low-rank activation checkpointing: the forward keeps only the
 *     bottleneck activations and the rms statistics; the backward
 *     recomputes the rest inside the block                      (section 2.2);
 *   - one tensor-parallel share of a bottleneck pair (BTP): a column slice of
 *     the up projection, SiLU on the sharded activation, a row slice of the
 *     next down projection, emitting partial sums and per-row partial
 *     sums of squares with no cross-share reduction            (section 2.1).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous tensors.
 *     Weights use the math layout [in, out] (the product is x @ A).
 *   - "dtype" tensors hold BOOST_DT_BF16 (bfloat16) or BOOST_DT_F32 values
 *     as selected by desc->dtype: activations, weights, gains and the
 *     activation-shaped outputs (Y, dx, p, dz). The saved bottleneck H, the
 *     statistics and every weight/gain gradient are always fp32.
 *   - Dimensions: T (tokens) >= 1, any value. Every other dimension (d, r,
 *     d_out, ffn, d_shard) must be a positive multiple of 64; G in [1, 16].
 *     Every tensor must be smaller than 2 GiB, and so must every buffer the
 *     library carves from a workspace (the workspace itself may be larger);
 *     a descriptor that would need a larger workspace buffer is refused with
 *     BOOST_ERR_UNSUPPORTED by *_workspace_size and by the call itself.
 *     Pointers must be 16-byte aligned.
 *   - Ownership: the caller owns every buffer. The library allocates no
 *     device memory, frees nothing, keeps no pointer after return and never
 *     synchronises. Work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) in stream order and runs asynchronously. The block and
 *     MLP backward calls fork their weight-gradient products onto a side
 *     stream through an event recorded on `stream`, and make `stream` wait
 *     for them before returning - on every return path, errors included,
 *     once anything was forked - so all results are ordered on `stream`
 *     exactly as if everything ran on it; stream capture of `stream`
 *     captures both. The BTP share backward runs on `stream` alone.
 *   - State: besides the loaded kernels, the library keeps one side stream
 *     and four events per host thread and device, created on first use
 *     with the default priority and kept until the process ends (no device
 *     memory). Two block or MLP backward calls made from one host thread
 *     on different streams share that thread's side stream, so their
 *     weight-gradient products run one after the other (results are
 *     unaffected; only the overlap between the two calls is lost).
 *   - Outputs are overwritten, never accumulated into. Inputs must not
 *     overlap outputs or the workspace.
 *   - Workspace: `ws` is device scratch of at least the size returned by the
 *     matching *_workspace_size call; its contents on entry are ignored and
 *     on return are unspecified. Concurrent calls on different streams need
 *     different workspaces.
 *   - Errors: arguments are validated before anything is launched, in the
 *     order ABI version, enums, dimensions, pointers, alignment, overlap,
 *     workspace size. On error nothing is launched, outputs are untouched,
 *     and a BOOST_ERR_* status is returned; boost_last_error_detail() then
 *     names the failing argument (thread-local). A failed launch returns
 *     BOOST_ERR_LAUNCH. Device faults surface at the caller's next
 *     synchronisation. No C++ exception crosses this interface.
 *   - Results are run-to-run bit-identical: every reduction has a fixed
 *     order and no floating-point atomics are used.
 */
#ifndef BOOST_LRBLOCK_H
#define BOOST_LRBLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BOOST_ABI_VERSION 1

enum {
  BOOST_OK = 0,
  BOOST_ERR_INVALID_VALUE = 1, /* null pointer, bad dimension or enum */
  BOOST_ERR_UNSUPPORTED = 2,   /* valid but outside what the kernels cover */
  BOOST_ERR_MISALIGNED = 3,    /* pointer not 16-byte aligned */
  BOOST_ERR_ALIASING = 4,      /* an output overlaps an input or another output */
  BOOST_ERR_WORKSPACE = 5,     /* ws too small (or NULL with nonzero need) */
  BOOST_ERR_VERSION = 6,       /* desc->abi_version != BOOST_ABI_VERSION */
  BOOST_ERR_LAUNCH = 7         /* a kernel launch failed */
};

enum { BOOST_DT_F32 = 0, BOOST_DT_BF16 = 1 };
/* Bottleneck activation between the factors: identity (SVD-style) or SiLU
 * (CoLA), BOOST summary pages, section 4. */
enum { BOOST_ACT_IDENTITY = 0, BOOST_ACT_SILU = 1 };

/* ------------------------------------------------------------------------
 * Grouped low-rank block: QKV-style (G groups sharing one normalised input)
 * or an O-projection (G = 1, norm = 0).
 *
 * Forward (norm = 1):  sumsq_t = sum_i x_ti^2
 *                      rho_t   = (sumsq_t / d_norm + eps)^(-1/2)
 *                      H       = rho * ((x * g) @ A_cat)          [T, G*r] fp32
 *                      Y_j     = act(H_j) @ B_j   j = 0..G-1      [G, T, d_out]
 * with H_j the columns j*r..(j+1)*r-1 of H. This equals plain RMSNorm
 * followed by the G separate down products (Online-RMSNorm and grouping,
 * section 2.2). With norm = 0, H = x @ A_cat and g/sumsq are unused.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t abi_version; /* BOOST_ABI_VERSION */
  int32_t dtype;       /* BOOST_DT_* */
  int32_t act;         /* BOOST_ACT_* */
  int32_t norm;        /* 1: Online-RMSNorm of x with gain g; 0: none */
  int64_t T, d, r, G, d_out;
  int64_t d_norm;      /* mean-square divisor, >= d (the global width) */
  float eps;           /* >= 0, added to the mean square inside the root */
} boost_lrblock_desc;

/* Bytes of workspace for the forward (is_bwd = 0) or backward (1). */
int boost_lrblock_workspace_size(const boost_lrblock_desc* desc, int is_bwd, size_t* bytes);

/* Forward. Inputs: x[T,d], g[d] (may be NULL iff norm = 0), A_cat[d,G*r],
 * B[G,r,d_out] (dtype). Outputs: Y[G,T,d_out] (dtype), H[T,G*r] fp32 (the
 * saved bottleneck), sumsq[T] fp32 (may be NULL iff norm = 0). */
int boost_lrblock_fwd(const boost_lrblock_desc* desc, const void* x, const void* g,
                      const void* A_cat, const void* B, void* Y, float* H, float* sumsq,
                      void* ws, size_t ws_bytes, void* stream);

/* The forward above with no workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation). Its scratch (the transposed down
 * weights and act(H)) lives in a fixed 64 MiB array that the library holds
 * on each device it runs on until the process ends; it calls no allocator. A
 * descriptor whose forward workspace (boost_lrblock_workspace_size with
 * is_bwd = 0) exceeds 64 MiB is refused with BOOST_ERR_UNSUPPORTED (the
 * 1B-shaped QKV forward, T = 16384, d = 2048, r = 512, G = 3, needs 54 MiB).
 * Every call on a device shares that device's array: calls that may overlap
 * on one device (different streams, different host threads) race and give
 * undefined results; serialise them. Nothing in the scratch needs to start
 * at zero. Results are bit-identical to boost_lrblock_fwd. */
int boost_lrblock_fwd_noalloc(const boost_lrblock_desc* desc, const void* x, const void* g,
                              const void* A_cat, const void* B, void* Y, float* H, float* sumsq,
                              void* stream);

/* Backward with low-rank activation checkpointing (section 2.2): from the
 * inputs, the saved H and sumsq, and dY[G,T,d_out] (dtype) only; act(H),
 * act'(H) and rho are recomputed. Outputs: dx[T,d] (dtype), dg[d] fp32 (NULL
 * iff norm = 0), dA_cat[d,G*r] fp32, dB[G,r,d_out] fp32. */
int boost_lrblock_bwd(const boost_lrblock_desc* desc, const void* x, const void* g,
                      const void* A_cat, const void* B, const float* H, const float* sumsq,
                      const void* dY, void* dx, float* dg, float* dA_cat, float* dB,
                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Low-rank SwiGLU MLP: two grouped blocks around a SwiGLU.
 *   H1 = rho * ((x * g) @ A1_cat)        [T,2r] fp32, saved
 *   Yg = act(H1_0) @ B1_0, Yu = act(H1_1) @ B1_1        [T,ffn]
 *   M  = SiLU(Yg) * Yu                                   [T,ffn]
 *   H2 = M @ A2                          [T,r] fp32, saved
 *   Y  = act(H2) @ B2                                    [T,d]
 * SwiGLU always uses SiLU; act is the bottleneck activation. The divisor of
 * the mean square is d.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t abi_version;
  int32_t dtype;
  int32_t act;
  int32_t reserved; /* must be 0 */
  int64_t T, d, r, ffn;
  float eps;
} boost_lrmlp_desc;

int boost_lrmlp_workspace_size(const boost_lrmlp_desc* desc, int is_bwd, size_t* bytes);

/* Forward. Inputs (dtype): x[T,d], g[d], A1_cat[d,2r], B1[2,r,ffn],
 * A2[ffn,r], B2[r,d]. Outputs: Y[T,d] (dtype), H1[T,2r], H2[T,r],
 * sumsq[T] (fp32). */
int boost_lrmlp_fwd(const boost_lrmlp_desc* desc, const void* x, const void* g,
                    const void* A1_cat, const void* B1, const void* A2, const void* B2,
                    void* Y, float* H1, float* H2, float* sumsq,
                    void* ws, size_t ws_bytes, void* stream);

/* Backward from the inputs, the saved H1, H2, sumsq and dY[T,d] (dtype).
 * The SwiGLU operands Yg, Yu and M are recomputed inside the block.
 * Outputs: dx[T,d] (dtype); dg[d], dA1_cat[d,2r], dB1[2,r,ffn], dA2[ffn,r],
 * dB2[r,d] (fp32). */
int boost_lrmlp_bwd(const boost_lrmlp_desc* desc, const void* x, const void* g,
                    const void* A1_cat, const void* B1, const void* A2, const void* B2,
                    const float* H1, const float* H2, const float* sumsq, const void* dY,
                    void* dx, float* dg, float* dA1_cat, float* dB1, float* dA2, float* dB2,
                    void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Chaining blocks into a decoder layer (Online-RMSNorm, section 2.2: the
 * statistic of a block's input is produced where that input is produced).
 * The *_chained entry points extend the calls above; passing NULL for every
 * extra argument gives exactly the plain call.
 *   residual[T,d_out] (dtype, G = 1 only): the up product writes
 *       Y = residual + S @ B (one rounding), e.g. h2 = x + O(a).
 *   sumsq_next[T] (fp32 out, G = 1 only): the row sums of squares of the
 *       stored Y (the dtype values, squared and summed in fp32) - the next
 *       block's Online-RMSNorm statistic, formed from per-tile-column
 *       partials in a fixed order.
 *   sumsq_in[T] (fp32, norm = 1 only): the statistic of x from its producer;
 *       the down product then takes its 1/rms row scale from it instead of
 *       summing the squares of x itself. `sumsq` may then be NULL; when not
 *       NULL it receives a copy.
 *   dx_add[T,d] (dtype, backward, norm = 1 only): added to dx in the
 *       input-gradient epilogue (the residual path of the layer's gradient).
 * The forward workspace sizes above already cover the chained forms.
 * ------------------------------------------------------------------------ */
int boost_lrblock_fwd_chained(const boost_lrblock_desc* desc, const void* x, const void* g,
                              const void* A_cat, const void* B, const void* residual,
                              const float* sumsq_in, void* Y, float* H, float* sumsq,
                              float* sumsq_next, void* ws, size_t ws_bytes, void* stream);

int boost_lrblock_bwd_chained(const boost_lrblock_desc* desc, const void* x, const void* g,
                              const void* A_cat, const void* B, const float* H,
                              const float* sumsq, const void* dY, const void* dx_add, void* dx,
                              float* dg, float* dA_cat, float* dB, void* ws, size_t ws_bytes,
                              void* stream);

int boost_lrmlp_fwd_chained(const boost_lrmlp_desc* desc, const void* x, const void* g,
                            const void* A1_cat, const void* B1, const void* A2, const void* B2,
                            const void* residual, const float* sumsq_in, void* Y, float* H1,
                            float* H2, float* sumsq, float* sumsq_next, void* ws,
                            size_t ws_bytes, void* stream);

int boost_lrmlp_bwd_chained(const boost_lrmlp_desc* desc, const void* x, const void* g,
                            const void* A1_cat, const void* B1, const void* A2, const void* B2,
                            const float* H1, const float* H2, const float* sumsq, const void* dY,
                            const void* dx_add, void* dx, float* dg, float* dA1_cat, float* dB1,
                            float* dA2, float* dB2, void* ws, size_t ws_bytes, void* stream);

/* Attention stand-in between a layer's QKV and O blocks (the attention core
 * is not part of the bottleneck block): a[T,d] = q + k + v for qkv[3,T,d]
 * (dtype; summed exactly in fp64, then rounded to fp32 and, for bf16, from
 * there to bf16), and its backward dqkv[3,T,d] = (da, da, da). d must be a
 * multiple of 64. */
int boost_attn_standin_fwd(int dtype, int64_t T, int64_t d, const void* qkv, void* a, void* stream);
int boost_attn_standin_bwd(int dtype, int64_t T, int64_t d, const void* da, void* dqkv, void* stream);

/* ------------------------------------------------------------------------
 * One tensor-parallel share of a bottleneck pair (BTP, section 2.1):
 *   u = z @ B_s            (column slice of the up projection)  [T,d_shard]
 *   a = SiLU(u)            (op on the sharded activation)
 *   s = rowsum(a^2)        (local Online-RMSNorm statistic)     [T] fp32
 *   p = (a * g_s) @ A_s    (row slice of the next down projection) [T,r]
 * No cross-share sum and no 1/rms scale are applied here: the caller's one
 * exchange sums p and s over the shares.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t abi_version;
  int32_t dtype;
  int64_t T, r, d_shard;
} boost_btp_share_desc;

int boost_btp_share_workspace_size(const boost_btp_share_desc* desc, int is_bwd, size_t* bytes);

/* Forward. Inputs (dtype): z[T,r], B_s[r,d_shard], g_s[d_shard],
 * A_s[d_shard,r]. Outputs: p[T,r] (dtype), s[T] fp32. */
int boost_btp_share_fwd(const boost_btp_share_desc* desc, const void* z, const void* B_s,
                        const void* g_s, const void* A_s, void* p, float* s,
                        void* ws, size_t ws_bytes, void* stream);

/* Backward given the gradients of the share's own outputs, dp[T,r] (dtype)
 * and ds[T] (fp32); u and a are recomputed from z. Outputs: dz[T,r] (dtype,
 * this share's partial), dB_s[r,d_shard], dg_s[d_shard], dA_s[d_shard,r]
 * (fp32). */
int boost_btp_share_bwd(const boost_btp_share_desc* desc, const void* z, const void* B_s,
                        const void* g_s, const void* A_s, const void* dp, const float* ds,
                        void* dz, float* dB_s, float* dg_s, float* dA_s,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Status and version.
 * ------------------------------------------------------------------------ */
const char* boost_status_string(int status);  /* static string; never NULL */
const char* boost_last_error_detail(void);    /* thread-local; "" if none */
int boost_abi_version(void);                  /* BOOST_ABI_VERSION */

/* ------------------------------------------------------------------------
 * Kernel timing (measurement support, off by default). While enabled, every
 * launch whose kernel label contains `name_filter` (all launches if NULL or
 * "") is timed by a pair of hipEvents on the launch stream: a GEMM launch
 * passes them to hipExtLaunchKernelGGL, which records them at the kernel's
 * start and end (the timed span still includes the dispatch, a few
 * microseconds); the element-wise passes record them around their launches.
 * The events are timing-only (no system-scope fence). They are created
 * here, up to max_records pairs; launches beyond that are not timed. boost_profiler_report synchronises on the recorded events and
 * writes one line per label, "label count total_ms", into buf (NUL
 * terminated, truncated to len). disable destroys the events. Not
 * thread-safe: enable, run, report and disable from one host thread.
 * ------------------------------------------------------------------------ */
int boost_profiler_enable(const char* name_filter, int max_records);
int boost_profiler_report(char* buf, size_t len);
int boost_profiler_disable(void);

/* Measurement switch, off by default (on = 1 sets it, 0 clears it; any
 * other value is BOOST_ERR_INVALID_VALUE). While set, backward passes
 * enqueue their weight-gradient products on the caller's stream instead of
 * the side stream, so every launch runs with no other kernel of the call
 * beside it and a timed launch measures that product alone. Results are
 * bit-identical either way (the same kernels compute the same sums); only
 * the overlap, and so the wall time of a backward, changes. Read when a
 * backward call starts; process-global and not thread-safe, like the timer. */
int boost_profiler_serialize(int on);

#ifdef __cplusplus
}
#endif

#endif /* BOOST_LRBLOCK_H */
