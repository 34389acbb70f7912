/*
 * distri_patch.h - C ABI of the MI355X (gfx950) library for one device's
 * share of a DistriFusion patch layer under displaced patch parallelism.
 *
 * The method (DistriFusion, "Distributed Parallel Inference for
 * High-Resolution Diffusion Models") splits the latent image into row
 * patches, one per device.  After the first synchronous steps each device
 * computes its own patch with fresh activations and takes the context of the
 * other patches from the previous denoising step, exchanged asynchronously
 * ("DistriFusion：高分辨率扩散模型的分布式并行推理", dongaigc.com mirror of the
 * project README, section 概述, figure (c); meens.ai catalog page, section 2).
 * The layers it wraps are Conv2d, self-attention and GroupNorm
 * ("DistriFusion源码探秘：从DistriUNetPP到DistriAttentionTP的模块设计原理",
 * section "Patch Parallelism的实现原理", items 1-3).  This library holds the
 * per-device arithmetic of those layers; on one GPU the other patches' stale
 * activations are ordinary device memory.
 *
 * Geometry.  A full map has B images of H rows x W columns.  It is split into
 * n row bands of h = H / n rows; patch i owns rows [i*h, (i+1)*h) and, as a
 * token sequence (token = row * W + col), tokens [i*Lq, (i+1)*Lq) with
 * Lq = h*W.  L = H*W is the full token count.
 *
 * Conventions shared by every entry point.
 *  - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *    row-major with the layouts given per call.  The library allocates
 *    nothing and keeps no state between calls.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    default stream).  Calls return without synchronising; results are ready
 *    when the stream reaches that point.  Calls are thread-safe.
 *  - Outputs must not overlap inputs (DISTRI_ERR_ALIAS).
 *  - Every argument is validated on the host before any HIP call; a bad
 *    argument returns its status code with nothing enqueued.  A call whose
 *    output has no elements returns DISTRI_OK without touching the GPU (its
 *    pointers may then be NULL).  A failed launch returns DISTRI_ERR_HIP.
 *  - Tensor pointers must be 16-byte aligned (DISTRI_ERR_ALIGN), except for
 *    distri_refresh_stale, which needs only element alignment.
 *  - bf16 values are IEEE-754 binary32 truncated to the top 16 bits; every
 *    kernel rounds its fp32 results to bf16 with round-to-nearest-even.
 *  - distri_last_error() returns a thread-local text naming the argument
 *    that the last failing call on this thread rejected.
 */
#ifndef DISTRI_PATCH_H
#define DISTRI_PATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DISTRI_PATCH_ABI_VERSION 1

typedef enum { DISTRI_F32 = 0, DISTRI_BF16 = 1 } distri_dtype;

typedef enum {
    DISTRI_OK = 0,
    DISTRI_ERR_NULL = 1,        /* a required pointer is NULL */
    DISTRI_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
    DISTRI_ERR_DTYPE = 3,       /* dtype not one of distri_dtype */
    DISTRI_ERR_ALIGN = 4,       /* pointer not aligned as required */
    DISTRI_ERR_UNSUPPORTED = 5, /* valid, but outside what the kernels handle */
    DISTRI_ERR_WORKSPACE = 6,   /* workspace missing or too small */
    DISTRI_ERR_HIP = 7,         /* the HIP runtime reported an error */
    DISTRI_ERR_ALIAS = 8        /* an output overlaps an input */
} distri_status;

/* (B, H, W, n, i): batch, full-map rows, columns, patch count, this patch. */
typedef struct {
    int64_t batch, height, width, n_patches, patch;
} distri_patch_geom;

int distri_abi_version(void);
const char *distri_status_str(int status);
const char *distri_last_error(void);

/*
 * distri_patch_self_attn - self-attention of patch i over the fresh + stale
 * token map (DistriSelfAttentionPP in the source walkthrough, section
 * "Patch Parallelism的实现原理", item 2; stale context per the README
 * mirror, section 概述, figure (c)).
 *
 * For every image b, head hd and local query row r:
 *   out[b, r, hd, :] = sum_t softmax_t(scale * <q[b, r, hd, :], K^[b, t, hd, :]>) V^[b, t, hd, :]
 * over all L tokens t, where K^/V^ row t is k_fresh/v_fresh[b, t - i*Lq] for
 * t in [i*Lq, (i+1)*Lq) and k_stale/v_stale[b, t] otherwise.  No mask.  The
 * stale maps' rows of patch i are never read.
 *
 *   q, k_fresh, v_fresh, out   [B, Lq, heads, head_dim]   dtype
 *   k_stale, v_stale           [B, L,  heads, head_dim]   dtype
 *   scale                      finite and > 0 (1/sqrt(head_dim) for SDXL)
 *   workspace                  >= distri_patch_self_attn_workspace_size()
 *                              bytes of device memory (may be NULL if that
 *                              size is 0); contents on entry are ignored.
 * head_dim must be 64 and H*W*heads*head_dim below 2^31
 * (DISTRI_ERR_UNSUPPORTED otherwise).  The bf16 path may split the keys of
 * some query tiles into chunks; the workspace then holds their partial
 * results.  Its size is a function of (g, heads, head_dim, dtype) alone: the
 * split is planned for a 256-compute-unit MI355X, and the same plan runs
 * unchanged (in more rounds) on a device with fewer.  The workspace must not
 * overlap any input or out (DISTRI_ERR_ALIAS).
 * Arithmetic: fp32 inputs are computed in fp32 throughout.  bf16 inputs: the
 * scores Q K^T on bf16 MFMA with fp32 accumulation, the softmax in fp32, and
 * the weighted sum of V on f16 MFMA with fp32 accumulation (the weights
 * rounded to f16, which keeps their error well inside the output's bf16
 * rounding).  V is therefore taken as f16: every V element must be finite
 * with magnitude below 65504 (a larger one becomes inf); elements below
 * 2^-14 in magnitude are carried with absolute error under 2^-25.
 */
int distri_patch_self_attn_workspace_size(const distri_patch_geom *g, int64_t heads,
                                          int64_t head_dim, int dtype, size_t *bytes);
int distri_patch_self_attn(const distri_patch_geom *g, int64_t heads, int64_t head_dim,
                           float scale, int dtype, const void *q, const void *k_fresh,
                           const void *v_fresh, const void *k_stale, const void *v_stale,
                           void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * distri_patch_cross_attn - cross-attention of patch i's queries over a
 * context shared by every patch (the text encoder's tokens, already
 * projected; the wrapped cross-attention of the source walkthrough, section
 * "Patch Parallelism的实现原理", item 2).  Nothing in it is stale: the
 * context is the same on every device and step, so a patch needs no other
 * patch's data.  For every image b, head and local query r:
 *   out[b, r, head, :] = softmax_t(scale * q[b, r, head, :] . k_ctx[b, t, head, :]) v_ctx
 * over the ctx_len context tokens t.
 *
 *   q, out          [B, Lq, heads, head_dim]   dtype
 *   k_ctx, v_ctx    [B, ctx_len, heads, head_dim] dtype
 *   workspace       >= distri_patch_cross_attn_workspace_size() bytes
 * head_dim must be 64 and ctx_len >= 1.  In bf16 with ctx_len <= 128 the
 * whole context of one (image, head) is held on chip and the workspace size
 * is 0; otherwise the self-attention kernels run with L = ctx_len, under the
 * same limits as distri_patch_self_attn.  Arithmetic and the range of v_ctx
 * are those of distri_patch_self_attn (f16 weighted sum of V in bf16); the
 * workspace must not overlap any input or out.
 */
int distri_patch_cross_attn_workspace_size(const distri_patch_geom *g, int64_t heads,
                                           int64_t head_dim, int64_t ctx_len, int dtype,
                                           size_t *bytes);
int distri_patch_cross_attn(const distri_patch_geom *g, int64_t heads, int64_t head_dim,
                            int64_t ctx_len, float scale, int dtype, const void *q,
                            const void *k_ctx, const void *v_ctx, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * distri_patch_conv3x3_halo - 3x3 convolution (stride 1, zero padding 1) of
 * patch i (DistriConv2dPP, source walkthrough, item 1).  The input rows just
 * above and below the patch (the halo) come from the previous step's stale
 * map: row i*h-1 if i > 0 and row (i+1)*h if i < n-1; outside the image the
 * padding is zero.
 *
 *   y[b, r, c, o] = bias[o] + sum_{kh,kw,ci} w[o, kh, kw, ci] * X^[b, i*h+r+kh-1, c+kw-1, ci]
 *
 *   x_fresh  [B, h, W, Cin]       dtype  (NHWC)
 *   x_stale  [B, H, W, Cin]       dtype  (only the two halo rows are read)
 *   weight   [Cout, 3, 3, Cin]    dtype
 *   bias     [Cout] fp32 or NULL
 *   y        [B, h, W, Cout]      dtype
 * bf16 requires Cin % 64 == 0, and B*H*W*Cin, B*H*W*Cout and Cout*9*Cin below
 * 2^31 (DISTRI_ERR_UNSUPPORTED); any Cout.
 */
int distri_patch_conv3x3_halo(const distri_patch_geom *g, int64_t c_in, int64_t c_out,
                              int dtype, const void *x_fresh, const void *x_stale,
                              const void *weight, const float *bias, void *y, void *stream);

/*
 * distri_async_groupnorm - corrected asynchronous GroupNorm of patch i
 * (DistriGroupNorm, source walkthrough, item 3; default sync mode per the
 * README mirror's --sync_mode flag).  Per image b and group g (C/G
 * consecutive channels):
 *   m1, m2  = E[x], E[x^2] over this patch's h*W*(C/G) fresh values
 *   mu      = (m1 + sum_{j != i} stale_moments[b, j, g, 0]) / n
 *   e2      = (m2 + sum_{j != i} stale_moments[b, j, g, 1]) / n
 *   rstd    = 1 / sqrt(max(e2 - mu^2, 0) + eps)
 *   y       = (x - mu) * rstd * gamma[c] + beta[c]
 *   fresh_moments[b, g, :] = (m1, m2)
 * Slot i of stale_moments is never read.  With the other slots equal to the
 * per-patch moments of the previous step's map this is GroupNorm of the
 * hybrid map.
 *
 *   x_fresh, y      [B, h, W, C]  dtype (NHWC)
 *   stale_moments   [B, n, G, 2]  fp32
 *   gamma, beta     [C] fp32, or NULL for 1 and 0
 *   fresh_moments   [B, G, 2]     fp32 (output)
 *   workspace       >= distri_async_groupnorm_workspace_size() bytes;
 *                   contents on entry are ignored
 * C must be a multiple of 8 for bf16 and of 4 for fp32, and at most 4096
 * (bf16) / 2048 (fp32); G at most 256 (DISTRI_ERR_UNSUPPORTED).  The
 * result is deterministic (fixed summation order, no atomics).
 */
int distri_async_groupnorm_workspace_size(const distri_patch_geom *g, int64_t channels,
                                          int64_t groups, int dtype, size_t *bytes);
int distri_async_groupnorm(const distri_patch_geom *g, int64_t channels, int64_t groups,
                           float eps, int dtype, const void *x_fresh,
                           const float *stale_moments, const float *gamma, const float *beta,
                           void *y, float *fresh_moments, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * distri_async_groupnorm_noalloc - distri_async_groupnorm for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no workspace and calls
 * no allocating routine; the caller still passes every input and output,
 * with the same arguments, layouts, limits and results as
 * distri_async_groupnorm (the same kernels run).
 *
 * Its scratch is a static device array of 2 MiB that the library holds on
 * each device it runs on until the process ends (its address is looked up
 * once per device, at the first call with that device current).  A shape
 * whose scratch need (distri_async_groupnorm_workspace_size()) exceeds 2 MiB
 * returns DISTRI_ERR_UNSUPPORTED with nothing enqueued; the SDXL shapes need
 * at most a few hundred KB.  Every call on one device shares that device's
 * array and leaves its contents behind (nothing in it needs clearing): calls
 * that overlap on one device - on different streams or threads without
 * ordering between them - race, and must be serialised by the caller.
 */
int distri_async_groupnorm_noalloc(const distri_patch_geom *g, int64_t channels, int64_t groups,
                                   float eps, int dtype, const void *x_fresh,
                                   const float *stale_moments, const float *gamma,
                                   const float *beta, void *y, float *fresh_moments, void *stream);

/*
 * distri_async_groupnorm_silu - distri_async_groupnorm followed by SiLU,
 * y = z / (1 + exp(-z)) with z the normalised, affine value (GroupNorm then
 * SiLU opens each SDXL ResNet block, whose GroupNorm the wrapped module of the
 * source walkthrough, item 3, replaces).  Same arguments, layouts, limits and
 * workspace; y is rounded once from fp32.
 */
int distri_async_groupnorm_silu(const distri_patch_geom *g, int64_t channels, int64_t groups,
                                float eps, int dtype, const void *x_fresh,
                                const float *stale_moments, const float *gamma,
                                const float *beta, void *y, float *fresh_moments,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * distri_group_moments - raw group moments of patch i written straight into
 * its slot of a moment table:
 *   table[b, i, g, :] = (E[x], E[x^2]) over the patch's h*W*(C/G) values
 * Other slots are left unchanged.  This fills the table before the first
 * asynchronous step and, in a synchronous step, shares every patch's current
 * moments before any patch normalises (the first denoising steps run
 * synchronously: README mirror, section 概述, figure (c), and the paper
 * page's implementation details).  Same values as the fresh_moments of
 * distri_async_groupnorm (same kernels, same summation order).
 *
 *   x_fresh  [B, h, W, C] dtype     table  [B, n, G, 2] fp32
 *   workspace  >= distri_async_groupnorm_workspace_size() bytes
 * Same channel and group limits as distri_async_groupnorm; a patch with no
 * pixels (W == 0) is DISTRI_ERR_SHAPE.
 */
int distri_group_moments(const distri_patch_geom *g, int64_t channels, int64_t groups, int dtype,
                         const void *x_fresh, float *table, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * distri_refresh_stale - make this step's fresh slice the next step's stale
 * context (the reuse of the previous step's activations, README mirror,
 * section 概述, figure (c)):
 *   stale[b, i*h + r, :] = fresh[b, r, :]   for r in [0, h)
 * Other rows of stale are left unchanged.  Bitwise copy.
 *
 *   fresh  [B, h, row_elems]   stale  [B, H, row_elems]   dtype
 * K/V maps use row_elems = W*heads*head_dim, conv inputs W*C, and the
 * GroupNorm moment table the geometry (B, n, 1, n, i) with row_elems = 2*G
 * and DISTRI_F32.
 */
int distri_refresh_stale(const distri_patch_geom *g, int64_t row_elems, int dtype,
                         const void *fresh, void *stale, void *stream);

/*
 * distri_refresh_stale_maps - the same refresh for all of a layer's stale
 * maps in one launch (the K and V maps of its attention, the input of its
 * conv, its GroupNorm moment table: every activation the next step reuses,
 * README mirror, section 概述, figure (c)).  Map m of count:
 *   stale_m[b, i*rows_m + r, :] = fresh_m[b, r, :]   for r in [0, rows_m)
 * with fresh_m [B, rows_m, row_elems_m] and stale_m [B, n*rows_m,
 * row_elems_m] of dtype_m; B, n and i come from g (H and W only have to
 * form a valid geometry).  rows_m is H/n for feature maps and K/V maps
 * (row_elems W*C, resp. W*heads*head_dim) and 1 for a moment table
 * (row_elems 2*G, DISTRI_F32).  Other rows are left unchanged; bitwise copy.
 *
 *   count   0..DISTRI_REFRESH_MAX_MAPS (DISTRI_ERR_UNSUPPORTED above)
 *   maps    host array of count descriptors (read during the call only)
 * A map with no elements is skipped.  Pointers must be aligned to their
 * element size (DISTRI_ERR_ALIGN); a stale map may not overlap any fresh
 * map or another stale map (DISTRI_ERR_ALIAS).  Maps whose rows are whole
 * 16-byte vectors at 16-byte aligned addresses (all SDXL maps) are copied
 * by one kernel launch; any other map gets a launch of its own on the same
 * stream.  Every check runs before anything is enqueued.
 */
#define DISTRI_REFRESH_MAX_MAPS 8
typedef struct distri_refresh_map {
    int64_t rows;       /* rows of the fresh slice per image */
    int64_t row_elems;  /* elements per row */
    int dtype;          /* DISTRI_BF16 or DISTRI_F32 */
    const void *fresh;  /* device, [B, rows, row_elems] */
    void *stale;        /* device, [B, n * rows, row_elems] */
} distri_refresh_map;
int distri_refresh_stale_maps(const distri_patch_geom *g, int count, const distri_refresh_map *maps,
                              void *stream);

/*
 * distri_patch_qkv_proj - Q/K/V projection of patch i's hidden states (the
 * projections that the wrapped self-attention holds: source walkthrough,
 * section "Patch Parallelism的实现原理", item 2), with the refresh of the
 * stale K/V maps folded in.  For every image b and patch token t:
 *   [q | k | v][b, t, :] = bias + w_qkv * x[b, t, :]      (each [C] of [3C])
 * and, when k_stale / v_stale are given, their rows of patch i take the new
 * values (k_stale[b, i*Lq + t, :] = k[b, t, :], likewise v): this step's
 * fresh K/V become the next step's stale context (README mirror, section
 * 概述, figure (c)) without a separate distri_refresh_stale.  Attention never
 * reads the stale maps' own rows, so they may be written before it runs.
 *
 *   x                   [B, h, W, C] = [B, Lq, C]   dtype (token-major)
 *   w_qkv               [3C, C] dtype: rows 0..C-1 Q, C..2C-1 K, 2C..3C-1 V
 *   bias                [3C] fp32 or NULL
 *   q, k_fresh, v_fresh [B, Lq, C] dtype (outputs; [B, Lq, heads, 64] for
 *                       distri_patch_self_attn when C = heads * 64)
 *   k_stale, v_stale    [B, H*W, C] dtype or NULL (rows of patch i written)
 * bf16 requires C % 64 == 0; C <= 65536 and B*Lq < 2^31
 * (DISTRI_ERR_UNSUPPORTED).  bf16 inputs use bf16 MFMA with fp32
 * accumulation; each output is rounded to bf16 once and the stale copy holds
 * the same bits.
 */
int distri_patch_qkv_proj(const distri_patch_geom *g, int64_t channels, int dtype,
                          const void *x, const void *w_qkv, const float *bias, void *q,
                          void *k_fresh, void *v_fresh, void *k_stale, void *v_stale,
                          void *stream);

/*
 * distri_patch_out_proj - output projection of the patch's attention result
 * (same module as above):
 *   y[b, t, :] = bias + w_o * o[b, t, :]
 *   o, y   [B, Lq, C] dtype      w_o  [C, C] dtype      bias [C] fp32 or NULL
 * Same limits as distri_patch_qkv_proj.
 */
int distri_patch_out_proj(const distri_patch_geom *g, int64_t channels, int dtype,
                          const void *o, const void *w_o, const float *bias, void *y,
                          void *stream);

/*
 * Patch block: the wrapped layers chained at patch granularity for one
 * denoising step (conv, self-attention and GroupNorm are the module types the
 * source walkthrough wraps, section "Patch Parallelism的实现原理"):
 *
 *   g1 = SiLU(GN1(x))                  async GroupNorm, stale table gn1
 *   h  = conv3x3(g1) + conv_b           halo rows from the stale map conv_in
 *   n2 = GN2(h)                         async GroupNorm, stale table gn2
 *   q, k, v = n2 w_qkv^T + b_qkv        K / V rows written into the k, v maps
 *   o  = softmax(scale q K^T) V         K, V: this patch fresh, others stale
 *   y  = o w_o^T + b_o
 *
 * Every stale read comes from state_in; this step's fresh values (g1 rows,
 * GN moments, K and V rows) go to patch i's rows / slots of state_out, which
 * become the next step's stale context.  state_out may be state_in itself
 * (one device's buffers: a patch never reads its own stale rows), or a
 * second set of buffers, so that all n patches of one step can run on one
 * device against the same previous state.
 */
typedef struct {
    int64_t channels; /* C = heads * 64 */
    int64_t groups;   /* GroupNorm groups G (both norms) */
    int64_t heads;
    float eps;        /* GroupNorm eps */
    float scale;      /* attention scale, > 0 (1/8 for head_dim 64) */
    const float *gn1_gamma, *gn1_beta; /* [C] fp32 or NULL */
    const void *conv_w;                /* [C, 3, 3, C] dtype */
    const float *conv_b;               /* [C] fp32 or NULL */
    const float *gn2_gamma, *gn2_beta; /* [C] fp32 or NULL */
    const void *w_qkv;                 /* [3C, C] dtype: Q, K, V rows */
    const float *b_qkv;                /* [3C] fp32 or NULL */
    const void *w_o;                   /* [C, C] dtype */
    const float *b_o;                  /* [C] fp32 or NULL */
} distri_block_weights;

typedef struct {
    float *gn1;    /* [B, n, G, 2] fp32: per-patch raw moments of x */
    void *conv_in; /* [B, H, W, C] dtype: g1 of every patch */
    float *gn2;    /* [B, n, G, 2] fp32: per-patch raw moments of h */
    void *k, *v;   /* [B, H*W, C] dtype */
} distri_block_state;

/*
 * distri_patch_block - one asynchronous step of the block for patch i.
 *   x [B, h, W, C] dtype -> y [B, Lq, C] dtype
 * Limits: C = heads * 64, C % 64 == 0, the GroupNorm limits, and those of
 * the ops above.  Every pointer 16-byte aligned.  The states' maps must not
 * overlap x, y, the weights or the workspace, and state_out's maps must
 * either be state_in's or not overlap them (DISTRI_ERR_ALIAS).
 * workspace >= distri_patch_block_workspace_size() bytes.
 */
int distri_patch_block_workspace_size(const distri_patch_geom *g,
                                      const distri_block_weights *w, int dtype, size_t *bytes);
int distri_patch_block(const distri_patch_geom *g, const distri_block_weights *w, int dtype,
                       const void *x, void *y, const distri_block_state *state_in,
                       const distri_block_state *state_out, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * distri_patch_block_sync - the synchronous (warm-up) step of the block for
 * all n patches on one device: before any patch reads another's activations
 * of a stage, every patch has produced them, so the result is the block over
 * the whole image, and afterwards `state` holds every patch's current values
 * (the asynchronous steps' first stale context).  g->patch is ignored.
 *   x  [n][B, h, W, C] dtype (patch-major)  ->  y  [n][B, Lq, C] dtype
 *   state  as above; its previous contents are never read
 * workspace >= distri_patch_block_sync_workspace_size() bytes.
 */
int distri_patch_block_sync_workspace_size(const distri_patch_geom *g,
                                           const distri_block_weights *w, int dtype,
                                           size_t *bytes);
int distri_patch_block_sync(const distri_patch_geom *g, const distri_block_weights *w, int dtype,
                            const void *x, void *y, const distri_block_state *state,
                            void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DISTRI_PATCH_H */
