// Patch block runner: the wrapped layers of one SDXL block chained at patch
// granularity ("DistriFusion源码探秘：从DistriUNetPP到DistriAttentionTP的模块
// 设计原理", section "Patch Parallelism的实现原理": conv, self-attention and
// GroupNorm are the layers that the patch-parallel UNet wraps), in the two
// step kinds of the method ("DistriFusion：高分辨率扩散模型的分布式并行推理",
// README mirror, section 概述, figure (c)): the synchronous warm-up step, in
// which every patch sees the others' current activations, and the
// asynchronous step, in which it sees the previous step's.
//
// Host code only: it validates once, carves its workspace and enqueues the
// op kernels on one stream.  No allocation, no synchronisation.
#include "abi_check.h"

using namespace dp_abi;

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Sizes {
    size_t slice;     // bytes of one patch activation [B, h, W, C] = [B, Lq, C]
    size_t map;       // bytes of a full map [B, H, W, C]
    size_t table;     // bytes of a moment table [B, n, G, 2] fp32
    size_t gn_ws;     // GroupNorm workspace
    size_t attn_ws;   // attention workspace
};

Sizes sizes_of(const dp::Geom& g, const distri_block_weights* w, int dtype) {
    const size_t eb = size_t(elem_bytes_of(dtype));
    Sizes z;
    z.slice = size_t(g.B * g.lq() * w->channels) * eb;
    z.map = size_t(g.B * g.L() * w->channels) * eb;
    z.table = size_t(g.B * g.n * w->groups * 2) * 4;
    z.gn_ws = dp::groupnorm_workspace_bytes(g, w->channels, w->groups, int(eb));
    z.attn_ws = dp::attention_workspace_bytes(g, w->heads, dtype == DISTRI_BF16);
    return z;
}

// async: [g1 / n2][h / o][q][k][v][gn ws][attention ws]
size_t async_bytes(const Sizes& z) {
    return 5 * align256(z.slice) + align256(z.gn_ws) + align256(z.attn_ws);
}
// sync: [g1 of all patches / q of all][h of all][k of all][v of all][n2][o][gn ws][attention ws]
size_t sync_bytes(const Sizes& z, int64_t n) {
    return 4 * align256(z.slice * size_t(n)) + 2 * align256(z.slice) + align256(z.gn_ws) +
           align256(z.attn_ws);
}

int check_weights(const distri_patch_geom* g, const distri_block_weights* w, int dtype) {
    DP_CHECK(w != nullptr, DISTRI_ERR_NULL, "weights pointer is NULL");
    int st = check_gn_shape(g, w->channels, w->groups, dtype);
    if (st) return st;
    st = check_attn_shape(g, w->heads, 64, dtype);
    if (st) return st;
    DP_CHECK(w->channels == w->heads * 64, DISTRI_ERR_SHAPE, "channels must equal heads * 64");
    DP_CHECK(std::isfinite(w->eps) && w->eps >= 0.f, DISTRI_ERR_SHAPE, "eps must be finite and >= 0");
    DP_CHECK(std::isfinite(w->scale) && w->scale > 0.f, DISTRI_ERR_SHAPE,
             "scale must be finite and > 0");
    const dp::Geom gg = to_geom(g);
    const int64_t C = w->channels;
    DP_CHECK(gg.B * gg.H * gg.W * C < (int64_t(1) << 31) && 9 * C * C < (int64_t(1) << 31),
             DISTRI_ERR_UNSUPPORTED, "block tensors must stay below 2^31 elements");
    DP_CHECK(dp::proj_launch_fits(gg.B * gg.lq(), 3 * C), DISTRI_ERR_UNSUPPORTED,
             "projection output too large for one launch");
    return DISTRI_OK;
}

// Inputs and outputs of one call, for the pointer checks.  `field` tags the
// state maps (0 = not a state map): an output may coincide exactly with the
// input of the same field (an in-place state), and overlap nothing else.
struct Buf {
    const void* p;
    size_t bytes;
    int field;
};

int check_buffers(const Buf* ins, int nin, const Buf* outs, int nout) {
    for (int a = 0; a < nin; ++a)
        DP_CHECK(ins[a].bytes == 0 || aligned16(ins[a].p), DISTRI_ERR_ALIGN,
                 "block pointers must be 16-byte aligned");
    for (int a = 0; a < nout; ++a)
        DP_CHECK(outs[a].bytes == 0 || aligned16(outs[a].p), DISTRI_ERR_ALIGN,
                 "block pointers must be 16-byte aligned");
    for (int a = 0; a < nout; ++a) {
        for (int b = a + 1; b < nout; ++b)
            DP_CHECK(!overlaps({outs[a].p, outs[a].bytes}, {outs[b].p, outs[b].bytes}),
                     DISTRI_ERR_ALIAS, "block outputs overlap each other");
        for (int b = 0; b < nin; ++b) {
            if (!overlaps({outs[a].p, outs[a].bytes}, {ins[b].p, ins[b].bytes})) continue;
            DP_CHECK(outs[a].field != 0 && outs[a].field == ins[b].field && outs[a].p == ins[b].p,
                     DISTRI_ERR_ALIAS, "a block output overlaps an input");
        }
    }
    return DISTRI_OK;
}

int check_state(const distri_block_state* s) {
    DP_CHECK(s != nullptr, DISTRI_ERR_NULL, "state pointer is NULL");
    DP_CHECK(s->gn1 && s->conv_in && s->gn2 && s->k && s->v, DISTRI_ERR_NULL,
             "a state map pointer is NULL");
    return DISTRI_OK;
}

int weight_bufs(const distri_block_weights* w, int dtype, Buf* out) {
    const size_t eb = size_t(elem_bytes_of(dtype));
    const int64_t C = w->channels;
    const size_t cb = size_t(C) * 4;
    int k = 0;
    out[k++] = {w->gn1_gamma, w->gn1_gamma ? cb : 0, 0};
    out[k++] = {w->gn1_beta, w->gn1_beta ? cb : 0, 0};
    out[k++] = {w->conv_w, size_t(9 * C * C) * eb, 0};
    out[k++] = {w->conv_b, w->conv_b ? cb : 0, 0};
    out[k++] = {w->gn2_gamma, w->gn2_gamma ? cb : 0, 0};
    out[k++] = {w->gn2_beta, w->gn2_beta ? cb : 0, 0};
    out[k++] = {w->w_qkv, size_t(3 * C * C) * eb, 0};
    out[k++] = {w->b_qkv, w->b_qkv ? 3 * cb : 0, 0};
    out[k++] = {w->w_o, size_t(C * C) * eb, 0};
    out[k++] = {w->b_o, w->b_o ? cb : 0, 0};
    return k;
}

int state_bufs(const distri_block_state* s, const Sizes& z, Buf* out) {
    out[0] = {s->gn1, z.table, 1};
    out[1] = {s->conv_in, z.map, 2};
    out[2] = {s->gn2, z.table, 3};
    out[3] = {s->k, z.map, 4};
    out[4] = {s->v, z.map, 5};
    return 5;
}

#define HIP_TRY(expr)                              \
    do {                                           \
        hipError_t e_ = (expr);                    \
        if (e_ != hipSuccess) return hip_status(e_); \
    } while (0)

// One asynchronous step of patch g.i: stale reads from `in`, fresh writes to
// `out`, temporaries in the workspace.
int run_async(const dp::Geom& g, const distri_block_weights* w, bool bf16, const void* x, void* y,
              const distri_block_state* in, const distri_block_state* out, char* ws,
              const Sizes& z, hipStream_t s) {
    const int64_t C = w->channels, G = w->groups;
    const int eb = bf16 ? 2 : 4;
    char* g1 = ws;                         // later n2
    char* h = g1 + align256(z.slice);      // later o
    char* q = h + align256(z.slice);
    char* k = q + align256(z.slice);
    char* v = k + align256(z.slice);
    char* gn_ws = v + align256(z.slice);
    char* attn_ws = gn_ws + align256(z.gn_ws);
    HIP_TRY(dp::launch_groupnorm(g, C, G, w->eps, bf16, dp::kGnNormalizeSilu, x, in->gn1,
                                 w->gn1_gamma, w->gn1_beta, g1, out->gn1 + g.i * G * 2,
                                 g.n * G * 2, gn_ws, s));
    HIP_TRY(dp::launch_conv3x3(g, C, C, bf16, g1, in->conv_in, w->conv_w, w->conv_b, h, s));
    HIP_TRY(dp::launch_refresh(g, g.W * C, eb, g1, out->conv_in, s));
    HIP_TRY(dp::launch_groupnorm(g, C, G, w->eps, bf16, dp::kGnNormalize, h, in->gn2,
                                 w->gn2_gamma, w->gn2_beta, g1, out->gn2 + g.i * G * 2,
                                 g.n * G * 2, gn_ws, s));
    HIP_TRY(dp::launch_qkv_proj(g, C, bf16, g1, w->w_qkv, w->b_qkv, q, k, v, out->k, out->v, s));
    HIP_TRY(dp::launch_attention(g, w->heads, w->scale, bf16, q, k, v, in->k, in->v, h, attn_ws,
                                 s));
    HIP_TRY(dp::launch_out_proj(g, C, bf16, h, w->w_o, w->b_o, y, s));
    return DISTRI_OK;
}

// The synchronous step of all n patches: each stage runs for every patch
// before the next stage reads the others' values.
int run_sync(dp::Geom g, const distri_block_weights* w, bool bf16, const char* x, char* y,
             const distri_block_state* st, char* ws, const Sizes& z, hipStream_t s) {
    const int64_t C = w->channels, G = w->groups, n = g.n;
    const int eb = bf16 ? 2 : 4;
    const size_t S = z.slice;
    char* g1_all = ws;                                  // later q of all patches
    char* h_all = g1_all + align256(S * size_t(n));
    char* k_all = h_all + align256(S * size_t(n));
    char* v_all = k_all + align256(S * size_t(n));
    char* n2 = v_all + align256(S * size_t(n));
    char* o = n2 + align256(S);
    char* gn_ws = o + align256(S);
    char* attn_ws = gn_ws + align256(z.gn_ws);
    const int64_t tstride = n * G * 2;
    for (g.i = 0; g.i < n; ++g.i)
        HIP_TRY(dp::launch_groupnorm(g, C, G, 0.f, bf16, dp::kGnMomentsOnly, x + g.i * S, nullptr,
                                     nullptr, nullptr, nullptr, st->gn1 + g.i * G * 2, tstride,
                                     gn_ws, s));
    for (g.i = 0; g.i < n; ++g.i) {
        char* g1 = g1_all + g.i * S;
        HIP_TRY(dp::launch_groupnorm(g, C, G, w->eps, bf16, dp::kGnNormalizeSilu, x + g.i * S,
                                     st->gn1, w->gn1_gamma, w->gn1_beta, g1,
                                     st->gn1 + g.i * G * 2, tstride, gn_ws, s));
        HIP_TRY(dp::launch_refresh(g, g.W * C, eb, g1, st->conv_in, s));
    }
    for (g.i = 0; g.i < n; ++g.i)
        HIP_TRY(dp::launch_conv3x3(g, C, C, bf16, g1_all + g.i * S, st->conv_in, w->conv_w,
                                   w->conv_b, h_all + g.i * S, s));
    for (g.i = 0; g.i < n; ++g.i)
        HIP_TRY(dp::launch_groupnorm(g, C, G, 0.f, bf16, dp::kGnMomentsOnly, h_all + g.i * S,
                                     nullptr, nullptr, nullptr, nullptr, st->gn2 + g.i * G * 2,
                                     tstride, gn_ws, s));
    char* q_all = g1_all;
    for (g.i = 0; g.i < n; ++g.i) {
        HIP_TRY(dp::launch_groupnorm(g, C, G, w->eps, bf16, dp::kGnNormalize, h_all + g.i * S,
                                     st->gn2, w->gn2_gamma, w->gn2_beta, n2,
                                     st->gn2 + g.i * G * 2, tstride, gn_ws, s));
        HIP_TRY(dp::launch_qkv_proj(g, C, bf16, n2, w->w_qkv, w->b_qkv, q_all + g.i * S,
                                    k_all + g.i * S, v_all + g.i * S, st->k, st->v, s));
    }
    for (g.i = 0; g.i < n; ++g.i) {
        HIP_TRY(dp::launch_attention(g, w->heads, w->scale, bf16, q_all + g.i * S,
                                     k_all + g.i * S, v_all + g.i * S, st->k, st->v, o, attn_ws,
                                     s));
        HIP_TRY(dp::launch_out_proj(g, C, bf16, o, w->w_o, w->b_o, y + g.i * S, s));
    }
    return DISTRI_OK;
}

}  // namespace

extern "C" {

int distri_patch_block_workspace_size(const distri_patch_geom* g, const distri_block_weights* w,
                                      int dtype, size_t* bytes) {
    DP_CHECK(bytes != nullptr, DISTRI_ERR_NULL, "bytes pointer is NULL");
    int st = check_weights(g, w, dtype);
    if (st) return st;
    *bytes = async_bytes(sizes_of(to_geom(g), w, dtype));
    return DISTRI_OK;
}

int distri_patch_block_sync_workspace_size(const distri_patch_geom* g,
                                           const distri_block_weights* w, int dtype,
                                           size_t* bytes) {
    DP_CHECK(bytes != nullptr, DISTRI_ERR_NULL, "bytes pointer is NULL");
    int st = check_weights(g, w, dtype);
    if (st) return st;
    const dp::Geom gg = to_geom(g);
    *bytes = sync_bytes(sizes_of(gg, w, dtype), gg.n);
    return DISTRI_OK;
}

int distri_patch_block(const distri_patch_geom* g, const distri_block_weights* w, int dtype,
                       const void* x, void* y, const distri_block_state* state_in,
                       const distri_block_state* state_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
    int st = check_weights(g, w, dtype);
    if (st) return st;
    const dp::Geom gg = to_geom(g);
    const Sizes z = sizes_of(gg, w, dtype);
    if (z.slice == 0) return DISTRI_OK;
    DP_CHECK(x && y && w->conv_w && w->w_qkv && w->w_o, DISTRI_ERR_NULL, "a tensor pointer is NULL");
    st = check_state(state_in);
    if (st) return st;
    st = check_state(state_out);
    if (st) return st;
    const size_t need = async_bytes(z);
    DP_CHECK(workspace != nullptr && workspace_bytes >= need, DISTRI_ERR_WORKSPACE,
             "block workspace missing or too small");
    Buf ins[16], outs[8];
    int nin = 0;
    ins[nin++] = {x, z.slice, 0};
    nin += weight_bufs(w, dtype, ins + nin);
    nin += state_bufs(state_in, z, ins + nin);
    int nout = 0;
    outs[nout++] = {y, z.slice, 0};
    outs[nout++] = {workspace, need, 0};
    nout += state_bufs(state_out, z, outs + nout);
    st = check_buffers(ins, nin, outs, nout);
    if (st) return st;
    return run_async(gg, w, dtype == DISTRI_BF16, x, y, state_in, state_out,
                     static_cast<char*>(workspace), z, static_cast<hipStream_t>(stream));
}

int distri_patch_block_sync(const distri_patch_geom* g, const distri_block_weights* w, int dtype,
                            const void* x, void* y, const distri_block_state* state,
                            void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_weights(g, w, dtype);
    if (st) return st;
    const dp::Geom gg = to_geom(g);
    const Sizes z = sizes_of(gg, w, dtype);
    if (z.slice == 0) return DISTRI_OK;
    DP_CHECK(x && y && w->conv_w && w->w_qkv && w->w_o, DISTRI_ERR_NULL, "a tensor pointer is NULL");
    st = check_state(state);
    if (st) return st;
    const size_t need = sync_bytes(z, gg.n);
    DP_CHECK(workspace != nullptr && workspace_bytes >= need, DISTRI_ERR_WORKSPACE,
             "block workspace missing or too small");
    Buf ins[16], outs[8];
    int nin = 0;
    ins[nin++] = {x, z.slice * size_t(gg.n), 0};
    nin += weight_bufs(w, dtype, ins + nin);
    int nout = 0;
    outs[nout++] = {y, z.slice * size_t(gg.n), 0};
    outs[nout++] = {workspace, need, 0};
    nout += state_bufs(state, z, outs + nout);
    st = check_buffers(ins, nin, outs, nout);
    if (st) return st;
    return run_sync(gg, w, dtype == DISTRI_BF16, static_cast<const char*>(x),
                    static_cast<char*>(y), state, static_cast<char*>(workspace), z,
                    static_cast<hipStream_t>(stream));
}

}  // extern "C"
