// C ABI of the patch-layer library: host-side argument validation and
// dispatch to the gfx950 kernels.  Every check runs before any HIP call, so a
// rejected call enqueues nothing and touches no device state.
#include "abi_check.h"

namespace dp {

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    if (dev < 64) cached[dev] = cus;
    return cus;
}

}  // namespace dp

namespace dp_abi {
thread_local char g_last_error[256] = "";
}  // namespace dp_abi

using namespace dp_abi;

namespace {

// use_scratch: the allocation-free form, whose workspace is the library's
// own scratch array (workspace / workspace_bytes ignored).
int groupnorm_entry(int mode, const distri_patch_geom* g, int64_t channels, int64_t groups,
                    float eps, int dtype, const void* x_fresh, const float* stale_moments,
                    const float* gamma, const float* beta, void* y, float* fresh_moments,
                    void* workspace, size_t workspace_bytes, void* stream,
                    bool use_scratch = false) {
    int st = check_gn_shape(g, channels, groups, dtype);
    if (st) return st;
    DP_CHECK(std::isfinite(eps) && eps >= 0.f, DISTRI_ERR_SHAPE, "eps must be finite and >= 0");
    const dp::Geom gg = to_geom(g);
    const size_t eb = size_t(elem_bytes_of(dtype));
    const size_t xbytes = size_t(gg.B * gg.h() * gg.W * channels) * eb;
    if (xbytes == 0) return DISTRI_OK;
    DP_CHECK(x_fresh && stale_moments && y && fresh_moments, DISTRI_ERR_NULL,
             "a tensor pointer is NULL");
    DP_CHECK(aligned16(x_fresh) && aligned16(stale_moments) && aligned16(gamma) &&
                 aligned16(beta) && aligned16(y) && aligned16(fresh_moments),
             DISTRI_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const size_t need = dp::groupnorm_workspace_bytes(gg, channels, groups, int(eb));
    if (use_scratch) {
        DP_CHECK(need <= dp::kGnScratchBytes, DISTRI_ERR_UNSUPPORTED,
                 "this shape needs more GroupNorm scratch than the 2 MiB the allocation-free form "
                 "holds: use distri_async_groupnorm with a workspace");
        workspace = nullptr;  // not an argument of this form; no overlap to check
    } else {
        DP_CHECK(workspace != nullptr && workspace_bytes >= need, DISTRI_ERR_WORKSPACE,
                 "groupnorm workspace missing or too small");
        DP_CHECK(aligned16(workspace), DISTRI_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    const size_t table = size_t(gg.B * gg.n * groups * 2) * 4;
    const size_t fm = size_t(gg.B * groups * 2) * 4;
    const size_t cb = size_t(channels) * 4;
    const Range outs[3] = {{y, xbytes}, {fresh_moments, fm}, {workspace, need}};
    const Range ins[4] = {{x_fresh, xbytes}, {stale_moments, table}, {gamma, gamma ? cb : 0},
                          {beta, beta ? cb : 0}};
    for (const Range& o : outs)
        for (const Range& in : ins)
            DP_CHECK(!overlaps(o, in), DISTRI_ERR_ALIAS, "an output overlaps an input");
    DP_CHECK(!overlaps(outs[0], outs[1]) && !overlaps(outs[0], outs[2]) &&
                 !overlaps(outs[1], outs[2]),
             DISTRI_ERR_ALIAS, "outputs overlap each other");
    if (use_scratch) {
        const hipError_t e = dp::groupnorm_scratch(&workspace);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(dp::launch_groupnorm(gg, channels, groups, eps, dtype == DISTRI_BF16, mode,
                                           x_fresh, stale_moments, gamma, beta, y, fresh_moments,
                                           groups * 2, workspace,
                                           static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int distri_abi_version(void) { return DISTRI_PATCH_ABI_VERSION; }

const char* distri_status_str(int status) {
    switch (status) {
        case DISTRI_OK: return "ok";
        case DISTRI_ERR_NULL: return "null pointer";
        case DISTRI_ERR_SHAPE: return "invalid shape";
        case DISTRI_ERR_DTYPE: return "invalid dtype";
        case DISTRI_ERR_ALIGN: return "misaligned pointer";
        case DISTRI_ERR_UNSUPPORTED: return "unsupported configuration";
        case DISTRI_ERR_WORKSPACE: return "workspace missing or too small";
        case DISTRI_ERR_HIP: return "HIP runtime error";
        case DISTRI_ERR_ALIAS: return "output overlaps an input";
        default: return "unknown status";
    }
}

const char* distri_last_error(void) { return g_last_error; }

int distri_patch_self_attn_workspace_size(const distri_patch_geom* g, int64_t heads,
                                          int64_t head_dim, int dtype, size_t* bytes) {
    DP_CHECK(bytes != nullptr, DISTRI_ERR_NULL, "bytes pointer is NULL");
    int st = check_attn_shape(g, heads, head_dim, dtype);
    if (st) return st;
    *bytes = dp::attention_workspace_bytes(to_geom(g), heads, dtype == DISTRI_BF16);
    return DISTRI_OK;
}

int distri_patch_self_attn(const distri_patch_geom* g, int64_t heads, int64_t head_dim,
                           float scale, int dtype, const void* q, const void* k_fresh,
                           const void* v_fresh, const void* k_stale, const void* v_stale,
                           void* out, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_attn_shape(g, heads, head_dim, dtype);
    if (st) return st;
    DP_CHECK(std::isfinite(scale) && scale > 0.f, DISTRI_ERR_SHAPE, "scale must be finite and > 0");
    const dp::Geom gg = to_geom(g);
    const size_t eb = size_t(elem_bytes_of(dtype));
    const size_t local = size_t(gg.B * gg.lq() * heads * head_dim) * eb;
    const size_t full = size_t(gg.B * gg.L() * heads * head_dim) * eb;
    if (local == 0) return DISTRI_OK;
    DP_CHECK(q && k_fresh && v_fresh && k_stale && v_stale && out, DISTRI_ERR_NULL,
             "a tensor pointer is NULL");
    DP_CHECK(aligned16(q) && aligned16(k_fresh) && aligned16(v_fresh) && aligned16(k_stale) &&
                 aligned16(v_stale) && aligned16(out),
             DISTRI_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const Range o{out, local};
    DP_CHECK(!overlaps(o, {q, local}) && !overlaps(o, {k_fresh, local}) &&
                 !overlaps(o, {v_fresh, local}) && !overlaps(o, {k_stale, full}) &&
                 !overlaps(o, {v_stale, full}),
             DISTRI_ERR_ALIAS, "out overlaps an input");
    const size_t need = dp::attention_workspace_bytes(gg, heads, dtype == DISTRI_BF16);
    if (need > 0) {
        DP_CHECK(workspace != nullptr && workspace_bytes >= need, DISTRI_ERR_WORKSPACE,
                 "attention workspace missing or too small");
        DP_CHECK(aligned16(workspace), DISTRI_ERR_ALIGN, "workspace must be 16-byte aligned");
        const Range w{workspace, need};
        DP_CHECK(!overlaps(w, o) && !overlaps(w, {q, local}) && !overlaps(w, {k_fresh, local}) &&
                     !overlaps(w, {v_fresh, local}) && !overlaps(w, {k_stale, full}) &&
                     !overlaps(w, {v_stale, full}),
                 DISTRI_ERR_ALIAS, "workspace overlaps an input or out");
    }
    return hip_status(dp::launch_attention(gg, heads, scale, dtype == DISTRI_BF16, q, k_fresh,
                                           v_fresh, k_stale, v_stale, out, workspace,
                                           static_cast<hipStream_t>(stream)));
}

int distri_patch_cross_attn_workspace_size(const distri_patch_geom* g, int64_t heads,
                                           int64_t head_dim, int64_t ctx_len, int dtype,
                                           size_t* bytes) {
    DP_CHECK(bytes != nullptr, DISTRI_ERR_NULL, "bytes pointer is NULL");
    int st = check_cross_shape(g, heads, head_dim, ctx_len, dtype);
    if (st) return st;
    const dp::Geom gg = to_geom(g);
    const bool bf16 = dtype == DISTRI_BF16;
    *bytes = bf16 && dp::cross_attention_short(gg.lq(), ctx_len, heads)
                 ? 0
                 : dp::attention_workspace_bytes(gg.B, gg.lq(), ctx_len, heads, bf16);
    return DISTRI_OK;
}

int distri_patch_cross_attn(const distri_patch_geom* g, int64_t heads, int64_t head_dim,
                            int64_t ctx_len, float scale, int dtype, const void* q,
                            const void* k_ctx, const void* v_ctx, void* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
    int st = check_cross_shape(g, heads, head_dim, ctx_len, dtype);
    if (st) return st;
    DP_CHECK(std::isfinite(scale) && scale > 0.f, DISTRI_ERR_SHAPE, "scale must be finite and > 0");
    const dp::Geom gg = to_geom(g);
    const size_t eb = size_t(elem_bytes_of(dtype));
    const size_t local = size_t(gg.B * gg.lq() * heads * head_dim) * eb;
    const size_t ctx = size_t(gg.B * ctx_len * heads * head_dim) * eb;
    if (local == 0) return DISTRI_OK;
    DP_CHECK(q && k_ctx && v_ctx && out, DISTRI_ERR_NULL, "a tensor pointer is NULL");
    DP_CHECK(aligned16(q) && aligned16(k_ctx) && aligned16(v_ctx) && aligned16(out),
             DISTRI_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const Range o{out, local};
    DP_CHECK(!overlaps(o, {q, local}) && !overlaps(o, {k_ctx, ctx}) && !overlaps(o, {v_ctx, ctx}),
             DISTRI_ERR_ALIAS, "out overlaps an input");
    const bool bf16 = dtype == DISTRI_BF16;
    const bool short_ctx = bf16 && dp::cross_attention_short(gg.lq(), ctx_len, heads);
    const size_t need =
        short_ctx ? 0 : dp::attention_workspace_bytes(gg.B, gg.lq(), ctx_len, heads, bf16);
    if (need > 0) {
        DP_CHECK(workspace != nullptr && workspace_bytes >= need, DISTRI_ERR_WORKSPACE,
                 "attention workspace missing or too small");
        DP_CHECK(aligned16(workspace), DISTRI_ERR_ALIGN, "workspace must be 16-byte aligned");
        const Range w{workspace, need};
        DP_CHECK(!overlaps(w, o) && !overlaps(w, {q, local}) && !overlaps(w, {k_ctx, ctx}) &&
                     !overlaps(w, {v_ctx, ctx}),
                 DISTRI_ERR_ALIAS, "workspace overlaps an input or out");
    }
    if (short_ctx)  // the whole context held in LDS
        return hip_status(dp::launch_cross_attention(gg.B, gg.lq(), ctx_len, heads, scale, q, k_ctx,
                                                     v_ctx, out, static_cast<hipStream_t>(stream)));
    // every key is a context token: the fresh range starts past the context
    return hip_status(dp::launch_attention_rows(gg.B, gg.lq(), ctx_len, ctx_len, heads, scale,
                                                bf16, q, k_ctx, v_ctx, k_ctx,
                                                v_ctx, out, workspace,
                                                static_cast<hipStream_t>(stream)));
}

int distri_patch_conv3x3_halo(const distri_patch_geom* g, int64_t c_in, int64_t c_out,
                              int dtype, const void* x_fresh, const void* x_stale,
                              const void* weight, const float* bias, void* y, void* stream) {
    int st = check_geom(g);
    if (st) return st;
    st = check_dtype(dtype);
    if (st) return st;
    DP_CHECK(c_in >= 1 && c_out >= 1, DISTRI_ERR_SHAPE, "c_in and c_out must be >= 1");
    DP_CHECK(c_in <= 65536 && c_out <= 65536, DISTRI_ERR_UNSUPPORTED, "channels above 65536");
    const dp::Geom gg = to_geom(g);
    if (dtype == DISTRI_BF16) {
        DP_CHECK(c_in % 64 == 0, DISTRI_ERR_UNSUPPORTED, "bf16 conv needs c_in % 64 == 0");
        DP_CHECK(gg.B * gg.H * gg.W * c_in < (int64_t(1) << 31) &&
                     gg.B * gg.H * gg.W * c_out < (int64_t(1) << 31) &&
                     c_out * 9 * c_in < (int64_t(1) << 31),
                 DISTRI_ERR_UNSUPPORTED, "bf16 conv tensors must stay below 2^31 elements");
    }
    const size_t eb = size_t(elem_bytes_of(dtype));
    const size_t ybytes = size_t(gg.B * gg.h() * gg.W * c_out) * eb;
    if (ybytes == 0) return DISTRI_OK;
    const size_t xf_bytes = size_t(gg.B * gg.h() * gg.W * c_in) * eb;
    const size_t xs_bytes = size_t(gg.B * gg.H * gg.W * c_in) * eb;
    const size_t w_bytes = size_t(c_out * 9 * c_in) * eb;
    const bool need_stale = gg.n > 1;
    DP_CHECK(x_fresh && weight && y && (x_stale || !need_stale), DISTRI_ERR_NULL,
             "a tensor pointer is NULL");
    DP_CHECK(aligned16(x_fresh) && aligned16(x_stale) && aligned16(weight) && aligned16(y) &&
                 aligned16(bias),
             DISTRI_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const Range o{y, ybytes};
    DP_CHECK(!overlaps(o, {x_fresh, xf_bytes}) && !overlaps(o, {x_stale, xs_bytes}) &&
                 !overlaps(o, {weight, w_bytes}) &&
                 !overlaps(o, {bias, bias ? size_t(c_out) * 4 : 0}),
             DISTRI_ERR_ALIAS, "y overlaps an input");
    return hip_status(dp::launch_conv3x3(gg, c_in, c_out, dtype == DISTRI_BF16, x_fresh, x_stale,
                                         weight, bias, y, static_cast<hipStream_t>(stream)));
}

int distri_async_groupnorm_workspace_size(const distri_patch_geom* g, int64_t channels,
                                          int64_t groups, int dtype, size_t* bytes) {
    DP_CHECK(bytes != nullptr, DISTRI_ERR_NULL, "bytes pointer is NULL");
    int st = check_gn_shape(g, channels, groups, dtype);
    if (st) return st;
    *bytes = dp::groupnorm_workspace_bytes(to_geom(g), channels, groups, elem_bytes_of(dtype));
    return DISTRI_OK;
}

int distri_async_groupnorm(const distri_patch_geom* g, int64_t channels, int64_t groups,
                           float eps, int dtype, const void* x_fresh,
                           const float* stale_moments, const float* gamma, const float* beta,
                           void* y, float* fresh_moments, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return groupnorm_entry(dp::kGnNormalize, g, channels, groups, eps, dtype, x_fresh,
                           stale_moments, gamma, beta, y, fresh_moments, workspace,
                           workspace_bytes, stream);
}

int distri_async_groupnorm_noalloc(const distri_patch_geom* g, int64_t channels, int64_t groups,
                                   float eps, int dtype, const void* x_fresh,
                                   const float* stale_moments, const float* gamma,
                                   const float* beta, void* y, float* fresh_moments, void* stream) {
    return groupnorm_entry(dp::kGnNormalize, g, channels, groups, eps, dtype, x_fresh,
                           stale_moments, gamma, beta, y, fresh_moments, nullptr, 0, stream,
                           true);
}

int distri_async_groupnorm_silu(const distri_patch_geom* g, int64_t channels, int64_t groups,
                                float eps, int dtype, const void* x_fresh,
                                const float* stale_moments, const float* gamma,
                                const float* beta, void* y, float* fresh_moments,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return groupnorm_entry(dp::kGnNormalizeSilu, g, channels, groups, eps, dtype, x_fresh,
                           stale_moments, gamma, beta, y, fresh_moments, workspace,
                           workspace_bytes, stream);
}

int distri_group_moments(const distri_patch_geom* g, int64_t channels, int64_t groups, int dtype,
                         const void* x_fresh, float* table, void* workspace,
                         size_t workspace_bytes, void* stream) {
    int st = check_gn_shape(g, channels, groups, dtype);
    if (st) return st;
    const dp::Geom gg = to_geom(g);
    const size_t eb = size_t(elem_bytes_of(dtype));
    const size_t xbytes = size_t(gg.B * gg.h() * gg.W * channels) * eb;
    if (gg.B == 0) return DISTRI_OK;
    DP_CHECK(gg.h() * gg.W > 0, DISTRI_ERR_SHAPE, "the patch holds no pixels: moments undefined");
    DP_CHECK(x_fresh && table, DISTRI_ERR_NULL, "a tensor pointer is NULL");
    DP_CHECK(aligned16(x_fresh) && aligned16(table), DISTRI_ERR_ALIGN,
             "tensor pointers must be 16-byte aligned");
    const size_t need = dp::groupnorm_workspace_bytes(gg, channels, groups, int(eb));
    DP_CHECK(workspace != nullptr && workspace_bytes >= need, DISTRI_ERR_WORKSPACE,
             "groupnorm workspace missing or too small");
    DP_CHECK(aligned16(workspace), DISTRI_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t tbytes = size_t(gg.B * gg.n * groups * 2) * 4;
    DP_CHECK(!overlaps({table, tbytes}, {x_fresh, xbytes}) &&
                 !overlaps({workspace, need}, {x_fresh, xbytes}) &&
                 !overlaps({workspace, need}, {table, tbytes}),
             DISTRI_ERR_ALIAS, "table, workspace and x_fresh must not overlap");
    return hip_status(dp::launch_groupnorm(gg, channels, groups, 0.f, dtype == DISTRI_BF16,
                                           dp::kGnMomentsOnly, x_fresh, nullptr, nullptr, nullptr,
                                           nullptr, table + gg.i * groups * 2,
                                           gg.n * groups * 2, workspace,
                                           static_cast<hipStream_t>(stream)));
}

int distri_refresh_stale(const distri_patch_geom* g, int64_t row_elems, int dtype,
                         const void* fresh, void* stale, void* stream) {
    int st = check_geom(g);
    if (st) return st;
    st = check_dtype(dtype);
    if (st) return st;
    DP_CHECK(row_elems >= 0, DISTRI_ERR_SHAPE, "row_elems must be >= 0");
    DP_CHECK(row_elems <= (int64_t(1) << 32), DISTRI_ERR_UNSUPPORTED, "row_elems above 2^32");
    const dp::Geom gg = to_geom(g);
    const size_t eb = size_t(elem_bytes_of(dtype));
    const size_t fbytes = size_t(gg.B * gg.h() * row_elems) * eb;
    if (fbytes == 0) return DISTRI_OK;
    DP_CHECK(fresh && stale, DISTRI_ERR_NULL, "a tensor pointer is NULL");
    DP_CHECK((reinterpret_cast<uintptr_t>(fresh) % eb) == 0 &&
                 (reinterpret_cast<uintptr_t>(stale) % eb) == 0,
             DISTRI_ERR_ALIGN, "pointers must be aligned to the element size");
    const size_t sbytes = size_t(gg.B * gg.H * row_elems) * eb;
    DP_CHECK(!overlaps({stale, sbytes}, {fresh, fbytes}), DISTRI_ERR_ALIAS,
             "stale overlaps fresh");
    return hip_status(dp::launch_refresh(gg, row_elems, int(eb), fresh, stale,
                                         static_cast<hipStream_t>(stream)));
}

int distri_refresh_stale_maps(const distri_patch_geom* g, int count, const distri_refresh_map* maps,
                              void* stream) {
    int st = check_geom(g);
    if (st) return st;
    DP_CHECK(count >= 0, DISTRI_ERR_SHAPE, "count must be >= 0");
    DP_CHECK(count <= DISTRI_REFRESH_MAX_MAPS, DISTRI_ERR_UNSUPPORTED,
             "more than DISTRI_REFRESH_MAX_MAPS maps");
    DP_CHECK(count == 0 || maps != nullptr, DISTRI_ERR_NULL, "maps is NULL");
    static_assert(DISTRI_REFRESH_MAX_MAPS == dp::kRefreshMaxMaps, "map limit");
    const dp::Geom gg = to_geom(g);
    dp::RefreshMap rm[DISTRI_REFRESH_MAX_MAPS];
    Range fr[DISTRI_REFRESH_MAX_MAPS], sr[DISTRI_REFRESH_MAX_MAPS];
    for (int k = 0; k < count; ++k) {
        const distri_refresh_map& m = maps[k];
        st = check_dtype(m.dtype);
        if (st) return st;
        DP_CHECK(m.rows >= 0 && m.row_elems >= 0, DISTRI_ERR_SHAPE,
                 "map rows and row_elems must be >= 0");
        DP_CHECK(m.rows <= (int64_t(1) << 32) && m.row_elems <= (int64_t(1) << 32),
                 DISTRI_ERR_UNSUPPORTED, "map rows or row_elems above 2^32");
        const size_t eb = size_t(elem_bytes_of(m.dtype));
        const size_t fbytes = size_t(gg.B * m.rows * m.row_elems) * eb;
        DP_CHECK(fbytes == 0 || (m.fresh && m.stale), DISTRI_ERR_NULL, "a map pointer is NULL");
        DP_CHECK((reinterpret_cast<uintptr_t>(m.fresh) % eb) == 0 &&
                     (reinterpret_cast<uintptr_t>(m.stale) % eb) == 0,
                 DISTRI_ERR_ALIGN, "map pointers must be aligned to the element size");
        fr[k] = {m.fresh, fbytes};
        sr[k] = {m.stale, fbytes ? size_t(gg.B * gg.n * m.rows * m.row_elems) * eb : 0};
        rm[k] = {m.rows, m.row_elems, int(eb), m.fresh, m.stale};
    }
    for (int k = 0; k < count; ++k)
        for (int j = 0; j < count; ++j) {
            DP_CHECK(!overlaps(sr[k], fr[j]), DISTRI_ERR_ALIAS, "a stale map overlaps a fresh map");
            DP_CHECK(j == k || !overlaps(sr[k], sr[j]), DISTRI_ERR_ALIAS,
                     "two stale maps overlap");
        }
    return hip_status(dp::launch_refresh_maps(gg, count, rm, static_cast<hipStream_t>(stream)));
}


int distri_patch_qkv_proj(const distri_patch_geom* g, int64_t channels, int dtype, const void* x,
                          const void* w_qkv, const float* bias, void* q, void* k_fresh,
                          void* v_fresh, void* k_stale, void* v_stale, void* stream) {
    int st = check_geom(g);
    if (st) return st;
    st = check_dtype(dtype);
    if (st) return st;
    DP_CHECK(channels >= 1, DISTRI_ERR_SHAPE, "channels must be >= 1");
    DP_CHECK(channels <= 65536, DISTRI_ERR_UNSUPPORTED, "channels above 65536");
    if (dtype == DISTRI_BF16)
        DP_CHECK(channels % 64 == 0, DISTRI_ERR_UNSUPPORTED, "bf16 projections need channels % 64 == 0");
    const dp::Geom gg = to_geom(g);
    DP_CHECK(gg.B * gg.lq() < (int64_t(1) << 31), DISTRI_ERR_UNSUPPORTED,
             "batch * patch tokens must stay below 2^31");
    DP_CHECK(dp::proj_launch_fits(gg.B * gg.lq(), 3 * channels), DISTRI_ERR_UNSUPPORTED,
             "projection output too large for one launch");
    const size_t eb = size_t(elem_bytes_of(dtype));
    const size_t tok = size_t(gg.B * gg.lq() * channels) * eb;
    if (tok == 0) return DISTRI_OK;
    DP_CHECK(x && w_qkv && q && k_fresh && v_fresh, DISTRI_ERR_NULL, "a tensor pointer is NULL");
    DP_CHECK(aligned16(x) && aligned16(w_qkv) && aligned16(bias) && aligned16(q) &&
                 aligned16(k_fresh) && aligned16(v_fresh) && aligned16(k_stale) && aligned16(v_stale),
             DISTRI_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    const size_t full = size_t(gg.B * gg.L() * channels) * eb;
    const Range ins[3] = {{x, tok}, {w_qkv, size_t(3 * channels * channels) * eb},
                          {bias, bias ? size_t(3 * channels) * 4 : 0}};
    const Range outs[5] = {{q, tok}, {k_fresh, tok}, {v_fresh, tok}, {k_stale, k_stale ? full : 0},
                           {v_stale, v_stale ? full : 0}};
    for (const Range& o : outs)
        for (const Range& in : ins)
            DP_CHECK(!overlaps(o, in), DISTRI_ERR_ALIAS, "an output overlaps an input");
    for (int a = 0; a < 5; ++a)
        for (int b = a + 1; b < 5; ++b)
            DP_CHECK(!overlaps(outs[a], outs[b]), DISTRI_ERR_ALIAS, "outputs overlap each other");
    return hip_status(dp::launch_qkv_proj(gg, channels, dtype == DISTRI_BF16, x, w_qkv, bias, q,
                                          k_fresh, v_fresh, k_stale, v_stale,
                                          static_cast<hipStream_t>(stream)));
}

int distri_patch_out_proj(const distri_patch_geom* g, int64_t channels, int dtype, const void* o,
                          const void* w_o, const float* bias, void* y, void* stream) {
    int st = check_geom(g);
    if (st) return st;
    st = check_dtype(dtype);
    if (st) return st;
    DP_CHECK(channels >= 1, DISTRI_ERR_SHAPE, "channels must be >= 1");
    DP_CHECK(channels <= 65536, DISTRI_ERR_UNSUPPORTED, "channels above 65536");
    if (dtype == DISTRI_BF16)
        DP_CHECK(channels % 64 == 0, DISTRI_ERR_UNSUPPORTED, "bf16 projections need channels % 64 == 0");
    const dp::Geom gg = to_geom(g);
    DP_CHECK(gg.B * gg.lq() < (int64_t(1) << 31), DISTRI_ERR_UNSUPPORTED,
             "batch * patch tokens must stay below 2^31");
    DP_CHECK(dp::proj_launch_fits(gg.B * gg.lq(), channels), DISTRI_ERR_UNSUPPORTED,
             "projection output too large for one launch");
    const size_t eb = size_t(elem_bytes_of(dtype));
    const size_t tok = size_t(gg.B * gg.lq() * channels) * eb;
    if (tok == 0) return DISTRI_OK;
    DP_CHECK(o && w_o && y, DISTRI_ERR_NULL, "a tensor pointer is NULL");
    DP_CHECK(aligned16(o) && aligned16(w_o) && aligned16(bias) && aligned16(y), DISTRI_ERR_ALIGN,
             "tensor pointers must be 16-byte aligned");
    const Range out{y, tok};
    DP_CHECK(!overlaps(out, {o, tok}) && !overlaps(out, {w_o, size_t(channels * channels) * eb}) &&
                 !overlaps(out, {bias, bias ? size_t(channels) * 4 : 0}),
             DISTRI_ERR_ALIAS, "y overlaps an input");
    return hip_status(dp::launch_out_proj(gg, channels, dtype == DISTRI_BF16, o, w_o, bias, y,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"
