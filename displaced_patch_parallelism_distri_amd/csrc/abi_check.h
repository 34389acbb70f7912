// Argument checks shared by the C-ABI entry points (host code, internal).
// Every check runs before any HIP call: a rejected call enqueues nothing.
#pragma once

#include "../../include/distri_patch.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>

#include "dp_common.h"

namespace dp_abi {

// message of the last failed call on this thread (distri_last_error)
extern thread_local char g_last_error[256];

inline int fail(int status, const char* fmt, const char* what) {
    std::snprintf(g_last_error, sizeof(g_last_error), fmt, what);
    return status;
}

#define DP_CHECK(cond, status, msg)                                \
    do {                                                           \
        if (!(cond)) return ::dp_abi::fail((status), "%s", (msg)); \
    } while (0)

inline int elem_bytes_of(int dtype) { return dtype == DISTRI_F32 ? 4 : 2; }

// Geometry rules shared by every call.
inline int check_geom(const distri_patch_geom* g) {
    DP_CHECK(g != nullptr, DISTRI_ERR_NULL, "geometry pointer is NULL");
    DP_CHECK(g->batch >= 0 && g->height >= 0 && g->width >= 0, DISTRI_ERR_SHAPE,
             "batch, height and width must be >= 0");
    DP_CHECK(g->n_patches >= 1, DISTRI_ERR_SHAPE, "n_patches must be >= 1");
    DP_CHECK(g->patch >= 0 && g->patch < g->n_patches, DISTRI_ERR_SHAPE,
             "patch must lie in [0, n_patches)");
    DP_CHECK(g->height % g->n_patches == 0, DISTRI_ERR_SHAPE,
             "height must be a multiple of n_patches");
    DP_CHECK(g->batch <= 65535, DISTRI_ERR_UNSUPPORTED, "batch above 65535");
    // keep every element offset far from int64 overflow
    DP_CHECK(g->height <= (int64_t(1) << 24) && g->width <= (int64_t(1) << 24), DISTRI_ERR_UNSUPPORTED,
             "height or width above 2^24");
    return DISTRI_OK;
}

inline int check_dtype(int dtype) {
    DP_CHECK(dtype == DISTRI_F32 || dtype == DISTRI_BF16, DISTRI_ERR_DTYPE,
             "dtype must be DISTRI_F32 or DISTRI_BF16");
    return DISTRI_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    const void* p;
    size_t bytes;
};
inline bool overlaps(Range a, Range b) {
    if (a.bytes == 0 || b.bytes == 0 || a.p == nullptr || b.p == nullptr) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

inline dp::Geom to_geom(const distri_patch_geom* g) {
    return dp::Geom{g->batch, g->height, g->width, g->n_patches, g->patch};
}

inline int hip_status(hipError_t e) {
    if (e == hipSuccess) return DISTRI_OK;
    std::snprintf(g_last_error, sizeof(g_last_error), "HIP error: %s", hipGetErrorString(e));
    return DISTRI_ERR_HIP;
}

inline int check_attn_shape(const distri_patch_geom* g, int64_t heads, int64_t head_dim, int dtype) {
    int st = check_geom(g);
    if (st) return st;
    st = check_dtype(dtype);
    if (st) return st;
    DP_CHECK(heads >= 1 && head_dim >= 1, DISTRI_ERR_SHAPE, "heads and head_dim must be >= 1");
    DP_CHECK(heads <= 65535 / (g->batch > 0 ? g->batch : 1), DISTRI_ERR_UNSUPPORTED,
             "batch * heads above 65535");
    DP_CHECK(head_dim == 64, DISTRI_ERR_UNSUPPORTED, "head_dim must be 64");
    // the kernels index one image's tokens with 32-bit offsets
    DP_CHECK(g->height * g->width * heads * head_dim < (int64_t(1) << 31), DISTRI_ERR_UNSUPPORTED,
             "height * width * heads * head_dim must stay below 2^31");
    return DISTRI_OK;
}

inline int check_cross_shape(const distri_patch_geom* g, int64_t heads, int64_t head_dim,
                             int64_t ctx_len, int dtype) {
    int st = check_geom(g);
    if (st) return st;
    st = check_dtype(dtype);
    if (st) return st;
    DP_CHECK(heads >= 1 && head_dim >= 1, DISTRI_ERR_SHAPE, "heads and head_dim must be >= 1");
    DP_CHECK(ctx_len >= 1, DISTRI_ERR_SHAPE, "ctx_len must be >= 1");
    DP_CHECK(heads <= 65535 / (g->batch > 0 ? g->batch : 1), DISTRI_ERR_UNSUPPORTED,
             "batch * heads above 65535");
    DP_CHECK(head_dim == 64, DISTRI_ERR_UNSUPPORTED, "head_dim must be 64");
    const int64_t lq = (g->height / g->n_patches) * g->width;
    DP_CHECK(lq * heads * head_dim < (int64_t(1) << 31) &&
                 ctx_len * heads * head_dim < (int64_t(1) << 31),
             DISTRI_ERR_UNSUPPORTED, "tokens * heads * head_dim must stay below 2^31");
    return DISTRI_OK;
}

inline int check_gn_shape(const distri_patch_geom* g, int64_t C, int64_t G, int dtype) {
    int st = check_geom(g);
    if (st) return st;
    st = check_dtype(dtype);
    if (st) return st;
    DP_CHECK(C >= 1 && G >= 1 && C % G == 0, DISTRI_ERR_SHAPE,
             "channels and groups must be >= 1 with channels % groups == 0");
    const int vec = 16 / elem_bytes_of(dtype);
    DP_CHECK(C % vec == 0, DISTRI_ERR_UNSUPPORTED,
             "channels must be a multiple of 8 (bf16) or 4 (fp32)");
    DP_CHECK(C / vec <= 512, DISTRI_ERR_UNSUPPORTED, "channels above 4096 (bf16) / 2048 (fp32)");
    DP_CHECK(G <= 256, DISTRI_ERR_UNSUPPORTED, "more than 256 groups");
    return DISTRI_OK;
}

}  // namespace dp_abi
