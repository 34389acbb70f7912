// Shared device-side helpers and the internal launcher interface of the
// gfx950 patch-layer library.  Internal to the HIP library; not part of the
// C ABI (include/distri_patch.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32.  Widening is exact; narrowing is round-to-nearest-even
// (the compiler emits v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(uint32_t(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Two packed fp32 values -> two f16, round to nearest even (gfx950:
// v_cvt_pk_f16_f32).  Values beyond the f16 range become +-inf.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2 v;
    v.x = (_Float16)lo;
    v.y = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
// A word of two bf16 -> the same two values as f16.  Exact for magnitudes in
// [2^-14, 65504] and for zero; smaller values round to the f16 subnormal
// grid (absolute error below 2^-25), larger ones (|v| >= 65536) become inf.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// Element-type traits for the two storage dtypes: a 16-byte vector holds
// VEC elements.
struct Bf16T {
    typedef uint16_t elem;
    static constexpr int VEC = 8;
    __device__ static float to_f32(elem e) { return bf16_to_f32(e); }
    __device__ static elem from_f32(float f) { return f32_to_bf16(f); }
    __device__ static void unpack(const u32x4& v, float* out) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[2 * j] = __uint_as_float(v[j] << 16);
            out[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
        }
    }
    __device__ static u32x4 pack(const float* in) {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(in[2 * j], in[2 * j + 1]);
        return v;
    }
};
struct F32T {
    typedef float elem;
    static constexpr int VEC = 4;
    __device__ static float to_f32(elem e) { return e; }
    __device__ static elem from_f32(float f) { return f; }
    __device__ static void unpack(const u32x4& v, float* out) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = __uint_as_float(v[j]);
    }
    __device__ static u32x4 pack(const float* in) {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __float_as_uint(in[j]);
        return v;
    }
};

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Direct global -> LDS tile loads (gfx950 global_load_lds_dwordx4).
#define DP_LDS __attribute__((address_space(3)))

// byte address in LDS of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((const DP_LDS void*)(p)));
}

// One 16-byte load per lane straight into LDS: lane l's 16 bytes at `src`
// land at LDS byte address lds_base + 16 l (lds_base is wave-uniform).  No
// register receives the data and no LDS store instruction is issued.
// Written in asm: with the compiler's builtin for this load, the compiler
// waits for every outstanding load into LDS before any LDS read, which
// serialises a multi-stage pipeline; callers wait with s_waitcnt vmcnt
// (vmcnt_imm below) before the barrier that precedes a stage's use, and
// keep nothing of their own in flight across it.  The load takes its LDS
// address from m0, a register the compiler reserves: the asm saves m0,
// sets it and restores it, so whatever the compiler keeps there survives.
__device__ __forceinline__ void global_load_lds16(const void* src, uint32_t lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(m0)
        : "memory");
}

// s_waitcnt immediate for vmcnt(n), n < 16 (gfx9 encoding: expcnt and
// lgkmcnt left free)
constexpr int vmcnt_imm(int n) { return 0x0F70 + n; }

// ---------------------------------------------------------------------------
// Internal launchers.  Arguments are already validated by the ABI layer.
struct Geom {
    int64_t B, H, W, n, i;
    int64_t h() const { return H / n; }
    int64_t lq() const { return (H / n) * W; }
    int64_t L() const { return H * W; }
};

// Compute units of the current device (cached per device), or -1.
int device_cus();

hipError_t launch_refresh(const Geom& g, int64_t row_elems, int elem_bytes, const void* fresh,
                          void* stale, hipStream_t s);
// Several maps of one patch at once: map k's fresh [B, rows, row_elems]
// goes to rows [i*rows, (i+1)*rows) of its stale [B, n*rows, row_elems].
constexpr int kRefreshMaxMaps = 8;
struct RefreshMap {
    int64_t rows, row_elems;
    int elem_bytes;
    const void* fresh;
    void* stale;
};
hipError_t launch_refresh_maps(const Geom& g, int count, const RefreshMap* maps, hipStream_t s);

size_t groupnorm_workspace_bytes(const Geom& g, int64_t C, int64_t G, int elem_bytes);
// The GroupNorm scratch array of the allocation-free entry point: its size,
// and its address on the current device (looked up once per device).
constexpr size_t kGnScratchBytes = size_t(2) << 20;
hipError_t groupnorm_scratch(void** ptr);
// mode: plain normalise, normalise then SiLU, or moments only (y, the
// stale table and gamma / beta unused).  fresh_moments[b * fm_stride + 2g
// + {0, 1}] receives (E[x], E[x^2]) of image b, group g over the slice.
enum GnMode { kGnNormalize = 0, kGnNormalizeSilu = 1, kGnMomentsOnly = 2 };
hipError_t launch_groupnorm(const Geom& g, int64_t C, int64_t G, float eps, bool bf16, int mode,
                            const void* x, const float* stale_moments, const float* gamma,
                            const float* beta, void* y, float* fresh_moments, int64_t fm_stride,
                            void* ws, hipStream_t s);

size_t attention_workspace_bytes(const Geom& g, int64_t heads, bool bf16);
size_t attention_workspace_bytes(int64_t B, int64_t lq, int64_t L, int64_t heads, bool bf16);
hipError_t launch_attention(const Geom& g, int64_t heads, float scale, bool bf16, const void* q,
                            const void* kf, const void* vf, const void* ks, const void* vs,
                            void* out, void* ws, hipStream_t s);
// The same kernels with the token ranges given directly: lq queries per
// image against L key/value tokens, of which [own_lo, own_lo + lq) come from
// kf / vf ([B, lq, heads, 64]) and the rest from ks / vs ([B, L, heads, 64]).
// own_lo >= L makes every key come from ks / vs (cross-attention).
hipError_t launch_attention_rows(int64_t B, int64_t lq, int64_t L, int64_t own_lo, int64_t heads,
                                 float scale, bool bf16, const void* q, const void* kf,
                                 const void* vf, const void* ks, const void* vs, void* out,
                                 void* ws, hipStream_t s);

// Cross-attention over a context of at most kCrossCtxMax tokens, held in LDS
// whole (bf16 only): q / out [B, lq, heads, 64], k / v [B, ctx, heads, 64].
// No workspace.  cross_attention_short() says whether a shape takes it.
constexpr int kCrossCtxMax = 128;
bool cross_attention_short(int64_t lq, int64_t ctx, int64_t heads);
hipError_t launch_cross_attention(int64_t B, int64_t lq, int64_t ctx, int64_t heads, float scale,
                                  const void* q, const void* k, const void* v, void* out,
                                  hipStream_t s);

hipError_t launch_qkv_proj(const Geom& g, int64_t C, bool bf16, const void* x, const void* w_qkv,
                           const float* bias, void* q, void* k, void* v, void* k_stale,
                           void* v_stale, hipStream_t s);
hipError_t launch_out_proj(const Geom& g, int64_t C, bool bf16, const void* o, const void* w_o,
                           const float* bias, void* y, hipStream_t s);
// whether an M x N projection output fits one launch's grid
bool proj_launch_fits(int64_t M, int64_t N);

hipError_t launch_conv3x3(const Geom& g, int64_t cin, int64_t cout, bool bf16, const void* xf,
                          const void* xs, const void* w, const float* bias, void* y,
                          hipStream_t s);

}  // namespace dp
