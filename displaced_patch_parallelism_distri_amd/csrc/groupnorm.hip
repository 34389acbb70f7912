// Corrected asynchronous GroupNorm of one patch (DistriGroupNorm: "DistriFusion
// 源码探秘：从DistriUNetPP到DistriAttentionTP的模块设计原理", section "Patch
// Parallelism的实现原理", item 3; the default --sync_mode of the README mirror
// "DistriFusion：高分辨率扩散模型的分布式并行推理", sections COCO 质量 / 延迟).
//
// Group statistics of the whole image are formed from this patch's fresh raw
// moments and the other patches' moments of the previous step:
//   mu = (m1 + sum_{j!=i} M1[j]) / n,  e2 = (m2 + sum_{j!=i} M2[j]) / n,
//   rstd = 1 / sqrt(max(e2 - mu^2, 0) + eps),  y = (x - mu) rstd gamma + beta.
//
// Memory-bound.  Two forms:
//  * one launch (gn_fused, the SDXL shapes and most others): every block is
//    resident at once and keeps its chunk of x in registers across a
//    grid-wide hand-off, so x is read from HBM once and y written once; the
//    kernel's comment below has the details;
//  * three launches, for slices too large to hold in the registers of
//    kFusedMaxBlocks blocks (more than 16 pixels per thread) or more images
//    than that:
//   1. gn_moments   - coalesced pass over x [B, h*W, C] (NHWC).  A block is a
//                     (rows x vectors-per-pixel) grid of threads: thread
//                     (row, col) owns one 16-byte channel vector of KV pixels
//                     of its chunk (row, row + rows, ...) and issues all KV
//                     loads before using any, so the whole slice is in flight
//                     at once.  Per-channel fp32 sums are folded into
//                     per-group sums in LDS and written to the workspace
//                     [B][chunks][G][2].
//   2. gn_finalize  - one block per image: fixed-order fp64 reduction of the
//                     chunk sums, the fresh/stale mix, the clamp, and the
//                     per-channel affine a_c = rstd gamma_c,
//                     b_c = beta_c - mu a_c (workspace [B][C][2]).  All of its
//                     global loads are issued before any result is needed.
//   3. gn_normalize - second coalesced pass: y = x a_c + b_c, optionally
//                     followed by SiLU (y / (1 + e^-y), the activation that
//                     follows GroupNorm in SDXL's ResNet blocks), rounded (RNE).
// A moments-only form writes the patch's raw moments alone.  Deterministic:
// no floating-point atomics, every sum has a fixed order.
#include "dp_common.h"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace dp {

// Scratch of the allocation-free entry point (distri_async_groupnorm_noalloc):
// the chunk sums and per-channel affine that the other entry points keep in
// a caller's workspace.  One copy per device, alive until the process ends;
// host code reaches it only through the address hipGetSymbolAddress returns
// for the current device (groupnorm_scratch).  Nothing in it must start at
// zero: every value is written before it is read within a call.
static __device__ __align__(256) unsigned char scratch[kGnScratchBytes];

namespace {

constexpr int kTargetBlocks = 256;
constexpr int kMaxThreads = 512;
constexpr int kMaxKV = 16;

struct GnPlan {
    int vpp;        // 16-byte vectors per pixel
    int rows;       // pixel rows of a block
    int threads;    // vpp * rows
    int kv;         // pixels per thread (power of two)
    int64_t chunks; // chunks (blocks) per image; a chunk is rows * kv pixels
};

GnPlan plan_gn(const Geom& g, int64_t C, int elem_bytes) {
    GnPlan p;
    p.vpp = int(C / (16 / elem_bytes));
    p.rows = kMaxThreads / p.vpp > 0 ? kMaxThreads / p.vpp : 1;
    p.threads = p.vpp * p.rows;
    const int64_t P = g.h() * g.W;
    const int64_t B = g.B > 0 ? g.B : 1;
    const int64_t per_image = kTargetBlocks / B > 0 ? kTargetBlocks / B : 1;
    // pixels per thread: a power of two (the kernels are instantiated per
    // value), the largest that still gives about kTargetBlocks blocks
    const int64_t want = ceil_div(ceil_div(P, p.rows), per_image);
    p.kv = 1;
    while (p.kv * 2 <= want && p.kv * 2 <= kMaxKV) p.kv *= 2;
    p.chunks = ceil_div(P, int64_t(p.rows) * p.kv);
    return p;
}

struct GnWorkspace {
    float* partial;   // [B][chunks][G][2]
    float* affine;    // [B][C][2]
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

GnWorkspace carve(void* ws, const Geom& g, const GnPlan& p, int64_t C, int64_t G) {
    char* base = static_cast<char*>(ws);
    GnWorkspace w;
    w.partial = reinterpret_cast<float*>(base);
    base += align256(size_t(g.B * p.chunks * G * 2) * sizeof(float));
    w.affine = reinterpret_cast<float*>(base);
    return w;
}

size_t workspace_bytes(const Geom& g, const GnPlan& p, int64_t C, int64_t G) {
    return align256(size_t(g.B * p.chunks * G * 2) * sizeof(float)) +
           size_t(g.B * C * 2) * sizeof(float);
}

// Thread (row, col) of chunk `chunk` loads channel vector col of pixels
// p0 + row + k * rows, k < KV.  Every load is issued unconditionally (a
// pixel past the slice re-reads the last pixel) so that all KV are in
// flight together; `valid` marks the real ones.
template <int KV>
__device__ __forceinline__ void load_chunk(const void* __restrict__ x, int64_t P, int vpp,
                                           int rows, int64_t b, int64_t chunk, int row, int col,
                                           u32x4 (&v)[KV], bool (&valid)[KV]) {
    const int64_t p0 = chunk * rows * KV + row;
    const u32x4* src = reinterpret_cast<const u32x4*>(x) + (b * P) * vpp + col;
#pragma unroll
    for (int k = 0; k < KV; ++k) {
        const int64_t p = p0 + int64_t(k) * rows;
        valid[k] = p < P;
        v[k] = src[(p < P ? p : P - 1) * vpp];
    }
    // keep the scheduler from moving the first uses above the later loads
    __builtin_amdgcn_sched_barrier(0);
}

struct GnArgs {
    const void* x;
    void* y;
    int64_t P;       // pixels per image in the slice
    int C, vpp, rows, G;
    int64_t chunks;
    int64_t n, patch;
    double count;    // values per (image, group) in the slice
    float eps;
    const float* stale_moments;
    const float* gamma;
    const float* beta;
    float* fresh_moments;
    int64_t fm_stride;  // floats between images in fresh_moments
    GnWorkspace ws;
};

// Statistics and affine of image blockIdx.x from all its chunk sums.  Every
// global load is issued before any result is needed: the chunk sums, the
// other patches' stale moments and gamma / beta.
constexpr int kFinThreads = 512;
constexpr int kMaxChanPerThread = 8;  // C <= 4096

template <bool MOMENTS_ONLY>
__global__ __launch_bounds__(kFinThreads) void gn_finalize(GnArgs a) {
    extern __shared__ double red[];  // [slices][G][2], then (mu, rstd) [G][2]
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x, T = blockDim.x, G = a.G;
    const int slices = T / G > 0 ? T / G : 1;
    double* stat = red + 2 * slices * G;

    // gamma / beta of channels tid, tid + T, ...
    float gam[kMaxChanPerThread], bet[kMaxChanPerThread];
#pragma unroll
    for (int u = 0; u < kMaxChanPerThread; ++u) {
        gam[u] = 1.f;
        bet[u] = 0.f;
    }
    if (a.gamma) {
#pragma unroll
        for (int u = 0; u < kMaxChanPerThread; ++u) gam[u] = a.gamma[min(tid + u * T, a.C - 1)];
    }
    if (a.beta) {
#pragma unroll
        for (int u = 0; u < kMaxChanPerThread; ++u) bet[u] = a.beta[min(tid + u * T, a.C - 1)];
    }
    // the other patches' stale moments of group tid (G <= 256 < T): the
    // first 8 patches' loads go out now, the sum is formed after the chunk
    // sums' loads are out too
    const uint64_t* tab = reinterpret_cast<const uint64_t*>(a.stale_moments) + b * a.n * G +
                          (tid < G ? tid : 0);
    uint64_t st[8];
    if (!MOMENTS_ONLY) {
#pragma unroll
        for (int u = 0; u < 8; ++u) st[u] = tab[(u < a.n ? u : a.n - 1) * G];
    }
    // thread (slice, g) adds chunks slice, slice + slices, ... in fp64 (16
    // loads in flight; the index is clamped and the extra terms dropped by a
    // select, so the loads need no branches); the slices are then added in
    // order.
    const uint64_t* pp = reinterpret_cast<const uint64_t*>(a.ws.partial) + b * a.chunks * G;
    for (int t = tid; t < slices * G; t += T) {
        const int g = t % G, sl = t / G;
        double a1 = 0.0, a2 = 0.0;
        for (int64_t k0 = sl; k0 < a.chunks; k0 += 16 * int64_t(slices)) {
            uint64_t w[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int64_t k = k0 + int64_t(u) * slices;
                w[u] = pp[(k < a.chunks ? k : a.chunks - 1) * G + g];
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const bool in = k0 + int64_t(u) * slices < a.chunks;
                a1 += in ? double(__uint_as_float(uint32_t(w[u]))) : 0.0;
                a2 += in ? double(__uint_as_float(uint32_t(w[u] >> 32))) : 0.0;
            }
        }
        red[2 * (sl * G + g)] = a1;
        red[2 * (sl * G + g) + 1] = a2;
    }
    double st1 = 0.0, st2 = 0.0;
    for (int64_t j0 = 0; j0 < (MOMENTS_ONLY ? 0 : a.n); j0 += 8) {
        if (j0 > 0) {
#pragma unroll
            for (int u = 0; u < 8; ++u) st[u] = tab[(j0 + u < a.n ? j0 + u : a.n - 1) * G];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool in = j0 + u < a.n && j0 + u != a.patch;
            st1 += in ? double(__uint_as_float(uint32_t(st[u]))) : 0.0;
            st2 += in ? double(__uint_as_float(uint32_t(st[u] >> 32))) : 0.0;
        }
    }
    __syncthreads();
    if (tid < G) {
        const int g = tid;
        double s1 = 0.0, s2 = 0.0;
        for (int sl = 0; sl < slices; ++sl) {
            s1 += red[2 * (sl * G + g)];
            s2 += red[2 * (sl * G + g) + 1];
        }
        const double m1 = s1 / a.count, m2 = s2 / a.count;
        a.fresh_moments[b * a.fm_stride + g * 2 + 0] = float(m1);
        a.fresh_moments[b * a.fm_stride + g * 2 + 1] = float(m2);
        if (MOMENTS_ONLY) return;
        const double e1 = (m1 + st1) / double(a.n);
        const double e2 = (m2 + st2) / double(a.n);
        double var = e2 - e1 * e1;
        if (var < 0.0) var = 0.0;
        stat[2 * g] = e1;
        stat[2 * g + 1] = 1.0 / sqrt(var + double(a.eps));
    }
    if (MOMENTS_ONLY) return;
    __syncthreads();
    const int cg = a.C / G;
#pragma unroll
    for (int u = 0; u < kMaxChanPerThread; ++u) {
        const int c = tid + u * T;
        if (c < a.C) {
            const int g = c / cg;
            const double aa = stat[2 * g + 1] * double(gam[u]);
            a.ws.affine[(b * a.C + c) * 2 + 0] = float(aa);
            a.ws.affine[(b * a.C + c) * 2 + 1] = float(double(bet[u]) - stat[2 * g] * aa);
        }
    }
}

template <class T, int KV>
__global__ __launch_bounds__(kMaxThreads) void gn_moments(GnArgs a) {
    extern __shared__ float lds[];  // [2][rows][C]
    const int64_t b = blockIdx.y, chunk = blockIdx.x;
    const int tid = threadIdx.x;
    const int C = a.C, rows = a.rows, G = a.G;
    const int col = tid % a.vpp, row = tid / a.vpp;
    u32x4 v[KV];
    bool valid[KV];
    load_chunk<KV>(a.x, a.P, a.vpp, rows, b, chunk, row, col, v, valid);
    float s[T::VEC], ss[T::VEC];
#pragma unroll
    for (int j = 0; j < T::VEC; ++j) s[j] = ss[j] = 0.f;
#pragma unroll
    for (int k = 0; k < KV; ++k) {
        float f[T::VEC];
        T::unpack(v[k], f);
#pragma unroll
        for (int j = 0; j < T::VEC; ++j) {
            const float e = valid[k] ? f[j] : 0.f;
            s[j] += e;
            ss[j] = fmaf(e, e, ss[j]);
        }
    }
    // C * row + VEC * col floats is a multiple of 16 bytes
#pragma unroll
    for (int q = 0; q < T::VEC / 4; ++q) {
        *reinterpret_cast<f32x4*>(&lds[row * C + col * T::VEC + 4 * q]) =
            f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
        *reinterpret_cast<f32x4*>(&lds[rows * C + row * C + col * T::VEC + 4 * q]) =
            f32x4{ss[4 * q], ss[4 * q + 1], ss[4 * q + 2], ss[4 * q + 3]};
    }
    __syncthreads();
    // channel totals over the block's rows (fixed order), into row 0
    for (int t = tid; t < 2 * C; t += blockDim.x) {
        const int stat = t / C, c = t % C;
        float* col0 = lds + stat * rows * C + c;
        float acc = col0[0];
        for (int r = 1; r < rows; ++r) acc += col0[r * C];
        col0[0] = acc;
    }
    __syncthreads();
    const int cg = C / G;
    for (int task = tid; task < 2 * G; task += blockDim.x) {
        const int g = task >> 1, stat = task & 1;
        const float* src = lds + stat * rows * C + g * cg;
        float acc = 0.f;
        for (int c = 0; c < cg; ++c) acc += src[c];
        a.ws.partial[((b * a.chunks + chunk) * G + g) * 2 + stat] = acc;
    }
}

template <class T, int KV, bool SILU>
__global__ __launch_bounds__(kMaxThreads) void gn_normalize(GnArgs a) {
    const int64_t b = blockIdx.y, chunk = blockIdx.x;
    const int tid = threadIdx.x;
    const int col = tid % a.vpp, row = tid / a.vpp;
    u32x4 v[KV];
    bool valid[KV];
    load_chunk<KV>(a.x, a.P, a.vpp, a.rows, b, chunk, row, col, v, valid);
    // (a_c, b_c) of this thread's VEC channels: VEC/2 16-byte loads
    const f32x4* af = reinterpret_cast<const f32x4*>(a.ws.affine + (b * a.C + col * T::VEC) * 2);
    f32x4 ab[T::VEC / 2];
#pragma unroll
    for (int q = 0; q < T::VEC / 2; ++q) ab[q] = af[q];
    const int64_t p0 = chunk * a.rows * KV + row;
    u32x4* dst = reinterpret_cast<u32x4*>(a.y) + (b * a.P) * a.vpp + col;
#pragma unroll
    for (int k = 0; k < KV; ++k) {
        if (valid[k]) {
            float f[T::VEC];
            T::unpack(v[k], f);
#pragma unroll
            for (int j = 0; j < T::VEC; ++j) {
                f[j] = fmaf(f[j], ab[j / 2][2 * (j % 2)], ab[j / 2][2 * (j % 2) + 1]);
                if (SILU) f[j] = f[j] / (1.f + __expf(-f[j]));
            }
            __builtin_nontemporal_store(T::pack(f), dst + (p0 + int64_t(k) * a.rows) * a.vpp);
        }
    }
}


// ---------------------------------------------------------------------------
// Single-launch form.  Every block of the launch is resident at once (at
// most kFusedMaxBlocks blocks, checked against the device's occupancy before
// launch), so a block can keep its chunk of x in registers across a
// grid-wide hand-off and the slice is read from HBM once:
//   1. load the chunk (all loads in flight together), per-group fp32 sums of
//      x and x^2 -> the block's slot of the workspace, then its flag;
//   2. wait until every block of its image has raised its flag (block 0:
//      every block of the launch);
//   3. every block reduces its image's slots in the same fixed order (so all
//      blocks hold bit-identical statistics), mixes in the stale moments,
//      clamps, and normalises the chunk still held in registers.
// x comes in and y goes out through buffer resources spanning one image's
// slice, whose range checks replace the tail masks.
// The flags carry a value unique to the call, derived from a count of the
// calls made on the workspace that the workspace itself holds (and each call
// advances once every block has read it), so the workspace needs no clearing
// between calls, a graph replay is a new call as well, and calls on
// different workspaces are independent.  The count is stored scrambled, so
// that whatever a fresh or reused workspace holds decodes to an arbitrary
// count, whose flag value the memory does not hold.  Slots and flags are
// written with agent-scope atomic stores (coherent across the XCDs' L2
// caches), the flag after the slot stores have completed; flags and then
// slots are read with agent-scope atomic loads.  The wait is bounded: a
// block that times out (a launch that could not be made resident, which the
// occupancy check rules out) turns its output to NaN instead of hanging.
// Measured on MI355X at the SDXL 3840 shapes, one launch takes about 16
// us (level a, 36.9 MB moved) and 12-13.5 us (level b, 18.4 MB), against
// 20.4 and 20.2 us for the three-launch form: the x loads complete about 6 us after
// the first block starts, and the hand-off (slot stores, flags, slot loads)
// adds a chain of dependent memory round trips of about 1-2.5 us each.
constexpr int kFusedMaxBlocks = 192;  // 128-256 measured: 192 is 2-4% ahead at the SDXL shapes
constexpr int kFusedThreads = 512;
constexpr int kFusedMaxKV = 16;
constexpr int kSpinLimit = 1 << 20;  // polls of ~100 cycles: ~50 ms

struct FusedPlan {
    bool ok;
    int vpp, rows, threads, kv;
    int64_t chunks;  // per image
};

FusedPlan plan_fused(const Geom& g, int64_t C, int elem_bytes) {
    FusedPlan p{};
    p.vpp = int(C / (16 / elem_bytes));
    p.rows = kFusedThreads / p.vpp > 0 ? kFusedThreads / p.vpp : 1;
    p.threads = p.vpp * p.rows;
    const int64_t P = g.h() * g.W;
    const int64_t B = g.B > 0 ? g.B : 1;
    const int64_t per_image = kFusedMaxBlocks / B;
    if (per_image < 1 || P < 1) return p;
    const int64_t kv = ceil_div(ceil_div(P, p.rows), per_image);
    if (kv > kFusedMaxKV) return p;
    p.kv = int(kv);
    p.chunks = ceil_div(P, int64_t(p.rows) * p.kv);
    p.ok = B * p.chunks <= kFusedMaxBlocks;
    return p;
}

// workspace: [call count (256 bytes)][flags (kFusedMaxBlocks u64)][slots]
size_t fused_flag_bytes() { return 256 + align256(size_t(kFusedMaxBlocks) * sizeof(uint64_t)); }

size_t fused_workspace_bytes(const Geom& g, const FusedPlan& p, int64_t G) {
    return fused_flag_bytes() + size_t(g.B * p.chunks * G * 2) * sizeof(float);
}

struct GnFusedArgs {
    const void* x;
    void* y;
    int64_t P;       // pixels per image in the slice
    int C, vpp, rows, G, kv, nblocks;
    int64_t chunks;  // per image
    int64_t n, patch;
    double inv_count;  // 1 / values per (image, group) in the slice
    double inv_n;      // 1 / patches
    float eps;
    const float* stale_moments;
    const float* gamma;
    const float* beta;
    float* fresh_moments;
    int64_t fm_stride;
    uint64_t* epoch;   // the workspace's call count, scrambled
    uint64_t* flags;   // [B * chunks]
    float* partial;    // [B][chunks][G][2]
};

constexpr uint64_t kEpochKey = 0x6A09E667F3BCC909ull;
// buffer resources: raw (stride 0) byte ranges; the resource's fourth word
// for gfx9-family targets, and the cache-policy bit of a nontemporal access
constexpr int kBufferFlags = 0x00020000;
constexpr int kNontemporal = 2;
constexpr uint32_t kPastEnd = 0xFFFFFFF0u;  // an offset past every resource's end
// zeros standing in for a missing gamma / beta (never written: static
// device storage starts zeroed)
__device__ float gn_zeros[4096];
// a call's flag value: its count scrambled by an odd multiplier (a bijection)
__device__ __forceinline__ uint64_t call_token(uint64_t epoch) {
    return ((epoch + 1) * 0x9E3779B97F4A7C15ull) ^ 0xD1B54A32D192ED03ull;
}

template <class T, int KVMAX, int MODE>
__global__ __launch_bounds__(kFusedThreads) void gn_fused(GnFusedArgs a) {
    // [2][rows][C] fp32 per-channel sums, then [2G][S] group partials
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ double stat[2 * 256];  // (mu, rstd) of each group
    __shared__ int timed_out;
    const int64_t b = blockIdx.x / a.chunks, chunk = blockIdx.x % a.chunks;
    const int tid = threadIdx.x, lane = tid & 63, nthr = blockDim.x;
    const int C = a.C, rows = a.rows, G = a.G, vpp = a.vpp;
    const int col = tid % vpp, row = tid / vpp;
    constexpr int VEC = T::VEC;

    // 1. the chunk: pixels p0 + k * rows, k < kv, all loads issued together,
    // through buffer resources spanning image b's slice: a pixel past the
    // slice (the last chunk's tail) or a k >= kv gets an offset past the
    // resource's end, which loads zeros (and stores nothing) without a
    // branch or a memory access.  Byte offsets are 32-bit: an image's slice
    // holds at most kFusedMaxBlocks * kFusedThreads * kFusedMaxKV vectors.
    const int P = int(a.P);
    const int p0 = int(chunk) * rows * a.kv + row;
    const int img_bytes = P * vpp * 16;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(reinterpret_cast<const u32x4*>(a.x) + b * a.P * vpp), 0, img_bytes,
        kBufferFlags);
    uint32_t off[KVMAX];
#pragma unroll
    for (int k = 0; k < KVMAX; ++k)
        off[k] = k < a.kv ? uint32_t(((p0 + k * rows) * vpp + col) * 16) : kPastEnd;
    u32x4 v[KVMAX];
#pragma unroll
    for (int k = 0; k < KVMAX; ++k) v[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off[k], 0, 0);
    // the call count, loaded behind the chunk by wave 0 alone (the only wave
    // that uses it).  Every block reads the count before raising its flag,
    // and the count advances only after every flag is up.  It was last
    // written by an earlier kernel, so a plain load sees it, and the blocks
    // of an XCD share one L2 fetch of it.
    uint64_t epoch = 0;
    if (tid < 64) epoch = *a.epoch ^ kEpochKey;
    __builtin_amdgcn_sched_barrier(0);

    float s[VEC], ss[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) s[j] = ss[j] = 0.f;
#pragma unroll
    for (int k = 0; k < KVMAX; ++k) {
        if (k < a.kv) {
            float f[VEC];
            T::unpack(v[k], f);  // zeros past the slice
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                s[j] += f[j];
                ss[j] = fmaf(f[j], f[j], ss[j]);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
        *reinterpret_cast<f32x4*>(&lds[row * C + col * VEC + 4 * q]) =
            f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
        *reinterpret_cast<f32x4*>(&lds[rows * C + row * C + col * VEC + 4 * q]) =
            f32x4{ss[4 * q], ss[4 * q + 1], ss[4 * q + 2], ss[4 * q + 3]};
    }
    if (tid == 0) timed_out = 0;
    __syncthreads();
    // group partials in one pass: task (pair, part) adds the rows x
    // channel-subset of its group (part-th run of cpt channels), S parts per
    // pair; wave 0 then adds the S parts in order
    const int cg = C / G, pairs = 2 * G;
    const int S = nthr / pairs > 0 ? nthr / pairs : 1;
    const int cpt = (cg + S - 1) / S;
    float* part = lds + 2 * rows * C;
    for (int t = tid; t < pairs * S; t += nthr) {
        const int pr = t / S, pt = t % S, g = pr >> 1, which = pr & 1;
        const int c0 = g * cg + pt * cpt, c1 = min(c0 + cpt, (g + 1) * cg);
        const float* base = lds + which * rows * C;
        float acc = 0.f;
        for (int r = 0; r < rows; ++r)
            for (int c = c0; c < c1; ++c) acc += base[r * C + c];
        part[t] = acc;
    }
    __syncthreads();
    // The block's slot, then its flag, both written by wave 0 with
    // agent-scope atomic stores, which are coherent across the XCDs' L2
    // caches by themselves (they complete at the memory side).  The flag
    // store is ordered after the slot stores by waiting for the wave's
    // stores to complete (the compiler fences keep the compiler from moving
    // the stores across the wait).  A release store would also write back
    // this XCD's whole L2, which only non-atomic data needs: there is none
    // to publish.
    const uint64_t token = call_token(epoch);
    if (tid < 64) {
        uint32_t* slot = reinterpret_cast<uint32_t*>(a.partial) + (b * a.chunks + chunk) * pairs;
        for (int pr = lane; pr < pairs; pr += 64) {
            float acc = 0.f;
            for (int pt = 0; pt < S; ++pt) acc += part[pr * S + pt];
            __hip_atomic_store(slot + pr, __float_as_uint(acc), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0)
            __hip_atomic_store(a.flags + blockIdx.x, token, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    const bool waits = MODE != kGnMomentsOnly || chunk == 0;
    if (!waits) return;  // moments only: one block per image finishes the job

    // what only the last phase needs, loaded while the flags come up: gamma /
    // beta of this thread's VEC channels and the other patches' stale
    // moments of group tid (the first 8 patches)
    // (a missing gamma / beta reads zeros, and gamma gets 1 added: the loads
    // stay unconditional, so no branch makes the wave wait for them here)
    const f32x4* gsrc = reinterpret_cast<const f32x4*>((a.gamma ? a.gamma : gn_zeros) + col * VEC);
    const f32x4* bsrc = reinterpret_cast<const f32x4*>((a.beta ? a.beta : gn_zeros) + col * VEC);
    const float gplus = a.gamma ? 0.f : 1.f;
    f32x4 gam[VEC / 4], bet[VEC / 4];
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
        gam[q] = gsrc[q];
        bet[q] = bsrc[q];
    }
    // lanes per group in the last phase: L consecutive lanes of one wave
    // reduce a group (L a power of two, L * G at most the block's threads)
    int L = 1;
    while (L < 64 && 2 * L * G <= nthr) L *= 2;
    const int my_g = tid / L < G ? tid / L : G - 1;
    const uint64_t* tab =
        reinterpret_cast<const uint64_t*>(a.stale_moments) + b * a.n * G + my_g;
    uint64_t st[8];
    if (MODE != kGnMomentsOnly) {
#pragma unroll
        for (int u = 0; u < 8; ++u) st[u] = tab[(u < a.n ? u : a.n - 1) * G];
    }

    // 2. wait for the flags of image b's blocks (block 0 waits for every
    // block of the launch, since it then advances the call count); wave 0
    // polls, 64 flags per pass
    if (tid < 64) {
        const int f0 = blockIdx.x == 0 ? 0 : int(b * a.chunks);
        const int f1 = blockIdx.x == 0 ? a.nblocks : int((b + 1) * a.chunks);
        int spins = 0;
        for (;;) {
            int ok = 1;
            for (int k = f0 + lane; k < f1; k += 64)
                ok &= __hip_atomic_load(a.flags + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      token;
            if (__all(ok)) break;
            if (++spins > kSpinLimit) {
                if (lane == 0) timed_out = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        // no acquire fence: the slots are read below with agent-scope atomic
        // loads, coherent by themselves, issued only after the polling loop
        // has ended (an acquire would invalidate this XCD's whole L2, which
        // only later non-atomic loads of published data need: there are none)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // every block has read the count: advance it for the next call
        if (blockIdx.x == 0 && lane == 0)
            __hip_atomic_store(a.epoch, (epoch + 1) ^ kEpochKey, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();

    // 3. statistics of image b from all its slots, in one fixed order (the
    // same in every block): lane r of group g's L lanes adds, in fp64, the
    // slots r, r + L, r + 2L, ... (its loads issued together); an xor
    // butterfly over the L lanes then leaves the identical total in each
    // (fp addition is commutative, so partner lanes form the same sums).
    const uint64_t* slots = reinterpret_cast<const uint64_t*>(a.partial) + b * a.chunks * G;
    const int r = tid % L;
    const bool owner = tid < L * G;
    double a1 = 0.0, a2 = 0.0;
    if (owner) {
        for (int64_t k0 = r; k0 < a.chunks; k0 += 16 * int64_t(L)) {
            uint64_t w[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int64_t k = k0 + int64_t(u) * L;
                w[u] = k < a.chunks ? __hip_atomic_load(slots + k * G + my_g, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                a1 += double(__uint_as_float(uint32_t(w[u])));
                a2 += double(__uint_as_float(uint32_t(w[u] >> 32)));
            }
        }
    }
    for (int m = 1; m < L; m <<= 1) {
        a1 += __shfl_xor(a1, m);
        a2 += __shfl_xor(a2, m);
    }
    if (owner && r == 0) {
        const int g = my_g;
        double st1 = 0.0, st2 = 0.0;
        for (int64_t j0 = 0; j0 < (MODE == kGnMomentsOnly ? 0 : a.n); j0 += 8) {
            if (j0 > 0) {
#pragma unroll
                for (int u = 0; u < 8; ++u) st[u] = tab[(j0 + u < a.n ? j0 + u : a.n - 1) * G];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const bool in = j0 + u < a.n && j0 + u != a.patch;
                st1 += in ? double(__uint_as_float(uint32_t(st[u]))) : 0.0;
                st2 += in ? double(__uint_as_float(uint32_t(st[u] >> 32))) : 0.0;
            }
        }
        const double m1 = a1 * a.inv_count, m2 = a2 * a.inv_count;
        if (chunk == 0) {
            a.fresh_moments[b * a.fm_stride + g * 2 + 0] = float(m1);
            a.fresh_moments[b * a.fm_stride + g * 2 + 1] = float(m2);
        }
        if (MODE != kGnMomentsOnly) {
            const double e1 = (m1 + st1) * a.inv_n;
            const double e2 = (m2 + st2) * a.inv_n;
            double var = e2 - e1 * e1;
            if (var < 0.0) var = 0.0;
            stat[2 * g] = e1;
            stat[2 * g + 1] = timed_out ? __builtin_nan("") : 1.0 / sqrt(var + double(a.eps));
        }
    }
    if (MODE == kGnMomentsOnly) return;
    __syncthreads();

    // normalise the chunk held in registers: y = x a_c + b_c
    float af[VEC], bf[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        const int g = (col * VEC + j) / cg;
        const double aa = stat[2 * g + 1] * double(gam[j / 4][j % 4] + gplus);
        af[j] = float(aa);
        bf[j] = float(double(bet[j / 4][j % 4]) - stat[2 * g] * aa);
    }
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<u32x4*>(a.y) + b * a.P * vpp, 0, img_bytes, kBufferFlags);
#pragma unroll
    for (int k = 0; k < KVMAX; ++k) {
        if (k < a.kv) {
            // the packed chunk is what stays live across the hand-off: an
            // opaque touch keeps the compiler from holding the unpacked fp32
            // values of the first pass (twice the registers) instead
            asm volatile("" : "+v"(v[k]));
            float f[VEC];
            T::unpack(v[k], f);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                f[j] = fmaf(f[j], af[j], bf[j]);
                if (MODE == kGnNormalizeSilu) f[j] = f[j] / (1.f + __expf(-f[j]));
            }
            // past the slice: dropped (nontemporal: y is not read again here)
            __builtin_amdgcn_raw_buffer_store_b128(T::pack(f), ry, off[k], 0, kNontemporal);
        }
    }
}

// Launches the single-launch form if the device holds the whole grid at
// once (blocks per CU at the kernel's largest LDS use x compute units);
// `launched` says whether it did.
template <class T, int KVMAX, int MODE>
hipError_t launch_fused(const FusedPlan& p, const GnFusedArgs& a, hipStream_t s, bool& launched) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> resident[kMaxDevices];  // blocks per CU, 0 = not asked yet
    launched = false;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipSuccess;
    const size_t lds_max = (size_t(2) * kFusedThreads * 8 + kFusedThreads) * sizeof(float);
    int per_cu = resident[dev].load();
    if (per_cu == 0) {
        int nb = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, gn_fused<T, KVMAX, MODE>,
                                                          kFusedThreads, lds_max);
        if (e != hipSuccess) return e;
        per_cu = nb > 0 ? nb : -1;
        resident[dev].store(per_cu);
    }
    const int cus = device_cus();
    if (per_cu < 0 || cus <= 0 || int64_t(per_cu) * cus < a.nblocks) return hipSuccess;
    const size_t lds = (size_t(2) * a.rows * a.C + kFusedThreads) * sizeof(float);
    hipLaunchKernelGGL((gn_fused<T, KVMAX, MODE>), dim3(unsigned(a.nblocks)), dim3(p.threads), lds,
                       s, a);
    launched = true;
    return hipGetLastError();
}

template <class T, int MODE>
hipError_t launch_fused_mode(const FusedPlan& p, const GnFusedArgs& a, hipStream_t s,
                             bool& launched) {
    if (p.kv <= 4) return launch_fused<T, 4, MODE>(p, a, s, launched);
    if (p.kv <= 8) return launch_fused<T, 8, MODE>(p, a, s, launched);
    return launch_fused<T, kFusedMaxKV, MODE>(p, a, s, launched);
}

template <class T>
hipError_t run_fused(const Geom& g, const FusedPlan& p, int64_t C, int64_t G, float eps, int mode,
                     const void* x, const float* stale_moments, const float* gamma,
                     const float* beta, void* y, float* fresh_moments, int64_t fm_stride, void* ws,
                     hipStream_t s, bool& launched) {
    GnFusedArgs a;
    a.x = x;
    a.y = y;
    a.P = g.h() * g.W;
    a.C = int(C);
    a.vpp = p.vpp;
    a.rows = p.rows;
    a.G = int(G);
    a.kv = p.kv;
    a.chunks = p.chunks;
    a.nblocks = int(g.B * p.chunks);
    a.n = g.n;
    a.patch = g.i;
    a.inv_count = 1.0 / (double(a.P) * double(C / G));
    a.inv_n = 1.0 / double(g.n);
    a.eps = eps;
    a.stale_moments = stale_moments;
    a.gamma = gamma;
    a.beta = beta;
    a.fresh_moments = fresh_moments;
    a.fm_stride = fm_stride;
    char* base = static_cast<char*>(ws);
    a.epoch = reinterpret_cast<uint64_t*>(base);
    a.flags = reinterpret_cast<uint64_t*>(base + 256);
    a.partial = reinterpret_cast<float*>(base + fused_flag_bytes());
    switch (mode) {
        case kGnNormalize: return launch_fused_mode<T, kGnNormalize>(p, a, s, launched);
        case kGnNormalizeSilu: return launch_fused_mode<T, kGnNormalizeSilu>(p, a, s, launched);
        default: return launch_fused_mode<T, kGnMomentsOnly>(p, a, s, launched);
    }
}

template <class T, int KV>
hipError_t run_kv(const GnPlan& p, const GnArgs& a, int64_t B, int mode, hipStream_t s) {
    dim3 grid(unsigned(p.chunks), unsigned(B));
    const size_t lds = size_t(2) * p.rows * a.C * sizeof(float);
    hipLaunchKernelGGL((gn_moments<T, KV>), grid, dim3(p.threads), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int slices = kFinThreads / a.G;
    const size_t lds_fin = (size_t(slices) * 2 * a.G + 2 * a.G) * sizeof(double);
    if (mode == kGnMomentsOnly) {
        hipLaunchKernelGGL(gn_finalize<true>, dim3(unsigned(B)), dim3(kFinThreads), lds_fin, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(gn_finalize<false>, dim3(unsigned(B)), dim3(kFinThreads), lds_fin, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mode == kGnNormalizeSilu)
        hipLaunchKernelGGL((gn_normalize<T, KV, true>), grid, dim3(p.threads), 0, s, a);
    else
        hipLaunchKernelGGL((gn_normalize<T, KV, false>), grid, dim3(p.threads), 0, s, a);
    return hipGetLastError();
}

template <class T>
hipError_t run(const Geom& g, int64_t C, int64_t G, float eps, int mode, const void* x,
               const float* stale_moments, const float* gamma, const float* beta, void* y,
               float* fresh_moments, int64_t fm_stride, void* ws, hipStream_t s) {
    const FusedPlan fp = plan_fused(g, C, int(sizeof(typename T::elem)));
    if (fp.ok) {
        bool launched = false;
        const hipError_t e = run_fused<T>(g, fp, C, G, eps, mode, x, stale_moments, gamma, beta, y,
                                          fresh_moments, fm_stride, ws, s, launched);
        if (e != hipSuccess || launched) return e;
    }
    const GnPlan p = plan_gn(g, C, int(sizeof(typename T::elem)));
    GnArgs a;
    a.x = x;
    a.y = y;
    a.P = g.h() * g.W;
    a.C = int(C);
    a.vpp = p.vpp;
    a.rows = p.rows;
    a.G = int(G);
    a.chunks = p.chunks;
    a.n = g.n;
    a.patch = g.i;
    a.count = double(a.P) * double(C / G);
    a.eps = eps;
    a.stale_moments = stale_moments;
    a.gamma = gamma;
    a.beta = beta;
    a.fresh_moments = fresh_moments;
    a.fm_stride = fm_stride;
    a.ws = carve(ws, g, p, C, G);
    switch (p.kv) {
        case 1: return run_kv<T, 1>(p, a, g.B, mode, s);
        case 2: return run_kv<T, 2>(p, a, g.B, mode, s);
        case 4: return run_kv<T, 4>(p, a, g.B, mode, s);
        case 8: return run_kv<T, 8>(p, a, g.B, mode, s);
        default: return run_kv<T, kMaxKV>(p, a, g.B, mode, s);
    }
}

}  // namespace

size_t groupnorm_workspace_bytes(const Geom& g, int64_t C, int64_t G, int elem_bytes) {
    const size_t three = workspace_bytes(g, plan_gn(g, C, elem_bytes), C, G);
    const FusedPlan fp = plan_fused(g, C, elem_bytes);
    return fp.ok ? std::max(three, fused_workspace_bytes(g, fp, G)) : three;
}

hipError_t groupnorm_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // once per device, with that device current: each device holds its
        // own copy of the array at its own address
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_groupnorm(const Geom& g, int64_t C, int64_t G, float eps, bool bf16, int mode,
                            const void* x, const float* stale_moments, const float* gamma,
                            const float* beta, void* y, float* fresh_moments, int64_t fm_stride,
                            void* ws, hipStream_t s) {
    if (bf16)
        return run<Bf16T>(g, C, G, eps, mode, x, stale_moments, gamma, beta, y, fresh_moments,
                          fm_stride, ws, s);
    return run<F32T>(g, C, G, eps, mode, x, stale_moments, gamma, beta, y, fresh_moments,
                     fm_stride, ws, s);
}

}  // namespace dp
