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
// Memory-bound; three launches:
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
// A moments-only form runs 1 and 2 and writes the patch's raw moments alone.
// Deterministic: no atomics, every sum has a fixed order.  The second read of
// x is normally served from L2 / the Infinity Cache: a chunk is read by the
// same XCD in both passes and the slice is tens of MB.
#include "dp_common.h"

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
    return workspace_bytes(g, plan_gn(g, C, elem_bytes), C, G);
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
