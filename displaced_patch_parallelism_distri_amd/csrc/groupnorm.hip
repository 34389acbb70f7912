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
//                     (row, col) owns one 16-byte channel vector of every
//                     R-th pixel of its chunk, so a row of threads reads whole
//                     pixels contiguously.  Per-channel fp32 partials are
//                     folded into per-group partials in LDS and written to
//                     the workspace [B][chunks][G][2].
//   2. gn_finalize  - per (group, image): fp64 sum of the chunk partials in a
//                     fixed order, the fresh/stale mix, the clamp, and the
//                     per-channel affine (a_c = rstd gamma_c,
//                     b_c = beta_c - mu a_c) written to the workspace.
//   3. gn_normalize - second coalesced pass: y = x a_c + b_c, rounded (RNE).
// Deterministic: no atomics; every sum has a fixed order.
#include "dp_common.h"

namespace dp {
namespace {

constexpr int kTargetBlocks = 512;
constexpr int kUnroll = 4;

struct GnPlan {
    int vpp;        // 16-byte vectors per pixel
    int rows;       // pixel rows per block iteration
    int threads;    // vpp * rows
    int64_t ppc;    // pixels per chunk
    int64_t chunks; // chunks per image
};

GnPlan plan_gn(const Geom& g, int64_t C, int elem_bytes) {
    GnPlan p;
    const int vec = 16 / elem_bytes;
    p.vpp = int(C / vec);
    int gcd = 64, a = p.vpp;
    while (a != 0) {
        int t = gcd % a;
        gcd = a;
        a = t;
    }
    p.rows = 64 / gcd;
    while (p.vpp * p.rows < 256) p.rows *= 2;
    if (p.vpp * p.rows > 1024) p.rows = 1024 / p.vpp > 0 ? 1024 / p.vpp : 1;
    p.threads = p.vpp * p.rows;
    const int64_t P = g.h() * g.W;
    int64_t per_image = kTargetBlocks / (g.B > 0 ? g.B : 1);
    if (per_image < 1) per_image = 1;
    int64_t ppc = ceil_div(P, per_image);
    ppc = ceil_div(ppc, p.rows) * p.rows;
    if (ppc < 4 * p.rows) ppc = 4 * p.rows;
    p.ppc = ppc;
    p.chunks = ceil_div(P, ppc);
    return p;
}

template <class T>
__global__ __launch_bounds__(1024) void gn_moments(const typename T::elem* __restrict__ x,
                                                   int64_t P, int C, int vpp, int rows, int G,
                                                   int64_t ppc, int64_t chunks,
                                                   float* __restrict__ partial) {
    extern __shared__ float lds[];  // [2][rows][C], then [2][C] channel totals
    const int64_t b = blockIdx.y, chunk = blockIdx.x;
    const int tid = threadIdx.x;
    const int col = tid % vpp, row = tid / vpp;
    const int64_t p0 = chunk * ppc;
    const int64_t p1 = p0 + ppc < P ? p0 + ppc : P;
    float s[T::VEC], ss[T::VEC];
#pragma unroll
    for (int j = 0; j < T::VEC; ++j) s[j] = ss[j] = 0.f;
    const u32x4* base = reinterpret_cast<const u32x4*>(x + b * P * C) + col;
    // kUnroll independent 16-byte loads in flight per thread
    for (int64_t p = p0 + row; p < p1; p += int64_t(kUnroll) * rows) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t pu = p + int64_t(u) * rows;
            v[u] = pu < p1 ? base[pu * vpp] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float f[T::VEC];
            T::unpack(v[u], f);
#pragma unroll
            for (int j = 0; j < T::VEC; ++j) {
                s[j] += f[j];
                ss[j] = fmaf(f[j], f[j], ss[j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < T::VEC; ++j) {
        lds[row * C + col * T::VEC + j] = s[j];
        lds[rows * C + row * C + col * T::VEC + j] = ss[j];
    }
    __syncthreads();
    // channel totals over the block's rows (fixed order)
    float* tot = lds + 2 * rows * C;
    for (int t = tid; t < 2 * C; t += blockDim.x) {
        const int stat = t / C, c = t % C;
        float acc = 0.f;
        for (int r = 0; r < rows; ++r) acc += lds[stat * rows * C + r * C + c];
        tot[stat * C + c] = acc;
    }
    __syncthreads();
    const int cg = C / G;
    for (int task = tid; task < 2 * G; task += blockDim.x) {
        const int g = task >> 1, stat = task & 1;
        const float* src = tot + stat * C + g * cg;
        float acc = 0.f;
        for (int c = 0; c < cg; ++c) acc += src[c];
        partial[((b * chunks + chunk) * G + g) * 2 + stat] = acc;
    }
}

// One block per (group, image): fixed-order fp64 reduction of the chunk
// partials, the fresh/stale mix and the clamp, then the per-channel affine.
__global__ __launch_bounds__(256) void gn_finalize(const float* __restrict__ partial,
                                                   int64_t chunks, int C, int G, int64_t n,
                                                   int64_t patch, double count, float eps,
                                                   const float* __restrict__ stale_moments,
                                                   const float* __restrict__ gamma,
                                                   const float* __restrict__ beta,
                                                   float* __restrict__ fresh_moments,
                                                   float* __restrict__ affine) {
    __shared__ double red[2][256];
    __shared__ double stats[2];
    const int g = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x;
    double s1 = 0.0, s2 = 0.0;
    const float* pp = partial + (b * chunks * G + g) * 2;
    for (int64_t k = tid; k < chunks; k += 256) {
        s1 += double(pp[k * G * 2 + 0]);
        s2 += double(pp[k * G * 2 + 1]);
    }
    red[0][tid] = s1;
    red[1][tid] = s2;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) {
            red[0][tid] += red[0][tid + w];
            red[1][tid] += red[1][tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        const double m1 = red[0][0] / count, m2 = red[1][0] / count;
        fresh_moments[(b * G + g) * 2 + 0] = float(m1);
        fresh_moments[(b * G + g) * 2 + 1] = float(m2);
        double e1 = m1, e2 = m2;
        for (int64_t j = 0; j < n; ++j) {
            if (j == patch) continue;
            e1 += double(stale_moments[((b * n + j) * G + g) * 2 + 0]);
            e2 += double(stale_moments[((b * n + j) * G + g) * 2 + 1]);
        }
        e1 /= double(n);
        e2 /= double(n);
        double var = e2 - e1 * e1;
        if (var < 0.0) var = 0.0;
        stats[0] = e1;
        stats[1] = 1.0 / sqrt(var + double(eps));
    }
    __syncthreads();
    const int cg = C / G;
    const double mu = stats[0], rstd = stats[1];
    for (int c = g * cg + tid; c < (g + 1) * cg; c += 256) {
        const double ga = gamma ? double(gamma[c]) : 1.0;
        const double be = beta ? double(beta[c]) : 0.0;
        const double a = rstd * ga;
        affine[(b * C + c) * 2 + 0] = float(a);
        affine[(b * C + c) * 2 + 1] = float(be - mu * a);
    }
}

template <class T>
__global__ __launch_bounds__(1024) void gn_normalize(const typename T::elem* __restrict__ x,
                                                     typename T::elem* __restrict__ y, int64_t P,
                                                     int C, int vpp, int rows, int64_t ppc,
                                                     const float* __restrict__ affine) {
    const int64_t b = blockIdx.y, chunk = blockIdx.x;
    const int tid = threadIdx.x;
    const int col = tid % vpp, row = tid / vpp;
    float a[T::VEC], c0[T::VEC];
    const float* af = affine + (b * C + col * T::VEC) * 2;
#pragma unroll
    for (int j = 0; j < T::VEC; ++j) {
        a[j] = af[2 * j];
        c0[j] = af[2 * j + 1];
    }
    const int64_t p0 = chunk * ppc;
    const int64_t p1 = p0 + ppc < P ? p0 + ppc : P;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + b * P * C) + col;
    u32x4* dst = reinterpret_cast<u32x4*>(y + b * P * C) + col;
    for (int64_t p = p0 + row; p < p1; p += int64_t(kUnroll) * rows) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t pu = p + int64_t(u) * rows;
            if (pu < p1) v[u] = src[pu * vpp];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t pu = p + int64_t(u) * rows;
            if (pu < p1) {
                float f[T::VEC];
                T::unpack(v[u], f);
#pragma unroll
                for (int j = 0; j < T::VEC; ++j) f[j] = fmaf(f[j], a[j], c0[j]);
                dst[pu * vpp] = T::pack(f);
            }
        }
    }
}

template <class T>
hipError_t run(const Geom& g, int64_t C, int64_t G, float eps, const void* x,
               const float* stale_moments, const float* gamma, const float* beta, void* y,
               float* fresh_moments, void* ws, hipStream_t s) {
    const GnPlan p = plan_gn(g, C, int(sizeof(typename T::elem)));
    const int64_t P = g.h() * g.W;
    float* partial = static_cast<float*>(ws);
    float* affine = partial + g.B * p.chunks * G * 2;
    const size_t lds = size_t(2) * (p.rows + 1) * C * sizeof(float);
    dim3 grid(unsigned(p.chunks), unsigned(g.B));
    hipLaunchKernelGGL(gn_moments<T>, grid, dim3(p.threads), lds, s,
                       static_cast<const typename T::elem*>(x), P, int(C), p.vpp, p.rows, int(G),
                       p.ppc, p.chunks, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gn_finalize, dim3(unsigned(G), unsigned(g.B)), dim3(256), 0, s, partial, p.chunks,
                       int(C), int(G), g.n, g.i, double(P) * double(C / G), eps, stale_moments,
                       gamma, beta, fresh_moments, affine);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gn_normalize<T>, grid, dim3(p.threads), 0, s,
                       static_cast<const typename T::elem*>(x),
                       static_cast<typename T::elem*>(y), P, int(C), p.vpp, p.rows, p.ppc,
                       affine);
    return hipGetLastError();
}

}  // namespace

size_t groupnorm_workspace_bytes(const Geom& g, int64_t C, int64_t G, int elem_bytes) {
    const GnPlan p = plan_gn(g, C, elem_bytes);
    return size_t(g.B * p.chunks * G * 2 + g.B * C * 2) * sizeof(float);
}

hipError_t launch_groupnorm(const Geom& g, int64_t C, int64_t G, float eps, bool bf16,
                            const void* x, const float* stale_moments, const float* gamma,
                            const float* beta, void* y, float* fresh_moments, void* ws,
                            hipStream_t s) {
    if (bf16)
        return run<Bf16T>(g, C, G, eps, x, stale_moments, gamma, beta, y, fresh_moments, ws, s);
    return run<F32T>(g, C, G, eps, x, stale_moments, gamma, beta, y, fresh_moments, ws, s);
}

}  // namespace dp
