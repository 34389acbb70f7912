// 3x3 convolution of one row patch with a stale halo (DistriConv2dPP:
// "DistriFusion源码探秘：从DistriUNetPP到DistriAttentionTP的模块设计原理", section
// "Patch Parallelism的实现原理", item 1; the neighbouring patches' boundary rows
// are the previous step's activations, "DistriFusion：高分辨率扩散模型的分布式并
// 行推理", README mirror, section 概述, figure (c)).
//
//   y[b, r, c, o] = bias[o] + sum_{kh, kw, ci} w[o, kh, kw, ci] X^[b, i*h + r + kh - 1, c + kw - 1, ci]
//
// X^ rows inside the patch are the fresh slice; row i*h-1 (if i > 0) and row
// (i+1)*h (if i < n-1) come from the stale full map; everything outside the
// image is zero.
//
// bf16 kernel: implicit GEMM on MFMA with M = B*h*W output pixels, N = Cout,
// K = 9*Cin ordered (kh, kw, ci).  A block computes a 128 x 128 (pixel x
// cout) tile with 4 waves of 64 x 64 (2 x 2 v_mfma_f32_32x32x16_bf16 tiles).
// K advances 32 channels of one tap at a time; the A tile rows are gathered
// per pixel from the fresh slice, the stale halo row or zero, as 16-byte
// channel vectors (NHWC keeps a pixel's channels contiguous) - the halo is
// never materialised.  The weight tile comes from [Cout][3][3][Cin], which
// is already K-contiguous per output channel.  Both tiles are staged in
// double-buffered LDS.
// fp32 kernel: one thread per output element, direct sum; parity-grade.
#include "dp_common.h"

namespace dp {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int APITCH = BK + 8;  // LDS row pitch (bf16 elements): 80 bytes
constexpr int BPITCH = BK + 8;

struct ConvArgs {
    const uint16_t* xf;
    const uint16_t* xs;
    const uint16_t* w;
    const float* bias;
    uint16_t* y;
    int64_t M;  // B*h*W
    int64_t h, W, H;
    int64_t n, i;
    int cin, cout;
};

// Pointer to channel ci0 of hybrid-map pixel (b, local row rr, col cc), or
// nullptr where the padding is zero.
__device__ __forceinline__ const uint16_t* pixel_ptr(const ConvArgs& a, int64_t b, int64_t rr,
                                                     int64_t cc) {
    if (cc < 0 || cc >= a.W) return nullptr;
    if (rr >= 0 && rr < a.h) return a.xf + ((b * a.h + rr) * a.W + cc) * a.cin;
    if (rr == -1) {
        if (a.i == 0) return nullptr;
        return a.xs + ((b * a.H + a.i * a.h - 1) * a.W + cc) * a.cin;
    }
    if (a.i == a.n - 1) return nullptr;
    return a.xs + ((b * a.H + (a.i + 1) * a.h) * a.W + cc) * a.cin;
}

__global__ __launch_bounds__(256, 2) void conv_bf16_kernel(ConvArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][BM * APITCH];
    __shared__ __attribute__((aligned(16))) uint16_t b_lds[2][BN * BPITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, g = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = int64_t(blockIdx.x) * BM;
    const int n0 = int(blockIdx.y) * BN;

    // loader mapping: chunk id = tid + 256*j -> row id>>2, channel group id&3
    int64_t pb[2], pr[2], pc[2];
    bool pvalid[2];
    int lrow[2], lc4[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int id = tid + 256 * j;
        lrow[j] = id >> 2;
        lc4[j] = id & 3;
        const int64_t m = m0 + lrow[j];
        pvalid[j] = m < a.M;
        const int64_t mm = pvalid[j] ? m : 0;
        const int64_t hw = a.h * a.W;
        pb[j] = mm / hw;
        pr[j] = (mm % hw) / a.W;
        pc[j] = mm % a.W;
    }
    const int cin = a.cin;
    const int kchunks = cin / BK;
    const int nk = 9 * kchunks;

    u32x4 ar[2], br[2];
    auto gload = [&](int k) {
        const int tap = k / kchunks;
        const int ci0 = (k - tap * kchunks) * BK;
        const int kh = tap / 3, kw = tap - kh * 3;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint16_t* p =
                pvalid[j] ? pixel_ptr(a, pb[j], pr[j] + kh - 1, pc[j] + kw - 1) : nullptr;
            ar[j] = p ? *reinterpret_cast<const u32x4*>(p + ci0 + lc4[j] * 8) : u32x4{0, 0, 0, 0};
            const int n = n0 + lrow[j];
            br[j] = n < a.cout ? *reinterpret_cast<const u32x4*>(
                                     a.w + (int64_t(n) * 9 + tap) * cin + ci0 + lc4[j] * 8)
                               : u32x4{0, 0, 0, 0};
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            *reinterpret_cast<u32x4*>(&a_lds[buf][lrow[j] * APITCH + lc4[j] * 8]) = ar[j];
            *reinterpret_cast<u32x4*>(&b_lds[buf][lrow[j] * BPITCH + lc4[j] * 8]) = br[j];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    gload(0);
    lstore(0);
    __syncthreads();
    for (int k = 0; k < nk; ++k) {
        const int cur = k & 1;
        if (k + 1 < nk) gload(k + 1);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = *reinterpret_cast<const bf16x8*>(
                    &a_lds[cur][(wm * 64 + i * 32 + lr) * APITCH + ks * 16 + g * 8]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *reinterpret_cast<const bf16x8*>(
                    &b_lds[cur][(wn * 64 + j * 32 + lr) * BPITCH + ks * 16 + g * 8]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (k + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: acc[i][j][e] is pixel m0 + wm*64 + i*32 + 8*(e/4) + 4g + e%4,
    // cout n0 + wn*64 + j*32 + lr
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + lr;
        if (n >= a.cout) continue;
        const float bias = a.bias ? a.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (m < a.M) a.y[m * a.cout + n] = f32_to_bf16(acc[i][j][e] + bias);
            }
    }
}

// ----------------------------------------------------------------- fp32 path
struct ConvArgsF32 {
    const float* xf;
    const float* xs;
    const float* w;
    const float* bias;
    float* y;
    int64_t M, h, W, H, n, i;
    int cin, cout;
};

__global__ __launch_bounds__(256) void conv_f32_kernel(ConvArgsF32 a) {
    const int64_t total = a.M * a.cout;
    for (int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * 256) {
        const int64_t m = idx / a.cout;
        const int o = int(idx % a.cout);
        const int64_t hw = a.h * a.W;
        const int64_t b = m / hw, r = (m % hw) / a.W, c = m % a.W;
        float acc = a.bias ? a.bias[o] : 0.f;
        for (int kh = 0; kh < 3; ++kh) {
            const int64_t rr = r + kh - 1;
            const float* row = nullptr;
            if (rr >= 0 && rr < a.h)
                row = a.xf + (b * a.h + rr) * a.W * a.cin;
            else if (rr == -1 && a.i > 0)
                row = a.xs + (b * a.H + a.i * a.h - 1) * a.W * a.cin;
            else if (rr == a.h && a.i < a.n - 1)
                row = a.xs + (b * a.H + (a.i + 1) * a.h) * a.W * a.cin;
            if (!row) continue;
            for (int kw = 0; kw < 3; ++kw) {
                const int64_t cc = c + kw - 1;
                if (cc < 0 || cc >= a.W) continue;
                const float* xp = row + cc * a.cin;
                const float* wp = a.w + (int64_t(o) * 9 + kh * 3 + kw) * a.cin;
                for (int ci = 0; ci < a.cin; ++ci) acc = fmaf(wp[ci], xp[ci], acc);
            }
        }
        a.y[idx] = acc;
    }
}

}  // namespace

hipError_t launch_conv3x3(const Geom& g, int64_t cin, int64_t cout, bool bf16, const void* xf,
                          const void* xs, const void* w, const float* bias, void* y,
                          hipStream_t s) {
    const int64_t M = g.B * g.h() * g.W;
    if (bf16) {
        ConvArgs a;
        a.xf = static_cast<const uint16_t*>(xf);
        a.xs = static_cast<const uint16_t*>(xs);
        a.w = static_cast<const uint16_t*>(w);
        a.bias = bias;
        a.y = static_cast<uint16_t*>(y);
        a.M = M;
        a.h = g.h();
        a.W = g.W;
        a.H = g.H;
        a.n = g.n;
        a.i = g.i;
        a.cin = int(cin);
        a.cout = int(cout);
        dim3 grid(unsigned(ceil_div(M, BM)), unsigned(ceil_div(cout, BN)));
        hipLaunchKernelGGL(conv_bf16_kernel, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    ConvArgsF32 a;
    a.xf = static_cast<const float*>(xf);
    a.xs = static_cast<const float*>(xs);
    a.w = static_cast<const float*>(w);
    a.bias = bias;
    a.y = static_cast<float*>(y);
    a.M = M;
    a.h = g.h();
    a.W = g.W;
    a.H = g.H;
    a.n = g.n;
    a.i = g.i;
    a.cin = int(cin);
    a.cout = int(cout);
    int64_t blocks = ceil_div(M * cout, 256);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(conv_f32_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dp
