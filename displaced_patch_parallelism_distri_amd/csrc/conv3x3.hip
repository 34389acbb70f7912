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
// K = 9*Cin ordered (kh, kw, ci).  A block computes a BM x 160 (pixel x
// cout) tile with 4 waves in a 2 x 2 grid of (BM/2) x 80 wave tiles made of
// v_mfma_f32_16x16x32_bf16 tiles.  Cout = 640 and 1280 are 4 and 8 tiles
// of 160; BM (128 or 64) is picked per shape so that the grid gives about
// two blocks per CU (two blocks are resident per CU).
//  * K advances 64 channels of one tap per step.  The A rows are gathered
//    per pixel from the fresh slice, the stale halo row or zero (NHWC keeps a
//    pixel's channels contiguous, so a row is 8 x 16-byte vectors); the halo
//    is never materialised.  A thread's source pixels are decoded once; the
//    three row sources are re-selected only when the tap changes.
//  * The weight tile comes from [Cout][3][3][Cin], already K-contiguous per
//    output channel.
//  * Both tiles go from global memory straight into LDS
//    (global_load_lds_dwordx4: no registers, no LDS store instructions),
//    double-buffered: the loads of step s+1 are in flight while step s
//    computes; one wait and one barrier per step.  LDS rows are 128 bytes
//    with the 16-byte chunks XOR-swizzled by (row / 2) % 8, which keeps the
//    ds_read_b128 operand reads free of bank conflicts without padding
//    (2 x 72 KB fit per CU); a load's LDS slot is fixed by its lane, so each
//    thread reads the logical chunk that the swizzle puts in its slot.
//  * Blocks are remapped so that each XCD takes every cout slice of one
//    contiguous range of pixel tiles: a pixel row is fetched into the XCD's
//    L2 once for all slices and stays there for the neighbouring taps, and
//    a step's weights (all slices, 64 channels) are shared by the XCD's
//    blocks.  (Measured on MI355X against slice-major order: same time at
//    Cout 640 / BM 128, 4% faster at Cout 1280 / BM 64.)
// fp32 kernel: one thread per output element, direct sum; parity-grade.
#include "dp_common.h"

namespace dp {
namespace {

constexpr int BN = 160, BK = 64;
constexpr int WN = 80, NT = WN / 16;  // wave tile columns, 16-wide MFMA tiles
constexpr int B_CHUNKS = BN * 8 / 256;  // 16-byte chunks per thread per step

// The zero padding's source: an A row of a padded tap (outside the image, or
// a halo row at the image edge) reads its channels [0, Cin) from here, so the
// loaded values go to LDS without a select.  Never written; Cin <= 65536.
__device__ __attribute__((aligned(16))) uint16_t conv_zeros[65536];

struct ConvArgs {
    const uint16_t* xf;
    const uint16_t* xs;
    const uint16_t* w;
    const float* bias;
    uint16_t* y;
    int M;  // B*h*W
    int h, W, H;
    int n, i;
    int cin, cout;
    int mtiles, ntiles;
};

constexpr int kVmcnt0 = vmcnt_imm(0);

// 16-byte chunk position of chunk `c` of LDS row `r`
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int BM>
__global__ __launch_bounds__(256, 2) void conv_bf16_kernel(ConvArgs a) {
    constexpr int WM = BM / 2, MT = WM / 16;
    constexpr int A_CHUNKS = BM * 8 / 256;
    // the two tile buffers, and after the K loop the bf16 output tile
    // [BM][OUT_PITCH] staged for 16-byte stores
    constexpr int OUT_PITCH = BN + 8;  // 336-byte rows: 4 rows apart land on other banks
    static_assert(BM * OUT_PITCH <= 2 * (BM + BN) * BK, "output tile fits the tile buffers");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * BK];
    uint16_t (*a_lds)[BM * BK] = reinterpret_cast<uint16_t (*)[BM * BK]>(smem);
    uint16_t (*b_lds)[BN * BK] = reinterpret_cast<uint16_t (*)[BN * BK]>(smem + 2 * BM * BK);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware tile order: logical tiles run pixel-tile-major with the cout
    // slices inner; the blocks of one XCD (physical id % 8) take a
    // contiguous logical range
    const int ntot = a.mtiles * a.ntiles;
    const int n8 = ntot - ntot % 8;
    const int pw = blockIdx.x;
    const int logical = pw < n8 ? (pw % 8) * (n8 / 8) + pw / 8 : pw;
    const int mt = logical / a.ntiles, nt = logical % a.ntiles;
    const int m0 = mt * BM, n0 = nt * BN;

    // ---- A loader: chunk c = tid + 256 j -> row c / 8, 16-byte chunk c % 8
    int ab[A_CHUNKS], ar[A_CHUNKS], acol[A_CHUNKS];
    bool avalid[A_CHUNKS];
    const int akc = tid & 7;
    const int hw = a.h * a.W;
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) {
        const int row = (tid >> 3) + 32 * j;
        const int m = m0 + row;
        avalid[j] = m < a.M;
        const int mm = avalid[j] ? m : 0;
        ab[j] = mm / hw;
        const int rem = mm - ab[j] * hw;
        ar[j] = rem / a.W;
        acol[j] = rem - ar[j] * a.W;
    }
    const uint16_t* aptr[A_CHUNKS];  // pixel base of the current tap (or the zeros)
    auto set_tap = [&](int tap) {
        const int kh = tap / 3, kw = tap - kh * 3;
#pragma unroll
        for (int j = 0; j < A_CHUNKS; ++j) {
            const int rr = ar[j] + kh - 1, cc = acol[j] + kw - 1;
            bool ok = avalid[j] && cc >= 0 && cc < a.W;
            const uint16_t* p = a.xf;
            if (rr >= 0 && rr < a.h) {
                p = a.xf + ((size_t(ab[j]) * a.h + rr) * a.W + cc) * a.cin;
            } else if (rr < 0) {
                ok = ok && a.i > 0;
                p = a.xs + ((size_t(ab[j]) * a.H + size_t(a.i) * a.h - 1) * a.W + cc) * a.cin;
            } else {
                ok = ok && a.i < a.n - 1;
                p = a.xs + ((size_t(ab[j]) * a.H + size_t(a.i + 1) * a.h) * a.W + cc) * a.cin;
            }
            aptr[j] = ok ? p : conv_zeros;
        }
    };

    // ---- B loader: chunk c = tid + 256 j -> weight row c / 8, chunk c % 8
    const uint16_t* bptr[B_CHUNKS];
    bool bok[B_CHUNKS];
#pragma unroll
    for (int j = 0; j < B_CHUNKS; ++j) {
        const int row = (tid >> 3) + 32 * j;
        bok[j] = n0 + row < a.cout;
        bptr[j] = a.w + size_t(bok[j] ? n0 + row : 0) * 9 * a.cin + akc * 8;
    }

    const int kchunks = a.cin / BK;
    const int nsteps = 9 * kchunks;
    // Tile loads straight into LDS: instruction j of wave w writes LDS
    // granules j*256 + w*64 + lane, i.e. row (tid >> 3) + 32 j at physical
    // chunk tid & 7, so the thread reads the logical chunk stored there.
    // Padding rows read zeros and weight rows past Cout read row 0 (they
    // feed only output columns that are never stored).  Their completion is
    // the explicit wait at the top of each step (global_load_lds16).
    int alc[A_CHUNKS], blc[B_CHUNKS];
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) alc[j] = swz((tid >> 3) + 32 * j, akc) * 8;
#pragma unroll
    for (int j = 0; j < B_CHUNKS; ++j) blc[j] = swz((tid >> 3) + 32 * j, akc) * 8 - akc * 8;
    const uint32_t wslot = uint32_t(wave) * 64 * 16;
    auto tile_load = [&](int s, int buf) {
        const int tap = s / kchunks;
        const int ci0 = (s - tap * kchunks) * BK;
        if (ci0 == 0) set_tap(tap);
        const uint32_t al = lds_addr(&a_lds[buf][0]) + wslot;
        const uint32_t bl = lds_addr(&b_lds[buf][0]) + wslot;
#pragma unroll
        for (int j = 0; j < A_CHUNKS; ++j) global_load_lds16(aptr[j] + ci0 + alc[j], al + j * 256 * 16);
#pragma unroll
        for (int j = 0; j < B_CHUNKS; ++j)
            global_load_lds16(bptr[j] + tap * a.cin + ci0 + blc[j], bl + j * 256 * 16);
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Both k32 halves' operand fragments are read first, so the second
    // half's LDS reads are in flight while the first half's MFMAs run.
    auto compute = [&](int cur) {
        bf16x8 af[BK / 32][MT], bf[BK / 32][NT];
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int row = wm * WM + i * 16 + l16;
                af[kk][i] = *reinterpret_cast<const bf16x8*>(&a_lds[cur][row * BK + swz(row, kk * 4 + lq) * 8]);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int row = wn * WN + j * 16 + l16;
                bf[kk][j] = *reinterpret_cast<const bf16x8*>(&b_lds[cur][row * BK + swz(row, kk * 4 + lq) * 8]);
            }
        }
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk][i], bf[kk][j], acc[i][j], 0, 0, 0);
    };
    // step s: its loads are done, then the barrier (every wave's share is
    // in LDS and every wave has left step s - 1, whose buffer the loads of
    // step s + 1 then take), then compute.  Nothing of the compiler's own
    // is in flight when the first load is issued.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    tile_load(0, 0);
    for (int s = 0; s < nsteps; ++s) {
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
        if (s + 1 < nsteps) tile_load(s + 1, (s + 1) & 1);
        compute(s & 1);
    }

    // epilogue: acc[i][j][e] is pixel m0 + wm*WM + i*16 + 4*lq + e,
    // cout n0 + wn*80 + j*16 + l16.  With Cout a multiple of 8 the tile is
    // staged in LDS as bf16 and written out in 16-byte pieces of a pixel's
    // channel run (whole 64-byte segments instead of 2-byte scatters);
    // otherwise each element is stored on its own.
    const bool vec_out = (a.cout % 8) == 0 && (reinterpret_cast<uintptr_t>(a.y) % 16) == 0;
    if (vec_out) {
        __syncthreads();  // every wave is past its last tile read
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int c = wn * WN + j * 16 + l16;
            const int n = n0 + c;
            const float bias = (a.bias && n < a.cout) ? a.bias[n] : 0.f;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = wm * WM + i * 16 + 4 * lq + e;
                    smem[r * OUT_PITCH + c] = f32_to_bf16(acc[i][j][e] + bias);
                }
        }
        __syncthreads();
        constexpr int CHUNKS = BN / 8;  // 16-byte pieces per tile row
        const int ncol = a.cout - n0 < BN ? (a.cout - n0) / 8 : CHUNKS;
        for (int t = tid; t < BM * CHUNKS; t += 256) {
            const int r = t / CHUNKS, ch = t - r * CHUNKS;
            const int m = m0 + r;
            if (m < a.M && ch < ncol)
                *reinterpret_cast<u32x4*>(a.y + size_t(m) * a.cout + n0 + ch * 8) =
                    *reinterpret_cast<const u32x4*>(&smem[r * OUT_PITCH + ch * 8]);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = n0 + wn * WN + j * 16 + l16;
        if (n >= a.cout) continue;
        const float bias = a.bias ? a.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * WM + i * 16 + 4 * lq + e;
                if (m < a.M) a.y[size_t(m) * a.cout + n] = f32_to_bf16(acc[i][j][e] + bias);
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
        a.M = int(M);
        a.h = int(g.h());
        a.W = int(g.W);
        a.H = int(g.H);
        a.n = int(g.n);
        a.i = int(g.i);
        a.cin = int(cin);
        a.cout = int(cout);
        a.ntiles = int(ceil_div(cout, BN));
        // two blocks are resident per CU: take the 128-row tile only when
        // it still gives at least ~1.6 blocks per CU
        const int64_t t128 = ceil_div(M, 128) * a.ntiles;
        const bool big = t128 * 10 >= int64_t(device_cus()) * 16;
        a.mtiles = int(ceil_div(M, big ? 128 : 64));
        const unsigned grid = unsigned(a.mtiles) * unsigned(a.ntiles);
        if (big)
            hipLaunchKernelGGL(conv_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(conv_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
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

