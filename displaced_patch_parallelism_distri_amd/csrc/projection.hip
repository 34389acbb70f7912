// Token-wise projections of the patch's attention layer (the Q/K/V and output
// projections that the wrapped self-attention holds: "DistriFusion源码探秘：
// 从DistriUNetPP到DistriAttentionTP的模块设计原理", section "Patch
// Parallelism的实现原理", item 2):
//
//   y[m, o] = bias[o] + sum_c w[o, c] x[m, c]      m < M = B*Lq, o < N
//
// The Q/K/V form stacks the three weights (N = 3C) and routes output column
// o to q, k or v (o / C).  Its epilogue also writes the k and v values into
// this patch's rows of the stale K/V maps: that is the refresh which makes
// this step's fresh K/V the next step's stale context ("DistriFusion：高分辨
// 率扩散模型的分布式并行推理", README mirror, section 概述, figure (c)), done
// here instead of by a separate copy.  Attention never reads the stale map's
// own rows, so writing them before the attention call is safe.
//
// bf16 kernel: a GEMM on v_mfma_f32_16x16x32_bf16 with the structure of the
// conv kernel - a BM x 160 block tile, 4 waves in a 2 x 2 grid of
// (BM/2) x 80 wave tiles, 64-wide K steps through swizzled double-buffered
// LDS filled by direct global -> LDS loads one step ahead - minus the halo
// gather: A rows are contiguous token rows.
// fp32 kernel: one thread per output element, direct sum; parity-grade.
#include "dp_common.h"

namespace dp {
namespace {

constexpr int BN = 160, BK = 64;
constexpr int WN = 80, NT = WN / 16;
constexpr int B_CHUNKS = BN * 8 / 256;

// Where output column o goes: part p = o / part_cols (0 .. parts-1) of width
// part_cols; dst[p] is [M][part_cols]; stale[p], if set, is [B][L][part_cols]
// and receives rows i*Lq .. i*Lq + Lq - 1 of image b for m = b*Lq + t.
struct Route {
    void* dst[3];
    void* stale[3];
    int part_cols;
    int lq;       // tokens per image in the patch
    int64_t L;    // tokens per image in the full map
    int64_t own;  // first token of the patch (i * Lq)
};

struct ProjArgs {
    const uint16_t* x;
    const uint16_t* w;
    const float* bias;
    int M, K, N;
    int mtiles, ntiles;
    Route r;
};

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

constexpr int kVmcnt0 = vmcnt_imm(0);

template <int BM>
__global__ __launch_bounds__(256, 2) void proj_bf16_kernel(ProjArgs a) {
    constexpr int WM = BM / 2, MT = WM / 16;
    constexpr int A_CHUNKS = BM * 8 / 256;
    // one LDS block: the A and B double buffers during the K loop, the
    // output tile (row stride CS) in the epilogue
    constexpr int CS = BN + 8;
    static_assert(BM * CS <= 2 * (BM + BN) * BK, "output tile must fit the LDS buffers");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * BK];
    uint16_t (*a_lds)[BM * BK] = reinterpret_cast<uint16_t (*)[BM * BK]>(smem);
    uint16_t (*b_lds)[BN * BK] = reinterpret_cast<uint16_t (*)[BN * BK]>(smem + 2 * BM * BK);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware tile order: logical tiles run row-tile-major with the
    // output-column slices inner, and each XCD (physical id % 8) takes a
    // contiguous logical range, so an XCD's blocks share each row tile of
    // the input in its L2 across all column slices.  (Measured on MI355X
    // against slice-major order, which kept each XCD on one or two slices'
    // weights: Q/K/V 13% and 4% faster, output projection 3% and 8% faster
    // at the 640- and 1280-channel SDXL 3840 levels, bit-identical.)
    const int ntot = a.mtiles * a.ntiles;
    const int n8 = ntot - ntot % 8;
    const int pw = blockIdx.x;
    const int logical = pw < n8 ? (pw % 8) * (n8 / 8) + pw / 8 : pw;
    const int mt = logical / a.ntiles, nt = logical % a.ntiles;
    const int m0 = mt * BM, n0 = nt * BN;

    // Tile loads straight into LDS (global_load_lds_dwordx4): instruction j
    // of wave w writes LDS granules j*256 + w*64 + lane, i.e. row
    // (tid >> 3) + 32 j at physical chunk tid & 7, so the thread reads the
    // logical chunk the row's swizzle stores there.  Rows past M / N re-read
    // row 0: they feed only outputs that are never stored.  Their completion
    // is the explicit wait at the top of each step (global_load_lds16).
    const int akc = tid & 7;
    const uint16_t* aptr[A_CHUNKS];
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) {
        const int row = (tid >> 3) + 32 * j;
        const int m = m0 + row;
        aptr[j] = a.x + size_t(m < a.M ? m : 0) * a.K + swz(row, akc) * 8;
    }
    const uint16_t* bptr[B_CHUNKS];
#pragma unroll
    for (int j = 0; j < B_CHUNKS; ++j) {
        const int row = (tid >> 3) + 32 * j;
        const int n = n0 + row;
        bptr[j] = a.w + size_t(n < a.N ? n : 0) * a.K + swz(row, akc) * 8;
    }

    const int nsteps = a.K / BK;
    const uint32_t wslot = uint32_t(wave) * 64 * 16;
    auto tile_load = [&](int s, int buf) {
        const uint32_t al = lds_addr(&a_lds[buf][0]) + wslot;
        const uint32_t bl = lds_addr(&b_lds[buf][0]) + wslot;
#pragma unroll
        for (int j = 0; j < A_CHUNKS; ++j) global_load_lds16(aptr[j] + s * BK, al + j * 256 * 16);
#pragma unroll
        for (int j = 0; j < B_CHUNKS; ++j) global_load_lds16(bptr[j] + s * BK, bl + j * 256 * 16);
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int cur) {
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            bf16x8 af[MT], bf[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int row = wm * WM + i * 16 + l16;
                af[i] = *reinterpret_cast<const bf16x8*>(&a_lds[cur][row * BK + swz(row, kk * 4 + lq) * 8]);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int row = wn * WN + j * 16 + l16;
                bf[j] = *reinterpret_cast<const bf16x8*>(&b_lds[cur][row * BK + swz(row, kk * 4 + lq) * 8]);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
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
    __syncthreads();  // every wave is done with the K-loop buffers

    // epilogue, through LDS so that every global store is 16 bytes: acc[i][j][e]
    // (row wm*WM + i*16 + 4*lq + e, column wn*80 + j*16 + l16 of the tile)
    // plus the bias goes to the tile in LDS as bf16 (after the barrier above
    // the K-loop buffers are free); then each thread stores rows
    // of 8 columns.  N and the part width are multiples of 64, so 8 columns
    // never straddle a part or the end of N.
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int c = wn * WN + j * 16 + l16;
        const float bias = a.bias ? a.bias[min(n0 + c, a.N - 1)] : 0.f;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                smem[(wm * WM + i * 16 + 4 * lq + e) * CS + c] = f32_to_bf16(acc[i][j][e] + bias);
    }
    __syncthreads();
    const Route& rt = a.r;
    constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
    for (int ch = tid; ch < BM * CPR; ch += 256) {
        const int row = ch / CPR, cc = ch - row * CPR;
        const int m = m0 + row, n = n0 + cc * 8;
        if (m >= a.M || n >= a.N) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(&smem[row * CS + cc * 8]);
        const int part = n / rt.part_cols;
        const int col = n - part * rt.part_cols;
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(rt.dst[part]) + size_t(m) * rt.part_cols + col) = v;
        if (uint16_t* stale = static_cast<uint16_t*>(rt.stale[part])) {
            const int b = m / rt.lq, t = m - b * rt.lq;
            *reinterpret_cast<u32x4*>(stale + (b * rt.L + rt.own + t) * rt.part_cols + col) = v;
        }
    }
}

// ----------------------------------------------------------------- fp32 path
struct ProjArgsF32 {
    const float* x;
    const float* w;
    const float* bias;
    int64_t M, K, N;
    Route r;
};

__global__ __launch_bounds__(256) void proj_f32_kernel(ProjArgsF32 a) {
    const int64_t total = a.M * a.N;
    const Route& rt = a.r;
    for (int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * 256) {
        const int64_t m = idx / a.N;
        const int n = int(idx % a.N);
        const float* xp = a.x + m * a.K;
        const float* wp = a.w + int64_t(n) * a.K;
        float acc = a.bias ? a.bias[n] : 0.f;
        for (int64_t c = 0; c < a.K; ++c) acc = fmaf(wp[c], xp[c], acc);
        const int part = n / rt.part_cols;
        const int col = n - part * rt.part_cols;
        static_cast<float*>(rt.dst[part])[m * rt.part_cols + col] = acc;
        if (rt.stale[part]) {
            const int64_t b = m / rt.lq, t = m - b * rt.lq;
            static_cast<float*>(rt.stale[part])[(b * rt.L + rt.own + t) * rt.part_cols + col] = acc;
        }
    }
}

hipError_t launch(int64_t M, int64_t K, int64_t N, bool bf16, const void* x, const void* w,
                  const float* bias, const Route& r, hipStream_t s) {
    if (bf16) {
        ProjArgs a;
        a.x = static_cast<const uint16_t*>(x);
        a.w = static_cast<const uint16_t*>(w);
        a.bias = bias;
        a.M = int(M);
        a.K = int(K);
        a.N = int(N);
        a.r = r;
        a.ntiles = int(ceil_div(N, BN));
        // two blocks are resident per CU: the 128-row tile when it still
        // gives at least ~1.6 blocks per CU
        const int64_t t128 = ceil_div(M, 128) * a.ntiles;
        const bool big = t128 * 10 >= int64_t(device_cus()) * 16;
        a.mtiles = int(ceil_div(M, big ? 128 : 64));
        const unsigned grid = unsigned(a.mtiles) * unsigned(a.ntiles);
        if (big)
            hipLaunchKernelGGL(proj_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(proj_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    ProjArgsF32 a;
    a.x = static_cast<const float*>(x);
    a.w = static_cast<const float*>(w);
    a.bias = bias;
    a.M = M;
    a.K = K;
    a.N = N;
    a.r = r;
    int64_t blocks = ceil_div(M * N, 256);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(proj_f32_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool proj_launch_fits(int64_t M, int64_t N) {
    // the bf16 grid holds ceil(M / 64) x ceil(N / 160) blocks of 256 threads
    // at most, and a grid's thread count must stay below 2^32
    return ceil_div(M, 64) * ceil_div(N, BN) < (int64_t(1) << 24);
}

hipError_t launch_qkv_proj(const Geom& g, int64_t C, bool bf16, const void* x, const void* w_qkv,
                           const float* bias, void* q, void* k, void* v, void* k_stale,
                           void* v_stale, hipStream_t s) {
    Route r;
    r.dst[0] = q;
    r.dst[1] = k;
    r.dst[2] = v;
    r.stale[0] = nullptr;
    r.stale[1] = k_stale;
    r.stale[2] = v_stale;
    r.part_cols = int(C);
    r.lq = int(g.lq());
    r.L = g.L();
    r.own = g.i * g.lq();
    return launch(g.B * g.lq(), C, 3 * C, bf16, x, w_qkv, bias, r, s);
}

hipError_t launch_out_proj(const Geom& g, int64_t C, bool bf16, const void* o, const void* w_o,
                           const float* bias, void* y, hipStream_t s) {
    Route r;
    r.dst[0] = y;
    r.dst[1] = r.dst[2] = nullptr;
    r.stale[0] = r.stale[1] = r.stale[2] = nullptr;
    r.part_cols = int(C);
    r.lq = int(g.lq());
    r.L = g.L();
    r.own = g.i * g.lq();
    return launch(g.B * g.lq(), C, C, bf16, o, w_o, bias, r, s);
}

}  // namespace dp
