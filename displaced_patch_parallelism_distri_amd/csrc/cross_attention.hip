// Cross-attention of patch queries over a short shared context (the text
// encoder's tokens that the wrapped cross-attention of "DistriFusion源码探秘：
// 从DistriUNetPP到DistriAttentionTP的模块设计原理", section "Patch
// Parallelism的实现原理", item 2, attends to; nothing in it is stale):
//
//   out[b, r, hd] = softmax_t(scale <q[b, r, hd], k[b, t, hd]>) . v[b, t, hd],  t < ctx
//
// For ctx <= 128 every key of one (image, head) fits in LDS at once, so the
// key loop of the self-attention kernel (tiles, online softmax, partial
// chunks) is not needed: a block stages the whole context of its (image,
// head) once and its 4 waves then stream 32-query blocks through it, each
// block in one pass with the exact row max:
//  * K row-major (bf16) and V transposed (V^T[d][key]) in LDS as f16, keys
//    past ctx zero;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (a lane holds 16 keys of one
//    query per 32-key block, as in the self-attention kernel), keys past ctx
//    set to -inf, the row max over all keys in registers plus one exchange
//    between the half-waves;
//  * P = exp2(s c - max c) rounded to f16 straight into the PV MFMA's B
//    operand (v_mfma_f32_32x32x16_f16: 11 significant bits for the weights,
//    against bf16's 8), the row sum over the same rounded values; 16-key
//    groups that lie wholly past ctx are skipped.  V elements of magnitude
//    65536 or more become inf in f16 (a documented input range);
//  * the next query block's Q is loaded while the current one computes, and
//    O leaves through 16-byte stores after one lane exchange.
// The grid runs all heads of one token range next to each other, so blocks
// in flight read and write whole token rows of Q and O.
#include "dp_common.h"

#include <math.h>

namespace dp {
namespace {

constexpr int D = 64;          // head dim
constexpr int NW = 4;          // waves per block
constexpr int KPITCH = D + 8;  // LDS row pitch of K (bf16 elements)
constexpr int kBlocksPerCu = 3; // blocks resident per CU (3 waves per SIMD)
// dword 3 of a raw (unformatted, 32-bit data format) buffer resource on gfx9
constexpr int kRawBufferFlags = 0x00020000;

struct CtxArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    int lq;      // queries per image
    int ctx;     // context tokens per image
    int heads;
    int bh;      // images * heads
    int nqb;     // 32-query blocks per image
    int nchunk;  // blocks per (image, head); chunk j runs query blocks
                 // [j * nqb / nchunk, (j + 1) * nqb / nchunk)
    float c;     // scale * log2(e)
};

template <int NKB>
__global__ __launch_bounds__(256, 3) void attn_ctx_bf16_kernel(CtxArgs a) {
    constexpr int NK = NKB * 32;      // keys held (ctx rounded up to 32)
    constexpr int VPITCH = NK + 4;    // V^T row pitch: 2 x odd dwords, no bank conflicts
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[NK * KPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * VPITCH];
    const f16x2 kOnes = {(_Float16)1.0f, (_Float16)1.0f};

    const int bh = int(blockIdx.x % unsigned(a.bh));
    const int chunk = int(blockIdx.x / unsigned(a.bh));
    const int b = bh / a.heads, hd = bh % a.heads;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, g = lane >> 5;
    const int64_t rs = int64_t(a.heads) * D;  // elements between consecutive tokens

    // Q and O of image b as raw buffers over its lq token rows: a row past
    // lq reads as zero and its stores are dropped by the hardware range
    // check, so the last, partial query block needs no clamp or branch (a
    // branch around the stores made the compiler wait for them before the
    // next block's Q could be used).  Byte offsets stay below 2^32: the ABI
    // bounds lq * heads * 64 below 2^31.
    const int64_t img = int64_t(b) * a.lq * a.heads * D;
    const uint32_t img_bytes = uint32_t(int64_t(a.lq) * rs * 2);
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.q + img), 0, int(img_bytes), kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t ors =
        __builtin_amdgcn_make_buffer_rsrc(a.out + img, 0, int(img_bytes), kRawBufferFlags);
    const uint32_t lane_off = uint32_t((hd * D + g * 8) * 2);  // bytes within a token row
    const uint32_t row_bytes = uint32_t(rs * 2);
    // this wave's query blocks: qb0, qb0 + NW, ... below qend
    const int qb0 = int(int64_t(chunk) * a.nqb / a.nchunk) + wave;
    const int qend = int(int64_t(chunk + 1) * a.nqb / a.nchunk);
    auto qload = [&](int qblk, bf16x8 (&qf)[4]) {
        const uint32_t off = uint32_t(qblk * 32 + lr) * row_bytes + lane_off;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, int(off + ks * 32), 0, 0));
    };
    bf16x8 qf[4];
    if (qb0 < qend) qload(qb0, qf);

    // stage the context: K rows and V^T columns; keys past ctx are zero
    {
        const uint16_t* kb = a.k + (int64_t(b) * a.ctx * a.heads + hd) * D;
        const uint16_t* vb = a.v + (int64_t(b) * a.ctx * a.heads + hd) * D;
        for (int idx = tid; idx < NK * 8; idx += 256) {
            const int t = idx >> 3, c8 = idx & 7;
            const u32x4 kv = t < a.ctx ? *reinterpret_cast<const u32x4*>(kb + t * rs + c8 * 8)
                                       : u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4*>(&k_lds[t * KPITCH + c8 * 8]) = kv;
        }
        for (int idx = tid; idx < NK * 4; idx += 256) {
            const int t2 = idx >> 3, c8 = idx & 7;  // key pair (2 t2, 2 t2 + 1), dims c8*8..
            const int t = 2 * t2;
            const u32x4 v0 = t < a.ctx ? *reinterpret_cast<const u32x4*>(vb + t * rs + c8 * 8)
                                       : u32x4{0, 0, 0, 0};
            const u32x4 v1 = t + 1 < a.ctx ? *reinterpret_cast<const u32x4*>(vb + (t + 1) * rs + c8 * 8)
                                           : u32x4{0, 0, 0, 0};
            // dims 2j and 2j + 1 of keys (t, t + 1), each pair as f16
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = pack_f16x2(__uint_as_float(v0[j] << 16), __uint_as_float(v1[j] << 16));
                const uint32_t hi = pack_f16x2(__uint_as_float(v0[j] & 0xffff0000u),
                                               __uint_as_float(v1[j] & 0xffff0000u));
                *reinterpret_cast<uint32_t*>(&v_lds[(c8 * 8 + 2 * j) * VPITCH + t]) = lo;
                *reinterpret_cast<uint32_t*>(&v_lds[(c8 * 8 + 2 * j + 1) * VPITCH + t]) = hi;
            }
        }
    }
    __syncthreads();

    const int koff0 = lr * KPITCH + g * 8;
    // one 32-query block: S, the next block's Q load, softmax, PV, O stores
    auto run_block = [&](const int qblk) {
        // S^T = K Q^T: s[kb] holds keys kb*32 + 8*(j/4) + 4g + j%4 of query
        // lr.  K is read from LDS on every query block: the empty asm keeps
        // the compiler from hoisting the reads and holding all of K in
        // registers, which would leave too few for the rest.
        int koff = koff0;
        asm volatile("" : "+v"(koff));
        f32x16 s[NKB];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8 ka =
                    *reinterpret_cast<const bf16x8*>(&k_lds[koff + kb * 32 * KPITCH + ks * 16]);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? f32x16{} : s[kb],
                                                                0, 0, 0);
            }
        // Q of the next query block into the same registers; its latency
        // hides behind this block's softmax, PV and stores
        if (qblk + NW < qend) qload(qblk + NW, qf);
        if (a.ctx < NK) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = (NKB - 1) * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
                if (key >= a.ctx) s[NKB - 1][j] = -INFINITY;
            }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, s[kb][j]);
        // the other half-wave holds the other 16 keys of each 32-key block
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false,
                                                         false);
        const float mneg = -__builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.c;

        // P in f16 and its row sum; O^T = V^T P^T.  B operand slot e of the
        // k-step (kb, h2) holds key kb*32 + h2*16 + (e/4)*8 + 4g + e%4 (the
        // S^T accumulator layout); the V^T operand reads those same keys.
        f32x16 o[2] = {f32x16{}, f32x16{}};
        float rsum = 0.f;
        // V^T operands of 16-key group gi = 2 kb + h2 for both 32-dim halves
        auto vread = [&](int gi, f16x8 (&va)[2]) {
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const uint16_t* vp = &v_lds[(db * 32 + lr) * VPITCH + gi * 16 + 4 * g];
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8);
                va[db] = __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
        };
        // groups wholly past ctx hold only masked keys and are skipped; the
        // next group's V^T is read before this group's exponentials
        const int ngroups = (a.ctx + 15) / 16 < 2 * NKB ? (a.ctx + 15) / 16 : 2 * NKB;
        f16x8 vcur[2], vnext[2];
        vread(0, vcur);
#pragma unroll
        for (int gi = 0; gi < 2 * NKB; ++gi) {
            if (gi >= ngroups) break;
            if (gi + 1 < ngroups) vread(gi + 1, vnext);
            const int kb = gi >> 1, h2 = gi & 1;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = pack_f16x2(__builtin_amdgcn_exp2f(fmaf(s[kb][h2 * 8 + 2 * e], a.c, mneg)),
                                  __builtin_amdgcn_exp2f(fmaf(s[kb][h2 * 8 + 2 * e + 1], a.c, mneg)));
            const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
            rsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w0), kOnes, rsum, false);
            rsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w1), kOnes, rsum, false);
            rsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w2), kOnes, rsum, false);
            rsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w3), kOnes, rsum, false);
            const f16x8 p = __builtin_bit_cast(f16x8, u32x4{w0, w1, w2, w3});
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vcur[db], p, o[db], 0, 0, 0);
                vcur[db] = vnext[db];
            }
        }
        const float inv = 1.0f / (rsum + __shfl_xor(rsum, 32));

        // O^T accumulator: lane holds dims db*32 + 8*jg + 4g + 0..3 of query
        // lr.  One swap between the half-waves per pair (jg0, jg1) gives the
        // lower half-wave dims 8*jg0 .. +8 and the upper one 8*jg1 .. +8.
        const uint32_t orow = uint32_t(qblk * 32 + lr) * row_bytes + uint32_t(hd * D * 2);
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
                const int j0 = 2 * jp, j1 = 2 * jp + 1;
                u32x2 x0, x1;
                x0[0] = pack_bf16x2(o[db][4 * j0] * inv, o[db][4 * j0 + 1] * inv);
                x0[1] = pack_bf16x2(o[db][4 * j0 + 2] * inv, o[db][4 * j0 + 3] * inv);
                x1[0] = pack_bf16x2(o[db][4 * j1] * inv, o[db][4 * j1 + 1] * inv);
                x1[1] = pack_bf16x2(o[db][4 * j1 + 2] * inv, o[db][4 * j1 + 3] * inv);
                const auto e0 = __builtin_amdgcn_permlane32_swap(x0[0], x1[0], false, false);
                const auto e1 = __builtin_amdgcn_permlane32_swap(x0[1], x1[1], false, false);
                const u32x4 w = {e0[0], e1[0], e0[1], e1[1]};
                __builtin_amdgcn_raw_buffer_store_b128(w, ors, int(orow + (db * 32 + 8 * (g ? j1 : j0)) * 2), 0, 0);
            }
    };
    // The first block runs outside the loop, so that every entry into the
    // loop has the same loads and stores in flight (the previous block's Q
    // prefetch, then its O stores) and the compiler's wait for Q does not
    // also wait for those stores.
    if (qb0 < qend) {
        run_block(qb0);
        for (int qblk = qb0 + NW; qblk < qend; qblk += NW) run_block(qblk);
    }
}

}  // namespace

bool cross_attention_short(int64_t lq, int64_t ctx, int64_t heads) {
    // the buffer byte offsets of the last query block, rows past lq
    // included, must stay below 2^32
    return ctx >= 1 && ctx <= kCrossCtxMax && ceil_div(lq, 32) * 32 * heads * D * 2 < (int64_t(1) << 32);
}

hipError_t launch_cross_attention(int64_t B, int64_t lq, int64_t ctx, int64_t heads, float scale,
                                  const void* q, const void* k, const void* v, void* out,
                                  hipStream_t s) {
    if (B == 0 || lq == 0) return hipSuccess;
    if (!cross_attention_short(lq, ctx, heads)) return hipErrorInvalidValue;
    CtxArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.out = static_cast<uint16_t*>(out);
    a.lq = int(lq);
    a.ctx = int(ctx);
    a.heads = int(heads);
    a.bh = int(B * heads);
    a.nqb = int(ceil_div(lq, 32));
    a.c = scale * 1.4426950408889634f;
    // about kBlocksPerCu blocks per CU in all, each on one (image, head)
    // and a contiguous range of its query blocks (at least one per wave)
    const int cus = device_cus() > 0 ? device_cus() : 256;
    const int64_t per_bh = (int64_t(kBlocksPerCu) * cus + a.bh / 2) / a.bh;
    const int64_t most = ceil_div(a.nqb, NW);
    a.nchunk = int(per_bh < 1 ? 1 : per_bh > most ? most : per_bh);
    const int64_t chunks = a.nchunk;
    const int64_t grid = chunks * a.bh;
    if (grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    switch ((ctx + 31) / 32) {
        case 1: attn_ctx_bf16_kernel<1><<<dim3(unsigned(grid)), dim3(256), 0, s>>>(a); break;
        case 2: attn_ctx_bf16_kernel<2><<<dim3(unsigned(grid)), dim3(256), 0, s>>>(a); break;
        case 3: attn_ctx_bf16_kernel<3><<<dim3(unsigned(grid)), dim3(256), 0, s>>>(a); break;
        default: attn_ctx_bf16_kernel<4><<<dim3(unsigned(grid)), dim3(256), 0, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace dp
