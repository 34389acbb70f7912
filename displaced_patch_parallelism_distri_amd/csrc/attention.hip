// Patch self-attention over fresh + stale K/V (DistriSelfAttentionPP:
// "DistriFusion源码探秘：从DistriUNetPP到DistriAttentionTP的模块设计原理", section
// "Patch Parallelism的实现原理", item 2; the other patches' K/V are the previous
// step's activations per "DistriFusion：高分辨率扩散模型的分布式并行推理", README
// mirror, section 概述, figure (c)).
//
//   out[b, r, hd] = softmax_t(scale <q[b, r, hd], K^[b, t, hd]>) . V^[b, t, hd]
//
// where token t < L of K^/V^ is the fresh local row when t lies in the
// patch's own token range [i*Lq, (i+1)*Lq) and the stale row otherwise.  No
// concatenated K/V is built: each K/V tile row picks its base pointer as it
// is loaded.
//
// bf16 kernel (gfx950, bf16 MFMA, fp32 accumulation):
//  * block = 4 waves x 64 queries; every wave keeps its Q^T fragments in
//    registers for the whole key loop;
//  * key tiles of 64 rows are staged in LDS, double-buffered: K row-major
//    (MFMA A operand for S^T = K Q^T) and V transposed to V^T[d][key] while it
//    is written (A operand for O^T = V^T P^T), so every MFMA operand is a
//    plain ds_read;
//  * S is computed transposed (keys x queries) with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 keys of ONE query per 32x32 block, so the row max and
//    row sum are in-lane reductions plus one exchange between the two
//    half-waves;
//  * online softmax in the log2 domain (exp2(s*scale*log2e - m)) with the
//    exact running max; O and l are rescaled only when some row of the wave
//    saw a new max (a wave-uniform branch that long key loops mostly skip);
//    the row sum l adds the bf16-rounded P (v_dot2_f32_bf16) so numerator and
//    denominator carry the same rounding - a row dominated by one key then
//    returns that key's V exactly;
//  * P is rounded to bf16 and fed straight from the S^T accumulators into the
//    PV MFMA as its B operand (the accumulator layout already matches the
//    operand layout, with the V^T reads permuted to agree).
// fp32 kernel: one thread per query, K/V tiles in LDS, fp32 online softmax
// with expf; used for fp32 inputs (parity-grade, small workloads).
#include "dp_common.h"

#include <math.h>

namespace dp {
namespace {

constexpr int D = 64;        // head dim
constexpr int KT = 64;       // keys per tile
constexpr int NWAVES = 4;    // waves per block
constexpr int QB = 2;        // 32-query blocks per wave
constexpr int QTILE = NWAVES * QB * 32;
constexpr int KPITCH = D + 8;   // LDS row pitch of K (bf16 elements)
constexpr int VPITCH = KT + 4;  // LDS row pitch of V^T (bf16 elements)

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* kf;
    const uint16_t* vf;
    const uint16_t* ks;
    const uint16_t* vs;
    uint16_t* out;
    int64_t lq;      // local queries per image
    int64_t L;       // tokens per image
    int64_t own_lo;  // first token of the patch
    int heads;
    float c;         // scale * log2(e)
};

__device__ __forceinline__ const uint16_t* token_row(const uint16_t* fresh, const uint16_t* stale,
                                                     int64_t b, int64_t hd, int64_t t,
                                                     const AttnArgs& a) {
    const int64_t rel = t - a.own_lo;
    if (rel >= 0 && rel < a.lq) return fresh + ((b * a.lq + rel) * a.heads + hd) * D;
    return stale + ((b * a.L + t) * a.heads + hd) * D;
}

__device__ __forceinline__ uint32_t half_of(const u32x4& v, int e) {
    const uint32_t w = v[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
    const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT * KPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VPITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, g = lane >> 5;
    const int64_t bh = blockIdx.y;
    const int64_t b = bh / a.heads, hd = bh % a.heads;
    const int64_t q0 = int64_t(blockIdx.x) * QTILE + wave * (QB * 32);

    // Q^T fragments (MFMA B operand): lane holds query q0+qb*32+lr, dims
    // ks*16 + g*8 .. +8.
    bf16x8 qf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        int64_t row = q0 + qb * 32 + lr;
        if (row > a.lq - 1) row = a.lq - 1;
        const uint16_t* qp = a.q + ((b * a.lq + row) * a.heads + hd) * D + g * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
    }

    // tile-load mapping: K rows kk and kk+32, V rows 2u and 2u+1, 8 dims each
    const int c8 = tid & 7;
    const int kk = tid >> 3;
    u32x4 kr[2], vr[2];
    const int64_t ntiles = ceil_div(a.L, KT);

    auto gload = [&](int64_t kt) {
        const int64_t t0 = kt * KT;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t t = t0 + kk + 32 * j;
            if (t < a.L)
                kr[j] = *reinterpret_cast<const u32x4*>(token_row(a.kf, a.ks, b, hd, t, a) + c8 * 8);
            else
                kr[j] = u32x4{0, 0, 0, 0};
            const int64_t tv = t0 + 2 * kk + j;
            if (tv < a.L)
                vr[j] = *reinterpret_cast<const u32x4*>(token_row(a.vf, a.vs, b, hd, tv, a) + c8 * 8);
            else
                vr[j] = u32x4{0, 0, 0, 0};
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *reinterpret_cast<u32x4*>(&k_lds[buf][(kk + 32 * j) * KPITCH + c8 * 8]) = kr[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = half_of(vr[0], e) | (half_of(vr[1], e) << 16);
            *reinterpret_cast<uint32_t*>(&v_lds[buf][(c8 * 8 + e) * VPITCH + 2 * kk]) = w;
        }
    };

    f32x16 o[2][QB];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[db][qb] = f32x16{};
    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;
    }

    gload(0);
    lstore(0);
    __syncthreads();

    for (int64_t kt = 0; kt < ntiles; ++kt) {
        const int cur = int(kt & 1);
        if (kt + 1 < ntiles) gload(kt + 1);

        // S^T = K Q^T : s[kb][qb] covers keys kb*32.. and queries qb*32..
        f32x16 s[2][QB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
                    &k_lds[cur][(kb * 32 + lr) * KPITCH + ks * 16 + g * 8]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][ks], s[kb][qb],
                                                                        0, 0, 0);
            }
        }
        // keys past the end of the map (last tile only)
        if ((kt + 1) * KT > a.L) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int64_t key = kt * KT + kb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
                    if (key >= a.L)
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) s[kb][qb][j] = -INFINITY;
                }
        }

        bf16x8 p[2][QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = s[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][qb][j]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m[qb], mx * a.c);
            // exact running max; the rescale is skipped when no row of the
            // wave saw a larger score (wave-uniform branch)
            if (__any(mnew > m[qb])) {
                const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
                l[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < 2; ++db) o[db][qb] *= alpha;
                m[qb] = mnew;
            }
            const float mneg = -m[qb];
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    bf16x8 v;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][qb][h2 * 8 + e], a.c, mneg));
                    p[kb][qb][h2] = v;
                    // the row sum adds the bf16-rounded p that the PV MFMA
                    // multiplies, so the normalisation matches the numerator
#pragma unroll
                    for (int e = 0; e < 8; e += 2)
                        rs = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[e], v[e + 1]}, kOnes, rs, false);
                }
            }
            l[qb] += rs;
        }

        // O^T += V^T P^T.  B operand slot e of k-step (kb, h2) holds key
        // kb*32 + h2*16 + (e/4)*8 + 4g + e%4 (the S^T accumulator layout), so
        // the V^T operand reads those same keys: two 4-key runs.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    const uint16_t* vp =
                        &v_lds[cur][(db * 32 + lr) * VPITCH + kb * 32 + h2 * 16 + 4 * g];
                    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vp);
                    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vp + 8);
                    const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[kb][qb][h2],
                                                                            o[db][qb], 0, 0, 0);
                }
            }
        }

        if (kt + 1 < ntiles) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: O = O^T / l, lane writes 4-dim runs of its query row
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float ltot = l[qb] + __shfl_xor(l[qb], 32);
        const float inv = 1.0f / ltot;
        const int64_t row = q0 + qb * 32 + lr;
        if (row < a.lq) {
            uint16_t* op = a.out + ((b * a.lq + row) * a.heads + hd) * D;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int jg = 0; jg < 4; ++jg) {
                    u32x2 w;
                    w[0] = pack_bf16x2(o[db][qb][4 * jg] * inv, o[db][qb][4 * jg + 1] * inv);
                    w[1] = pack_bf16x2(o[db][qb][4 * jg + 2] * inv, o[db][qb][4 * jg + 3] * inv);
                    *reinterpret_cast<u32x2*>(op + db * 32 + 8 * jg + 4 * g) = w;
                }
        }
    }
}

// ----------------------------------------------------------------- fp32 path
struct AttnArgsF32 {
    const float* q;
    const float* kf;
    const float* vf;
    const float* ks;
    const float* vs;
    float* out;
    int64_t lq, L, own_lo;
    int heads;
    float scale;
};

__device__ __forceinline__ const float* token_row_f32(const float* fresh, const float* stale,
                                                      int64_t b, int64_t hd, int64_t t,
                                                      const AttnArgsF32& a) {
    const int64_t rel = t - a.own_lo;
    if (rel >= 0 && rel < a.lq) return fresh + ((b * a.lq + rel) * a.heads + hd) * D;
    return stale + ((b * a.L + t) * a.heads + hd) * D;
}

__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgsF32 a) {
    __shared__ float k_s[KT][D];
    __shared__ float v_s[KT][D];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int64_t b = bh / a.heads, hd = bh % a.heads;
    const int64_t row = int64_t(blockIdx.x) * 64 + tid;
    const int64_t rowc = row < a.lq ? row : a.lq - 1;
    float q[D], o[D];
    const float* qp = a.q + ((b * a.lq + rowc) * a.heads + hd) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) {
        q[e] = qp[e];
        o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int64_t t0 = 0; t0 < a.L; t0 += KT) {
        const int nk = int(a.L - t0 < KT ? a.L - t0 : KT);
        for (int idx = tid; idx < nk * (D / 4); idx += 64) {
            const int key = idx / (D / 4), c4 = idx % (D / 4);
            reinterpret_cast<f32x4*>(&k_s[key][0])[c4] =
                reinterpret_cast<const f32x4*>(token_row_f32(a.kf, a.ks, b, hd, t0 + key, a))[c4];
            reinterpret_cast<f32x4*>(&v_s[key][0])[c4] =
                reinterpret_cast<const f32x4*>(token_row_f32(a.vf, a.vs, b, hd, t0 + key, a))[c4];
        }
        __syncthreads();
        for (int key = 0; key < nk; ++key) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) dot = fmaf(q[e], k_s[key][e], dot);
            const float sc = dot * a.scale;
            if (sc > m) {
                const float corr = expf(m - sc);
                l *= corr;
#pragma unroll
                for (int e = 0; e < D; ++e) o[e] *= corr;
                m = sc;
            }
            const float p = expf(sc - m);
            l += p;
#pragma unroll
            for (int e = 0; e < D; ++e) o[e] = fmaf(p, v_s[key][e], o[e]);
        }
        __syncthreads();
    }
    if (row < a.lq) {
        float* op = a.out + ((b * a.lq + row) * a.heads + hd) * D;
        const float inv = 1.0f / l;
#pragma unroll
        for (int e = 0; e < D; ++e) op[e] = o[e] * inv;
    }
}

}  // namespace

size_t attention_workspace_bytes(const Geom&, int64_t, bool) { return 0; }

hipError_t launch_attention(const Geom& g, int64_t heads, float scale, bool bf16, const void* q,
                            const void* kf, const void* vf, const void* ks, const void* vs,
                            void* out, void*, hipStream_t s) {
    const int64_t lq = g.lq();
    if (bf16) {
        AttnArgs a;
        a.q = static_cast<const uint16_t*>(q);
        a.kf = static_cast<const uint16_t*>(kf);
        a.vf = static_cast<const uint16_t*>(vf);
        a.ks = static_cast<const uint16_t*>(ks);
        a.vs = static_cast<const uint16_t*>(vs);
        a.out = static_cast<uint16_t*>(out);
        a.lq = lq;
        a.L = g.L();
        a.own_lo = g.i * lq;
        a.heads = int(heads);
        a.c = scale * 1.4426950408889634f;
        dim3 grid(unsigned(ceil_div(lq, QTILE)), unsigned(g.B * heads));
        hipLaunchKernelGGL(attn_bf16_kernel, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    AttnArgsF32 a;
    a.q = static_cast<const float*>(q);
    a.kf = static_cast<const float*>(kf);
    a.vf = static_cast<const float*>(vf);
    a.ks = static_cast<const float*>(ks);
    a.vs = static_cast<const float*>(vs);
    a.out = static_cast<float*>(out);
    a.lq = lq;
    a.L = g.L();
    a.own_lo = g.i * lq;
    a.heads = int(heads);
    a.scale = scale;
    dim3 grid(unsigned(ceil_div(lq, 64)), unsigned(g.B * heads));
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace dp
