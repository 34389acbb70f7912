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
//  * block = 8 waves x 64 queries (a 512-query tile of one image and head),
//    one block per CU; every wave keeps its Q^T fragments in registers for
//    the whole key loop;
//  * work plan: with P = one block per CU running at once, whole (tile,
//    head, image) tasks are handed out in full rounds of P blocks; the tasks
//    left over are split along the keys into S chunks (S from a small cost
//    model) so the last round also fills the machine, and a combine kernel
//    merges the chunks' partial (O, max, sum).  Block ids are remapped so
//    that the blocks one XCD runs at the same time hold neighbouring tiles of
//    the same head and walk the same keys together, sharing K/V tiles in that
//    XCD's L2;
//  * key tiles of 64 rows go from global memory straight into LDS
//    (global_load_lds_dwordx4: no registers, no LDS store instructions) in
//    three stages, the loads two tiles ahead of their use.  K and V are
//    both kept row-major, each row's 16-byte granules XOR-swizzled so that
//    the operand reads hit every LDS bank evenly: K rows are the MFMA A
//    operand of S^T = K Q^T (ds_read_b128), and the V^T operand of O^T =
//    V^T P^T comes from the transposing read ds_read_b64_tr_b16 (a 16-lane
//    group turns 16 4-element row pieces into 4-key columns);
//  * S is computed transposed (keys x queries) with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 keys of ONE query per 32x32 block, so the row max and
//    row sum are in-lane reductions plus one exchange between the two
//    half-waves;
//  * online softmax in the log2 domain (exp2(s*scale*log2e - m)) against a
//    reference max m that moves only when needed: each tile first forms P
//    with the current m and no row max at all; only if some lane's sum of P
//    leaves [0, kSumLimit] (the first tile, where m = -inf, or a score above
//    m by about log2(kSumLimit)) does the wave take a rare, wave-uniform
//    branch that forms S again, takes the row max, rescales O and l and
//    recomputes P.  P then stays at most kSumLimit, which bf16 and the fp32
//    accumulators carry with the same relative precision.  The row sum l
//    adds the bf16-rounded P (v_dot2_f32_bf16) so numerator and denominator
//    carry the same rounding - a row dominated by one key then returns that
//    key's V exactly;
//  * P is rounded to bf16 and fed straight from the S^T accumulators into the
//    PV MFMA as its B operand (the accumulator layout already matches the
//    operand layout, with the V^T reads permuted to agree).
// fp32 kernel: one thread per query, K/V tiles in LDS, fp32 online softmax
// with expf; used for fp32 inputs (parity-grade, small workloads).
#include "dp_common.h"

#include <math.h>

#include <type_traits>

namespace dp {
namespace {

constexpr int D = 64;        // head dim
constexpr int KT = 64;       // keys per tile
constexpr int NWAVES = 8;    // waves per block (4 or 8)
constexpr int BLOCKS_PER_CU = 8 / NWAVES;  // two waves per SIMD either way
constexpr int TROWS = KT * 8 / (NWAVES * 64);  // K (and V) tile rows one thread loads
constexpr int QB = 2;        // 32-query blocks per wave
constexpr int QTILE = NWAVES * QB * 32;
constexpr int NSTAGE = 3;       // K/V tile stages in LDS (loads run two tiles ahead)
constexpr int kPartialCost = 3; // cost of one partial write + merge, in key tiles
constexpr float kSumLimit = 4096.0f;  // largest lane sum of P kept without moving the max

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
constexpr int kVmcnt0 = vmcnt_imm(0);
constexpr int kVmcntTile = vmcnt_imm(2 * TROWS);  // one tile's loads per thread

// 16-byte granule swizzles of a K and a V tile row.  K: the 32 rows of an
// operand read spread over all eight granule positions; V: the eight rows
// of a transposing read land on both halves of the granule range.
__device__ __forceinline__ int k_swizzle(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int v_swizzle(int row) { return ((row >> 1) & 1) * 4; }

// Work plan shared by the host launcher and both kernels.
struct Plan {
    int64_t tasks;  // images * heads * query tiles
    int nqt, nkt;   // query tiles per (image, head); key tiles
    int P;          // blocks resident at once (multiple of 8)
    int64_t F;      // tasks run whole, in full rounds of P blocks
    int R;          // tasks left over, each split into S key chunks
    int S;
    int nfull;      // query tiles per (image, head) that hold QTILE queries
    int64_t grid() const { return F + int64_t(R) * S; }
    // Task order: every (image, head)'s full query tiles first, head after
    // head, then the partial last tiles of all heads.  The partial tiles (one
    // wave of queries at level a) thus fall into the key-split remainder
    // instead of taking a CU for a whole round of full tasks.
    __host__ __device__ void tile_of(int64_t task, int64_t& bh, int& qt) const {
        const int64_t nf = tasks / nqt * nfull;  // tasks on full tiles
        if (task < nf) {
            bh = task / nfull;
            qt = int(task % nfull);
        } else {
            bh = task - nf;
            qt = nqt - 1;
        }
    }
    int64_t partials() const { return S > 1 ? int64_t(R) * S : 0; }
};

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* kf;
    const uint16_t* vf;
    const uint16_t* ks;
    const uint16_t* vs;
    uint16_t* out;
    float* part_o;   // [partials][D][QTILE]  unnormalised O
    float* part_ml;  // [partials][QTILE][2]  (running max, sum)
    int lq;          // local queries per image
    int L;           // tokens per image
    int own_lo;      // first token of the patch
    int heads;
    float c;         // scale * log2(e)
    Plan plan;
};

Plan make_plan(int64_t B, int64_t heads, int64_t lq, int64_t L, int cus) {
    Plan p;
    p.nqt = int(ceil_div(lq, QTILE));
    p.nfull = int(lq / QTILE);
    p.nkt = int(ceil_div(L, KT));
    p.tasks = B * heads * p.nqt;
    p.P = BLOCKS_PER_CU * (cus > 4 ? cus : 4);
    p.P -= p.P % 8;
    p.F = (p.tasks / p.P) * p.P;
    p.R = int(p.tasks - p.F);
    p.S = 1;
    if (p.R > 0) {
        int64_t best = -1;
        const int smax = p.nkt < 32 ? p.nkt : 32;
        for (int S = 1; S <= smax; ++S) {
            const int64_t rounds = ceil_div(int64_t(p.R) * S, p.P);
            const int64_t cost = rounds * (ceil_div(p.nkt, S) + (S > 1 ? kPartialCost : 0));
            if (best < 0 || cost < best) {
                best = cost;
                p.S = S;
            }
        }
    }
    return p;
}

// Physical position w of n blocks -> logical index, so that the blocks the
// hardware places on one XCD (w % 8) get one contiguous logical range.
__device__ __forceinline__ int xcd_remap(int w, int n) {
    const int n8 = n - n % 8;
    if (w >= n8) return w;
    return (w % 8) * (n8 / 8) + w / 8;
}

__global__ __launch_bounds__(NWAVES * 64, BLOCKS_PER_CU) void attn_bf16_kernel(AttnArgs a) {
    // NSTAGE stages of [K tile | V tile], each 64 rows x 128 bytes, row t's
    // 16-byte granule c stored at position c ^ swizzle(t)
    __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[NSTAGE][2][KT * D];
    const bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
    const Plan& pl = a.plan;

    // ---- which (task, key range) this block owns
    const int64_t bid = blockIdx.x;
    int64_t task, part = -1;
    int kt0, kt1;
    if (bid < pl.F) {
        task = (bid / pl.P) * pl.P + xcd_remap(int(bid % pl.P), pl.P);
        kt0 = 0;
        kt1 = pl.nkt;
    } else {
        const int i2 = xcd_remap(int(bid - pl.F), pl.R * pl.S);
        const int c = i2 / pl.R, r = i2 % pl.R;
        task = pl.F + r;
        kt0 = int(int64_t(c) * pl.nkt / pl.S);
        kt1 = int(int64_t(c + 1) * pl.nkt / pl.S);
        if (pl.S > 1) part = int64_t(r) * pl.S + c;
    }
    int64_t bh;
    int qt;
    pl.tile_of(task, bh, qt);
    const int64_t b = bh / a.heads, hd = bh % a.heads;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, g = lane >> 5;
    const int q0 = qt * QTILE + wave * (QB * 32);
    const int rs = a.heads * D;  // elements between consecutive tokens

    // Q^T fragments (MFMA B operand): lane holds query q0+qb*32+lr, dims
    // ks*16 + g*8 .. +8.
    bf16x8 qf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        int row = q0 + qb * 32 + lr;
        if (row > a.lq - 1) row = a.lq - 1;
        const uint16_t* qp = a.q + (b * a.lq * a.heads + hd) * D + int64_t(row) * rs + g * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
    }

    // Tile loads: thread tid loads 16 bytes of K and of V from token rows
    // kt*64 + (tid >> 3) + j * NWAVES * 8 (j < TROWS) of the tile; its lane
    // slot in LDS is granule tid & 7 of that row, so it reads the granule
    // that the row's swizzle puts there.  A token row comes from the fresh slice inside the patch,
    // else from the stale map (32-bit offsets: the ABI bounds L * heads * D
    // below 2^31); rows past the map are clamped to its last row, whose keys
    // the last tile masks.  Their completion is the explicit vmcnt wait at
    // the top of each tile (global_load_lds16).
    const int c8 = tid & 7;
    const uint16_t* kst = a.ks + (b * a.L * a.heads + hd) * D;
    const uint16_t* vst = a.vs + (b * a.L * a.heads + hd) * D;
    const uint16_t* kfr = a.kf + (b * a.lq * a.heads + hd) * D;
    const uint16_t* vfr = a.vf + (b * a.lq * a.heads + hd) * D;
    auto tile_load = [&](int kt, int stage) {
#pragma unroll
        for (int j = 0; j < TROWS; ++j) {
            const int krow = (tid >> 3) + j * NWAVES * 8;
            int t = kt * KT + krow;
            if (t > a.L - 1) t = a.L - 1;
            const int rel = t - a.own_lo;
            const bool fresh = unsigned(rel) < unsigned(a.lq);
            const int off = (fresh ? rel : t) * rs;
            const uint16_t* kp = (fresh ? kfr : kst) + off + (c8 ^ k_swizzle(krow)) * 8;
            const uint16_t* vp = (fresh ? vfr : vst) + off + (c8 ^ v_swizzle(krow)) * 8;
            const uint32_t slot = uint32_t(j * NWAVES * 64 + wave * 64) * 16;
            global_load_lds16(kp, lds_addr(&kv_lds[stage][0][0]) + slot);
            global_load_lds16(vp, lds_addr(&kv_lds[stage][1][0]) + slot);
        }
    };
    // K operand (row kb*32 + lr, dims ks*16 + g*8 ..): granule 2 ks + g of
    // the row, swizzled; the row's swizzle depends on lr only
    const int ksw = k_swizzle(lr);
    // V^T operand by transposing read: within each 16-lane group (i = lane
    // & 15) lane i hands over the 4 dims (16 ((lane >> 4) & 1) + 4 (i & 3))..
    // of key row 4g + (i >> 2) of an 8-key run and receives dim
    // 16 ((lane >> 4) & 1) + i of keys 4g .. 4g + 3: the lane's MFMA row
    // db*32 + lr.  vlane[db]: its byte address within the run.
    const int ti = lane & 15;
    const int vrow = 4 * g + (ti >> 2);
    uint32_t vlane[2];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
        const int gran = (db * 4 + 2 * ((lane >> 4) & 1) + ((ti & 3) >> 1)) ^ v_swizzle(vrow);
        vlane[db] = uint32_t(vrow * 128 + gran * 16 + (ti & 1) * 8);
    }

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

    // one key tile: prefetch the next tile into registers, S^T on MFMA,
    // online softmax, PV on MFMA, then stage the prefetched tile in LDS.
    // kMask (a std::integral_constant) masks keys past the end of the map;
    // only the map's last, partial tile needs it.
    // A wave whose 64 queries all lie past the patch (the last query tile of
    // a map whose Lq is not a multiple of 512) only loads and syncs, which
    // leaves its SIMD to the wave of the block that shares it.
    const bool wave_active = q0 < a.lq;
    // S^T = K Q^T of LDS stage `cur` for query blocks qb in [q_lo, q_hi):
    // s[kb][qb] covers keys kb*32.. and queries qb*32..; keys past the map
    // (kMask) get -inf
    auto qk = [&](int cur, int kt, f32x16 (&s)[2][QB], int q_lo, int q_hi, auto kMask) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
                    &kv_lds[cur][0][(kb * 32 + lr) * D + (((2 * ks + g) ^ ksw) * 8)]);
#pragma unroll
                for (int qb = q_lo; qb < q_hi; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        ka, qf[qb][ks], ks == 0 ? f32x16{} : s[kb][qb], 0, 0, 0);
            }
        }
        if (decltype(kMask)::value) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = kt * KT + kb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
                    if (key >= a.L)
#pragma unroll
                        for (int qb = q_lo; qb < q_hi; ++qb) s[kb][qb][j] = -INFINITY;
                }
        }
    };
    // P = exp2(s * c - m[qb]) rounded to bf16, and the lane's sum of those
    // rounded values (the row sum adds the bf16-rounded p that the PV MFMA
    // multiplies, so the normalisation matches the numerator)
    auto softmax = [&](const f32x16 (&s)[2][QB], int qb, bf16x8 (&p)[2][2]) {
        const float mneg = -m[qb];
        float rsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16x2(
                        __builtin_amdgcn_exp2f(fmaf(s[kb][qb][h2 * 8 + 2 * e], a.c, mneg)),
                        __builtin_amdgcn_exp2f(fmaf(s[kb][qb][h2 * 8 + 2 * e + 1], a.c, mneg)));
                // (scalar words on purpose: passing vector elements w[e]
                // straight to the builtin made hipcc read w[0] four times)
                const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
                rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), kOnes, rsum, false);
                rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), kOnes, rsum, false);
                rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), kOnes, rsum, false);
                rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), kOnes, rsum, false);
                p[kb][h2] = __builtin_bit_cast(bf16x8, u32x4{w0, w1, w2, w3});
            }
        }
        return rsum;
    };

    // one key tile: prefetch the next tile into registers, S^T on MFMA, then
    // per 32-query block the online softmax and PV on MFMA (the PV of one
    // block overlaps the softmax of the next), then stage the prefetched tile
    // in LDS.  kMask (a std::integral_constant) masks keys past the end of
    // the map; only the map's last, partial tile needs it.
    // A wave whose 64 queries all lie past the patch (the last query tile of
    // a map whose Lq is not a multiple of 512) only loads and syncs, which
    // leaves its SIMD to the wave of the block that shares it.
    auto tile = [&](int kt, auto kMask) {
        const int cur = (kt - kt0) % NSTAGE;
        // this thread's loads of tile kt are done (those of tile kt + 1,
        // 2 TROWS per thread, may still be in flight); after the barrier every
        // wave's share is in LDS and every wave has left tile kt - 1, whose
        // stage the loads of tile kt + 2 then take
        if (kt + 1 < kt1)
            __builtin_amdgcn_s_waitcnt(kVmcntTile);
        else
            __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
        if (kt + 2 < kt1) tile_load(kt + 2, (kt + 2 - kt0) % NSTAGE);
        if (wave_active) {
            f32x16 s[2][QB];
            // one query block after the other, so that the second block's
            // MFMAs can overlap the first block's softmax
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) qk(cur, kt, s, qb, qb + 1, kMask);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                // fast path: P against the current reference max, no row max
                bf16x8 p[2][2];
                float rsum = softmax(s, qb, p);
                // the reference max moves only when some lane's sum of P
                // leaves [0, kSumLimit] (always on the first tile, where m =
                // -inf, and whenever a score exceeds m by about
                // log2(kSumLimit)): then this block's S is formed again, the
                // row max taken, O and l rescaled and P recomputed.  A
                // wave-uniform, rare branch; S is recomputed rather than kept
                // so that it holds no registers across the fast path.
                if (__any(!(rsum <= kSumLimit))) {
                    qk(cur, kt, s, qb, qb + 1, kMask);
                    float mx = s[0][qb][0];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, s[kb][qb][j]);
                    // the other half-wave holds the other 16 keys of each 32-key block
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                                     __float_as_uint(mx), false, false);
                    mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.c;
                    const float mnew = __builtin_fmaxf(m[qb], mx);
                    const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
                    l[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < 2; ++db) o[db][qb] *= alpha;
                    m[qb] = mnew;
                    rsum = softmax(s, qb, p);
                }
                l[qb] += rsum;

                // O^T += V^T P^T.  B operand slot e of k-step (kb, h2) holds
                // key kb*32 + h2*16 + (e/4)*8 + 4g + e%4 (the S^T accumulator
                // layout), so the V^T operand reads those same keys: two
                // 4-key runs.
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                        for (int db = 0; db < 2; ++db) {
                            const uint32_t vb =
                                lds_addr(&kv_lds[cur][1][0]) + vlane[db] + (kb * 32 + h2 * 16) * 128;
                            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DP_LDS i16x4*)(vb));
                            const i16x4 hi =
                                __builtin_amdgcn_ds_read_tr16_b64_v4i16((DP_LDS i16x4*)(vb + 8 * 128));
                            const bf16x8 va = __builtin_bit_cast(
                                bf16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[kb][h2], o[db][qb],
                                                                                0, 0, 0);
                        }
                    }
                }
            }
        }
    };

    // Q is in registers before the first tile load is issued, so that the
    // compiler has no load of its own in flight inside the key loop (its
    // wait for one would also wait for the tile loads)
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    tile_load(kt0, 0);
    if (kt0 + 1 < kt1) tile_load(kt0 + 1, 1);
    const int full_end = (kt1 == pl.nkt && a.L % KT != 0) ? kt1 - 1 : kt1;
    for (int kt = kt0; kt < full_end; ++kt) tile(kt, std::false_type{});
    if (full_end < kt1) tile(full_end, std::true_type{});

    if (part < 0) {
        // whole task: O = O^T / l, lane writes 4-dim runs of its query row
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float inv = 1.0f / (l[qb] + __shfl_xor(l[qb], 32));
            const int row = q0 + qb * 32 + lr;
            if (row < a.lq) {
                uint16_t* op = a.out + (b * a.lq * a.heads + hd) * D + int64_t(row) * rs;
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
    } else {
        // one key chunk of a split task: unnormalised O^T, max and sum
        float* po = a.part_o + part * D * QTILE;
        float* pml = a.part_ml + part * QTILE * 2;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float ltot = l[qb] + __shfl_xor(l[qb], 32);
            const int row = wave * (QB * 32) + qb * 32 + lr;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    po[(db * 32 + 8 * (j >> 2) + 4 * g + (j & 3)) * QTILE + row] = o[db][qb][j];
            if (g == 0) {
                pml[row * 2 + 0] = m[qb];
                pml[row * 2 + 1] = ltot;
            }
        }
    }
}

// Merge the S key chunks of each split task.  Block (task, dim group of 8):
// one thread per query row; the chunk weights exp2(m_c - M) are recomputed
// by every dim group (S values), the partial O reads are coalesced across
// the rows and S * 8 loads per thread stay in flight together.
constexpr int kCombineDims = 8;

__global__ __launch_bounds__(QTILE) void attn_combine_kernel(AttnArgs a) {
    const Plan& pl = a.plan;
    const int r = blockIdx.x;
    const int d0 = blockIdx.y * kCombineDims;
    const int64_t task = pl.F + r;
    int64_t bh;
    int qt;
    pl.tile_of(task, bh, qt);
    const int64_t b = bh / a.heads, hd = bh % a.heads;
    const int row = threadIdx.x;
    const int qrow = qt * QTILE + row;
    if (qrow >= a.lq) return;
    const int64_t p0 = int64_t(r) * pl.S;
    float M = -INFINITY;
    for (int c = 0; c < pl.S; ++c) M = fmaxf(M, a.part_ml[((p0 + c) * QTILE + row) * 2]);
    float acc[kCombineDims];
#pragma unroll
    for (int d = 0; d < kCombineDims; ++d) acc[d] = 0.f;
    float lsum = 0.f;
    for (int c = 0; c < pl.S; ++c) {
        const float* ml = a.part_ml + ((p0 + c) * QTILE + row) * 2;
        const float w = __builtin_amdgcn_exp2f(ml[0] - M);
        lsum = fmaf(w, ml[1], lsum);
        const float* po = a.part_o + ((p0 + c) * D + d0) * QTILE + row;
#pragma unroll
        for (int d = 0; d < kCombineDims; ++d) acc[d] = fmaf(w, po[d * QTILE], acc[d]);
    }
    const float inv = 1.0f / lsum;
    uint16_t* op = a.out + (b * a.lq * a.heads + hd) * D + int64_t(qrow) * a.heads * D + d0;
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
    *reinterpret_cast<u32x4*>(op) = w;
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

size_t attention_workspace_bytes(int64_t B, int64_t lq, int64_t L, int64_t heads, bool bf16) {
    if (!bf16) return 0;
    const int cus = device_cus();
    if (cus <= 0) return 0;
    const Plan p = make_plan(B, heads, lq, L, cus);
    return size_t(p.partials()) * QTILE * (D + 2) * sizeof(float);
}

size_t attention_workspace_bytes(const Geom& g, int64_t heads, bool bf16) {
    return attention_workspace_bytes(g.B, g.lq(), g.L(), heads, bf16);
}

hipError_t launch_attention(const Geom& g, int64_t heads, float scale, bool bf16, const void* q,
                            const void* kf, const void* vf, const void* ks, const void* vs,
                            void* out, void* ws, hipStream_t s) {
    return launch_attention_rows(g.B, g.lq(), g.L(), g.i * g.lq(), heads, scale, bf16, q, kf, vf,
                                 ks, vs, out, ws, s);
}

hipError_t launch_attention_rows(int64_t B, int64_t lq, int64_t L, int64_t own_lo, int64_t heads,
                                 float scale, bool bf16, const void* q, const void* kf,
                                 const void* vf, const void* ks, const void* vs, void* out,
                                 void* ws, hipStream_t s) {
    if (bf16) {
        const int cus = device_cus();
        if (cus <= 0) return hipErrorNoDevice;
        AttnArgs a;
        a.q = static_cast<const uint16_t*>(q);
        a.kf = static_cast<const uint16_t*>(kf);
        a.vf = static_cast<const uint16_t*>(vf);
        a.ks = static_cast<const uint16_t*>(ks);
        a.vs = static_cast<const uint16_t*>(vs);
        a.out = static_cast<uint16_t*>(out);
        a.plan = make_plan(B, heads, lq, L, cus);
        a.part_o = static_cast<float*>(ws);
        a.part_ml = a.part_o + a.plan.partials() * D * QTILE;
        a.lq = int(lq);
        a.L = int(L);
        a.own_lo = int(own_lo);
        a.heads = int(heads);
        a.c = scale * 1.4426950408889634f;
        hipLaunchKernelGGL(attn_bf16_kernel, dim3(unsigned(a.plan.grid())), dim3(NWAVES * 64), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.plan.partials() == 0) return e;
        hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned(a.plan.R), D / kCombineDims), dim3(QTILE),
                           0, s, a);
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
    a.L = L;
    a.own_lo = own_lo;
    a.heads = int(heads);
    a.scale = scale;
    dim3 grid(unsigned(ceil_div(lq, 64)), unsigned(B * heads));
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace dp
