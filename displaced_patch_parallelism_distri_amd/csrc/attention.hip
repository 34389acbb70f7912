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
// bf16 kernel (gfx950, bf16 MFMA for the scores, f16 MFMA for the weighted
// sum, fp32 accumulation):
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
//    four stages, the loads three tiles ahead of their use.  K and V are
//    both kept row-major, each row's 16-byte granules XOR-swizzled so that
//    the operand reads hit every LDS bank evenly: K rows are the MFMA A
//    operand of S^T = K Q^T (ds_read_b128), and the V^T operand of O^T =
//    V^T P^T comes from the transposing read ds_read_b64_tr_b16 (a 16-lane
//    group turns 16 4-element row pieces into 4-key columns);
//  * the PV product runs in f16 (v_mfma_f32_32x32x16_f16): P rounded to f16
//    carries 11 significant bits against bf16's 8, which keeps the error of
//    the weights well below the output's own bf16 rounding.  Each V tile is
//    rewritten in LDS from bf16 to f16 once per block, a tile ahead of its
//    use (8 elements per thread), so the waves read f16 operands directly.
//    The bf16 -> f16 map is exact for |v| in [2^-14, 65504]; V elements of
//    magnitude 65536 or more become inf (a documented input range);
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
//    recomputes P.  P then stays at most kSumLimit, which f16 and the fp32
//    accumulators carry with the same relative precision.  The row sum l
//    adds the f16-rounded P (in f16 pairs, widened once per tile), so
//    numerator and denominator carry the same rounding of P;
//  * P is rounded to f16 and fed straight from the S^T accumulators into the
//    PV MFMA as its B operand (the accumulator layout already matches the
//    operand layout, with the V^T reads permuted to agree);
//  * MFMA / softmax overlap across waves (the key loop's comment has the
//    details): a wave's tile work splits into an MFMA phase and a VALU
//    (softmax) phase, and the two waves that share a SIMD run them in
//    opposite order, so one issues MFMAs while the other runs its softmax.
//    gfx950 co-issues exp / fma / cvt work of one wave beside another
//    wave's MFMAs, but hardly the dot instructions, so the softmax sums P
//    without them.
// fp32 kernel: one thread per query, K/V tiles in LDS, fp32 online softmax
// with expf; used for fp32 inputs (parity-grade, small workloads).
#include "dp_common.h"

#include <math.h>

#include <type_traits>

namespace dp {
namespace {

constexpr int D = 64;        // head dim
constexpr int KT = 64;       // keys per tile
constexpr int NWAVES = 8;    // waves per block: two per SIMD, waves w and w+4 sharing one
constexpr int BLOCKS_PER_CU = 1;
constexpr int TROWS = KT * 8 / (NWAVES * 64);  // K (and V) tile rows one thread loads
constexpr int QB = 2;        // 32-query blocks per wave
constexpr int QTILE = NWAVES * QB * 32;
constexpr int NSTAGE = 4;       // K/V tile stages in LDS (loads run three tiles ahead)
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

__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

// acc + lo(w) + hi(w) in fp32, for a word w of two f16: each half is widened
// exactly (v_fma_mix_f32 with an f16 operand).  Ends the softmax's row sum:
// on gfx950 v_dot2_f32_f16 would take one instruction per word, but the dot
// instructions do not issue beside another wave's MFMAs, which the key loop
// relies on.
__device__ __forceinline__ float add_f16x2(uint32_t w, float acc) {
    asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "+v"(acc)
        : "v"(w));
    return acc;
}

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
    __host__ __device__ __forceinline__ void tile_of(int64_t task, int64_t& bh, int& qt) const {
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

// The work plan is made for a fixed machine of kPlanCUs compute units (an
// MI355X), so that the workspace it needs is a function of the call's sizes
// alone; on a device with fewer CUs the same grid runs in more rounds.
constexpr int kPlanCUs = 256;

Plan make_plan(int64_t B, int64_t heads, int64_t lq, int64_t L, int cus = kPlanCUs) {
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
    // 16-byte granule c stored at position c ^ swizzle(t).  K stays bf16; a
    // V tile arrives as bf16 and is rewritten in place as f16 before its PV.
    __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[NSTAGE][2][KT * D];
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
    // Tiles whose 64 rows all lie inside the map: the thread's row pointers
    // advance by one tile stride (a wave-uniform offset), the fresh / stale
    // choice is one compare and two selects, the LDS slot is wave-uniform.
    // The map's last, partial tile takes the clamped per-row path below.
    static_assert(TROWS == 1, "one K and one V row per thread and tile");
    const int krow0 = tid >> 3;
    const uint64_t kst0 = reinterpret_cast<uint64_t>(kst + int64_t(krow0) * rs + (c8 ^ k_swizzle(krow0)) * 8);
    const uint64_t vst0 = reinterpret_cast<uint64_t>(vst + int64_t(krow0) * rs + (c8 ^ v_swizzle(krow0)) * 8);
    // fresh rows: row t sits at (t - own_lo) * rs of the fresh slice; the
    // address is formed for every row but used only where the row is fresh
    const uint64_t fshift = uint64_t(int64_t(a.own_lo) * rs * 2);
    const uint64_t kfr0 = reinterpret_cast<uint64_t>(kfr + int64_t(krow0) * rs + (c8 ^ k_swizzle(krow0)) * 8) - fshift;
    const uint64_t vfr0 = reinterpret_cast<uint64_t>(vfr + int64_t(krow0) * rs + (c8 ^ v_swizzle(krow0)) * 8) - fshift;
    const uint32_t wslot = uint32_t(__builtin_amdgcn_readfirstlane(wave)) * 64 * 16;
    const int full_tiles = a.L / KT;
    auto tile_load = [&](int kt, int stage) {
        if (kt < full_tiles) {
            // bytes from tile 0: below 2^32, as the map's bytes are (the ABI
            // bounds L * heads * D below 2^31 elements)
            const uint32_t d = __builtin_amdgcn_readfirstlane(uint32_t(kt) * uint32_t(KT * 2 * rs));
            const bool fresh = unsigned(kt * KT + krow0 - a.own_lo) < unsigned(a.lq);
            const uint16_t* kp = reinterpret_cast<const uint16_t*>((fresh ? kfr0 : kst0) + d);
            const uint16_t* vp = reinterpret_cast<const uint16_t*>((fresh ? vfr0 : vst0) + d);
            global_load_lds16(kp, lds_addr(&kv_lds[stage][0][0]) + wslot);
            global_load_lds16(vp, lds_addr(&kv_lds[stage][1][0]) + wslot);
            return;
        }
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
    // V tile of a stage, bf16 -> f16 in place: each thread rewrites 16-byte
    // pieces of it (which piece does not matter: the map is element-wise).
    // The PV product then multiplies f16 P by f16 V.
    auto convert_v = [&](int stage) {
#pragma unroll
        for (int j = 0; j < TROWS; ++j) {
            u32x4* vp = reinterpret_cast<u32x4*>(&kv_lds[stage][1][0]) + tid + j * NWAVES * 64;
            const u32x4 w = *vp;
            u32x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = bf16x2_to_f16x2(w[e]);
            *vp = h;
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

    // A wave whose 64 queries all lie past the patch (the last query tile of
    // a map whose Lq is not a multiple of 512) only loads and syncs, which
    // leaves its SIMD to the wave of the block that shares it.
    const bool wave_active = __builtin_amdgcn_readfirstlane(q0) < a.lq;  // wave-uniform
    // A wave whose second query block lies past the patch (8 or 32 queries
    // left in the map's last tile) runs the MFMAs and softmax of its first
    // block only, in an instance of the key loop of its own (chosen once,
    // so the common loop keeps its registers and schedule); its second
    // block keeps O = 0, l = 0, and no row of it is written.  (Measured on
    // MI355X: 0.5% / 0.3% faster at the SDXL 3840 levels, bit-identical.)
    const bool one_qb = __builtin_amdgcn_readfirstlane(q0 + 32) >= a.lq;  // wave-uniform
    const std::integral_constant<int, 1> kOneQB{};
    const std::integral_constant<int, 2> kTwoQB{};
    auto stage_of = [&](int kt) { return (kt - kt0) & (NSTAGE - 1); };

    // S^T = K Q^T of query block qb over the key tile in `stage`: s[kb] holds
    // keys kb*32 + 8*(j/4) + 4g + j%4 (j < 16) of query qb*32 + lr.  The two
    // accumulators alternate, so dependent MFMAs are never back to back.
    auto qk = [&](int stage, int qb, f32x16 (&s)[2]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
                    &kv_lds[stage][0][(kb * 32 + lr) * D + (((2 * ks + g) ^ ksw) * 8)]);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][ks],
                                                                ks == 0 ? f32x16{} : s[kb], 0, 0, 0);
            }
        }
    };
    // S^T of both query blocks over the key tile in `stage`, each K fragment
    // read once for the two MFMAs that use it
    auto qk2 = [&](int stage, f32x16 (&sa)[2], f32x16 (&sb)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
                    &kv_lds[stage][0][(kb * 32 + lr) * D + (((2 * ks + g) ^ ksw) * 8)]);
                sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[0][ks],
                                                                 ks == 0 ? f32x16{} : sa[kb], 0, 0, 0);
                sb[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[1][ks],
                                                                 ks == 0 ? f32x16{} : sb[kb], 0, 0, 0);
            }
        }
    };
    // keys of the map's last, partial tile that lie past L: score -inf.
    // Element (kb, j) holds tile key kb*32 + 8*(j/4) + (j%4) + 4g; it is
    // masked when 4g >= (valid keys in the tile) - (its lane-free part), a
    // compare of one lane value with a scalar per element, so nothing here
    // is worth hoisting out of the rare branch that calls it.
    const int g4 = 4 * g;
    auto mask_keys = [&](int kt, f32x16 (&s)[2]) {
        const int nvalid = __builtin_amdgcn_readfirstlane(a.L - kt * KT);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (g4 >= nvalid - (kb * 32 + 8 * (j >> 2) + (j & 3))) s[kb][j] = -INFINITY;
    };
    // P = exp2(s * c - m) rounded to f16, and the lane's sum of those
    // rounded values (the row sum adds the f16-rounded p that the PV MFMA
    // multiplies, so the normalisation matches the numerator).  The 32
    // values are summed as f16 pairs in a tree of v_pk_add_f16 (15
    // instructions instead of 32 widening adds; measured on MI355X, 1.5-1.8%
    // faster), then the two halves are widened: each half sums 16 values
    // with f16's 11-bit relative rounding per add.  A half that passes
    // 65504 becomes inf, which fails the caller's [0, kSumLimit] check and
    // takes the rescue branch, exactly as a large fp32 sum would.
    // p[kb][h2] is the B operand of k-step (kb, h2) of O^T = V^T P^T: the
    // S^T accumulator layout is already that operand's layout.
    auto softmax = [&](const f32x16 (&s)[2], float mneg, f16x8 (&p)[2][2]) {
        f16x2 part[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_f16x2(__builtin_amdgcn_exp2f(fmaf(s[kb][h2 * 8 + 2 * e], a.c, mneg)),
                                      __builtin_amdgcn_exp2f(fmaf(s[kb][h2 * 8 + 2 * e + 1], a.c, mneg)));
                part[kb][h2] = (as_f16x2(w[0]) + as_f16x2(w[1])) + (as_f16x2(w[2]) + as_f16x2(w[3]));
                p[kb][h2] = __builtin_bit_cast(f16x8, u32x4{w[0], w[1], w[2], w[3]});
            }
        }
        const f16x2 t = (part[0][0] + part[0][1]) + (part[1][0] + part[1][1]);
        return add_f16x2(__builtin_bit_cast(uint32_t, t), 0.f);
    };
    // The rare branch of the lazy maximum: the reference max of block qb
    // moves only when some lane's sum of P leaves [0, kSumLimit] (always on
    // the first tile, where m = -inf, and whenever a score exceeds m by about
    // log2(kSumLimit)).  Then S is formed again from the tile in LDS (so it
    // holds no registers across the common path), the row max taken, O and l
    // rescaled and P recomputed.
    auto rescue = [&](int stage, int kt, int qb, f32x16 (&s)[2], f16x8 (&p)[2][2], bool masked) {
        qk(stage, qb, s);
        if (masked) mask_keys(kt, s);
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, s[kb][j]);
        // the other half-wave holds the other 16 keys of each 32-key block
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.c;
        const float mnew = __builtin_fmaxf(m[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db) o[db][qb] *= alpha;
        m[qb] = mnew;
        return softmax(s, -mnew, p);
    };

    // The key loop, software-pipelined so that each run of VALU work (one
    // query block's softmax) has 16 independent MFMAs beside it, and each K
    // and V^T fragment read from LDS serves both query blocks:
    //   A(t): softmax of block 1, tile t    |  S of blocks 0 and 1, tile t+1
    //   B(t): softmax of block 0, tile t+1  |  PV of blocks 0 and 1, tile t
    // Iteration t starts with S of block 1 over tile t in s1 and P of block 0
    // over tile t in p0.  One barrier per tile, before A(t): after it tile
    // t+1 is in LDS (for S in A(t)), V of tile t is f16 and visible
    // (converted after the previous barrier), and every wave is past its
    // last read of tile t-1, whose stage the loads of tile t+3 then take.
    // In the last iteration A forms S over the next stage anyway (whatever it
    // holds) and B's softmax of it is discarded; the V conversion of that
    // stage is as harmless.  Keys past L exist only in the map's last tile:
    // its S is masked in a branch between phases, so that each phase stays
    // one block of straight-line code that the scheduler interleaves.
    // The key loop.  Each tile's work of a wave splits into an MFMA phase and
    // a VALU phase:
    //   alpha(k): PV of both query blocks over tile k (P of tile k), then S of
    //             both blocks over tile k+1 - MFMAs and their LDS operand reads;
    //   beta(j):  the online softmax of both blocks over S of tile j -> P of
    //             tile j - VALU work.
    // A CU holds two waves per SIMD, waves w and w+4.  Waves 4-7 run each tile
    // as alpha(k) then beta(k+1); waves 0-3 as beta(k) then alpha(k), half a
    // tile behind.  So while one wave of a SIMD issues its MFMA phase the
    // other issues its VALU phase.  (gfx950 overlaps an MFMA-only wave with
    // a VALU-only wave on one SIMD well; with short alternating phases, as
    // here, a register-only probe overlapped them far less.  Measured with
    // the tile loads in, this order still beats both groups running the
    // same order.)  The VALU phase is the longer one, and the issue arbiter
    // favours the older waves (0-3) when both have VALU work, so those run
    // the softmax first.  The tile loads and the V conversion ride in the
    // VALU phase of both groups.
    // One barrier per tile, before both groups' work on tile k: after it tile
    // k+1 is in LDS (S over it in alpha(k)), V of tile k is f16 and visible
    // (converted during tile k-1), and every wave is past its last read of
    // tile k-1, whose stage the loads of tile k+3 then take.
    const int grp = __builtin_amdgcn_readfirstlane(1 - (wave >> 2));  // wave-uniform
    const int masked_kt = a.L % KT != 0 && kt1 == pl.nkt ? kt1 - 1 : -1;
    f32x16 s[QB][2];
    f16x8 p[QB][2][2];
    // alpha issues every LDS operand read well before the MFMA that uses it:
    // the 16 V^T reads of tile k first, the 8 K fragments of tile k+1 after
    // the first PV MFMAs, then the MFMAs back to back - so that the phase
    // does not stall on LDS latency between MFMAs.  One block of straight-
    // line code: after the last tile it forms S over the next stage anyway
    // (whatever that holds) and no softmax reads it.
    auto alpha = [&](int kt, auto nq) __attribute__((always_inline)) {
        constexpr int NQ = decltype(nq)::value;  // query blocks with queries in the patch
        const int cs = stage_of(kt), ns = stage_of(kt + 1);
        f16x8 va[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kb = i / 4, h2 = (i / 2) % 2, db = i % 2;
            const uint32_t vb = lds_addr(&kv_lds[cs][1][0]) + vlane[db] + (kb * 32 + h2 * 16) * 128;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DP_LDS i16x4*)(vb));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DP_LDS i16x4*)(vb + 8 * 128));
            va[i] = __builtin_bit_cast(f16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
        bf16x8 ka[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kb = i / 4, h2 = (i / 2) % 2, db = i % 2;
            o[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i], p[0][kb][h2], o[db][0], 0, 0, 0);
            if (NQ > 1)
                o[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i], p[1][kb][h2], o[db][1], 0, 0, 0);
            if (i == 1) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int jkb = j / 4, jks = j % 4;
                    ka[j] = *reinterpret_cast<const bf16x8*>(
                        &kv_lds[ns][0][(jkb * 32 + lr) * D + (((2 * jks + g) ^ ksw) * 8)]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kb = j / 4, ks = j % 4;
            s[0][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j], qf[0][ks],
                                                               ks == 0 ? f32x16{} : s[0][kb], 0, 0, 0);
            if (NQ > 1)
                s[1][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j], qf[1][ks],
                                                                   ks == 0 ? f32x16{} : s[1][kb], 0, 0, 0);
        }
        // the issue order above, which the scheduler would otherwise undo
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);      // DS read: V^T of tile k
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NQ, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);       // DS read: K of tile k+1
        __builtin_amdgcn_sched_group_barrier(0x008, 14 * NQ, 0); // MFMA
    };
    // Both query blocks' softmax is issued before either range check: the
    // check is a wave-uniform branch on the end of a block's dependency chain
    // (exp -> pack -> sum tree -> widen), so checking each block at once
    // left that chain's latency exposed.  (Measured on MI355X, interleaved
    // A/B: 1.3-1.8% faster at level a, 0.4-0.8% at level b, output
    // bit-identical; moving the tile loads and V conversion in between as
    // well was 2-5% slower.)  A block's rescue touches only its own m, l, O
    // and P, so the order of the two is immaterial.
    auto beta = [&](int kt, auto nq) __attribute__((always_inline)) {
        constexpr int NQ = decltype(nq)::value;
        const bool masked = kt == masked_kt;
        if (masked) {
#pragma unroll
            for (int qb = 0; qb < NQ; ++qb) mask_keys(kt, s[qb]);
        }
        float r[QB];
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) r[qb] = softmax(s[qb], -m[qb], p[qb]);
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) {
            if (__any(!(r[qb] <= kSumLimit))) r[qb] = rescue(stage_of(kt), kt, qb, s[qb], p[qb], masked);
            l[qb] += r[qb];
        }
    };
    auto chores = [&](int kt) {
        if (kt + 3 < kt1) tile_load(kt + 3, stage_of(kt + 3));
        if (kt + 1 < kt1) convert_v(stage_of(kt + 1));
    };

    // Q is in registers before the first tile load is issued, so that the
    // compiler has no load of its own in flight inside the key loop (its
    // wait for one would also wait for the tile loads)
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    tile_load(kt0, 0);
    if (kt0 + 1 < kt1) tile_load(kt0 + 1, 1);
    if (kt0 + 2 < kt1) tile_load(kt0 + 2, 2);
    if (kt0 + 2 < kt1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * TROWS));
    else if (kt0 + 1 < kt1)
        __builtin_amdgcn_s_waitcnt(kVmcntTile);
    else
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    convert_v(0);
    // The key loop for waves with `nq` query blocks in the patch: both
    // instances run the same tile loads, conversions and barriers.
    auto key_loop = [&](auto nq) __attribute__((always_inline)) {
        constexpr int NQ = decltype(nq)::value;
        // S over the first tile; waves 4-7 also its softmax (their first
        // phase in the loop is alpha, which needs P)
        if (wave_active) {
            if (NQ > 1) qk2(0, s[0], s[1]);
            else qk(0, 0, s[0]);
            if (grp == 0) beta(kt0, nq);
        }
        // Both groups run the same sequence alpha(k), beta(k+1), alpha(k+1),
        // ...; the barrier of tile k falls before alpha(k) for waves 0-3 and
        // before beta(k) for waves 4-7, which puts the two waves of a SIMD
        // half a tile apart.
        for (int kt = kt0; kt < kt1; ++kt) {
            if (kt + 2 < kt1)
                __builtin_amdgcn_s_waitcnt(kVmcntTile);
            else
                __builtin_amdgcn_s_waitcnt(kVmcnt0);
            __syncthreads();
            if (grp != 0) {
                chores(kt);
                if (wave_active) beta(kt, nq);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (wave_active) alpha(kt, nq);
            __builtin_amdgcn_sched_barrier(0);
            if (grp == 0) {
                chores(kt);
                if (wave_active && kt + 1 < kt1) beta(kt + 1, nq);
            }
        }
    };
    if (one_qb)
        key_loop(kOneQB);
    else
        key_loop(kTwoQB);

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
    const Plan p = make_plan(B, heads, lq, L);
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
        AttnArgs a;
        a.q = static_cast<const uint16_t*>(q);
        a.kf = static_cast<const uint16_t*>(kf);
        a.vf = static_cast<const uint16_t*>(vf);
        a.ks = static_cast<const uint16_t*>(ks);
        a.vs = static_cast<const uint16_t*>(vs);
        a.out = static_cast<uint16_t*>(out);
        a.plan = make_plan(B, heads, lq, L);
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
