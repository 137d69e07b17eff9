// fa_fwd.hip -- forward pass of exact attention on gfx950.
//
// Method (mlapandio "FlashAttention: IO-aware exact attention", flash half of
// the naive-vs-flash diagram and "Four ideas"): a workgroup keeps a block of
// query rows on chip and streams the key/value blocks of its head through LDS.
// For every query row it keeps a running max m, a running sum l and an
// unnormalised output O, rescales them when the max rises, and writes O / l
// once, plus the logsumexp m + ln l. No score ever reaches device memory.
//
// gfx950 design (prior art on the pages targets A100/H100; these choices are
// this kernel's own, backed by measurements on MI355X):
//  * The softmax is vector-ALU work that must overlap the MFMAs. One wave per
//    SIMD hides only about 2 VALU instructions under each 32x32x16 MFMA; two
//    waves per SIMD hide most of them. So a workgroup is 8 waves (2 per SIMD),
//    each owning 32 query rows (256 rows per workgroup, at most 256 registers
//    per wave), or at d = 128 up to 16384 rows per head and on small grids 4
//    waves over 128 rows with two workgroups per CU (fwd_waves). At d = 64 a score costs half the MFMA work for the same
//    softmax work, and the wave's loop fits in 156 registers: large grids take
//    12 waves (3 per SIMD, 384 rows), 10.8% less time on a 2 x 64-head,
//    16384-row causal forward. At d = 128 a third wave per SIMD does not fit
//    this loop (168 registers); the loop without the cross-chunk pipelining
//    does, and measured no faster than two pipelined waves.
//  * Keys are streamed in tiles of 64 through LDS with direct global->LDS
//    loads: K in 3 buffers, V in 2, one barrier per tile. Tiles are stored
//    densely with XOR-swizzled 16-byte chunks (fa_device.h): K by row for the
//    16-byte row reads, V by 64-byte quarter for the transposing reads. Every
//    read stays bank-conflict-free, and a copy moves whole 1 KiB blocks of data
//    only: 2 loads per wave per tile for each of K and V at d = 128 (padded
//    rows took 3 each, part of them duplicates).
//  * Inside each wave the work runs in chunks of 32 keys, software-pipelined by
//    hand: the MFMAs for the scores of chunk c+1 are interleaved with the exp /
//    sum / pack work of chunk c, and the P.V MFMAs of chunk c with the row max
//    of chunk c+1.
//  * The scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16. A lane then holds one query row and 16 keys per
//    32 x 32 block. The row max needs a single cross-lane step (lane l with
//    l ^ 32), and the fp32 accumulator registers become, after rounding to
//    bf16, the B operand of O^T += V^T P^T with no data movement. V^T is read
//    with ds_read_b64_tr_b16 in the matching key order.
//  * exp2 with scale * log2(e) folded into one FMA, x = S * scale * log2(e) - m,
//    computed for the next chunk beside the P.V MFMAs of the current one. The
//    reference m is not the running max: it starts at the first chunk's max
//    and moves only when a chunk's probabilities under it grow too large (a
//    lane's 16 values sum past 2^16, or overflow). That chunk is then redone
//    with the exact max, O and l rescaled. So no row max is computed for the
//    other chunks, and every P stays at most 2^16. Any reference value cancels
//    in O / l and m + ln l, so the result is the same (the fp64 model in
//    oracle/online.py checks this rule). In bf16, though, a stale reference
//    leaves a peaked row's dominant probability at some 2^x with x > 0 that
//    rounds by up to 2^-8 relative, about 0.01 on a value of 4. So O is
//    divided by the sum of the bf16 probabilities themselves: the weights
//    then sum to one as used, and the dominant value's rounding cancels, so
//    the bound need not keep the reference near the max: 2^16 redoes fewer
//    chunks than 2^8 (4% less time on a forward whose K rows are partly four
//    times larger), with the same errors in every parity test. The
//    matrix cores form that sum (two more MFMAs per chunk, ones * P^T): the
//    forward is bound by its vector-ALU issue, and one v_dot2 per pair cost
//    8.7% of its time. LSE keeps the fp32 sum.
//  * Causal: chunks above a wave's diagonal are skipped; the diagonal chunk and
//    the ragged last chunk are masked element-wise. Workgroups run heaviest
//    q-tile first (longest-processing-time order). Workgroups of one head set
//    map to one XCD, so their K/V re-reads hit the same L2.
#include <atomic>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int kWM = 32;        // query rows per wave
constexpr int kBN = 64;        // keys per LDS tile
constexpr float kSumMax = 65536.0f;   // largest partial sum of P accepted without a new reference

// d = 64 and 128: 8 waves, two per SIMD (at most 256 registers each); d = 128
// takes 4 waves (128 rows, two workgroups per CU) up to 16384 rows per head and
// on small grids (fwd_waves). d = 64
// also has a 12-wave form, three per SIMD (its pipelined loop needs 156
// registers, within the 168 of three waves), for large grids (fwd_waves). d =
// 256: a wave's Q and O alone take 192 registers, so 4 waves, one per SIMD (up
// to 512 registers), and 128 rows per workgroup; its 3 K + 2 V tiles of 32 KiB
// fill the 160 KiB of LDS.
// PAD: the tensors' rows hold fewer than D values (a multiple of 8); the
// tiles' columns past them stay zero (CopyPlanSwz with PAD), so every product
// over D columns equals the product over the real ones.
template <int D, bool PAD = false, int W = (D == 256 ? 4 : 8)>
struct FwdCfg {
    static constexpr int DS = D / 16, DB = D / 32;
    static constexpr int WAVES = W;
    // Waves that copy: a tile is 16 (d = 128) or 8 (d = 64) blocks of 1 KiB,
    // so with 12 waves the first 8 copy and the other 4 only compute.
    static constexpr int CW = W > 8 ? 8 : W;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BM = kWM * WAVES;                       // query rows per workgroup
    static constexpr int L = 2 * D;                              // bytes per K / V row
    static constexpr int KT = kBN * L, VT = kBN * L;
    static constexpr int LDS = 3 * KT + 2 * VT;
    using PlanK = CopyPlanSwz<L, kBN, CW, RowKey<L>, PAD>;
    using PlanV = CopyPlanSwz<L, kBN, CW, TrKey<L>, PAD>;
};

// Workgroup id -> (rank, bh). Workgroups are handed to the 8 XCDs round-robin,
// so when the head count is a multiple of 8 each XCD gets a contiguous block of
// heads (whole GQA groups) and walks its q-tiles in rank order.
__device__ __forceinline__ void unmap_block(int bid, int nbh, int& rank, int& bh) {
    if ((nbh & 7) == 0) {
        const int x = bid & 7, r = bid >> 3, hpx = nbh >> 3;
        rank = r / hpx;
        bh = x * hpx + (r - rank * hpx);
    } else {
        rank = bid / nbh;
        bh = bid - rank * nbh;
    }
}

// ---- per-wave pieces of one 32-key chunk (32 query rows per wave) ----
// A chunk is half h of a 64-key tile. Scores S^T = K Q^T: lane holds query
// column l32 and keys (i/4)*8 + hh*4 + i%4 of register i.
//
// Lane bases (bytes, swizzle folded in; L = 2D bytes per row):
//   K: kbase = l32 * L + ((hh ^ k0) << 4) + ((key >> 1) << 5), key = swz_key(l32),
//      k0 = key & 1; chunk pair ds of the row is at (tile + kbase) ^ (ds << 5);
//   V: vbase = vr * L + (tr_key(vr) << 6) + ((g & 1) * 16 + 4 * (lane & 3)) * 2
//      with vr = (lane & 15) >> 2 + 4 * hh, g = lane >> 4; the 64-byte quarter
//      db is at (tile + vbase) ^ (db << 6).
// Row offsets that are multiples of 8 leave both keys unchanged, and tiles
// start on L-byte boundaries, so the XOR can act on the whole address.

// K fragment ds of chunk half h: the A operand of the score MFMAs (row l32,
// d = ds*16 + hh*8 .. +7).
template <int D>
__device__ __forceinline__ u32x4 k_frag(const FA_LDS uint8_t* __restrict__ Kt, int kbase, int h, int ds) {
    const uint32_t a = ((uint32_t)(uintptr_t)Kt + (uint32_t)kbase) ^ (uint32_t)(ds << 5);
    return *reinterpret_cast<const FA_LDS u32x4*>((const FA_LDS uint8_t*)(uintptr_t)a + h * 32 * FwdCfg<D>::L);
}

// V^T fragment f = (kc, db) of chunk half h: the A operand of the P.V MFMAs,
// read transposed so that its k slots run over keys in the order the P operand
// uses: slot hh*8 + t holds key kc*16 + (t/4)*8 + hh*4 + t%4.
template <int D>
__device__ __forceinline__ u32x4 v_frag(const FA_LDS uint8_t* __restrict__ Vt, int vbase, int h, int f) {
    constexpr int DB = FwdCfg<D>::DB, L = FwdCfg<D>::L;
    const int kc = f / DB, db = f % DB;
    const uint32_t a = ((uint32_t)(uintptr_t)Vt + (uint32_t)vbase) ^ (uint32_t)(db << 6);
    const FA_LDS uint8_t* p = (const FA_LDS uint8_t*)(uintptr_t)a + (h * 32 + kc * 16) * L;
    return cat(lds_read_trb(p, 0), lds_read_trb(p, 8 * L));
}

template <int D>
__device__ __forceinline__ f32x16 scores(const FA_LDS uint8_t* __restrict__ Kt, int kbase, int h,
                                         const u32x4 (&qf)[D / 16]) {
    f32x16 s = zero16();
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) s = mfma32(k_frag<D>(Kt, kbase, h, ds), qf[ds], s);
    return s;
}

// Diagonal or ragged chunk: scores (or x values) of invisible keys become -inf,
// so their probabilities are exact zeros. With a sliding window (WIN) the keys
// at or before qrow - win are invisible too.
template <bool WIN = false>
__device__ __forceinline__ void mask_scores(f32x16& s, int key0, int qrow, int N, bool causal, int hh,
                                            int win = 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int key = key0 + (i >> 2) * 8 + hh * 4 + (i & 3);
        // (rows past N, never stored, keep all keys below N so their max stays finite)
        if (key >= N || (causal && key > qrow) || (WIN && qrow < N && key <= qrow - win)) s[i] = -INFINITY;
    }
}

// Row max of a chunk in log2 units. Every chunk a wave computes has a visible
// key in every row, or the row is past N (finite scores, never stored). With a
// positive scale_log2 (the host keeps it >= 1e-30) the max commutes with it.
__device__ __forceinline__ float chunk_max(const f32x16& s, float sl2) {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    return fmaxf(mx, swap_half(mx)) * sl2;
}

// P~ = exp2(x) for pack pi = 0..7 of a chunk holding x = S*sl2 - m (16-key
// half kc = pi / 4, dword t = pi % 4): registers kc*8 + 2t and +1, rounded to a
// bf16 pair, which is k slot pair (2t, 2t+1) of the P^T operand of half kc.
__device__ __forceinline__ void exp_pack_one(const f32x16& x, int pi, float& ls, u32x4 (&pp)[2]) {
    const int kc = pi >> 2, t = pi & 3, i = kc * 8 + 2 * t;
    const float p0 = fast_exp2(x[i]);
    const float p1 = fast_exp2(x[i + 1]);
    ls = pi == 0 ? p0 + p1 : ls + (p0 + p1);   // the chunk's first pair starts the sum (no 0 + x)
    pp[kc][t] = pack_bf16(p0, p1);
}

// The A operand of all-ones bf16 values: ones * P^T sums, for every query row
// (lane column), the bf16 probabilities the P.V MFMA takes, over both lane
// halves' keys. Every register of the accumulator then holds that row sum.
__device__ __forceinline__ u32x4 ones_bf16() {
    const uint32_t one2 = 0x3F803F80u;
    return u32x4{one2, one2, one2, one2};
}

// The reference check after a chunk's exps (ls: this lane's sum, pp: packs).
// Unless some lane's sum exceeds kSumMax or is not finite, every P of the chunk
// is at most kSumMax and nothing happens. Otherwise the wave moves m up to the
// exact running max (m + the chunk's max of x, both lane halves), rescales O
// and l by 2^(m_old - m_new), shifts x and redoes the exps.
template <int D>
__device__ __forceinline__ void check_reference(f32x16& x, float& m, float& l, f32x16& lsum, f32x16 (&o)[D / 32],
                                                float& ls, u32x4 (&pp)[2]) {
    if (__ballot(!(ls <= kSumMax))) {
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
        const float delta = fmaxf(fmaxf(mx, swap_half(mx)), 0.f);
        const float alpha = fast_exp2(-delta);
        l *= alpha;
        lsum[0] *= alpha;   // the only entry the epilogue reads
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        m += delta;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] -= delta;
        ls = 0.f;
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) exp_pack_one(x, pi, ls, pp);
    }
}

// Softmax and O^T += V^T P^T for one chunk (not pipelined: a wave's last chunk).
template <int D>
__device__ __forceinline__ void softmax_pv(const FA_LDS uint8_t* __restrict__ Vt, int vbase, int h,
                                           f32x16& x, float& m, float& l, f32x16& lsum, f32x16 (&o)[D / 32]) {
    constexpr int DB = D / 32;
    u32x4 pp[2];
    float ls = 0.f;
#pragma unroll
    for (int pi = 0; pi < 8; ++pi) exp_pack_one(x, pi, ls, pp);
    check_reference<D>(x, m, l, lsum, o, ls, pp);
    l += ls;
    lsum = mfma32(ones_bf16(), pp[0], lsum);
    lsum = mfma32(ones_bf16(), pp[1], lsum);
#pragma unroll
    for (int f = 0; f < 2 * DB; ++f) o[f % DB] = mfma32(v_frag<D>(Vt, vbase, h, f), pp[f / DB], o[f % DB]);
}

// The global->LDS copies of one tile iteration (K tile j+2, V tile j+1). When
// the iteration's first chunk is pipelined they go out one 1 KiB load at a time
// inside its MFMA steps (2 * D/16 of them): item i at step 1 + i * SP. A wave
// waits at each such load until the memory pipeline takes it, so a burst of
// loads before the MFMAs stalls both waves of a SIMD together right after the
// tile barrier; spread out, each load costs about one issue slot. Otherwise
// (the chunk is the wave's last, or past it) `bulk` issues them all at once.
// ON = false issues nothing. GUARD: the workgroup has more waves than copy
// (FwdCfg::CW); the others skip their items.
template <int D, bool ON, bool PAD = false, bool GUARD = false, int W = FwdCfg<D>::WAVES>
struct FwdCopies {
    using PlanK = typename FwdCfg<D, PAD, W>::PlanK;
    using PlanV = typename FwdCfg<D, PAD, W>::PlanV;
    static constexpr int NK = PlanK::NT, NI = PlanK::NT + PlanV::NT, SP = 2 * (D / 16) / NI;
    static_assert(SP >= 1, "copy items fit the steps");
    const PlanK* pk;
    const PlanV* pv;
    BufRes rk, rv;
    uint32_t koff, voff;
    FA_LDS uint8_t* Kw;
    FA_LDS uint8_t* Vw;
    int w;
    template <int step>
    __device__ __forceinline__ void at() const {
        if constexpr (ON && step >= 1 && (step - 1) % SP == 0 && (step - 1) / SP < NI) {
            constexpr int i = (step - 1) / SP;
            const int ws = __builtin_amdgcn_readfirstlane(w);
            if constexpr (GUARD) {
                if (ws >= FwdCfg<D, PAD, W>::CW) return;
            }
            if constexpr (i < NK)
                pk->copy_one(i, rk, koff, Kw, ws);
            else
                pv->copy_one(i - NK, rv, voff, Vw, ws);
        }
    }
    __device__ __forceinline__ void bulk() const {
        if constexpr (ON) {
            if constexpr (GUARD) {
                if (__builtin_amdgcn_readfirstlane(w) >= FwdCfg<D, PAD, W>::CW) return;
            }
            pk->copy(rk, koff, Kw, w);
            pv->copy(rv, voff, Vw, w);
        }
    }
};

// One pipelined chunk, interleaved by hand. Each step is closed by a scheduling
// barrier, so the compiler keeps the order written here and only reorders
// inside a step.
//   phase 1 (DS steps): scores of the next chunk (one MFMA per K fragment, each
//            fragment read two steps ahead) with the exp / row sum / bf16 pack
//            of the current chunk; step r also reads V^T fragment r of the
//            current chunk, which phase 2 consumes at least DS steps later;
//   then the reference check (check_reference);
//   phase 2 (2*DB = DS steps): O^T += V^T P^T of the current chunk with
//            x = S*sl2 - m of the next chunk, in place.
// ka holds the first two K fragments of this chunk's score MFMAs on entry;
// phase 2 reads those of the following chunk into it (half hnn of tile Knn),
// so no chunk starts by waiting for its first LDS reads.
// cp issues its copy items at step r of phase 1 and step DS + f of phase 2.
template <int D, int H, class CP>
__device__ __forceinline__ void pipelined_chunk(const FA_LDS uint8_t* __restrict__ Kn, int kbase, int hn,
                                                const FA_LDS uint8_t* __restrict__ Knn, int hnn,
                                                const FA_LDS uint8_t* __restrict__ Vt, int vbase, int h,
                                                const u32x4 (&qf)[D / 16], f32x16& sc, f32x16& sn,
                                                float& m, float& l, f32x16& lsum, float sl2, f32x16 (&o)[D / 32],
                                                u32x4 (&ka)[2], const CP& cp, const u32x4& ones) {
    constexpr int DS = D / 16, DB = D / 32, NF = 2 * DB;
    // the 8 packs of the current chunk over the DS phase-1 steps: PPS per step,
    // on every PEVERY-th step (d = 256: one pack every other step)
    constexpr int PPS = DS <= 8 ? 8 / DS : 1;
    constexpr int PEVERY = DS <= 8 ? 1 : DS / 8;
    constexpr int EPS = 16 / NF;     // next-chunk registers turned into x per phase-2 step
    static_assert(NF == DS, "one V^T fragment read per phase-1 step");
    u32x4 pp[2];
    u32x4 vf[NF];
    float ls = 0.f;
    // The last chunk exponentiates the same x values; an empty asm statement
    // marks them as changed here, so the compiler cannot hoist this chunk's
    // exps above the branch between the two, out of the MFMA steps below.
#pragma unroll
    for (int i = 0; i < 16; i += 2) asm volatile("" : "+v"(sc[i]), "+v"(sc[i + 1]));
    sn = zero16();
    u32x4 a0 = ka[0];
    u32x4 a1 = ka[1];
    // Phase 1 (score MFMAs interleaved with the softmax) runs at a raised wave
    // priority, phase 2 at the normal one: when the two waves of a SIMD want to
    // issue at once, the one in phase 1 goes first. Measured on MI355X: about
    // 4% less forward time than equal priorities (any raised level alike, and
    // raising phase 2 instead gains half as much).
    __builtin_amdgcn_s_setprio(1);
    static_for<DS>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        u32x4 a2 = a1;
        if constexpr (r + 2 < DS) a2 = k_frag<D>(Kn, kbase, hn, r + 2);
        vf[r] = v_frag<D>(Vt, vbase, h, r);
        sn = mfma32(a0, qf[r], sn);
        if constexpr (r % PEVERY == 0) {
#pragma unroll
            for (int c = 0; c < PPS; ++c) exp_pack_one(sc, (r / PEVERY) * PPS + c, ls, pp);
        }
        cp.template at<r>();
        asm volatile("" : "+v"(ls));
        __builtin_amdgcn_sched_barrier(0);
        a0 = a1;
        a1 = a2;
    });
    check_reference<D>(sc, m, l, lsum, o, ls, pp);
    l += ls;
    __builtin_amdgcn_s_setprio(0);
    static_for<NF>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        o[f % DB] = mfma32(vf[f], pp[f / DB], o[f % DB]);
        if constexpr (f == 1 || f == NF - 1) lsum = mfma32(ones, pp[f == 1 ? 0 : 1], lsum);
#pragma unroll
        for (int c = 0; c < EPS; ++c) sn[f * EPS + c] = fmaf(sn[f * EPS + c], sl2, -m);
        if constexpr (f == 2 || f == 3) ka[f - 2] = k_frag<D>(Knn, kbase, hnn, f - 2);
        cp.template at<DS + f>();
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Per-wave state of the forward loop.
template <int D>
struct FwdState {
    u32x4 qf[D / 16];          // Q as the B operand
    f32x16 o[D / 32];          // O^T accumulators
    f32x16 sA, sB;             // x = S*sl2 - m of the current chunk / scores of the next (alternating)
    u32x4 ka[2];               // first two K fragments of the next pipelined chunk's score MFMAs
    float m, l;                // reference (log2 units), this lane's share of the row sum
    f32x16 lsum;               // ones * P^T: the row sum of the bf16 probabilities the P.V MFMA takes
    u32x4 ones;                // the all-ones A operand of the row-sum MFMA, held across the loop
};

// Sliding window: where a wave's keys start. A wave skips the chunks before
// its first one (firstc) and, at that chunk, takes as its reference the exact
// max over it and the next chunk: together they hold a visible key for every
// row of the wave (the first row's window starts in chunk firstc, so the last
// row's starts at most 31 keys later, and the diagonal chunk has each row's own
// key), while one chunk alone may hold none for some rows.
struct Window {
    int firstc;   // first chunk with a visible key for some row of the wave
    int win;      // window size
    int r0;       // the wave's first row
};

// Chunk c = 2j + H. sc holds its scores; the next chunk's go to sn.
// Kc: the K tile holding this chunk; Kn: the K tile holding the next chunk;
// Kr1: K tile j+1, which holds chunk c+2 (half H); Vt: this chunk's V tile.
// cp carries the iteration's copies (first chunk only).
template <int D, int H, bool CP, bool WIN, bool PAD, bool GUARD, int W>
__device__ __forceinline__ void fwd_chunk(FwdState<D>& st, int c, f32x16& sc, f32x16& sn,
                                          const FA_LDS uint8_t* __restrict__ Kc,
                                          const FA_LDS uint8_t* __restrict__ Kn,
                                          const FA_LDS uint8_t* __restrict__ Kr1,
                                          const FA_LDS uint8_t* __restrict__ Vt, int kbase, int vbase,
                                          bool causal, int qrow, int N, int lastc, float sl2, int hh,
                                          const FwdCopies<D, CP, PAD, GUARD, W>& cp, const Window& wd) {
    if (c > lastc) {
        cp.bulk();
        return;
    }
    if constexpr (WIN) {
        if (c < wd.firstc) {
            cp.bulk();
            return;
        }
        if (c == wd.firstc) {
            sc = scores<D>(Kc, kbase, H, st.qf);
            mask_scores<true>(sc, c * 32, qrow, N, true, hh, wd.win);
            float mx = chunk_max(sc, sl2);
            if (c < lastc) {
                f32x16 s1 = scores<D>(Kn, kbase, H ^ 1, st.qf);
                mask_scores<true>(s1, c * 32 + 32, qrow, N, true, hh, wd.win);
                mx = fmaxf(mx, chunk_max(s1, sl2));
                st.ka[0] = k_frag<D>(Kn, kbase, H ^ 1, 0);
                st.ka[1] = k_frag<D>(Kn, kbase, H ^ 1, 1);
            }
            st.m = mx;
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[i] = fmaf(sc[i], sl2, -st.m);
        }
    }
    if ((causal && c * 32 + 31 > qrow - (qrow & 31)) || (c * 32 + 32 > N))
        mask_scores<WIN>(sc, c * 32, qrow, N, causal, hh, wd.win);
    else if (WIN && c * 32 < wd.r0 + 32 - wd.win)
        mask_scores<true>(sc, c * 32, qrow, N, causal, hh, wd.win);
    if (c < lastc) {
        pipelined_chunk<D, H>(Kn, kbase, H ^ 1, Kr1, H, Vt, vbase, H, st.qf, sc, sn, st.m, st.l, st.lsum, sl2,
                              st.o, st.ka, cp, st.ones);
    } else {
        cp.bulk();
        softmax_pv<D>(Vt, vbase, H, sc, st.m, st.l, st.lsum, st.o);
    }
}

// One 64-key tile j: start the copies of K tile j+2 (into Kw) and V tile j+1
// (into Vw), then compute chunks 2j and 2j+1 from K tiles j, j+1 (Kr0, Kr1)
// and V tile j (Vr). All five buffers are distinct during the iteration; the
// __restrict__ qualifiers say so, which lets the compiler see that the LDS
// reads do not touch the LDS the in-flight global->LDS copies write, so it does
// not wait for those copies before each read.
template <int D, bool WIN, bool PAD, bool GUARD, int W>
__device__ __forceinline__ void fwd_iteration(FwdState<D>& st, int j, int nt,
                                              const typename FwdCfg<D, PAD, W>::PlanK& pk,
                                              const typename FwdCfg<D, PAD, W>::PlanV& pv, BufRes rk, BufRes rv,
                                              FA_LDS uint8_t* __restrict__ Kw,
                                              FA_LDS uint8_t* __restrict__ Vw,
                                              const FA_LDS uint8_t* __restrict__ Kr0,
                                              const FA_LDS uint8_t* __restrict__ Kr1,
                                              const FA_LDS uint8_t* __restrict__ Vr, int kbase, int vbase,
                                              bool valid, bool causal, int qrow, int N, int lastc,
                                              float sl2, int w, int lane, const Window& wd, int dr) {
    // dr: elements per row in the tensors (D, or fewer with PAD).
    // Tiles j + 1 and j + 2 may lie past the last one: their copies then read
    // past the resource (zeros) into buffers no chunk reads any more (those of
    // tiles j - 1 and j - 2).
    const FwdCopies<D, true, PAD, GUARD, W> cp{&pk, &pv, rk, rv, (uint32_t)(j + 2) * kBN * dr * 2,
                                            (uint32_t)(j + 1) * kBN * dr * 2, Kw, Vw, w};
    if (valid) {
        const int hh = lane >> 5;
        fwd_chunk<D, 0, true, WIN, PAD, GUARD, W>(st, 2 * j, st.sA, st.sB, Kr0, Kr0, Kr1, Vr, kbase, vbase, causal,
                                               qrow, N, lastc, sl2, hh, cp, wd);
        fwd_chunk<D, 1, false, WIN, PAD, GUARD, W>(st, 2 * j + 1, st.sB, st.sA, Kr0, Kr1, Kr1, Vr, kbase, vbase,
                                                causal, qrow, N, lastc, sl2, hh,
                                                FwdCopies<D, false, PAD, GUARD, W>{}, wd);
    } else {
        cp.bulk();
    }
}

// The causal flag is a run-time argument: it only changes the tile ranges and
// the mask of each wave's last chunk, so one instance per head dimension
// serves both cases.
template <int D, bool WIN, bool PAD, int W>
__global__ __launch_bounds__(64 * W, 1) void fwd_kernel(FwdParams p) {
    using C = FwdCfg<D, PAD, W>;
    constexpr bool GUARD = C::WAVES > C::CW;
    constexpr int DS = C::DS, DB = C::DB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];
    FA_LDS uint8_t* Ks = (FA_LDS uint8_t*)smem;          // 3 K tiles
    FA_LDS uint8_t* Vs = Ks + 3 * C::KT;                   // 2 V tiles

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5, g = lane >> 4;
    const bool causal = p.causal != 0;
    constexpr int kBM = C::BM;
    const int nqt = (p.N + kBM - 1) / kBM;
    int rank, bh;
    unmap_block(blockIdx.x, p.B * p.Hq, rank, bh);
    // Causal: the heaviest q-tiles first. The work of a tile depends only on
    // its index, so with packed sequences this order is heaviest first too.
    const int qt = causal ? nqt - 1 - rank : rank;
    if (p.cu_seqlens) {
        // Packed sequences differ in length, so an XCD must not own whole
        // sequences: read the index K/V-head-major, (hkv, b, g), so that each
        // XCD's block of indices is one K/V head (its G query heads) of every
        // sequence. The load is then even over the XCDs and a K/V head's
        // re-reads stay in one L2.
        const int g = bh % p.G, u = bh / p.G;
        const int bb = u % p.B, kv = u / p.B;
        bh = bb * p.Hq + kv * p.G + g;
    }
    const int b = bh / p.Hq, hq = bh - b * p.Hq, hkv = hq / p.G;
    int N = p.N;
    size_t qrow0 = (size_t)bh * N, kvrow0 = ((size_t)b * p.Hkv + hkv) * N;   // first row of the head
    if (p.cu_seqlens) {
        // packed: this sequence's rows; the bounds are clamped so that any
        // cu_seqlens keeps every access inside the [H, total] arrays
        const int s0 = min(max(p.cu_seqlens[b], 0), p.total);
        N = min(max(p.cu_seqlens[b + 1] - s0, 0), min(p.N, p.total - s0));
        qrow0 = (size_t)hq * p.total + s0;
        kvrow0 = (size_t)hkv * p.total + s0;
    }
    const int q0 = qt * kBM;
    if (q0 >= N) return;          // a q-tile past a shorter packed sequence (whole workgroup)
    // elements per row in the tensors: D, or with PAD the real head dimension
    // (a multiple of 8 below D); columns past it are zeros in every tile
    const int dr = PAD ? p.d : D;
    const uint16_t* Qg = p.q + qrow0 * dr;
    const uint16_t* Kg = p.k + kvrow0 * dr;
    const uint16_t* Vg = p.v + kvrow0 * dr;

    const int r0 = q0 + w * kWM;                 // this wave's first query row
    const int qrow = r0 + l32;                   // this lane's query row
    const int ntk = (N + kBN - 1) / kBN;
    const int nt = causal ? min(ntk, (q0 + kBM - 1) / kBN + 1) : ntk;
    // sliding window: the workgroup's first tile, and this wave's first chunk
    const int win = WIN ? p.window : 0;
    const int js = WIN ? max(0, q0 - win + 1) / kBN : 0;
    const Window wd{WIN ? max(0, r0 - win + 1) / 32 : 0, win, r0};
    const bool wave_valid = r0 < N;
    // last 32-key chunk this wave computes (causal: the diagonal chunk, keys r0 .. r0+31)
    const int nck = (N + 31) / 32;
    const int lastc = causal ? min(nck - 1, r0 / 32) : nck - 1;
    const float sl2 = p.scale_log2;
    const int kkey = swz_key<C::L>(l32);
    const int kbase = l32 * C::L + ((hh ^ (kkey & 1)) << 4) + ((kkey >> 1) << 5);
    const int vr = ((lane & 15) >> 2) + 4 * hh;
    const int vbase = vr * C::L + (tr_key<C::L>(vr) << 6) + ((g & 1) * 16 + 4 * (lane & 3)) * 2;

    FwdState<D> st;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
        st.qf[ds] = gload16(Qg + (size_t)qrow * dr + ds * 16 + hh * 8, qrow < N && (!PAD || ds * 16 + hh * 8 < dr));
#pragma unroll
    for (int db = 0; db < DB; ++db) st.o[db] = zero16();
    st.m = 0.f;
    st.l = 0.f;
    st.lsum = zero16();
    // Held in registers for the whole loop (the compiler would otherwise
    // rebuild the constant before every chunk's row-sum MFMAs: two moves per
    // chunk; 0.6% of the forward's time with the first-pair start of the row sum).
    st.ones = ones_bf16();
    asm volatile("" : "+v"(st.ones));

    // K and V through buffer resources covering the head's N rows: rows of a
    // ragged last tile past N read as zeros (their scores are masked).
    const BufRes rk = make_bufres(Kg, (uint32_t)N * dr * 2);
    const BufRes rv = make_bufres(Vg, (uint32_t)N * dr * 2);
    typename C::PlanK pk;
    typename C::PlanV pv;
    pk.init(w, lane, dr, dr);
    pv.init(w, lane, dr, dr);
    if (PAD) {   // the columns no copy writes must read as zeros
        lds_zero(Ks, C::LDS, tid, C::THREADS);
        __syncthreads();
    }

    // K tiles js, js+1 and V tile js before the loop (js = 0 without a window),
    // in the buffers the loop's index arithmetic expects for them.
    if (!GUARD || w < C::CW) {
        pk.copy(rk, (uint32_t)js * kBN * dr * 2, Ks + (js % 3) * C::KT, w);
        if (nt > js + 1) pk.copy(rk, (uint32_t)(js + 1) * kBN * dr * 2, Ks + ((js + 1) % 3) * C::KT, w);
        pv.copy(rv, (uint32_t)js * kBN * dr * 2, Vs + (js & 1) * C::VT, w);
    }
    wait_vmem();
    __syncthreads();

    if (!WIN && wave_valid) {
        // The first reference is chunk 0's exact (masked) max, so every row has
        // l >= 1 from then on; chunk 0 then holds x.
        st.sA = scores<D>(Ks, kbase, 0, st.qf);
        st.ka[0] = k_frag<D>(Ks, kbase, 1, 0);   // chunk 1's keys: tile 0, second half
        st.ka[1] = k_frag<D>(Ks, kbase, 1, 1);
        if ((causal && 31 > r0) || 32 > N) mask_scores(st.sA, 0, qrow, N, causal, hh);
        st.m = chunk_max(st.sA, sl2);
#pragma unroll
        for (int i = 0; i < 16; ++i) st.sA[i] = fmaf(st.sA[i], sl2, -st.m);
    }
    for (int j = js; j < nt; ++j) {
        fwd_iteration<D, WIN, PAD, GUARD, W>(st, j, nt, pk, pv, rk, rv, Ks + ((j + 2) % 3) * C::KT,
                                   Vs + ((j + 1) & 1) * C::VT, Ks + (j % 3) * C::KT, Ks + ((j + 1) % 3) * C::KT,
                                   Vs + (j & 1) * C::VT, kbase, vbase, wave_valid, causal, qrow, N, lastc, sl2, w,
                                   lane, wd, dr);
        wait_vmem();
        __syncthreads();
    }

    if (wave_valid && qrow < N) {
        uint16_t* Og = p.o + (qrow0 + qrow) * dr;
        // O is divided by the sum of the bf16 probabilities the P.V products
        // took, so each row's weights sum to one as used: a peaked row keeps
        // its dominant value's weight at 1 whatever that probability rounded
        // to (the reference need not sit at the row's max). The logsumexp
        // takes the fp32 sum.
        const float lt = st.l + swap_half(st.l);
        const float inv = 1.f / st.lsum[0];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 val;
                val[0] = pack_bf16(st.o[db][u * 4 + 0] * inv, st.o[db][u * 4 + 1] * inv);
                val[1] = pack_bf16(st.o[db][u * 4 + 2] * inv, st.o[db][u * 4 + 3] * inv);
                if (!PAD || db * 32 + u * 8 + hh * 4 < dr)
                    *reinterpret_cast<u32x2*>(Og + db * 32 + u * 8 + hh * 4) = val;
            }
        if (hh == 0) p.lse[qrow0 + qrow] = (st.m + __log2f(lt)) * kLn2;
    }
}

// Compute units of the current GPU, read once per device.
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Waves per workgroup. d = 64 takes 12 (three per SIMD; measured on MI355X:
// 10.8% less time on a 2 x 64-head, 16384-row causal forward, the same
// results bit for bit) unless the grid is small: 384-row workgroups then leave
// more of the last round of workgroups idle than the faster waves recover
// (4 x 16 heads of 2048 rows, causal: 4.6% more time; 2 x 16 heads of 4096
// rows, not causal: 19% more). The choice compares rounds of one workgroup per
// CU times rows per workgroup, a 12-wave row taking 0.9 of the time.
template <int D>
int fwd_waves(int B, int Hq, int N) {
    if constexpr (D == 128) {
        // 4-wave workgroups over 128 rows (two share a CU: 228-236 registers
        // and 80 KiB of LDS each) against 8-wave ones over 256 rows, measured
        // on MI355X: 9-17% less time on grids of fewer than two 256-row
        // workgroups per CU, 2-3% less on larger grids up to 16384 rows per
        // head. Longer rows on large grids keep 8 waves, which copy each K/V
        // tile for twice the rows (2.7% faster at 65536 rows).
        const long long g8 = (long long)B * Hq * ((N + 255) / 256);
        return (N <= 16384 || g8 < 2 * cu_count()) ? 4 : 8;
    } else if constexpr (D != 64) {
        return FwdCfg<D>::WAVES;
    } else {
        const long long bh = (long long)B * Hq, cu = cu_count();
        const long long r8 = (bh * ((N + 255) / 256) + cu - 1) / cu;
        const long long r12 = (bh * ((N + 383) / 384) + cu - 1) / cu;
        return r12 * 384 * 9 < r8 * 256 * 10 ? 12 : 8;
    }
}

template <int D, int W>
hipError_t launch_fwd_w(const FwdParams& p, hipStream_t stream) {
    using C = FwdCfg<D, false, W>;
    const int nqt = (p.N + C::BM - 1) / C::BM;
    const int grid = p.B * p.Hq * nqt;
    const bool pad = p.d != D;
    if (p.window > 0) {
        if (pad) hipLaunchKernelGGL((fwd_kernel<D, true, true, W>), dim3(grid), dim3(C::THREADS), 0, stream, p);
        else hipLaunchKernelGGL((fwd_kernel<D, true, false, W>), dim3(grid), dim3(C::THREADS), 0, stream, p);
    } else {
        if (pad) hipLaunchKernelGGL((fwd_kernel<D, false, true, W>), dim3(grid), dim3(C::THREADS), 0, stream, p);
        else hipLaunchKernelGGL((fwd_kernel<D, false, false, W>), dim3(grid), dim3(C::THREADS), 0, stream, p);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
    if constexpr (D == 64) {
        if (fwd_waves<D>(p.B, p.Hq, p.N) == 12) return launch_fwd_w<D, 12>(p, stream);
    }
    if constexpr (D == 128) {
        if (fwd_waves<D>(p.B, p.Hq, p.N) == 4) return launch_fwd_w<D, 4>(p, stream);
    }
    return launch_fwd_w<D, FwdCfg<D>::WAVES>(p, stream);
}

template <int D, int W>
Geometry geometry_w(int B, int Hq, int N) {
    using C = FwdCfg<D, false, W>;
    Geometry g;
    g.block_m = C::BM;
    g.block_n = kBN;
    g.threads = C::THREADS;
    g.grid = B * Hq * ((N + C::BM - 1) / C::BM);
    g.lds_bytes = C::LDS;
    return g;
}

template <int D>
Geometry geometry_t(int B, int Hq, int N) {
    if constexpr (D == 64) {
        if (fwd_waves<D>(B, Hq, N) == 12) return geometry_w<D, 12>(B, Hq, N);
    }
    if constexpr (D == 128) {
        if (fwd_waves<D>(B, Hq, N) == 4) return geometry_w<D, 4>(B, Hq, N);
    }
    return geometry_w<D, FwdCfg<D>::WAVES>(B, Hq, N);
}

}  // namespace

Geometry fwd_geometry(int B, int Hq, int N, int d, int causal) {
    (void)causal;
    const int D = padded_dim(d);
    return D == 256 ? geometry_t<256>(B, Hq, N) : D == 128 ? geometry_t<128>(B, Hq, N) : geometry_t<64>(B, Hq, N);
}

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
    const int D = padded_dim(p.d);
    if (D == 256) return launch_fwd_t<256>(p, stream);
    return D == 128 ? launch_fwd_t<128>(p, stream) : launch_fwd_t<64>(p, stream);
}

}  // namespace fa
