// fa_decode.hip -- a few query rows against a long key/value sequence (decode).
//
// What is computed: exact softmax attention, as in the forward pass, for the
// newest Nq tokens of a sequence whose Nk keys and values are cached. The
// mlapandio page "FlashAttention: IO-aware exact attention" points out that
// tiling does not help here ("Two notes", and the end of the naive-vs-flash
// diagram): one step reads the whole cache once and does little arithmetic per
// byte, so the memory read bounds it. The online softmax of that page ("Four
// ideas") still applies, and its logsumexp makes results over disjoint key
// ranges combinable: L = log sum_r exp(L_r), O = sum_r exp(L_r - L) O_r.
//
// gfx950 design:
//  * The bound is HBM bandwidth, so the kernel's job is to keep every CU
//    reading. The keys of each K/V head are split into ranges of whole 64-key
//    tiles, enough ranges that the grid holds about one workgroup per CU; a
//    workgroup streams its range once through a ring of LDS stages filled by
//    direct global->LDS loads (three tiles in flight while one is used: one
//    tile in flight left each CU waiting on memory latency) and leaves a
//    partial result. A second kernel merges the ranges by their logsumexp.
//  * The G = Hq / Hkv query heads that share a K/V head read it together: the
//    G * Nq rows of such a group (contiguous in q, o and lse) form the MFMA
//    row dimension, so the cache is read once per group, not once per head.
//  * A workgroup is 4 waves over up to 128 rows, one wave per 32-row block.
//    Groups of at most 64 rows (one or two blocks) leave waves over; then two
//    waves take each block, one per 32-key half of every tile, and fold their
//    results together through LDS at the end.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16),
//    from K tiles stored with XOR-swizzled 16-byte chunks, and P feeds
//    O^T += V^T P^T from its accumulator registers; V^T is read with
//    ds_read_b64_tr_b16 from quarter-swizzled tiles. These are the forward
//    kernel's tile layouts.
//  * The softmax keeps the exact running max per 32-key chunk and rescales O
//    and l only when some row's max rises: the arithmetic is far below the
//    memory time, so the forward's rarer reference moves buy nothing here.
#include <math.h>

#include <algorithm>
#include <climits>
#include <mutex>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int kDW = 4;                 // waves per workgroup
constexpr int kDThreads = 64 * kDW;
constexpr int kDBN = 64;               // keys per LDS tile
constexpr int kDRows = 128;            // query rows per workgroup
constexpr int kDTarget = 256;          // workgroups the split aims for (one per CU)
// Running max before any visible key. It is finite, so exp2(m_old - m_new)
// stays defined (it is 0 once a real score arrives), while masked scores
// (-inf) give exact zeros under it.
constexpr float kNoMax = -1e30f;

// PAD: tensor rows hold fewer than D values (a multiple of 8); tile columns
// past them stay zero (CopyPlanSwz with PAD). Every tile row keeps at least
// one source chunk, so each copy instruction still issues (with some lanes
// off) and the vmcnt accounting of the ring holds.
template <int D, bool PAD = false>
struct DecCfg {
    static constexpr int DS = D / 16, DB = D / 32, L = 2 * D;
    static constexpr int KT = kDBN * L;             // one K or V tile
    static constexpr int STAGE = 2 * KT;            // K tile, then V tile
    // ring stages: 128 KiB of LDS (d = 256: two stages of 64 KiB, one tile in
    // flight while one is used)
    static constexpr int NS = D == 256 ? 2 : D == 128 ? 4 : 8;
    static constexpr int LDS = NS * STAGE;
    using PlanK = CopyPlanSwz<L, kDBN, kDW, RowKey<L>, PAD>;
    using PlanV = CopyPlanSwz<L, kDBN, kDW, TrKey<L>, PAD>;
    static constexpr int LOADS = PlanK::NT + PlanV::NT;   // copy loads per wave per tile
    static_assert((NS - 2) * LOADS <= 63, "the loads of the tiles in flight fit vmcnt");
    // per-lane state a wave hands to its partner in the final fold
    static constexpr int FOLD = DB * 16 + 2;
    static_assert(2 * 64 * FOLD * 4 <= LDS, "the fold fits the tile memory");
};

template <int D>
struct DecWave {
    u32x4 qf[D / 16];          // Q as the B operand of the score MFMAs
    f32x16 o[D / 32];          // O^T accumulators
    float m;                   // running max of the row, log2 units
    float l;                   // this lane's share of the row sum
};

// LDS fragment reads. The tile ring keeps copies of later tiles in flight
// while a tile is read; the compiler cannot tell the stages apart across loop
// iterations and would wait for every copy before each read it sees. So the
// reads are asm statements, and the chunk waits for them itself (lgkmcnt).
__device__ __forceinline__ u32x4 lds_b128(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr_b64(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}
// s_waitcnt lgkmcnt(N), then the values read so far count as changed here, so
// no use of them moves above the wait.
template <int N, int C>
__device__ __forceinline__ void lds_wait(u32x4 (&f)[C]) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
#pragma unroll
    for (int i = 0; i < C; ++i) asm volatile("" : "+v"(f[i]));
}

// K fragment ds of a 32-key chunk (A operand of the score MFMAs: key l32,
// d = ds*16 + hh*8 .. +7). Kc is the chunk's first row in a swizzled tile;
// chunk offsets are multiples of 32 rows, which leave the XOR bits alone.
__device__ __forceinline__ u32x4 dec_k_frag(const FA_LDS uint8_t* Kc, int kbase, int ds) {
    return lds_b128(((uint32_t)(uintptr_t)Kc + (uint32_t)kbase) ^ (uint32_t)(ds << 5));
}

// V^T fragment f = (kc, db) of a chunk, read transposed in the key order of the
// P operand: slot hh*8 + t holds key kc*16 + (t/4)*8 + hh*4 + t%4.
template <int D, int F>
__device__ __forceinline__ u32x4 dec_v_frag(const FA_LDS uint8_t* Vc, int vbase) {
    constexpr int DB = D / 32, L = 2 * D;
    constexpr int kc = F / DB, db = F % DB;
    const uint32_t a = (((uint32_t)(uintptr_t)Vc + (uint32_t)vbase) ^ (uint32_t)(db << 6));
    return cat(lds_tr_b64<kc * 16 * L>(a), lds_tr_b64<kc * 16 * L + 8 * L>(a));
}

// The d = 256 instance reads through the compiler's own LDS loads instead.
// Its 48 fragment registers per chunk (128 registers) do not fit beside O
// while asm loads are in flight: an asm load's output counts as written when
// the statement ends, so the compiler may copy or reuse that register before
// the data lands. With the builtins the compiler places every wait itself.
// (With its two-stage ring, each wait for the copy in flight costs little.)
template <int D>
__device__ __forceinline__ u32x4 dec_k_frag_b(const FA_LDS uint8_t* Kc, int kbase, int ds) {
    const uint32_t a = ((uint32_t)(uintptr_t)Kc + (uint32_t)kbase) ^ (uint32_t)(ds << 5);
    return *reinterpret_cast<const FA_LDS u32x4*>((const FA_LDS uint8_t*)(uintptr_t)a);
}
template <int D, int F>
__device__ __forceinline__ u32x4 dec_v_frag_b(const FA_LDS uint8_t* Vc, int vbase) {
    constexpr int DB = D / 32, L = 2 * D;
    constexpr int kc = F / DB, db = F % DB;
    const uint32_t a = (((uint32_t)(uintptr_t)Vc + (uint32_t)vbase) ^ (uint32_t)(db << 6));
    const FA_LDS uint8_t* p = (const FA_LDS uint8_t*)(uintptr_t)a;
    return cat(lds_read_trb(p, kc * 16 * L), lds_read_trb(p, kc * 16 * L + 8 * L));
}

// One 32-key chunk starting at key0: scores, mask, online softmax, P.V.
// pos: the lane's row position (keys > pos are invisible); Nk: keys past it
// are invisible; lo: keys <= lo are invisible (a sliding window; INT_MIN
// without one); mask: whether any key of the chunk can be invisible.
template <int D>
__device__ __forceinline__ void dec_chunk(DecWave<D>& st, const FA_LDS uint8_t* __restrict__ Kc,
                                          const FA_LDS uint8_t* __restrict__ Vc, int kbase, int vbase,
                                          int key0, int Nk, int pos, int lo, bool mask, float sl2, int hh) {
    constexpr int DS = D / 16, DB = D / 32;
    // All fragment reads go out first: the K reads feed the score MFMAs, the
    // V^T reads land while the softmax runs.
    constexpr bool ASM = D != 256;
    u32x4 kf[DS], vf[2 * DB];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) kf[ds] = ASM ? dec_k_frag(Kc, kbase, ds) : dec_k_frag_b<D>(Kc, kbase, ds);
    static_for<2 * DB>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        if constexpr (ASM)
            vf[f] = dec_v_frag<D, f>(Vc, vbase);
        else
            vf[f] = dec_v_frag_b<D, f>(Vc, vbase);
    });
    // K done; the V^T reads (2 per fragment) may still be in flight
    if constexpr (ASM) lds_wait<(4 * DB < 15 ? 4 * DB : 15)>(kf);
    f32x16 s = zero16();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) s = mfma32(kf[ds], st.qf[ds], s);
    if (mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = key0 + (i >> 2) * 8 + hh * 4 + (i & 3);
            if (key >= Nk || key > pos || key <= lo) s[i] = -INFINITY;
        }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, swap_half(mx)) * sl2;       // sl2 > 0: the max commutes with the scale
    const float mn = fmaxf(st.m, mx);
    if (__ballot(mn > st.m)) {
        const float a = fast_exp2(st.m - mn);
        st.l *= a;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.o[db][i] *= a;
    }
    st.m = mn;
    // P = exp2(S*sl2 - m) <= 1, packed to bf16 as the B operand of O^T += V^T P^T:
    // registers kc*8 + 2t, +1 form k slot pair (2t, 2t+1) of 16-key half kc.
    u32x4 pp[2];
    float ls = 0.f;
#pragma unroll
    for (int pi = 0; pi < 8; ++pi) {
        const int kc = pi >> 2, t = pi & 3, i = kc * 8 + 2 * t;
        const float p0 = fast_exp2(fmaf(s[i], sl2, -mn));
        const float p1 = fast_exp2(fmaf(s[i + 1], sl2, -mn));
        ls += p0 + p1;
        pp[kc][t] = pack_bf16(p0, p1);
    }
    st.l += ls;
    if constexpr (ASM) lds_wait<0>(vf);
#pragma unroll
    for (int f = 0; f < 2 * DB; ++f) st.o[f % DB] = mfma32(vf[f], pp[f / DB], st.o[f % DB]);
}

// s_waitcnt vmcnt(ahead * LOADS): this wave's copies of all but the `ahead`
// most recent tiles have landed (loads complete in order for vmcnt).
template <int LOADS, int NS>
__device__ __forceinline__ void wait_tiles(int ahead) {
    static_for<NS - 1>([&](auto ac) {
        constexpr int A = decltype(ac)::value;
        if (ahead == A) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(A * LOADS));
    });
}

// One tile iteration: start the copy of a later tile (when there is one) into
// stage W, then use the current tile from stage R.
template <int D, bool PAD>
__device__ __forceinline__ void dec_iteration(DecWave<D>& st, const typename DecCfg<D, PAD>::PlanK& pk,
                                              const typename DecCfg<D, PAD>::PlanV& pv, BufRes rk, BufRes rv,
                                              bool copy_next, uint32_t noff, FA_LDS uint8_t* __restrict__ W,
                                              const FA_LDS uint8_t* __restrict__ R, int w, bool active,
                                              int h0, int h1, int key0, int Nk, int pos, int lo, int mfrom,
                                              int mto, float sl2, int kbase, int vbase, int hh) {
    using C = DecCfg<D>;
    if (copy_next) {
        pk.copy(rk, noff, W, w);
        pv.copy(rv, noff, W + C::KT, w);
    }
    if (!active) return;
    for (int h = h0; h < h1; ++h) {
        const int kc = key0 + 32 * h;
        if (kc >= Nk) break;
        dec_chunk<D>(st, R + h * 32 * C::L, R + C::KT + h * 32 * C::L, kbase, vbase, kc, Nk, pos, lo,
                     kc + 32 > mfrom || kc <= mto, sl2, hh);
    }
}

template <int D, bool PAD>
__global__ __launch_bounds__(kDThreads, 1) void decode_split_kernel(DecParams p) {
    using C = DecCfg<D, PAD>;
    constexpr int DB = C::DB, NS = C::NS;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];
    FA_LDS uint8_t* ring = (FA_LDS uint8_t*)smem;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5, g = lane >> 4;
    const int split = blockIdx.x % p.nsplit;
    const int rest = blockIdx.x / p.nsplit;
    const int rblk = rest % p.nrb, grp = rest / p.nrb;
    const int M = p.M, Nk = p.Nk;
    // keys in use for this batch entry: the first L of its Nk cache rows
    int L = Nk;
    if (p.seqlens_k) L = min(max(p.seqlens_k[grp / p.Hkv], 0), Nk);

    // waves -> (32-row block, key half)
    const int rows_here = min(kDRows, M - rblk * kDRows);
    const int nb = (rows_here + 31) / 32;
    int rb, kw;
    bool active;
    if (p.pair) {                 // nb is 1 or 2: two waves per block
        active = w < 2 * nb;
        rb = w % nb;
        kw = w / nb;
    } else {
        active = w < nb;
        rb = w;
        kw = 0;
    }
    const int h0 = p.pair ? kw : 0, h1 = p.pair ? kw + 1 : 2;
    const int r = rblk * kDRows + rb * 32 + l32;          // this lane's row in the group
    const bool row_ok = active && r < M;
    // causal: row r is token L - Nq + (r % Nq); keys after it are invisible
    // (a negative position: the row sees no key)
    const int pos = (p.causal && row_ok) ? L - p.Nq + r % p.Nq : 0x7fffffff;
    // sliding window: keys at or before lo are invisible to this row
    const int lo = (p.window > 0 && row_ok) ? pos - p.window : INT_MIN;
    // chunks ending after mfrom, or starting at or before mto, may hold
    // invisible keys (mto: the last row's window start - 1)
    const int mfrom = p.causal ? L - p.Nq + 1 : L;
    const int mto = p.window > 0 ? L - 1 - p.window : INT_MIN;

    // this range's tiles that hold keys in use (none: the range reports an
    // empty result). With a window the ranges start at the tile of the first
    // row's first visible key, so earlier tiles are never read.
    const int ntile = (L + kDBN - 1) / kDBN;
    const int tf = p.window > 0 ? max(0, L - p.Nq - p.window + 1) / kDBN : 0;
    const int t0 = tf + split * p.tps;
    const int nt = min(p.tps, ntile - t0);

    const float sl2 = p.scale_log2;
    const int kkey = swz_key<C::L>(l32);
    const int kbase = l32 * C::L + ((hh ^ (kkey & 1)) << 4) + ((kkey >> 1) << 5);
    const int vr = ((lane & 15) >> 2) + 4 * hh;
    const int vbase = vr * C::L + (tr_key<C::L>(vr) << 6) + ((g & 1) * 16 + 4 * (lane & 3)) * 2;

    DecWave<D> st;
    // elements per row in the tensors: D, or with PAD the real head dimension
    const int dr = PAD ? p.d : D;
    // Q through a buffer resource over this workgroup's rows: rows past the
    // group's M (and lanes of idle waves) read zeros, with no branch; so do
    // the padding columns (an offset past the resource, which is < 2^17 bytes).
    const int rq = active ? r : M;
    const BufRes rq_res = make_bufres(p.q + ((size_t)grp * M + rblk * kDRows) * dr, (uint32_t)rows_here * dr * 2);
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
        const int col = ds * 16 + hh * 8;
        const uint32_t qoff = (!PAD || col < dr) ? (uint32_t)((rq - rblk * kDRows) * dr + col) * 2u : 0x7FFFFFF0u;
        st.qf[ds] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq_res, qoff, 0, 0));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) st.o[db] = zero16();
    st.m = kNoMax;
    st.l = 0.f;

    // K and V through buffer resources over the group's Nk rows: rows of a
    // ragged last tile past Nk read as zeros (and are masked).
    const uint16_t* Kg = p.k + (size_t)grp * Nk * dr;
    const uint16_t* Vg = p.v + (size_t)grp * Nk * dr;
    const BufRes rk = make_bufres(Kg, (uint32_t)Nk * dr * 2);
    const BufRes rv = make_bufres(Vg, (uint32_t)Nk * dr * 2);
    typename C::PlanK pk;
    typename C::PlanV pv;
    pk.init(w, lane, dr, dr);
    pv.init(w, lane, dr, dr);
    const uint32_t kTileBytes = kDBN * dr * 2;
    if (PAD) {   // the columns no copy writes must read as zeros
        lds_zero(ring, C::LDS, tid, kDThreads);
        __syncthreads();
    }
    if (nt > 0) {
    // Ring of NS stages: tiles j+1 .. j+NS-2 stay in flight while tile j is
    // used, and tile j+NS-1 goes into the stage tile j-1 used. The first NS-1
    // copies are issued unconditionally (a range shorter than that re-copies
    // its last tile into stages no iteration reads), so the number of loads
    // behind the Q loads is fixed and the wait for Q below is exact.
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) {
        const uint32_t off = (uint32_t)(t0 + min(t, nt - 1)) * kTileBytes;
        pk.copy(rk, off, ring + t * C::STAGE, w);
        pv.copy(rv, off, ring + t * C::STAGE + C::KT, w);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 1) * C::LOADS));
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) asm volatile("" : "+v"(st.qf[ds]));
    for (int j = 0; j < nt; ++j) {
        // tile j has landed for every wave; every wave is done with tile j-1
        wait_tiles<C::LOADS, NS>(min(NS - 2, nt - 1 - j));
        // A plain s_barrier: the barrier intrinsic would make the compiler wait
        // for every copy in flight first. The LDS reads are asm statements that
        // wait for themselves, and the memory clobber keeps the copies in order.
        asm volatile("s_barrier" ::: "memory");
        const int jn = j + NS - 1;
        dec_iteration<D, PAD>(st, pk, pv, rk, rv, jn < nt, (uint32_t)(t0 + jn) * kTileBytes,
                         ring + (jn % NS) * C::STAGE, ring + (j % NS) * C::STAGE, w, active, h0, h1,
                         (t0 + j) * kDBN, L, pos, lo, mfrom, mto, sl2, kbase, vbase, hh);
    }
    }

    if (p.pair) {
        // Fold the second wave of each row block into the first: lane-private
        // round trip through the (now unused) tile memory.
        __syncthreads();
        float* fold = (float*)smem;
        if (active && kw == 1) {
            float* dst = fold + (size_t)(rb * 64 + lane) * C::FOLD;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) dst[db * 16 + i] = st.o[db][i];
            dst[DB * 16] = st.m;
            dst[DB * 16 + 1] = st.l;
        }
        __syncthreads();
        if (active && kw == 0) {
            const float* src = fold + (size_t)(rb * 64 + lane) * C::FOLD;
            const float m1 = src[DB * 16], l1 = src[DB * 16 + 1];
            const float mm = fmaxf(st.m, m1);
            const float a0 = fast_exp2(st.m - mm), a1 = fast_exp2(m1 - mm);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) st.o[db][i] = st.o[db][i] * a0 + src[db * 16 + i] * a1;
            st.l = st.l * a0 + l1 * a1;
            st.m = mm;
        }
        if (kw == 1) active = false;
    }

    if (!active) return;
    const float lt = st.l + swap_half(st.l);
    if (r >= M) return;
    if (p.nsplit == 1) {
        // a single range: the final result (a row that sees no key gets
        // O = 0 and LSE = -inf)
        uint16_t* Og = p.o + ((size_t)grp * M + r) * dr;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
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
        if (hh == 0) p.lse[(size_t)grp * M + r] = lt > 0.f ? (st.m + __log2f(lt)) * kLn2 : -INFINITY;
        return;
    }
    // partial result of this range: normalised O and log2 of the sum (a row
    // that saw no key here gets O = 0 and -inf, weight 0 in the merge)
    const size_t slot = ((size_t)grp * p.nsplit + split) * M + r;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* Pg = p.part_o + slot * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f32x4 val;
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = st.o[db][u * 4 + e] * inv;
            *reinterpret_cast<f32x4*>(Pg + db * 32 + u * 8 + hh * 4) = val;
        }
    if (hh == 0) p.part_lse[slot] = lt > 0.f ? st.m + __log2f(lt) : -INFINITY;
}

// Merge of the key ranges: one workgroup per query row. With L_r the ranges'
// log2 sums and mx = max_r L_r, weights w_r = exp2(L_r - mx); O = sum w_r O_r /
// sum w_r and LSE = (mx + log2 sum w_r) * ln 2. A row with no finite L_r saw
// no key at all: O = 0 and LSE = -inf. Thread t takes 4 output values (column c) of the
// ranges r = g, g + SG, ... (group g): the loads of all ranges go out
// together instead of one range after another.
template <int D, bool PAD>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecParams p) {
    constexpr int C4 = D / 4;             // 4-value columns of a row
    constexpr int SG = 256 / C4;          // range groups
    __shared__ f32x4 part[256];
    __shared__ float wpart[SG];
    __shared__ float wmax[4];
    const int t = threadIdx.x, c = t % C4, g = t / C4;
    const long long row = blockIdx.x;
    const int M = p.M, S = p.nsplit;
    const int grp = (int)(row / M), r = (int)(row - (long long)grp * M);
    const float* pl = p.part_lse + (size_t)grp * S * M + r;
    const float* po = p.part_o + ((size_t)grp * S * M + r) * D + c * 4;
    float mx = -INFINITY;
    for (int s = t; s < S; s += 256) mx = fmaxf(mx, pl[(size_t)s * M]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((t & 63) == 0) wmax[t >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float mref = mx == -INFINITY ? 0.f : mx;       // all weights 0 then, not NaN
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
#pragma unroll 4
    for (int s = g; s < S; s += SG) {
        const float wt = fast_exp2(pl[(size_t)s * M] - mref);
        const f32x4 x = *reinterpret_cast<const f32x4*>(po + (size_t)s * M * D);
        wsum += wt;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(wt, x[e], acc[e]);
    }
    part[t] = acc;
    if (c == 0) wpart[g] = wsum;
    __syncthreads();
    if (g != 0) return;
#pragma unroll
    for (int k = 1; k < SG; ++k) {
        const f32x4 x = part[k * C4 + c];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += x[e];
    }
    float wt = 0.f;
#pragma unroll
    for (int k = 0; k < SG; ++k) wt += wpart[k];
    const float inv = wt > 0.f ? 1.f / wt : 0.f;
    u32x2 val;
    val[0] = pack_bf16(acc[0] * inv, acc[1] * inv);
    val[1] = pack_bf16(acc[2] * inv, acc[3] * inv);
    const int dr = PAD ? p.d : D;
    if (!PAD || c * 4 < dr) *reinterpret_cast<u32x2*>(p.o + (size_t)row * dr + c * 4) = val;
    if (c == 0) p.lse[row] = wt > 0.f ? (mx + __log2f(wt)) * kLn2 : -INFINITY;
}

template <int D, bool PAD>
hipError_t launch_decode_t(const DecParams& p, hipStream_t stream) {
    const long long grid = (long long)p.B * p.Hkv * p.nrb * p.nsplit;
    hipLaunchKernelGGL((decode_split_kernel<D, PAD>), dim3((unsigned)grid), dim3(kDThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    const long long rows = (long long)p.B * p.Hq * p.Nq;
    hipLaunchKernelGGL((decode_merge_kernel<D, PAD>), dim3((unsigned)rows), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecParams& p, hipStream_t stream) {
    return p.d == D ? launch_decode_t<D, false>(p, stream) : launch_decode_t<D, true>(p, stream);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

DecPlan dec_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int window) {
    DecPlan pl{};
    const int G = Hq / Hkv;
    pl.M = G * Nq;
    pl.nrb = (pl.M + kDRows - 1) / kDRows;
    pl.pair = pl.M <= 64 ? 1 : 0;
    // tiles a row group can need: all of them, or with a window the tiles
    // from the first row's first visible key to the end of the cache
    long long ntile = (Nk + kDBN - 1) / kDBN;
    if (window > 0) ntile = std::min(ntile, ((long long)Nq + window - 1 + kDBN - 1) / kDBN + 1);
    const long long base = (long long)B * Hkv * pl.nrb;
    long long tps = (ntile * base + kDTarget - 1) / kDTarget;
    tps = tps < 1 ? 1 : (tps > ntile ? ntile : tps);
    pl.tps = (int)tps;
    pl.nsplit = (int)((ntile + tps - 1) / tps);
    if (pl.nsplit > 1) {
        const size_t n = (size_t)B * Hkv * pl.nsplit * pl.M;
        pl.part_lse = 0;
        pl.part_o = align256(n * 4);
        pl.total = pl.part_o + align256(n * (size_t)padded_dim(d) * 4);   // partial O rows hold D values
    }
    return pl;
}

hipError_t launch_decode(const DecParams& p, hipStream_t stream) {
    const int D = padded_dim(p.d);
    if (D == 256) return launch_decode_d<256>(p, stream);
    return D == 128 ? launch_decode_d<128>(p, stream) : launch_decode_d<64>(p, stream);
}

// ---------------------------------------------------------------- static scratch
// Device memory for the per-range partial results of callers that cannot
// allocate (flash_attn_decode_noalloc). Every GPU the library runs on holds
// its own copy until the process ends. In host code `scratch` names a host-side
// stand-in, not the device array: kernels and copies only ever get the address
// that hipGetSymbolAddress returns for the current device.
namespace {
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void** out) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    // once per device, with that device current (it is: hipGetDevice above)
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    if (!g_scratch_ptr[dev]) return hipErrorInvalidSymbol;
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace fa
