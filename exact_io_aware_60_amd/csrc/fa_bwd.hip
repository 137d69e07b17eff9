// fa_bwd.hip -- backward pass of exact attention on gfx950.
//
// Method: the forward keeps only O and one logsumexp per query row; the
// backward rebuilds every probability from them, P_ij = exp(S_ij - LSE_i),
// instead of reading a stored score matrix (mlapandio "FlashAttention: IO-aware
// exact attention", "Four ideas", recomputation item; techtrendtracker "Flash
// Attention: memory-efficient transformers", "Recomputation in the Backward
// Pass"). The gradient formulas are the chain rule of softmax attention for the
// loss sum(dO * O):
//   D_i   = sum_c dO_ic O_ic                 (row dot)
//   dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij q_i   (dK/dV kernel)
//   dQ_i  = scale sum_j dS_ij k_j                              (dQ kernel)
// dK and dV sum over the query heads that share the K/V head.
//
// Precision. The four products that take P or dS as an operand run on fp16
// MFMA operands. fp16 keeps 11 significant bits where bf16 keeps 8, at the same
// MFMA rate, so rounding P and dS costs 8x less accuracy. A first kernel finds
// max |x| of q, k, v and dout. The preparation kernel then writes fp16 copies
// of them scaled by powers of two (max |x| * scale lies in [2^13, 2^14)). A
// bf16 value x converts exactly when |x| >= 2^-30 max |x| of its tensor (its
// scaled value then keeps 8 significant bits above fp16's subnormal spacing
// 2^-24); smaller values become fp16 subnormals or zero, off by at most
// 2^-38 max |x|. It also derives a scale for dS from the bound
// |dS_ij| <= 2 d max|dO| max|V|, so dS values far below that bound (for
// example every dS of a head whose dO is 2^-20 times another head's) lose
// relative precision in the same way; their absolute error stays below
// 2^-25 times the bound's scale. The scales are undone in fp32 in each
// epilogue.
//
// The row dot D. The forward stores O in bf16, and its P.V product rounds P to
// bf16, so a D formed from the stored O is off by about one bf16 ulp of O per
// element. dS = P (dP - D) turns that into dQ and dK errors of several 1e-2
// when the softmax is peaked. The dQ kernel therefore also sums the exact row
// dot D'_i = sum_j P_ij dP_ij from the probabilities it rebuilds, together
// with PK_i = sum_j P_ij k_j. dS is linear in D, so dQ computed with the
// approximate D plus (D - D') PK equals dQ computed with D'. The dK/dV kernel
// runs after it and uses D'. (Forming D' instead as D + sum_j dS_ij, one
// v_dot2_f32_f16 per packed dS pair in place of one FMA per element, measured
// 3.7% slower: each dot2 waits for the packed product just before it.)
//
// Two passes, no atomics: the dQ kernel owns a block of query rows and walks the
// keys; the dK/dV kernel owns a block of keys and walks the query rows. Each
// output element is written once, so results are bit-reproducible. The cost is
// recomputing S and dP in the dQ pass.
//
// Operand layouts. All products use v_mfma_f32_32x32x16_f16 (layouts in
// fa_device.h), and every operand is read from LDS with conflict-free 16-byte
// row reads (ds_read_b128 delivers about 220 B/clk per CU on MI355X, the
// transposing ds_read_b64_tr_b16 at most about 145 and only 70 with four
// waves). The contractions over query rows (dV, dK) and over keys (dQ) need an
// operand with consecutive rows at a fixed column, so the preparation kernel
// writes transposed copies of q, dout and k ([d][rows] per head). Their rows
// are stored in the k order of the operand they meet: the fp32 accumulator of
// S or dP, reused in register order as the other operand, holds in slot s of
// lane half hh the row 16c + 8(s/4) + 4hh + s%4, so position p of every group
// of 16 holds row p with bits 2 and 3 swapped. All copies are padded to a
// multiple of 128 rows with zero data, D = 0 and LSE = +inf, so no tile reads
// past an array and padding rows carry P = 0.
//
// Data flow at d = 128 on grids of 512 or more such workgroups (eight waves per
// workgroup, two per SIMD; smaller grids run the four-wave form below):
//  * dK/dV: a workgroup owns 256 keys, 32 per wave. K stays in registers as
//    the B operand of S = Q K^T; V, the B operand of dP = dO V^T, sits in LDS
//    (the workgroup's 256 rows), since two waves per SIMD leave each at most
//    256 registers. Each step streams 32 query rows of one query head of the
//    group (Q and dO rows, their transposes, LSE and D) through two LDS
//    stages. The steps walk the row blocks from the last one down, all heads
//    of the group per block, so workgroups running side by side read the same
//    rows from L2. S and dP leave one key per lane; P and dS in fp16 feed
//    dV^T += dO^T P and dK^T += Q^T dS.
//  * dQ: a workgroup owns 256 query rows, 32 per wave. Q stays in registers,
//    dO sits in LDS; tiles of 32 keys (K and V rows, K^T) stream through two
//    stages. S^T = K Q^T and dP^T = V dO^T leave one query row per lane; P^T
//    and dS^T in fp16 feed dQ^T += K^T dS^T and PK^T += K^T P^T.
// In both, a step's MFMAs run in four phases (the two score products, then
// the two gradient products), with the exp / dS work interleaved by hand
// between them and the next step's copy spread over the slots; the other wave
// of the SIMD fills the gaps. Per MFMA a step copies half the bytes of a
// four-wave workgroup over 128 keys or rows.
// Data flow at d <= 64, and at d = 128 on small grids (four waves per
// workgroup, one per SIMD in the workgroup; two workgroups per CU at d <= 64):
//  * dQ: a workgroup owns 128 query rows, 32 per wave, whose Q and dO rows
//    stay in registers as MFMA operands. Tiles of 64 keys (K and V rows, K^T)
//    stream through three LDS stages. The loop is software-pipelined across
//    tiles: the MFMAs of tile j's scores run beside the dQ products of tile
//    j-1, and the exp / dS work of tile j spreads over the slots in between.
//  * dK/dV: a workgroup owns 128 keys, 32 per wave, held in registers as MFMA
//    operands. Each step streams 64 query rows of one query head of the group
//    through two LDS stages, in the order above. Inside a step the exp / dS
//    work is interleaved by hand with the MFMAs.
// (d = 256 splits the accumulated columns over two workgroups; see below.)
// Only tiles that cross the causal diagonal (and, in dQ, the ragged last key
// tile) take an element-wise mask, on a plain unpipelined path.
#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int kThreads = 256;   // 4 waves

// Per-lane fragment addresses in a stage of either backward kernel. Row tiles
// ([64 x D], padded rows of SR bytes) are read at one lane base plus constants:
// row(b, ds) is row b*32 + l32, d = ds*16 + hh*8 ... Transposed tiles
// ([D x 64]) are read through T (Swz128 or PadRows): t.read(tile, b*32, c) is
// d row b*32 + l32, positions c*16 + hh*8 ... Swizzled row tiles would need a
// table of eight lane offsets, which the register budget of these kernels does
// not have.
template <int SR, class T>
struct LaneAddr {
    int rbase;          // l32 * SR + hh * 16
    T t;
    __device__ __forceinline__ void init(int l32, int hh) {
        rbase = l32 * SR + hh * 16;
        t.init(l32, hh);
    }
    __device__ __forceinline__ int row(int b, int ds) const { return rbase + b * 32 * SR + ds * 32; }
};

// Keeps a value in place: the compiler may not move its computation across a
// scheduling barrier that follows.
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

// Bounded masks (sliding window or packed sequences), as the first key a row
// sees and the first row that no longer sees a key. Window W: rows r see keys
// r - W + 1 .. r. Packed sequences: the keys of the row's own sequence up to
// the row. Offsets are clamped to [0, N], so any cu_seqlens keeps every bound
// inside the arrays; rows and keys at or past N get N.
struct Bounds {
    const int* cu;   // packed offsets (nseq + 1 entries), or null for a window
    int nseq, win, N;
    // index s with cu[s] <= x < cu[s+1] (the last such s when sequences are empty)
    __device__ __forceinline__ int seq_of(int x) const {
        int lo = 0, hi = nseq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (min(max(cu[mid], 0), N) <= x) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    }
    __device__ __forceinline__ int first_key(int r) const {      // of row r
        if (!cu) return r - win + 1;
        return r >= N ? N : min(max(cu[seq_of(r)], 0), N);
    }
    __device__ __forceinline__ int row_end(int k) const {        // first row past key k's reach
        if (!cu) return k + win;
        return k >= N ? N : min(max(cu[seq_of(k) + 1], 0), N);
    }
};

// Workgroup id -> (rank, unit). Workgroups are handed to the 8 XCDs
// round-robin; when the unit count is a multiple of 8, each XCD gets a
// contiguous block of units and walks them in rank order, so the units that
// share K/V (or Q/dO) rows share one L2.
__device__ __forceinline__ void unmap_block(int bid, int nunits, int& rank, int& unit) {
    if ((nunits & 7) == 0) {
        const int x = bid & 7, r = bid >> 3, upx = nunits >> 3;
        rank = r / upx;
        unit = x * upx + (r - rank * upx);
    } else {
        rank = bid / nunits;
        unit = bid - rank * nunits;
    }
}

// The same hand-out, unit-major: each XCD takes its units one after another,
// all ranks of a unit in rank order, so the workgroups an XCD runs side by
// side belong to one unit and read the same rows through its L2.
__device__ __forceinline__ void unmap_block_unit_major(int bid, int nunits, int nranks, int& rank, int& unit) {
    if ((nunits & 7) == 0) {
        const int x = bid & 7, r = bid >> 3, upx = nunits >> 3;
        const int u = r / nranks;
        rank = r - u * nranks;
        unit = x * upx + u;
    } else {
        unmap_block(bid, nunits, rank, unit);
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }


// ---------------------------------------------------------------- preparation
// Tensors the preparation kernels read, in this order: q, k, v, dout.
__device__ __forceinline__ void prep_tensor(const BwdParams& p, int t, const uint16_t*& src,
                                            uint16_t*& dst, long long& chunks) {
    const long long nq = (long long)p.B * p.Hq * p.N * p.d / 8;
    const long long nk = (long long)p.B * p.Hkv * p.N * p.d / 8;
    if (t == 0) { src = p.q; dst = p.q16; chunks = nq; }
    else if (t == 1) { src = p.k; dst = p.k16; chunks = nk; }
    else if (t == 2) { src = p.v; dst = p.v16; chunks = nk; }
    else { src = p.dout; dst = p.do16; chunks = nq; }
}

__device__ __forceinline__ uint32_t max_mag8(const u32x4& x) {
    uint32_t m = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        m = max(m, x[t] & 0x7FFFu);
        m = max(m, (x[t] >> 16) & 0x7FFFu);
    }
    return m;
}

// Max over the workgroup of a per-thread value; every thread gets the result.
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = max(max(red[0], red[1]), max(red[2], red[3]));
    return v;
}

// Partial max |x| (as bf16 magnitude bits: for finite values the integer order
// of the low 15 bits is the order of |x|) of q, k, v and dout per workgroup.
__global__ __launch_bounds__(kThreads) void bwd_max_kernel(BwdParams p) {
    __shared__ uint32_t red[4];
    for (int t = 0; t < 4; ++t) {
        const uint16_t* src;
        uint16_t* dst;
        long long chunks;
        prep_tensor(p, t, src, dst, chunks);
        uint32_t m = 0;
        for (long long c = (long long)blockIdx.x * kThreads + threadIdx.x; c < chunks;
             c += (long long)gridDim.x * kThreads)
            m = max(m, max_mag8(*reinterpret_cast<const u32x4*>(src + c * 8)));
        m = block_max(m, red);
        if (threadIdx.x == 0) p.part[t * p.npart + blockIdx.x] = m;
    }
}

// Power-of-two exponent s such that max * 2^s lies in [2^13, 2^14); 0 for max = 0.
__device__ __forceinline__ int scale_exp(uint32_t mag_bits) {
    if (mag_bits == 0) return 0;
    int e;
    frexpf(__uint_as_float(mag_bits << 16), &e);   // max = f * 2^e, 0.5 <= f < 1
    return 14 - e;
}

// Position of row r of a group of 16 in a transposed copy, and back (bits 2 and
// 3 swapped: the map is its own inverse). Bits above 3 pass through.
__device__ __forceinline__ int perm16(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Rows [row0, row0 + 64) of one head: the fp16 copy (x * f) and, when dstT is
// set, the transposed copy of the same rows. Rows >= N are written as zeros,
// and so are columns >= dr: source rows hold dr values (a multiple of 8, at
// most D), the copies D.
// `tr` is a [64][D/2 + 1]-word LDS buffer (odd row pitch: the column reads of
// the transpose hit distinct banks).
template <int D>
__device__ __forceinline__ void conv_tile(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                          uint16_t* __restrict__ dstT, int row0, int N, int Np, float f,
                                          uint32_t* tr, int dr) {
    constexpr int CPR = D / 8;
    constexpr int CH = 64 * CPR / kThreads;
    constexpr int TW = D / 2 + 1;
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
        const int chunk = u * kThreads + tid;
        const int r = chunk / CPR, c = chunk % CPR;
        const int row = row0 + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row < N && c * 8 < dr) x = *reinterpret_cast<const u32x4*>(src + (size_t)row * dr + c * 8);
        u32x4 y;
#pragma unroll
        for (int t = 0; t < 4; ++t) y[t] = pack_f16(bf16_lo(x[t]) * f, bf16_hi(x[t]) * f);
        *reinterpret_cast<u32x4*>(dst + (size_t)row * D + c * 8) = y;
        if (dstT) {
#pragma unroll
            for (int t = 0; t < 4; ++t) tr[r * TW + c * 4 + t] = y[t];
        }
    }
    if (dstT) {   // uniform over the workgroup
        __syncthreads();
        // [D][64] block: 8 chunks of 16 bytes per d row; chunk cc holds positions
        // cc*8 .. cc*8+7, i.e. rows perm16(position).
        constexpr int TCH = D * 8 / kThreads;
#pragma unroll
        for (int u = 0; u < TCH; ++u) {
            const int idx = u * kThreads + tid;
            const int dd = idx >> 3, cc = idx & 7;
            const int sh = (dd & 1) * 16;
            u32x4 z;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t lo = tr[perm16(cc * 8 + 2 * t) * TW + (dd >> 1)] >> sh;
                const uint32_t hi = tr[perm16(cc * 8 + 2 * t + 1) * TW + (dd >> 1)] >> sh;
                z[t] = (lo & 0xFFFFu) | (hi << 16);
            }
            *reinterpret_cast<u32x4*>(dstT + (size_t)dd * Np + row0 + cc * 8) = z;
        }
        __syncthreads();
    }
}

// Scales; fp16 copies (row and transposed); per padded row D * 2^sS and
// LSE * log2(e) (0 and +inf on padding rows).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdParams p) {
    __shared__ uint32_t red[4];
    __shared__ uint32_t tr[64 * (D / 2 + 1)];
    int sx[4];
    uint32_t mags[4];
    for (int t = 0; t < 4; ++t) {
        uint32_t m = 0;
        for (int i = threadIdx.x; i < p.npart; i += kThreads) m = max(m, p.part[t * p.npart + i]);
        mags[t] = block_max(m, red);
        sx[t] = scale_exp(mags[t]);
    }
    // |dS| <= |dP| + |D| <= 2 d max|dO| max|V| < 2^(1 + log2 d + eO + eV), with
    // max|X| < 2^eX = 2^(14 - sX).
    constexpr int LOG2D = D == 256 ? 8 : (D == 128 ? 7 : 6);
    const int eO = 14 - sx[3], eV = 14 - sx[2];
    const int sS = (mags[3] == 0 || mags[2] == 0) ? 0 : 14 - (1 + LOG2D + eO + eV);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        p.scales[0] = ldexpf(p.scale_log2, -(sx[0] + sx[1]));        // S' -> log2-scaled S
        p.scales[1] = ldexpf(1.f, sS - sx[3] - sx[2]);               // dP' -> dP * 2^sS
        p.scales[2] = ldexpf(1.f, -sx[3]);                           // dV' -> dV
        p.scales[3] = ldexpf(p.scale, -(sx[0] + sS));                // dK' -> dK
        p.scales[4] = ldexpf(p.scale, -(sx[1] + sS));                // dQ' -> dQ
        p.scales[5] = ldexpf(1.f, sS);
        p.scales[6] = 0.f;
        p.scales[7] = 0.f;
    }
    const int N = p.N, Np = p.Np, nrb = Np / 64;
    // Tiles of 64 rows: q, dout (with transposes), k (with transpose), v.
    const long long tq = (long long)p.B * p.Hq * nrb, tk = (long long)p.B * p.Hkv * nrb;
    const long long ntiles = 2 * tq + 2 * tk;
    for (long long t = blockIdx.x; t < ntiles; t += gridDim.x) {
        int which;
        long long r;
        if (t < tq) { which = 0; r = t; }
        else if (t < 2 * tq) { which = 3; r = t - tq; }
        else if (t < 2 * tq + tk) { which = 1; r = t - 2 * tq; }
        else { which = 2; r = t - 2 * tq - tk; }
        const long long h = r / nrb;
        const int rb = (int)(r - h * nrb);
        const uint16_t* src;
        uint16_t* dst;
        uint16_t* dstT;
        if (which == 0) { src = p.q; dst = p.q16; dstT = p.qT16; }
        else if (which == 1) { src = p.k; dst = p.k16; dstT = p.kT16; }
        else if (which == 2) { src = p.v; dst = p.v16; dstT = nullptr; }
        else { src = p.dout; dst = p.do16; dstT = p.doT16; }
        conv_tile<D>(src + (size_t)h * N * p.d, dst + (size_t)h * Np * D,
                     dstT ? dstT + (size_t)h * D * Np : nullptr, rb * 64, N, Np, ldexpf(1.f, sx[which]), tr, p.d);
    }
    // Row dot: D / 8 lanes share one row (16 bytes each).
    constexpr int LPR = D / 8;
    constexpr int RPB = kThreads / LPR;
    const float fS = ldexpf(1.f, sS);
    const long long rows = (long long)p.B * p.Hq * Np;
    const int sub = threadIdx.x % LPR;
    for (long long base = (long long)blockIdx.x * RPB; base < rows; base += (long long)gridDim.x * RPB) {
        const long long rp = base + threadIdx.x / LPR;
        const long long bh = rp / Np;
        const int q = (int)(rp - bh * Np);
        const bool real = rp < rows && q < N && sub * 8 < p.d;
        const long long row = bh * N + q;
        float acc = 0.f;
        if (real) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(p.o + row * p.d + sub * 8);
            const u32x4 g = *reinterpret_cast<const u32x4*>(p.dout + row * p.d + sub * 8);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc = fmaf(bf16_lo(a[t]), bf16_lo(g[t]), acc);
                acc = fmaf(bf16_hi(a[t]), bf16_hi(g[t]), acc);
            }
        }
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (rp < rows && sub == 0) {
            p.delta[rp] = real ? acc * fS : 0.f;
            p.lse2[rp] = real ? p.lse[row] * kLog2e : INFINITY;
        }
    }
}

// ---------------------------------------------------------------- dK / dV
constexpr int kKV_WG = 128;   // keys per workgroup
constexpr int kKV_W = 32;     // keys per wave
constexpr int kKV_Q = 64;     // query rows per step

// The four-wave dK/dV kernel: d <= 64 (D = 64), and d = 128 on grids too small
// for the eight-wave form (use_eight_wave).
template <int D>
struct KvCfg {
    static constexpr int DS = D / 16, DB = D / 32;
    static constexpr int SR = RowPad<D>::STRIDE;       // Q, dO rows: [64][D], padded rows
    static constexpr int RT = padded_tile_bytes<SR, kKV_Q>();
    static constexpr int TT = D * 2 * kKV_Q;            // Q^T, dO^T: [D][64], swizzled
    static constexpr int QR = 0, DOR = RT, QT = 2 * RT, DOT = 2 * RT + TT;
    static constexpr int L2 = 2 * RT + 2 * TT, DD = L2 + 4 * kKV_Q;   // 64 floats each
    static constexpr int STAGE = DD + 4 * kKV_Q;
    static constexpr int LDS = 2 * STAGE;
    // MFMA slots of a step, in order: S rows 0-31 (DS), dP rows 0-31 (DS),
    // S rows 32-63, dP rows 32-63, dV chunks 0-1 (2 DB), dK chunks 0-1,
    // dV chunks 2-3, dK chunks 2-3.
    static constexpr int NS = 8 * DS;
    // The 64 softmax tasks of a step (P of rows 0-31, dS of rows 0-31, P of
    // rows 32-63, dS of rows 32-63; 16 registers each) are spread evenly over
    // the slots [START, END): from two slots after the first S block is
    // complete to the first slot of dK chunks 2-3. Each group starts after its
    // inputs are complete and ends before the slot that consumes it.
    static constexpr int START = DS + 1;
    static constexpr int END = 4 * DS + 6 * DB;
    using PlanR = CopyPlan<D, SR, kKV_Q, 4>;
    using PlanT = CopyPlanSwz<2 * kKV_Q, D, 4>;
    using Addr = LaneAddr<SR, Swz128>;
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(QT % 128 == 0 && DOT % 128 == 0 && STAGE % 128 == 0, "swizzled tiles start on 128 bytes");
};

template <int D>
__host__ __device__ constexpr int kv_task_begin(int n) {
    const int t = (n - KvCfg<D>::START) * 64 / (KvCfg<D>::END - KvCfg<D>::START);
    return t < 0 ? 0 : (t > 64 ? 64 : t);
}

template <int D>
struct KvState {
    u32x4 kf[D / 16], vf[D / 16];   // K, V as the B operand: lane holds key l32, d = ds*16 + hh*8 .. +7
    f32x16 dk[D / 32], dv[D / 32];  // dK^T, dV^T: lane holds key l32, d rows db*32 + (i/4)*8 + hh*4 + i%4
};

// Where one step's data sits: the byte offsets, in the resources of the K/V
// head's query-head group, of 64 rows from q0 of group member g.
struct KvRes {
    BufRes q, dout, qt, dot, l2, dd;
};
struct KvSrc {
    uint32_t rows;   // q16 / do16 rows
    uint32_t tr;     // qT16 / doT16 columns
    uint32_t row4;   // lse2 / delta
};

// The copy of the next step, spread over the MFMA slots of a pipelined step.
// A wave waits at each direct-to-LDS load until the memory pipeline accepts it
// (about 1 KiB per 20 cycles per CU), so loads issued back to back stall it for
// a long stretch; one load every few MFMAs hides under them.
template <int D>
struct KvNext {
    const typename KvCfg<D>::PlanR& pr;
    const typename KvCfg<D>::PlanT& pt;
    const KvRes& rs;
    KvSrc x;
    int ws;     // wave index (scalar)
    int lane;
};

// Copy item c of a step (one 1 KiB block per wave each): [0, NR) Q rows,
// [NR, 2NR) dO rows, then NT blocks of Q^T and NT of dO^T, and last the LSE
// and D rows (waves 0 and 2 copy LSE, 1 and 3 copy D: the same bytes twice).
template <int D, int c>
__device__ __forceinline__ void kv_copy_item(const KvNext<D>& nx, FA_LDS uint8_t* __restrict__ st) {
    using C = KvCfg<D>;
    constexpr int NR = C::PlanR::NT, NT = C::PlanT::NT;
    if constexpr (c < 2 * NR) {
        nx.pr.copy_one(c % NR, c < NR ? nx.rs.q : nx.rs.dout, nx.x.rows, st + (c < NR ? C::QR : C::DOR), nx.ws);
    } else if constexpr (c < 2 * NR + 2 * NT) {
        constexpr int k = c - 2 * NR;
        nx.pt.copy_one(k % NT, k < NT ? nx.rs.qt : nx.rs.dot, nx.x.tr, st + (k < NT ? C::QT : C::DOT), nx.ws);
    } else {
        const bool odd = nx.ws & 1;
        bload_lds4(odd ? nx.rs.dd : nx.rs.l2, nx.lane * 4, nx.x.row4, st + (odd ? C::DD : C::L2));
    }
}

// Fragment addresses: la.row(qb, ds) for the Q / dO row operands,
// la.t.read(tile, db*32, qc) for the transposed ones; lbase = hh * 16 for the per-row
// LSE / D values.

// One unmasked step, interleaved by hand: MFMA slot n issues its MFMA, starts
// the LDS read of slot n + 3's operand and runs its share of the softmax
// tasks; a scheduling barrier closes every slot.
// With COPY, the next step's copy into `wst` is issued item by item, one item
// every SP slots.
template <int D, bool COPY>
__device__ __forceinline__ void kv_step(const FA_LDS uint8_t* __restrict__ st, KvState<D>& S,
                                        const typename KvCfg<D>::Addr& la, int lbase, float sl2, float c1, const KvNext<D>* nx,
                                        FA_LDS uint8_t* __restrict__ wst) {
    using C = KvCfg<D>;
    constexpr int DS = C::DS, DB = C::DB, NS = C::NS, PF = 3;
    constexpr int NITEM = 2 * C::PlanR::NT + 2 * C::PlanT::NT + 1, SP = NS / NITEM;
    static_assert(SP >= 1 && 1 + (NITEM - 1) * SP < NS, "copy items fit the slots");
    f32x16 s[2], dp[2];
    u32x4 pp[4], dsp[4];
    // LSE (P tasks) or D (dS tasks) of task group g = t / 4, loaded one group
    // ahead into lb[g % 2]. (Loading a half's 16 values at once kept up to 48
    // of them live and pushed 51 more registers into AGPRs: 0.6% slower.)
    f32x4 lb[2];
    auto lse_d = [&](auto gc) {
        constexpr int g = decltype(gc)::value, grp = g / 4, h = grp >> 1, u = g % 4;
        lb[g % 2] = *reinterpret_cast<const FA_LDS f32x4*>(st + ((grp & 1) ? C::DD : C::L2) + lbase + h * 128 + u * 32);
    };
    u32x4 ring[PF + 1];
    // Transposed operands: chunk pair qc of d rows db*32 + l32 lies at
    // ((st + b0) ^ (qc << 5)) + tile + db*32*128. The address of pair qc is
    // formed once, at its first read, and serves the 2*DB reads of that pair in
    // the dO^T and Q^T tiles (tile offsets are multiples of 128 bytes).
    const uint32_t tb = (uint32_t)(uintptr_t)st + (uint32_t)la.t.b0;
    uint32_t tx[4];

    auto frag = [&](auto nc) -> u32x4 {
        constexpr int n = decltype(nc)::value;
        if constexpr (n < 4 * DS) {
            constexpr int ph = n / DS, ds = n % DS, qb = ph >> 1;
            return lds_read16b(st, la.row(qb, ds) + ((ph & 1) ? C::DOR : C::QR));
        } else {
            constexpr int m = n - 4 * DS, grp = m / (2 * DB);
            constexpr int qc = (grp >> 1) * 2 + (m % (2 * DB)) / DB, db = m % DB;
            if constexpr ((grp & 1) == 0 && db == 0) {
                if constexpr (qc == 0) tx[0] = tb;
                else asm volatile("v_xor_b32 %0, %1, %2" : "=v"(tx[qc]) : "i"(qc << 5), "v"(tb));
            }
            const FA_LDS uint8_t* a = (const FA_LDS uint8_t*)(uintptr_t)tx[qc];
            return *reinterpret_cast<const FA_LDS u32x4*>(a + ((grp & 1) ? C::QT : C::DOT) + db * 32 * 128);
        }
    };
    auto mfma_at = [&](auto nc, const u32x4& a) {
        constexpr int n = decltype(nc)::value;
        if constexpr (n < 4 * DS) {
            constexpr int ph = n / DS, ds = n % DS, qb = ph >> 1;
            if constexpr ((ph & 1) == 0)
                s[qb] = mfma32h(a, S.kf[ds], ds == 0 ? zero16() : s[qb]);
            else
                dp[qb] = mfma32h(a, S.vf[ds], ds == 0 ? zero16() : dp[qb]);
        } else {
            constexpr int m = n - 4 * DS, grp = m / (2 * DB);
            constexpr int qc = (grp >> 1) * 2 + (m % (2 * DB)) / DB, db = m % DB;
            if constexpr ((grp & 1) == 0)
                S.dv[db] = mfma32h(a, pp[qc], S.dv[db]);
            else
                S.dk[db] = mfma32h(a, dsp[qc], S.dk[db]);
        }
    };
    // Task t: group t/16 (P rows 0-31, dS rows 0-31, P rows 32-63, dS rows
    // 32-63), register i = t%16 of the half, which is row h*32 + (i/4)*8 +
    // hh*4 + i%4. P = exp2(S' sl2 - LSE log2 e); dS 2^sS = P (dP' c1 - D 2^sS).
    // Register pair (2w, 2w+1) of 16-row chunk qc is k-slot pair w of the
    // chunk's B operand.
    auto task = [&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int grp = t / 16, i = t % 16, h = grp >> 1;
        constexpr int e = i % 4, qc = 2 * h + i / 8, w = (i % 8) / 2, g = t / 4;
        if constexpr (e == 0 && g + 1 < 16) lse_d(std::integral_constant<int, g + 1>{});
        if constexpr ((grp & 1) == 0) {
            const float x = fast_exp2(fmaf(s[h][i], sl2, -lb[g % 2][e]));
            s[h][i] = x;
            if constexpr (i & 1) {
                uint32_t v = pack_f16(s[h][i - 1], x);
                pin(v);
                pp[qc][w] = v;
            }
        } else {
            // dS = P (dP c1 - D): the difference in fp32, the product of the fp16
            // pair with the P pair already packed for the dV MFMA (v_pk_mul_f16)
            const float t = fmaf(dp[h][i], c1, -lb[g % 2][e]);
            dp[h][i] = t;
            if constexpr (i & 1) {
                uint32_t v = mul_f16x2(pp[qc][w], pack_f16(dp[h][i - 1], t));
                pin(v);
                dsp[qc][w] = v;
            }
        }
    };

    static_for<PF>([&](auto nc) { ring[decltype(nc)::value] = frag(nc); });
    lse_d(std::integral_constant<int, 0>{});
    static_for<NS>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        mfma_at(nc, ring[n % (PF + 1)]);
        if constexpr (n + PF < NS) ring[(n + PF) % (PF + 1)] = frag(std::integral_constant<int, n + PF>{});
        if constexpr (COPY && n >= 1 && (n - 1) % SP == 0 && (n - 1) / SP < NITEM)
            kv_copy_item<D, (n - 1) / SP>(*nx, wst);
        constexpr int t0 = kv_task_begin<D>(n), t1 = kv_task_begin<D>(n + 1);
        static_for<t1 - t0>([&](auto k) { task(std::integral_constant<int, t0 + decltype(k)::value>{}); });
        __builtin_amdgcn_sched_barrier(0);
    });
}

// A step that crosses the causal diagonal: keys above a row get P = 0. With a
// bounded mask (WIN: sliding window or packed sequences) so do rows at or past
// kend, the first row that no longer sees this lane's key, and rows before
// kbeg, the first row that sees it (packed sequences without the causal mask:
// its sequence's start). Unpipelined; a few per head and wave.
template <int D, bool WIN>
__device__ __forceinline__ void kv_step_masked(const FA_LDS uint8_t* __restrict__ st, KvState<D>& S,
                                               const typename KvCfg<D>::Addr& la, int lbase, int q0, int key, float sl2,
                                               float c1, int hh, bool causal, int kbeg, int kend) {
    using C = KvCfg<D>;
    constexpr int DS = C::DS, DB = C::DB;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        s[qb] = zero16();
        dp[qb] = zero16();
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            s[qb] = mfma32h(lds_read16b(st, la.row(qb, ds) + C::QR), S.kf[ds], s[qb]);
            dp[qb] = mfma32h(lds_read16b(st, la.row(qb, ds) + C::DOR), S.vf[ds], dp[qb]);
        }
    u32x4 pp[4], dsp[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 lv = *reinterpret_cast<const FA_LDS f32x4*>(st + C::L2 + lbase + (qb * 32 + u * 8) * 4);
            const f32x4 dv4 = *reinterpret_cast<const FA_LDS f32x4*>(st + C::DD + lbase + (qb * 32 + u * 8) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = u * 4 + e;
                const int q = q0 + qb * 32 + u * 8 + hh * 4 + e;
                float x = fast_exp2(fmaf(s[qb][i], sl2, -lv[e]));
                if ((causal && key > q) || (WIN && (q < kbeg || q >= kend))) x = 0.f;
                s[qb][i] = x;
                dp[qb][i] = x * fmaf(dp[qb][i], c1, -dv4[e]);
            }
        }
#pragma unroll
    for (int qc = 0; qc < 4; ++qc)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int i = (qc & 1) * 8 + 2 * w;
            pp[qc][w] = pack_f16(s[qc >> 1][i], s[qc >> 1][i + 1]);
            dsp[qc][w] = pack_f16(dp[qc >> 1][i], dp[qc >> 1][i + 1]);
        }
#pragma unroll
    for (int qc = 0; qc < 4; ++qc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            S.dv[db] = mfma32h(la.t.read(st + C::DOT, db * 32, qc), pp[qc], S.dv[db]);
            S.dk[db] = mfma32h(la.t.read(st + C::QT, db * 32, qc), dsp[qc], S.dk[db]);
        }
}

template <int D>
__device__ __forceinline__ void kv_copy(const typename KvCfg<D>::PlanR& pr, const typename KvCfg<D>::PlanT& pt,
                                        const KvRes& rs, const KvSrc& x, FA_LDS uint8_t* __restrict__ st, int w,
                                        int lane) {
    using C = KvCfg<D>;
    pr.copy(rs.q, x.rows, st + C::QR, w);
    pr.copy(rs.dout, x.rows, st + C::DOR, w);
    pt.copy(rs.qt, x.tr, st + C::QT, w);
    pt.copy(rs.dot, x.tr, st + C::DOT, w);
    if (w == 0) bload_lds4(rs.l2, lane * 4, x.row4, st + C::L2);
    if (w == 1) bload_lds4(rs.dd, lane * 4, x.row4, st + C::DD);
}

// Step j: start the copy of step j+1 into stage `wst` (if any), then compute
// step j from stage `rst`. The two stages are distinct; the __restrict__
// qualifiers tell the compiler so, and it then reads `rst` without waiting for
// the copies into `wst`. mode: 0 idle, 1 unmasked, 2 diagonal.
template <int D, bool WIN>
__device__ __forceinline__ void kv_iteration(KvState<D>& S, const typename KvCfg<D>::PlanR& pr,
                                             const typename KvCfg<D>::PlanT& pt, const KvRes& rs, bool issue,
                                             const KvSrc& nx,
                                             FA_LDS uint8_t* __restrict__ wst,
                                             const FA_LDS uint8_t* __restrict__ rst, int mode, int q0, int key,
                                             const typename KvCfg<D>::Addr& la, int lbase, float sl2, float c1, int w,
                                             int lane, bool causal, int kbeg, int kend) {
    if (issue) kv_copy<D>(pr, pt, rs, nx, wst, w, lane);
    if (mode == 1)
        kv_step<D, false>(rst, S, la, lbase, sl2, c1, nullptr, nullptr);
    else if (mode == 2)
        kv_step_masked<D, WIN>(rst, S, la, lbase, q0, key, sl2, c1, lane >> 5, causal, kbeg, kend);
}

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
    using C = KvCfg<D>;
    constexpr int DS = C::DS, DB = C::DB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N, Np = p.Np, G = p.G;
    const bool causal = p.causal != 0;
    int kt, bkv;
    // kt = 0 first: the most query rows when causal
    unmap_block_unit_major(blockIdx.x, p.B * p.Hkv, (N + kKV_WG - 1) / kKV_WG, kt, bkv);
    const int b = bkv / p.Hkv, hkv = bkv - b * p.Hkv;
    const int k0 = kt * kKV_WG;
    const int kw0 = k0 + w * kKV_W;
    const int key = kw0 + l32;                       // < Np: padded rows are zero
    const float sl2 = p.scales[0], c1 = p.scales[1];

    KvState<D> S;
    {
        const uint16_t* Kg = p.k16 + ((size_t)bkv * Np + key) * D;
        const uint16_t* Vg = p.v16 + ((size_t)bkv * Np + key) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            S.kf[ds] = *reinterpret_cast<const u32x4*>(Kg + ds * 16 + hh * 8);
            S.vf[ds] = *reinterpret_cast<const u32x4*>(Vg + ds * 16 + hh * 8);
        }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        S.dk[db] = zero16();
        S.dv[db] = zero16();
    }

    // Steps: row blocks from the last one down to qs (rows before the block's
    // first key see none of it under the causal mask), all G heads per block.
    // With a bounded mask only rows below qe see a key of this workgroup, and
    // packed sequences without the causal mask start at the first key's
    // sequence (qs, rounded down to a row block).
    const Bounds bd{p.cu_seqlens, p.nseq, p.window, N};
    const int kend = WIN ? bd.row_end(key) : 0;     // this lane's key
    const bool lbnd = WIN && !causal;
    const int kbeg = lbnd ? bd.first_key(key) : 0;  // first row that sees this lane's key
    const int qs = causal ? k0 : (lbnd ? bd.first_key(k0) / kKV_Q * kKV_Q : 0);
    const int qe = WIN ? min(N, bd.row_end(k0 + kKV_WG - 1)) : N;
    const int nrb = (qe - qs + kKV_Q - 1) / kKV_Q;
    const int nsteps = G * nrb;
    const int qtop = qs + (nrb - 1) * kKV_Q;
    KvRes rs;
    {
        const size_t bh0 = (size_t)b * p.Hq + (size_t)hkv * G;   // first query head of the group
        const uint32_t nrow = (uint32_t)G * Np;
        rs.q = make_bufres(p.q16 + bh0 * Np * D, nrow * D * 2);
        rs.dout = make_bufres(p.do16 + bh0 * Np * D, nrow * D * 2);
        rs.qt = make_bufres(p.qT16 + bh0 * D * Np, nrow * D * 2);
        rs.dot = make_bufres(p.doT16 + bh0 * D * Np, nrow * D * 2);
        rs.l2 = make_bufres(p.lse2 + bh0 * Np, nrow * 4);
        rs.dd = make_bufres(p.delta + bh0 * Np, nrow * 4);
    }
    auto src_of = [&](int j) {
        const uint32_t g = j % G;
        const uint32_t q0 = qtop - (j / G) * kKV_Q;
        KvSrc x;
        x.rows = (g * Np + q0) * D * 2;
        x.tr = g * D * Np * 2 + q0 * 2;
        x.row4 = (g * Np + q0) * 4;
        return x;
    };
    typename C::PlanR pr;
    typename C::PlanT pt;
    pr.init(w, lane, D);
    pt.init(w, lane, Np);
    typename C::Addr la;
    la.init(l32, hh);
    const int lbase = hh * 16;
    FA_LDS uint8_t* st0 = (FA_LDS uint8_t*)smem;

    kv_copy<D>(pr, pt, rs, src_of(0), st0, w, lane);
    wait_vmem();
    __syncthreads();
    // Steps with q0 >= k0 + 128 (all but the last two row blocks when causal)
    // are unmasked for every wave, and run on one code path. A wave whose keys
    // lie past N runs them too (its keys are zero padding; never stored).
    // With a bounded mask the top row blocks t >= tfar (q0 = qs + 64 t) hold
    // rows past some key's reach (the workgroup's first key reaches least far);
    // they come first (jT steps, per wave), and the steady blocks are t in
    // [tnear, tfar). The bottom blocks t < tnear hold rows before some key's
    // first row: the causal diagonal (two blocks), or, for packed sequences
    // without the causal mask, rows before the last key's sequence start.
    const int tfar = WIN ? max(0, bd.row_end(k0) - qs) / kKV_Q : 0;
    const int tnear = lbnd ? (max(0, bd.first_key(min(k0 + kKV_WG - 1, N - 1)) - qs) + kKV_Q - 1) / kKV_Q : 2;
    const int nfar = WIN ? max(0, nrb - tfar) : 0;
    const int jT = G * nfar;
    int nsteady = WIN ? G * max(0, min(tfar, nrb) - tnear)
                      : (causal ? G * max(0, nrb - 2) : nsteps - 1);   // each has a next step to copy
    if (lbnd) nsteady = min(nsteady, max(0, nsteps - jT - 1));
    const int kend_w0 = WIN ? bd.row_end(kw0) : 0, kend_w31 = WIN ? bd.row_end(kw0 + kKV_W - 1) : 0;
    const int kbeg_w0 = lbnd ? bd.first_key(kw0) : 0;
    const int kbeg_w31 = lbnd ? bd.first_key(min(kw0 + kKV_W - 1, N - 1)) : 0;
    auto per_wave_step = [&](int j) {
        const int q0 = qtop - (j / G) * kKV_Q;
        const bool active = kw0 < N && (!causal || q0 + kKV_Q - 1 >= kw0) && (!WIN || q0 < kend_w31) &&
                            (!lbnd || q0 + kKV_Q - 1 >= kbeg_w0);
        const int mode = !active ? 0
                                 : (((causal && q0 < kw0 + kKV_W - 1) || (WIN && q0 + kKV_Q - 1 >= kend_w0) ||
                                     (lbnd && q0 < kbeg_w31)) ? 2 : 1);
        const bool issue = j + 1 < nsteps;
        const KvSrc nx = src_of(issue ? j + 1 : j);
        FA_LDS uint8_t* wst = st0 + ((j + 1) & 1) * C::STAGE;
        const FA_LDS uint8_t* rst = st0 + (j & 1) * C::STAGE;
        kv_iteration<D, WIN>(S, pr, pt, rs, issue, nx, wst, rst, mode, q0, key, la, lbase, sl2, c1, w, lane, causal,
                             kbeg, kend);
        wait_vmem();
        __syncthreads();
    };
    for (int j = 0; j < jT; ++j) per_wave_step(j);
    for (int j = jT; j < jT + nsteady; ++j) {
        const KvNext<D> nx{pr, pt, rs, src_of(j + 1), __builtin_amdgcn_readfirstlane(w), lane};
        FA_LDS uint8_t* wst = st0 + ((j + 1) & 1) * C::STAGE;
        const FA_LDS uint8_t* rst = st0 + (j & 1) * C::STAGE;
        kv_step<D, true>(rst, S, la, lbase, sl2, c1, &nx, wst);
        wait_vmem();
        __syncthreads();
    }
    for (int j = jT + nsteady; j < nsteps; ++j) per_wave_step(j);

    // dK^T / dV^T blocks: lane holds key l32, d rows db*32 + u*8 + hh*4 + 0..3.
    if (key < N) {
        // rows of dr = p.d values (D, or fewer: the copies' columns past them are zero)
        const int dr = p.d;
        uint16_t* dKg = p.dk + ((size_t)bkv * N + key) * dr;
        uint16_t* dVg = p.dv + ((size_t)bkv * N + key) * dr;
        const float fk = p.scales[3], fv = p.scales[2];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 a, c;
                a[0] = pack_bf16(S.dk[db][u * 4 + 0] * fk, S.dk[db][u * 4 + 1] * fk);
                a[1] = pack_bf16(S.dk[db][u * 4 + 2] * fk, S.dk[db][u * 4 + 3] * fk);
                c[0] = pack_bf16(S.dv[db][u * 4 + 0] * fv, S.dv[db][u * 4 + 1] * fv);
                c[1] = pack_bf16(S.dv[db][u * 4 + 2] * fv, S.dv[db][u * 4 + 3] * fv);
                if (db * 32 + u * 8 + hh * 4 < dr) {
                    *reinterpret_cast<u32x2*>(dKg + db * 32 + u * 8 + hh * 4) = a;
                    *reinterpret_cast<u32x2*>(dVg + db * 32 + u * 8 + hh * 4) = c;
                }
            }
    }
}

// ---------------------------------------------------------------- dK / dV, eight waves
// The d = 128 form (every mask). A workgroup owns 256 keys, 32 per wave,
// with two waves per SIMD, and each step streams 32 query rows. Every
// byte a step copies then serves twice as many keys as in the four-wave form,
// so each MFMA costs half as many copy instructions, and a SIMD has a second
// wave to issue from while one waits on a copy, an LDS read or its softmax
// work. Two waves per SIMD allow at most 256 registers each, which the dK and
// dV accumulators (128), the K operand (32) and one step's S, dP and packed P
// and dS leave room for only if V is not also held in registers: it sits in
// LDS (the workgroup's 256 rows, 68 KiB) and is read as the dP product's B
// operand, one more 16-byte read per dP MFMA.
constexpr int kKV8_WG = 256;     // keys per workgroup
constexpr int kKV8_Q = 32;       // query rows per step
constexpr int kThreads8 = 512;   // 8 waves, two per SIMD

// Transposed [D x 32] tiles have 64-byte rows: 16-byte chunk c of row r sits
// at chunk position c ^ ((r >> 2) & 3). The 16 rows that 16 lanes read at one
// logical chunk then fill the 16 bank groups of a 256-byte line.
struct Key64 {
    __host__ __device__ static constexpr int key(int r) { return (r >> 2) & 3; }
};

template <int D>
struct Kv8Cfg {
    static constexpr int DS = D / 16, DB = D / 32;
    static constexpr int SR = RowPad<D>::STRIDE;             // Q, dO and V rows: padded
    static constexpr int RT = padded_tile_bytes<SR, kKV8_Q>();
    static constexpr int TL = 2 * kKV8_Q;                    // bytes per transposed row
    static constexpr int TT = D * TL;
    static constexpr int QR = 0, DOR = RT, QT = 2 * RT, DOT = 2 * RT + TT;
    static constexpr int L2 = 2 * RT + 2 * TT, DD = L2 + 256;   // 64 floats each (one 64-lane load)
    static constexpr int STAGE = DD + 256;
    static constexpr int VR = 2 * STAGE;                     // V rows of the workgroup's keys
    static constexpr int LDS = VR + kKV8_WG * SR;
    // MFMA slots of a step, DS each, in order: S = Q K^T, dP = dO V^T, then
    // dV^T += dO^T P and dK^T += Q^T dS over the two 16-row chunks.
    static constexpr int NS = 4 * DS;
    // The 16 P tasks run over PSPAN slots from two slots after S is complete,
    // the 16 dS tasks over DSPAN slots after the last P task: the tasks keep
    // one order, which the one-group-ahead LSE / D loads rely on. P of rows
    // 0-15 is done before the first dV slot, dS of rows 0-15 before the first
    // dK slot.
    static constexpr int PSTART = DS + 1, PSPAN = 10, DSTART = PSTART + PSPAN, DSPAN = 9;
    using PlanR = CopyPlan<D, SR, kKV8_Q, 8>;
    using PlanT = CopyPlanSwz<TL, D, 8, Key64>;
    static_assert(D == 128, "the eight-wave form is built for d = 128");
    static_assert(PlanR::NB == 9 && PlanR::NT == 2, "a row tile is 8 blocks of 1 KiB and a ninth, partial one");
    static_assert(PlanT::NT == 1, "one transposed block per wave");
    static_assert(2 * DB == DS, "the dV and dK products take DS slots each");
    // P of rows 0-15 (tasks 0-7) ends before slot 2 DS (dV, chunk 0), of rows
    // 16-31 before 2 DS + DB (chunk 1); dS likewise before 3 DS and 3 DS + DB.
    static_assert(PSTART + (7 * PSPAN + 15) / 16 < 2 * DS && PSTART + PSPAN <= 2 * DS + DB, "P before dV");
    static_assert(DSTART + (7 * DSPAN + 15) / 16 < 3 * DS && DSTART + DSPAN <= 3 * DS + DB, "dS before dK");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// First of 16 tasks spread over `span` slots from slot `start` that slot n runs.
__host__ __device__ constexpr int kv8_task_begin(int n, int start, int span) {
    const int t = (n - start) * 16 / span;
    return t < 0 ? 0 : (t > 16 ? 16 : t);
}

template <int D>
struct Kv8State {
    u32x4 kf[D / 16];                 // K as the B operand: lane holds key l32, d = ds*16 + hh*8 .. +7
    f32x16 dk[D / 32], dv[D / 32];    // dK^T, dV^T: lane holds key l32, d rows db*32 + (i/4)*8 + hh*4 + i%4
};

// Per-lane byte offsets: row(ds) in a row tile (row l32 of the step, d =
// ds*16 + hh*8), tb[qc] in a transposed tile (d row l32 of a 32-row block,
// rows qc*16 + hh*8 .. +7 of the step), V rows from vt.
struct Kv8Addr {
    int rbase;    // l32 * SR + hh * 16
    int tb[2];
    int lbase;    // hh * 16: this lane half's rows in the LSE / D arrays
    __device__ __forceinline__ void init(int l32, int hh, int sr) {
        rbase = l32 * sr + hh * 16;
        const int key = Key64::key(l32);
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) tb[qc] = l32 * 64 + (((2 * qc + hh) ^ key) << 4);
        lbase = hh * 16;
    }
};

template <int D>
struct Kv8Next {
    const typename Kv8Cfg<D>::PlanR& pr;
    const typename Kv8Cfg<D>::PlanT& pt;
    const KvRes& rs;
    KvSrc x;
    int ws;     // wave index (scalar)
    int lane;
};

// Copy item c of a step for wave ws: 0 its block of the Q rows, 1 of the dO
// rows, 2 of Q^T, 3 of dO^T; 4 the rest, one item each for waves 0-3: the
// last (partial) block of the Q rows, of the dO rows, the LSE and the D rows.
template <int D, int c>
__device__ __forceinline__ void kv8_copy_item(const Kv8Next<D>& nx, FA_LDS uint8_t* __restrict__ st) {
    using C = Kv8Cfg<D>;
    if constexpr (c == 0) nx.pr.copy_one(0, nx.rs.q, nx.x.rows, st + C::QR, nx.ws);
    else if constexpr (c == 1) nx.pr.copy_one(0, nx.rs.dout, nx.x.rows, st + C::DOR, nx.ws);
    else if constexpr (c == 2) nx.pt.copy_one(0, nx.rs.qt, nx.x.tr, st + C::QT, nx.ws);
    else if constexpr (c == 3) nx.pt.copy_one(0, nx.rs.dot, nx.x.tr, st + C::DOT, nx.ws);
    else {
        if (nx.ws == 0) nx.pr.copy_one(1, nx.rs.q, nx.x.rows, st + C::QR, nx.ws);
        else if (nx.ws == 1) nx.pr.copy_one(1, nx.rs.dout, nx.x.rows, st + C::DOR, nx.ws);
        else if (nx.ws == 2) bload_lds4(nx.rs.l2, nx.lane * 4, nx.x.row4, st + C::L2);
        else if (nx.ws == 3) bload_lds4(nx.rs.dd, nx.lane * 4, nx.x.row4, st + C::DD);
    }
}

template <int D>
__device__ __forceinline__ void kv8_copy(const Kv8Next<D>& nx, FA_LDS uint8_t* __restrict__ st) {
    static_for<5>([&](auto c) { kv8_copy_item<D, decltype(c)::value>(nx, st); });
}

// One unmasked step, interleaved by hand: slot n issues its MFMA, starts the
// LDS reads of slot n + 3's operands and runs its share of the softmax tasks;
// a scheduling barrier closes every slot. With COPY, the next step's copy
// items go out one every SP slots.
template <int D, bool COPY>
__device__ __forceinline__ void kv8_step(const FA_LDS uint8_t* __restrict__ st, Kv8State<D>& S, const Kv8Addr& la,
                                         const FA_LDS uint8_t* __restrict__ vt, float sl2, float c1,
                                         const Kv8Next<D>* nx, FA_LDS uint8_t* __restrict__ wst) {
    using C = Kv8Cfg<D>;
    constexpr int DS = C::DS, DB = C::DB, NS = C::NS, PF = 3, NITEM = 5, SP = NS / (NITEM + 1);
    static_assert(SP >= 1 && 1 + (NITEM - 1) * SP < NS, "copy items fit the slots");
    f32x16 s, dp;
    u32x4 pp[2], dsp[2];
    f32x4 lb[2];
    // LSE (groups 0-3, P tasks) or D (groups 4-7, dS tasks) of task group g,
    // rows u*8 + hh*4 + 0..3 with u = g % 4, loaded one group ahead.
    auto lse_d = [&](auto gc) {
        constexpr int g = decltype(gc)::value;
        lb[g % 2] = *reinterpret_cast<const FA_LDS f32x4*>(st + (g >= 4 ? C::DD : C::L2) + la.lbase + (g % 4) * 32);
    };
    u32x4 ra[PF + 1], rb[PF + 1];
    auto frag = [&](auto nc) {
        constexpr int n = decltype(nc)::value, r = n % (PF + 1);
        if constexpr (n < DS) {
            ra[r] = lds_read16b(st, la.rbase + C::QR + n * 32);
        } else if constexpr (n < 2 * DS) {
            ra[r] = lds_read16b(st, la.rbase + C::DOR + (n - DS) * 32);
            rb[r] = lds_read16b(vt, (n - DS) * 32);
        } else {
            constexpr int m = n - 2 * DS, grp = m / (2 * DB), qc = (m % (2 * DB)) / DB, db = m % DB;
            ra[r] = lds_read16b(st + la.tb[qc], (grp ? C::QT : C::DOT) + db * 32 * C::TL);
        }
    };
    auto mfma_at = [&](auto nc) {
        constexpr int n = decltype(nc)::value, r = n % (PF + 1);
        if constexpr (n < DS) {
            s = mfma32h(ra[r], S.kf[n], n == 0 ? zero16() : s);
        } else if constexpr (n < 2 * DS) {
            dp = mfma32h(ra[r], rb[r], n == DS ? zero16() : dp);
        } else {
            constexpr int m = n - 2 * DS, grp = m / (2 * DB), qc = (m % (2 * DB)) / DB, db = m % DB;
            if constexpr (grp == 0)
                S.dv[db] = mfma32h(ra[r], pp[qc], S.dv[db]);
            else
                S.dk[db] = mfma32h(ra[r], dsp[qc], S.dk[db]);
        }
    };
    // Task t < 16: P of register i = t (row (i/4)*8 + hh*4 + i%4), P =
    // exp2(S' sl2 - LSE log2 e); task 16 + i: dS 2^sS = P (dP' c1 - D 2^sS),
    // the difference in fp32, the product with the packed fp16 P pair. Register
    // pair (2w, 2w+1) of 16-row chunk qc = i / 8 is k-slot pair w of the
    // chunk's B operand.
    auto task = [&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int i = t % 16, e = i % 4, qc = i / 8, wp = (i % 8) / 2, g = t / 4;
        if constexpr (e == 0 && g + 1 < 8) lse_d(std::integral_constant<int, g + 1>{});
        if constexpr (t < 16) {
            const float x = fast_exp2(fmaf(s[i], sl2, -lb[g % 2][e]));
            s[i] = x;
            if constexpr (i & 1) {
                uint32_t v = pack_f16(s[i - 1], x);
                pin(v);
                pp[qc][wp] = v;
            }
        } else {
            const float y = fmaf(dp[i], c1, -lb[g % 2][e]);
            dp[i] = y;
            if constexpr (i & 1) {
                uint32_t v = mul_f16x2(pp[qc][wp], pack_f16(dp[i - 1], y));
                pin(v);
                dsp[qc][wp] = v;
            }
        }
    };

    static_for<PF>([&](auto nc) { frag(nc); });
    lse_d(std::integral_constant<int, 0>{});
    static_for<NS>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        // The S and dP slots (with the P tasks) run at a raised wave priority,
        // the products at the normal one: when both waves of a SIMD can issue,
        // the one forming scores goes first. Measured on MI355X: 3.0% less
        // time for dK/dV and 2.2% for dQ than equal priorities.
        if constexpr (n == 0) __builtin_amdgcn_s_setprio(1);
        if constexpr (n == 2 * DS) __builtin_amdgcn_s_setprio(0);
        mfma_at(nc);
        if constexpr (n + PF < NS) frag(std::integral_constant<int, n + PF>{});
        if constexpr (COPY && n >= 1 && (n - 1) % SP == 0 && (n - 1) / SP < NITEM)
            kv8_copy_item<D, (n - 1) / SP>(*nx, wst);
        constexpr int p0 = kv8_task_begin(n, C::PSTART, C::PSPAN), p1 = kv8_task_begin(n + 1, C::PSTART, C::PSPAN);
        static_for<p1 - p0>([&](auto k) { task(std::integral_constant<int, p0 + decltype(k)::value>{}); });
        constexpr int d0 = kv8_task_begin(n, C::DSTART, C::DSPAN), d1 = kv8_task_begin(n + 1, C::DSTART, C::DSPAN);
        static_for<d1 - d0>([&](auto k) { task(std::integral_constant<int, 16 + d0 + decltype(k)::value>{}); });
        __builtin_amdgcn_sched_barrier(0);
    });
}

// A step that crosses the causal diagonal: keys above a row get P = 0. With a
// bounded mask (WIN) so do rows at or past kend, the first row that no longer
// sees this lane's key, and rows before kbeg, the first row that sees it.
// Unpipelined; a few per head and wave.
template <int D, bool WIN>
__device__ __forceinline__ void kv8_step_masked(const FA_LDS uint8_t* __restrict__ st, Kv8State<D>& S,
                                                const Kv8Addr& la, const FA_LDS uint8_t* __restrict__ vt, int q0,
                                                int key, float sl2, float c1, int hh, bool causal, int kbeg,
                                                int kend) {
    using C = Kv8Cfg<D>;
    constexpr int DS = C::DS, DB = C::DB;
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
        s = mfma32h(lds_read16b(st, la.rbase + C::QR + ds * 32), S.kf[ds], s);
        dp = mfma32h(lds_read16b(st, la.rbase + C::DOR + ds * 32), lds_read16b(vt, ds * 32), dp);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const f32x4 lv = *reinterpret_cast<const FA_LDS f32x4*>(st + C::L2 + la.lbase + u * 32);
        const f32x4 dv4 = *reinterpret_cast<const FA_LDS f32x4*>(st + C::DD + la.lbase + u * 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = u * 4 + e;
            const int q = q0 + u * 8 + hh * 4 + e;
            float x = fast_exp2(fmaf(s[i], sl2, -lv[e]));
            if ((causal && key > q) || (WIN && (q < kbeg || q >= kend))) x = 0.f;
            s[i] = x;
            dp[i] = x * fmaf(dp[i], c1, -dv4[e]);
        }
    }
    u32x4 pp[2], dsp[2];
#pragma unroll
    for (int qc = 0; qc < 2; ++qc)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int i = qc * 8 + 2 * w;
            pp[qc][w] = pack_f16(s[i], s[i + 1]);
            dsp[qc][w] = pack_f16(dp[i], dp[i + 1]);
        }
#pragma unroll
    for (int qc = 0; qc < 2; ++qc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const FA_LDS uint8_t* a = st + la.tb[qc] + db * 32 * C::TL;
            S.dv[db] = mfma32h(lds_read16b(a, C::DOT), pp[qc], S.dv[db]);
            S.dk[db] = mfma32h(lds_read16b(a, C::QT), dsp[qc], S.dk[db]);
        }
}

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads8, 1) void bwd_dkdv8_kernel(BwdParams p) {
    using C = Kv8Cfg<D>;
    constexpr int DS = C::DS, DB = C::DB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N, Np = p.Np, G = p.G;
    const bool causal = p.causal != 0;
    int kt, bkv;
    // kt = 0 first: the most query rows when causal
    unmap_block_unit_major(blockIdx.x, p.B * p.Hkv, (N + kKV8_WG - 1) / kKV8_WG, kt, bkv);
    const int k0 = kt * kKV8_WG;
    const int kw0 = k0 + w * kKV_W;
    const int key = kw0 + l32;
    // Np is a multiple of 128 and kw0 of 32, so a wave's 32 keys lie all
    // below Np or all at or past it; past it there are no copies to read
    // (zero operands instead; such keys are never stored).
    const bool has_keys = kw0 < Np;
    const float sl2 = p.scales[0], c1 = p.scales[1];

    Kv8State<D> S;
    {
        const size_t row = (size_t)bkv * Np + (has_keys ? key : 0);
        const uint16_t* Kg = p.k16 + row * D;
        const uint16_t* Vg = p.v16 + row * D;
        FA_LDS uint8_t* vrow = (FA_LDS uint8_t*)smem + C::VR + (w * kKV_W + l32) * C::SR + hh * 16;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            S.kf[ds] = gload16(Kg + ds * 16 + hh * 8, has_keys);
            *reinterpret_cast<FA_LDS u32x4*>(vrow + ds * 32) = gload16(Vg + ds * 16 + hh * 8, has_keys);
        }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        S.dk[db] = zero16();
        S.dv[db] = zero16();
    }

    // Steps: 32-row blocks from the last one down to qs, all G heads per block
    // (rows before the block's first key see none of it under the causal
    // mask). With a bounded mask only rows below qe see a key of this
    // workgroup, and packed sequences without the causal mask start at the
    // first key's sequence (qs, rounded down to a row block).
    const Bounds bd{p.cu_seqlens, p.nseq, p.window, N};
    const int kend = WIN ? bd.row_end(key) : 0;     // this lane's key
    const bool lbnd = WIN && !causal;
    const int kbeg = lbnd ? bd.first_key(key) : 0;  // first row that sees this lane's key
    const int qs = causal ? k0 : (lbnd ? bd.first_key(k0) / kKV8_Q * kKV8_Q : 0);
    const int qe = WIN ? min(N, bd.row_end(min(k0 + kKV8_WG - 1, N - 1))) : N;
    const int nrb = (qe - qs + kKV8_Q - 1) / kKV8_Q;
    const int nsteps = G * nrb;
    const int qtop = qs + (nrb - 1) * kKV8_Q;
    KvRes rs;
    {
        const size_t bh0 = (size_t)(bkv / p.Hkv) * p.Hq + (size_t)(bkv % p.Hkv) * G;   // first query head
        const uint32_t nrow = (uint32_t)G * Np;
        rs.q = make_bufres(p.q16 + bh0 * Np * D, nrow * D * 2);
        rs.dout = make_bufres(p.do16 + bh0 * Np * D, nrow * D * 2);
        rs.qt = make_bufres(p.qT16 + bh0 * D * Np, nrow * D * 2);
        rs.dot = make_bufres(p.doT16 + bh0 * D * Np, nrow * D * 2);
        rs.l2 = make_bufres(p.lse2 + bh0 * Np, nrow * 4);
        rs.dd = make_bufres(p.delta + bh0 * Np, nrow * 4);
    }
    auto src_of = [&](int j) {
        const uint32_t g = j % G;
        const uint32_t q0 = qtop - (j / G) * kKV8_Q;
        KvSrc x;
        x.rows = (g * Np + q0) * D * 2;
        x.tr = g * D * Np * 2 + q0 * 2;
        x.row4 = (g * Np + q0) * 4;
        return x;
    };
    typename C::PlanR pr;
    typename C::PlanT pt;
    pr.init(w, lane, D);
    pt.init(w, lane, Np);
    Kv8Addr la;
    la.init(l32, hh, C::SR);
    FA_LDS uint8_t* st0 = (FA_LDS uint8_t*)smem;
    const FA_LDS uint8_t* vt = st0 + C::VR + (w * kKV_W + l32) * C::SR + hh * 16;

    kv8_copy<D>(Kv8Next<D>{pr, pt, rs, src_of(0), __builtin_amdgcn_readfirstlane(w), lane}, st0);
    wait_vmem();
    __syncthreads();
    // Row blocks t in [tnear, tfar) (q0 = qs + 32 t) are unmasked for every
    // wave and run on one code path, with the next step's copy spread over the
    // MFMA slots: all but the last eight blocks when causal. A wave whose keys
    // lie past N runs them too (zero or padding keys, never stored). With a
    // bounded mask the top blocks t >= tfar hold rows past some key's reach (the
    // workgroup's first key reaches least far); they come first (jT steps, per
    // wave). The bottom blocks t < tnear hold rows before some key's first row:
    // the causal diagonal, or, for packed sequences without the causal mask,
    // rows before the last key's sequence start.
    const int tfar = WIN ? max(0, bd.row_end(k0) - qs) / kKV8_Q : 0;
    const int tnear = lbnd ? (max(0, bd.first_key(min(k0 + kKV8_WG - 1, N - 1)) - qs) + kKV8_Q - 1) / kKV8_Q
                           : kKV8_WG / kKV8_Q;
    const int nfar = WIN ? max(0, nrb - tfar) : 0;
    const int jT = G * nfar;
    int nsteady = WIN ? G * max(0, min(tfar, nrb) - tnear)
                      : (causal ? G * max(0, nrb - kKV8_WG / kKV8_Q) : nsteps - 1);   // each has a next step
    if (lbnd) nsteady = min(nsteady, max(0, nsteps - jT - 1));
    const int kend_w0 = WIN ? bd.row_end(kw0) : 0, kend_w31 = WIN ? bd.row_end(kw0 + kKV_W - 1) : 0;
    const int kbeg_w0 = lbnd ? bd.first_key(kw0) : 0;
    const int kbeg_w31 = lbnd ? bd.first_key(min(kw0 + kKV_W - 1, N - 1)) : 0;
    // A step where each wave is idle (no row of the step sees its keys),
    // masked or unmasked.
    auto per_wave_step = [&](int j) {
        const int q0 = qtop - (j / G) * kKV8_Q;
        const bool active = kw0 < N && (!causal || q0 + kKV8_Q - 1 >= kw0) && (!WIN || q0 < kend_w31) &&
                            (!lbnd || q0 + kKV8_Q - 1 >= kbeg_w0);
        const int mode = !active ? 0
                                 : (((causal && q0 < kw0 + kKV_W - 1) || (WIN && q0 + kKV8_Q - 1 >= kend_w0) ||
                                     (lbnd && q0 < kbeg_w31)) ? 2 : 1);
        FA_LDS uint8_t* wst = st0 + ((j + 1) & 1) * C::STAGE;
        const FA_LDS uint8_t* rst = st0 + (j & 1) * C::STAGE;
        if (j + 1 < nsteps) kv8_copy<D>(Kv8Next<D>{pr, pt, rs, src_of(j + 1), __builtin_amdgcn_readfirstlane(w), lane}, wst);
        if (mode == 1)
            kv8_step<D, false>(rst, S, la, vt, sl2, c1, nullptr, nullptr);
        else if (mode == 2)
            kv8_step_masked<D, WIN>(rst, S, la, vt, q0, key, sl2, c1, hh, causal, kbeg, kend);
        wait_vmem();
        __syncthreads();
    };
    for (int j = 0; j < jT; ++j) per_wave_step(j);
    for (int j = jT; j < jT + nsteady; ++j) {
        const Kv8Next<D> nx{pr, pt, rs, src_of(j + 1), __builtin_amdgcn_readfirstlane(w), lane};
        FA_LDS uint8_t* wst = st0 + ((j + 1) & 1) * C::STAGE;
        const FA_LDS uint8_t* rst = st0 + (j & 1) * C::STAGE;
        kv8_step<D, true>(rst, S, la, vt, sl2, c1, &nx, wst);
        wait_vmem();
        __syncthreads();
    }
    for (int j = jT + nsteady; j < nsteps; ++j) per_wave_step(j);

    // dK^T / dV^T blocks: lane holds key l32, d rows db*32 + u*8 + hh*4 + 0..3.
    if (key < N) {
        const int dr = p.d;
        uint16_t* dKg = p.dk + ((size_t)bkv * N + key) * dr;
        uint16_t* dVg = p.dv + ((size_t)bkv * N + key) * dr;
        const float fk = p.scales[3], fv = p.scales[2];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 a, c;
                a[0] = pack_bf16(S.dk[db][u * 4 + 0] * fk, S.dk[db][u * 4 + 1] * fk);
                a[1] = pack_bf16(S.dk[db][u * 4 + 2] * fk, S.dk[db][u * 4 + 3] * fk);
                c[0] = pack_bf16(S.dv[db][u * 4 + 0] * fv, S.dv[db][u * 4 + 1] * fv);
                c[1] = pack_bf16(S.dv[db][u * 4 + 2] * fv, S.dv[db][u * 4 + 3] * fv);
                if (db * 32 + u * 8 + hh * 4 < dr) {
                    *reinterpret_cast<u32x2*>(dKg + db * 32 + u * 8 + hh * 4) = a;
                    *reinterpret_cast<u32x2*>(dVg + db * 32 + u * 8 + hh * 4) = c;
                }
            }
    }
}

// ---------------------------------------------------------------- dQ
constexpr int kQ_WG = 128;   // query rows per workgroup
constexpr int kQ_W = 32;     // query rows per wave
constexpr int kQ_N = 64;     // keys per tile

template <int D>
struct QCfg {
    static constexpr int DS = D / 16, DB = D / 32;
    static constexpr int SR = RowPad<D>::STRIDE;      // K, V rows: [64][D], padded rows
    static constexpr int RT = padded_tile_bytes<SR, kQ_N>();
    // K^T: [D][64]. D = 64: dense 128-byte rows, XOR-swizzled as the dK/dV
    // kernel's transposed tiles, so that three stages (78 KiB) leave room for
    // a second workgroup per CU (two waves per SIMD; the kernel needs at most
    // 256 registers there). D = 128 (grids too small for the eight-wave form):
    // padded rows, which measured faster here than swizzled ones.
    static constexpr bool TSWZ = D == 64;
    static constexpr int ST = RowPad<kQ_N>::STRIDE;
    static constexpr int TT = TSWZ ? D * 2 * kQ_N : padded_tile_bytes<ST, D>();
    static constexpr int KR = 0, VR = RT, KT = 2 * RT;
    static constexpr int STAGE = 2 * RT + TT;
    static constexpr int LDS = 3 * STAGE;             // tiles j-1 (K^T), j, j+1
    // MFMA slots of a pipelined tile, DS each, in order: dQ/PK products of the
    // previous tile for key chunk 0, chunk 1; S^T keys 0-31; dP^T keys 0-31;
    // products of the previous tile for chunks 2, 3; S^T keys 32-63; dP^T keys
    // 32-63. A product slot pair (2m, 2m+1) shares one K^T operand.
    static constexpr int NS = 8 * DS;
    // The 64 softmax tasks of a tile start two slots after its first S^T block
    // is complete and run one per NS/64 slots; the last ones fall into the next
    // tile's first slots. Each group of 16 starts after its inputs are complete
    // and ends before the product that consumes it.
    static constexpr int START = 3 * DS + 1;
    using PlanR = CopyPlan<D, SR, kQ_N, 4>;
    using PlanT = std::conditional_t<TSWZ, CopyPlanSwz<2 * kQ_N, D, 4>, CopyPlan<kQ_N, ST, D, 4>>;
    using Addr = LaneAddr<SR, std::conditional_t<TSWZ, Swz128, PadRows<ST>>>;
    static constexpr int PER_CU = TSWZ ? 2 : 1;       // workgroups per CU
    static_assert(LDS * PER_CU <= 160 * 1024, "LDS budget");
    static_assert(!TSWZ || (KT % 128 == 0 && STAGE % 128 == 0), "swizzled tiles start on 128 bytes");
};

// First softmax task of linear slot x (x counts from the tile's slot 0 and
// runs past NS into the next tile).
template <int D>
__host__ __device__ constexpr int dq_task_begin(int x) {
    const int t = (x - QCfg<D>::START) * 64 / QCfg<D>::NS;
    return t < 0 ? 0 : (t > 64 ? 64 : t);
}

template <int D>
struct QState {
    u32x4 qf[D / 16], dof[D / 16];   // Q, dO as the B operand: lane holds row l32, d = ds*16 + hh*8 ..
    f32x16 dq[D / 32], pk[D / 32];   // dQ^T, PK^T: lane holds row l32, d rows db*32 + (i/4)*8 + hh*4 + i%4
    f32x16 s[2], dp[2];              // S^T, dP^T of keys kb*32 + (i/4)*8 + hh*4 + i%4
    u32x4 pp[4], dsp[4];             // fp16 P^T, dS^T per 16-key chunk, as the B operand
    float l2, dd, dacc;              // LSE log2 e, D 2^sS, running sum of P dP'
};

// Softmax task t of the tile whose S^T / dP^T are in S.s / S.dp: group t/16
// (P keys 0-31, dS keys 0-31, P keys 32-63, dS keys 32-63), register i = t%16.
template <int D, int t>
__device__ __forceinline__ void dq_task(QState<D>& S, float sl2, float c1) {
    constexpr int grp = t / 16, i = t % 16, h = grp >> 1;
    constexpr int kc = 2 * h + i / 8, w = (i % 8) / 2;
    if constexpr ((grp & 1) == 0) {
        const float x = fast_exp2(fmaf(S.s[h][i], sl2, -S.l2));
        S.s[h][i] = x;
        if constexpr (i & 1) {
            uint32_t v = pack_f16(S.s[h][i - 1], x);
            pin(v);
            S.pp[kc][w] = v;
        }
    } else {
        // dS = P (dP c1 - D): the difference in fp32, the product of the fp16
        // pair with the P pair already packed for the PK MFMA (v_pk_mul_f16)
        const float dpv = S.dp[h][i];
        S.dacc = fmaf(S.s[h][i], dpv, S.dacc);
        const float y = fmaf(dpv, c1, -S.dd);
        S.dp[h][i] = y;
        if constexpr (i & 1) {
            uint32_t v = mul_f16x2(S.pp[kc][w], pack_f16(S.dp[h][i - 1], y));
            pin(v);
            S.dsp[kc][w] = v;
        }
    }
}

// The copy of the next tile, spread over the MFMA slots of a pipelined tile
// (see KvNext): NR items of K rows, NR of V rows, then NT of K^T.
template <int D>
struct QNext {
    const typename QCfg<D>::PlanR& pr;
    const typename QCfg<D>::PlanT& pt;
    BufRes rk, rv, rkt;
    uint32_t rows, tr;   // byte offsets of the tile in the row / transposed copies
    int ws;              // wave index (scalar)
};

template <int D, int c>
__device__ __forceinline__ void dq_copy_item(const QNext<D>& nx, FA_LDS uint8_t* __restrict__ st) {
    using C = QCfg<D>;
    constexpr int NR = C::PlanR::NT;
    if constexpr (c < 2 * NR)
        nx.pr.copy_one(c % NR, c < NR ? nx.rk : nx.rv, nx.rows, st + (c < NR ? C::KR : C::VR), nx.ws);
    else
        nx.pt.copy_one(c - 2 * NR, nx.rkt, nx.tr, st + C::KT, nx.ws);
}

// One pipelined tile: `cur` holds tile j (K, V rows), `prv` tile j-1 (K^T).
// PREV = false for a wave's first tile (no previous products or tasks).
// Fragment addresses: la.row(kb, ds) for K / V rows, la.t.read(tile, db*32, kc) for K^T.
// With COPY, the next tile's copy into `wst` is issued one item every SP slots.
template <int D, bool PREV, bool COPY>
__device__ __forceinline__ void dq_pipe(QState<D>& S, const FA_LDS uint8_t* __restrict__ cur,
                                        const FA_LDS uint8_t* __restrict__ prv, const typename QCfg<D>::Addr& la,
                                        float sl2, float c1, const QNext<D>* nx, FA_LDS uint8_t* __restrict__ wst) {
    using C = QCfg<D>;
    constexpr int DS = C::DS, NS = C::NS, PF = 3, START = C::START;
    constexpr int NITEM = 2 * C::PlanR::NT + C::PlanT::NT, SP = NS / NITEM;
    static_assert(SP >= 1 && 1 + (NITEM - 1) * SP < NS, "copy items fit the slots");
    // product group g -> key chunk of the previous tile
    constexpr int kc_of[8] = {0, 1, -1, -1, 2, 3, -1, -1};
    u32x4 ring[PF + 1];

    auto has_read = [](auto nc) constexpr {
        constexpr int n = decltype(nc)::value;
        constexpr int g = n / DS, m = n % DS;
        constexpr bool prod = g == 0 || g == 1 || g == 4 || g == 5;
        return prod ? (PREV && m % 2 == 0) : true;
    };
    auto frag = [&](auto nc) -> u32x4 {
        constexpr int n = decltype(nc)::value;
        constexpr int g = n / DS, m = n % DS;
        if constexpr (kc_of[g] >= 0) {
            constexpr int db = m / 2;
            return la.t.read(prv + C::KT, db * 32, kc_of[g]);
        } else {
            constexpr int kb = g >= 6 ? 1 : 0;
            return lds_read16b(cur, la.row(kb, m) + ((g & 1) ? C::VR : C::KR));
        }
    };
    auto mfma_at = [&](auto nc, const u32x4& a) {
        constexpr int n = decltype(nc)::value;
        constexpr int g = n / DS, m = n % DS;
        if constexpr (kc_of[g] >= 0) {
            if constexpr (PREV) {
                constexpr int db = m / 2, kc = kc_of[g];
                if constexpr (m % 2 == 0) S.pk[db] = mfma32h(a, S.pp[kc], S.pk[db]);
                else S.dq[db] = mfma32h(a, S.dsp[kc], S.dq[db]);
            }
        } else {
            constexpr int kb = g >= 6 ? 1 : 0;
            if constexpr ((g & 1) == 0) S.s[kb] = mfma32h(a, S.qf[m], m == 0 ? zero16() : S.s[kb]);
            else S.dp[kb] = mfma32h(a, S.dof[m], m == 0 ? zero16() : S.dp[kb]);
        }
    };

    // operand reads of slots 0 .. PF-1
    static_for<PF>([&](auto nc) {
        if constexpr (has_read(nc)) ring[decltype(nc)::value % (PF + 1)] = frag(nc);
    });
    static_for<NS>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        // a product slot without a read of its own uses its pair's operand
        constexpr int src = has_read(nc) ? n : n - 1;
        if constexpr (!(kc_of[n / DS] >= 0) || PREV) mfma_at(nc, ring[src % (PF + 1)]);
        if constexpr (n + PF < NS) {
            using NX = std::integral_constant<int, n + PF>;
            if constexpr (has_read(NX{})) ring[(n + PF) % (PF + 1)] = frag(NX{});
        }
        if constexpr (COPY && n >= 1 && (n - 1) % SP == 0 && (n - 1) / SP < NITEM)
            dq_copy_item<D, (n - 1) / SP>(*nx, wst);
        if constexpr (n < START) {
            if constexpr (PREV) {
                constexpr int t0 = dq_task_begin<D>(n + NS), t1 = dq_task_begin<D>(n + NS + 1);
                static_for<t1 - t0>([&](auto k) { dq_task<D, t0 + decltype(k)::value>(S, sl2, c1); });
            }
        } else {
            constexpr int t0 = dq_task_begin<D>(n), t1 = dq_task_begin<D>(n + 1);
            static_for<t1 - t0>([&](auto k) { dq_task<D, t0 + decltype(k)::value>(S, sl2, c1); });
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Finish the last pipelined tile: its remaining softmax tasks, then all of its
// dQ / PK products (K^T from `prv`).
template <int D>
__device__ __forceinline__ void dq_drain(QState<D>& S, const FA_LDS uint8_t* __restrict__ prv, const typename QCfg<D>::Addr& la,
                                         float sl2, float c1) {
    using C = QCfg<D>;
    constexpr int t0 = dq_task_begin<D>(C::NS);
    static_for<64 - t0>([&](auto k) { dq_task<D, t0 + decltype(k)::value>(S, sl2, c1); });
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const u32x4 a = la.t.read(prv + C::KT, db * 32, kc);
            S.pk[db] = mfma32h(a, S.pp[kc], S.pk[db]);
            S.dq[db] = mfma32h(a, S.dsp[kc], S.dq[db]);
        }
}

// A tile with masked entries (the causal diagonal or keys >= N), complete and
// unpipelined. Keys past N are zero rows in the copies but would still get
// P = exp2(-LSE), so they are masked like the ones above the diagonal.
template <int D, bool WIN>
__device__ __forceinline__ void dq_masked(QState<D>& S, const FA_LDS uint8_t* __restrict__ cur,
                                          const typename QCfg<D>::Addr& la, int key0, int qrow, int N, bool causal, float sl2,
                                          float c1, int hh, int lbq, int ubq) {
    using C = QCfg<D>;
    constexpr int DS = C::DS, DB = C::DB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        S.s[kb] = zero16();
        S.dp[kb] = zero16();
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            S.s[kb] = mfma32h(lds_read16b(cur, la.row(kb, ds) + C::KR), S.qf[ds], S.s[kb]);
            S.dp[kb] = mfma32h(lds_read16b(cur, la.row(kb, ds) + C::VR), S.dof[ds], S.dp[kb]);
        }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kk = key0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
            float x = fast_exp2(fmaf(S.s[kb][i], sl2, -S.l2));
            if (kk >= N || (causal && kk > qrow) || (WIN && (kk < lbq || kk >= ubq))) x = 0.f;
            const float dpv = S.dp[kb][i];
            S.dacc = fmaf(x, dpv, S.dacc);
            S.s[kb][i] = x;
            S.dp[kb][i] = x * fmaf(dpv, c1, -S.dd);
        }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int i = (kc & 1) * 8 + 2 * w;
            S.pp[kc][w] = pack_f16(S.s[kc >> 1][i], S.s[kc >> 1][i + 1]);
            S.dsp[kc][w] = pack_f16(S.dp[kc >> 1][i], S.dp[kc >> 1][i + 1]);
        }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const u32x4 a = la.t.read(cur + C::KT, db * 32, kc);
            S.pk[db] = mfma32h(a, S.pp[kc], S.pk[db]);
            S.dq[db] = mfma32h(a, S.dsp[kc], S.dq[db]);
        }
}

// Tile j of the workgroup loop: start the copy of tile j+1 into `wst` (if
// any), then this wave's work on tile j (`cur`; tile j-1 in `prv`). The three
// stages are distinct (the __restrict__ qualifiers say so).
// Tiles [jw1, jfull) are unmasked for this wave and pipelined, tiles
// [jfull, jlast] are masked, later tiles leave the wave idle. Without a window
// jw0 = jw1 = 0; with one, tiles before jw0 hold no visible key for the wave
// and tiles [jw0, jw1) cross its rows' window starts (masked).
template <int D>
__device__ __forceinline__ void dq_copy(const typename QCfg<D>::PlanR& pr, const typename QCfg<D>::PlanT& pt,
                                        BufRes rk, BufRes rv, BufRes rkt, int j, FA_LDS uint8_t* __restrict__ st,
                                        int w) {
    using C = QCfg<D>;
    const uint32_t rows = (uint32_t)j * kQ_N * D * 2, tr = (uint32_t)j * kQ_N * 2;
    pr.copy(rk, rows, st + C::KR, w);
    pr.copy(rv, rows, st + C::VR, w);
    pt.copy(rkt, tr, st + C::KT, w);
}

template <int D, bool WIN>
__device__ __forceinline__ void dq_iteration(QState<D>& S, const typename QCfg<D>::PlanR& pr,
                                             const typename QCfg<D>::PlanT& pt, bool issue, BufRes rk,
                                             BufRes rv, BufRes rkt, int jn,
                                             FA_LDS uint8_t* __restrict__ wst,
                                             const FA_LDS uint8_t* __restrict__ cur,
                                             const FA_LDS uint8_t* __restrict__ prv, int j, int jfull,
                                             int jlast, const typename QCfg<D>::Addr& la, int qrow, int N, bool causal,
                                             float sl2, float c1, int w, int jw0, int jw1, int lbq, int ubq) {
    if (issue) dq_copy<D>(pr, pt, rk, rv, rkt, jn, wst, w);
    if (WIN && j < jw0) return;
    if (j >= jw1 && j < jfull) {
        if (j == jw1) dq_pipe<D, false, false>(S, cur, prv, la, sl2, c1, nullptr, nullptr);
        else dq_pipe<D, true, false>(S, cur, prv, la, sl2, c1, nullptr, nullptr);
    } else {
        if (j == jfull && jfull > jw1) dq_drain<D>(S, prv, la, sl2, c1);
        if (j <= jlast)
            dq_masked<D, WIN>(S, cur, la, j * kQ_N, qrow, N, causal, sl2, c1, (threadIdx.x >> 5) & 1, lbq, ubq);
    }
}

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads, QCfg<D>::PER_CU) void bwd_dq_kernel(BwdParams p) {
    using C = QCfg<D>;
    constexpr int DS = C::DS, DB = C::DB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N, Np = p.Np;
    const bool causal = p.causal != 0;
    const int nqt = (N + kQ_WG - 1) / kQ_WG;
    int rank, bh;
    unmap_block_unit_major(blockIdx.x, p.B * p.Hq, nqt, rank, bh);
    const int qt = causal ? nqt - 1 - rank : rank;   // heaviest first when causal
    const int b = bh / p.Hq, hq = bh - b * p.Hq;
    const size_t bkv = (size_t)b * p.Hkv + hq / p.G;
    const BufRes rk = make_bufres(p.k16 + bkv * Np * D, (uint32_t)Np * D * 2);
    const BufRes rv = make_bufres(p.v16 + bkv * Np * D, (uint32_t)Np * D * 2);
    const BufRes rkt = make_bufres(p.kT16 + bkv * D * Np, (uint32_t)Np * D * 2);
    const float sl2 = p.scales[0], c1 = p.scales[1];

    const int q0 = qt * kQ_WG;
    const int r0 = q0 + w * kQ_W;
    const int qrow = r0 + l32;                       // < Np: padded rows are zero
    const int ntk = (N + kQ_N - 1) / kQ_N;
    const int nfull = N / kQ_N;                      // key tiles with no key >= N
    // Bounded mask (sliding window or packed sequences): tiles before jw0 hold
    // no visible key of the wave, tiles [jw0, jw1) cross its rows' first keys;
    // the loop starts at wave 0's jw0, and the uniform pipelined tiles start
    // after every wave's jw1. A row's first key never decreases along the rows.
    // Packed sequences without the causal mask also end each row's keys at its
    // sequence's end (ub, this bound never decreases along the rows either).
    const Bounds bd{p.cu_seqlens, p.nseq, p.window, N};
    const bool ubnd = WIN && !causal;
    auto ub_of = [&](int r) { return bd.row_end(min(r, N - 1)); };   // keys of row r end before this
    const int nt = causal ? min(ntk, (q0 + kQ_WG - 1) / kQ_N + 1)
                          : (ubnd ? max(1, min(ntk, (ub_of(q0 + kQ_WG - 1) + kQ_N - 1) / kQ_N)) : ntk);
    // Tiles [0, jfull) are unmasked for this wave, [jfull, jlast] masked.
    // jA (wave 0's jfull) <= every wave's jfull: tiles below it run one code
    // path on all waves. A wave past N runs those too (its rows are zero
    // padding with P = 0) and then idles.
    const int jA = causal ? min(nfull, q0 / kQ_N) : (ubnd ? min(nfull, ub_of(q0) / kQ_N) : nfull);
    int jfull = causal ? min(nfull, r0 / kQ_N) : (ubnd ? min(nfull, ub_of(r0) / kQ_N) : nfull);
    int jlast = causal ? min(ntk - 1, (r0 + kQ_W - 1) / kQ_N)
                       : (ubnd ? min(ntk - 1, max(0, ub_of(r0 + kQ_W - 1) - 1) / kQ_N) : ntk - 1);
    const int lbq = WIN ? bd.first_key(qrow) : 0;   // this lane's row
    const int ubq = ubnd ? bd.row_end(qrow) : N;
    auto jw1_of = [&](int r) {                       // first tile the wave of rows r.. sees in full
        const int f = bd.first_key(r + kQ_W - 1);
        return f > 0 ? (f + kQ_N - 1) / kQ_N : 0;
    };
    int jw0 = WIN ? max(0, bd.first_key(r0)) / kQ_N : 0;
    int jw1 = WIN ? jw1_of(r0) : 0;
    const int jst = WIN ? max(0, bd.first_key(q0)) / kQ_N : 0;
    const int jU0 = WIN ? jw1_of(q0 + kQ_WG - kQ_W) + 1 : 1;
    if (r0 >= N) {
        jfull = jA;
        jlast = -1;
        jw0 = jw1 = WIN ? jw1_of(q0) : 0;
    }

    QState<D> S;
    {
        const size_t ro = ((size_t)bh * Np + qrow) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            S.qf[ds] = *reinterpret_cast<const u32x4*>(p.q16 + ro + ds * 16 + hh * 8);
            S.dof[ds] = *reinterpret_cast<const u32x4*>(p.do16 + ro + ds * 16 + hh * 8);
        }
        S.l2 = p.lse2[(size_t)bh * Np + qrow];
        S.dd = p.delta[(size_t)bh * Np + qrow];
        S.dacc = 0.f;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        S.dq[db] = zero16();
        S.pk[db] = zero16();
    }
    typename C::PlanR pr;
    typename C::PlanT pt;
    pr.init(w, lane, D);
    pt.init(w, lane, Np);
    typename C::Addr la;
    la.init(l32, hh);
    FA_LDS uint8_t* st0 = (FA_LDS uint8_t*)smem;

    dq_copy<D>(pr, pt, rk, rv, rkt, jst, st0 + (jst % 3) * C::STAGE, w);
    wait_vmem();
    __syncthreads();
    // first tiles, where waves start their pipelines: tile 0 without a window
    if constexpr (!WIN) {
        dq_iteration<D, WIN>(S, pr, pt, nt > 1, rk, rv, rkt, 1, st0 + C::STAGE, st0, st0 + 2 * C::STAGE, 0, jfull,
                             jlast, la, qrow, N, causal, sl2, c1, w, 0, 0, 0, N);
        wait_vmem();
        __syncthreads();
    } else {
        for (int j = jst; j < min(jU0, nt); ++j) {
            dq_iteration<D, WIN>(S, pr, pt, j + 1 < nt, rk, rv, rkt, j + 1, st0 + ((j + 1) % 3) * C::STAGE,
                                 st0 + (j % 3) * C::STAGE, st0 + ((j + 2) % 3) * C::STAGE, j, jfull, jlast, la, qrow,
                                 N, causal, sl2, c1, w, jw0, jw1, lbq, ubq);
            wait_vmem();
            __syncthreads();
        }
    }
    // steady state: every wave pipelines, and there is a next tile to copy
    const int jS = min(jA, nt - 1);
    for (int j = jU0; j < jS; ++j) {
        FA_LDS uint8_t* wst = st0 + ((j + 1) % 3) * C::STAGE;
        const FA_LDS uint8_t* cur = st0 + (j % 3) * C::STAGE;
        const FA_LDS uint8_t* prv = st0 + ((j + 2) % 3) * C::STAGE;
        const QNext<D> nx{pr, pt, rk, rv, rkt, (uint32_t)(j + 1) * kQ_N * D * 2, (uint32_t)(j + 1) * kQ_N * 2,
                          __builtin_amdgcn_readfirstlane(w)};
        dq_pipe<D, true, true>(S, cur, prv, la, sl2, c1, &nx, wst);
        wait_vmem();
        __syncthreads();
    }
    // the diagonal / ragged tiles, where waves differ
    for (int j = max(jU0, jS); j < nt; ++j) {
        FA_LDS uint8_t* wst = st0 + ((j + 1) % 3) * C::STAGE;
        const FA_LDS uint8_t* cur = st0 + (j % 3) * C::STAGE;
        const FA_LDS uint8_t* prv = st0 + ((j + 2) % 3) * C::STAGE;
        dq_iteration<D, WIN>(S, pr, pt, j + 1 < nt, rk, rv, rkt, j + 1, wst, cur, prv, j, jfull, jlast, la,
                             qrow, N, causal, sl2, c1, w, jw0, jw1, lbq, ubq);
        wait_vmem();
        __syncthreads();
    }
    if (jfull == nt && nt > jw1) dq_drain<D>(S, st0 + ((nt - 1) % 3) * C::STAGE, la, sl2, c1);

    // exact row dot (the lane halves hold half of the keys each), in units of 2^sS
    const float dx = (S.dacc + swap_half(S.dacc)) * c1;
    if (r0 < N && qrow < N) {
        const int dr = p.d;   // rows of dr values (D, or fewer: padded copies)
        uint16_t* dQg = p.dq + ((size_t)bh * N + qrow) * dr;
        const float sc = p.scales[4];
        const float corr = S.dd - dx;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float v4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v4[t] = fmaf(corr, S.pk[db][u * 4 + t], S.dq[db][u * 4 + t]) * sc;
                u32x2 val;
                val[0] = pack_bf16(v4[0], v4[1]);
                val[1] = pack_bf16(v4[2], v4[3]);
                if (db * 32 + u * 8 + hh * 4 < dr) *reinterpret_cast<u32x2*>(dQg + db * 32 + u * 8 + hh * 4) = val;
            }
        if (hh == 0) p.delta[(size_t)bh * Np + qrow] = dx;   // for the dK/dV kernel
    }
}

// ---------------------------------------------------------------- dQ, eight waves
// The d = 128 form (every mask), built like the eight-wave dK/dV
// kernel: a workgroup owns 256 query rows, 32 per wave, two waves per SIMD,
// and each step streams a tile of 32 keys. Q stays in registers; dO, the
// other row operand, sits in LDS (the workgroup's 256 rows) and is read as the
// dP^T product's B operand. Each tile is complete within its step (S^T, dP^T,
// then the PK^T and dQ^T products), so two stages suffice.
constexpr int kQ8_WG = 256;    // query rows per workgroup
constexpr int kQ8_N = 32;      // keys per tile

template <int D>
struct Q8Cfg {
    static constexpr int DS = D / 16, DB = D / 32;
    static constexpr int SR = RowPad<D>::STRIDE;             // K, V and dO rows: padded
    static constexpr int RT = padded_tile_bytes<SR, kQ8_N>();
    static constexpr int TL = 2 * kQ8_N;                     // bytes per K^T row
    static constexpr int TT = D * TL;
    static constexpr int KR = 0, VR = RT, KT = 2 * RT;
    static constexpr int STAGE = 2 * RT + TT;
    static constexpr int DOR = 2 * STAGE;                    // dO rows of the workgroup
    static constexpr int LDS = DOR + kQ8_WG * SR;
    // MFMA slots of a tile, DS each: S^T = K Q^T, dP^T = V dO^T, PK^T += K^T P^T
    // and dQ^T += K^T dS^T over the two 16-key chunks. The 16 P tasks, then the
    // 16 dS tasks, run as in the eight-wave dK/dV step.
    static constexpr int NS = 4 * DS;
    static constexpr int PSTART = DS + 1, PSPAN = 10, DSTART = PSTART + PSPAN, DSPAN = 9;
    using PlanR = CopyPlan<D, SR, kQ8_N, 8>;
    using PlanT = CopyPlanSwz<TL, D, 8, Key64>;
    static_assert(D == 128, "the eight-wave form is built for d = 128");
    static_assert(PlanR::NB == 9 && PlanR::NT == 2, "a row tile is 8 blocks of 1 KiB and a ninth, partial one");
    static_assert(PlanT::NT == 1, "one transposed block per wave");
    static_assert(2 * DB == DS, "the PK and dQ products take DS slots each");
    static_assert(PSTART + (7 * PSPAN + 15) / 16 < 2 * DS && PSTART + PSPAN <= 2 * DS + DB, "P before PK");
    static_assert(DSTART + (7 * DSPAN + 15) / 16 < 3 * DS && DSTART + DSPAN <= 3 * DS + DB, "dS before dQ");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int D>
struct Q8State {
    u32x4 qf[D / 16];                // Q as the B operand: lane holds row l32, d = ds*16 + hh*8 ..
    f32x16 dq[D / 32], pk[D / 32];   // dQ^T, PK^T: lane holds row l32, d rows db*32 + (i/4)*8 + hh*4 + i%4
    float l2, dd, dacc;              // LSE log2 e, D 2^sS, running sum of P dP'
};

template <int D>
struct Q8Next {
    const typename Q8Cfg<D>::PlanR& pr;
    const typename Q8Cfg<D>::PlanT& pt;
    BufRes rk, rv, rkt;
    uint32_t rows, tr;   // byte offsets of the tile in the row / transposed copies
    int ws;              // wave index (scalar)
};

// Copy item c of a tile for wave ws: 0 its block of the K rows, 1 of the V
// rows, 2 of K^T; 3 the last (partial) block of the K rows (wave 0) or of the
// V rows (wave 1).
template <int D, int c>
__device__ __forceinline__ void dq8_copy_item(const Q8Next<D>& nx, FA_LDS uint8_t* __restrict__ st) {
    using C = Q8Cfg<D>;
    if constexpr (c == 0) nx.pr.copy_one(0, nx.rk, nx.rows, st + C::KR, nx.ws);
    else if constexpr (c == 1) nx.pr.copy_one(0, nx.rv, nx.rows, st + C::VR, nx.ws);
    else if constexpr (c == 2) nx.pt.copy_one(0, nx.rkt, nx.tr, st + C::KT, nx.ws);
    else {
        if (nx.ws == 0) nx.pr.copy_one(1, nx.rk, nx.rows, st + C::KR, nx.ws);
        else if (nx.ws == 1) nx.pr.copy_one(1, nx.rv, nx.rows, st + C::VR, nx.ws);
    }
}

template <int D>
__device__ __forceinline__ void dq8_copy(const Q8Next<D>& nx, FA_LDS uint8_t* __restrict__ st) {
    static_for<4>([&](auto c) { dq8_copy_item<D, decltype(c)::value>(nx, st); });
}

// One unmasked tile, interleaved by hand as kv8_step: slot n issues its MFMA,
// starts the LDS reads of slot n + 3's operands and runs its share of the
// softmax tasks. With COPY, the next tile's copy items go out one every SP slots.
template <int D, bool COPY>
__device__ __forceinline__ void dq8_step(const FA_LDS uint8_t* __restrict__ st, Q8State<D>& S, const Kv8Addr& la,
                                         const FA_LDS uint8_t* __restrict__ dot, float sl2, float c1,
                                         const Q8Next<D>* nx, FA_LDS uint8_t* __restrict__ wst) {
    using C = Q8Cfg<D>;
    constexpr int DS = C::DS, DB = C::DB, NS = C::NS, PF = 2, NITEM = 4, SP = NS / (NITEM + 1);
    static_assert(SP >= 1 && 1 + (NITEM - 1) * SP < NS, "copy items fit the slots");
    f32x16 s, dp;
    u32x4 pp[2], dsp[2];
    u32x4 ra[PF + 1], rb[PF + 1];
    auto frag = [&](auto nc) {
        constexpr int n = decltype(nc)::value, r = n % (PF + 1);
        if constexpr (n < DS) {
            ra[r] = lds_read16b(st, la.rbase + C::KR + n * 32);
        } else if constexpr (n < 2 * DS) {
            ra[r] = lds_read16b(st, la.rbase + C::VR + (n - DS) * 32);
            rb[r] = lds_read16b(dot, (n - DS) * 32);
        } else {
            constexpr int m = n - 2 * DS, kc = (m % (2 * DB)) / DB, db = m % DB;
            ra[r] = lds_read16b(st + la.tb[kc], C::KT + db * 32 * C::TL);
        }
    };
    auto mfma_at = [&](auto nc) {
        constexpr int n = decltype(nc)::value, r = n % (PF + 1);
        if constexpr (n < DS) {
            s = mfma32h(ra[r], S.qf[n], n == 0 ? zero16() : s);
        } else if constexpr (n < 2 * DS) {
            dp = mfma32h(ra[r], rb[r], n == DS ? zero16() : dp);
        } else {
            constexpr int m = n - 2 * DS, grp = m / (2 * DB), kc = (m % (2 * DB)) / DB, db = m % DB;
            if constexpr (grp == 0)
                S.pk[db] = mfma32h(ra[r], pp[kc], S.pk[db]);
            else
                S.dq[db] = mfma32h(ra[r], dsp[kc], S.dq[db]);
        }
    };
    // Task t < 16: P^T of register i = t (key (i/4)*8 + hh*4 + i%4 of the
    // tile), P = exp2(S' sl2 - LSE log2 e); task 16 + i: the exact row dot's
    // term P dP' and dS 2^sS = P (dP' c1 - D 2^sS), the difference in fp32, the
    // product with the packed fp16 P pair. Register pair (2w, 2w+1) of 16-key
    // chunk kc = i / 8 is k-slot pair w of the chunk's B operand.
    auto task = [&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int i = t % 16, kc = i / 8, wp = (i % 8) / 2;
        if constexpr (t < 16) {
            const float x = fast_exp2(fmaf(s[i], sl2, -S.l2));
            s[i] = x;
            if constexpr (i & 1) {
                uint32_t v = pack_f16(s[i - 1], x);
                pin(v);
                pp[kc][wp] = v;
            }
        } else {
            const float dpv = dp[i];
            S.dacc = fmaf(s[i], dpv, S.dacc);
            const float y = fmaf(dpv, c1, -S.dd);
            dp[i] = y;
            if constexpr (i & 1) {
                uint32_t v = mul_f16x2(pp[kc][wp], pack_f16(dp[i - 1], y));
                pin(v);
                dsp[kc][wp] = v;
            }
        }
    };

    static_for<PF>([&](auto nc) { frag(nc); });
    static_for<NS>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        // The S and dP slots (with the P tasks) run at a raised wave priority,
        // the products at the normal one: when both waves of a SIMD can issue,
        // the one forming scores goes first. Measured on MI355X: 3.0% less
        // time for dK/dV and 2.2% for dQ than equal priorities.
        if constexpr (n == 0) __builtin_amdgcn_s_setprio(1);
        if constexpr (n == 2 * DS) __builtin_amdgcn_s_setprio(0);
        mfma_at(nc);
        if constexpr (n + PF < NS) frag(std::integral_constant<int, n + PF>{});
        if constexpr (COPY && n >= 1 && (n - 1) % SP == 0 && (n - 1) / SP < NITEM)
            dq8_copy_item<D, (n - 1) / SP>(*nx, wst);
        constexpr int p0 = kv8_task_begin(n, C::PSTART, C::PSPAN), p1 = kv8_task_begin(n + 1, C::PSTART, C::PSPAN);
        static_for<p1 - p0>([&](auto k) { task(std::integral_constant<int, p0 + decltype(k)::value>{}); });
        constexpr int d0 = kv8_task_begin(n, C::DSTART, C::DSPAN), d1 = kv8_task_begin(n + 1, C::DSTART, C::DSPAN);
        static_for<d1 - d0>([&](auto k) { task(std::integral_constant<int, 16 + d0 + decltype(k)::value>{}); });
        __builtin_amdgcn_sched_barrier(0);
    });
}

// A tile with masked entries (the causal diagonal, keys >= N, and with a
// bounded mask (WIN) keys outside [lbq, ubq), this lane's row's first key and
// end), unpipelined. Keys past N are zero rows in the copies but would still
// get P = exp2(-LSE), so they are masked like the ones above the diagonal.
template <int D, bool WIN>
__device__ __forceinline__ void dq8_masked(const FA_LDS uint8_t* __restrict__ st, Q8State<D>& S, const Kv8Addr& la,
                                           const FA_LDS uint8_t* __restrict__ dot, int key0, int qrow, int N,
                                           bool causal, float sl2, float c1, int hh, int lbq, int ubq) {
    using C = Q8Cfg<D>;
    constexpr int DS = C::DS, DB = C::DB;
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
        s = mfma32h(lds_read16b(st, la.rbase + C::KR + ds * 32), S.qf[ds], s);
        dp = mfma32h(lds_read16b(st, la.rbase + C::VR + ds * 32), lds_read16b(dot, ds * 32), dp);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int kk = key0 + (i >> 2) * 8 + hh * 4 + (i & 3);
        float x = fast_exp2(fmaf(s[i], sl2, -S.l2));
        if (kk >= N || (causal && kk > qrow) || (WIN && (kk < lbq || kk >= ubq))) x = 0.f;
        const float dpv = dp[i];
        S.dacc = fmaf(x, dpv, S.dacc);
        s[i] = x;
        dp[i] = x * fmaf(dpv, c1, -S.dd);
    }
    u32x4 pp[2], dsp[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int i = kc * 8 + 2 * w;
            pp[kc][w] = pack_f16(s[i], s[i + 1]);
            dsp[kc][w] = pack_f16(dp[i], dp[i + 1]);
        }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const u32x4 a = lds_read16b(st + la.tb[kc], C::KT + db * 32 * C::TL);
            S.pk[db] = mfma32h(a, pp[kc], S.pk[db]);
            S.dq[db] = mfma32h(a, dsp[kc], S.dq[db]);
        }
}

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads8, 1) void bwd_dq8_kernel(BwdParams p) {
    using C = Q8Cfg<D>;
    constexpr int DS = C::DS, DB = C::DB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N, Np = p.Np;
    const bool causal = p.causal != 0;
    const int nqt = (N + kQ8_WG - 1) / kQ8_WG;
    int rank, bh;
    unmap_block_unit_major(blockIdx.x, p.B * p.Hq, nqt, rank, bh);
    const int qt = causal ? nqt - 1 - rank : rank;   // heaviest first when causal
    const int b = bh / p.Hq, hq = bh - b * p.Hq;
    const size_t bkv = (size_t)b * p.Hkv + hq / p.G;
    const BufRes rk = make_bufres(p.k16 + bkv * Np * D, (uint32_t)Np * D * 2);
    const BufRes rv = make_bufres(p.v16 + bkv * Np * D, (uint32_t)Np * D * 2);
    const BufRes rkt = make_bufres(p.kT16 + bkv * D * Np, (uint32_t)Np * D * 2);
    const float sl2 = p.scales[0], c1 = p.scales[1];

    const int q0 = qt * kQ8_WG;
    const int r0 = q0 + w * kQ_W;
    const int qrow = r0 + l32;
    // Np is a multiple of 128 and r0 of 32, so a wave's 32 rows lie all below
    // Np or all at or past it; past it they are zero operands with P = 0.
    const bool has_rows = r0 < Np;
    const int ntk = (N + kQ8_N - 1) / kQ8_N;
    const int nfull = N / kQ8_N;                     // key tiles with no key >= N
    // Bounded mask (sliding window or packed sequences): a row's first key
    // never decreases along the rows, nor does its last one for packed
    // sequences without the causal mask (ub, the end of the row's sequence).
    const Bounds bd{p.cu_seqlens, p.nseq, p.window, N};
    const bool ubnd = WIN && !causal;
    auto ub_of = [&](int r) { return bd.row_end(min(r, N - 1)); };   // keys of row r end before this
    const int nt = causal ? min(ntk, (q0 + kQ8_WG - 1) / kQ8_N + 1)
                          : (ubnd ? max(1, min(ntk, (ub_of(q0 + kQ8_WG - 1) + kQ8_N - 1) / kQ8_N)) : ntk);
    // For this wave, tiles before jw0 hold no visible key, tiles [jw0, jw1)
    // cross its rows' first keys (masked), tiles [jw1, jfull) are unmasked,
    // tiles [jfull, jlast] masked (the causal diagonal, keys >= N, its rows'
    // last keys), later ones idle. Without a window jw0 = jw1 = 0. jA (wave
    // 0's jfull) <= every wave's jfull and jU (the last wave's jw1) >= every
    // wave's jw1, so the tiles in [jU, jA) run one code path on all waves,
    // with the next tile's copy spread over the slots. A wave past N runs
    // those too (its rows have P = 0) and otherwise idles.
    const int jA = causal ? min(nfull, q0 / kQ8_N) : (ubnd ? min(nfull, ub_of(q0) / kQ8_N) : nfull);
    int jfull = causal ? min(nfull, r0 / kQ8_N) : (ubnd ? min(nfull, ub_of(r0) / kQ8_N) : nfull);
    int jlast = causal ? min(ntk - 1, (r0 + kQ_W - 1) / kQ8_N)
                       : (ubnd ? min(ntk - 1, max(0, ub_of(r0 + kQ_W - 1) - 1) / kQ8_N) : ntk - 1);
    const int lbq = WIN ? bd.first_key(qrow) : 0;   // this lane's row
    const int ubq = ubnd ? bd.row_end(qrow) : N;
    auto jw1_of = [&](int r) {                       // first tile the wave of rows r.. sees in full
        const int f = bd.first_key(r + kQ_W - 1);
        return f > 0 ? (f + kQ8_N - 1) / kQ8_N : 0;
    };
    const int jw0 = WIN ? max(0, bd.first_key(r0)) / kQ8_N : 0;
    const int jw1 = WIN ? jw1_of(r0) : 0;
    const int jst = WIN ? max(0, bd.first_key(q0)) / kQ8_N : 0;      // wave 0's jw0
    const int jU = WIN ? jw1_of(q0 + kQ8_WG - kQ_W) : 0;
    if (r0 >= N) {
        jfull = jA;
        jlast = -1;
    }

    Q8State<D> S;
    {
        const size_t ro = ((size_t)bh * Np + (has_rows ? qrow : 0)) * D;
        FA_LDS uint8_t* drow = (FA_LDS uint8_t*)smem + C::DOR + (w * kQ_W + l32) * C::SR + hh * 16;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            S.qf[ds] = gload16(p.q16 + ro + ds * 16 + hh * 8, has_rows);
            *reinterpret_cast<FA_LDS u32x4*>(drow + ds * 32) = gload16(p.do16 + ro + ds * 16 + hh * 8, has_rows);
        }
        S.l2 = has_rows ? p.lse2[(size_t)bh * Np + qrow] : INFINITY;
        S.dd = has_rows ? p.delta[(size_t)bh * Np + qrow] : 0.f;
        S.dacc = 0.f;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        S.dq[db] = zero16();
        S.pk[db] = zero16();
    }
    typename C::PlanR pr;
    typename C::PlanT pt;
    pr.init(w, lane, D);
    pt.init(w, lane, Np);
    Kv8Addr la;
    la.init(l32, hh, C::SR);
    FA_LDS uint8_t* st0 = (FA_LDS uint8_t*)smem;
    const FA_LDS uint8_t* dot = st0 + C::DOR + (w * kQ_W + l32) * C::SR + hh * 16;
    auto next = [&](int j) {
        return Q8Next<D>{pr, pt, rk, rv, rkt, (uint32_t)j * kQ8_N * D * 2, (uint32_t)j * kQ8_N * 2,
                         __builtin_amdgcn_readfirstlane(w)};
    };

    dq8_copy<D>(next(jst), st0 + (jst & 1) * C::STAGE);
    wait_vmem();
    __syncthreads();
    auto per_wave_tile = [&](int j) {
        const FA_LDS uint8_t* cur = st0 + (j & 1) * C::STAGE;
        if (j + 1 < nt) dq8_copy<D>(next(j + 1), st0 + ((j + 1) & 1) * C::STAGE);
        if (!(WIN && j < jw0) && j <= jlast) {
            if (j >= jw1 && j < jfull)
                dq8_step<D, false>(cur, S, la, dot, sl2, c1, nullptr, nullptr);
            else
                dq8_masked<D, WIN>(cur, S, la, dot, j * kQ8_N, qrow, N, causal, sl2, c1, hh, lbq, ubq);
        }
        wait_vmem();
        __syncthreads();
    };
    const int jS = min(jA, nt - 1);   // each has a next tile to copy
    for (int j = jst; j < min(jU, nt); ++j) per_wave_tile(j);
    for (int j = max(jst, jU); j < jS; ++j) {
        const Q8Next<D> nx = next(j + 1);
        dq8_step<D, true>(st0 + (j & 1) * C::STAGE, S, la, dot, sl2, c1, &nx, st0 + ((j + 1) & 1) * C::STAGE);
        wait_vmem();
        __syncthreads();
    }
    for (int j = max(max(jst, jU), jS); j < nt; ++j) per_wave_tile(j);

    // exact row dot (the lane halves hold half of the keys each), in units of 2^sS
    const float dx = (S.dacc + swap_half(S.dacc)) * c1;
    if (qrow < N) {
        const int dr = p.d;   // rows of dr values (D, or fewer: padded copies)
        uint16_t* dQg = p.dq + ((size_t)bh * N + qrow) * dr;
        const float sc = p.scales[4];
        const float corr = S.dd - dx;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float v4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v4[t] = fmaf(corr, S.pk[db][u * 4 + t], S.dq[db][u * 4 + t]) * sc;
                u32x2 val;
                val[0] = pack_bf16(v4[0], v4[1]);
                val[1] = pack_bf16(v4[2], v4[3]);
                if (db * 32 + u * 8 + hh * 4 < dr) *reinterpret_cast<u32x2*>(dQg + db * 32 + u * 8 + hh * 4) = val;
            }
        if (hh == 0) p.delta[(size_t)bh * Np + qrow] = dx;   // for the dK/dV kernel
    }
}

// ---------------------------------------------------------------- d = 256: split head dimension
// A wave's K and V (dK/dV pass) or Q and dO (dQ pass) over all 256 columns take
// 128 registers, and the four accumulators of the full width 256 more: no room
// for the scores. So each gradient pass runs two workgroups per tile, one per
// half of the accumulated columns (kSplitDH = 128): both compute S and dP over
// all 256 columns, and each accumulates its half of dK, dV (or dQ, PK). This
// trades work (S and dP are computed twice) for a register budget that fits.
//
// A row tile of 256 columns is 33 KiB, so the LDS holds one set of a step's
// tiles, not two. A step has two phases that read different tiles, though:
// S and dP (phase A) read the row tiles (and LSE, D), the gradient products
// (phase B) the transposed tiles. So the next step's row tiles are copied as
// soon as phase A is done everywhere, and land during phase B; the next
// transposed tiles are copied after phase B, and land during the next phase
// A. Loads complete in issue order, so a wave waits for the row tiles by
// leaving only the transposed copies outstanding (vmcnt), and every step
// runs the plain masked path.
constexpr int kSplitDH = 128;

template <int D>
struct KvSplitCfg {
    static constexpr int DS = D / 16, DBH = kSplitDH / 32;
    static constexpr int SR = RowPad<D>::STRIDE;          // Q, dO rows: [64][D], padded rows
    static constexpr int RT = padded_tile_bytes<SR, kKV_Q>();
    static constexpr int TT = kSplitDH * 2 * kKV_Q;        // Q^T, dO^T of one half: [DH][64], swizzled
    static constexpr int QR = 0, DOR = RT, QT = 2 * RT, DOT = 2 * RT + TT;
    // LSE and D rows (64 floats each) in two sets, by step parity: a step's
    // set stays intact while the next step's copy fills the other one
    static constexpr int L2 = 2 * RT + 2 * TT, DD = L2 + 4 * kKV_Q, LD2 = 8 * kKV_Q;
    static constexpr int LDS = L2 + 2 * LD2;               // one stage of tiles
    using PlanR = CopyPlan<D, SR, kKV_Q, 4>;
    using PlanT = CopyPlanSwz<2 * kKV_Q, kSplitDH, 4>;
    using Addr = LaneAddr<SR, Swz128>;
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(QT % 128 == 0 && DOT % 128 == 0, "swizzled tiles start on 128 bytes");
};

template <int D>
struct KvSplitState {
    u32x4 kf[D / 16], vf[D / 16];          // K, V as the B operand (all columns)
    f32x16 dk[kSplitDH / 32], dv[kSplitDH / 32];   // dK^T, dV^T of this workgroup's half
};

// One step of 64 query rows against the wave's 32 keys, every entry masked as
// in kv_step_masked (causal: keys above the row; bounded masks: rows outside
// [kbeg, kend)). Phase A: S and dP over all columns for rows 0-31, then for
// rows 32-63 with the softmax of rows 0-31 (P, dS and their fp16 packs) spread
// over those MFMAs, one register per two MFMAs. `mid` then runs (the
// workgroup's hand-over between the phases). Phase B: dV^T += dO^T P and
// dK^T += Q^T dS over this half's columns for rows 0-31 with the softmax of
// rows 32-63 spread over them, then for rows 32-63. ld: the byte offset of
// the step's set of LSE and D rows, which the next step's copy leaves alone.
template <int D, bool WIN, class MID>
__device__ __forceinline__ void kv_split_step(const FA_LDS uint8_t* __restrict__ st, KvSplitState<D>& S,
                                              const typename KvSplitCfg<D>::Addr& la, int lbase, int ld, int q0,
                                              int key, float sl2, float c1, int hh, bool causal, int kbeg, int kend,
                                              const MID& mid) {
    using C = KvSplitCfg<D>;
    constexpr int DS = C::DS, DBH = C::DBH;
    f32x16 s[2], dp[2];
    f32x4 lv[4], dv4[4];
    u32x4 pp[4], dsp[4];
    auto stats = [&](int qb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            lv[u] = *reinterpret_cast<const FA_LDS f32x4*>(st + C::L2 + ld + lbase + (qb * 32 + u * 8) * 4);
            dv4[u] = *reinterpret_cast<const FA_LDS f32x4*>(st + C::DD + ld + lbase + (qb * 32 + u * 8) * 4);
        }
    };
    // register i of rows qb*32..: row q0 + qb*32 + (i/4)*8 + hh*4 + i%4
    auto soft = [&](auto qbc, auto ic) {
        constexpr int qb = decltype(qbc)::value, i = decltype(ic)::value;
        constexpr int u = i / 4, e = i % 4, qc = 2 * qb + i / 8, w = (i % 8) / 2;
        const int q = q0 + qb * 32 + u * 8 + hh * 4 + e;
        float x = fast_exp2(fmaf(s[qb][i], sl2, -lv[u][e]));
        if ((causal && key > q) || (WIN && (q < kbeg || q >= kend))) x = 0.f;
        s[qb][i] = x;
        dp[qb][i] = x * fmaf(dp[qb][i], c1, -dv4[u][e]);
        if constexpr (i & 1) {
            pp[qc][w] = pack_f16(s[qb][i - 1], s[qb][i]);
            dsp[qc][w] = pack_f16(dp[qb][i - 1], dp[qb][i]);
        }
    };
    s[0] = zero16();
    dp[0] = zero16();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
        s[0] = mfma32h(lds_read16b(st, la.row(0, ds) + C::QR), S.kf[ds], s[0]);
        dp[0] = mfma32h(lds_read16b(st, la.row(0, ds) + C::DOR), S.vf[ds], dp[0]);
    }
    s[1] = zero16();
    dp[1] = zero16();
    stats(0);
    // operands read PF slots ahead of their MFMA: a scheduling barrier closes
    // every slot, so no read could otherwise move ahead of it (one slot: the
    // register budget has no room for a deeper ring)
    constexpr int PF = 1;
    u32x4 ra[PF + 1][2];
    auto read_a = [&](auto dc) {
        constexpr int ds = decltype(dc)::value;
        ra[ds % (PF + 1)][0] = lds_read16b(st, la.row(1, ds) + C::QR);
        ra[ds % (PF + 1)][1] = lds_read16b(st, la.row(1, ds) + C::DOR);
    };
    static_for<PF>([&](auto dc) { read_a(dc); });
    static_for<DS>([&](auto dc) {
        constexpr int ds = decltype(dc)::value;
        if constexpr (ds + PF < DS) read_a(std::integral_constant<int, ds + PF>{});
        s[1] = mfma32h(ra[ds % (PF + 1)][0], S.kf[ds], s[1]);
        dp[1] = mfma32h(ra[ds % (PF + 1)][1], S.vf[ds], dp[1]);
        static_for<16 / DS>([&](auto k) { soft(std::integral_constant<int, 0>{}, std::integral_constant<int, ds * (16 / DS) + decltype(k)::value>{}); });
        __builtin_amdgcn_sched_barrier(0);
    });
    mid();
    stats(1);
    u32x4 rb[PF + 1][2];
    auto read_b = [&](auto mc) {
        constexpr int m = decltype(mc)::value, qc = m / DBH, db = m % DBH;
        rb[m % (PF + 1)][0] = la.t.read(st + C::DOT, db * 32, qc);
        rb[m % (PF + 1)][1] = la.t.read(st + C::QT, db * 32, qc);
    };
    static_for<PF>([&](auto mc) { read_b(mc); });
    static_for<2 * DBH>([&](auto mc) {
        constexpr int m = decltype(mc)::value, qc = m / DBH, db = m % DBH;
        if constexpr (m + PF < 2 * DBH) read_b(std::integral_constant<int, m + PF>{});
        S.dv[db] = mfma32h(rb[m % (PF + 1)][0], pp[qc], S.dv[db]);
        S.dk[db] = mfma32h(rb[m % (PF + 1)][1], dsp[qc], S.dk[db]);
        static_for<16 / (2 * DBH)>([&](auto k) { soft(std::integral_constant<int, 1>{}, std::integral_constant<int, m * (16 / (2 * DBH)) + decltype(k)::value>{}); });
        __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int qc = 2; qc < 4; ++qc)
#pragma unroll
        for (int db = 0; db < DBH; ++db) {
            S.dv[db] = mfma32h(la.t.read(st + C::DOT, db * 32, qc), pp[qc], S.dv[db]);
            S.dk[db] = mfma32h(la.t.read(st + C::QT, db * 32, qc), dsp[qc], S.dk[db]);
        }
}

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_split_kernel(BwdParams p) {
    using C = KvSplitCfg<D>;
    constexpr int DS = C::DS, DBH = C::DBH;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];
    FA_LDS uint8_t* st = (FA_LDS uint8_t*)smem;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N, Np = p.Np, G = p.G;
    const bool causal = p.causal != 0;
    int kt, unit;
    unmap_block_unit_major(blockIdx.x, p.B * p.Hkv * 2, (N + kKV_WG - 1) / kKV_WG, kt, unit);
    const int half = unit & 1, bkv = unit >> 1;
    const int b = bkv / p.Hkv, hkv = bkv - b * p.Hkv;
    const int k0 = kt * kKV_WG, kw0 = k0 + w * kKV_W, key = kw0 + l32;   // key < Np: padded rows are zero
    const float sl2 = p.scales[0], c1 = p.scales[1];

    KvSplitState<D> S;
    {
        const uint16_t* Kg = p.k16 + ((size_t)bkv * Np + key) * D;
        const uint16_t* Vg = p.v16 + ((size_t)bkv * Np + key) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            S.kf[ds] = *reinterpret_cast<const u32x4*>(Kg + ds * 16 + hh * 8);
            S.vf[ds] = *reinterpret_cast<const u32x4*>(Vg + ds * 16 + hh * 8);
        }
    }
#pragma unroll
    for (int db = 0; db < DBH; ++db) {
        S.dk[db] = zero16();
        S.dv[db] = zero16();
    }
    // the row blocks that can see a key of this workgroup (as bwd_dkdv_kernel)
    const Bounds bd{p.cu_seqlens, p.nseq, p.window, N};
    const int kend = WIN ? bd.row_end(key) : 0;
    const bool lbnd = WIN && !causal;
    const int kbeg = lbnd ? bd.first_key(key) : 0;
    const int qs = causal ? k0 : (lbnd ? bd.first_key(k0) / kKV_Q * kKV_Q : 0);
    const int qe = WIN ? min(N, bd.row_end(k0 + kKV_WG - 1)) : N;
    const int nrb = max(0, (qe - qs + kKV_Q - 1) / kKV_Q);
    const int nsteps = G * nrb;

    KvRes rs;
    {
        const size_t bh0 = (size_t)b * p.Hq + (size_t)hkv * G;
        const uint32_t nrow = (uint32_t)G * Np;
        rs.q = make_bufres(p.q16 + bh0 * Np * D, nrow * D * 2);
        rs.dout = make_bufres(p.do16 + bh0 * Np * D, nrow * D * 2);
        rs.qt = make_bufres(p.qT16 + bh0 * D * Np, nrow * D * 2);
        rs.dot = make_bufres(p.doT16 + bh0 * D * Np, nrow * D * 2);
        rs.l2 = make_bufres(p.lse2 + bh0 * Np, nrow * 4);
        rs.dd = make_bufres(p.delta + bh0 * Np, nrow * 4);
    }
    typename C::PlanR pr;
    typename C::PlanT pt;
    pr.init(w, lane, D);
    pt.init(w, lane, Np);
    typename C::Addr la;
    la.init(l32, hh);
    const int lbase = hh * 16;
    // step j: query head g = j % G, rows q0 = qs + (j / G) * 64
    auto copy_rows = [&](int j) {   // Q, dO rows, LSE and D (set j & 1): 2 * NT + 1 loads per wave
        const uint32_t g = j % G;
        const int q0 = qs + (j / G) * kKV_Q;
        const uint32_t rows = (g * Np + q0) * D * 2;
        const uint32_t row4 = (g * Np + q0) * 4;
        const int ld = (j & 1) * C::LD2;
        pr.copy(rs.q, rows, st + C::QR, w);
        pr.copy(rs.dout, rows, st + C::DOR, w);
        // waves 0 and 2 copy LSE, 1 and 3 copy D (the same bytes twice)
        if ((w & 1) == 0) bload_lds4(rs.l2, lane * 4, row4, st + C::L2 + ld);
        else bload_lds4(rs.dd, lane * 4, row4, st + C::DD + ld);
    };
    auto copy_tr = [&](int j) {     // this half's Q^T, dO^T: 2 * NT loads per wave
        const uint32_t g = j % G;
        const int q0 = qs + (j / G) * kKV_Q;
        const uint32_t tr = (g * D + half * kSplitDH) * Np * 2 + q0 * 2;
        pt.copy(rs.qt, tr, st + C::QT, w);
        pt.copy(rs.dot, tr, st + C::DOT, w);
    };
    if (nsteps > 0) {
        copy_rows(0);
        copy_tr(0);
    }
    for (int j = 0; j < nsteps; ++j) {
        const int q0 = qs + (j / G) * kKV_Q;
        wait_vmem_n<2 * C::PlanT::NT>();   // this step's rows (its transposed tiles may be in flight)
        __syncthreads();
        kv_split_step<D, WIN>(st, S, la, lbase, (j & 1) * C::LD2, q0, key, sl2, c1, hh, causal, kbeg, kend, [&]() {
            wait_vmem();                    // this step's transposed tiles
            __syncthreads();                // ... everywhere, and the row tiles are free
            if (j + 1 < nsteps) copy_rows(j + 1);
        });
        __syncthreads();                    // the transposed tiles are free
        if (j + 1 < nsteps) copy_tr(j + 1);
    }
    if (key < N) {
        const int dr = p.d;
        uint16_t* dKg = p.dk + ((size_t)bkv * N + key) * dr + half * kSplitDH;
        uint16_t* dVg = p.dv + ((size_t)bkv * N + key) * dr + half * kSplitDH;
        const float fk = p.scales[3], fv = p.scales[2];
#pragma unroll
        for (int db = 0; db < DBH; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 a, c;
                a[0] = pack_bf16(S.dk[db][u * 4 + 0] * fk, S.dk[db][u * 4 + 1] * fk);
                a[1] = pack_bf16(S.dk[db][u * 4 + 2] * fk, S.dk[db][u * 4 + 3] * fk);
                c[0] = pack_bf16(S.dv[db][u * 4 + 0] * fv, S.dv[db][u * 4 + 1] * fv);
                c[1] = pack_bf16(S.dv[db][u * 4 + 2] * fv, S.dv[db][u * 4 + 3] * fv);
                if (half * kSplitDH + db * 32 + u * 8 + hh * 4 < dr) {
                    *reinterpret_cast<u32x2*>(dKg + db * 32 + u * 8 + hh * 4) = a;
                    *reinterpret_cast<u32x2*>(dVg + db * 32 + u * 8 + hh * 4) = c;
                }
            }
    }
}

template <int D>
struct QSplitCfg {
    static constexpr int DS = D / 16, DBH = kSplitDH / 32;
    static constexpr int SR = RowPad<D>::STRIDE;          // K, V rows: [64][D], padded rows
    static constexpr int RT = padded_tile_bytes<SR, kQ_N>();
    static constexpr int ST = RowPad<kQ_N>::STRIDE;       // K^T of one half: [DH][64], padded rows
    static constexpr int TT = padded_tile_bytes<ST, kSplitDH>();
    static constexpr int KR = 0, VR = RT, KT = 2 * RT;
    static constexpr int LDS = 2 * RT + TT;               // one stage
    using PlanR = CopyPlan<D, SR, kQ_N, 4>;
    using PlanT = CopyPlan<kQ_N, ST, kSplitDH, 4>;
    using Addr = LaneAddr<SR, PadRows<ST>>;
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int D>
struct QSplitState {
    u32x4 qf[D / 16], dof[D / 16];                 // Q, dO as the B operand (all columns)
    f32x16 dq[kSplitDH / 32], pk[kSplitDH / 32];   // dQ^T, PK^T of this workgroup's half
    float l2, dd, dacc;                             // LSE log2 e, D 2^sS, running sum of P dP'
};

// One tile of 64 keys, every entry masked as in dq_masked; the exact row dot
// sums over all columns of dP, so both halves form the same value. Phase A:
// S and dP over all columns for keys 0-31, then keys 32-63 with the softmax of
// keys 0-31 spread over those MFMAs; `mid` runs; phase B: PK^T += K^T P^T and
// dQ^T += K^T dS^T over this half's columns for keys 0-31 with the softmax of
// keys 32-63 spread over them, then for keys 32-63.
template <int D, bool WIN, class MID>
__device__ __forceinline__ void dq_split_step(QSplitState<D>& S, const FA_LDS uint8_t* __restrict__ cur,
                                              const typename QSplitCfg<D>::Addr& la, int key0, int qrow, int N,
                                              bool causal, float sl2, float c1, int hh, int lbq, int ubq,
                                              const MID& mid) {
    using C = QSplitCfg<D>;
    constexpr int DS = C::DS, DBH = C::DBH;
    f32x16 s[2], dp[2];
    u32x4 pp[4], dsp[4];
    // register i of keys kb*32..: key key0 + kb*32 + (i/4)*8 + hh*4 + i%4
    auto soft = [&](auto kbc, auto ic) {
        constexpr int kb = decltype(kbc)::value, i = decltype(ic)::value;
        constexpr int kc = 2 * kb + i / 8, w = (i % 8) / 2;
        const int kk = key0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
        float x = fast_exp2(fmaf(s[kb][i], sl2, -S.l2));
        if (kk >= N || (causal && kk > qrow) || (WIN && (kk < lbq || kk >= ubq))) x = 0.f;
        const float dpv = dp[kb][i];
        S.dacc = fmaf(x, dpv, S.dacc);
        s[kb][i] = x;
        dp[kb][i] = x * fmaf(dpv, c1, -S.dd);
        if constexpr (i & 1) {
            pp[kc][w] = pack_f16(s[kb][i - 1], s[kb][i]);
            dsp[kc][w] = pack_f16(dp[kb][i - 1], dp[kb][i]);
        }
    };
    s[0] = zero16();
    dp[0] = zero16();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
        s[0] = mfma32h(lds_read16b(cur, la.row(0, ds) + C::KR), S.qf[ds], s[0]);
        dp[0] = mfma32h(lds_read16b(cur, la.row(0, ds) + C::VR), S.dof[ds], dp[0]);
    }
    s[1] = zero16();
    dp[1] = zero16();
    // operands read PF slots ahead of their MFMA (a scheduling barrier closes
    // every slot)
    constexpr int PF = 2;
    u32x4 ra[PF + 1][2];
    auto read_a = [&](auto dc) {
        constexpr int ds = decltype(dc)::value;
        ra[ds % (PF + 1)][0] = lds_read16b(cur, la.row(1, ds) + C::KR);
        ra[ds % (PF + 1)][1] = lds_read16b(cur, la.row(1, ds) + C::VR);
    };
    static_for<PF>([&](auto dc) { read_a(dc); });
    static_for<DS>([&](auto dc) {
        constexpr int ds = decltype(dc)::value;
        if constexpr (ds + PF < DS) read_a(std::integral_constant<int, ds + PF>{});
        s[1] = mfma32h(ra[ds % (PF + 1)][0], S.qf[ds], s[1]);
        dp[1] = mfma32h(ra[ds % (PF + 1)][1], S.dof[ds], dp[1]);
        static_for<16 / DS>([&](auto k) { soft(std::integral_constant<int, 0>{}, std::integral_constant<int, ds * (16 / DS) + decltype(k)::value>{}); });
        __builtin_amdgcn_sched_barrier(0);
    });
    mid();
    u32x4 rb[PF + 1];
    auto read_b = [&](auto mc) {
        constexpr int m = decltype(mc)::value, kc = m / DBH, db = m % DBH;
        rb[m % (PF + 1)] = la.t.read(cur + C::KT, db * 32, kc);
    };
    static_for<PF>([&](auto mc) { read_b(mc); });
    static_for<2 * DBH>([&](auto mc) {
        constexpr int m = decltype(mc)::value, kc = m / DBH, db = m % DBH;
        if constexpr (m + PF < 2 * DBH) read_b(std::integral_constant<int, m + PF>{});
        S.pk[db] = mfma32h(rb[m % (PF + 1)], pp[kc], S.pk[db]);
        S.dq[db] = mfma32h(rb[m % (PF + 1)], dsp[kc], S.dq[db]);
        static_for<16 / (2 * DBH)>([&](auto k) { soft(std::integral_constant<int, 1>{}, std::integral_constant<int, m * (16 / (2 * DBH)) + decltype(k)::value>{}); });
        __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int kc = 2; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < DBH; ++db) {
            const u32x4 a = la.t.read(cur + C::KT, db * 32, kc);
            S.pk[db] = mfma32h(a, pp[kc], S.pk[db]);
            S.dq[db] = mfma32h(a, dsp[kc], S.dq[db]);
        }
}

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_split_kernel(BwdParams p) {
    using C = QSplitCfg<D>;
    constexpr int DS = C::DS, DBH = C::DBH;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];
    FA_LDS uint8_t* cur = (FA_LDS uint8_t*)smem;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N, Np = p.Np;
    const bool causal = p.causal != 0;
    const int nqt = (N + kQ_WG - 1) / kQ_WG;
    int rank, unit;
    unmap_block_unit_major(blockIdx.x, p.B * p.Hq * 2, nqt, rank, unit);
    const int half = unit & 1, bh = unit >> 1;
    const int qt = causal ? nqt - 1 - rank : rank;
    const int b = bh / p.Hq, hq = bh - b * p.Hq;
    const size_t bkv = (size_t)b * p.Hkv + hq / p.G;
    const BufRes rk = make_bufres(p.k16 + bkv * Np * D, (uint32_t)Np * D * 2);
    const BufRes rv = make_bufres(p.v16 + bkv * Np * D, (uint32_t)Np * D * 2);
    const BufRes rkt = make_bufres(p.kT16 + (bkv * D + half * kSplitDH) * Np, (uint32_t)Np * kSplitDH * 2);
    const float sl2 = p.scales[0], c1 = p.scales[1];

    const int q0 = qt * kQ_WG, r0 = q0 + w * kQ_W, qrow = r0 + l32;   // qrow < Np
    const int ntk = (N + kQ_N - 1) / kQ_N;
    const Bounds bd{p.cu_seqlens, p.nseq, p.window, N};
    const bool ubnd = WIN && !causal;
    auto ub_of = [&](int r) { return bd.row_end(min(r, N - 1)); };
    const int nt = causal ? min(ntk, (q0 + kQ_WG - 1) / kQ_N + 1)
                          : (ubnd ? max(1, min(ntk, (ub_of(q0 + kQ_WG - 1) + kQ_N - 1) / kQ_N)) : ntk);
    const int jst = WIN ? max(0, bd.first_key(q0)) / kQ_N : 0;
    const int lbq = WIN ? bd.first_key(qrow) : 0;
    const int ubq = ubnd ? bd.row_end(qrow) : N;

    QSplitState<D> S;
    {
        const size_t ro = ((size_t)bh * Np + qrow) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            S.qf[ds] = *reinterpret_cast<const u32x4*>(p.q16 + ro + ds * 16 + hh * 8);
            S.dof[ds] = *reinterpret_cast<const u32x4*>(p.do16 + ro + ds * 16 + hh * 8);
        }
        S.l2 = p.lse2[(size_t)bh * Np + qrow];
        S.dd = p.delta[(size_t)bh * Np + qrow];
        S.dacc = 0.f;
    }
#pragma unroll
    for (int db = 0; db < DBH; ++db) {
        S.dq[db] = zero16();
        S.pk[db] = zero16();
    }
    typename C::PlanR pr;
    typename C::PlanT pt;
    pr.init(w, lane, D);
    pt.init(w, lane, Np);
    typename C::Addr la;
    la.init(l32, hh);
    // K, V rows of key tile j (2 * NT loads per wave), this half's K^T (NT)
    auto copy_rows = [&](int j) {
        pr.copy(rk, (uint32_t)j * kQ_N * D * 2, cur + C::KR, w);
        pr.copy(rv, (uint32_t)j * kQ_N * D * 2, cur + C::VR, w);
    };
    auto copy_tr = [&](int j) { pt.copy(rkt, (uint32_t)j * kQ_N * 2, cur + C::KT, w); };
    if (jst < nt) {
        copy_rows(jst);
        copy_tr(jst);
    }
    for (int j = jst; j < nt; ++j) {
        wait_vmem_n<C::PlanT::NT>();      // this tile's rows (its K^T may be in flight)
        __syncthreads();
        dq_split_step<D, WIN>(S, cur, la, j * kQ_N, qrow, N, causal, sl2, c1, hh, lbq, ubq, [&]() {
            wait_vmem();                  // this tile's K^T
            __syncthreads();              // ... everywhere, and the row tiles are free
            if (j + 1 < nt) copy_rows(j + 1);
        });
        __syncthreads();                  // K^T is free
        if (j + 1 < nt) copy_tr(j + 1);
    }
    const float dx = (S.dacc + swap_half(S.dacc)) * c1;
    if (qrow < N) {
        const int dr = p.d;
        uint16_t* dQg = p.dq + ((size_t)bh * N + qrow) * dr + half * kSplitDH;
        const float sc = p.scales[4];
        const float corr = S.dd - dx;
#pragma unroll
        for (int db = 0; db < DBH; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float v4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v4[t] = fmaf(corr, S.pk[db][u * 4 + t], S.dq[db][u * 4 + t]) * sc;
                u32x2 val;
                val[0] = pack_bf16(v4[0], v4[1]);
                val[1] = pack_bf16(v4[2], v4[3]);
                if (half * kSplitDH + db * 32 + u * 8 + hh * 4 < dr)
                    *reinterpret_cast<u32x2*>(dQg + db * 32 + u * 8 + hh * 4) = val;
            }
        // both halves form the same value; one stores it for the dK/dV kernel
        if (hh == 0 && half == 0) p.delta[(size_t)bh * Np + qrow] = dx;
    }
}

// ---------------------------------------------------------------- launchers
template <int D>
hipError_t launch_prep_t(const BwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_max_kernel, dim3(p.npart), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long tiles = 2LL * p.B * (p.Hq + p.Hkv) * (p.Np / 64);
    const int grid = (int)(tiles < 8192 ? tiles : 8192);
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// The eight-wave d = 128 gradient kernels cover 256 keys (rows) per
// workgroup, twice the four-wave ones, and hold one workgroup per CU. Below
// two such workgroups per compute unit the grid leaves CUs idle through the
// causal tail, and the four-wave form (twice the workgroups) measured faster:
// grids of 64 to 256 eight-wave workgroups ran 19-48% slower than the
// four-wave form, while grids of 512 or more ran 3-8% faster.
constexpr int kEightWaveMinGrid = 512;
inline bool use_eight_wave(int grid8) { return grid8 >= kEightWaveMinGrid; }

template <int D>
hipError_t launch_dkdv_t(const BwdParams& p, hipStream_t stream) {
    const bool bounded = p.window > 0 || p.cu_seqlens;
    if constexpr (D == 128) {   // the eight-wave form on large grids
        const int grid = p.B * p.Hkv * ((p.N + kKV8_WG - 1) / kKV8_WG);
        if (!use_eight_wave(grid)) {
            const int grid4 = p.B * p.Hkv * ((p.N + kKV_WG - 1) / kKV_WG);
            if (bounded)
                hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3(grid4), dim3(kThreads), 0, stream, p);
            else
                hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3(grid4), dim3(kThreads), 0, stream, p);
            return hipGetLastError();
        }
        if (bounded)
            hipLaunchKernelGGL((bwd_dkdv8_kernel<D, true>), dim3(grid), dim3(kThreads8), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_dkdv8_kernel<D, false>), dim3(grid), dim3(kThreads8), 0, stream, p);
    } else {
        const int grid = p.B * p.Hkv * ((p.N + kKV_WG - 1) / kKV_WG);
        if (bounded)
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_dq_t(const BwdParams& p, hipStream_t stream) {
    const bool bounded = p.window > 0 || p.cu_seqlens;
    if constexpr (D == 128) {   // the eight-wave form on large grids
        const int grid = p.B * p.Hq * ((p.N + kQ8_WG - 1) / kQ8_WG);
        if (!use_eight_wave(grid)) {
            const int grid4 = p.B * p.Hq * ((p.N + kQ_WG - 1) / kQ_WG);
            if (bounded)
                hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3(grid4), dim3(kThreads), 0, stream, p);
            else
                hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3(grid4), dim3(kThreads), 0, stream, p);
            return hipGetLastError();
        }
        if (bounded)
            hipLaunchKernelGGL((bwd_dq8_kernel<D, true>), dim3(grid), dim3(kThreads8), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_dq8_kernel<D, false>), dim3(grid), dim3(kThreads8), 0, stream, p);
    } else {
        const int grid = p.B * p.Hq * ((p.N + kQ_WG - 1) / kQ_WG);
        if (bounded)
            hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_split_t(const BwdParams& p, hipStream_t stream) {
    const int grid = p.B * p.Hkv * 2 * ((p.N + kKV_WG - 1) / kKV_WG);
    if (p.window > 0 || p.cu_seqlens)
        hipLaunchKernelGGL((bwd_dkdv_split_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_dkdv_split_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dq_split_t(const BwdParams& p, hipStream_t stream) {
    const int grid = p.B * p.Hq * 2 * ((p.N + kQ_WG - 1) / kQ_WG);
    if (p.window > 0 || p.cu_seqlens)
        hipLaunchKernelGGL((bwd_dq_split_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_dq_split_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

BwdWorkspace bwd_workspace_layout(int B, int Hq, int Hkv, int N, int d) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BwdWorkspace w;
    w.Np = (N + kRowPad - 1) / kRowPad * kRowPad;
    const size_t rows = (size_t)B * Hq * w.Np;
    const size_t Dp = (size_t)padded_dim(d);   // the copies hold D = padded_dim(d) columns
    const size_t nq = rows * Dp, nk = (size_t)B * Hkv * w.Np * Dp;
    const size_t chunks = (size_t)B * Hq * N * d / 8;
    const size_t want = (chunks + kThreads - 1) / kThreads;
    w.npart = (int)(want < 1024 ? (want > 0 ? want : 1) : 1024);
    size_t off = 0;
    w.delta = off; off += up(rows * 4);
    w.lse2 = off; off += up(rows * 4);
    w.q16 = off; off += up(nq * 2);
    w.k16 = off; off += up(nk * 2);
    w.v16 = off; off += up(nk * 2);
    w.do16 = off; off += up(nq * 2);
    w.qT16 = off; off += up(nq * 2);
    w.doT16 = off; off += up(nq * 2);
    w.kT16 = off; off += up(nk * 2);
    w.part = off; off += up((size_t)4 * w.npart * 4);
    w.scales = off; off += 256;
    w.total = off;
    return w;
}

hipError_t launch_bwd_stage(const BwdParams& p, int stage, hipStream_t stream) {
    if (padded_dim(p.d) == 256) {
        if (stage == 0) return launch_prep_t<256>(p, stream);
        if (stage == 1) return launch_dq_split_t<256>(p, stream);
        return launch_dkdv_split_t<256>(p, stream);
    }
    const bool d128 = padded_dim(p.d) == 128;
    if (stage == 0) return d128 ? launch_prep_t<128>(p, stream) : launch_prep_t<64>(p, stream);
    if (stage == 1) return d128 ? launch_dq_t<128>(p, stream) : launch_dq_t<64>(p, stream);
    return d128 ? launch_dkdv_t<128>(p, stream) : launch_dkdv_t<64>(p, stream);
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
    for (int stage = 0; stage < 3; ++stage) {
        const hipError_t e = launch_bwd_stage(p, stage, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fa
