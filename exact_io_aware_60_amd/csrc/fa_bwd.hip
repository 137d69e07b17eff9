// fa_bwd.hip -- backward pass of exact attention on gfx950.
//
// Method: the forward keeps only O and one logsumexp per query row; the
// backward rebuilds every probability from them, P_ij = exp(S_ij - LSE_i),
// instead of reading a stored score matrix (mlapandio "FlashAttention: IO-aware
// exact attention", "Four ideas", recomputation item; techtrendtracker "Flash
// Attention: memory-efficient transformers", "Recomputation in the Backward
// Pass"). The gradient formulas are the chain rule of softmax attention for the
// loss sum(dO * O):
//   D_i   = sum_c dO_ic O_ic                 (row dot, first kernel)
//   dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij q_i   (second kernel)
//   dQ_i  = scale sum_j dS_ij k_j                              (third kernel)
// dK and dV sum over the query heads that share the K/V head.
//
// Precision. The four products that take P or dS as an operand run on fp16
// MFMA operands. fp16 keeps 11 significant bits where bf16 keeps 8, at the same
// MFMA rate, so rounding P and dS costs 8x less accuracy. The first kernel
// finds max |x| of q, k, v and dout. A preparation kernel then writes fp16
// copies of them scaled by powers of two (max |x| * scale lies in
// [2^13, 2^14)), so every bf16 value converts exactly. It also derives a scale
// for dS from the bound |dS_ij| <= 2 d max|dO| max|V|. The scales are undone
// in fp32 in each epilogue.
//
// The row dot D. The forward stores O in bf16, and its P.V product rounds P to
// bf16, so a D formed from the stored O is off by about one bf16 ulp of O per
// element. dS = P (dP - D) turns that into dQ and dK errors of several 1e-2
// when the softmax is peaked. The dQ kernel therefore also sums the exact row
// dot D'_i = sum_j P_ij dP_ij from the probabilities it rebuilds, together
// with PK_i = sum_j P_ij k_j. dS is linear in D, so dQ computed with the
// approximate D plus (D - D') PK equals dQ computed with D'. The dK/dV kernel
// runs after it and uses D'.
//
// Two passes, no atomics: the dQ kernel owns a block of query rows and walks the
// keys; the dK/dV kernel owns a block of keys and walks the query rows. Each
// output element is written once, so results are bit-reproducible. The cost is
// recomputing S and dP in the dQ pass.
//
// Data flow per kernel, using 32x32x16 MFMA for every product (the
// operand layouts are listed in fa_device.h):
//  * dQ: a workgroup of 4 waves owns 256 query rows (64 per wave). Their Q and
//    dO rows sit in LDS for the whole kernel, and 32-key tiles of K and V
//    stream through double-buffered LDS. S^T = K Q^T and dP^T = V dO^T leave
//    one query row per lane, and dS^T and P^T in fp16 feed dQ^T += K^T dS^T and
//    PK^T += K^T P^T, with K^T from the LDS transpose read.
//  * dK/dV: a workgroup of 4 waves owns 128 keys, 32 per wave, held in
//    registers as MFMA operands. Per step it streams 64 query rows of Q and dO
//    (plus their LSE and D) through double-buffered LDS. S = Q K^T and
//    dP = dO V^T leave one key per lane and 16 query rows per lane, which after
//    rounding to fp16 are directly the operands of dV^T += dO^T P and
//    dK^T += Q^T dS. dO^T and Q^T come from the LDS transpose read.
// Both kernels skip the tiles that the causal mask hides completely, mask the
// diagonal and ragged tiles element-wise, and run the heaviest workgroups
// first.
#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int kThreads = 256;

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

// Scales, fp16 copies, and per row D * 2^sS and LSE * log2(e).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdParams p) {
    __shared__ uint32_t red[4];
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
    constexpr int LOG2D = D == 128 ? 7 : 6;
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
    for (int t = 0; t < 4; ++t) {
        const uint16_t* src;
        uint16_t* dst;
        long long chunks;
        prep_tensor(p, t, src, dst, chunks);
        const float f = ldexpf(1.f, sx[t]);
        for (long long c = (long long)blockIdx.x * kThreads + threadIdx.x; c < chunks;
             c += (long long)gridDim.x * kThreads) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(src + c * 8);
            u32x4 y;
#pragma unroll
            for (int u = 0; u < 4; ++u) y[u] = pack_f16(bf16_lo(x[u]) * f, bf16_hi(x[u]) * f);
            *reinterpret_cast<u32x4*>(dst + c * 8) = y;
        }
    }
    // Row dot: D / 8 lanes share one row (16 bytes each).
    constexpr int LPR = D / 8;
    constexpr int RPB = kThreads / LPR;
    const float fS = ldexpf(1.f, sS);
    const long long rows = (long long)p.B * p.Hq * p.N;
    const int sub = threadIdx.x % LPR;
    for (long long base = (long long)blockIdx.x * RPB; base < rows; base += (long long)gridDim.x * RPB) {
        const long long row = base + threadIdx.x / LPR;
        float acc = 0.f;
        if (row < rows) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(p.o + row * D + sub * 8);
            const u32x4 g = *reinterpret_cast<const u32x4*>(p.dout + row * D + sub * 8);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc = fmaf(bf16_lo(a[t]), bf16_lo(g[t]), acc);
                acc = fmaf(bf16_hi(a[t]), bf16_hi(g[t]), acc);
            }
        }
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (row < rows && sub == 0) {
            p.delta[row] = acc * fS;
            p.lse2[row] = p.lse[row] * kLog2e;
        }
    }
}

// ---------------------------------------------------------------- dK / dV
constexpr int kKV_WG = 128;  // keys per workgroup
constexpr int kKV_W = 32;    // keys per wave
constexpr int kKV_Q = 64;    // query rows per step

// One step for one wave: 64 query rows against the wave's 32 keys.
// Qt/dOt: [64][D] bf16 tiles (swizzle mode 2), L2t/Dt: 64 floats.
// `key` is this lane's key; `masked` is set when the step touches the causal
// diagonal or a ragged edge.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_step(const FA_LDS uint16_t* Qt, const FA_LDS uint16_t* dOt,
                                          const FA_LDS float* L2t, const FA_LDS float* Dt,
                                          const u32x4 (&kf)[D / 16], const u32x4 (&vf)[D / 16],
                                          f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], bool masked,
                                          int q0, int key, int N, float sl2, float c1, int lane) {
    constexpr int DS = D / 16, DB = D / 32;
    const int l32 = lane & 31, hh = lane >> 5;

    // S = Q K^T and dP = dO V^T: lane holds key column l32, rows qb*32 + (i/4)*8 + hh*4 + i%4.
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
            const int off = swz<D, 2>(qb * 32 + l32, ds * 2 + hh);
            s[qb] = mfma32h(lds_read16(Qt, off), kf[ds], s[qb]);
            dp[qb] = mfma32h(lds_read16(dOt, off), vf[ds], dp[qb]);
        }

    // P = exp2(S * scale * log2e - L2); dS * 2^sS = P (dP' * c1 - D * 2^sS).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = qb * 32 + u * 8 + hh * 4;
            const f32x4 lv = *reinterpret_cast<const FA_LDS f32x4*>(L2t + r);
            const f32x4 dv4 = *reinterpret_cast<const FA_LDS f32x4*>(Dt + r);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = u * 4 + t;
                float x = fast_exp2(fmaf(s[qb][i], sl2, -lv[t]));
                if (masked) {
                    const int q = q0 + r + t;
                    if (key >= N || q >= N || (CAUSAL && key > q)) x = 0.f;
                }
                s[qb][i] = x;
                dp[qb][i] = x * fmaf(dp[qb][i], c1, -dv4[t]);
            }
        }

    // fp16 operands. k slot t of chunk qc is query row qc*16 + (t/4)*8 + hh*4 + t%4,
    // which is register (qc & 1) * 8 + t of block qc >> 1.
    u32x4 pp[4], dsp[4];
#pragma unroll
    for (int qc = 0; qc < 4; ++qc)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = (qc & 1) * 8 + 2 * t;
            pp[qc][t] = pack_f16(s[qc >> 1][i], s[qc >> 1][i + 1]);
            dsp[qc][t] = pack_f16(dp[qc >> 1][i], dp[qc >> 1][i + 1]);
        }

    // dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T read transposed in the same row order.
    const int g = lane >> 4;
#pragma unroll
    for (int qc = 0; qc < 4; ++qc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int dcol = db * 32 + (g & 1) * 16 + 4 * (lane & 3);
            const int qrow = qc * 16 + (g >> 1) * 4 + ((lane & 15) >> 2);
            const int o0 = swz<D, 2>(qrow, dcol >> 3) + (dcol & 7);
            const int o1 = swz<D, 2>(qrow + 8, dcol >> 3) + (dcol & 7);
            dv[db] = mfma32h(cat(lds_read_tr(dOt, o0), lds_read_tr(dOt, o1)), pp[qc], dv[db]);
            dk[db] = mfma32h(cat(lds_read_tr(Qt, o0), lds_read_tr(Qt, o1)), dsp[qc], dk[db]);
        }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
    constexpr int CPR = D / 8, DS = D / 16, DB = D / 32;
    constexpr int QT = kKV_Q * D;                  // elements per Q or dO tile
    constexpr int LCH = kKV_Q * CPR / kThreads;    // chunks each thread copies per tile
    constexpr int STAGE = 2 * QT + 4 * kKV_Q;      // Q, dO, then 64 floats of L2 and of D
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N, G = p.G;
    const int nkt = (N + kKV_WG - 1) / kKV_WG;
    int kt, bkv;
    unmap_block(blockIdx.x, p.B * p.Hkv, kt, bkv);  // kt = 0 first: the most query rows when causal
    const int b = bkv / p.Hkv, hkv = bkv - b * p.Hkv;
    (void)nkt;
    const int k0 = kt * kKV_WG;
    const int kw0 = k0 + w * kKV_W;
    const int key = kw0 + l32;
    const uint16_t* Kg = p.k16 + (size_t)bkv * N * D;
    const uint16_t* Vg = p.v16 + (size_t)bkv * N * D;
    const float sl2 = p.scales[0], c1 = p.scales[1];

    // K and V as the B operand of S = Q K^T and dP = dO V^T: lane holds key
    // column l32 and d = ds*16 + hh*8 .. +7. Keys past N read row N-1 (masked later).
    u32x4 kf[DS], vf[DS];
    {
        const size_t kr = (size_t)min(key, N - 1) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            kf[ds] = *reinterpret_cast<const u32x4*>(Kg + kr + ds * 16 + hh * 8);
            vf[ds] = *reinterpret_cast<const u32x4*>(Vg + kr + ds * 16 + hh * 8);
        }
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = zero16();
        dv[db] = zero16();
    }

    const int qs = CAUSAL ? k0 : 0;                 // rows before the block's first key see none of it
    const int nqs = (N - qs + kKV_Q - 1) / kKV_Q;   // query steps per head
    const int nsteps = G * nqs;

    // Copy step j (head g, rows q0..q0+63) into stage `buf`. Rows past N read
    // row N-1; their probabilities are masked to zero.
    auto issue = [&](int j, int buf) {
        const int g = j / nqs;
        const int q0 = qs + (j - g * nqs) * kKV_Q;
        const size_t bh = (size_t)b * p.Hq + (size_t)hkv * G + g;
        const uint16_t* Qg = p.q16 + bh * N * D;
        const uint16_t* dOg = p.do16 + bh * N * D;
        FA_LDS uint16_t* st = (FA_LDS uint16_t*)smem + buf * STAGE;
#pragma unroll
        for (int u = 0; u < LCH; ++u) {
            const int slot = u * kThreads + tid;
            int row, c;
            unswz<D, 2>(slot, row, c);
            const size_t src = (size_t)min(q0 + row, N - 1) * D + c * 8;
            gload_lds16(Qg + src, st + (u * kThreads + w * 64) * 8);
            gload_lds16(dOg + src, st + QT + (u * kThreads + w * 64) * 8);
        }
        const size_t r = bh * N + min(q0 + lane, N - 1);
        if (w == 0) gload_lds4(p.lse2 + r, (FA_LDS float*)(st + 2 * QT));
        if (w == 1) gload_lds4(p.delta + r, (FA_LDS float*)(st + 2 * QT) + kKV_Q);
    };

    issue(0, 0);
    wait_vmem();
    __syncthreads();
    for (int j = 0; j < nsteps; ++j) {
        const int buf = j & 1;
        if (j + 1 < nsteps) issue(j + 1, buf ^ 1);
        const int g = j / nqs;
        const int q0 = qs + (j - g * nqs) * kKV_Q;
        const bool active = kw0 < N && (!CAUSAL || q0 + kKV_Q - 1 >= kw0);
        if (active) {
            const bool masked = (CAUSAL && kw0 + kKV_W - 1 > q0) || (q0 + kKV_Q > N) || (kw0 + kKV_W > N);
            const FA_LDS uint16_t* st = (const FA_LDS uint16_t*)smem + buf * STAGE;
            const FA_LDS float* lt = (const FA_LDS float*)(st + 2 * QT);
            dkdv_step<D, CAUSAL>(st, st + QT, lt, lt + kKV_Q, kf, vf, dk, dv, masked, q0, key, N,
                                 sl2, c1, lane);
        }
        wait_vmem();
        __syncthreads();
    }

    // dK^T / dV^T blocks: lane holds key l32, d rows db*32 + u*8 + hh*4 + 0..3.
    if (key < N) {
        uint16_t* dKg = p.dk + (size_t)bkv * N * D + (size_t)key * D;
        uint16_t* dVg = p.dv + (size_t)bkv * N * D + (size_t)key * D;
        const float fk = p.scales[3], fv = p.scales[2];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 a, c;
                a[0] = pack_bf16(dk[db][u * 4 + 0] * fk, dk[db][u * 4 + 1] * fk);
                a[1] = pack_bf16(dk[db][u * 4 + 2] * fk, dk[db][u * 4 + 3] * fk);
                c[0] = pack_bf16(dv[db][u * 4 + 0] * fv, dv[db][u * 4 + 1] * fv);
                c[1] = pack_bf16(dv[db][u * 4 + 2] * fv, dv[db][u * 4 + 3] * fv);
                *reinterpret_cast<u32x2*>(dKg + db * 32 + u * 8 + hh * 4) = a;
                *reinterpret_cast<u32x2*>(dVg + db * 32 + u * 8 + hh * 4) = c;
            }
    }
}

// ---------------------------------------------------------------- dQ
constexpr int kQ_WG = 256;  // query rows per workgroup
constexpr int kQ_W = 64;    // query rows per wave
constexpr int kQ_N = 32;    // keys per tile

// One key tile for one wave: S^T = K Q^T, dP^T = V dO^T, then
//   dQ^T += K^T dS^T   with dS formed from the preparation's D (from the stored O),
//   PK^T += K^T P^T    and D'_i += sum_j P_ij dP_ij (the exact row dot).
// The epilogue corrects dQ by (D - D') PK, which is exact because dS is linear in D.
// Q and dO are read from the workgroup's LDS copies (Qw, dOw).
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_tile(const FA_LDS uint16_t* Kt, const FA_LDS uint16_t* Vt,
                                        const FA_LDS uint16_t* dOw, const FA_LDS uint16_t* Qw,
                                        f32x16 (&dq)[D / 32][2], f32x16 (&pk)[D / 32][2],
                                        float (&dacc)[2], const float (&l2)[2], const float (&dd)[2],
                                        bool masked, int key0, int r0, int wrow0, int N, float sl2,
                                        float c1, int lane) {
    constexpr int DS = D / 16, DB = D / 32;
    const int l32 = lane & 31, hh = lane >> 5;

    // lane holds query column l32 of block qb, keys (i/4)*8 + hh*4 + i%4.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        s[qb] = zero16();
        dp[qb] = zero16();
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
        const u32x4 ka = lds_read16(Kt, swz<D, 2>(l32, ds * 2 + hh));
        const u32x4 va = lds_read16(Vt, swz<D, 0>(l32, ds * 2 + hh));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int off = swz<D, 0>(wrow0 + qb * 32 + l32, ds * 2 + hh);
            s[qb] = mfma32h(ka, lds_read16(Qw, off), s[qb]);
            dp[qb] = mfma32h(va, lds_read16(dOw, off), dp[qb]);
        }
    }

    // P and dS, packed to fp16 pairs as soon as each pair is ready.
    u32x4 dsp[2][2], pp[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = r0 + qb * 32 + l32;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            float x[2], y[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float xe = fast_exp2(fmaf(s[qb][i + e], sl2, -l2[qb]));
                if (masked) {
                    const int kk = key0 + ((i + e) >> 2) * 8 + hh * 4 + ((i + e) & 3);
                    if (kk >= N || (CAUSAL && kk > q)) xe = 0.f;
                }
                const float t = dp[qb][i + e] * c1;     // dP * 2^sS
                acc = fmaf(xe, t, acc);
                x[e] = xe;
                y[e] = xe * (t - dd[qb]);
            }
            pp[qb][i >> 3][(i & 7) >> 1] = pack_f16(x[0], x[1]);
            dsp[qb][i >> 3][(i & 7) >> 1] = pack_f16(y[0], y[1]);
        }
        dacc[qb] += acc;
    }

    const int g = lane >> 4;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int dcol = db * 32 + (g & 1) * 16 + 4 * (lane & 3);
            const int krow = kc * 16 + (g >> 1) * 4 + ((lane & 15) >> 2);
            const u32x4 a = cat(lds_read_tr(Kt, swz<D, 2>(krow, dcol >> 3) + (dcol & 7)),
                                lds_read_tr(Kt, swz<D, 2>(krow + 8, dcol >> 3) + (dcol & 7)));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                dq[db][qb] = mfma32h(a, dsp[qb][kc], dq[db][qb]);
                pk[db][qb] = mfma32h(a, pp[qb][kc], pk[db][qb]);
            }
        }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdParams p) {
    constexpr int CPR = D / 8, DS = D / 16, DB = D / 32;
    constexpr int TILE = kQ_N * D;
    constexpr int LCH = kQ_N * CPR / kThreads;
    constexpr int OCH = kQ_WG * CPR / kThreads;    // dO chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE + 2 * kQ_WG * D];
    FA_LDS uint16_t* Ks = (FA_LDS uint16_t*)smem;
    FA_LDS uint16_t* Vs = Ks + 2 * TILE;
    FA_LDS uint16_t* dOs = Ks + 4 * TILE;
    FA_LDS uint16_t* Qs = dOs + kQ_WG * D;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N;
    const int nqt = (N + kQ_WG - 1) / kQ_WG;
    int rank, bh;
    unmap_block(blockIdx.x, p.B * p.Hq, rank, bh);
    const int qt = CAUSAL ? nqt - 1 - rank : rank;
    const int b = bh / p.Hq, hq = bh - b * p.Hq, hkv = hq / p.G;
    const uint16_t* Qg = p.q16 + (size_t)bh * N * D;
    const uint16_t* dOg = p.do16 + (size_t)bh * N * D;
    const uint16_t* Kg = p.k16 + ((size_t)b * p.Hkv + hkv) * N * D;
    const uint16_t* Vg = p.v16 + ((size_t)b * p.Hkv + hkv) * N * D;
    const float sl2 = p.scales[0], c1 = p.scales[1];

    const int q0 = qt * kQ_WG;
    const int r0 = q0 + w * kQ_W;
    const int ntk = (N + kQ_N - 1) / kQ_N;
    const int nt = CAUSAL ? min(ntk, (q0 + kQ_WG - 1) / kQ_N + 1) : ntk;
    const bool wave_valid = r0 < N;
    const int wave_last = CAUSAL ? min(ntk - 1, (r0 + kQ_W - 1) / kQ_N) : ntk - 1;

    auto issue_tile = [&](int j, int buf) {
#pragma unroll
        for (int u = 0; u < LCH; ++u) {
            const int slot = u * kThreads + tid;
            int row, c;
            unswz<D, 2>(slot, row, c);
            gload_lds16(Kg + (size_t)min(j * kQ_N + row, N - 1) * D + c * 8,
                        Ks + buf * TILE + (u * kThreads + w * 64) * 8);
            unswz<D, 0>(slot, row, c);
            gload_lds16(Vg + (size_t)min(j * kQ_N + row, N - 1) * D + c * 8,
                        Vs + buf * TILE + (u * kThreads + w * 64) * 8);
        }
    };

    // The workgroup's Q and dO rows, once (rows past N read row N-1; never stored).
    // Both are read as the B operand: lane holds query column l32 of a 32-row
    // block, d = ds*16 + hh*8 .. +7.
#pragma unroll
    for (int u = 0; u < OCH; ++u) {
        const int slot = u * kThreads + tid;
        int row, c;
        unswz<D, 0>(slot, row, c);
        const size_t src = (size_t)min(q0 + row, N - 1) * D + c * 8;
        gload_lds16(dOg + src, dOs + (u * kThreads + w * 64) * 8);
        gload_lds16(Qg + src, Qs + (u * kThreads + w * 64) * 8);
    }

    float l2[2], dd[2], dacc[2] = {0.f, 0.f};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qrow = r0 + qb * 32 + l32;
        const bool ok = qrow < N;
        l2[qb] = ok ? p.lse2[(size_t)bh * N + qrow] : 0.f;
        dd[qb] = ok ? p.delta[(size_t)bh * N + qrow] : 0.f;
    }
    f32x16 dq[DB][2], pk[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            dq[db][qb] = zero16();
            pk[db][qb] = zero16();
        }

    issue_tile(0, 0);
    wait_vmem();
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        if (j + 1 < nt) issue_tile(j + 1, buf ^ 1);
        if (wave_valid && j <= wave_last) {
            const int key0 = j * kQ_N;
            const bool masked = (CAUSAL && key0 + kQ_N - 1 > r0) || (key0 + kQ_N > N);
            dq_tile<D, CAUSAL>(Ks + buf * TILE, Vs + buf * TILE, dOs, Qs, dq, pk, dacc, l2, dd, masked,
                               key0, r0, w * kQ_W, N, sl2, c1, lane);
        }
        wait_vmem();
        __syncthreads();
    }

    if (wave_valid) {
        uint16_t* dQg = p.dq + (size_t)bh * N * D;
        const float sc = p.scales[4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qrow = r0 + qb * 32 + l32;
            // exact row dot (both lane halves hold half of the keys), in units of 2^sS
            const float dx = dacc[qb] + swap_half(dacc[qb]);
            const float corr = dd[qb] - dx;
            if (qrow < N) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        float v4[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            v4[t] = fmaf(corr, pk[db][qb][u * 4 + t], dq[db][qb][u * 4 + t]) * sc;
                        u32x2 val;
                        val[0] = pack_bf16(v4[0], v4[1]);
                        val[1] = pack_bf16(v4[2], v4[3]);
                        *reinterpret_cast<u32x2*>(dQg + (size_t)qrow * D + db * 32 + u * 8 + hh * 4) = val;
                    }
                if (hh == 0) p.delta[(size_t)bh * N + qrow] = dx;   // for the dK/dV kernel
            }
        }
    }
}

// ---------------------------------------------------------------- launchers
template <int D>
hipError_t launch_prep_t(const BwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_max_kernel, dim3(p.npart), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long chunks = (long long)p.B * p.Hq * p.N * D / 8;
    const long long want = (chunks + kThreads - 1) / kThreads;
    const int grid = (int)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdParams& p, hipStream_t stream) {
    const int grid = p.B * p.Hkv * ((p.N + kKV_WG - 1) / kKV_WG);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdParams& p, hipStream_t stream) {
    const int grid = p.B * p.Hq * ((p.N + kQ_WG - 1) / kQ_WG);
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

BwdWorkspace bwd_workspace_layout(int B, int Hq, int Hkv, int N, int d) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t rows = (size_t)B * Hq * N;
    const size_t nq = rows * d, nk = (size_t)B * Hkv * N * d;
    BwdWorkspace w;
    const size_t chunks = nq / 8;
    const size_t want = (chunks + kThreads - 1) / kThreads;
    w.npart = (int)(want < 1024 ? (want > 0 ? want : 1) : 1024);
    size_t off = 0;
    w.delta = off; off += up(rows * 4);
    w.lse2 = off; off += up(rows * 4);
    w.q16 = off; off += up(nq * 2);
    w.k16 = off; off += up(nk * 2);
    w.v16 = off; off += up(nk * 2);
    w.do16 = off; off += up(nq * 2);
    w.part = off; off += up((size_t)4 * w.npart * 4);
    w.scales = off; off += 256;
    w.total = off;
    return w;
}

hipError_t launch_bwd_stage(const BwdParams& p, int stage, hipStream_t stream) {
    const bool c = p.causal != 0;
    if (stage == 0) return p.d == 128 ? launch_prep_t<128>(p, stream) : launch_prep_t<64>(p, stream);
    if (stage == 1) {
        if (p.d == 128) return c ? launch_dq_t<128, true>(p, stream) : launch_dq_t<128, false>(p, stream);
        return c ? launch_dq_t<64, true>(p, stream) : launch_dq_t<64, false>(p, stream);
    }
    if (p.d == 128) return c ? launch_dkdv_t<128, true>(p, stream) : launch_dkdv_t<128, false>(p, stream);
    return c ? launch_dkdv_t<64, true>(p, stream) : launch_dkdv_t<64, false>(p, stream);
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
    for (int stage = 0; stage < 3; ++stage) {
        const hipError_t e = launch_bwd_stage(p, stage, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fa
