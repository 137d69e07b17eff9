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
// Two passes, no atomics: the dK/dV kernel owns a block of keys and walks the
// query rows; the dQ kernel owns a block of query rows and walks the keys. Each
// output element is written once, so results are bit-reproducible. The cost is
// recomputing S and dP in the dQ pass.
//
// Data flow per kernel, using v_mfma_f32_32x32x16_bf16 for every product (the
// operand layouts are listed in fa_device.h):
//  * dK/dV: a workgroup of 4 waves owns 128 keys, 32 per wave, held in
//    registers as MFMA operands. Per step it streams 64 query rows of Q and dO
//    (plus their LSE and D) through double-buffered LDS. S = Q K^T and
//    dP = dO V^T leave one key per lane and 16 query rows per lane, which after
//    rounding to bf16 are directly the operands of dV^T += dO^T P and
//    dK^T += Q^T dS. dO^T and Q^T come from the LDS transpose read.
//  * dQ: a workgroup of 4 waves owns 256 query rows (64 per wave, Q and dO in
//    registers) and streams 32-key tiles of K and V through double-buffered LDS.
//    S^T = K Q^T and dP^T = V dO^T leave one query row per lane, and dS^T in
//    bf16 feeds dQ^T += K^T dS^T with K^T from the LDS transpose read.
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

// ---------------------------------------------------------------- row dot
// D_i = sum_c dO_ic O_ic in fp32, and L2_i = LSE_i * log2(e). D / 8 lanes share
// one row (16 bytes each); grid-stride over rows.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                           const uint16_t* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           float* __restrict__ delta,
                                                           float* __restrict__ lse2, long long rows) {
    constexpr int LPR = D / 8;
    constexpr int RPB = kThreads / LPR;
    const int sub = threadIdx.x % LPR;
    for (long long base = (long long)blockIdx.x * RPB; base < rows; base += (long long)gridDim.x * RPB) {
        const long long row = base + threadIdx.x / LPR;
        float acc = 0.f;
        if (row < rows) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + sub * 8);
            const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + sub * 8);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc = fmaf(bf16_lo(a[t]), bf16_lo(g[t]), acc);
                acc = fmaf(bf16_hi(a[t]), bf16_hi(g[t]), acc);
            }
        }
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (row < rows && sub == 0) {
            delta[row] = acc;
            lse2[row] = lse[row] * kLog2e;
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
                                          int q0, int key, int N, float sl2, int lane) {
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
            s[qb] = mfma32(lds_read16(Qt, off), kf[ds], s[qb]);
            dp[qb] = mfma32(lds_read16(dOt, off), vf[ds], dp[qb]);
        }

    // P = exp2(S * scale * log2e - L2), dS = P (dP - D).
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
                dp[qb][i] = x * (dp[qb][i] - dv4[t]);
            }
        }

    // bf16 operands. k slot t of chunk qc is query row qc*16 + (t/4)*8 + hh*4 + t%4,
    // which is register (qc & 1) * 8 + t of block qc >> 1.
    u32x4 pp[4], dsp[4];
#pragma unroll
    for (int qc = 0; qc < 4; ++qc)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = (qc & 1) * 8 + 2 * t;
            pp[qc][t] = pack_bf16(s[qc >> 1][i], s[qc >> 1][i + 1]);
            dsp[qc][t] = pack_bf16(dp[qc >> 1][i], dp[qc >> 1][i + 1]);
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
            dv[db] = mfma32(cat(lds_read_tr(dOt, o0), lds_read_tr(dOt, o1)), pp[qc], dv[db]);
            dk[db] = mfma32(cat(lds_read_tr(Qt, o0), lds_read_tr(Qt, o1)), dsp[qc], dk[db]);
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
    const uint16_t* Kg = p.k + (size_t)bkv * N * D;
    const uint16_t* Vg = p.v + (size_t)bkv * N * D;

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
        const uint16_t* Qg = p.q + bh * N * D;
        const uint16_t* dOg = p.dout + bh * N * D;
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
                                 p.scale_log2, lane);
        }
        wait_vmem();
        __syncthreads();
    }

    // dK^T / dV^T blocks: lane holds key l32, d rows db*32 + u*8 + hh*4 + 0..3.
    if (key < N) {
        uint16_t* dKg = p.dk + (size_t)bkv * N * D + (size_t)key * D;
        uint16_t* dVg = p.dv + (size_t)bkv * N * D + (size_t)key * D;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 a, c;
                a[0] = pack_bf16(dk[db][u * 4 + 0] * sc, dk[db][u * 4 + 1] * sc);
                a[1] = pack_bf16(dk[db][u * 4 + 2] * sc, dk[db][u * 4 + 3] * sc);
                c[0] = pack_bf16(dv[db][u * 4 + 0], dv[db][u * 4 + 1]);
                c[1] = pack_bf16(dv[db][u * 4 + 2], dv[db][u * 4 + 3]);
                *reinterpret_cast<u32x2*>(dKg + db * 32 + u * 8 + hh * 4) = a;
                *reinterpret_cast<u32x2*>(dVg + db * 32 + u * 8 + hh * 4) = c;
            }
    }
}

// ---------------------------------------------------------------- dQ
constexpr int kQ_WG = 256;  // query rows per workgroup
constexpr int kQ_W = 64;    // query rows per wave
constexpr int kQ_N = 32;    // keys per tile

// One key tile for one wave: S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_tile(const FA_LDS uint16_t* Kt, const FA_LDS uint16_t* Vt,
                                        const u32x4 (&qf)[2][D / 16], const u32x4 (&of)[2][D / 16],
                                        f32x16 (&dq)[D / 32][2], const float (&l2)[2],
                                        const float (&dd)[2], bool masked, int key0, int r0, int N,
                                        float sl2, int lane) {
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
            s[qb] = mfma32(ka, qf[qb][ds], s[qb]);
            dp[qb] = mfma32(va, of[qb][ds], dp[qb]);
        }
    }

    u32x4 dsp[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = r0 + qb * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = fast_exp2(fmaf(s[qb][i], sl2, -l2[qb]));
            if (masked) {
                const int kk = key0 + (i >> 2) * 8 + hh * 4 + (i & 3);
                if (kk >= N || (CAUSAL && kk > q)) x = 0.f;
            }
            dp[qb][i] = x * (dp[qb][i] - dd[qb]);
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                dsp[qb][kc][t] = pack_bf16(dp[qb][kc * 8 + 2 * t], dp[qb][kc * 8 + 2 * t + 1]);
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
            for (int qb = 0; qb < 2; ++qb) dq[db][qb] = mfma32(a, dsp[qb][kc], dq[db][qb]);
        }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdParams p) {
    constexpr int CPR = D / 8, DS = D / 16, DB = D / 32;
    constexpr int TILE = kQ_N * D;
    constexpr int LCH = kQ_N * CPR / kThreads;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];
    FA_LDS uint16_t* Ks = (FA_LDS uint16_t*)smem;
    FA_LDS uint16_t* Vs = Ks + 2 * TILE;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N;
    const int nqt = (N + kQ_WG - 1) / kQ_WG;
    int rank, bh;
    unmap_block(blockIdx.x, p.B * p.Hq, rank, bh);
    const int qt = CAUSAL ? nqt - 1 - rank : rank;
    const int b = bh / p.Hq, hq = bh - b * p.Hq, hkv = hq / p.G;
    const uint16_t* Qg = p.q + (size_t)bh * N * D;
    const uint16_t* dOg = p.dout + (size_t)bh * N * D;
    const uint16_t* Kg = p.k + ((size_t)b * p.Hkv + hkv) * N * D;
    const uint16_t* Vg = p.v + ((size_t)b * p.Hkv + hkv) * N * D;

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

    // Q and dO as the B operand: lane holds query column l32 of block qb, d = ds*16 + hh*8 .. +7.
    u32x4 qf[2][DS], of[2][DS];
    float l2[2], dd[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qrow = r0 + qb * 32 + l32;
        const bool ok = qrow < N;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            qf[qb][ds] = gload16(Qg + (size_t)qrow * D + ds * 16 + hh * 8, ok);
            of[qb][ds] = gload16(dOg + (size_t)qrow * D + ds * 16 + hh * 8, ok);
        }
        l2[qb] = ok ? p.lse2[(size_t)bh * N + qrow] : 0.f;
        dd[qb] = ok ? p.delta[(size_t)bh * N + qrow] : 0.f;
    }
    f32x16 dq[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) dq[db][qb] = zero16();

    issue_tile(0, 0);
    wait_vmem();
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        if (j + 1 < nt) issue_tile(j + 1, buf ^ 1);
        if (wave_valid && j <= wave_last) {
            const int key0 = j * kQ_N;
            const bool masked = (CAUSAL && key0 + kQ_N - 1 > r0) || (key0 + kQ_N > N);
            dq_tile<D, CAUSAL>(Ks + buf * TILE, Vs + buf * TILE, qf, of, dq, l2, dd, masked, key0, r0,
                               N, p.scale_log2, lane);
        }
        wait_vmem();
        __syncthreads();
    }

    if (wave_valid) {
        uint16_t* dQg = p.dq + (size_t)bh * N * D;
        const float sc = p.scale;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qrow = r0 + qb * 32 + l32;
            if (qrow < N) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        u32x2 val;
                        val[0] = pack_bf16(dq[db][qb][u * 4 + 0] * sc, dq[db][qb][u * 4 + 1] * sc);
                        val[1] = pack_bf16(dq[db][qb][u * 4 + 2] * sc, dq[db][qb][u * 4 + 3] * sc);
                        *reinterpret_cast<u32x2*>(dQg + (size_t)qrow * D + db * 32 + u * 8 + hh * 4) = val;
                    }
            }
        }
    }
}

// ---------------------------------------------------------------- launchers
template <int D>
hipError_t launch_pre_t(const BwdParams& p, hipStream_t stream) {
    const long long rows = (long long)p.B * p.Hq * p.N;
    constexpr int RPB = kThreads / (D / 8);
    const long long want = (rows + RPB - 1) / RPB;
    const int grid = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, p.o, p.dout, p.lse,
                       p.delta, p.lse2, rows);
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

size_t bwd_workspace_bytes(long long rows) {
    const size_t one = ((size_t)rows * sizeof(float) + 255) & ~(size_t)255;
    return 2 * one;
}

hipError_t launch_bwd_stage(const BwdParams& p, int stage, hipStream_t stream) {
    const bool c = p.causal != 0;
    if (stage == 0) return p.d == 128 ? launch_pre_t<128>(p, stream) : launch_pre_t<64>(p, stream);
    if (stage == 1) {
        if (p.d == 128) return c ? launch_dkdv_t<128, true>(p, stream) : launch_dkdv_t<128, false>(p, stream);
        return c ? launch_dkdv_t<64, true>(p, stream) : launch_dkdv_t<64, false>(p, stream);
    }
    if (p.d == 128) return c ? launch_dq_t<128, true>(p, stream) : launch_dq_t<128, false>(p, stream);
    return c ? launch_dq_t<64, true>(p, stream) : launch_dq_t<64, false>(p, stream);
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
    for (int stage = 0; stage < 3; ++stage) {
        const hipError_t e = launch_bwd_stage(p, stage, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fa
