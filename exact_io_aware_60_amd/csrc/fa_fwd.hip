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
// this kernel's own):
//  * One workgroup = 4 waves = 256 query rows. Each wave owns 64 rows, and one
//    wave runs per SIMD with up to 512 registers. 64 rows per wave halve the LDS
//    bytes per MFMA flop against 32-row waves. That matters because every wave
//    reads the whole K and V tile out of LDS.
//  * Keys are streamed in tiles of 64. K and V tiles are double-buffered in LDS
//    (64 KiB at d = 128). The next tile is loaded into registers while the
//    current one is computed, then written to the other buffer. One barrier per
//    tile.
//  * The scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16. A lane then holds one query row and 16 keys per
//    32 x 32 block. The row max needs a single cross-lane step (lane l with
//    l ^ 32), and the fp32 accumulator registers become, after rounding to
//    bf16, the B operand of O^T += V^T P^T with no data movement. V^T is read
//    with ds_read_b64_tr_b16 in the matching key order.
//  * exp2 with scale * log2(e) folded into one FMA. The reference max moves
//    only when a tile's max exceeds it by more than 2^8; otherwise the rescale
//    of O is skipped. Any reference value cancels in O / l and m + ln l, so the
//    result is the same (the fp64 model in oracle/online.py checks this).
//  * Causal: tiles above a wave's diagonal are skipped; the diagonal tile and
//    the ragged last tile are masked element-wise. Workgroups run heaviest
//    q-tile first (longest-processing-time order). Workgroups of one head set
//    map to one XCD, so their K/V re-reads hit the same L2.
#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int kBM = 256;       // query rows per workgroup
constexpr int kWM = 64;        // query rows per wave
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves
constexpr float kTau = 8.0f;   // lazy-max threshold, log2 units

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

// One key tile for one wave: S^T = K Q^T, mask, online-softmax update, O^T += V^T P^T.
// `masked` (uniform over the wave) is set for the diagonal tile under the causal
// mask and for the ragged last tile. Masked scores become -inf; with a positive
// scale_log2 (the host keeps it >= 1e-30) they turn into exact zeros.
template <int D, bool CAUSAL>
__device__ __forceinline__ void fwd_tile(const FA_LDS uint16_t* Kt, const FA_LDS uint16_t* Vt,
                                         const u32x4 (&qf)[2][D / 16], f32x16 (&o)[D / 32][2],
                                         float (&m)[2], float (&l)[2], bool masked, int key0, int r0,
                                         int N, float sl2, int lane) {
    constexpr int DS = D / 16, DB = D / 32;
    const int l32 = lane & 31, hh = lane >> 5;

    f32x16 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb][qb] = zero16();

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            const u32x4 a = lds_read16(Kt, swz<D, 0>(kb * 32 + l32, ds * 2 + hh));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma32(a, qf[qb][ds], s[kb][qb]);
        }

    if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
                    const int qrow = r0 + qb * 32 + l32;
                    if (key >= N || (CAUSAL && key > qrow)) s[kb][qb][i] = -INFINITY;
                }
    }

    // Row max of this tile, in log2 units; every active tile has a visible key per row.
    float mc[2];
    bool need[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        mx = fmaxf(mx, swap_half(mx));
        mc[qb] = mx * sl2;
        need[qb] = mc[qb] > m[qb] + kTau;
    }
    if (__ballot(need[0] || need[1])) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float mn = need[qb] ? mc[qb] : m[qb];
            const float alpha = fast_exp2(m[qb] - mn);
            l[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][qb][i] *= alpha;
            m[qb] = mn;
        }
    }

    // P~ = exp2(scale*log2e*S - m), row sums, and the bf16 B operand of the next product.
    u32x4 pp[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float x = fast_exp2(fmaf(s[kb][qb][i], sl2, -m[qb]));
                s[kb][qb][i] = x;
                ls += x;
            }
        l[qb] += ls;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                pp[qb][kc][t] = pack_bf16(s[kc >> 1][qb][(kc & 1) * 8 + 2 * t],
                                          s[kc >> 1][qb][(kc & 1) * 8 + 2 * t + 1]);
    }

    // O^T += V^T P^T. k slot s of chunk kc is key kc*16 + (s/4)*8 + hh*4 + s%4.
    const int g = lane >> 4;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int dcol = db * 32 + (g & 1) * 16 + 4 * (lane & 3);
            const int krow = kc * 16 + (g >> 1) * 4 + ((lane & 15) >> 2);
            const u32x2 t0 = lds_read_tr(Vt, swz<D, 1>(krow, dcol >> 3) + (dcol & 7));
            const u32x2 t1 = lds_read_tr(Vt, swz<D, 1>(krow + 8, dcol >> 3) + (dcol & 7));
            const u32x4 a = cat(t0, t1);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) o[db][qb] = mfma32(a, pp[qb][kc], o[db][qb]);
        }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdParams p) {
    constexpr int CPR = D / 8;                   // 16-byte chunks per row
    constexpr int DS = D / 16, DB = D / 32;
    constexpr int TILE = kBN * D;                // elements per K or V tile
    constexpr int LCH = kBN * CPR / kThreads;    // chunks each thread copies per tile
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];
    FA_LDS uint16_t* Ks = (FA_LDS uint16_t*)smem;
    FA_LDS uint16_t* Vs = Ks + 2 * TILE;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N;
    const int nqt = (N + kBM - 1) / kBM;
    int rank, bh;
    unmap_block(blockIdx.x, p.B * p.Hq, rank, bh);
    const int qt = CAUSAL ? nqt - 1 - rank : rank;
    const int b = bh / p.Hq, hq = bh - b * p.Hq, hkv = hq / p.G;
    const uint16_t* Qg = p.q + (size_t)bh * N * D;
    const uint16_t* Kg = p.k + ((size_t)b * p.Hkv + hkv) * N * D;
    const uint16_t* Vg = p.v + ((size_t)b * p.Hkv + hkv) * N * D;

    const int q0 = qt * kBM;
    const int r0 = q0 + w * kWM;
    const int ntk = (N + kBN - 1) / kBN;
    const int nt = CAUSAL ? min(ntk, (q0 + kBM - 1) / kBN + 1) : ntk;
    const bool wave_valid = r0 < N;
    const int wave_last = CAUSAL ? min(ntk - 1, r0 / kBN) : ntk - 1;

    // Copy K/V tile j into LDS buffer `buf`. Thread chunk u fills 16-byte slot
    // u*256 + tid; the global chunk is the one the swizzle puts there. Rows past
    // N read row N-1 (finite data, and their scores are masked).
    auto issue_tile = [&](int j, int buf) {
#pragma unroll
        for (int u = 0; u < LCH; ++u) {
            const int slot = u * kThreads + tid;
            FA_LDS uint16_t* kdst = Ks + buf * TILE + (u * kThreads + w * 64) * 8;
            FA_LDS uint16_t* vdst = Vs + buf * TILE + (u * kThreads + w * 64) * 8;
            int row, c;
            unswz<D, 0>(slot, row, c);
            gload_lds16(Kg + (size_t)min(j * kBN + row, N - 1) * D + c * 8, kdst);
            unswz<D, 1>(slot, row, c);
            gload_lds16(Vg + (size_t)min(j * kBN + row, N - 1) * D + c * 8, vdst);
        }
    };

    u32x4 qf[2][DS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qrow = r0 + qb * 32 + l32;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            qf[qb][ds] = gload16(Qg + (size_t)qrow * D + ds * 16 + hh * 8, qrow < N);
    }

    f32x16 o[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) o[db][qb] = zero16();
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

    issue_tile(0, 0);
    wait_vmem();
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        if (j + 1 < nt) issue_tile(j + 1, buf ^ 1);
        if (wave_valid && j <= wave_last) {
            const int key0 = j * kBN;
            const bool masked = (CAUSAL && key0 + kBN - 1 > r0) || (key0 + kBN > N);
            fwd_tile<D, CAUSAL>(Ks + buf * TILE, Vs + buf * TILE, qf, o, m, l, masked, key0, r0, N,
                                p.scale_log2, lane);
        }
        wait_vmem();
        __syncthreads();
    }

    if (wave_valid) {
        uint16_t* Og = p.o + (size_t)bh * N * D;
        float* Lg = p.lse + (size_t)bh * N;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float lt = l[qb] + swap_half(l[qb]);
            const float inv = 1.f / lt;
            const int qrow = r0 + qb * 32 + l32;
            if (qrow < N) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        u32x2 val;
                        val[0] = pack_bf16(o[db][qb][u * 4 + 0] * inv, o[db][qb][u * 4 + 1] * inv);
                        val[1] = pack_bf16(o[db][qb][u * 4 + 2] * inv, o[db][qb][u * 4 + 3] * inv);
                        *reinterpret_cast<u32x2*>(Og + (size_t)qrow * D + db * 32 + u * 8 + hh * 4) = val;
                    }
                if (hh == 0) Lg[qrow] = (m[qb] + __log2f(lt)) * kLn2;
            }
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
    const int nqt = (p.N + kBM - 1) / kBM;
    const int grid = p.B * p.Hq * nqt;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

Geometry fwd_geometry(int B, int Hq, int N, int d, int causal) {
    (void)causal;
    Geometry g;
    g.block_m = kBM;
    g.block_n = kBN;
    g.threads = kThreads;
    g.grid = B * Hq * ((N + kBM - 1) / kBM);
    g.lds_bytes = 4 * kBN * d * 2;
    return g;
}

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
    if (p.d == 128) return p.causal ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
    return p.causal ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
}

}  // namespace fa
