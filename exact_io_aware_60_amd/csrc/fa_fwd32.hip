// fa_fwd32.hip -- forward pass of exact attention on fp32 inputs.
//
// The same computation as the bf16 forward (mlapandio "FlashAttention: IO-aware
// exact attention", "Four ideas": K/V tiles streamed on chip, a running max and
// sum per row, O rescaled exactly, one logsumexp per row written), for callers
// whose Q, K and V are fp32 and should not be rounded to bf16 first: O and the
// logsumexp come out in fp32.
//
// gfx950 design:
//  * Both products on v_mfma_f32_32x32x2_f32 (fp32 operands, fp32
//    accumulation): Sᵀ = K·Qᵀ takes d/2 instructions per 32x32 block and
//    Oᵀ += Vᵀ·Pᵀ 16 per 32 columns of d. Lane l supplies row l % 32 and k slot
//    l / 32 of each operand.
//  * A wave holds 32 query rows; Q sits in registers as the B operand (d/2
//    values per lane: columns 2s + l/32). Four waves share 32-key tiles of K
//    (stored transposed, 32 keys + 1 pad per row) and V (rows padded by 8
//    floats, so the two lane halves, 4 keys apart, read disjoint banks),
//    loaded with 16-byte global reads.
//  * The scores keep the C layout: lane l holds query l % 32 and keys
//    (r / 4) * 8 + (l / 32) * 4 + r % 4 of register r. Those registers are the
//    B operand of P·V as they stand, with the A operand reading the same keys
//    of V, so P never leaves its registers.
//  * Online softmax in the textbook form: the running max is exact, the
//    correction exp2(m_old - m_new) is applied to O and the sum at every tile.
//  * Causal: tiles past a wave's last row are skipped; the diagonal and the
//    ragged last tile are masked.
//  * Several workgroups per CU (34 KiB of LDS each at d = 128, 17 KiB at
//    d = 64): the launch bounds ask for two at d = 128 (192 registers, two
//    waves per SIMD) and three at d = 64 (122 registers, which lets four run).
//    Each wave's score and P.V products are chains of dependent fp32 MFMAs,
//    so more waves per SIMD hide their latency. Measured on MI355X against one
//    workgroup per CU (286 registers at d = 128): 61.1 -> 46.0 ms on a
//    2 x 32-head, 16384-row causal forward, 0.613 -> 0.563 ms on 4 x 16 heads
//    of 2048 rows at d = 64, same results bit for bit. Three per CU at
//    d = 128 spills (168 registers): 49.3 ms.
// Head dimensions: any multiple of 8 up to 128 (zero columns past d).
#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int k32Waves = 4;
constexpr int k32Threads = 64 * k32Waves;
constexpr int k32WM = 32;                       // query rows per wave
constexpr int k32BM = k32WM * k32Waves;         // query rows per workgroup
constexpr int k32BN = 32;                       // keys per tile

template <int D>
struct F32Cfg {
    static constexpr int KP = k32BN + 1;        // Kᵀ tile row pitch (floats)
    static constexpr int VP = D + 8;            // V tile row pitch (floats)
    static constexpr int KT = D * KP;           // floats
    static constexpr int VT = k32BN * VP;
    static constexpr int NB = D / 32;           // 32-column blocks of O
};

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// key (within a 32-key tile) held by register r of lane half hh
__device__ __forceinline__ int key_of(int r, int hh) { return (r >> 2) * 8 + hh * 4 + (r & 3); }

template <int D>
__global__ __launch_bounds__(k32Threads, D == 64 ? 3 : 2) void fwd32_kernel(Fwd32Params p) {
    using C = F32Cfg<D>;
    __shared__ float Kt[C::KT];
    __shared__ __attribute__((aligned(16))) float Vs[C::VT];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int N = p.N, d = p.d;
    const bool causal = p.causal != 0;
    const int nqt = (N + k32BM - 1) / k32BM;
    const int bh = blockIdx.x / nqt;
    const int qt = causal ? nqt - 1 - (blockIdx.x - bh * nqt) : blockIdx.x - bh * nqt;   // heavy tiles first
    const int b = bh / p.Hq, hq = bh - b * p.Hq;
    const int bkv = b * p.Hkv + hq / p.G;
    const int q0 = qt * k32BM, r0 = q0 + w * k32WM, qrow = r0 + l32;
    const int ntk = (N + k32BN - 1) / k32BN;
    const int nt = causal ? min(ntk, (q0 + k32BM - 1) / k32BN + 1) : ntk;   // tiles the workgroup needs
    const int last = causal ? min(ntk - 1, (r0 + k32WM - 1) / k32BN) : ntk - 1;
    const bool wave_valid = r0 < N;

    // Q row qrow, columns 2s + hh, as the B operand (zeros past d and N)
    float qf[D / 2];
    {
        const float* Qg = p.q + ((size_t)bh * N + min(qrow, N - 1)) * d;
        const bool ok = qrow < N;
#pragma unroll
        for (int c4 = 0; c4 < D / 4; ++c4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (ok && c4 * 4 < d) x = *reinterpret_cast<const float4*>(Qg + c4 * 4);
            qf[2 * c4] = hh ? x.y : x.x;
            qf[2 * c4 + 1] = hh ? x.w : x.z;
        }
    }

    const float* Kg = p.k + (size_t)bkv * N * d;
    const float* Vg = p.v + (size_t)bkv * N * d;
    f32x16 o[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) o[nb] = zero16();
    float m = -INFINITY, l = 0.f;

    for (int j = 0; j < nt; ++j) {
        __syncthreads();   // the previous tile is no longer read
        // 32 keys x D columns of K (transposed) and V, 16 bytes per thread and step
#pragma unroll
        for (int c = tid; c < k32BN * D / 4; c += k32Threads) {
            const int key = c / (D / 4), col = (c - key * (D / 4)) * 4;
            const int gk = j * k32BN + key;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (gk < N && col < d) {
                kx = *reinterpret_cast<const float4*>(Kg + (size_t)gk * d + col);
                vx = *reinterpret_cast<const float4*>(Vg + (size_t)gk * d + col);
            }
            Kt[(col + 0) * C::KP + key] = kx.x;
            Kt[(col + 1) * C::KP + key] = kx.y;
            Kt[(col + 2) * C::KP + key] = kx.z;
            Kt[(col + 3) * C::KP + key] = kx.w;
            *reinterpret_cast<float4*>(&Vs[key * C::VP + col]) = vx;
        }
        __syncthreads();
        if (!wave_valid || j > last) continue;

        // Sᵀ = K·Qᵀ: lane holds query l32, keys key_of(r, hh)
        f32x16 s = zero16();
#pragma unroll
        for (int k2 = 0; k2 < D / 2; ++k2) s = mfma_f32(Kt[(2 * k2 + hh) * C::KP + l32], qf[k2], s);

        const bool masked = (causal && j == last) || (j + 1) * k32BN > N;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = s[r] * p.scale_log2;
            if (masked) {
                const int key = j * k32BN + key_of(r, hh);
                if (key >= N || (causal && key > qrow)) x = -INFINITY;
            }
            s[r] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, swap_half(mx));
        const float mn = fmaxf(m, mx);
        // a row that has seen no key yet keeps m = -inf and weight 0
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = mn == -INFINITY ? 0.f : fast_exp2(s[r] - mn);
            s[r] = e;
            ls += e;
        }
        m = mn;
        l = fmaf(l, alpha, ls);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) o[nb][i] *= alpha;
        }
        // Oᵀ += Vᵀ·Pᵀ over the tile's 32 keys, k slots (register r, lane half)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float* vrow = &Vs[key_of(r, hh) * C::VP + l32];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) o[nb] = mfma_f32(vrow[nb * 32], s[r], o[nb]);
        }
    }

    if (wave_valid && qrow < N) {
        const float lt = l + swap_half(l);
        const float inv = 1.f / lt;
        float* Og = p.o + ((size_t)bh * N + qrow) * d;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = nb * 32 + g * 8 + hh * 4;
                if (col < d)
                    *reinterpret_cast<float4*>(Og + col) = make_float4(o[nb][g * 4] * inv, o[nb][g * 4 + 1] * inv,
                                                                      o[nb][g * 4 + 2] * inv, o[nb][g * 4 + 3] * inv);
            }
        if (hh == 0) p.lse[(size_t)bh * N + qrow] = (m + __log2f(lt)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd32(const Fwd32Params& p, hipStream_t stream) {
    const int grid = p.B * p.Hq * ((p.N + k32BM - 1) / k32BM);
    if (p.d <= 64)
        hipLaunchKernelGGL((fwd32_kernel<64>), dim3(grid), dim3(k32Threads), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd32_kernel<128>), dim3(grid), dim3(k32Threads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
