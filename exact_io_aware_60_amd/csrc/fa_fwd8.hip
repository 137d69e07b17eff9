// fa_fwd8.hip -- forward pass of exact attention on 8-bit floating-point inputs.
//
// FlashAttention-3 runs its forward pass in FP8 with block scaling (mlapandio
// "FlashAttention: IO-aware exact attention", "Generations"; wishwiki
// "FlashAttention", "Evolution: FlashAttention-2 and -3"), and the first page's
// "Honest limits" notes that FP8 changes the rounding. This kernel takes Q, K
// and V as OCP E4M3 codes with one fp32 scale per run of R rows of each head
// (flash_attn_quantize_e4m3; V in the transposed layout of
// flash_attn_quantize_e4m3_vt), computes softmax(scale * Q K^T) V of the
// dequantised values code * scale, and writes O in bf16 and the logsumexp.
//
// gfx950 design:
//  * Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
//    scales: twice the bf16 MFMA rate (64 cycles for 4x the work of a 32-cycle
//    32x32x16 bf16 MFMA, measured). A lane's 32 operand bytes sit at the k
//    slots (lane half, byte): the same slot in A and B (checked on MI355X),
//    so any assignment of keys or columns to (half, byte) that both operands
//    share is a valid product.
//  * S^T = K Q^T over 64 columns per MFMA: byte b of lane half hh holds column
//    hh * 32 + b of a 64-column block, in K (from LDS) and Q (registers) alike.
//    As in the bf16 forward, a lane then holds one query row and 16 keys of a
//    32-key half: keys (i / 4) * 8 + hh * 4 + i % 4 of register i.
//  * O^T += V^T P^T over 64 keys per MFMA: byte b = c * 16 + i of lane half hh
//    holds the probability of key c * 32 + (i / 4) * 8 + hh * 4 + i % 4 (half c,
//    register i: the score registers, converted in register order). The
//    quantiser writes V transposed with each group of 64 keys in that order,
//    so the V^T operand is two 16-byte LDS reads per lane.
//  * Block scales in fp32: the score scale s_q * s_k * scale * log2(e) is one
//    FMA with the reference, and the V scale enters as an offset of the exp:
//    exp2(x + log2(s_v / s_vmax)) = P * s_v / s_vmax, so the probabilities the
//    MFMA takes already carry V's block scale relative to the head's largest
//    one (at most 1: the E4M3 range is kept for the largest values). O is
//    multiplied by s_vmax at the end.
//  * P is rounded to E4M3 (3 mantissa bits). O is divided by the sum of the
//    rounded probabilities as the products took them (an all-ones A operand
//    times P^T, one MFMA per 64 keys, divided by the tile's V scale ratio): the
//    weights then sum to one as used, and a dominant probability's rounding
//    cancels. The logsumexp takes the fp32 sum.
//  * The reference max follows the bf16 forward's rule with a tighter bound:
//    the first tile's exact max, then a new exact max only when some lane's
//    sum of its 32 probabilities (times the V ratio) passes 2^8, so every
//    E4M3 value stays at most 2^8 (the format's largest is 448).
//  * 12 waves of 32 query rows, three per SIMD (at most 168 registers each):
//    the kernel is bound by vector-ALU issue, and a third wave per SIMD
//    hides more of it under the matrix instructions than two (measured on
//    MI355X: 3.27 -> 2.86 ms on a 2 x 32-head, 16384-row causal forward,
//    though 14 registers spill at d = 128). 64-key tiles stream through LDS
//    with direct buffer->LDS loads into padded rows (K: D + 16 bytes, V^T: 80
//    bytes; 16-byte reads of 16 consecutive rows then hit distinct banks),
//    two buffers each, one barrier per tile.
//  * Causal: a wave skips tiles past its diagonal and masks the diagonal tile
//    and the ragged last tile; heaviest q-tiles first.
// Head dimensions 64 and 128; R a multiple of 64, so a wave's rows share one
// Q scale and a tile's keys one K and one V scale.
#include "fa_device.h"
#include "fa_params.h"

namespace fa {
namespace {

constexpr int k8Waves = 12;
constexpr int k8Threads = 64 * k8Waves;
constexpr int k8WM = 32;                   // query rows per wave
constexpr int k8BM = k8WM * k8Waves;       // query rows per workgroup
constexpr int k8BN = 64;                   // keys per tile
constexpr float k8SumMax = 256.0f;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16e __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
    // E4M3 operands (format 0) with unit E8M0 block scales (127 = 2^0)
    const f32x16e r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, __builtin_bit_cast(f32x16e, c), 0, 0,
                                                                      0, 127, 0, 127);
    return __builtin_bit_cast(f32x16, r);
}

__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
    i32x8 r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

template <int D>
struct F8Cfg {
    static constexpr int DK = D / 64;                         // score MFMAs per 32-key half
    static constexpr int DB = D / 32;                         // O^T blocks of 32 columns
    static constexpr int KS = D + 16;                         // K tile row stride (bytes)
    static constexpr int VS = k8BN + 16;                      // V^T tile row stride (bytes)
    static constexpr int KT = padded_tile_bytes<KS, k8BN>();
    static constexpr int VT = padded_tile_bytes<VS, D>();
    static constexpr int LDS = 2 * KT + 2 * VT;
    // copy plans count 16-bit units: a K row is D bytes, a V^T tile row 64
    using PlanK = CopyPlan<D / 2, KS, k8BN, k8Waves>;
    using PlanV = CopyPlan<k8BN / 2, VS, D, k8Waves>;
};

// Workgroup id -> (rank, bh); as in the bf16 forward, each XCD takes a
// contiguous block of heads when the head count is a multiple of 8.
__device__ __forceinline__ void unmap_block8(int bid, int nbh, int& rank, int& bh) {
    if ((nbh & 7) == 0) {
        const int x = bid & 7, r = bid >> 3, hpx = nbh >> 3;
        rank = r / hpx;
        bh = x * hpx + (r - rank * hpx);
    } else {
        rank = bid / nbh;
        bh = bid - rank * nbh;
    }
}

template <int D>
__device__ __forceinline__ f32x16 scores8(const FA_LDS uint8_t* Kt, int h, int l32, int hh, const i32x8 (&qf)[D / 64]) {
    using C = F8Cfg<D>;
    f32x16 s = zero16();
#pragma unroll
    for (int db = 0; db < C::DK; ++db) {
        const FA_LDS uint8_t* a = Kt + (h * 32 + l32) * C::KS + db * 64 + hh * 32;
        s = mfma8(cat8(lds_read16b(a, 0), lds_read16b(a, 16)), qf[db], s);
    }
    return s;
}

template <int D>
__global__ __launch_bounds__(k8Threads, 1) void fwd8_kernel(Fwd8Params p) {
    using C = F8Cfg<D>;
    constexpr int DK = C::DK, DB = C::DB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];
    FA_LDS uint8_t* Ks = (FA_LDS uint8_t*)smem;          // 2 K tiles
    FA_LDS uint8_t* Vs = Ks + 2 * C::KT;                   // 2 V^T tiles

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const bool causal = p.causal != 0;
    const int N = p.N, Np = p.Np, R = p.rows;
    const int nqt = (N + k8BM - 1) / k8BM;
    int rank, bh;
    unmap_block8(blockIdx.x, p.B * p.Hq, rank, bh);
    const int qt = causal ? nqt - 1 - rank : rank;
    const int b = bh / p.Hq, hq = bh - b * p.Hq;
    const int bkv = b * p.Hkv + hq / p.G;
    const int q0 = qt * k8BM, r0 = q0 + w * k8WM, qrow = r0 + l32;
    const int ntk = (N + k8BN - 1) / k8BN;
    const int nt = causal ? min(ntk, (q0 + k8BM - 1) / k8BN + 1) : ntk;
    const bool wave_valid = r0 < N;
    const int last = causal ? min(ntk - 1, (r0 + k8WM - 1) / k8BN) : ntk - 1;   // this wave's last tile
    const int nrun = (N + R - 1) / R;

    // Q as the B operand: byte hh * 32 + b of each 64-column block
    i32x8 qf[DK];
    {
        const uint8_t* Qg = p.q + ((size_t)bh * N + qrow) * D;
#pragma unroll
        for (int db = 0; db < DK; ++db) {
            const bool ok = qrow < N;
            const u32x4 lo = ok ? *reinterpret_cast<const u32x4*>(Qg + db * 64 + hh * 32) : u32x4{0u, 0u, 0u, 0u};
            const u32x4 hi = ok ? *reinterpret_cast<const u32x4*>(Qg + db * 64 + hh * 32 + 16) : u32x4{0u, 0u, 0u, 0u};
            qf[db] = cat8(lo, hi);
        }
    }
    const float sq = p.q_scales[(size_t)bh * nrun + min(qrow, N - 1) / R];
    // the head's largest V scale: the V ratios s_v / s_vmax are at most 1
    float svmax = 0.f;
    for (int t = tid; t < nrun; t += k8Threads) svmax = fmaxf(svmax, p.v_scales[(size_t)bkv * nrun + t]);
    {
        __shared__ float red[k8Waves];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) svmax = fmaxf(svmax, __shfl_xor(svmax, off));
        if (lane == 0) red[w] = svmax;
        __syncthreads();
        svmax = red[0];
#pragma unroll
        for (int i = 1; i < k8Waves; ++i) svmax = fmaxf(svmax, red[i]);
    }

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16();
    float m = 0.f, l = 0.f, lsum = 0.f;
    const uint32_t one8 = 0x38383838u;   // E4M3 1.0 in every byte
    i32x8 ones = {(int)one8, (int)one8, (int)one8, (int)one8, (int)one8, (int)one8, (int)one8, (int)one8};

    const BufRes rk = make_bufres(p.k + (size_t)bkv * N * D, (uint32_t)N * D);
    const BufRes rv = make_bufres(p.vt + (size_t)bkv * D * Np, (uint32_t)D * Np);
    typename C::PlanK pk;
    typename C::PlanV pv;
    pk.init(w, lane, D / 2);
    pv.init(w, lane, Np / 2);
    pk.copy(rk, 0u, Ks, w);
    pv.copy(rv, 0u, Vs, w);
    wait_vmem();
    __syncthreads();

    // The K/V scale run of tile j: runs hold R / 64 whole tiles, so the run
    // advances by counting, and the values derived from its scales change
    // only at a run's first tile. The next run's scales are fetched a run
    // ahead (uniform addresses: scalar loads).
    const int tpr = R / k8BN;
    int run = 0, jr = 0;
    float sk_next = p.k_scales[(size_t)bkv * nrun], sv_next = p.v_scales[(size_t)bkv * nrun];
    float sk = 0.f, lrv = 0.f, inv_rv = 1.f;

    for (int j = 0; j < nt; ++j) {
        FA_LDS uint8_t* Kt = Ks + (j & 1) * C::KT;
        FA_LDS uint8_t* Vt = Vs + (j & 1) * C::VT;
        if (j + 1 < nt) {   // the next tile into the other buffers (uniform)
            pk.copy(rk, (uint32_t)(j + 1) * k8BN * D, Ks + ((j + 1) & 1) * C::KT, w);
            pv.copy(rv, (uint32_t)(j + 1) * k8BN, Vs + ((j + 1) & 1) * C::VT, w);
        }
        if (jr == 0) {
            sk = sk_next;
            const float sv = sv_next;
            lrv = __log2f(sv / svmax);       // <= 0: the run's V ratio, log2
            inv_rv = svmax / sv;
            if (run + 1 < nrun) {
                sk_next = p.k_scales[(size_t)bkv * nrun + run + 1];
                sv_next = p.v_scales[(size_t)bkv * nrun + run + 1];
            }
        }
        // the tile's body; MASKED for the diagonal and the ragged last tile
        auto tile = [&](auto masked_c) {
            constexpr bool MASKED = decltype(masked_c)::value;
            const float cs = sq * sk * p.scale_log2;     // score code units -> log2 units
                f32x16 s[2];
                s[0] = scores8<D>(Kt, 0, l32, hh, qf);
                s[1] = scores8<D>(Kt, 1, l32, hh, qf);
                if constexpr (MASKED) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = j * k8BN + h * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
                            if (key >= N || (causal && key > qrow)) s[h][i] = -INFINITY;
                        }
                }
                if (j == 0) {   // the first reference: this tile's exact (masked) max
                    float mx = -INFINITY;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
                    m = fmaxf(mx, swap_half(mx)) * cs;
                }
                // x = S cs - m + log2(s_v / s_vmax); P~ r = exp2(x)
                float ls = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        s[h][i] = fmaf(s[h][i], cs, lrv - m);
                        const float e = fast_exp2(s[h][i]);
                        ls += e;
                        s[h][i] = e;
                    }
                if (__ballot(!(ls <= k8SumMax))) {
                    // a new reference: the exact max (in units of P~), then O, l
                    // and the rounded sum rescaled and the exps redone
                    float mx = -INFINITY;
                    // recover x from the exps is not exact; recompute the scores
                    s[0] = scores8<D>(Kt, 0, l32, hh, qf);
                    s[1] = scores8<D>(Kt, 1, l32, hh, qf);
                    if constexpr (MASKED) {
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const int key = j * k8BN + h * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
                                if (key >= N || (causal && key > qrow)) s[h][i] = -INFINITY;
                            }
                    }
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
                    mx = fmaxf(mx, swap_half(mx)) * cs;
                    const float delta = fmaxf(mx - m, 0.f);
                    const float alpha = fast_exp2(-delta);
                    m += delta;
                    l *= alpha;
                    lsum *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
                    ls = 0.f;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const float e = fast_exp2(fmaf(s[h][i], cs, lrv - m));
                            ls += e;
                            s[h][i] = e;
                        }
                }
                // P~ r rounded to E4M3: byte c * 16 + i <- half c, register i
                i32x8 pp;
#pragma unroll
                for (int wd = 0; wd < 8; ++wd) {
                    const int h = wd >> 2, i = (wd & 3) * 4;
                    // the second conversion overwrites the other half, so the
                    // first one may write over its own (dead) input
                    int v = __builtin_amdgcn_cvt_pk_fp8_f32(s[h][i], s[h][i + 1], __float_as_int(s[h][i]), false);
                    v = __builtin_amdgcn_cvt_pk_fp8_f32(s[h][i + 2], s[h][i + 3], v, true);
                    pp[wd] = v;
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const FA_LDS uint8_t* a = Vt + (db * 32 + l32) * C::VS + hh * 32;
                    o[db] = mfma8(cat8(lds_read16b(a, 0), lds_read16b(a, 16)), pp, o[db]);
                }
                const f32x16 t = mfma8(ones, pp, zero16());
                lsum = fmaf(t[0], inv_rv, lsum);
                l = fmaf(ls, inv_rv, l);
        };
        if (wave_valid && j <= last) {
            if ((causal && j == last) || (j + 1) * k8BN > N) tile(std::true_type{});
            else tile(std::false_type{});
        }
        if (++jr == tpr) {
            jr = 0;
            ++run;
        }
        // d = 64: keeps the ones operand resident rather than rebuilt every
        // tile (at d = 128 its 8 registers would spill at three waves per SIMD)
        if constexpr (D == 64) asm volatile("" : "+v"(ones));
        wait_vmem();
        __syncthreads();
    }

    if (wave_valid && qrow < N) {
        uint16_t* Og = p.o + ((size_t)bh * N + qrow) * D;
        const float lt = l + swap_half(l);
        const float f = svmax / lsum;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x2 val;
                val[0] = pack_bf16(o[db][u * 4 + 0] * f, o[db][u * 4 + 1] * f);
                val[1] = pack_bf16(o[db][u * 4 + 2] * f, o[db][u * 4 + 3] * f);
                *reinterpret_cast<u32x2*>(Og + db * 32 + u * 8 + hh * 4) = val;
            }
        if (hh == 0) p.lse[(size_t)bh * N + qrow] = (m + __log2f(lt)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd8(const Fwd8Params& p, hipStream_t stream) {
    const int grid = p.B * p.Hq * ((p.N + k8BM - 1) / k8BM);
    if (p.d == 128)
        hipLaunchKernelGGL((fwd8_kernel<128>), dim3(grid), dim3(k8Threads), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd8_kernel<64>), dim3(grid), dim3(k8Threads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
