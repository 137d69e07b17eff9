// fa_quant.hip -- block quantisation of bfloat16 tensors to 8-bit E4M3 codes.
//
// FlashAttention-3 runs its forward in FP8 with block scaling (the mlapandio
// page "FlashAttention: IO-aware exact attention", "Generations"; the wishwiki
// page "FlashAttention", "Evolution: FlashAttention-2 and -3"). The pages give no format,
// so the codes follow the OCP 8-bit floating point E4M3 definition (sign, 4
// exponent bits with bias 7, 3 mantissa bits, no infinities, largest finite
// value 448), which is the FP8 format gfx950's matrix cores read.
//
// One scale per run of `rows` rows of each (b, h) slab, the last run ragged.
// In fp32: amax = max |x| over the run, inv = 448 / amax (correctly rounded),
// code = E4M3(x * inv) rounded to nearest, ties to even, saturating at 448,
// and the stored scale is amax / 448 (correctly rounded), so x ~ code * scale.
// An all-zero run gets inv = scale = 1. A run whose amax is below 2^-64 is
// multiplied by 2^64 first (exact), which keeps 448 / amax finite; its codes
// are those of the scaled run and its scale is (2^64 amax / 448) * 2^-64.
//
// One workgroup per run: a first sweep takes amax from the bf16 magnitude bits
// (integer max of finite values), a second re-reads the run (from L2) and
// writes 8 codes per lane per step. The work is HBM bound: 2 bytes read and 1
// written per element, plus the second read when the run does not stay in L2.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace fa {
namespace {

constexpr int kQThreads = 256;

// E4M3 code of a finite fp32 value: nearest, ties to even, |y| >= 448 -> 448.
// Below 2^-6 the codes are the multiples of 2^-9 (code = the multiple's count,
// 8 being the smallest normal 2^-6). Above, rounding the fp32 pattern to its
// top 3 mantissa bits (adding just under half an ulp of the kept bits plus the
// kept lowest bit) gives nearest-even, a carry moving into the exponent; the
// fp32 exponent bias 127 becomes 7 by subtracting 120 << 3.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t b = __float_as_uint(y);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t u = b & 0x7fffffffu;
    uint32_t c;
    if (u >= 0x43e00000u) c = 0x7eu;                                       // 448 and above
    else if (u < 0x3c800000u) c = (uint32_t)rintf(__uint_as_float(u) * 512.0f);
    else c = ((u + 0x7ffffu + ((u >> 20) & 1u)) >> 20) - 960u;
    return sign | c;
}

// The larger magnitude (bf16 bits without the sign) of a word's two values.
__device__ __forceinline__ uint32_t mag2(uint32_t w) {
    w &= 0x7fff7fffu;
    return max(w & 0xffffu, w >> 16);
}

__device__ __forceinline__ float bf16_lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(kQThreads) void quant_e4m3_kernel(const uint16_t* __restrict__ x,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales, int N, int d,
                                                               int rows, int nruns) {
    __shared__ uint32_t red[kQThreads / 64];
    const int run = (int)(blockIdx.x % (unsigned)nruns);
    const long long bh = (long long)(blockIdx.x / (unsigned)nruns);
    const long long r0 = (long long)run * rows;
    const long long r1 = r0 + rows < N ? r0 + rows : N;
    const long long base = (bh * N + r0) * d;
    const int chunks = (int)((r1 - r0) * d / 8);                            // d is a multiple of 8
    const uint4* src = reinterpret_cast<const uint4*>(x + base);

    uint32_t m = 0;
    for (int c = threadIdx.x; c < chunks; c += kQThreads) {
        const uint4 w = src[c];
        m = max(m, max(max(mag2(w.x), mag2(w.y)), max(mag2(w.z), mag2(w.w))));
    }
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));

    // A run below 2^-64 (bf16 exponent field under 63) is taken times 2^64
    // first, exactly, so that 448 / amax cannot overflow; its stored scale is
    // scaled back by 2^-64.
    const bool tiny = m < (63u << 7);
    const float up = tiny ? 0x1p64f : 1.0f;
    const float amax = __fmul_rn(__uint_as_float(m << 16), up);
    const float inv = m ? __fdiv_rn(448.0f, amax) : 1.0f;
    if (threadIdx.x == 0)
        scales[bh * nruns + run] = m ? __fmul_rn(__fdiv_rn(amax, 448.0f), tiny ? 0x1p-64f : 1.0f) : 1.0f;

    uint2* dst = reinterpret_cast<uint2*>(codes + base);
    for (int c = threadIdx.x; c < chunks; c += kQThreads) {
        const uint4 w = src[c];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        uint32_t out[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t c0 = e4m3_code(__fmul_rn(__fmul_rn(bf16_lo_f(ws[2 * t]), up), inv));
            const uint32_t c1 = e4m3_code(__fmul_rn(__fmul_rn(bf16_hi_f(ws[2 * t]), up), inv));
            const uint32_t c2 = e4m3_code(__fmul_rn(__fmul_rn(bf16_lo_f(ws[2 * t + 1]), up), inv));
            const uint32_t c3 = e4m3_code(__fmul_rn(__fmul_rn(bf16_hi_f(ws[2 * t + 1]), up), inv));
            out[t] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
        }
        dst[c] = make_uint2(out[0], out[1]);
    }
}

// The same quantisation of V, written transposed for the FP8 forward's
// O^T += V^T P^T products: codes_t [BH, d, Np] with Np = N rounded up to 64,
// and inside every group of 64 keys position p holds key
//   ((p % 32) / 16) * 32 + ((p % 16) / 4) * 8 + (p / 32) * 4 + p % 4,
// the key whose probability sits at the same k slot of the product's other
// operand (byte p % 32 of lane half p / 32). Keys past N get code 0. Runs are
// whole groups of 64 keys (rows % 64 == 0), so a workgroup owns its groups.
__global__ __launch_bounds__(kQThreads) void quant_e4m3_vt_kernel(const uint16_t* __restrict__ x,
                                                                  uint8_t* __restrict__ codes_t,
                                                                  float* __restrict__ scales, int N, int Np,
                                                                  int d, int rows, int nruns) {
    __shared__ uint32_t red[kQThreads / 64];
    const int run = (int)(blockIdx.x % (unsigned)nruns);
    const long long bh = (long long)(blockIdx.x / (unsigned)nruns);
    const long long r0 = (long long)run * rows;
    const long long r1 = r0 + rows < N ? r0 + rows : N;
    const long long base = (bh * N + r0) * d;
    const int chunks = (int)((r1 - r0) * d / 8);
    const uint4* src = reinterpret_cast<const uint4*>(x + base);

    uint32_t m = 0;
    for (int c = threadIdx.x; c < chunks; c += kQThreads) {
        const uint4 w = src[c];
        m = max(m, max(max(mag2(w.x), mag2(w.y)), max(mag2(w.z), mag2(w.w))));
    }
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const bool tiny = m < (63u << 7);
    const float up = tiny ? 0x1p64f : 1.0f;
    const float amax = __fmul_rn(__uint_as_float(m << 16), up);
    const float inv = m ? __fdiv_rn(448.0f, amax) : 1.0f;
    if (threadIdx.x == 0)
        scales[bh * nruns + run] = m ? __fmul_rn(__fdiv_rn(amax, 448.0f), tiny ? 0x1p-64f : 1.0f) : 1.0f;

    // The run's key groups, every column: a thread writes 4 consecutive
    // positions of one transposed row, one word (the keys they hold follow
    // the map above).
    const int g0 = (int)(r0 / 64), ng = (int)((r0 + rows < Np ? r0 + rows : Np) - r0 + 63) / 64;
    const long long words = (long long)ng * d * 16;
    uint8_t* dst = codes_t + bh * (long long)d * Np;
    for (long long wi = threadIdx.x; wi < words; wi += kQThreads) {
        const int g = g0 + (int)(wi / (d * 16));
        const int rem = (int)(wi % (d * 16));
        const int col = rem / 16, p0 = (rem % 16) * 4;
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = p0 + e;
            const int t = ((p % 32) / 16) * 32 + ((p % 16) / 4) * 8 + (p / 32) * 4 + p % 4;
            const long long key = (long long)g * 64 + t;
            uint32_t c = 0;
            if (key < N) {
                const uint16_t b = x[(bh * N + key) * d + col];
                c = e4m3_code(__fmul_rn(__fmul_rn(__uint_as_float((uint32_t)b << 16), up), inv));
            }
            word |= c << (8 * e);
        }
        *reinterpret_cast<uint32_t*>(dst + (long long)col * Np + (long long)g * 64 + p0) = word;
    }
}

}  // namespace

hipError_t launch_quant_e4m3_vt(const void* x, void* codes_t, float* scales, int BH, int N, int d, int rows,
                                hipStream_t stream) {
    const int nruns = (int)(((long long)N + rows - 1) / rows);
    const int Np = (N + 63) / 64 * 64;
    const long long grid = (long long)BH * nruns;
    hipLaunchKernelGGL(quant_e4m3_vt_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(codes_t), scales, N, Np, d, rows, nruns);
    return hipGetLastError();
}

hipError_t launch_quant_e4m3(const void* x, void* codes, float* scales, int BH, int N, int d, int rows,
                             hipStream_t stream) {
    const int nruns = (int)(((long long)N + rows - 1) / rows);
    const long long grid = (long long)BH * nruns;
    hipLaunchKernelGGL(quant_e4m3_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<uint8_t*>(codes), scales, N, d, rows, nruns);
    return hipGetLastError();
}

}  // namespace fa
