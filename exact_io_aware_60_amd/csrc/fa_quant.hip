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
// One workgroup per run. A run of up to 256 x kQHold 16-byte chunks (rows * d
// <= 32768 elements) is read once: each thread keeps its chunks in registers
// while the workgroup takes amax from the bf16 magnitude bits (integer max of
// finite values), then writes their codes. A larger run is swept twice, the
// second sweep re-reading it. The work is HBM bound: 2 bytes read and 1
// written per element.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace fa {
namespace {

constexpr int kQThreads = 256;
constexpr int kQHold = 16;   // 16-byte chunks a thread holds when its run fits

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

__device__ __forceinline__ uint32_t mag8(const uint4& w) {
    return max(max(mag2(w.x), mag2(w.y)), max(mag2(w.z), mag2(w.w)));
}

// Codes of the 8 values of a 16-byte chunk, in order.
__device__ __forceinline__ uint2 codes8(const uint4& w, float up, float inv) {
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
    return make_uint2(out[0], out[1]);
}

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

    // the whole run in registers when it fits (a workgroup-uniform choice)
    const bool hold = chunks <= kQThreads * kQHold;
    uint4 held[kQHold];
    uint32_t m = 0;
    if (hold) {
#pragma unroll
        for (int i = 0; i < kQHold; ++i) {
            const int c = (int)threadIdx.x + i * kQThreads;
            held[i] = c < chunks ? src[c] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < kQHold; ++i) m = max(m, mag8(held[i]));
    } else {
        for (int c = threadIdx.x; c < chunks; c += kQThreads) m = max(m, mag8(src[c]));
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
    if (hold) {
#pragma unroll
        for (int i = 0; i < kQHold; ++i) {
            const int c = (int)threadIdx.x + i * kQThreads;
            if (c < chunks) dst[c] = codes8(held[i], up, inv);
        }
    } else {
        for (int c = threadIdx.x; c < chunks; c += kQThreads) dst[c] = codes8(src[c], up, inv);
    }
}

// The same quantisation of V, written transposed for the FP8 forward's
// O^T += V^T P^T products: codes_t [BH, d, Np] with Np = N rounded up to 64,
// and inside every group of 64 keys position p holds key
//   ((p % 32) / 16) * 32 + ((p % 16) / 4) * 8 + (p / 32) * 4 + p % 4,
// the key whose probability sits at the same k slot of the product's other
// operand (byte p % 32 of lane half p / 32). Keys past N get code 0. Runs are
// whole groups of 64 keys (rows % 64 == 0), so a workgroup owns its groups.
//
// Four consecutive keys 4j .. 4j+3 sit at four consecutive positions starting
// at pos4(4j), so a run that fits is read once, row-major and coalesced, each
// thread holding the 16-byte chunks of 4 consecutive keys at one 8-column
// offset. It writes their codes as one word per column into an LDS tile of
// the run's transposed rows (pitch R + 4 bytes), and the tile goes out in
// 16-byte pieces of the transposed rows. A larger run takes amax in one sweep
// and gathers its codes column by column in a second.
constexpr int kVtLds = 36864;   // bytes of the transposed tile

// Position of key k (k % 4 == 0) in its group of 64: the inverse of the map above.
__device__ __forceinline__ int pos4(int k) { return ((k >> 3) & 3) * 4 + (k >> 5) * 16 + ((k >> 2) & 1) * 32; }

__global__ __launch_bounds__(kQThreads) void quant_e4m3_vt_kernel(const uint16_t* __restrict__ x,
                                                                  uint8_t* __restrict__ codes_t,
                                                                  float* __restrict__ scales, int N, int Np,
                                                                  int d, int rows, int nruns) {
    __shared__ uint32_t red[kQThreads / 64];
    __shared__ __attribute__((aligned(16))) uint8_t T[kVtLds];
    const int run = (int)(blockIdx.x % (unsigned)nruns);
    const long long bh = (long long)(blockIdx.x / (unsigned)nruns);
    const long long r0 = (long long)run * rows;
    const long long r1 = r0 + rows < N ? r0 + rows : N;
    const long long base = (bh * N + r0) * d;
    const int chunks = (int)((r1 - r0) * d / 8);
    const uint4* src = reinterpret_cast<const uint4*>(x + base);
    const int nkeys = (int)(r1 - r0);
    const int g0 = (int)(r0 / 64), ng = (int)((r0 + rows < Np ? r0 + rows : Np) - r0 + 63) / 64;
    const int R = ng * 64, PT = R + 4, cq = d / 8;
    const int units = (R / 4) * cq;                            // (4 keys, 8 columns) each
    const bool hold = units <= kQThreads * (kQHold / 4) && d * PT <= kVtLds;

    uint4 held[kQHold];
    uint32_t m = 0;
    if (hold) {
#pragma unroll
        for (int j = 0; j < kQHold / 4; ++j) {
            const int u = (int)threadIdx.x + j * kQThreads;
            const int kq = u / cq, cc = u - kq * cq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = 4 * kq + i;
                held[4 * j + i] = u < units && key < nkeys ? src[key * cq + cc] : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int i = 0; i < kQHold; ++i) m = max(m, mag8(held[i]));
    } else {
        for (int c = threadIdx.x; c < chunks; c += kQThreads) m = max(m, mag8(src[c]));
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

    uint8_t* dst = codes_t + bh * (long long)d * Np;
    if (hold) {
#pragma unroll
        for (int j = 0; j < kQHold / 4; ++j) {
            const int u = (int)threadIdx.x + j * kQThreads;
            if (u < units) {
                const int kq = u / cq, cc = u - kq * cq;
                const int p0 = (4 * kq / 64) * 64 + pos4((4 * kq) % 64);
                uint2 c[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) c[i] = codes8(held[4 * j + i], up, inv);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sh = (e & 3) * 8;
                    const uint32_t b0 = ((e < 4 ? c[0].x : c[0].y) >> sh) & 0xffu;
                    const uint32_t b1 = ((e < 4 ? c[1].x : c[1].y) >> sh) & 0xffu;
                    const uint32_t b2 = ((e < 4 ? c[2].x : c[2].y) >> sh) & 0xffu;
                    const uint32_t b3 = ((e < 4 ? c[3].x : c[3].y) >> sh) & 0xffu;
                    *reinterpret_cast<uint32_t*>(&T[(cc * 8 + e) * PT + p0]) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
                }
            }
        }
        __syncthreads();
        // the tile's d rows of R bytes, in 16-byte pieces
        const int per_row = R / 16, pieces = d * per_row;
        uint8_t* out = dst + (long long)g0 * 64;
        const bool a16 = (reinterpret_cast<uintptr_t>(codes_t) & 15u) == 0;
        for (int u = threadIdx.x; u < pieces; u += kQThreads) {
            const int col = u / per_row, q = u - col * per_row;
            const uint32_t* t = reinterpret_cast<const uint32_t*>(&T[col * PT + q * 16]);
            const uint4 v = make_uint4(t[0], t[1], t[2], t[3]);
            uint8_t* o = out + (long long)col * Np + q * 16;
            if (a16) {
                *reinterpret_cast<uint4*>(o) = v;
            } else {
                uint32_t* o4 = reinterpret_cast<uint32_t*>(o);
                o4[0] = v.x; o4[1] = v.y; o4[2] = v.z; o4[3] = v.w;
            }
        }
        return;
    }

    // The run's key groups, every column: a thread writes 4 consecutive
    // positions of one transposed row, one word (the keys they hold follow
    // the map above).
    const long long words = (long long)ng * d * 16;
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
