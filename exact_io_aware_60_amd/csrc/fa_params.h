// fa_params.h -- argument blocks shared by the host launcher and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Padded width of a head dimension: the kernel instance that serves tensors
// whose rows hold d values (d a multiple of 8, 8 <= d <= 256). Tiles and the
// backward's copies hold D columns, the ones past d being zeros.
__host__ __device__ constexpr int padded_dim(int d) { return d <= 64 ? 64 : (d <= 128 ? 128 : 256); }

struct FwdParams {
    const uint16_t* q;   // bf16 [B, Hq, N, d]
    const uint16_t* k;   // bf16 [B, Hkv, N, d]
    const uint16_t* v;   // bf16 [B, Hkv, N, d]
    uint16_t* o;         // bf16 [B, Hq, N, d]
    float* lse;          // fp32 [B, Hq, N]
    int B, Hq, Hkv, N, d, G;
    int causal;
    float scale;         // softmax scale
    float scale_log2;    // scale * log2(e)
    // Packed sequences of different lengths (null: every sequence has N rows).
    // Then q/o are [Hq, total, d], k/v [Hkv, total, d], lse [Hq, total];
    // sequence b holds rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head,
    // and N is the longest sequence (it sizes the grid).
    const int* cu_seqlens;
    int total;
    // Sliding window (local attention, with the causal mask): row i keeps keys
    // i - window < j <= i. 0: no window.
    int window;
};

// Forward on fp32 inputs (fa_fwd32.hip): fp32 Q, K, V in, fp32 O and LSE out.
struct Fwd32Params {
    const float* q;      // fp32 [B, Hq, N, d]
    const float* k;      // fp32 [B, Hkv, N, d]
    const float* v;      // fp32 [B, Hkv, N, d]
    float* o;            // fp32 [B, Hq, N, d]
    float* lse;          // fp32 [B, Hq, N]
    int B, Hq, Hkv, N, d, G;
    int causal;
    float scale_log2;    // softmax scale * log2(e)
};

// Forward on 8-bit inputs (OCP E4M3 codes with one fp32 scale per run of
// `rows` rows of each head; fa_fwd8.hip).
struct Fwd8Params {
    const uint8_t* q;        // E4M3 [B, Hq, N, d]
    const float* q_scales;   // fp32 [B, Hq, ceil(N / rows)]
    const uint8_t* k;        // E4M3 [B, Hkv, N, d]
    const float* k_scales;   // fp32 [B, Hkv, ceil(N / rows)]
    const uint8_t* vt;       // E4M3 [B, Hkv, d, Np]: V transposed, keys in MFMA order (flash_attn_quantize_e4m3_vt)
    const float* v_scales;   // fp32 [B, Hkv, ceil(N / rows)]
    uint16_t* o;             // bf16 [B, Hq, N, d]
    float* lse;              // fp32 [B, Hq, N]
    int B, Hq, Hkv, N, Np, d, G, rows, causal;
    float scale_log2;        // softmax scale * log2(e)
};

struct BwdParams {
    const uint16_t* q;   // bf16 inputs, as in FwdParams
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const float* lse;
    const uint16_t* dout;
    uint16_t* dq;        // bf16 outputs
    uint16_t* dk;
    uint16_t* dv;
    // Workspace (device memory the caller provides; layout in bwd_workspace_layout).
    // Per-row arrays and the fp16 copies hold Np = N rounded up to a multiple of
    // kRowPad rows per head; rows N .. Np-1 are padding the preparation writes
    // (zero data, D = 0, LSE = +inf), so tiles never read past an array.
    float* delta;        // fp32 [B, Hq, Np]: row dot D times the dS scale
    float* lse2;         // fp32 [B, Hq, Np]: lse * log2(e)
    uint16_t* q16;       // fp16 [B, Hq, Np, d] copies of q, k, v, dout, each scaled by a power of two
    uint16_t* k16;       // fp16 [B, Hkv, Np, d]
    uint16_t* v16;
    uint16_t* do16;
    uint16_t* qT16;      // fp16 [B, Hq, d, Np] transposed copies of q, dout and k; inside every
    uint16_t* doT16;     // group of 16 rows the row order is permuted (bits 2 and 3 of the row
    uint16_t* kT16;      // index swapped), the k order of the MFMA operand they feed
    uint32_t* part;      // [4][npart] partial max |x| of q, k, v, dout (bf16 magnitude bits)
    float* scales;       // [8] derived constants, written by the preparation kernel
    int npart;           // workgroups of the max-reduction kernel
    int B, Hq, Hkv, N, d, G;
    int Np;              // padded rows per head
    int causal;
    float scale;
    float scale_log2;
    int window;          // sliding window with the causal mask (0: none), as in FwdParams
    // Packed sequences (null: none): the arrays are one sequence of N = total
    // rows per head, and sequence s holds rows cu_seqlens[s] .. cu_seqlens[s+1]-1.
    // With the causal mask a row then sees the keys from its sequence's start
    // to itself, a key is seen by the rows from itself to its sequence's end.
    const int* cu_seqlens;
    int nseq;
};

// Decode: a few query rows against a long key/value sequence. The M = G * Nq
// query rows that share a K/V head (a "group", index b * Hkv + hkv) are
// contiguous in q, o and lse. The keys of a group are split into nsplit ranges
// of tps 64-key tiles; a workgroup handles one (group, 128-row block, range)
// and, unless there is a single range, leaves a partial result that the merge
// kernel combines.
struct DecParams {
    const uint16_t* q;   // bf16 [B, Hq, Nq, d]
    const uint16_t* k;   // bf16 [B, Hkv, Nk, d]
    const uint16_t* v;   // bf16 [B, Hkv, Nk, d]
    uint16_t* o;         // bf16 [B, Hq, Nq, d]
    float* lse;          // fp32 [B, Hq, Nq]
    float* part_lse;     // fp32 [groups][nsplit][M]: log2 of the range's sum of exp2 (-inf: no key seen)
    float* part_o;       // fp32 [groups][nsplit][M][d]: the range's normalised output (0: no key seen)
    const int* seqlens_k;  // int32 [B] keys in use per batch entry (clamped to [0, Nk]), or null: all Nk
    int window;            // causal sliding window: row at position p sees keys p - window < j <= p (0: none)
    int B, Hq, Hkv, Nq, Nk, d, G, M;
    int causal;
    float scale_log2;
    int nrb;             // 128-row blocks per group
    int nsplit;          // key ranges per group
    int tps;             // 64-key tiles per range
    int pair;            // 1: two waves share each 32-row block, one per 32-key half of a tile
};

// Split plan and workspace layout of the decode (workspace offsets are
// 256-byte aligned; total = 0 when nsplit == 1 and the range kernel writes o
// and lse itself).
struct DecPlan {
    int M, nrb, nsplit, tps, pair;
    size_t part_lse, part_o, total;
};
DecPlan dec_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int window);

constexpr int kRowPad = 128;   // row padding unit of the backward workspace

// Byte offsets of the backward workspace arrays; every array starts on a
// 256-byte boundary.
struct BwdWorkspace {
    size_t delta, lse2, q16, k16, v16, do16, qT16, doT16, kT16, part, scales, total;
    int npart;
    int Np;
};
BwdWorkspace bwd_workspace_layout(int B, int Hq, int Hkv, int N, int d);

// Launchers (defined next to their kernels). They only enqueue work on the
// stream; they return the HIP status of the launch.
hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);
// One backward stage: 0 = preparation (scales, fp16 copies, row dot D,
// log2-scaled LSE), 1 = dQ (and the exact row dot), 2 = dK/dV.
hipError_t launch_bwd_stage(const BwdParams& p, int stage, hipStream_t stream);
hipError_t launch_decode(const DecParams& p, hipStream_t stream);
hipError_t launch_fwd8(const Fwd8Params& p, hipStream_t stream);
hipError_t launch_fwd32(const Fwd32Params& p, hipStream_t stream);

// Size of the decode's static scratch array (one per GPU; flash_attn_decode_noalloc).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
// Device address of the current GPU's scratch array, looked up once per GPU
// (hipGetSymbolAddress with that GPU current) and cached.
hipError_t decode_scratch(void** out);

// Launch geometry, exposed for logging and tests of the host logic.
struct Geometry {
    int block_m;      // query rows per workgroup
    int block_n;      // keys per streamed tile
    int threads;      // threads per workgroup
    int grid;         // workgroups
    int lds_bytes;    // LDS per workgroup
};
Geometry fwd_geometry(int B, int Hq, int N, int d, int causal);

}  // namespace fa
