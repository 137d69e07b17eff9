// fa_params.h -- argument blocks shared by the host launcher and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

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
};

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const float* lse;
    const uint16_t* dout;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* delta;        // fp32 [B, Hq, N] workspace: rowsum(dout * o)
    float* lse2;         // fp32 [B, Hq, N] workspace: lse * log2(e)
    int B, Hq, Hkv, N, d, G;
    int causal;
    float scale;
    float scale_log2;
};

// Launchers (defined next to their kernels). They only enqueue work on the
// stream; they return the HIP status of the launch.
hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);
// One backward stage: 0 = row dot D (and log2-scaled LSE), 1 = dK/dV, 2 = dQ.
hipError_t launch_bwd_stage(const BwdParams& p, int stage, hipStream_t stream);

// Launch geometry, exposed for logging and tests of the host logic.
struct Geometry {
    int block_m;      // query rows per workgroup
    int block_n;      // keys per streamed tile
    int threads;      // threads per workgroup
    int grid;         // workgroups
    int lds_bytes;    // LDS per workgroup
};
Geometry fwd_geometry(int B, int Hq, int N, int d, int causal);

// Bytes of backward workspace: D and the log2-scaled LSE, one fp32 each per
// query row, each array starting on a 256-byte boundary.
size_t bwd_workspace_bytes(long long rows);

}  // namespace fa
