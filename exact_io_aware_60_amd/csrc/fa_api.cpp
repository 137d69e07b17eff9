// fa_api.cpp -- the C ABI: argument validation, launch parameters, status codes.
//
// Every entry point checks its arguments before any HIP call, so an invalid
// call enqueues nothing; the checks need no GPU. Kernels are enqueued on the
// caller's stream; nothing here allocates, frees or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/flash_attn.h"
#include "fa_params.h"

namespace fa {
// fa_quant.hip: block E4M3 quantisation of a bf16 [BH, N, d] tensor (d a
// multiple of 8) into codes [BH, N, d] and one fp32 scale per run of `rows`
// rows, [BH, ceil(N / rows)].
hipError_t launch_quant_e4m3(const void* x, void* codes, float* scales, int BH, int N, int d, int rows,
                             hipStream_t stream);
// The same codes and scales with V written transposed for the FP8 forward:
// codes_t [BH, d, Np], Np = N rounded up to 64, keys of each 64-key group in
// the order of the forward's P operand; rows a multiple of 64.
hipError_t launch_quant_e4m3_vt(const void* x, void* codes_t, float* scales, int BH, int N, int d, int rows,
                                hipStream_t stream);
}  // namespace fa

namespace {

thread_local char g_hip_text[256] = "";

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Head dimensions: multiples of 8 from 8 to 256 in every pass. A d below 64,
// 128 or 256 runs on that instance with zero columns past d.
bool headdim_ok(int d, int dmax) { return d >= 8 && d <= dmax && d % 8 == 0; }

int check_shape(int B, int Hq, int Hkv, int N, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (!headdim_ok(d, 256)) return FA_ERR_HEADDIM;
    d = fa::padded_dim(d);   // the width the copies and tiles use
    // element counts and the largest launch grid must fit the kernels' index types
    const long double elems = (long double)B * Hq * N * d;
    if (elems >= 4.0e18L) return FA_ERR_SHAPE;
    const long double grid = (long double)B * Hq * ((N + 63) / 64);
    if (grid >= 2147483647.0L) return FA_ERR_SHAPE;
    // per-head element offsets of the (padded) backward copies are 32-bit, and
    // the bytes of one group of query heads sharing a K/V head fit a 32-bit
    // buffer range
    if ((long double)(N + fa::kRowPad) * d >= 2147483647.0L) return FA_ERR_SHAPE;
    if ((long double)(Hq / Hkv) * (N + fa::kRowPad) * d * 2 >= 4294967295.0L) return FA_ERR_SHAPE;
    return FA_OK;
}

int check_scale(float scale) {
    if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
    return FA_OK;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return FA_OK;
    std::snprintf(g_hip_text, sizeof(g_hip_text), "HIP launch failed: %s", hipGetErrorString(e));
    return FA_ERR_HIP;
}

void log_config(const char* pass, int B, int Hq, int Hkv, int N, int d, int causal) {
    static const bool enabled = [] {
        const char* e = std::getenv("FLASH_ATTN_LOG");
        return e && e[0] == '1';
    }();
    if (!enabled) return;
    const fa::Geometry g = fa::fwd_geometry(B, Hq, N, d, causal);
    std::fprintf(stderr,
                 "[flash_attn] %s B=%d Hq=%d Hkv=%d N=%d d=%d causal=%d: block_m=%d block_n=%d "
                 "threads=%d grid=%d lds=%dB\n",
                 pass, B, Hq, Hkv, N, d, causal, g.block_m, g.block_n, g.threads, g.grid, g.lds_bytes);
}

}  // namespace

extern "C" {

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                   int Hkv, int N, int d, int causal, float scale, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    int st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_ALIGN;
    log_config("fwd", B, Hq, Hkv, N, d, causal);
    fa::FwdParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.d = d; p.G = Hq / Hkv;
    p.causal = causal ? 1 : 0;
    p.scale = scale;
    p.scale_log2 = std::max(scale * 1.4426950408889634f, 1e-30f);
    p.cu_seqlens = nullptr;
    p.total = 0;
    p.window = 0;
    return hip_status(fa::launch_fwd(p, static_cast<hipStream_t>(stream)));
}

int flash_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq,
                       int Hkv, int N, int d, int causal, float scale, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (!headdim_ok(d, 128)) return FA_ERR_HEADDIM;
    int st = check_scale(scale);
    if (st != FA_OK) return st;
    if ((long double)B * Hq * N * d >= 4.0e18L) return FA_ERR_SHAPE;
    if ((long double)B * Hq * ((N + 127) / 128) >= 2147483647.0L) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
    log_config("fwd_f32", B, Hq, Hkv, N, d, causal);
    fa::Fwd32Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.d = d; p.G = Hq / Hkv;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = std::max(scale * 1.4426950408889634f, 1e-30f);
    return hip_status(fa::launch_fwd32(p, static_cast<hipStream_t>(stream)));
}

int flash_attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                          int Hkv, int N, int d, int window, float scale, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    int st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    if (window < 1) return FA_ERR_SHAPE;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_ALIGN;
    log_config("fwd_window", B, Hq, Hkv, N, d, 1);
    fa::FwdParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.d = d; p.G = Hq / Hkv;
    p.causal = 1;
    p.scale = scale;
    p.scale_log2 = std::max(scale * 1.4426950408889634f, 1e-30f);
    p.cu_seqlens = nullptr;
    p.total = 0;
    p.window = window;
    return hip_status(fa::launch_fwd(p, static_cast<hipStream_t>(stream)));
}

int flash_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int* cu_seqlens, int B, int max_seqlen, int total, int Hq, int Hkv, int d,
                          int causal, float scale, void* stream) {
    if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA_ERR_NULL;
    int st = check_shape(B, Hq, Hkv, max_seqlen, d);
    if (st != FA_OK) return st;
    if (total < 1 || (long double)Hq * total * d >= 4.0e18L) return FA_ERR_SHAPE;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
        return FA_ERR_ALIGN;
    log_config("fwd_varlen", B, Hq, Hkv, max_seqlen, d, causal);
    fa::FwdParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = max_seqlen; p.d = d; p.G = Hq / Hkv;
    p.causal = causal ? 1 : 0;
    p.scale = scale;
    p.scale_log2 = std::max(scale * 1.4426950408889634f, 1e-30f);
    p.cu_seqlens = cu_seqlens;
    p.total = total;
    p.window = 0;
    return hip_status(fa::launch_fwd(p, static_cast<hipStream_t>(stream)));
}

size_t flash_attn_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int causal) {
    (void)causal;
    if (check_shape(B, Hq, Hkv, N, d) != FA_OK) return 0;
    return fa::bwd_workspace_layout(B, Hq, Hkv, N, d).total;
}

}  // extern "C"

namespace {

// Shared by flash_attn_bwd and its stage entry points: validate, fill the
// parameter block, enqueue stages [first, last].
int bwd_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
               int causal, float scale, void* workspace, size_t workspace_bytes, void* stream,
               int first, int last, int window = 0, const int* cu_seqlens = nullptr, int nseq = 0) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    int st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return FA_ERR_ALIGN;
    if (!workspace || workspace_bytes < flash_attn_bwd_workspace_size(B, Hq, Hkv, N, d, causal))
        return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    if (first == 0) log_config("bwd", B, Hq, Hkv, N, d, causal);
    fa::BwdParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<const uint16_t*>(o);
    p.lse = lse;
    p.dout = static_cast<const uint16_t*>(dout);
    p.dq = static_cast<uint16_t*>(dq);
    p.dk = static_cast<uint16_t*>(dk);
    p.dv = static_cast<uint16_t*>(dv);
    const fa::BwdWorkspace w = fa::bwd_workspace_layout(B, Hq, Hkv, N, d);
    char* ws = static_cast<char*>(workspace);
    p.delta = reinterpret_cast<float*>(ws + w.delta);
    p.lse2 = reinterpret_cast<float*>(ws + w.lse2);
    p.q16 = reinterpret_cast<uint16_t*>(ws + w.q16);
    p.k16 = reinterpret_cast<uint16_t*>(ws + w.k16);
    p.v16 = reinterpret_cast<uint16_t*>(ws + w.v16);
    p.do16 = reinterpret_cast<uint16_t*>(ws + w.do16);
    p.qT16 = reinterpret_cast<uint16_t*>(ws + w.qT16);
    p.doT16 = reinterpret_cast<uint16_t*>(ws + w.doT16);
    p.kT16 = reinterpret_cast<uint16_t*>(ws + w.kT16);
    p.part = reinterpret_cast<uint32_t*>(ws + w.part);
    p.scales = reinterpret_cast<float*>(ws + w.scales);
    p.npart = w.npart;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.d = d; p.G = Hq / Hkv;
    p.Np = w.Np;
    p.causal = causal ? 1 : 0;
    p.scale = scale;
    p.scale_log2 = std::max(scale * 1.4426950408889634f, 1e-30f);
    p.window = window;
    p.cu_seqlens = cu_seqlens;
    p.nseq = nseq;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    for (int stage = first; stage <= last; ++stage) {
        st = hip_status(fa::launch_bwd_stage(p, stage, s));
        if (st != FA_OK) return st;
    }
    return FA_OK;
}

}  // namespace

extern "C" {

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                   int d, int causal, float scale, void* workspace, size_t workspace_bytes,
                   void* stream) {
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, workspace,
                      workspace_bytes, stream, 0, 2);
}

int flash_attn_bwd_preprocess(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, workspace,
                      workspace_bytes, stream, 0, 0);
}

int flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
                        int N, int d, int causal, float scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, workspace,
                      workspace_bytes, stream, 2, 2);
}

int flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                      int d, int causal, float scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, workspace,
                      workspace_bytes, stream, 1, 1);
}

namespace {

int check_decode_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (!headdim_ok(d, 256)) return FA_ERR_HEADDIM;
    d = fa::padded_dim(d);
    if (causal && Nq > Nk) return FA_ERR_SHAPE;
    // one K/V head fits a 32-bit buffer range with room for a ragged tile
    if ((long double)Nk * d * 2 >= 2147483648.0L) return FA_ERR_SHAPE;
    // rows of one group and their offsets, element counts, grids
    if ((long double)(Hq / Hkv) * Nq * d >= 2147483647.0L) return FA_ERR_SHAPE;
    if ((long double)B * Hq * Nq * d >= 4.0e18L || (long double)B * Hkv * Nk * d >= 4.0e18L) return FA_ERR_SHAPE;
    const long double rows = (long double)B * Hq * Nq;
    if (rows >= 2147483647.0L) return FA_ERR_SHAPE;
    const long double nrb = ((long double)(Hq / Hkv) * Nq + 127) / 128;
    if ((long double)B * Hkv * (nrb + 1) * 512 >= 2147483647.0L) return FA_ERR_SHAPE;
    return FA_OK;
}

}  // namespace

size_t flash_attn_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                                        int window) {
    if (check_decode_shape(B, Hq, Hkv, Nq, Nk, d, causal) != FA_OK) return 0;
    if (window < 0 || (window > 0 && !causal)) return 0;
    return fa::dec_plan(B, Hq, Hkv, Nq, Nk, d, window).total;
}

namespace {

// flash_attn_decode with the workspace checks done by the caller.
int decode_common(const void* q, const void* k, const void* v, void* o, float* lse, const int* seqlens_k,
                  int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int window, float scale,
                  void* workspace, size_t workspace_bytes, void* stream, bool noalloc);

}  // namespace

int flash_attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* seqlens_k, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                      int window, float scale, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_common(q, k, v, o, lse, seqlens_k, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, workspace,
                         workspace_bytes, stream, false);
}

int flash_attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* seqlens_k, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                              int causal, int window, float scale, void* stream) {
    return decode_common(q, k, v, o, lse, seqlens_k, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, nullptr, 0,
                         stream, true);
}

size_t flash_attn_decode_noalloc_max_bytes(void) { return fa::kDecodeScratchBytes; }

namespace {

int decode_common(const void* q, const void* k, const void* v, void* o, float* lse, const int* seqlens_k,
                  int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int window, float scale,
                  void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    int st = check_decode_shape(B, Hq, Hkv, Nq, Nk, d, causal);
    if (st != FA_OK) return st;
    if (window < 0 || (window > 0 && !causal)) return FA_ERR_SHAPE;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0)
        return FA_ERR_ALIGN;
    const fa::DecPlan pl = fa::dec_plan(B, Hq, Hkv, Nq, Nk, d, window);
    if (noalloc) {
        // the partial results go to this GPU's static scratch array
        if (pl.total > fa::kDecodeScratchBytes) return FA_ERR_SCRATCH;
        if (pl.total > 0) {
            const hipError_t e = fa::decode_scratch(&workspace);
            if (e != hipSuccess) return hip_status(e);
            workspace_bytes = fa::kDecodeScratchBytes;
        }
    }
    if (pl.total > 0) {
        if (!workspace || workspace_bytes < pl.total) return FA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FA_ERR_ALIGN;
    }
    fa::DecParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    char* ws = static_cast<char*>(workspace);
    p.part_lse = pl.total ? reinterpret_cast<float*>(ws + pl.part_lse) : nullptr;
    p.part_o = pl.total ? reinterpret_cast<float*>(ws + pl.part_o) : nullptr;
    p.seqlens_k = seqlens_k;
    p.window = window;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.d = d; p.G = Hq / Hkv; p.M = pl.M;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = std::max(scale * 1.4426950408889634f, 1e-30f);
    p.nrb = pl.nrb;
    p.nsplit = pl.nsplit;
    p.tps = pl.tps;
    p.pair = pl.pair;
    return hip_status(fa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

int flash_attn_quantize_e4m3(const void* x, void* codes, float* scales, int BH, int N, int d, int rows,
                             void* stream) {
    if (!x || !codes || !scales) return FA_ERR_NULL;
    if (BH < 1 || N < 1 || rows < 1) return FA_ERR_SHAPE;
    if (d < 8 || d % 8 != 0) return FA_ERR_HEADDIM;
    if (!aligned16(x) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
        return FA_ERR_ALIGN;
    // one workgroup per run; a run's element count and the grid are 32-bit
    const long long runs = (N + (long long)rows - 1) / rows;
    if ((long double)BH * runs >= 2147483647.0L) return FA_ERR_SHAPE;
    if ((long double)std::min(rows, N) * d >= 2147483647.0L) return FA_ERR_SHAPE;
    if ((long double)BH * N * d >= 4.0e18L) return FA_ERR_SHAPE;
    return hip_status(fa::launch_quant_e4m3(x, codes, scales, BH, N, d, rows, static_cast<hipStream_t>(stream)));
}

int flash_attn_quantize_e4m3_vt(const void* x, void* codes_t, float* scales, int BH, int N, int d, int rows,
                                void* stream) {
    if (!x || !codes_t || !scales) return FA_ERR_NULL;
    if (BH < 1 || N < 1 || rows < 64 || rows % 64 != 0) return FA_ERR_SHAPE;
    if (d < 8 || d % 8 != 0) return FA_ERR_HEADDIM;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(codes_t) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
        return FA_ERR_ALIGN;
    const long long Np = (N + 63LL) / 64 * 64;
    const long long runs = (N + (long long)rows - 1) / rows;
    if ((long double)BH * runs >= 2147483647.0L) return FA_ERR_SHAPE;
    if ((long double)std::min(rows, N) * d >= 2147483647.0L || (long double)Np * d >= 2147483647.0L)
        return FA_ERR_SHAPE;
    if ((long double)BH * Np * d >= 4.0e18L) return FA_ERR_SHAPE;
    return hip_status(fa::launch_quant_e4m3_vt(x, codes_t, scales, BH, N, d, rows, static_cast<hipStream_t>(stream)));
}

int flash_attn_fwd_e4m3(const void* q8, const float* q_scales, const void* k8, const float* k_scales,
                        const void* v8t, const float* v_scales, void* o, float* lse, int B, int Hq, int Hkv, int N,
                        int d, int causal, float scale, int rows, void* stream) {
    if (!q8 || !q_scales || !k8 || !k_scales || !v8t || !v_scales || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (rows < 64 || rows % 64 != 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    int st = check_scale(scale);
    if (st != FA_OK) return st;
    const long long Np = (N + 63LL) / 64 * 64;
    if ((long double)Np * d >= 2147483647.0L) return FA_ERR_SHAPE;            // one head's bytes, 32-bit
    if ((long double)B * Hq * ((N + 255) / 256) >= 2147483647.0L) return FA_ERR_SHAPE;
    if ((long double)B * Hq * Np * d >= 4.0e18L) return FA_ERR_SHAPE;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o) || !aligned16(lse) ||
        (reinterpret_cast<uintptr_t>(q_scales) & 3u) != 0 || (reinterpret_cast<uintptr_t>(k_scales) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(v_scales) & 3u) != 0)
        return FA_ERR_ALIGN;
    fa::Fwd8Params p;
    p.q = static_cast<const uint8_t*>(q8);
    p.q_scales = q_scales;
    p.k = static_cast<const uint8_t*>(k8);
    p.k_scales = k_scales;
    p.vt = static_cast<const uint8_t*>(v8t);
    p.v_scales = v_scales;
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.Np = (int)Np; p.d = d; p.G = Hq / Hkv; p.rows = rows;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = std::max(scale * 1.4426950408889634f, 1e-30f);
    return hip_status(fa::launch_fwd8(p, static_cast<hipStream_t>(stream)));
}

int flash_attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                          int d, int window, float scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (window < 1) return FA_ERR_SHAPE;
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, 1, scale, workspace,
                      workspace_bytes, stream, 0, 2, window);
}

int flash_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens, int B,
                          int max_seqlen, int total, int Hq, int Hkv, int d, int causal, float scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_seqlens) return FA_ERR_NULL;
    if (B < 1 || max_seqlen < 1) return FA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return FA_ERR_ALIGN;
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, 1, Hq, Hkv, total, d, causal ? 1 : 0, scale, workspace,
                      workspace_bytes, stream, 0, 2, 0, cu_seqlens, B);
}

const char* flash_attn_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "unsupported shape: B, Hq, Hkv, N must be >= 1, Hq % Hkv == 0, sizes in range";
        case FA_ERR_HEADDIM:
            return "unsupported head dimension: d must be a multiple of 8 from 8 to 256";
        case FA_ERR_ALIGN: return "a pointer is not 16-byte aligned (int32 length arrays: 4-byte)";
        case FA_ERR_WORKSPACE: return "workspace is NULL or too small";
        case FA_ERR_HIP: return g_hip_text[0] ? g_hip_text : "HIP launch failed";
        case FA_ERR_SCALE: return "scale must be finite and >= 0";
        case FA_ERR_SCRATCH:
            return "the call needs more partial-result memory than the static scratch holds "
                   "(flash_attn_decode_noalloc_max_bytes); use flash_attn_decode with a workspace";
        default: return "unknown status";
    }
}

const char* flash_attn_version(void) { return "0.8.0 gfx950"; }

int flash_attn_fwd_geometry(int B, int Hq, int Hkv, int N, int d, int causal, int* out) {
    if (!out) return FA_ERR_NULL;
    const int st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    const fa::Geometry g = fa::fwd_geometry(B, Hq, N, d, causal);
    out[0] = g.block_m;
    out[1] = g.block_n;
    out[2] = g.threads;
    out[3] = g.grid;
    out[4] = g.lds_bytes;
    return FA_OK;
}

}  // extern "C"
