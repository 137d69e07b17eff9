/*
 * flash_attn.h -- C ABI of an exact-attention library for AMD MI355X (gfx950).
 *
 * Operation. For each batch entry b and query head h:
 *
 *     O = softmax(scale * Q K^T [+ causal mask]) V
 *
 * Query head h reads key/value head h / (Hq / Hkv) (grouped-query attention;
 * Hq / Hkv consecutive query heads share one K/V head). Under the causal mask,
 * query row i sees key j iff j <= i. The forward pass also stores one
 * logsumexp value per query row,
 *
 *     LSE_i = ln sum_{visible j} exp(scale * q_i . k_j),
 *
 * and the backward pass rebuilds the probabilities from it, never from a stored
 * score matrix. The N x N score matrix is never written to device memory.
 * Sources: mlapandio "FlashAttention: IO-aware exact attention" (Definition;
 * the naive-vs-flash diagram, flash half; "Four ideas", recomputation item;
 * "Two notes" for grouped-query attention) and techtrendtracker "Flash
 * Attention: memory-efficient transformers" ("Recomputation in the Backward
 * Pass"). The scale, the mask convention and the head mapping are readings
 * of those pages; the pages fix none of them.
 *
 * Layout. Every tensor is contiguous, row-major [B, H, N, d] (d fastest) in
 * bfloat16, with H = Hq for q/o/dout/dq and H = Hkv for k/v/dk/dv. LSE is
 * contiguous [B, Hq, N] float32 (natural log). There are no stride arguments.
 *
 * Supported shapes: B, Hq, Hkv, N >= 1; Hq % Hkv == 0; d a multiple of 8 with
 * 8 <= d <= 256 in every entry point. A d below 64, 128 or 256 runs on the
 * kernels of that width with zero columns past d (tensors keep rows of d
 * values; 32 and 96 are common model shapes); d above 128 in the backward runs
 * gradient kernels that split the accumulated columns in halves of 128.
 * With D = d rounded up to 64, 128 or 256: B*Hq*N*D < 2^62; (N + 128) * D <
 * 2^31 and (Hq / Hkv) * (N + 128) * D * 2 < 2^32 (32-bit offsets inside one
 * head and one query-head group). scale must be finite and >= 0. Other
 * shapes return an error; there is no fallback path.
 *
 * Pointers are device pointers (hipMalloc'd or equivalent), 16-byte aligned.
 * `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 * work on `stream` and return at once; results are valid once the stream has
 * been synchronised. The library never allocates, frees or synchronises, keeps
 * no pointer after a call returns, and holds no mutable global state apart
 * from two per-GPU caches: the address of flash_attn_decode_noalloc's static
 * scratch (set once per GPU under a once-flag) and the compute-unit count the
 * forward's launch shape depends on (read once per GPU, atomically). Calls
 * from several host threads are therefore safe (flash_attn_decode_noalloc:
 * see its sharing rule). Calls on one stream run in order; the
 * caller orders calls on different streams that share buffers.
 *
 * Errors. Every entry point returns FA_OK (0) or a negative status and never
 * aborts. Arguments are checked before any HIP call, so an invalid call
 * enqueues nothing. FA_ERR_HIP means a launch failed; flash_attn_strerror()
 * then also carries the HIP error text of the calling thread's last failure.
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = -1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,     /* B, Hq, Hkv or N < 1, Hq % Hkv != 0, or sizes overflow */
    FA_ERR_HEADDIM = -3,   /* d not a multiple of 8 in [8, 256] */
    FA_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned (int32 length arrays: 4-byte) */
    FA_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required */
    FA_ERR_HIP = -6,       /* a kernel launch failed (see flash_attn_strerror) */
    FA_ERR_SCALE = -7,     /* scale is negative, NaN or infinite */
    FA_ERR_SCRATCH = -8    /* flash_attn_decode_noalloc: more partial results than its static scratch holds */
};

/*
 * Forward pass.
 *   q    in   bf16 [B, Hq,  N, d]
 *   k    in   bf16 [B, Hkv, N, d]
 *   v    in   bf16 [B, Hkv, N, d]
 *   o    out  bf16 [B, Hq,  N, d]   normalised output
 *   lse  out  fp32 [B, Hq,  N]      natural-log logsumexp of the scaled, masked scores
 * causal: 0 or 1. scale: the factor on q.k before the softmax (usually 1/sqrt(d)).
 * Inputs and outputs must not overlap.
 */
int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   void* stream);

/*
 * Forward pass on fp32 inputs: the computation of flash_attn_fwd (mlapandio
 * "FlashAttention: IO-aware exact attention", "Four ideas") for Q, K and V
 * that are fp32 and are not rounded first. Both products run on fp32 matrix
 * instructions with fp32 accumulation, the softmax statistics in fp32.
 *   q    in   fp32 [B, Hq,  N, d]
 *   k    in   fp32 [B, Hkv, N, d]
 *   v    in   fp32 [B, Hkv, N, d]
 *   o    out  fp32 [B, Hq,  N, d]   normalised output
 *   lse  out  fp32 [B, Hq,  N]      natural-log logsumexp of the scaled, masked scores
 * causal: 0 or 1. d: a multiple of 8 up to 128 (else FA_ERR_HEADDIM). Other
 * arguments and rules as in flash_attn_fwd. It runs at the fp32 matrix rate,
 * a sixteenth of the bf16 one.
 */
int flash_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                       int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                       void* stream);

/*
 * Forward pass with a sliding-window (local) causal mask: query row i sees keys
 * i - window < j <= i, its `window` most recent positions. Arguments, layout
 * and outputs as in flash_attn_fwd (causal is implied); window >= 1, and
 * window >= N gives the plain causal result. The mlapandio page
 * "FlashAttention: IO-aware exact attention" ("Honest limits") notes that such
 * masks need implementations of their own: here the causal tile skip is
 * extended to the band, so keys before a q-tile's window are never read.
 */
int flash_attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int N, int d, int window, float scale,
                          void* stream);

/*
 * Forward pass over packed sequences of different lengths (one launch for a
 * batch of prompts, no padding). Same computation as flash_attn_fwd for each
 * sequence on its own; the sequences share heads and nothing else.
 *   q           in   bf16 [Hq,  total, d]   sequence b is rows cu_seqlens[b] ..
 *   k, v        in   bf16 [Hkv, total, d]   cu_seqlens[b+1]-1 of every head
 *   o           out  bf16 [Hq,  total, d]
 *   lse         out  fp32 [Hq,  total]
 *   cu_seqlens  in   int32 [B + 1] device array: 0 = cu_seqlens[0] <= ... <=
 *                    cu_seqlens[B] = total, every length <= max_seqlen
 * max_seqlen sizes the grid (workgroups of q-tiles past a shorter sequence
 * exit at once). causal: within each sequence, row i sees keys j <= i.
 * Supported: B, max_seqlen, total, Hq, Hkv >= 1 and the limits of
 * flash_attn_fwd with N = max_seqlen. cu_seqlens is device data and is not
 * read on the host: offsets and lengths that break the rules above are
 * clamped in the kernel to [0, total] and [0, min(max_seqlen, total - offset)],
 * so no access leaves the arrays, but the affected sequences' results are
 * then unspecified. cu_seqlens must be 4-byte aligned.
 */
int flash_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int* cu_seqlens, int B, int max_seqlen, int total, int Hq, int Hkv,
                          int d, int causal, float scale, void* stream);

/*
 * Bytes of device workspace flash_attn_bwd needs for these arguments, or 0 for
 * shapes the backward rejects. Per head, rows are padded to Np = N rounded up
 * to a multiple of 128. The workspace holds two fp32 values per padded query
 * row (D = rowsum(dout * o) and LSE * log2(e)); fp16 copies of q, k, v and dout
 * scaled by powers of two, [.., Np, D]; transposed fp16 copies of q, dout and
 * k, [.., D, Np] (the operands of the backward's products), where D is d
 * rounded up to 64, 128 or 256 (the columns past d are zeros); and a few KiB of
 * reduction scratch. In all, about 4 * |q| + 3 * |k| bytes for the sizes
 * |q| = B*Hq*N*D*2 and |k| = B*Hkv*N*D*2, plus 8 bytes per query row.
 */
size_t flash_attn_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int causal);

/*
 * Backward pass for the loss sum(dout * O): given the forward's o and lse,
 * writes the gradients with respect to q, k and v (mlapandio "FlashAttention:
 * IO-aware exact attention", "Four ideas", recomputation item: P is rebuilt
 * from the stored logsumexp; techtrendtracker "Flash Attention:
 * memory-efficient transformers", "Recomputation in the Backward Pass").
 *   q, k, v, o, lse, dout   in   as in flash_attn_fwd; dout shaped like o
 *   dq                      out  bf16 [B, Hq,  N, d]
 *   dk, dv                  out  bf16 [B, Hkv, N, d]   summed over each K/V head's query group
 *   workspace               scratch, device memory of workspace_bytes >=
 *                           flash_attn_bwd_workspace_size(...); contents on
 *                           entry are ignored and on return are unspecified
 * Outputs must not overlap inputs or each other. Runs four kernels in order on
 * `stream`: max |x| of q, k, v, dout; preparation (scaled fp16 copies and
 * transposed copies, the row dot D from o, the log2-scaled LSE); dQ, which
 * also forms the exact row dot
 * D_i = sum_j P_ij dP_ij from the rebuilt probabilities, corrects its own
 * result with it and stores it; dK/dV, which uses that exact D. Deterministic:
 * the same inputs give bit-identical outputs (no atomics). Inputs must be
 * finite, with max|dout| * max|v| < 2^100 (the dS scale is derived from their
 * product).
 */
int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three stages of flash_attn_bwd, with its argument list and checks.
 * flash_attn_bwd is exactly preprocess (two kernels), dq, dkdv in that order
 * on one stream. They exist so that a caller can time or schedule the kernels
 * separately.
 *   preprocess  reads q, k, v, o, dout, lse; writes the workspace
 *   dq          reads the workspace (and lse); writes dq and the exact row dot
 *               into the workspace
 *   dkdv        reads the workspace; writes dk, dv
 * Each stage needs the workspace the previous stages wrote for the same
 * inputs; pointers a stage does not use must still be valid and aligned.
 */
int flash_attn_bwd_preprocess(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);
int flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);
int flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention of a few query rows over a long key/value sequence: the decode
 * step of generation, where each new token (or a short block of them) attends
 * to the whole key/value cache. The mlapandio page "FlashAttention: IO-aware
 * exact attention" notes that tiling does not speed this case up: it is bound
 * by reading the cache from memory ("Two notes"; end of the naive-vs-flash
 * diagram). So this entry point splits the keys of every K/V head into
 * ranges read by separate workgroups, which keeps the whole GPU reading, and
 * merges the per-range results by their logsumexp.
 *   q          in   bf16 [B, Hq,  Nq, d]    the newest Nq query rows
 *   k          in   bf16 [B, Hkv, Nk, d]    the key/value cache, Nk rows per head
 *   v          in   bf16 [B, Hkv, Nk, d]
 *   o          out  bf16 [B, Hq,  Nq, d]
 *   lse        out  fp32 [B, Hq,  Nq]       natural-log logsumexp, as in flash_attn_fwd
 *   seqlens_k  in   int32 [B] device array, or NULL: batch entry b uses the
 *              first L_b = seqlens_k[b] rows of its cache (clamped to
 *              [0, Nk]; rows past L_b are never read into the result). NULL:
 *              L_b = Nk for every entry.
 * causal: query row i is token L_b - Nq + i of the sequence the keys belong to
 * (the queries are its last Nq tokens) and sees keys j <= L_b - Nq + i.
 * causal = 0: every row sees all L_b keys. With Nq = Nk = L_b and causal = 1
 * the result is that of flash_attn_fwd. window > 0 (causal only) adds a
 * sliding window: row i also loses keys j <= L_b - Nq + i - window (as in
 * flash_attn_fwd_window), and only the cache tiles the window covers are
 * read. window = 0: no window. A row that sees no key at all (L_b = 0, or
 * L_b - Nq + i < 0) gets O = 0 and LSE = -inf.
 * Supported: B, Hq, Hkv, Nq, Nk >= 1; Hq % Hkv == 0; d as above (8 .. 256); Nq <= Nk
 * when causal; Nk * d * 2 < 2^31 bytes per K/V head. Any Nq is accepted; the path is made
 * for (Hq / Hkv) * Nq <= 128 query rows per K/V head, and larger counts read
 * the cache once per 128 rows. Inputs and outputs must not overlap.
 * workspace: device memory of workspace_bytes >=
 * flash_attn_decode_workspace_size(...) for the per-range partial results;
 * NULL is accepted when that size is 0. Contents on entry are ignored and on
 * return are unspecified. Runs two kernels on `stream` (the range kernel and
 * the merge), or one when the shape needs a single range per head. Results do
 * not depend on the stream or on earlier calls (no atomics).
 */
int flash_attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* seqlens_k, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      int causal, int window, float scale, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace flash_attn_decode needs for these arguments, or 0
 * when it needs none or rejects the shape (including window < 0, or a window
 * without the causal mask). It depends on the cache capacity Nk and the
 * window, not on seqlens_k. The workspace holds, for every
 * key range of every K/V head and every query row, one fp32 logsumexp and d
 * fp32 output values: about R * B * Hq * Nq * (d + 1) * 4 bytes for R ranges
 * per head (R is chosen from the shape so that the grid fills the GPU).
 */
size_t flash_attn_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                                        int window);

/*
 * flash_attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks, kernels and results as flash_attn_decode, without
 * the workspace: the per-range partial results go to a static device array of
 * flash_attn_decode_noalloc_max_bytes() bytes (32 MiB) that the library holds
 * on every GPU it runs on until the process ends. The call allocates and frees
 * nothing. Its first call on a GPU looks up that GPU's copy of the array
 * (hipGetSymbolAddress, with that GPU current) and caches the address; the
 * runtime loads the library's code object for that GPU then if it has not yet.
 *   Limit: shapes whose flash_attn_decode_workspace_size(...) exceeds the
 *   array return FA_ERR_SCRATCH and enqueue nothing (the largest plans, near
 *   67 MB, need 128 query rows per K/V head at d = 256 over few heads).
 *   Sharing: every call on one GPU uses the same array, and the partial results
 *   of a call live there from its range kernel to its merge kernel. Calls that
 *   overlap on one GPU (different streams, or host threads each enqueueing on
 *   its own stream) race and give unspecified results: the caller serialises
 *   them, for example by enqueueing them on one stream. Nothing in the array
 *   needs to start at zero (every partial slot a merge reads is written first
 *   by the same call), and the array keeps the last call's contents.
 */
int flash_attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* seqlens_k, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                              int causal, int window, float scale, void* stream);

/* Bytes of the static scratch array flash_attn_decode_noalloc uses on each GPU. */
size_t flash_attn_decode_noalloc_max_bytes(void);

/*
 * Backward pass of flash_attn_fwd_window: the gradients of sum(dout * O) under
 * the sliding-window causal mask (row i sees keys i - window < j <= i).
 * Arguments, workspace (flash_attn_bwd_workspace_size with causal = 1) and
 * behaviour as in flash_attn_bwd with causal = 1; o and lse must come from
 * flash_attn_fwd_window with the same window. window >= 1. Key tiles before a
 * row block's window and row blocks past a key block's window are not read.
 */
int flash_attn_bwd_window(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int N, int d, int window, float scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of flash_attn_fwd_varlen: the gradients of sum(dout * O) for
 * packed sequences, every sequence on its own.
 *   q, k, v, o, dout, dq, dk, dv   [H, total, d] as in flash_attn_fwd_varlen
 *   lse                            fp32 [Hq, total] from flash_attn_fwd_varlen
 *   cu_seqlens                     int32 [B + 1] device array, as there
 * workspace: flash_attn_bwd_workspace_size(1, Hq, Hkv, total, d, causal) bytes
 * (the packed arrays are one sequence of `total` rows to the preparation and
 * the workspace). With causal = 1 each row's keys run from its sequence's
 * start to itself; with causal = 0, over its whole sequence. The gradient
 * kernels read only those keys, as in flash_attn_bwd_window with a per-row
 * first (and, non-causal, last) key. max_seqlen is checked (>= 1) but not
 * otherwise needed.
 * Offsets are clamped in the kernels as in flash_attn_fwd_varlen.
 */
int flash_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          const int* cu_seqlens, int B, int max_seqlen, int total, int Hq, int Hkv,
                          int d, int causal, float scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Block quantisation of a bf16 tensor to 8-bit floating point codes, the input
 * form of an FP8 forward. FlashAttention-3 runs its forward in FP8 with block
 * scaling (mlapandio "FlashAttention: IO-aware exact attention", Generations;
 * wishwiki "FlashAttention", "Evolution: FlashAttention-2 and -3"); the pages fix no format.
 *
 *   x       bf16 [BH, N, d] contiguous (e.g. [B, H, N, d] with BH = B * H),
 *           finite values (a NaN or infinity gives unspecified codes for its run)
 *   codes   uint8 [BH, N, d]: OCP E4M3 codes (bias 7, 3 mantissa bits, no
 *           infinities, largest finite 448; 0x7F / 0xFF are NaN and never written)
 *   scales  fp32 [BH, ceil(N / rows)]: one per run of `rows` rows of a slab,
 *           the last run of a slab ragged
 *
 * Per run, in fp32: amax = max |x|, inv = 448 / amax, code = E4M3(x * inv)
 * rounded to nearest (ties to even) and saturated at 448, scale = amax / 448
 * (both divisions correctly rounded); an all-zero run gets scale 1. A run
 * with amax below 2^-64 is first multiplied by 2^64 (exact; 448 / amax would
 * overflow otherwise): its codes are those of the scaled run and its scale is
 * (2^64 amax / 448) * 2^-64. Then x ~ code * scale, within 2^-4 relative for
 * codes of magnitude >= 2^-6 (an fp32-subnormal scale, for amax below about
 * 2^-117, keeps at least 7 significant bits for any bf16 input).
 * d: a multiple of 8; rows >= 1. x and codes 16-byte aligned, scales 4-byte.
 * The caller owns every buffer; the call is asynchronous on `stream`.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (BH, N, rows < 1, or the run count or the
 * size beyond the 32-bit grid), FA_ERR_HEADDIM (d), FA_ERR_ALIGN, FA_ERR_HIP. */
int flash_attn_quantize_e4m3(const void* x, void* codes, float* scales, int BH, int N, int d, int rows,
                             void* stream);

/* The same quantisation of V, written for flash_attn_fwd_e4m3: codes and
 * scales as flash_attn_quantize_e4m3 computes them, with the codes stored
 * transposed and, inside each group of 64 keys, in the order of the FP8
 * forward's probability operand:
 *   x        bf16 [BH, N, d] contiguous, finite
 *   codes_t  uint8 [BH, d, Np], Np = N rounded up to a multiple of 64: row c of
 *            slab bh holds column c of every key; position p of key group g
 *            holds key 64 g + ((p % 32) / 16) * 32 + ((p % 16) / 4) * 8 +
 *            (p / 32) * 4 + p % 4 (a permutation of the group); keys past N
 *            hold code 0
 *   scales   fp32 [BH, ceil(N / rows)], as flash_attn_quantize_e4m3
 * rows: a multiple of 64. d: a multiple of 8. x 16-byte aligned, codes_t and
 * scales 4-byte. Errors as flash_attn_quantize_e4m3 (FA_ERR_SHAPE also for rows
 * not a multiple of 64). */
int flash_attn_quantize_e4m3_vt(const void* x, void* codes_t, float* scales, int BH, int N, int d, int rows,
                                void* stream);

/*
 * Forward pass on 8-bit inputs: FlashAttention-3's FP8 forward with block
 * scaling (mlapandio "FlashAttention: IO-aware exact attention",
 * "Generations"; wishwiki "FlashAttention", "Evolution: FlashAttention-2 and
 * -3"). The inputs are the dequantised values code * scale of
 *   q8, q_scales    flash_attn_quantize_e4m3 of q: E4M3 [B, Hq, N, d], fp32 [B, Hq, ceil(N / rows)]
 *   k8, k_scales    flash_attn_quantize_e4m3 of k: E4M3 [B, Hkv, N, d], fp32 [B, Hkv, ceil(N / rows)]
 *   v8t, v_scales   flash_attn_quantize_e4m3_vt of v: E4M3 [B, Hkv, d, Np], fp32 [B, Hkv, ceil(N / rows)]
 * and the outputs are as in flash_attn_fwd:
 *   o    out  bf16 [B, Hq, N, d]
 *   lse  out  fp32 [B, Hq, N]
 * Both products run on the FP8 matrix cores; the probabilities are rounded to
 * E4M3 for the P.V product (3 mantissa bits: the result is close to, not
 * within bf16 rounding of, the attention of the dequantised inputs; O is
 * normalised by the sum of the rounded probabilities, so their weights sum to
 * one as used). Scores and softmax statistics are fp32.
 * Supported: B, Hq, Hkv, N >= 1; Hq % Hkv == 0; d in {64, 128}; rows a
 * multiple of 64 (the same run length for q, k and v); Np * d < 2^31.
 * causal: 0 or 1 (row i sees keys j <= i). Code and output pointers 16-byte
 * aligned, scale arrays 4-byte. Asynchronous on `stream`; nothing allocated.
 */
int flash_attn_fwd_e4m3(const void* q8, const float* q_scales, const void* k8, const float* k_scales,
                        const void* v8t, const float* v_scales, void* o, float* lse, int B, int Hq, int Hkv, int N,
                        int d, int causal, float scale, int rows, void* stream);

/* Static text for a status code. For FA_ERR_HIP the text also holds the HIP
 * error string of the calling thread's last failed launch. Never NULL. */
const char* flash_attn_strerror(int status);

/* Library version and the GPU target it was compiled for, e.g. "0.8.0 gfx950". */
const char* flash_attn_version(void);

/*
 * Launch shape flash_attn_fwd would use for these arguments on the current GPU,
 * for logging and tests of the host logic (no GPU work, nothing enqueued):
 *   out[0] query rows per workgroup, out[1] keys per streamed tile,
 *   out[2] threads per workgroup, out[3] workgroups, out[4] LDS bytes per
 *   workgroup.
 * At d <= 64 the forward takes workgroups of 8 waves (256 rows) or, for large
 * grids, 12 waves (384 rows, three per SIMD); the choice depends on B * Hq, N
 * and the GPU's compute-unit count (256 assumed when no GPU is current).
 * Returns FA_ERR_NULL for a NULL out, or the status flash_attn_fwd would
 * return for a rejected shape (out is then left unchanged).
 */
int flash_attn_fwd_geometry(int B, int Hq, int Hkv, int N, int d, int causal, int* out);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H */
