/*
 * oracle.c -- plain, slow, fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The HIP path never calls it, and the
 * two share no code.
 *
 * What it computes: the textbook definition the FlashAttention pages say the
 * tiled algorithm reproduces exactly. The mlapandio page "FlashAttention:
 * IO-aware exact attention" (Definition; "Four ideas", online softmax item)
 * says the result is exact and ends equal to the ordinary softmax. The
 * wishwiki "FlashAttention" page ("The IO-Aware Insight") calls the outputs
 * identical to standard attention. So this file does not use the online
 * recurrence. For every query row it materialises the score row S and the
 * probability row P in full, as the "NAIVE" half of the mlapandio naive-vs-flash
 * diagram does, and takes the softmax in two passes (max, then sum).
 *
 *   scores   S_ij = s * sum_c q_ic k_jc            for visible keys j
 *   softmax  m_i = max_j S_ij,  e_ij = exp(S_ij - m_i),  l_i = sum_j e_ij
 *            P_ij = e_ij / l_i   (0 for masked keys)
 *   output   O_i = sum_j P_ij v_j
 *   LSE      L_i = m_i + ln l_i  (natural log of sum_j exp(S_ij))
 *
 * Key j is visible to query i when the mask is off, or when j <= pos_i under
 * the causal mask; a sliding window W > 0 (local attention) also hides keys
 * j <= pos_i - W, leaving the W most recent positions. pos_i is the query's position among the keys (pos_i = i when
 * queries and keys are the same sequence). Query head h reads key/value head
 * h / (Hq / Hkv) (grouped-query attention, mlapandio "Two notes").
 *
 * Backward: the pages say only that the backward pass rebuilds P from the
 * stored logsumexp (mlapandio "Four ideas", recomputation item; techtrendtracker
 * "Recomputation in the Backward Pass"). The gradients below are the chain rule
 * of the definition for the loss sum(dO * O):
 *   D_i   = sum_c dO_ic O_ic
 *   dP_ij = sum_c dO_ic v_jc
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = s sum_j dS_ij k_j
 *   dK_j  = s sum_{heads in group} sum_i dS_ij q_i
 *   dV_j  =   sum_{heads in group} sum_i P_ij dO_i
 * D_i is the row dot of dO with the forward's output. The backward's caller
 * hands in O as the forward stored it, and the interface stores O in bfloat16.
 * The backward functions therefore take a flag, o_bf16. When it is set, D_i is
 * formed from O_i rounded to bfloat16 (round to nearest, ties to even),
 * which models that storage step. When it is clear, D_i uses the exact fp64
 * O_i. Everything else stays exact fp64 in both modes.
 *
 * 8-bit inputs (test infrastructure for an FP8 forward, which the pages credit
 * to FlashAttention-3 with block scaling): an E4M3 codec and an fp32 block
 * quantiser, below. The attention on such inputs is the definition above on
 * the exactly dequantised values code * scale.
 *
 * Layout: every tensor is contiguous [B, H, N, d] float64 (d fastest);
 * LSE and D are [B, Hq, N]. Functions return 0, or -1 on bad arguments or
 * allocation failure.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int thread_id(void) {
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

static double dot(const double* a, const double* b, int d) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += a[c] * b[c];
    return acc;
}

/* x rounded to the nearest bfloat16 value (8 significant bits), ties to even.
 * frexp gives x = m * 2^e with 0.5 <= |m| < 1, so m * 2^8 holds the 8 kept
 * bits left of the point; nearbyint rounds it to nearest, ties to even, in the
 * default rounding mode. Normal bfloat16 range only (the attention outputs
 * here are far from its limits). */
static double round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    const double m = frexp(x, &e);
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

static int is_visible(int64_t pos_i, int j, int causal, int window) {
    return !causal || ((int64_t)j <= pos_i && (window <= 0 || (int64_t)j > pos_i - window));
}

/*
 * One query row against one key/value head.
 *   qi[d], kh[Nk*d], vh[Nk*d]  -> S[Nk], P[Nk] (scratch, filled), oi[d], *lse_i
 * Returns the number of visible keys.
 */
static int attend_row(const double* qi, const double* kh, const double* vh, int Nk, int d,
                      int64_t pos_i, int causal, int window, double s, double* S, double* P,
                      double* oi, double* lse_i) {
    int visible = 0;
    double m = -INFINITY;
    for (int j = 0; j < Nk; ++j) {
        if (is_visible(pos_i, j, causal, window)) {
            S[j] = s * dot(qi, kh + (size_t)j * d, d);
            if (S[j] > m) m = S[j];
            ++visible;
        } else {
            S[j] = -INFINITY;
        }
    }
    for (int c = 0; c < d; ++c) oi[c] = 0.0;
    if (visible == 0) {          /* no visible key: empty sum */
        for (int j = 0; j < Nk; ++j) P[j] = 0.0;
        *lse_i = -INFINITY;
        return 0;
    }
    double l = 0.0;
    for (int j = 0; j < Nk; ++j) {
        P[j] = is_visible(pos_i, j, causal, window) ? exp(S[j] - m) : 0.0;
        l += P[j];
    }
    for (int j = 0; j < Nk; ++j) P[j] /= l;
    for (int j = 0; j < Nk; ++j) {
        if (P[j] == 0.0) continue;
        const double* vj = vh + (size_t)j * d;
        for (int c = 0; c < d; ++c) oi[c] += P[j] * vj[c];
    }
    *lse_i = m + log(l);
    return visible;
}

static int check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    return 0;
}

/*
 * Forward. q [B,Hq,Nq,d], k,v [B,Hkv,Nk,d] -> o [B,Hq,Nq,d], lse [B,Hq,Nq].
 * qpos[Nq] gives each query row's position for the causal mask (NULL: row i
 * is position i); window > 0 limits a causal row to its `window` most recent
 * positions (0: no limit).
 */
int oracle_attn_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                    int B, int Hq, int Hkv, int Nq, int Nk, int d, const int64_t* qpos,
                    int causal, int window, double scale) {
    if (!q || !k || !v || !o || !lse || check_shape(B, Hq, Hkv, Nq, Nk, d)) return -1;
    const int G = Hq / Hkv;
    const int nt = max_threads();
    double* scratch = (double*)malloc(sizeof(double) * 2 * (size_t)Nk * nt);
    if (!scratch) return -1;
    const int64_t rows = (int64_t)B * Hq * Nq;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
        const int i = (int)(r % Nq);
        const int h = (int)((r / Nq) % Hq);
        const int b = (int)(r / ((int64_t)Nq * Hq));
        const int hk = h / G;
        const double* kh = k + ((size_t)b * Hkv + hk) * (size_t)Nk * d;
        const double* vh = v + ((size_t)b * Hkv + hk) * (size_t)Nk * d;
        double* S = scratch + (size_t)thread_id() * 2 * Nk;
        double* P = S + Nk;
        attend_row(q + (size_t)r * d, kh, vh, Nk, d, qpos ? qpos[i] : i, causal, window, scale, S, P,
                   o + (size_t)r * d, lse + r);
    }
    free(scratch);
    return 0;
}

/*
 * Probability matrix, for checking invariants at small sizes:
 * p [B,Hq,Nq,Nk] = softmax rows (0 on masked keys).
 */
int oracle_attn_probs(const double* q, const double* k, double* p, int B, int Hq, int Hkv, int Nq,
                      int Nk, int d, const int64_t* qpos, int causal, int window, double scale) {
    if (!q || !k || !p || check_shape(B, Hq, Hkv, Nq, Nk, d)) return -1;
    const int G = Hq / Hkv;
    double* S = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    double* zeros = (double*)calloc((size_t)Nk * d, sizeof(double));
    if (!S || !o || !zeros) { free(S); free(o); free(zeros); return -1; }
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h)
            for (int i = 0; i < Nq; ++i) {
                const size_t r = ((size_t)b * Hq + h) * Nq + i;
                const double* kh = k + ((size_t)b * Hkv + h / G) * (size_t)Nk * d;
                double lse;
                attend_row(q + r * d, kh, zeros, Nk, d, qpos ? qpos[i] : i, causal, window, scale, S,
                           p + r * Nk, o, &lse);
            }
    free(S); free(o); free(zeros);
    return 0;
}

/*
 * Gradient contributions of one query row i against one key/value head, for
 * the loss sum(dout * O) (definition in the header comment).
 *   fills S, P (scratch, length N), oi[d], *lse_i, *D_i
 *   dqi: receives dQ_i when not NULL
 *   dK_j, dV_j contributions are added to dk_acc / dv_acc at row slot[j];
 *   slot == NULL means slot j for every key, slot[j] < 0 skips key j.
 */
static void bwd_row(const double* qi, const double* doi, const double* kh, const double* vh,
                    int N, int d, int i, int causal, int window, double scale, double* S, double* P,
                    double* oi, double* lse_i, double* D_i, double* dqi, const int* slot,
                    double* dk_acc, double* dv_acc, int o_bf16, double* ostore) {
    attend_row(qi, kh, vh, N, d, i, causal, window, scale, S, P, oi, lse_i);
    for (int c = 0; c < d; ++c) ostore[c] = o_bf16 ? round_bf16(oi[c]) : oi[c];
    const double Di = dot(doi, ostore, d);
    *D_i = Di;
    if (dqi)
        for (int c = 0; c < d; ++c) dqi[c] = 0.0;
    for (int j = 0; j < N; ++j) {
        if (!is_visible(i, j, causal, window)) continue;
        const int sj = slot ? slot[j] : j;
        if (!dqi && sj < 0) continue;
        const double dPij = dot(doi, vh + (size_t)j * d, d);
        const double dSij = P[j] * (dPij - Di);
        const double* kj = kh + (size_t)j * d;
        if (dqi)
            for (int c = 0; c < d; ++c) dqi[c] += scale * dSij * kj[c];
        if (sj >= 0) {
            double* dkj = dk_acc + (size_t)sj * d;
            double* dvj = dv_acc + (size_t)sj * d;
            for (int c = 0; c < d; ++c) {
                dkj[c] += scale * dSij * qi[c];
                dvj[c] += P[j] * doi[c];
            }
        }
    }
}

/*
 * Backward, optionally restricted to some outputs, queries and keys the same
 * sequence (N). Inputs q, dout [B,Hq,N,d]; k, v [B,Hkv,N,d].
 *  rows (nrows entries, ascending, or NULL = every row): dq [B,Hq,nrows,d] gets
 *      dQ of those rows;
 *  keys (nkeys entries, or NULL = every key): dk, dv [B,Hkv,nkeys,d] get dK, dV
 *      of those keys (summed over the K/V head's query group);
 *  optional (may be NULL, only with rows == NULL): o [B,Hq,N,d], lse and D [B,Hq,N].
 * Every query row of every head still runs its full softmax, because dK_j and
 * dV_j sum over all rows. Rows are split over threads; each thread sums its
 * dK/dV contributions in a private buffer, and the buffers are added in thread
 * order afterwards.
 */
static int bwd_impl(const double* q, const double* k, const double* v, const double* dout,
                    const int64_t* rows, int nrows, const int64_t* keys, int nkeys, double* dq,
                    double* dk, double* dv, double* o_out, double* lse_out, double* D_out, int B,
                    int Hq, int Hkv, int N, int d, int causal, int window, double scale, int o_bf16) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || check_shape(B, Hq, Hkv, N, N, d)) return -1;
    if (!rows) nrows = N;
    if (!keys) nkeys = N;
    if (nrows < 0 || nkeys < 0 || (rows && (o_out || lse_out || D_out))) return -1;
    const int G = Hq / Hkv;
    const int nt = max_threads();
    const size_t head = (size_t)N * d, kout = (size_t)nkeys * d;
    int* slot = NULL;   /* key j -> output row, or -1 */
    int* rslot = NULL;  /* row i -> dq output row, or -1 */
    if (keys) {
        slot = (int*)malloc(sizeof(int) * (size_t)N);
        if (!slot) return -1;
        for (int j = 0; j < N; ++j) slot[j] = -1;
        for (int t = 0; t < nkeys; ++t) {
            if (keys[t] < 0 || keys[t] >= N) { free(slot); return -1; }
            slot[keys[t]] = t;
        }
    }
    if (rows) {
        rslot = (int*)malloc(sizeof(int) * (size_t)N);
        if (!rslot) { free(slot); return -1; }
        for (int i = 0; i < N; ++i) rslot[i] = -1;
        for (int t = 0; t < nrows; ++t) {
            if (rows[t] < 0 || rows[t] >= N) { free(slot); free(rslot); return -1; }
            rslot[rows[t]] = t;
        }
    }
    double* priv = (double*)calloc((size_t)nt * 2 * kout + 1, sizeof(double));
    double* rowbuf = (double*)malloc(sizeof(double) * (size_t)nt * (2 * (size_t)N + 2 * (size_t)d));
    if (!priv || !rowbuf) { free(priv); free(rowbuf); free(slot); free(rslot); return -1; }
    for (int b = 0; b < B; ++b) {
        for (int hk = 0; hk < Hkv; ++hk) {
            const double* kh = k + ((size_t)b * Hkv + hk) * head;
            const double* vh = v + ((size_t)b * Hkv + hk) * head;
            memset(priv, 0, sizeof(double) * (size_t)nt * 2 * kout);
            const int64_t nr = (int64_t)G * N;
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < nr; ++r) {
                const int g = (int)(r / N), i = (int)(r % N);
                const int h = hk * G + g;
                const size_t ri = (((size_t)b * Hq + h) * N + i);
                const int t = thread_id();
                double* S = rowbuf + (size_t)t * (2 * (size_t)N + 2 * (size_t)d);
                double* P = S + N;
                double* oi = P + N;
                double* ostore = oi + d;
                double* dqi = NULL;
                if (!rows) dqi = dq + ri * d;
                else if (rslot[i] >= 0) dqi = dq + (((size_t)b * Hq + h) * nrows + rslot[i]) * d;
                double lse_i, D_i;
                bwd_row(q + ri * d, dout + ri * d, kh, vh, N, d, i, causal, window, scale, S, P, oi, &lse_i,
                        &D_i, dqi, slot, priv + (size_t)t * 2 * kout, priv + (size_t)t * 2 * kout + kout,
                        o_bf16, ostore);
                if (o_out) memcpy(o_out + ri * d, oi, sizeof(double) * d);
                if (lse_out) lse_out[ri] = lse_i;
                if (D_out) D_out[ri] = D_i;
            }
            double* dkh = dk + ((size_t)b * Hkv + hk) * kout;
            double* dvh = dv + ((size_t)b * Hkv + hk) * kout;
            for (size_t e = 0; e < kout; ++e) { dkh[e] = 0.0; dvh[e] = 0.0; }
            for (int t = 0; t < nt; ++t) {
                const double* dk_t = priv + (size_t)t * 2 * kout;
                const double* dv_t = dk_t + kout;
                for (size_t e = 0; e < kout; ++e) { dkh[e] += dk_t[e]; dvh[e] += dv_t[e]; }
            }
        }
    }
    free(priv);
    free(rowbuf);
    free(slot);
    free(rslot);
    return 0;
}

/* Full backward: every dQ row and every dK/dV key, plus O, LSE and D (optional).
 * o_bf16: form D from O rounded to bfloat16 (see the header comment); window:
 * as in oracle_attn_fwd. */
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv, double* o_out, double* lse_out,
                    double* D_out, int B, int Hq, int Hkv, int N, int d, int causal, int window,
                    double scale, int o_bf16) {
    return bwd_impl(q, k, v, dout, NULL, 0, NULL, 0, dq, dk, dv, o_out, lse_out, D_out, B, Hq, Hkv,
                    N, d, causal, window, scale, o_bf16);
}

/* Sampled backward: dQ of the listed rows, dK/dV of the listed keys. */
int oracle_attn_bwd_sampled(const double* q, const double* k, const double* v, const double* dout,
                            const int64_t* rows, int nrows, const int64_t* keys, int nkeys,
                            double* dq_rows, double* dk_keys, double* dv_keys, int B, int Hq,
                            int Hkv, int N, int d, int causal, int window, double scale, int o_bf16) {
    if (!rows || !keys) return -1;
    return bwd_impl(q, k, v, dout, rows, nrows, keys, nkeys, dq_rows, dk_keys, dv_keys, NULL, NULL,
                    NULL, B, Hq, Hkv, N, d, causal, window, scale, o_bf16);
}

/* The bfloat16 rounding the stored-O mode applies, exposed so tests can pin it. */
int oracle_round_bf16(const double* x, double* y, int64_t n) {
    if ((!x || !y) && n > 0) return -1;
    for (int64_t t = 0; t < n; ++t) y[t] = round_bf16(x[t]);
    return 0;
}

/* ---- 8-bit floating point (OCP E4M3, the "fn" variant) and block scaling ----
 * FlashAttention-3 (Shah et al.) runs the forward in FP8 with block scaling;
 * the pages fix neither the format nor the scaling, so this follows the OCP
 * 8-bit floating point definition of E4M3: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, and one NaN pattern per sign (all
 * exponent and mantissa bits set). Exponent field 0 holds the subnormals
 * m * 2^-9. The largest finite magnitude is 1.75 * 2^8 = 448. */
static double e4m3_value(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double a;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) a = ldexp((double)m, -9);
    else a = ldexp(8.0 + m, e - 10);          /* (1 + m/8) * 2^(e-7) */
    return s ? -a : a;
}

/* x rounded to the nearest E4M3 value, ties to even, magnitudes at or above
 * 448 saturated to 448 (the reading taken for overflow; block scaling keeps
 * every scaled value at or below 448 up to one fp32 rounding), NaN to 0x7F. */
static uint8_t e4m3_code(float xf) {
    const double x = (double)xf;
    if (isnan(x)) return 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    const double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal spacing 2^-9; a count of 8 is the smallest normal, code 8 */
        return sign | (uint8_t)nearbyint(ldexp(a, 9));
    }
    int E;
    frexp(a, &E);                              /* a = f * 2^E, 0.5 <= f < 1 */
    int ee = E - 1;                            /* a = (1.x) * 2^ee, ee in [-6, 8] */
    double q = nearbyint(ldexp(a, 3 - ee));    /* 8 .. 16 eighths */
    if (q == 16.0) { q = 8.0; ++ee; }
    return sign | (uint8_t)(((ee + 7) << 3) | ((int)q - 8));
}

int oracle_e4m3_decode(const uint8_t* c, double* y, int64_t n) {
    if ((!c || !y) && n > 0) return -1;
    for (int64_t t = 0; t < n; ++t) y[t] = e4m3_value(c[t]);
    return 0;
}

int oracle_e4m3_encode(const float* x, uint8_t* c, int64_t n) {
    if ((!x || !c) && n > 0) return -1;
    for (int64_t t = 0; t < n; ++t) c[t] = e4m3_code(x[t]);
    return 0;
}

/* Block quantisation of a contiguous [BH, N, d] fp32 tensor: each run of R
 * rows of one (b, h) slab (the last one ragged) gets one scale. In fp32, as a
 * kernel would do it: amax = the largest |x| of the block, inv = 448 / amax
 * (one rounded division), code = E4M3(x * inv) (one rounded product), and the
 * stored dequantisation scale is amax / 448, so that x ~ code * scale. An
 * all-zero block gets inv = scale = 1. A block with amax below 2^-64 is taken
 * times 2^64 first (amax and every x; exact), so that 448 / amax stays finite,
 * and its stored scale is (2^64 amax / 448) * 2^-64 (two roundings). The
 * codes are then those of the block times 2^64. Scales are [BH, ceil(N / R)]. */
int oracle_quantize_e4m3_blocks(const float* x, uint8_t* codes, float* scales, int64_t BH, int N,
                                int d, int R) {
    if (!x || !codes || !scales || BH < 0 || N < 0 || d <= 0 || R <= 0) return -1;
    const int nb = (N + R - 1) / R;
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int b = 0; b < nb; ++b) {
            const int r0 = b * R, r1 = r0 + R < N ? r0 + R : N;
            const float* xb = x + (bh * N + r0) * (int64_t)d;
            uint8_t* cb = codes + (bh * N + r0) * (int64_t)d;
            const int64_t cnt = (int64_t)(r1 - r0) * d;
            float amax = 0.0f;
            for (int64_t t = 0; t < cnt; ++t) {
                const float a = fabsf(xb[t]);
                if (!(a <= FLT_MAX)) return -2;        /* NaN or infinite input */
                if (a > amax) amax = a;
            }
            /* below 2^-64, 448 / amax could overflow: the run is first scaled
             * up by 2^64 (exact), and the stored scale scaled back down */
            const int tiny = amax > 0.0f && amax < 0x1p-64f;
            const float up = tiny ? 0x1p64f : 1.0f;
            volatile float a = amax * up;
            volatile float inv = amax > 0.0f ? 448.0f / a : 1.0f;
            volatile float sc = amax > 0.0f ? a / 448.0f : 1.0f;
            volatile float sc_out = sc * (tiny ? 0x1p-64f : 1.0f);
            for (int64_t t = 0; t < cnt; ++t) {
                volatile float xs = xb[t] * up;
                volatile float y = xs * inv;
                cb[t] = e4m3_code(y);
            }
            sc = sc_out;
            scales[bh * nb + b] = sc;
        }
    }
    return 0;
}

int oracle_num_threads(void) { return max_threads(); }
