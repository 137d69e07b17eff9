"""Pins for the fp64 oracle: checks against facts other than the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with a closed form, a hand formula, an invariant, an independent
library implementation, finite differences, or high-precision arithmetic.
``tests/test_oracle_pins.py`` runs them on the in-tree oracle, and
``tests/test_oracle_mutants.py`` runs them on deliberately broken oracle builds.
A mistake planted anywhere in the oracle should trip at least one pin.

Sources of the facts: the FlashAttention pages say the method computes exact
softmax attention (mlapandio "FlashAttention: IO-aware exact attention",
Definition and "Four ideas"; wishwiki "FlashAttention", "The IO-Aware
Insight"). Everything else follows from the algebra of that definition.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(shape, seed, scale=1.0):
    return _rng(seed).standard_normal(shape) * scale


def _close(a, b, tol=TOL, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ tiny hand cases
def pin_one_token(orc):
    """N = 1: the only key has probability 1, so O = v, LSE = s q.k, dV = dO, dQ = dK = 0."""
    d = 5
    q, k, v, do = (_rand((1, 1, 1, d), s) for s in (1, 2, 3, 4))
    s = 0.37
    for causal in (False, True):
        o, lse = orc.fwd(q, k, v, causal, s)
        _close(o, v, what="N=1 O")
        _close(lse[0, 0, 0], s * float(q[0, 0, 0] @ k[0, 0, 0]), what="N=1 LSE")
        g = orc.bwd(q, k, v, do, causal, s)
        _close(g["dv"], do, what="N=1 dV")
        _close(g["dq"], 0 * q, what="N=1 dQ")
        _close(g["dk"], 0 * k, what="N=1 dK")


def pin_two_tokens(orc):
    """N = 2, by the logistic form of a two-way softmax: p = sigmoid(S_0 - S_1).

    O_i = p v_0 + (1 - p) v_1, LSE_i = max + log1p(exp(-|S_0 - S_1|)),
    dS_i0 = p (1 - p) dO_i.(v_0 - v_1) = -dS_i1, dQ_i = s dS_i0 (k_0 - k_1),
    dK_1 = -dK_0, dV_0 = sum_i p_i dO_i, dV_1 = sum_i (1 - p_i) dO_i.
    Causal: row 0 sees only key 0."""
    d = 3
    q, k, v, do = (_rand((1, 1, 2, d), s) for s in (11, 12, 13, 14))
    s = 0.8
    qq, kk, vv, dd = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    for causal in (False, True):
        o, lse = orc.fwd(q, k, v, causal, s)
        g = orc.bwd(q, k, v, do, causal, s)
        dq_ref = np.zeros((2, d))
        dk_ref = np.zeros((2, d))
        dv_ref = np.zeros((2, d))
        for i in range(2):
            S0, S1 = s * (qq[i] @ kk[0]), s * (qq[i] @ kk[1])
            if causal and i == 0:
                _close(o[0, 0, 0], vv[0], what="N=2 causal row 0 O")
                _close(lse[0, 0, 0], S0, what="N=2 causal row 0 LSE")
                dv_ref[0] += dd[0]
                continue
            p = 1.0 / (1.0 + math.exp(-(S0 - S1)))
            _close(o[0, 0, i], p * vv[0] + (1 - p) * vv[1], what=f"N=2 O row {i}")
            _close(lse[0, 0, i], max(S0, S1) + math.log1p(math.exp(-abs(S0 - S1))),
                   what=f"N=2 LSE row {i}")
            dS0 = p * (1 - p) * (dd[i] @ (vv[0] - vv[1]))
            dq_ref[i] = s * dS0 * (kk[0] - kk[1])
            dk_ref[0] += s * dS0 * qq[i]
            dk_ref[1] -= s * dS0 * qq[i]
            dv_ref[0] += p * dd[i]
            dv_ref[1] += (1 - p) * dd[i]
        _close(g["dq"][0, 0], dq_ref, what="N=2 dQ")
        _close(g["dk"][0, 0], dk_ref, what="N=2 dK")
        _close(g["dv"][0, 0], dv_ref, what="N=2 dV")


def pin_three_four_tokens_mp(orc):
    """N = 3 and 4 with explicit exp sums in 50-digit arithmetic (mpmath), using
    the ratio form O_i = sum_j v_j / sum_k exp(S_ik - S_ij)."""
    import mpmath as mp
    mp.mp.dps = 50
    for N in (3, 4):
        d = 3
        q, k, v = (_rand((1, 1, N, d), 20 + N * 3 + t) for t in range(3))
        s = 0.9
        for causal in (False, True):
            o, lse = orc.fwd(q, k, v, causal, s)
            for i in range(N):
                vis = [j for j in range(N) if (not causal or j <= i)]
                S = {j: mp.mpf(s) * mp.fsum(mp.mpf(q[0, 0, i, c]) * mp.mpf(k[0, 0, j, c]) for c in range(d))
                     for j in vis}
                for c in range(d):
                    ref = mp.fsum(mp.mpf(v[0, 0, j, c]) / mp.fsum(mp.exp(S[kk] - S[j]) for kk in vis) for j in vis)
                    _close(o[0, 0, i, c], float(ref), what=f"N={N} O[{i},{c}]")
                _close(lse[0, 0, i], float(mp.log(mp.fsum(mp.exp(S[j]) for j in vis))), what=f"N={N} LSE[{i}]")


# ------------------------------------------------------------------ closed forms / invariants
def pin_constant_v(orc):
    """All v_j equal to one vector v: O_i = v for every row; in the backward
    dQ = dK = 0 and dV_j = sum_i P_ij dO_i."""
    B, H, N, d = 1, 2, 9, 4
    q, k, do = _rand((B, H, N, d), 31), _rand((B, H, N, d), 32), _rand((B, H, N, d), 34)
    vrow = _rand((d,), 33)
    v = np.broadcast_to(vrow, (B, H, N, d)).copy()
    for causal in (False, True):
        o, _ = orc.fwd(q, k, v, causal, 0.6)
        _close(o, np.broadcast_to(vrow, o.shape), what="constant V O")
        g = orc.bwd(q, k, v, do, causal, 0.6)
        _close(g["dq"], 0 * q, tol=1e-11, what="constant V dQ")
        _close(g["dk"], 0 * k, tol=1e-11, what="constant V dK")
        P = orc.probs(q, k, causal, 0.6)
        _close(g["dv"], np.einsum("bhij,bhid->bhjd", P, do), what="constant V dV")


def pin_causal_row_zero(orc):
    """Causal row 0 sees key 0 only: O_0 = v_0, LSE_0 = s q_0.k_0, dQ_0 = 0."""
    B, H, N, d = 2, 2, 7, 6
    q, k, v, do = (_rand((B, H, N, d), 40 + t) for t in range(4))
    s = 0.45
    o, lse = orc.fwd(q, k, v, True, s)
    _close(o[:, :, 0], v[:, :, 0], what="causal row 0 O")
    _close(lse[:, :, 0], s * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), what="causal row 0 LSE")
    g = orc.bwd(q, k, v, do, True, s)
    _close(g["dq"][:, :, 0], 0 * q[:, :, 0], what="causal row 0 dQ")


def pin_uniform_scale_zero(orc):
    """scale = 0 makes every visible key equally likely: non-causal O_i = mean_j v_j
    and LSE_i = ln N; causal O_i = prefix mean over j <= i and LSE_i = ln(i+1)."""
    B, H, N, d = 1, 2, 11, 4
    q, k, v = (_rand((B, H, N, d), 50 + t) for t in range(3))
    o, lse = orc.fwd(q, k, v, False, 0.0)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), what="uniform O")
    _close(lse, np.full(lse.shape, math.log(N)), what="uniform LSE")
    o, lse = orc.fwd(q, k, v, True, 0.0)
    counts = np.arange(1, N + 1, dtype=np.float64)
    _close(o, np.cumsum(v, axis=2) / counts[None, None, :, None], what="prefix-mean O")
    _close(lse, np.broadcast_to(np.log(counts), lse.shape), what="prefix-mean LSE")


def pin_probability_rows(orc):
    """Rows of P are a probability distribution over the visible keys: entries
    >= 0, exactly 0 on masked keys, summing to 1. O is P times V."""
    B, H, N, d = 1, 3, 12, 5
    q, k, v = (_rand((B, H, N, d), 60 + t, 1.5) for t in range(3))
    for causal in (False, True):
        P = orc.probs(q, k, causal, 0.7)
        assert np.all(P >= 0), "negative probability"
        _close(P.sum(axis=-1), np.ones((B, H, N)), what="P row sums")
        if causal:
            assert np.all(P[..., np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]] == 0), "masked P != 0"
        o, _ = orc.fwd(q, k, v, causal, 0.7)
        _close(o, P @ v, what="O = P V")


def pin_key_translation(orc):
    """Adding one vector c to every key leaves O unchanged and shifts LSE_i by s q_i.c."""
    B, H, N, d = 1, 2, 10, 4
    q, k, v = (_rand((B, H, N, d), 70 + t) for t in range(3))
    c = _rand((d,), 74)
    s = 0.5
    for causal in (False, True):
        o1, l1 = orc.fwd(q, k, v, causal, s)
        o2, l2 = orc.fwd(q, k + c, v, causal, s)
        _close(o2, o1, tol=1e-11, what="translation O")
        _close(l2 - l1, s * (q @ c), tol=1e-11, what="translation LSE")


def pin_gqa_equals_repeated_mha(orc):
    """Grouped-query attention equals multi-head attention with each K/V head
    repeated G times in order; dK/dV are the group sums of the repeated-head ones."""
    B, Hq, Hkv, N, d = 2, 6, 2, 8, 4
    G = Hq // Hkv
    q, do = _rand((B, Hq, N, d), 80), _rand((B, Hq, N, d), 83)
    k, v = _rand((B, Hkv, N, d), 81), _rand((B, Hkv, N, d), 82)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        o1, l1 = orc.fwd(q, k, v, causal, 0.5)
        o2, l2 = orc.fwd(q, kr, vr, causal, 0.5)
        _close(o1, o2, what="GQA O")
        _close(l1, l2, what="GQA LSE")
        g1 = orc.bwd(q, k, v, do, causal, 0.5)
        g2 = orc.bwd(q, kr, vr, do, causal, 0.5)
        _close(g1["dq"], g2["dq"], what="GQA dQ")
        _close(g1["dk"], g2["dk"].reshape(B, Hkv, G, N, d).sum(2), what="GQA dK")
        _close(g1["dv"], g2["dv"].reshape(B, Hkv, G, N, d).sum(2), what="GQA dV")


def pin_head_permutation(orc):
    """Heads and batch entries are independent: permuting them permutes the outputs."""
    B, H, N, d = 2, 3, 6, 4
    q, k, v, do = (_rand((B, H, N, d), 90 + t) for t in range(4))
    perm_b, perm_h = [1, 0], [2, 0, 1]

    def p(x):
        return x[perm_b][:, perm_h]

    o1, l1 = orc.fwd(q, k, v, True, 0.4)
    o2, l2 = orc.fwd(p(q), p(k), p(v), True, 0.4)
    _close(o2, p(o1), what="permuted O")
    _close(l2, p(l1), what="permuted LSE")
    g1 = orc.bwd(q, k, v, do, True, 0.4)
    g2 = orc.bwd(p(q), p(k), p(v), p(do), True, 0.4)
    for key in ("dq", "dk", "dv"):
        _close(g2[key], p(g1[key]), what=f"permuted {key}")


def pin_last_row_and_positions(orc):
    """The causal last row sees every key, so it equals the non-causal last row.
    Query rows given with explicit positions give the same rows as the full run."""
    B, H, N, d = 1, 2, 13, 4
    q, k, v = (_rand((B, H, N, d), 100 + t) for t in range(3))
    oc, lc = orc.fwd(q, k, v, True, 0.6)
    on, ln = orc.fwd(q, k, v, False, 0.6)
    _close(oc[:, :, -1], on[:, :, -1], what="last row O")
    _close(lc[:, :, -1], ln[:, :, -1], what="last row LSE")
    rows = np.array([0, 4, 12], dtype=np.int64)
    os_, ls_ = orc.fwd(q[:, :, rows], k, v, True, 0.6, qpos=rows)
    _close(os_, oc[:, :, rows], what="row-subset O")
    _close(ls_, lc[:, :, rows], what="row-subset LSE")


def pin_gradient_sums(orc):
    """Each row of dS sums to 0, so sum_j dK_j = 0 per KV head; rows of P sum to 1,
    so sum_j dV_j = sum over the group's heads and rows of dO."""
    B, Hq, Hkv, N, d = 1, 4, 2, 10, 5
    q, do = _rand((B, Hq, N, d), 110), _rand((B, Hq, N, d), 113)
    k, v = _rand((B, Hkv, N, d), 111), _rand((B, Hkv, N, d), 112)
    for causal in (False, True):
        g = orc.bwd(q, k, v, do, causal, 0.7)
        _close(g["dk"].sum(axis=2), np.zeros((B, Hkv, d)), tol=1e-11, what="sum dK")
        _close(g["dv"].sum(axis=2), do.reshape(B, Hkv, Hq // Hkv, N, d).sum(axis=(2, 3)), tol=1e-11,
               what="sum dV")


def pin_large_logits(orc):
    """Scores near +-700 (exp would overflow fp64 without a max shift): O and
    LSE must match 50-digit arithmetic."""
    import mpmath as mp
    mp.mp.dps = 50
    N, d = 6, 2
    q = np.array([[30.0, -20.0]] * N)[None, None]
    k = _rand((1, 1, N, d), 120) * 25.0
    v = _rand((1, 1, N, d), 121)
    s = 1.0
    o, lse = orc.fwd(q, k, v, False, s)
    for i in range(N):
        S = [mp.mpf(s) * (mp.mpf(q[0, 0, i, 0]) * mp.mpf(k[0, 0, j, 0]) + mp.mpf(q[0, 0, i, 1]) * mp.mpf(k[0, 0, j, 1]))
             for j in range(N)]
        Z = mp.fsum(mp.exp(x) for x in S)
        _close(lse[0, 0, i], float(mp.log(Z)), tol=1e-9, what="large-logit LSE")
        for c in range(d):
            _close(o[0, 0, i, c], float(mp.fsum(mp.exp(S[j]) * mp.mpf(v[0, 0, j, c]) for j in range(N)) / Z),
                   what="large-logit O")


# ------------------------------------------------------------------ independent implementations
def pin_torch_sdpa(orc):
    """torch's own fp64 CPU attention (its math path) and autograd agree with the
    oracle on O and on the gradients of sum(dO * O); LSE against torch.logsumexp."""
    import torch
    torch.manual_seed(0)
    B, Hq, Hkv, N, d = 2, 4, 2, 17, 8
    G = Hq // Hkv
    q, do = _rand((B, Hq, N, d), 130), _rand((B, Hq, N, d), 133)
    k, v = _rand((B, Hkv, N, d), 131), _rand((B, Hkv, N, d), 132)
    s = 1.0 / math.sqrt(d)
    for causal in (False, True):
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        to = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), is_causal=causal, scale=s)
        (to * torch.tensor(do)).sum().backward()
        o, lse = orc.fwd(q, k, v, causal, s)
        _close(o, to.detach().numpy(), tol=1e-12, what="SDPA O")
        g = orc.bwd(q, k, v, do, causal, s)
        _close(g["dq"], tq.grad.numpy(), tol=1e-11, what="autograd dQ")
        _close(g["dk"], tk.grad.numpy(), tol=1e-11, what="autograd dK")
        _close(g["dv"], tv.grad.numpy(), tol=1e-11, what="autograd dV")
        scores = torch.tensor(q) @ torch.tensor(k).repeat_interleave(G, 1).transpose(-1, -2) * s
        if causal:
            scores = scores.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        _close(lse, torch.logsumexp(scores, -1).numpy(), what="logsumexp LSE")


def pin_finite_differences(orc):
    """Central differences of the loss sum(dO * O(Q, K, V)) match the analytic
    gradients (N <= 6, d <= 3, both masks, groups of 1 and 2 heads)."""
    h = 1e-6
    for (Hq, Hkv, causal) in ((1, 1, False), (2, 1, True), (2, 2, True), (2, 1, False)):
        B, N, d = 1, 5, 3
        q, do = _rand((B, Hq, N, d), 140 + Hq), _rand((B, Hq, N, d), 143)
        k, v = _rand((B, Hkv, N, d), 141 + Hkv), _rand((B, Hkv, N, d), 142)
        s = 0.7
        g = orc.bwd(q, k, v, do, causal, s)

        def loss(q_, k_, v_):
            o, _ = orc.fwd(q_, k_, v_, causal, s)
            return float((o * do).sum())

        for name, arr in (("dq", q), ("dk", k), ("dv", v)):
            num = np.zeros_like(arr)
            it = np.nditer(arr, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                plus, minus = arr.copy(), arr.copy()
                plus[idx] += h
                minus[idx] -= h
                args_p = {"dq": (plus, k, v), "dk": (q, plus, v), "dv": (q, k, plus)}[name]
                args_m = {"dq": (minus, k, v), "dk": (q, minus, v), "dv": (q, k, minus)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(g[name], num, tol=1e-7, what=f"finite-difference {name} (Hq={Hq},Hkv={Hkv},causal={causal})")


def pin_online_recurrence(orc):
    """The tiled online recurrence in fp64 (any block sizes, ragged edges, lazy
    reference max or the sum-triggered reference) reproduces the oracle's
    definition."""
    from oracle.online import online_attention
    N, d = 37, 6
    q, k, v = (_rand((1, 1, N, d), 150 + t, 1.5) for t in range(3))
    k[0, 0, 5] *= 4.0
    for causal in (False, True):
        o, lse = orc.fwd(q, k, v, causal, 0.6)
        for br, bc, tau in ((1, 1, 0.0), (3, 5, 0.0), (16, 16, 0.0), (7, 64, 0.0), (8, 4, 8 * math.log(2)),
                            (5, 3, 2.0)):
            om, lm = online_attention(q[0, 0], k[0, 0], v[0, 0], causal, 0.6, br, bc, tau)
            _close(om, o[0, 0], what=f"online O ({br}x{bc}, tau={tau:.2f})")
            _close(lm, lse[0, 0], what=f"online LSE ({br}x{bc}, tau={tau:.2f})")
        # the sum-triggered reference: tight (moves often), the FP8 forward's 2^8,
        # the bf16 forward's 2^16, and loose enough that it never moves after the
        # first block
        for br, bc, smax in ((4, 3, 1.5), (32, 32, 256.0), (32, 32, 65536.0), (6, 5, 1e30)):
            om, lm = online_attention(q[0, 0], k[0, 0], v[0, 0], causal, 0.6, br, bc, sum_max=smax)
            _close(om, o[0, 0], what=f"online O ({br}x{bc}, sum_max={smax:g})")
            _close(lm, lse[0, 0], what=f"online LSE ({br}x{bc}, sum_max={smax:g})")


def pin_sampled_backward(orc):
    """The sampled backward (dQ of chosen rows, dK/dV of chosen keys) equals the
    same rows and keys of the full backward, with GQA and both masks."""
    B, Hq, Hkv, N, d = 2, 4, 2, 23, 6
    q, do = _rand((B, Hq, N, d), 160), _rand((B, Hq, N, d), 163)
    k, v = _rand((B, Hkv, N, d), 161), _rand((B, Hkv, N, d), 162)
    rows = np.array([0, 3, 4, 11, 22], dtype=np.int64)
    keys = np.array([22, 1, 0, 9], dtype=np.int64)
    for causal in (False, True):
        full = orc.bwd(q, k, v, do, causal, 0.4)
        smp = orc.bwd_sampled(q, k, v, do, causal, 0.4, rows, keys)
        _close(smp["dq"], full["dq"][:, :, rows], what="sampled dQ")
        _close(smp["dk"], full["dk"][:, :, keys], what="sampled dK")
        _close(smp["dv"], full["dv"][:, :, keys], what="sampled dV")


def pin_round_bf16(orc):
    """The oracle's bfloat16 rounding agrees with torch's float32 -> bfloat16
    conversion (round to nearest, ties to even) on random values, on values
    exactly halfway between two bfloat16 neighbours, and on powers of two."""
    import torch
    rng = _rng(170)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))).astype(np.float32)
    base = x.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (base | np.uint32(0x8000)).view(np.float32)          # exactly half a bf16 ulp above base
    pow2 = np.exp2(np.arange(-30, 30)).astype(np.float32)
    for arr in (x, ties, -ties, pow2):
        want = torch.from_numpy(arr).to(torch.bfloat16).to(torch.float64).numpy()
        got = orc.round_bf16(arr.astype(np.float64))
        assert np.array_equal(got, want), "bf16 rounding disagrees with torch"
    assert orc.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert orc.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def pin_stored_o_mode(orc):
    """Forming D from O rounded to bfloat16 changes D to rowsum(dO * bf16(O)) and
    nothing else. dS is linear in D, so with dD = D_stored - D_exact:
    dQ_i moves by -s dD_i sum_j P_ij k_j, dK_j by -s sum_i P_ij dD_i q_i, dV
    not at all. When O is already a bfloat16 value (constant bf16 V), both
    modes agree exactly."""
    import torch
    B, Hq, Hkv, N, d = 1, 4, 2, 13, 6
    G = Hq // Hkv
    q, do = _rand((B, Hq, N, d), 180, 1.3), _rand((B, Hq, N, d), 183)
    k, v = _rand((B, Hkv, N, d), 181, 1.3), _rand((B, Hkv, N, d), 182)
    s = 0.6
    for causal in (False, True):
        ex = orc.bwd(q, k, v, do, causal, s, o_bf16=False)
        st = orc.bwd(q, k, v, do, causal, s, o_bf16=True)
        o_b = torch.from_numpy(ex["o"]).to(torch.bfloat16).to(torch.float64).numpy()
        _close(st["D"], (do * o_b).sum(-1), what="stored-O D")
        _close(st["o"], ex["o"], what="stored-O mode keeps the exact O output")
        dD = st["D"] - ex["D"]
        P = orc.probs(q, k, causal, s)
        kr, qr = np.repeat(k, G, axis=1), q
        dq_shift = -s * dD[..., None] * (P @ kr)
        dk_shift = (-s * np.einsum("bhij,bhi,bhic->bhjc", P, dD, qr)).reshape(B, Hkv, G, N, d).sum(2)
        _close(st["dq"], ex["dq"] + dq_shift, tol=1e-11, what="stored-O dQ shift")
        _close(st["dk"], ex["dk"] + dk_shift, tol=1e-11, what="stored-O dK shift")
        _close(st["dv"], ex["dv"], what="stored-O dV unchanged")
        rows = np.array([0, 5, 12], dtype=np.int64)
        keys = np.array([12, 3], dtype=np.int64)
        sm = orc.bwd_sampled(q, k, v, do, causal, s, rows, keys, o_bf16=True)
        _close(sm["dq"], st["dq"][:, :, rows], what="stored-O sampled dQ")
        _close(sm["dk"], st["dk"][:, :, keys], what="stored-O sampled dK")
    vb = np.broadcast_to(orc.round_bf16(_rand((d,), 184)), (B, Hkv, N, d)).copy()
    a = orc.bwd(q, k, vb, do, True, s, o_bf16=False)
    b = orc.bwd(q, k, vb, do, True, s, o_bf16=True)
    for key in ("dq", "dk", "dv", "D"):
        _close(a[key], b[key], tol=1e-13, what=f"bf16-exact O: {key}")


def pin_decode_positions(orc):
    """Short query blocks at the end of a long key sequence (decode): with row i
    placed at position Nk - Nq + i, the oracle equals (a) torch's fp64 SDPA with
    that bottom-right causal mask written out, (b) the last Nq rows of the
    square causal run whose final query rows are these queries, and (c) for a
    single query, the unmasked run (it sees every key)."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = 2, 6, 2, 3, 19, 8
    G = Hq // Hkv
    q = _rand((B, Hq, Nq, d), 190)
    k, v = _rand((B, Hkv, Nk, d), 191), _rand((B, Hkv, Nk, d), 192)
    s = 0.45
    pos = Nk - Nq + np.arange(Nq, dtype=np.int64)
    o, lse = orc.fwd(q, k, v, True, s, qpos=pos)
    mask = torch.tensor(np.arange(Nk)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k).repeat_interleave(G, 1), torch.tensor(v).repeat_interleave(G, 1),
        attn_mask=mask, scale=s)
    _close(o, ref.numpy(), tol=1e-12, what="decode O vs SDPA with explicit mask")
    sc = (torch.tensor(q) @ torch.tensor(k).repeat_interleave(G, 1).transpose(-1, -2) * s).masked_fill(~mask, float("-inf"))
    _close(lse, torch.logsumexp(sc, -1).numpy(), tol=1e-12, what="decode LSE vs logsumexp")
    qf = _rand((B, Hq, Nk, d), 193)
    qf[:, :, Nk - Nq:] = q
    of, lf = orc.fwd(qf, k, v, True, s)
    _close(o, of[:, :, Nk - Nq:], what="decode rows vs square causal rows")
    _close(lse, lf[:, :, Nk - Nq:], what="decode LSE vs square causal LSE")
    o1, l1 = orc.fwd(q[:, :, -1:], k, v, True, s, qpos=np.array([Nk - 1], dtype=np.int64))
    on, ln = orc.fwd(q[:, :, -1:], k, v, False, s)
    _close(o1, on, what="single decode row vs unmasked")
    _close(l1, ln, what="single decode LSE vs unmasked")


def pin_split_merge(orc):
    """Keys split into disjoint ranges: the per-range (O, LSE) pairs merge into the
    full result by LSE = ln sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r. This
    holds only if LSE is the full log-sum-exp (max included) and O the
    normalised output. With the causal decode mask, a range a row cannot see has
    LSE = -inf and weight 0."""
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 4, 23, 6
    q = _rand((B, Hq, Nq, d), 195, 1.5)
    k, v = _rand((B, Hkv, Nk, d), 196, 1.5), _rand((B, Hkv, Nk, d), 197)
    s = 0.7
    pos = Nk - Nq + np.arange(Nq, dtype=np.int64)
    cuts = [0, 7, 16, 21, Nk]          # the last range [21, 23) is beyond row 0's position 19
    for causal in (False, True):
        qp = pos if causal else None
        o, lse = orc.fwd(q, k, v, causal, s, qpos=qp)
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            rp = (pos - a) if causal else None
            parts.append(orc.fwd(q, k[:, :, a:b], v[:, :, a:b], causal, s, qpos=rp))
        L = np.stack([p[1] for p in parts])
        if causal:
            assert np.isneginf(L[-1][..., 0]).all(), "a range after a row's position must have LSE = -inf"
        top = L.max(0)
        wsum = np.exp(L - top).sum(0)
        Lm = top + np.log(wsum)
        Om = sum(np.exp(Lr - Lm)[..., None] * p[0] for Lr, p in zip(L, parts))
        _close(Lm, lse, what=f"merged LSE causal={causal}")
        _close(Om, o, what=f"merged O causal={causal}")


def pin_sliding_window(orc):
    """Local (sliding-window) causal attention: row i keeps keys i - W < j <= i.
    (a) W >= every position is plain causal; (b) W = 1 leaves only the diagonal
    key, so O_i = v_i and LSE_i = s q_i.k_i; (c) torch's fp64 SDPA with the band
    mask written out, also for decode rows placed at the end of the keys; (d) the
    probabilities vanish outside the band and sum to 1 inside it."""
    import torch
    B, Hq, Hkv, N, d = 1, 4, 2, 23, 6
    G = Hq // Hkv
    q = _rand((B, Hq, N, d), 200)
    k, v = _rand((B, Hkv, N, d), 201), _rand((B, Hkv, N, d), 202)
    s = 0.55
    oc, lc = orc.fwd(q, k, v, True, s)
    ow, lw = orc.fwd(q, k, v, True, s, window=N)
    _close(ow, oc, what="window N O")
    _close(lw, lc, what="window N LSE")
    o1, l1 = orc.fwd(q, k, v, True, s, window=1)
    _close(o1, np.repeat(v, G, axis=1), what="window 1 O")
    _close(l1, s * np.einsum("bhnd,bhnd->bhn", q, np.repeat(k, G, axis=1)), what="window 1 LSE")
    for W, Nq in ((5, N), (5, 3), (9, 1)):
        pos = N - Nq + np.arange(Nq, dtype=np.int64)
        qq = q[:, :, N - Nq:]
        o, lse = orc.fwd(qq, k, v, True, s, qpos=pos, window=W)
        j = np.arange(N)[None, :]
        band = (j <= pos[:, None]) & (j > pos[:, None] - W)
        mask = torch.tensor(band)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(qq), torch.tensor(k).repeat_interleave(G, 1), torch.tensor(v).repeat_interleave(G, 1),
            attn_mask=mask, scale=s)
        _close(o, ref.numpy(), tol=1e-12, what=f"window {W} Nq {Nq} O vs SDPA")
        sc = (torch.tensor(qq) @ torch.tensor(k).repeat_interleave(G, 1).transpose(-1, -2) * s).masked_fill(
            ~mask, float("-inf"))
        _close(lse, torch.logsumexp(sc, -1).numpy(), tol=1e-12, what=f"window {W} Nq {Nq} LSE")
        P = orc.probs(qq, k, True, s, qpos=pos, window=W)
        assert np.all(P[..., ~band] == 0.0), "probability outside the window"
        _close(P.sum(-1), np.ones(P.shape[:-1]), what="window rows sum to 1")


def pin_sliding_window_backward(orc):
    """Gradients under the sliding-window mask: torch's fp64 autograd through SDPA
    with the band mask written out, central finite differences on a tiny case,
    W >= N equal to plain causal, and the sampled backward equal to the full one."""
    import torch
    B, Hq, Hkv, N, d = 1, 4, 2, 19, 5
    G = Hq // Hkv
    q, do = _rand((B, Hq, N, d), 210), _rand((B, Hq, N, d), 213)
    k, v = _rand((B, Hkv, N, d), 211), _rand((B, Hkv, N, d), 212)
    s = 0.6
    for W in (1, 4, 7):
        j = np.arange(N)
        band = torch.tensor((j[None, :] <= j[:, None]) & (j[None, :] > j[:, None] - W))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), attn_mask=band, scale=s)
        (to * torch.tensor(do)).sum().backward()
        g = orc.bwd(q, k, v, do, True, s, window=W)
        _close(g["o"], to.detach().numpy(), tol=1e-12, what=f"window {W} O")
        _close(g["dq"], tq.grad.numpy(), tol=1e-11, what=f"window {W} dQ")
        _close(g["dk"], tk.grad.numpy(), tol=1e-11, what=f"window {W} dK")
        _close(g["dv"], tv.grad.numpy(), tol=1e-11, what=f"window {W} dV")
        rows, keys = np.array([0, 6, 18], dtype=np.int64), np.array([17, 2], dtype=np.int64)
        sm = orc.bwd_sampled(q, k, v, do, True, s, rows, keys, window=W)
        _close(sm["dq"], g["dq"][:, :, rows], what=f"window {W} sampled dQ")
        _close(sm["dk"], g["dk"][:, :, keys], what=f"window {W} sampled dK")
    gw, gc = orc.bwd(q, k, v, do, True, s, window=N), orc.bwd(q, k, v, do, True, s)
    for key in ("dq", "dk", "dv"):
        _close(gw[key], gc[key], what=f"window N {key}")
    # finite differences of sum(dO * O) in one K and one V entry, W = 3
    h, W = 1e-6, 3
    g = orc.bwd(q, k, v, do, True, s, window=W)
    for name, arr, idx in (("k", k, (0, 1, 9, 2)), ("v", v, (0, 0, 4, 3)), ("q", q, (0, 3, 12, 1))):
        xp, xm = arr.copy(), arr.copy()
        xp[idx] += h
        xm[idx] -= h
        args_p = {"q": q, "k": k, "v": v}
        args_m = dict(args_p)
        args_p[name], args_m[name] = xp, xm
        fp = float((orc.fwd(args_p["q"], args_p["k"], args_p["v"], True, s, window=W)[0] * do).sum())
        fm = float((orc.fwd(args_m["q"], args_m["k"], args_m["v"], True, s, window=W)[0] * do).sum())
        _close((fp - fm) / (2 * h), g["d" + name][idx], tol=1e-7, what=f"window FD d{name}")



# ---- 8-bit inputs: OCP E4M3 codes with fp32 block scales ----
# The pages credit FlashAttention-3 with an FP8 forward using block scaling
# (mlapandio "Generations"; wishwiki "FlashAttention", "Evolution:
# FlashAttention-2 and -3") and fix no format. These pins hold the oracle's E4M3 codec to
# torch's float8_e4m3fn (an independent library implementation of the same OCP
# format), to the format's closed forms, and its block quantiser to a
# brute-force numpy float32 recomputation.

def _torch_e4m3_values(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8).copy()).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3_codes(x32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32).copy()).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_codes(orc):
    """Every code decodes as the library does; closed forms of the format."""
    c = np.arange(256, dtype=np.uint8)
    v = orc.e4m3_decode(c)
    assert np.array_equal(v, _torch_e4m3_values(c), equal_nan=True), "E4M3 decode differs from float8_e4m3fn"
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0, "largest finite E4M3 magnitude is 1.75 * 2^8"
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9, "subnormals are m * 2^-9"
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x40] == 2.0, "normals are (1 + m/8) 2^(e-7)"
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isfinite(v).sum() == 254, "one NaN code per sign"
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes increase with their value"
    assert np.array_equal(v[0x80:0xFF], -pos) and math.copysign(1.0, v[0x80]) < 0, "sign bit mirrors"
    fin = c[np.isfinite(v)]
    assert np.array_equal(orc.e4m3_encode(v[np.isfinite(v)].astype(np.float32)), fin), "encode(decode(c)) != c"


def pin_e4m3_rounding(orc):
    """Nearest value with ties to even, saturation at 448, NaN to the NaN code."""
    v = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)           # 5 significant bits: exact in float32
    assert np.array_equal(mid.astype(np.float64), (v[:-1] + v[1:]) / 2)
    got = orc.e4m3_encode(mid)
    lo = np.arange(0x7E, dtype=np.uint8)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, want), "a tie does not go to the even code"
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    assert np.array_equal(orc.e4m3_encode(up), lo + 1) and np.array_equal(orc.e4m3_encode(dn), lo), "not nearest"
    rng = _rng(41)
    x = np.concatenate([rng.standard_normal(20000) * 60, rng.standard_normal(20000) * 2.0 ** -7,
                        rng.uniform(-464, 464, 20000)]).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(x), _torch_e4m3_codes(x)), "encode differs from float8_e4m3fn"
    big = np.array([448, 464, 480, 500, 1e6, 3e38, np.inf], dtype=np.float32)
    assert np.all(orc.e4m3_encode(big) == 0x7E) and np.all(orc.e4m3_encode(-big) == 0xFE), "saturation"
    assert orc.e4m3_encode(np.array([np.nan], dtype=np.float32))[0] & 0x7F == 0x7F, "NaN code"
    assert orc.e4m3_encode(np.array([-0.0], dtype=np.float32))[0] == 0x80, "negative zero keeps its sign"


def pin_e4m3_block_quantiser(orc):
    """Blocks of rows, one scale each, against a numpy float32 recomputation."""
    rng = _rng(43)
    B, H, N, d, R = 2, 3, 300, 16, 128                        # ragged last block of 44 rows
    x = (rng.standard_normal((B, H, N, d)) * rng.uniform(0.01, 30, (B, H, 1, 1))).astype(np.float32)
    x[1, 2, 128:256] = 0.0                                     # an all-zero block
    x[0, 1, 5, 3] = np.float32(1e4)                            # one outlier sets its block's scale
    codes, scales = orc.quantize_e4m3(x, R)
    nb = -(-N // R)
    assert scales.shape == (B, H, nb)
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                blk = x[b, h, j * R:(j + 1) * R]
                amax = np.float32(np.abs(blk).max())
                if amax == 0:
                    inv, sc = np.float32(1), np.float32(1)
                else:
                    inv, sc = np.float32(448) / amax, amax / np.float32(448)
                assert scales[b, h, j] == sc, f"scale of block {b, h, j}"
                want = _torch_e4m3_codes((blk * inv).astype(np.float32))
                assert np.array_equal(codes[b, h, j * R:(j + 1) * R], want), f"codes of block {b, h, j}"
                if amax > 0:
                    top = np.abs(blk) == amax
                    assert np.all(codes[b, h, j * R:(j + 1) * R][top] & 0x7F == 0x7E), "amax maps to 448"
    deq = orc.dequantize_e4m3(codes, scales, R)
    assert np.array_equal(deq, _torch_e4m3_values(codes) * np.repeat(scales.astype(np.float64), R, axis=2)[
        :, :, :N, None]), "dequantisation"
    s_full = np.repeat(scales.astype(np.float64), R, axis=2)[:, :, :N, None]
    y = np.abs(x.astype(np.float64)) / s_full
    normal = y >= 2.0 ** -6
    err = np.abs(deq - x)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6)), "relative error of a normal code"
    assert np.all(err[~normal] <= 2.0 ** -10 * s_full.repeat(d, axis=3)[~normal] * (1 + 1e-6)), "subnormal error"


def pin_e4m3_tiny_runs(orc):
    """Runs far below the normal range. A power-of-two factor on a run commutes
    with the quantiser: the run times 2^-k gets the codes of the run itself and
    its scale times 2^-k, as long as that scale stays a normal fp32 number. For
    a run whose max is below 2^-64 (where 448 / amax would overflow fp32), the
    codes still equal those of the run times 2^80, never hold a NaN pattern,
    map the run's max to 448, and dequantise within 2^-4 relative."""
    rng = _rng(53)
    R, d = 16, 8
    base = (rng.standard_normal((1, 4, 2 * R, d)) * 3).astype(np.float32)
    base[0, 3, R:] = 0.0
    base[0, 3, R, 0] = np.float32(0.75)                 # a run holding one nonzero value
    c0, s0 = orc.quantize_e4m3(base, R)
    for k in (20, 60, 100):                             # 2^-100 * 448 / 2^8.6 is still a normal scale
        ck, sk = orc.quantize_e4m3((base * np.float32(2.0 ** -k)).astype(np.float32), R)
        assert np.array_equal(ck, c0), f"codes of the run times 2^-{k}"
        assert np.array_equal(sk.astype(np.float64), s0.astype(np.float64) * 2.0 ** -k), f"scale times 2^-{k}"
    # the advisor's case: a run of [1e-37, 5e-38, 0, ...]
    x = np.zeros((1, 1, R, d), dtype=np.float32)
    x[0, 0, 0, 0], x[0, 0, 0, 1] = np.float32(1e-37), np.float32(5e-38)
    c, sc = orc.quantize_e4m3(x, R)
    c80, _ = orc.quantize_e4m3((x * np.float32(2.0 ** 80)).astype(np.float32), R)
    assert np.array_equal(c, c80), "tiny run: codes of the run times 2^80"
    assert c[0, 0, 0, 0] == 0x7E and np.all(c.reshape(-1)[2:] == 0), "max to 448, zeros to 0"
    assert not np.any((c & 0x7F) == 0x7F), "no NaN code"
    deq = orc.dequantize_e4m3(c, sc, R)
    nz = x != 0
    assert np.all(np.abs(deq[nz] - x[nz]) <= 2.0 ** -4 * np.abs(x[nz])), "tiny run dequantises within 2^-4"
    # bf16 subnormal inputs: the smallest bf16 magnitudes, scale an fp32 subnormal
    y = np.zeros((1, 1, R, d), dtype=np.float32)
    y[0, 0, 0, :3] = np.array([2.0 ** -133, -3 * 2.0 ** -133, 2.0 ** -127], dtype=np.float32)
    c, sc = orc.quantize_e4m3(y, R)
    assert 0 < sc[0, 0, 0] < 2.0 ** -126, "the scale is an fp32 subnormal here"
    assert c[0, 0, 0, 2] == 0x7E and not np.any((c & 0x7F) == 0x7F)
    deq = orc.dequantize_e4m3(c, sc, R)
    nz = y != 0
    assert np.all(np.abs(deq[nz] - y[nz]) <= 2.0 ** -4 * np.abs(y[nz])), "subnormal-scale run within 2^-4"


def pin_e4m3_forward(orc):
    """The forward on 8-bit inputs is the definition on the dequantised values:
    constant V codes give O = that value exactly; zero Q codes give the causal
    prefix mean of the dequantised V with LSE = ln(i + 1)."""
    rng = _rng(47)
    B, Hq, Hkv, N, d, R = 1, 4, 2, 200, 32, 64
    xq = rng.standard_normal((B, Hq, N, d)).astype(np.float32)
    xk = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    q8, qs = orc.quantize_e4m3(xq, R)
    k8, ks = orc.quantize_e4m3(xk, R)
    v8 = np.full((B, Hkv, N, d), 0x3B, dtype=np.uint8)      # 1.375
    vs = np.full((B, Hkv, -(-N // R)), 0.5, dtype=np.float32)
    o, lse = orc.fwd_e4m3(q8, k8, v8, qs, ks, vs, R, causal=True, scale=d ** -0.5)
    assert np.max(np.abs(o - 0.6875)) <= TOL, "constant V"
    xv = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v8, vs = orc.quantize_e4m3(xv, R)
    o, lse = orc.fwd_e4m3(np.zeros_like(q8), k8, v8, qs, ks, vs, R, causal=True, scale=d ** -0.5)
    vd = _torch_e4m3_values(v8) * np.repeat(vs.astype(np.float64), R, axis=2)[:, :, :N, None]
    cnt = np.arange(1, N + 1, dtype=np.float64)
    prefix = np.cumsum(vd, axis=2) / cnt[None, None, :, None]
    assert np.max(np.abs(o - np.repeat(prefix, Hq // Hkv, axis=1))) <= 1e-12, "zero Q: prefix mean"
    assert np.max(np.abs(lse - np.log(cnt))) <= 1e-12, "zero Q: LSE = ln(i + 1)"


PINS = [
    pin_one_token,
    pin_two_tokens,
    pin_three_four_tokens_mp,
    pin_constant_v,
    pin_causal_row_zero,
    pin_uniform_scale_zero,
    pin_probability_rows,
    pin_key_translation,
    pin_gqa_equals_repeated_mha,
    pin_head_permutation,
    pin_last_row_and_positions,
    pin_gradient_sums,
    pin_large_logits,
    pin_torch_sdpa,
    pin_finite_differences,
    pin_online_recurrence,
    pin_sampled_backward,
    pin_round_bf16,
    pin_stored_o_mode,
    pin_decode_positions,
    pin_split_merge,
    pin_sliding_window,
    pin_sliding_window_backward,
    pin_e4m3_codes,
    pin_e4m3_rounding,
    pin_e4m3_block_quantiser,
    pin_e4m3_tiny_runs,
    pin_e4m3_forward,
]
