"""Seeded synthetic inputs for exact-attention runs.

This module is shared by the fp64 oracle side and the HIP side. It holds no
attention arithmetic: it only draws random numbers, rounds them to the bf16 I/O
format, and names the workload shapes.

Workload shapes follow the shape families the FlashAttention pages use (the
2048-token sequence of the techtrendtracker post, "The Standard Attention
Bottleneck"; the 8-head, d = 128, long-prefill example of the mlapandio
"FlashAttention: IO-aware exact attention" page, "120K-token prefill" diagram).
No dataset is used; every tensor is N(0, 1) from a counter-based seed.

Seeding: tensor t of workload c is drawn from numpy's PCG64 seeded with
``SeedSequence([2026, c, t])``. Tensor ids: Q = 0, K = 1, V = 2, dO = 3, spike
positions = 4, row sample = 5, per-sequence cache lengths = 6. Each tensor has its own stream, so regenerating
one tensor never changes another.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO, TENSOR_SPIKE, TENSOR_ROWS, TENSOR_LENS = range(7)
ROOT_SEED = 2026


# ---------------------------------------------------------------- bf16 packing
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with round-to-nearest-even; return the
    16-bit patterns as uint16. NaN stays NaN (quiet bit set)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------- generators
def rng_for(cfg_id: int, tensor_id: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cfg_id, tensor_id, *extra])))


def normal_f32(shape, cfg_id: int, tensor_id: int, *extra: int) -> np.ndarray:
    """N(0, 1) float32 samples from the stream (cfg_id, tensor_id, *extra)."""
    return rng_for(cfg_id, tensor_id, *extra).standard_normal(size=shape, dtype=np.float32)


def normal_bf16(shape, cfg_id: int, tensor_id: int, *extra: int) -> np.ndarray:
    """N(0, 1) samples rounded to bf16; returned as uint16 bit patterns."""
    return bf16_round_bits(normal_f32(shape, cfg_id, tensor_id, *extra))


def spike_positions(B: int, Hkv: int, N: int, frac: float, cfg_id: int) -> np.ndarray:
    """For each (b, kv-head) pick round(frac * N) distinct key positions
    (seeded, without replacement). Returns int64 [B, Hkv, count], each row sorted."""
    count = int(round(frac * N))
    rng = rng_for(cfg_id, TENSOR_SPIKE)
    out = np.empty((B, Hkv, count), dtype=np.int64)
    for b in range(B):
        for h in range(Hkv):
            out[b, h] = np.sort(rng.choice(N, size=count, replace=False))
    return out


def sample_rows(N: int, count: int, cfg_id: int) -> np.ndarray:
    """`count` distinct query rows in [0, N), always containing 0 and N - 1,
    sorted ascending (int64)."""
    count = min(count, N)
    if count >= N:
        return np.arange(N, dtype=np.int64)
    rng = rng_for(cfg_id, TENSOR_ROWS)
    inner = rng.choice(np.arange(1, N - 1), size=max(count - 2, 0), replace=False) if N > 2 else np.array([], np.int64)
    rows = np.unique(np.concatenate([[0, N - 1], inner]).astype(np.int64))
    return rows


# ---------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    backward: bool
    fp32_source: bool = False      # inputs drawn in fp32, then rounded to bf16
    spike_frac: float = 0.0        # fraction of key positions whose K row is scaled
    spike_factor: float = 1.0
    oracle_groups: int | None = None   # (b, kv-head) groups the oracle checks; None = all
    oracle_rows: int | None = None     # query rows the oracle checks per head; None = all

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        """softmax scale 1/sqrt(d), rounded to float32 (the value passed to the kernels)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def describe(self) -> dict:
        return dict(workload=self.name, B=self.B, Hq=self.Hq, Hkv=self.Hkv, N=self.N, d=self.d,
                    causal=self.causal, passes="fwd+bwd" if self.backward else "fwd")


WORKLOADS = {
    "tiny": Workload(0, "tiny", 1, 1, 1, 256, 64, False, False, fp32_source=True),
    "mha2k": Workload(1, "mha2k", 4, 16, 16, 2048, 64, True, True),
    "spiky8k": Workload(2, "spiky8k", 1, 32, 32, 8192, 128, True, True, spike_frac=0.05, spike_factor=4.0),
    "gqa16k": Workload(3, "gqa16k", 2, 32, 8, 16384, 128, True, True, oracle_groups=2),
    "long128k": Workload(4, "long128k", 1, 8, 8, 131072, 128, True, False, oracle_rows=256),
    # gqa16k's shape and FLOP count with d = 64 (twice the heads), forward and backward
    "gqa16k_d64": Workload(13, "gqa16k_d64", 2, 64, 16, 16384, 64, True, True, oracle_rows=128),
    # gqa16k's shape and FLOP count with d = 256 (half the query heads), forward only
    "gqa16k_d256": Workload(11, "gqa16k_d256", 2, 16, 4, 16384, 256, True, True, oracle_rows=128),
}


def make_inputs(w: Workload, with_grad: bool | None = None) -> dict:
    """Generate the workload's tensors as bf16 bit patterns (uint16, [B, H, N, d]).

    Keys: 'q', 'k', 'v', and 'do' when a backward pass is wanted. For fp32-source
    workloads the unrounded float32 draws are also returned under 'q32', 'k32', 'v32'.
    """
    if with_grad is None:
        with_grad = w.backward
    qs, kvs = (w.B, w.Hq, w.N, w.d), (w.B, w.Hkv, w.N, w.d)
    out = {}
    if w.fp32_source:
        q32, k32, v32 = (normal_f32(qs, w.cfg_id, TENSOR_Q), normal_f32(kvs, w.cfg_id, TENSOR_K),
                         normal_f32(kvs, w.cfg_id, TENSOR_V))
        out.update(q32=q32, k32=k32, v32=v32)
        out.update(q=bf16_round_bits(q32), k=bf16_round_bits(k32), v=bf16_round_bits(v32))
    else:
        out["q"] = normal_bf16(qs, w.cfg_id, TENSOR_Q)
        out["k"] = normal_bf16(kvs, w.cfg_id, TENSOR_K)
        out["v"] = normal_bf16(kvs, w.cfg_id, TENSOR_V)
    if w.spike_frac > 0:
        pos = spike_positions(w.B, w.Hkv, w.N, w.spike_frac, w.cfg_id)
        k = bf16_bits_to_f32(out["k"])
        for b in range(w.B):
            for h in range(w.Hkv):
                k[b, h, pos[b, h], :] *= np.float32(w.spike_factor)
        # a power-of-two factor keeps every value exactly representable in bf16
        out["k"] = bf16_round_bits(k)
        out["spike_positions"] = pos
    if with_grad:
        out["do"] = normal_bf16(qs, w.cfg_id, TENSOR_DO)
    return out


def make_case(B: int, Hq: int, Hkv: int, N: int, d: int, seed: int, with_grad: bool = True,
              dist_scale: float = 1.0) -> dict:
    """Small seeded case for parity tests (cfg_id space 1000 + seed keeps these
    streams apart from the named workloads)."""
    cid = 1000 + seed
    qs, kvs = (B, Hq, N, d), (B, Hkv, N, d)
    f = np.float32(dist_scale)
    out = {
        "q": bf16_round_bits(normal_f32(qs, cid, TENSOR_Q) * f),
        "k": bf16_round_bits(normal_f32(kvs, cid, TENSOR_K) * f),
        "v": bf16_round_bits(normal_f32(kvs, cid, TENSOR_V)),
    }
    if with_grad:
        out["do"] = bf16_round_bits(normal_f32(qs, cid, TENSOR_DO))
    return out


# ---------------------------------------------------------------- decode workloads
@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Nq new query rows per head against a cache of Nk keys and values (the
    decode step of generation). The cache shapes are those of the long-sequence
    workloads above; the queries are the sequence's last Nq tokens."""
    cfg_id: int
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool = True
    ragged: bool = False     # per-sequence cache lengths, uniform in [Nk / 16, Nk]

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def describe(self) -> dict:
        return dict(workload=self.name, B=self.B, Hq=self.Hq, Hkv=self.Hkv, Nq=self.Nq, Nk=self.Nk, d=self.d,
                    causal=self.causal, ragged=self.ragged, passes="decode")


def decode_seqlens(w: DecodeWorkload) -> np.ndarray | None:
    """Cache rows in use per batch entry (int32 [B]) for a ragged decode workload, else None."""
    if not w.ragged:
        return None
    return rng_for(w.cfg_id, TENSOR_LENS).integers(w.Nk // 16, w.Nk, size=w.B, endpoint=True).astype(np.int32)


DECODE_WORKLOADS = {
    "decode_gqa16k": DecodeWorkload(5, "decode_gqa16k", 2, 32, 8, 1, 16384, 128),
    "decode_gqa16k_q16": DecodeWorkload(6, "decode_gqa16k_q16", 2, 32, 8, 16, 16384, 128),
    "decode_long128k": DecodeWorkload(7, "decode_long128k", 1, 8, 8, 1, 131072, 128),
    "decode_batch64": DecodeWorkload(8, "decode_batch64", 64, 32, 8, 1, 4096, 128),
    "decode_ragged64": DecodeWorkload(9, "decode_ragged64", 64, 32, 8, 1, 8192, 128, ragged=True),
    # decode_gqa16k's cache bytes at d = 256 (half the heads)
    "decode_gqa16k_d256": DecodeWorkload(12, "decode_gqa16k_d256", 2, 16, 4, 1, 16384, 256),
}


def make_decode_inputs(w: DecodeWorkload) -> dict:
    """q [B, Hq, Nq, d], k and v [B, Hkv, Nk, d], N(0, 1) rounded to bf16 (uint16 bits)."""
    return {
        "q": normal_bf16((w.B, w.Hq, w.Nq, w.d), w.cfg_id, TENSOR_Q),
        "k": normal_bf16((w.B, w.Hkv, w.Nk, w.d), w.cfg_id, TENSOR_K),
        "v": normal_bf16((w.B, w.Hkv, w.Nk, w.d), w.cfg_id, TENSOR_V),
    }


def make_decode_case(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int,
                     dist_scale: float = 1.0) -> dict:
    """Small seeded decode case (cfg_id space 3000 + seed)."""
    cid = 3000 + seed
    f = np.float32(dist_scale)
    return {
        "q": bf16_round_bits(normal_f32((B, Hq, Nq, d), cid, TENSOR_Q) * f),
        "k": bf16_round_bits(normal_f32((B, Hkv, Nk, d), cid, TENSOR_K) * f),
        "v": bf16_round_bits(normal_f32((B, Hkv, Nk, d), cid, TENSOR_V)),
    }


# ---------------------------------------------------------------- packed (variable-length) workloads
@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """B sequences of different lengths packed head by head: q [Hq, total, d],
    k/v [Hkv, total, d]; lengths uniform in [min_len, max_len] (seeded)."""
    cfg_id: int
    name: str
    B: int
    Hq: int
    Hkv: int
    min_len: int
    max_len: int
    d: int
    causal: bool = True

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def lengths(self) -> np.ndarray:
        return rng_for(self.cfg_id, TENSOR_LENS).integers(self.min_len, self.max_len, size=self.B,
                                                          endpoint=True).astype(np.int64)

    def describe(self) -> dict:
        return dict(workload=self.name, B=self.B, Hq=self.Hq, Hkv=self.Hkv, min_len=self.min_len,
                    max_len=self.max_len, d=self.d, causal=self.causal, passes="fwd (packed sequences)")


VARLEN_WORKLOADS = {
    # a prefill batch of 16 prompts of 512 .. 16384 tokens, with the GQA heads of the gqa16k workload
    "varlen_mix": VarlenWorkload(10, "varlen_mix", 16, 32, 8, 512, 16384, 128),
    # the same sequences and data without the causal mask (an encoder's packed batch)
    "varlen_mix_noncausal": VarlenWorkload(10, "varlen_mix_noncausal", 16, 32, 8, 512, 16384, 128, causal=False),
}


def cu_seqlens(lengths) -> np.ndarray:
    """int32 [B + 1] offsets of packed sequences."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


def make_varlen_inputs(w: VarlenWorkload) -> dict:
    lens = w.lengths()
    total = int(lens.sum())
    return {
        "q": normal_bf16((w.Hq, total, w.d), w.cfg_id, TENSOR_Q),
        "k": normal_bf16((w.Hkv, total, w.d), w.cfg_id, TENSOR_K),
        "v": normal_bf16((w.Hkv, total, w.d), w.cfg_id, TENSOR_V),
        "lengths": lens,
        "cu_seqlens": cu_seqlens(lens),
    }


def make_varlen_case(lengths, Hq: int, Hkv: int, d: int, seed: int) -> dict:
    """Small packed case (cfg_id space 4000 + seed)."""
    cid = 4000 + seed
    total = int(np.sum(lengths))
    return {
        "q": normal_bf16((Hq, total, d), cid, TENSOR_Q),
        "k": normal_bf16((Hkv, total, d), cid, TENSOR_K),
        "v": normal_bf16((Hkv, total, d), cid, TENSOR_V),
        "lengths": np.asarray(lengths, np.int64),
        "cu_seqlens": cu_seqlens(lengths),
    }
