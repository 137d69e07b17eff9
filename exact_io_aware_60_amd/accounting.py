"""Byte and FLOP accounting for exact attention (host arithmetic only).

Memory: a materialised score matrix holds N^2 values per head. The tiled method
keeps only Q, K, V and O (N x d each per head) plus one fp32 logsumexp per
query row (mlapandio "FlashAttention: IO-aware exact attention", text under the
memory-hierarchy diagram and the 120K-token prefill diagram; techtrendtracker
"Flash Attention: memory-efficient transformers", "The Standard Attention
Bottleneck").

FLOPs: the forward pass does two contractions of 2*d FLOP per visible
(query, key) pair; the count used for throughput is 4*B*Hq*N^2*d, halved under
the causal mask, and the backward is counted as 2.5 times the forward.
"""
from __future__ import annotations

LSE_BYTES = 4  # one fp32 logsumexp per query row


def score_count(N: int, heads: int = 1) -> int:
    """Entries of the N x N score matrix, over `heads` heads."""
    return heads * N * N


def naive_score_bytes(N: int, heads: int = 1, bytes_per_value: int = 2) -> int:
    """Bytes of a materialised score (or probability) matrix."""
    return score_count(N, heads) * bytes_per_value


def flash_qkvo_bytes(N: int, d: int, heads: int = 1, bytes_per_value: int = 2) -> int:
    """Bytes of Q, K, V and O (N x d each) per head, over `heads` heads."""
    return heads * 4 * N * d * bytes_per_value


def flash_lse_bytes(N: int, heads: int = 1) -> int:
    """Bytes of the per-row logsumexp the forward keeps for the backward."""
    return heads * N * LSE_BYTES


def flash_total_bytes(N: int, d: int, heads: int = 1, bytes_per_value: int = 2) -> int:
    """Everything the tiled method keeps in device memory: Q, K, V, O and LSE."""
    return flash_qkvo_bytes(N, d, heads, bytes_per_value) + flash_lse_bytes(N, heads)


def fwd_flop(B: int, Hq: int, N: int, d: int, causal: bool) -> float:
    """Forward FLOP as throughput is counted: 4*B*Hq*N^2*d, halved when causal."""
    return 4.0 * B * Hq * N * N * d / (2.0 if causal else 1.0)


def bwd_flop(B: int, Hq: int, N: int, d: int, causal: bool) -> float:
    """Backward FLOP as throughput is counted: 2.5 times the forward."""
    return 2.5 * fwd_flop(B, Hq, N, d, causal)


def visible_pairs(N: int, causal: bool) -> int:
    """Exact number of (query, key) pairs the mask leaves visible in one head."""
    return N * (N + 1) // 2 if causal else N * N
