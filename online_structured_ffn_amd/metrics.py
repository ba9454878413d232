"""Algorithmic HBM bytes and flops of each piece of the pruned gated-MLP path.

"Algorithmic" means what the method itself must move: every weight row it uses
read once, its inputs read once, its outputs written once.  Implementation
overheads (partial sums of split reductions, re-reads) are not counted, so a
kernel's achieved bandwidth on these bytes can only be lower than its raw
traffic rate.  e = element bytes (2 for bf16, 4 for fp32).
"""
from __future__ import annotations


def gateup_bytes(d: int, n_A: int, n_C: int, batch: int, e: int) -> int:
    """Gate/up GEMV over the rows R u C: both weight rows, x, the index list,
    z written, the candidate scores written."""
    return 2 * n_A * d * e + batch * d * e + 4 * n_A + 4 * batch * n_A + 4 * n_C


def select_bytes(n_C: int, k: int) -> int:
    return 4 * n_C + 4 * k * 2 + 4 * k


def down_bytes(d: int, n_live: int, batch: int, e: int, k: int = 0) -> int:
    """Down-projection over the live rows of W_downT: the rows, z of those rows,
    the index lists, y written."""
    return n_live * d * e + 4 * batch * n_live + 4 * (n_live + k) + 4 * batch * d


def decode_bytes(d: int, n_R: int, n_C: int, k: int, batch: int, e: int) -> int:
    """One pruned decode layer-step (the three stages)."""
    n_A = n_R + n_C
    n_live = n_R + k
    return gateup_bytes(d, n_A, n_C, batch, e) + select_bytes(n_C, k) + down_bytes(d, n_live, batch, e, k)


def dense_decode_bytes(d: int, d_ff: int, batch: int, e: int) -> int:
    return 3 * d_ff * d * e + batch * d * e + 4 * batch * d + 8 * batch * d_ff


def decode_flops(d: int, n_A: int, n_live: int, batch: int) -> int:
    return 2 * batch * d * (2 * n_A + n_live)


def importance_bytes(n_tokens: int, d: int, d_ff: int, e: int) -> int:
    """Prompt X once, W_up once, I written."""
    return n_tokens * d * e + d_ff * d * e + 4 * d_ff


def partition_bytes(n_tokens: int, d: int, d_ff: int, e: int) -> int:
    """Importance plus the select (I read, the three lists written)."""
    return importance_bytes(n_tokens, d, d_ff, e) + 4 * d_ff + 4 * d_ff


def prefill_ffn_flops(n_tokens: int, d: int, d_ff: int) -> int:
    return 6 * n_tokens * d * d_ff


# Launch shape of the batch-1 step with candidates (mirrors the library: one
# 512-thread workgroup runs the top-k, the others take static shares of C and
# R, one per 8 rows up to 255 of them, one workgroup per CU; a second launch
# adds their partial sums).
LINKED_THREADS = 512
LINKED_MAX_WORKERS = 255


def linked_workers(n_R: int, n_C: int) -> int:
    return max(1, min((n_R + n_C + 7) // 8, LINKED_MAX_WORKERS))


def linked_symbol(d: int, e: int) -> str:
    """The kernel symbol of the batch-1 step for row width d and element
    bytes e (its template takes the 16-byte vectors per thread: 1, 2 or 4)."""
    nv = -(-d // (LINKED_THREADS * (16 // e)))
    tname = "pop::bf16s" if e == 2 else "float"
    return f"pop::k_pop_linked<{tname}, {1 if nv <= 1 else 2 if nv <= 2 else 4}, false, false>"


def linked_bytes(d: int, n_R: int, n_C: int, k: int, e: int) -> int:
    """The single-launch batch-1 step (k_pop_linked): everything
    :func:`decode_bytes` counts except y's write, which the launch after it
    does (the per-workgroup partial sums are not counted)."""
    return decode_bytes(d, n_R, n_C, k, 1, e) - 4 * d


def linked_finish_bytes(d: int, n_R: int, n_C: int) -> int:
    """The launch after it (k_pop_finish): the per-workgroup partial sums
    read, y written."""
    return 4 * d * linked_workers(n_R, n_C) + 4 * d


def moe_decode_bytes(d: int, n_R: int, n_C: int, k: int, experts_reached: float, tokens: int, e: int) -> float:
    """One MoE decode layer-step: every reached expert's gate and up rows over
    R u C and W_downT rows over R u S, the tokens' inputs (once per routed
    pair) and outputs."""
    per_expert = 2 * (n_R + n_C) * d * e + (n_R + k) * d * e
    return experts_reached * per_expert + 2 * tokens * d * e + 4 * tokens * d


def attention_decode_bytes(d: int, n_heads: int, n_kv_heads: int, head_dim: int, n_keys: int, batch: int,
                           e: int) -> dict:
    """The attention half of one decode layer-step, per kernel: the q|k|v and
    output projections read their weights and inputs once and write their
    outputs (the partial sums of split reductions not counted); attention reads
    the n_keys cached keys and values of every sequence once; RMSNorm reads x
    and writes its output."""
    nqkv = (n_heads + 2 * n_kv_heads) * head_dim
    hd_all = n_heads * head_dim
    return {
        "qkv": d * nqkv * e + batch * d * e + batch * nqkv * 4,
        "attn": 2 * batch * n_kv_heads * n_keys * head_dim * e + batch * hd_all * 4 + batch * hd_all * e,
        "o": hd_all * d * e + batch * hd_all * e + batch * d * 4,
        "norms": 2 * (batch * d * 4 + batch * d * e),
    }
