"""KV-store byte accounting (oracle; test infrastructure only).

Basis: the FlashLoop abstract notes that every extra loop caches another set
of KV states (so a dense per-loop cache grows with K) and claims a KV-memory
reduction from residual quantization; the aiboss88.com tutorial (step 4, step
5) separates the recurrent (shared-block) KV from the rest, describes
last_loop as keeping the recurrent KV at single-pass size, and asks for
weights and KV to be reported separately.

Closed forms, with E = 2 * n_kv_heads * head_dim KV elements per token per
layer and the store formats of the library (bf16 dense rows; int8 / int4 codes
with one float16 scale per group of 32):

* dense prelude/coda layers: (P + Q) * E * 2 bytes per token;
* per_loop shared block: R * K * E * 2 per token;
* last_loop shared block: R * E * 2 per token;
* lazy shared block: base R * E * b_base per token, plus per loop k >= 2 one
  residual row (R * E * b_res) per stored token (the n recomputed prompt tokens,
  all prompt tokens at a refresh loop, and every decoded token), plus a 4-byte slot-map entry
  per (loop k >= 2, token), plus the column sets (4 bytes per column per
  (shared layer, KV head, sequence)).  b(16) = 2, b(8) = 1 + 2/32,
  b(4) = 1/2 + 2/32 bytes per element.
"""
from __future__ import annotations

from .select import n_selected


def row_bytes(n_elems: int, bits: int, group: int = 32) -> int:
    """Bytes of ``n_elems`` stored values at ``bits`` (16 = plain bf16 rows)."""
    if bits == 16:
        return 2 * n_elems
    if n_elems % group:
        raise ValueError("element count must be a multiple of the group")
    return n_elems * bits // 8 + (n_elems // group) * 2


def kv_bytes(shape, lazy, batch: int, prompt: int, tokens: int) -> dict:
    """Bytes occupied after a prefill of ``prompt`` tokens grown to ``tokens``.

    Returns ``{"dense_layers", "shared", "total", "per_token_shared",
    "per_token_total"}``; per-token figures divide by batch * tokens.
    """
    E = 2 * shape.n_kv_heads * shape.head_dim
    P, R, K, Q = shape.n_prelude, shape.n_shared, shape.n_loops, shape.n_coda
    dense = (P + Q) * batch * tokens * row_bytes(E, 16)
    if lazy.mode == "per_loop":
        shared = R * K * batch * tokens * row_bytes(E, 16)
    elif lazy.mode == "last_loop":
        shared = R * batch * tokens * row_bytes(E, 16)
    elif lazy.mode == "lazy":
        g = lazy.group
        base = R * batch * tokens * row_bytes(E, lazy.base_bits, g)
        n = n_selected(lazy.rho, prompt)
        p = int(getattr(lazy, "refresh_every", 0))
        # rows stored per loop k >= 2: the recomputed prompt tokens (all of them at a
        # refresh loop) and every decoded token
        stored = sum((prompt if p > 0 and (k - 1) % p == 0 else n) + (tokens - prompt) for k in range(2, K + 1))
        res = R * batch * stored * row_bytes(E, lazy.res_bits, g)
        slot_maps = (K - 1) * batch * tokens * 4
        cols = R * batch * shape.n_kv_heads * min(lazy.top_s, prompt) * 4
        shared = base + res + slot_maps + cols
    else:
        raise ValueError(lazy.mode)
    total = dense + shared
    denom = batch * tokens
    return {"dense_layers": dense, "shared": shared, "total": total,
            "per_token_shared": shared / denom, "per_token_total": total / denom}


def dense_per_loop_bytes_per_token(shape) -> int:
    """Shared-block bytes per token of the dense per-loop bf16 cache: 2 * R * K * E."""
    return 2 * shape.n_shared * shape.n_loops * 2 * shape.n_kv_heads * shape.head_dim


def effective_depth(shape) -> int:
    """Layer applications per token: P + R * K + Q (discosf.com section 3.1)."""
    return shape.n_prelude + shape.n_shared * shape.n_loops + shape.n_coda
