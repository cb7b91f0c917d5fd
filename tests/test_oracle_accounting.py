"""Pins of the KV-byte accounting (oracle.accounting) against values fixed outside it.

1. Worked per-token figures of the store formats at the named workloads (the
   byte arithmetic of the store format: base rows at 2 bytes (bf16) or 1 + 2/32
   (int8 codes plus one float16 scale per 32), int4 residual rows at 1/2 + 2/32,
   a 4-byte slot-map entry per (loop k >= 2, token); column sets excluded, since
   they are amortized over the prompt).  The figures are in
   tests/golden/kv_bytes_worked.json; each was worked by hand from those
   per-element sizes, not from the code under test.
2. The byte size of the oracle's own store arrays after a small prefill and a
   few decode steps (codes, scales, slot-map entries and column sets actually
   written, counted from the arrays), which must equal kv_bytes exactly.
3. The dense per-loop and last-loop caches: 2 bytes per element, R*K (per loop)
   or R (last loop) KV sets (aiboss88.com tutorial, step 4).
"""
import json
import math
import os

import numpy as np
import pytest

from cross_loop_kv_amd import inputs as I
from oracle import accounting
from oracle.model import LoopedOracle
from oracle.select import n_selected

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_bytes_worked.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_per_token_bytes_equal_worked_values(case):
    """Per prompt token and per decode token, lazy store (shared block), for a
    prompt length at which rho * T is an integer (so the kept fraction is exactly
    rho), with the column sets taken out; the worked values are the exact figures
    and their round-up to a whole byte."""
    wl = I.workload(case["workload"])
    s = wl.shape
    T = case["prompt"]
    n = n_selected(case["rho"], T)
    assert n == round(case["rho"] * T), "pick T with an integral rho * T"
    E = 2 * s.n_kv_heads * s.head_dim
    dense = accounting.dense_per_loop_bytes_per_token(s)
    assert dense == case["dense_per_loop"]
    for base_bits, key in ((16, "bf16_base"), (8, "int8_base")):
        lz = I.Lazy(mode="lazy", rho=case["rho"], top_s=case["top_s"], window=8, base_bits=base_bits,
                    res_bits=4)
        # prompt tokens only
        b = accounting.kv_bytes(s, lz, 1, T, T)
        cols = s.n_shared * s.n_kv_heads * min(case["top_s"], T) * 4
        per_tok = (b["shared"] - cols) / T
        assert abs(per_tok - case[key]["prompt_token_exact"]) < 1e-6, (key, per_tok)
        assert math.ceil(per_tok - 1e-9) == case[key]["prompt_token"], (key, per_tok)
        # one decode token stores its base row and one residual row per loop k >= 2
        b1 = accounting.kv_bytes(s, lz, 1, T, T + 1)
        dec = b1["shared"] - b["shared"]
        assert dec == case[key]["decode_token"], (key, dec)
    assert E == case["E"]


SMALL = I.Shape(vocab=64, d_model=64, n_heads=4, n_kv_heads=2, head_dim=32, ffn_dim=128, ffn_act="swiglu",
                n_prelude=1, n_shared=2, n_loops=3, n_coda=1)


@pytest.mark.parametrize("base_bits,res_bits,refresh", [(8, 4, 0), (16, 8, 0), (8, 16, 0), (16, 4, 2)])
def test_kv_bytes_equal_the_oracle_store_arrays(base_bits, res_bits, refresh):
    """After a prefill of T tokens and 3 decode steps, count what the oracle's arrays
    hold for the tokens present: base codes (1 byte, int8) plus float16 scales, or
    2-byte rows for a 16-bit base; each stored residual row at res_bits per element
    (int4 codes occupy half their int8 array) plus float16 scales; one int32 slot-map
    entry per (loop k >= 2, token); the int32 column sets; and 2-byte rows for the
    prelude/coda layers.  That count must equal kv_bytes."""
    s = SMALL
    B, T, steps = 2, 40, 3
    lz = I.Lazy(mode="lazy", rho=0.3, top_s=7, window=4, base_bits=base_bits, res_bits=res_bits,
                refresh_every=refresh)
    W = I.gen_weights(s, seed=3)
    m = LoopedOracle(s, lz, W, B, T + steps)
    m.prefill(I.gen_prompt_ids(s, B, T))
    for d in I.gen_decode_ids(s, B, steps):
        m.decode(d)
    t = T + steps
    R, K = s.n_shared, s.n_loops
    shared = 0
    for r in range(R):
        for kv in range(2):
            if base_bits == 16:
                shared += m.base[r][kv][:, :, :t, :].size * 2
            else:
                codes, sc = m.base[r][kv]
                shared += codes[:, :, :t, :].nbytes + sc[:, :, :t, :].nbytes
    for k in range(2, K + 1):
        used = [np.nonzero(m.slot[k - 1, b, :t] >= 0)[0].size for b in range(B)]
        for r in range(R):
            for kv in range(2):
                st = m.res[(k, r, kv)]
                for b in range(B):
                    if res_bits == 16:
                        shared += st[b][:, :used[b], :].size * 2
                    else:
                        codes, sc = st
                        cb = codes[b][:, :used[b], :].nbytes
                        shared += (cb // 2 if res_bits == 4 else cb) + sc[b][:, :used[b], :].nbytes
        shared += m.slot[k - 1][:, :t].nbytes
    shared += sum(np.asarray(c, np.int32).nbytes for r in range(R) for b in range(B) for c in m.S[r][b])
    dense = sum(x[:, :, :t, :].size * 2 for x in m.dense_k + m.dense_v)
    got = accounting.kv_bytes(s, lz, B, T, t)
    assert got["shared"] == shared
    assert got["total"] == shared + dense


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_dense_cache_bytes_equal_the_oracle_arrays(mode):
    s = SMALL
    B, T, steps = 2, 20, 2
    W = I.gen_weights(s, seed=4)
    m = LoopedOracle(s, I.Lazy(mode=mode), W, B, T + steps)
    m.prefill(I.gen_prompt_ids(s, B, T))
    for d in I.gen_decode_ids(s, B, steps):
        m.decode(d)
    t = T + steps
    sets = [x for k in range(s.n_loops) for x in m.loop_k[k] + m.loop_v[k]] if mode == "per_loop" \
        else m.last_k + m.last_v
    shared = sum(x[:, :, :t, :].size * 2 for x in sets)
    got = accounting.kv_bytes(s, I.Lazy(mode=mode), B, T, t)
    assert got["shared"] == shared
    # per token: 2 bytes x E elements x R*K (per loop) or R (last loop) KV sets
    E = 2 * s.n_kv_heads * s.head_dim
    assert got["shared"] == B * t * 2 * E * s.n_shared * (s.n_loops if mode == "per_loop" else 1)
