"""Pins of the oracle's looped forward (CPU only).

* K = 1 with a zero loop embedding equals a standard (P+R+Q)-layer pre-norm
  Transformer built from PyTorch library routines (the FlashLoop essay on
  nxmr.cn, section 6, recommends exactly this check: loop count 1 first).
* Dense looped == the unrolled weight-tied stack with the loop embedding added
  before each repetition (discosf.com sections 3.1, 3.2, 4.1), for prefill and
  for decode (decode must equal re-running the whole sequence).
* Effective depth P + R*K + Q and its printed instances.
* Lazy with rho = 1, all columns, bits 16/16 is bit-identical to dense.
* last_loop prefill is bit-identical to per_loop prefill; at K = 1 decode too.
* RoPE, attention with explicit column sets, column mass.
"""
import copy

import numpy as np
import pytest
import torch

from cross_loop_kv_amd import inputs as I
from oracle import accounting
from oracle.model import LoopedOracle, apply_rope, attend, rope_cos_sin, sparse_cols
from tests import torch_ref


def small_shape(**kw):
    s = I.Shape(vocab=300, d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, ffn_dim=192,
                ffn_act="swiglu", n_prelude=1, n_shared=2, n_loops=3, n_coda=1)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def tiny_shape(**kw):
    s = I.workload("tiny_1p2x2c1_t32").shape
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def max_abs_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def run_oracle(shape, lazy, W, ids, dec):
    B, T = ids.shape
    m = LoopedOracle(shape, lazy, W, B, T + len(dec))
    out = m.prefill(ids)
    depth_prefill = m.depth
    outs = [m.decode(d) for d in dec]
    return m, out, np.stack(outs, 0) if outs else None, depth_prefill


@pytest.mark.parametrize("mk", [tiny_shape, small_shape])
def test_k1_equals_standard_transformer(mk):
    s = mk(n_loops=1)
    W = I.gen_weights(s, seed=3)
    W["loop_emb"][:] = 0
    ids = I.gen_prompt_ids(s, 2, 24, seed=4)
    dec = I.gen_decode_ids(s, 2, 3, seed=5)
    m, out, dout, _ = run_oracle(s, I.Lazy(mode="per_loop"), W, ids, dec)
    for b in range(2):
        full = np.concatenate([ids[b], dec[:, b]])
        ref = torch_ref.unrolled_forward(W, s, full, loops=1, loop_emb=False).numpy()
        assert max_abs_rel(out[b], ref[:24]) < 2e-5
        assert max_abs_rel(dout[:, b], ref[24:]) < 2e-5


@pytest.mark.parametrize("mk,K", [(tiny_shape, 2), (small_shape, 3)])
def test_dense_looped_equals_unrolled_stack(mk, K):
    s = mk(n_loops=K)
    W = I.gen_weights(s, seed=6)
    W["loop_emb"] *= np.float32(50.0)   # make the loop embedding matter
    ids = I.gen_prompt_ids(s, 2, 20, seed=7)
    dec = I.gen_decode_ids(s, 2, 3, seed=8)
    m, out, dout, depth = run_oracle(s, I.Lazy(mode="per_loop"), W, ids, dec)
    assert depth == accounting.effective_depth(s) == s.n_prelude + s.n_shared * K + s.n_coda
    assert m.depth == depth          # a decode token runs the same stack
    for b in range(2):
        full = np.concatenate([ids[b], dec[:, b]])
        ref = torch_ref.unrolled_forward(W, s, full).numpy()
        assert max_abs_rel(out[b], ref[:20]) < 2e-5
        assert max_abs_rel(dout[:, b], ref[20:]) < 2e-5
    # dropping the loop embedding must change the result (the term is live)
    ref0 = torch_ref.unrolled_forward(W, s, ids[0], loop_emb=False).numpy()
    assert max_abs_rel(out[0], ref0) > 1e-3


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_input_reinjection_equals_unrolled_stack(mode):
    """The re-injection variant (aiboss88.com tutorial, step 3: the input representation
    passed into every loop) against an independently written float64 torch stack that
    adds the prelude output back before loops 2..K; it must differ from no re-injection."""
    s = small_shape(n_loops=3, input_reinject=True)
    W = I.gen_weights(s, seed=13)
    ids = I.gen_prompt_ids(s, 2, 20, seed=14)
    dec = I.gen_decode_ids(s, 2, 3, seed=15)
    _, out, dout, depth = run_oracle(s, I.Lazy(mode=mode), W, ids, dec)
    assert depth == accounting.effective_depth(s)
    for b in range(2):
        full = np.concatenate([ids[b], dec[:, b]])
        ref = torch_ref.unrolled_forward(W, s, full, reinject=True).numpy()
        assert max_abs_rel(out[b], ref[:20]) < 2e-5
        if mode == "per_loop":   # last_loop decode reads the last pass's KV only
            assert max_abs_rel(dout[:, b], ref[20:]) < 2e-5
    ref0 = torch_ref.unrolled_forward(W, s, ids[0], reinject=False).numpy()
    assert max_abs_rel(out[0], ref0) > 1e-3


def test_input_reinjection_is_inert_at_one_loop():
    """Loop 1 starts from the prelude output: with K = 1 re-injection changes nothing."""
    s = small_shape(n_loops=1)
    W = I.gen_weights(s, seed=16)
    ids = I.gen_prompt_ids(s, 1, 18, seed=17)
    dec = I.gen_decode_ids(s, 1, 2, seed=18)
    s1 = small_shape(n_loops=1, input_reinject=True)
    for lz in (I.Lazy(mode="per_loop"), I.Lazy(mode="lazy", rho=0.5, top_s=6, window=4, base_bits=8, res_bits=4)):
        _, a, ad, _ = run_oracle(s, lz, W, ids, dec)
        _, c, cd, _ = run_oracle(s1, lz, W, ids, dec)
        np.testing.assert_array_equal(a, c)
        np.testing.assert_array_equal(ad, cd)


@pytest.mark.parametrize("mode", ["per_loop", "lazy"])
@pytest.mark.parametrize("reinject", [False, True])
def test_call_loop_count_equals_model_with_that_many_loops(mode, reinject):
    """n_recurrent_loops chosen per call (aiboss88.com tutorial, step 3): running 2 of
    the 4 loops of a store laid out for 4 equals a model built with 2 loops (same
    weights, loop-embedding rows 0..1), bit for bit, prefill and decode; the depth is
    P + R*2 + Q."""
    s4 = small_shape(n_loops=4, input_reinject=reinject)
    s2 = small_shape(n_loops=2, input_reinject=reinject)
    W = I.gen_weights(s4, seed=19)
    W2 = dict(W)
    W2["loop_emb"] = W["loop_emb"][:2].copy()
    T, steps = 22, 3
    ids = I.gen_prompt_ids(s4, 2, T, seed=20)
    dec = I.gen_decode_ids(s4, 2, steps, seed=21)
    lz = (I.Lazy(mode="lazy", rho=0.4, top_s=8, window=5, base_bits=8, res_bits=4) if mode == "lazy"
          else I.Lazy(mode="per_loop"))
    m4 = LoopedOracle(s4, lz, W, 2, T + steps, n_loops=2)
    a = m4.prefill(ids)
    assert m4.depth == accounting.effective_depth(s2)
    ad = np.stack([m4.decode(d) for d in dec])
    _, c, cd, _ = run_oracle(s2, lz, W2, ids, dec)
    np.testing.assert_array_equal(a, c)
    np.testing.assert_array_equal(ad, cd)
    with pytest.raises(ValueError):
        LoopedOracle(s4, lz, W, 2, T + steps, n_loops=5)


def test_effective_depth_page_instances():
    mk = lambda p, r, k, q: I.Shape(1, 1, 1, 1, 32, 1, "gelu", p, r, k, q)
    # discosf.com section 3.1: 6 independent + 6 looped x3 + 6 independent -> depth 30, 18 stored
    assert accounting.effective_depth(mk(6, 6, 3, 6)) == 30
    assert mk(6, 6, 3, 6).n_layers_stored == 18
    # aiboss88.com step 2 / full example: 22 layers x 2 passes = 44; x1 = 22; x4 = 88
    assert [accounting.effective_depth(mk(0, 22, k, 0)) for k in (1, 2, 4)] == [22, 44, 88]
    # aiboss88.com step 3: 48 layers x 4 passes = 192 block applications
    assert accounting.effective_depth(mk(0, 48, 4, 0)) == 192
    # aiboss88.com lineage paragraph: 2 + 4 x 32 + 2 = 132 applications, 8 stored blocks
    assert accounting.effective_depth(mk(2, 4, 32, 2)) == 132 and mk(2, 4, 32, 2).n_layers_stored == 8
    # nxmr.cn section 4.2 table: 24 / 33 / 42 / 51 for loop counts 1..4 (8 + 9 x K + 7)
    assert [accounting.effective_depth(mk(8, 9, k, 7)) for k in (1, 2, 3, 4)] == [24, 33, 42, 51]


@pytest.mark.parametrize("mk,reinject", [(tiny_shape, False), (small_shape, False), (small_shape, True)])
def test_lazy_rho1_all_columns_is_bit_identical_to_dense(mk, reinject):
    s = mk(input_reinject=reinject)
    W = I.gen_weights(s, seed=9)
    T, steps = 24, 4
    ids = I.gen_prompt_ids(s, 2, T, seed=10)
    dec = I.gen_decode_ids(s, 2, steps, seed=11)
    _, d_out, d_dec, _ = run_oracle(s, I.Lazy(mode="per_loop"), W, ids, dec)
    lz = I.Lazy(mode="lazy", rho=1.0, top_s=T, window=T + steps, base_bits=16, res_bits=16)
    m, l_out, l_dec, depth = run_oracle(s, lz, W, ids, dec)
    np.testing.assert_array_equal(l_out, d_out)
    np.testing.assert_array_equal(l_dec, d_dec)
    assert depth == accounting.effective_depth(s)


def test_lazy_sparse_differs_from_dense():
    """With rho < 1 and few columns the lazy result is a different (approximate) function."""
    s = small_shape()
    W = I.gen_weights(s, seed=9)
    ids = I.gen_prompt_ids(s, 1, 40, seed=10)
    _, d_out, _, _ = run_oracle(s, I.Lazy(mode="per_loop"), W, ids, [])
    lz = I.Lazy(mode="lazy", rho=0.25, top_s=6, window=4, base_bits=8, res_bits=4)
    _, l_out, _, _ = run_oracle(s, lz, W, ids, [])
    assert 1e-4 < max_abs_rel(l_out, d_out) < 1.0


def test_last_loop_prefill_identical_and_k1_decode_identical():
    s = small_shape()
    W = I.gen_weights(s, seed=12)
    ids = I.gen_prompt_ids(s, 2, 16, seed=13)
    dec = I.gen_decode_ids(s, 2, 3, seed=14)
    _, p_out, p_dec, _ = run_oracle(s, I.Lazy(mode="per_loop"), W, ids, dec)
    _, l_out, l_dec, _ = run_oracle(s, I.Lazy(mode="last_loop"), W, ids, dec)
    np.testing.assert_array_equal(l_out, p_out)
    assert not np.array_equal(l_dec, p_dec)      # decode sees the overwritten rows
    s1 = small_shape(n_loops=1)
    _, _, p1, _ = run_oracle(s1, I.Lazy(mode="per_loop"), W, ids, dec)
    _, _, l1, _ = run_oracle(s1, I.Lazy(mode="last_loop"), W, ids, dec)
    np.testing.assert_array_equal(l1, p1)


# ---------------------------------------------------------------- RoPE
def test_rope_matches_complex_form_and_invariants():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 64)).astype(np.float32)
    pos = rng.integers(0, 70000, size=50)
    cos, sin = rope_cos_sin(pos, 64, 10000.0)
    y = apply_rope(x, cos, sin)
    ref = torch_ref.rope_complex(torch.as_tensor(x, dtype=torch.float64), pos, 10000.0).numpy()
    assert np.max(np.abs(y - ref)) < 1e-5 * np.max(np.abs(ref)) * 10
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-5)
    # q.k depends on the position difference only
    q = rng.standard_normal((1, 1, 64)).astype(np.float32)
    k = rng.standard_normal((1, 1, 64)).astype(np.float32)
    dots = []
    for shift in (0, 17, 1000):
        cq, sq = rope_cos_sin(np.array([40 + shift]), 64, 10000.0)
        ck, sk = rope_cos_sin(np.array([3 + shift]), 64, 10000.0)
        dots.append(float(np.sum(apply_rope(q, cq, sq) * apply_rope(k, ck, sk))))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-4)


# ---------------------------------------------------------------- attention
def test_attend_matches_masked_sdpa_brute_force():
    rng = np.random.default_rng(1)
    n, H, Hkv, hd, Tc = 30, 6, 2, 16, 30
    q = rng.standard_normal((n, H, hd)).astype(np.float32)
    K = rng.standard_normal((Hkv, Tc, hd)).astype(np.float32)
    V = rng.standard_normal((Hkv, Tc, hd)).astype(np.float32)
    S = [np.sort(rng.choice(Tc, 7, replace=False)).astype(np.int32) for _ in range(Hkv)]
    w = 4
    out = attend(q, K, V, lambda i, g: sparse_cols(i, S[g], w))
    # brute force: dense scores, boolean mask, library softmax attention in float64
    G = H // Hkv
    mask = np.zeros((H, n, Tc), bool)
    for h in range(H):
        for i in range(n):
            for j in range(Tc):
                mask[h, i, j] = (j <= i) and ((j in set(S[h // G].tolist())) or j > i - w)
    qt = torch.as_tensor(q, dtype=torch.float64).transpose(0, 1)
    kt = torch.as_tensor(K, dtype=torch.float64).repeat_interleave(G, dim=0)
    vt = torch.as_tensor(V, dtype=torch.float64).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.as_tensor(mask))
    ref = ref.transpose(0, 1).numpy()
    assert max_abs_rel(out, ref) < 1e-5


def test_attend_identical_keys_gives_mean_and_mass_sums():
    rng = np.random.default_rng(2)
    H, Hkv, hd, Tc = 4, 2, 8, 12
    q = rng.standard_normal((Tc, H, hd)).astype(np.float32)
    K = np.tile(rng.standard_normal((Hkv, 1, hd)).astype(np.float32), (1, Tc, 1))
    V = rng.standard_normal((Hkv, Tc, hd)).astype(np.float32)
    mass = np.zeros((Hkv, Tc), np.float32)
    out = attend(q, K, V, lambda i, g: np.arange(i + 1), mass=mass)
    for i in range(Tc):
        for h in range(H):
            np.testing.assert_allclose(out[i, h], V[h // 2, : i + 1].mean(0), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(mass.sum(1), (H // Hkv) * Tc, rtol=1e-5)
    # uniform probabilities: column j collects sum_{i >= j} 1/(i+1) per head
    exp = np.array([sum(1.0 / (i + 1) for i in range(j, Tc)) for j in range(Tc)]) * (H // Hkv)
    np.testing.assert_allclose(mass[0], exp, rtol=1e-5)


def test_sparse_cols_cover_dense_when_s_plus_w_large():
    S = np.arange(0, 10, dtype=np.int32)
    for i in range(30):
        np.testing.assert_array_equal(sparse_cols(i, S, 21), np.arange(i + 1))
    np.testing.assert_array_equal(sparse_cols(20, np.array([2, 5, 19], np.int32), 3), [2, 5, 18, 19, 20])


def test_column_mass_totals():
    s = small_shape()
    W = I.gen_weights(s, seed=15)
    T = 36
    ids = I.gen_prompt_ids(s, 2, T, seed=16)
    lz = I.Lazy(mode="lazy", rho=0.3, top_s=5, window=3, base_bits=16, res_bits=8)
    m, _, _, _ = run_oracle(s, lz, W, ids, [])
    G = s.n_heads // s.n_kv_heads
    for (r, b), mass in m.mass.items():
        np.testing.assert_allclose(mass.sum(axis=1), G * T, rtol=1e-4)
        for g in range(s.n_kv_heads):
            exp = sorted(sorted(range(T), key=lambda j: (-float(mass[g, j]), j))[:5])
            assert list(m.S[r][b][g]) == exp


def test_column_mass_matches_library_softmax_sums():
    """Mass = sum over queries and group heads of causal softmax probabilities (sharp scores)."""
    rng = np.random.default_rng(3)
    H, Hkv, hd, T = 4, 2, 8, 20
    q = (rng.standard_normal((T, H, hd)) * 3).astype(np.float32)
    K = (rng.standard_normal((Hkv, T, hd)) * 3).astype(np.float32)
    V = rng.standard_normal((Hkv, T, hd)).astype(np.float32)
    mass = np.zeros((Hkv, T), np.float32)
    attend(q, K, V, lambda i, g: np.arange(i + 1), mass=mass)
    qt = torch.as_tensor(q, dtype=torch.float64).transpose(0, 1)          # [H, T, hd]
    kt = torch.as_tensor(K, dtype=torch.float64).repeat_interleave(2, dim=0)
    sc = qt @ kt.transpose(1, 2) / np.sqrt(hd)
    sc = sc.masked_fill(~torch.tril(torch.ones(T, T, dtype=torch.bool)), float("-inf"))
    p = torch.softmax(sc, dim=-1)                                          # [H, T(q), T(k)]
    ref = p.sum(dim=1).view(Hkv, 2, T).sum(dim=1).numpy()
    np.testing.assert_allclose(mass, ref, rtol=2e-5, atol=1e-6)


def test_forced_codes_reproduce_the_source_oracle():
    """An oracle that takes another oracle's selections and codes reproduces it exactly."""
    s = small_shape()
    W = I.gen_weights(s, seed=19)
    ids = I.gen_prompt_ids(s, 2, 30, seed=20)
    dec = I.gen_decode_ids(s, 2, 2, seed=21)
    lz = I.Lazy(mode="lazy", rho=0.3, top_s=6, window=4, base_bits=8, res_bits=4)
    a = LoopedOracle(s, lz, W, 2, 32)
    oa = a.prefill(ids)
    da = [a.decode(d) for d in dec]
    b = LoopedOracle(s, lz, W, 2, 32)
    b.forced_tokens = dict(a.sel)
    b.forced_S = a.S
    b.forced_codes_from = a
    ob = b.prefill(ids)
    db = [b.decode(d) for d in dec]
    np.testing.assert_array_equal(oa, ob)
    for x, y in zip(da, db):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("rows,sparse", [("all", False), ("all", True), ("subset", True)])
def test_masked_attention_equals_row_by_row_attention(rows, sparse):
    """The masked, block-at-a-time form the model uses (attend_masked) gives the
    row-by-row gathered softmax (attend) for every row, several blocks and a ragged
    last block, dense causal or sparse (stable columns plus a window), with the
    column mass; only the summation order inside the products differs."""
    from oracle.model import attend_masked, causal_mask, sparse_mask
    rng = np.random.default_rng(23)
    T, H, Hkv, hd, w = 300, 4, 2, 32, 7
    q = rng.standard_normal((T, H, hd)).astype(np.float32)
    K = (rng.standard_normal((Hkv, T, hd)) * 2).astype(np.float32)
    V = rng.standard_normal((Hkv, T, hd)).astype(np.float32)
    S = [np.sort(rng.choice(T, 40, replace=False)).astype(np.int32) for _ in range(Hkv)]
    pos = np.arange(T) if rows == "all" else np.sort(rng.choice(T, 90, replace=False))
    if sparse:
        allowed = sparse_mask(S, w)
        cols_of = lambda i, g: sparse_cols(int(pos[i]), S[g], w)
    else:
        allowed = causal_mask
        cols_of = lambda i, g: np.arange(int(pos[i]) + 1)
    m1, m2 = np.zeros((Hkv, T), np.float32), np.zeros((Hkv, T), np.float32)
    a = attend_masked(q[pos], K, V, pos, allowed, mass=m1, block=64)
    b = attend(q[pos], K, V, cols_of, mass=m2)
    assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(b))
    assert np.max(np.abs(m1 - m2)) <= 1e-5 * np.max(np.abs(m2))
    # the mask is exactly the gathered column set
    for i in range(0, len(pos), 17):
        for g in range(Hkv):
            got = np.nonzero(allowed(pos[i:i + 1], np.arange(int(pos[i]) + 1), g)[0])[0]
            assert np.array_equal(got, cols_of(i, g))
