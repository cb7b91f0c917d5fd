"""Prefill at full size against the oracle, through the C ABI.

* The prefill workload at its own size: 2 + 4 x 4 + 2 layers, d 2048, 16 heads of 128
  (MHA), FFN 5632 SwiGLU, a 4096-token prompt, rho 0.25, top-s 256, window 128,
  bf16 base and int4 residuals; one sequence.
* The decode workload's prefill at its full context: d 2048, 16 query / 4 KV heads of
  128, FFN 5632, 4 loops, a 32768-token prompt, rho 0.1, top-s 1024, window 512, int8
  base and int4 residuals; one sequence and 1 shared layer in place of 48 (the
  kernels and their launch shapes are those of the 48-layer prefill: depth only
  repeats them).  It builds the store that decode reads: flash attention writing its
  log-sum-exp over 512 key tiles, the column mass over 32768 queries, top-1024 over
  32768 columns and the sparse rows over 1536 columns.

The oracle's token and column selections are injected (forced selection), and so are
its quantized codes (both sides take the same integer decisions on inputs that differ
by the GPU's bf16 products; the writer itself is compared bit for bit on identical
inputs in test_gpu_writer).  Every output row must agree within max-abs-relative
2e-2.  The GPU's own column selection (run
without forcing, on the same inputs) must be a valid top-1024 of the oracle's loop-1
mass up to a 5 % margin.
"""
import copy
import time

import numpy as np
import pytest
import torch

from cross_loop_kv_amd import binding as B
from cross_loop_kv_amd import inputs as I
from oracle.model import LoopedOracle
from tests.gpu_util import cached_weights, gpu_selection, inject_oracle_codes, log, max_abs_rel, oracle_selection

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _prefill_pair(shape, lz, T, force=True):
    W = cached_weights(shape, 0)
    ids = I.gen_prompt_ids(shape, 1, T)
    t0 = time.time()
    m = LoopedOracle(shape, lz, W, 1, T)
    o = m.prefill(ids)
    log(f"  oracle prefill {time.time() - t0:.1f}s")
    model = B.LoopedModel(shape, lz, W)
    st = model.store(1, T, T)
    if force:
        tok, cols = oracle_selection(m, shape, 1)
        st.force_selection(torch.from_numpy(tok).cuda(), torch.from_numpy(cols).cuda())
        inject_oracle_codes(st, m, shape, lz)
    g = model.prefill(st, torch.from_numpy(ids)).cpu().numpy()
    torch.cuda.synchronize()
    return m, model, st, o, g, ids


@pytest.mark.timeout(900)
def test_prefill_workload_at_full_size():
    wl = I.workload("prefill_2p4x4c2_b4_t4096")
    log(f"prefill workload: B=1 T={wl.prompt}")
    m, model, st, o, g, _ = _prefill_pair(wl.shape, wl.lazy, wl.prompt)
    e = max_abs_rel(g, o)
    log(f"  prefill vs fp32 oracle: {e:.3e}")
    assert np.isfinite(g).all() and e < TOL


@pytest.mark.timeout(900)
def test_decode_workload_prefill_at_full_context():
    wl = I.workload("deep_48x4_b8_ctx32k")
    s = copy.copy(wl.shape)
    s.n_shared = 1
    log(f"decode workload prefill: B=1 T={wl.prompt} R=1 K={s.n_loops}")
    m, model, st, o, g, ids = _prefill_pair(s, wl.lazy, wl.prompt)
    e = max_abs_rel(g, o)
    rows = np.max(np.abs(g - o), axis=-1) / np.max(np.abs(o))
    log(f"  prefill vs fp32 oracle: {e:.3e} (rows above 1e-2: {int((rows > 1e-2).sum())})")
    assert np.isfinite(g).all() and e < TOL
    # natural column selection on the same prompt: a valid top-1024 of the oracle's mass
    st2 = model.store(1, wl.prompt, wl.prompt)
    model.prefill(st2, torch.from_numpy(ids))
    torch.cuda.synchronize()
    _, cols = gpu_selection(st2, s, 1, wl.prompt)
    from tests.test_gpu_model import valid_top
    d = sum(valid_top(cols[0, 0, g_], m.mass[(0, 0)][g_], wl.lazy.top_s, 0.05) for g_ in range(s.n_kv_heads))
    log(f"  natural top-{wl.lazy.top_s} columns: {d} differ from the oracle's, all in near-ties")
