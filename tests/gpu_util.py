"""Helpers of the GPU parity tests: run the oracle and the HIP path on the same inputs."""
import copy
import sys
import time

import numpy as np
import torch

from cross_loop_kv_amd import binding as B
from cross_loop_kv_amd import inputs as I
from oracle.model import LoopedOracle


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_abs_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def oracle_selection(m, shape, batch):
    """Oracle's kept tokens [K-1, B, n] and column sets [R, B, Hkv, n_cols] as int32 arrays."""
    K, R, Hkv = shape.n_loops, shape.n_shared, shape.n_kv_heads
    tok = np.stack([np.stack([m.sel[(k, b)] for b in range(batch)]) for k in range(2, K + 1)]) \
        if K >= 2 else np.zeros((0, batch, 1), np.int32)
    cols = np.stack([np.stack([np.stack(m.S[r][b]) for b in range(batch)]) for r in range(R)])
    return tok.astype(np.int32), cols.astype(np.int32)


def store_region(store, ptr, nbytes, dtype):
    """A torch view of `nbytes` of the store buffer starting at device address `ptr`."""
    off = int(ptr) - store.buf.data_ptr()
    assert 0 <= off and off + nbytes <= store.buf.numel()
    return store.buf[off:off + nbytes].view(dtype)


def gpu_selection(store, shape, batch, prompt):
    """Kept prompt tokens per loop read back from the store's slot maps, and the column sets."""
    v = store.view()
    K, R, Hkv = shape.n_loops, shape.n_shared, shape.n_kv_heads
    Tm = store.max_tokens
    torch.cuda.synchronize()
    sm = store_region(store, v.slot_maps, (K - 1) * batch * Tm * 4, torch.int32)
    cols = store_region(store, v.columns, R * batch * Hkv * v.n_columns * 4, torch.int32)
    sm = sm.view(K - 1, batch, Tm)[:, :, :prompt].cpu().numpy()
    sel = {(k, b): np.nonzero(sm[k - 2, b] >= 0)[0] for k in range(2, K + 1) for b in range(batch)}
    return sel, cols.view(R, batch, Hkv, v.n_columns).cpu().numpy()


def run_pair(shape, lazy, batch, prompt, steps, seed=0, force=True, weights=None):
    """Prefill + `steps` decode steps on the oracle and the GPU; returns a result dict."""
    W = weights if weights is not None else I.gen_weights(shape, seed=seed)
    ids = I.gen_prompt_ids(shape, batch, prompt)
    dec = I.gen_decode_ids(shape, batch, steps)
    t0 = time.time()
    m = LoopedOracle(shape, lazy, W, batch, prompt + steps)
    o_out = m.prefill(ids)
    o_dec = [m.decode(d) for d in dec]
    t_oracle = time.time() - t0
    model = B.LoopedModel(shape, lazy, W)
    store = model.store(batch, prompt, prompt + steps)
    if lazy.mode == "lazy" and force:
        tok, cols = oracle_selection(m, shape, batch)
        store.force_selection(torch.from_numpy(tok).cuda() if tok.size else None,
                              torch.from_numpy(cols).cuda())
    g_out = model.prefill(store, torch.from_numpy(ids)).cpu().numpy()
    g_dec = [model.decode(store, torch.from_numpy(d)).cpu().numpy() for d in dec]
    torch.cuda.synchronize()
    res = dict(oracle=m, model=model, store=store, o_out=o_out, g_out=g_out, o_dec=o_dec, g_dec=g_dec,
               t_oracle=t_oracle, ids=ids, dec=dec)
    res["err_prefill"] = max_abs_rel(g_out, o_out)
    res["err_decode"] = [max_abs_rel(g, o) for g, o in zip(g_dec, o_dec)]
    return res
