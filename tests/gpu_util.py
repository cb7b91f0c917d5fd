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
    K, R, Hkv = m.K, shape.n_shared, shape.n_kv_heads
    # refresh loops keep every token and ignore their rows here: the first n stand in
    tok = np.stack([np.stack([m.sel[(k, b)][:m.n_sel] for b in range(batch)]) for k in range(2, K + 1)]) \
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
    Tm = v.row_stride
    torch.cuda.synchronize()
    sm = store_region(store, v.slot_maps, (K - 1) * batch * Tm * 4, torch.int32)
    cols = store_region(store, v.columns, R * batch * Hkv * v.n_columns * 4, torch.int32)
    sm = sm.view(K - 1, batch, Tm)[:, :, :prompt].cpu().numpy()
    sel = {(k, b): np.nonzero(sm[k - 2, b] >= 0)[0] for k in range(2, K + 1) for b in range(batch)}
    return sel, cols.view(R, batch, Hkv, v.n_columns).cpu().numpy()


def _pad_t(a, tpad):
    """Pad axis 2 (positions) of [B, Hkv, T, ...] to tpad."""
    out = np.zeros(a.shape[:2] + (tpad,) + a.shape[3:], a.dtype)
    out[:, :, : a.shape[2]] = a
    return out


def _interleave8(a):
    """[B, Hkv, Tp, X] -> [B, Hkv, Tp/8, X, 8] (blocks of 8 interleaved positions)."""
    B_, H_, Tp, X = a.shape
    return np.ascontiguousarray(a.reshape(B_, H_, Tp // 8, 8, X).transpose(0, 1, 2, 4, 3))


def _write(store, ptr, arr):
    raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
    store_region(store, ptr, raw.size, torch.uint8).copy_(torch.from_numpy(raw))


def inject_oracle_codes(store, m, shape, lazy):
    """Copy the oracle's int8 base codes and 4/8-bit residual codes (with their float16
    scales) into the GPU store, in the store's documented layout."""
    from oracle import quant
    v = store.view()
    B_, Hkv, hd = m.B, shape.n_kv_heads, shape.head_dim
    R, K, Tp = shape.n_shared, m.K, v.row_stride
    ng = hd // lazy.group
    if lazy.base_bits == 8:
        reg = B_ * Hkv * Tp * hd               # int8 elements of one (layer, K|V) region
        sreg = B_ * Hkv * Tp * ng * 2          # bytes of its scale region
        for r in range(R):
            for kv in range(2):
                codes, sc = m.base[r][kv]
                codes, sc = _pad_t(codes, Tp), _pad_t(sc.view(np.uint16), Tp)
                if kv == 1:
                    codes, sc = _interleave8(codes), _interleave8(sc)
                _write(store, v.base_codes + (2 * r + kv) * reg, codes)
                _write(store, v.base_scales + (2 * r + kv) * sreg, sc)
    if lazy.res_bits in (4, 8):
        rows = B_ * Hkv * v.slots
        for k in range(2, K + 1):
            for r in range(R):
                for kv in range(2):
                    codes, sc = m.res[(k, r, kv)]
                    reg = ((k - 2) * R + r) * 2 + kv
                    packed = quant.pack_int4(codes) if lazy.res_bits == 4 else codes.view(np.uint8)
                    _write(store, v.res_codes + reg * rows * v.res_row_bytes, packed)
                    _write(store, v.res_scales + reg * rows * ng * 2, sc.view(np.uint16))
    torch.cuda.synchronize()
    store.keep_codes(True)


_WEIGHTS = {}


def cached_weights(shape, seed):
    """I.gen_weights(shape, seed), kept for the next call with the same arguments (the
    full-width shapes take tens of seconds to draw); one entry is kept."""
    key = (repr(shape), seed)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        _WEIGHTS[key] = I.gen_weights(shape, seed=seed)
    return _WEIGHTS[key]


def run_pair(shape, lazy, batch, prompt, steps, seed=0, force=True, weights=None, force_codes=None,
             loops=None):
    """Prefill + `steps` decode steps on the oracle and the GPU; returns a result dict.

    force: inject the oracle's token and column selections.  force_codes (default:
    with int4 residuals): also inject the oracle's quantized codes (prefill and decode
    rows), so that both sides make the same integer decisions on inputs that differ by
    the GPU's bf16 products (an int4 step is amax/7 of a group, far more than that
    rounding).  The writer itself is compared bit for bit on identical inputs in
    test_gpu_writer, and the full-context decode tests run on the GPU's own codes.
    loops: run the shared block this many times (default: the shape's n_loops)."""
    W = weights if weights is not None else cached_weights(shape, seed)
    ids = I.gen_prompt_ids(shape, batch, prompt)
    dec = I.gen_decode_ids(shape, batch, steps)
    t0 = time.time()
    m = LoopedOracle(shape, lazy, W, batch, prompt + steps, n_loops=loops)
    o_out = m.prefill(ids)
    o_dec = [m.decode(d) for d in dec]
    t_oracle = time.time() - t0
    model = B.LoopedModel(shape, lazy, W)
    store = model.store(batch, prompt, prompt + steps, loops=loops)
    if lazy.mode == "lazy" and force:
        tok, cols = oracle_selection(m, shape, batch)
        store.force_selection(torch.from_numpy(tok).cuda() if tok.size else None,
                              torch.from_numpy(cols).cuda())
        if force_codes is None:
            force_codes = lazy.res_bits == 4
        if force_codes:
            inject_oracle_codes(store, m, shape, lazy)
    g_out = model.prefill(store, torch.from_numpy(ids)).cpu().numpy()
    g_dec = [model.decode(store, torch.from_numpy(d)).cpu().numpy() for d in dec]
    torch.cuda.synchronize()
    res = dict(oracle=m, model=model, store=store, o_out=o_out, g_out=g_out, o_dec=o_dec, g_dec=g_dec,
               t_oracle=t_oracle, ids=ids, dec=dec, forced_codes=bool(force and force_codes))
    res["err_prefill"] = max_abs_rel(g_out, o_out)
    res["err_decode"] = [max_abs_rel(g, o) for g, o in zip(g_dec, o_dec)]
    return res
