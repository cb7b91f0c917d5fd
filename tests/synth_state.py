"""A lazy KV-store state built on the host, as a prefill could leave it, for decode
parity at full context length (where a CPU prefill is out of reach), and its store
snapshot (the library's snapshot format: header, then the store buffer's leading
bytes in the layout lk_kv_store_view reports).

The state is random but well formed: int8 base codes with float16 group scales,
int4 (or int8) residual codes on the kept rows of every loop k >= 2 (a sorted random
subset of n_selected(rho, T) prompt positions, slots in position order), and a
sorted random stable-column set per (shared layer, KV head).  It holds no arithmetic
of the method; the oracle and the GPU both read it as their stored state."""
import ctypes

import numpy as np

from cross_loop_kv_amd import binding as B
from oracle import quant
from oracle.select import n_selected


def synthetic_lazy_state(shape, lazy, T, Tmax, seed, k_std=4.0, v_std=1.0, res_std=0.2):
    """One sequence's state (oracle layout, batch 1).  Base K/V elements have about
    k_std / v_std spread (so that loop-1 attention over T columns is peaked, not
    flat), residuals about res_std."""
    if lazy.base_bits != 8 or lazy.res_bits not in (4, 8):
        raise ValueError("synthetic states are built for int8 bases and int4/int8 residuals")
    rng = np.random.default_rng(seed)
    R, K, Hkv, hd, g = shape.n_shared, shape.n_loops, shape.n_kv_heads, shape.head_dim, lazy.group
    ng = hd // g
    n = n_selected(lazy.rho, T)
    slots = n + Tmax - T
    qres = 7 if lazy.res_bits == 4 else 127

    def codes(shape_, qmax):
        return rng.integers(-qmax, qmax + 1, size=shape_, dtype=np.int8)

    def scales(shape_, std, qmax):
        # a uniform code has spread about qmax / sqrt(3)
        s = std * np.sqrt(3.0) / qmax * rng.uniform(0.5, 1.5, size=shape_)
        return s.astype(np.float16)

    base = []
    for r in range(R):
        pair = []
        for kv, std in ((0, k_std), (1, v_std)):
            c = np.zeros((1, Hkv, Tmax, hd), np.int8)
            sc = np.zeros((1, Hkv, Tmax, ng), np.float16)
            c[0, :, :T] = codes((Hkv, T, hd), 127)
            sc[0, :, :T] = scales((Hkv, T, ng), std, 127)
            pair.append((c, sc))
        base.append(pair)
    slot = np.full((K, 1, Tmax), -1, np.int32)
    res = {}
    for k in range(2, K + 1):
        kept = np.sort(rng.choice(T, size=n, replace=False))
        slot[k - 1, 0, kept] = np.arange(n, dtype=np.int32)
        for r in range(R):
            for kv in range(2):
                c = np.zeros((1, Hkv, slots, hd), np.int8)
                sc = np.zeros((1, Hkv, slots, ng), np.float16)
                c[0, :, :n] = codes((Hkv, n, hd), qres)
                sc[0, :, :n] = scales((Hkv, n, ng), res_std, qres)
                res[(k, r, kv)] = (c, sc)
    ncols = min(lazy.top_s, T)
    S = [[[np.sort(rng.choice(T, size=ncols, replace=False)).astype(np.int32) for _ in range(Hkv)]]
         for _ in range(R)]
    return dict(T=T, base=base, res=res, slot=slot, S=S)


def _interleave8(a):
    """[Hkv, Tp, X] -> [Hkv, Tp/8, X, 8] (blocks of 8 interleaved positions)."""
    H_, Tp, X = a.shape
    return np.ascontiguousarray(a.reshape(H_, Tp // 8, 8, X).transpose(0, 1, 3, 2))


def snapshot_with_states(store, shape, lazy, states, loops=None):
    """A snapshot of `store` (allocated, not prefilled) in which sequence b holds
    states[b] (one sequence each, oracle layout, all of one prompt length T) and the
    other sequences hold empty rows, no kept tokens and the columns 0..n_cols-1;
    length = T."""
    v = store.view()
    R, K, Hkv, hd = shape.n_shared, shape.n_loops, shape.n_kv_heads, shape.head_dim
    if shape.n_prelude + shape.n_coda:
        raise ValueError("prelude/coda rows are not synthesized")
    Bn, Tp = store.batch, v.row_stride
    T = {st["T"] for st in states.values()}
    assert len(T) == 1
    T = T.pop()
    ng = hd // lazy.group
    hdr = ctypes.sizeof(B.lk_store_snapshot)
    n = ctypes.c_size_t()
    B._check(B.lib().lk_kv_store_export(store.s, None, 0, ctypes.byref(n), None))
    body_bytes = n.value - hdr
    buf = np.zeros(n.value, np.uint8)
    body = buf[hdr:]
    base0 = store.buf.data_ptr()

    def region(ptr, nbytes, dtype):
        off = int(ptr) - base0
        assert 0 <= off and off + nbytes <= body_bytes
        return body[off:off + nbytes].view(dtype)

    Tm = store.max_tokens
    assert Tm <= Tp and T == store.prompt
    sm = region(v.slot_maps, (K - 1) * Bn * Tp * 4, np.int32).reshape(K - 1, Bn, Tp)
    sm[:] = -1
    cols = region(v.columns, R * Bn * Hkv * v.n_columns * 4, np.int32).reshape(R, Bn, Hkv, v.n_columns)
    cols[:] = np.arange(v.n_columns, dtype=np.int32)
    for seq, state in states.items():
        _write_one(state, seq, region, v, shape, lazy, Bn)
        sm[:, seq, :Tm] = state["slot"][1:, 0]
        for r in range(R):
            cols[r, seq] = np.stack(state["S"][r][0])
    h = B.lk_store_snapshot.from_buffer(buf)
    h.magic, h.header_bytes, h.version = B.SNAPSHOT_MAGIC, hdr, B.SNAPSHOT_VERSION
    h.cfg, h.lazy = B.model_cfg(shape), B.lazy_cfg(lazy)
    h.batch, h.prompt_tokens, h.max_tokens = Bn, store.prompt, store.max_tokens
    h.loops = K if loops is None else loops
    h.tokens, h.prefilled, h.body_bytes = T, 1, body_bytes
    del h
    return buf


def _write_one(state, seq, region, v, shape, lazy, Bn):
    """Base and residual rows of one sequence into the snapshot body."""
    R, K, Hkv, hd = shape.n_shared, shape.n_loops, shape.n_kv_heads, shape.head_dim
    ng, Tp = hd // lazy.group, v.row_stride
    Tm = state["base"][0][0][0].shape[2]
    reg = Bn * Hkv * Tp * hd             # int8 codes of one (layer, K|V) base region
    sreg = Bn * Hkv * Tp * ng * 2        # bytes of its scales
    rows = Bn * Hkv * v.slots            # rows of one (loop, layer, K|V) residual region
    assert state["res"][(2, 0, 0)][0].shape[2] == v.slots
    for r in range(R):
        for kv in range(2):
            c, sc = state["base"][r][kv]
            cp = np.zeros((Hkv, Tp, hd), np.int8)
            cp[:, :Tm] = c[0]
            sp = np.zeros((Hkv, Tp, ng), np.uint16)
            sp[:, :Tm] = sc[0].view(np.uint16)
            if kv == 1:
                cp, sp = _interleave8(cp), _interleave8(sp)
            region(v.base_codes + (2 * r + kv) * reg, reg, np.int8).reshape(Bn, -1)[seq] = cp.reshape(-1)
            region(v.base_scales + (2 * r + kv) * sreg, sreg, np.uint16).reshape(Bn, -1)[seq] = sp.reshape(-1)
    for k in range(2, K + 1):
        for r in range(R):
            for kv in range(2):
                c, sc = state["res"][(k, r, kv)]
                g = ((k - 2) * R + r) * 2 + kv
                packed = quant.pack_int4(c[0]) if lazy.res_bits == 4 else c[0].view(np.uint8)
                region(v.res_codes + g * rows * v.res_row_bytes, rows * v.res_row_bytes, np.uint8) \
                    .reshape(Bn, -1)[seq] = packed.reshape(-1)
                region(v.res_scales + g * rows * ng * 2, rows * ng * 2, np.uint16) \
                    .reshape(Bn, -1)[seq] = sc[0].view(np.uint16).reshape(-1)
