"""C-ABI checks that need no GPU: symbols, struct layouts, validation, size queries."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from cross_loop_kv_amd import binding as B
from cross_loop_kv_amd import inputs as I
from oracle import accounting

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "looped_kv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lk_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    lib = B.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
        assert n in B.EXPORTED, n


def test_struct_layouts_match_the_header():
    prog = r"""
#include <stdio.h>
#include <stddef.h>
#include "looped_kv.h"
#define P(T, f) printf("%s.%s %zu\n", #T, #f, offsetof(T, f));
int main(void) {
  printf("lk_model_cfg %zu\nlk_lazy_cfg %zu\nlk_layer_weights %zu\nlk_weights %zu\nlk_store_view %zu\n"
         "lk_store_snapshot %zu\nlk_dbg_attn_args %zu\n",
         sizeof(lk_model_cfg), sizeof(lk_lazy_cfg), sizeof(lk_layer_weights), sizeof(lk_weights),
         sizeof(lk_store_view), sizeof(lk_store_snapshot), sizeof(lk_dbg_attn_args));
  P(lk_dbg_attn_args, q) P(lk_dbg_attn_args, q_half) P(lk_dbg_attn_args, cols) P(lk_dbg_attn_args, s_cap)
  P(lk_dbg_attn_args, r_cap) P(lk_dbg_attn_args, qpos) P(lk_dbg_attn_args, n_rows) P(lk_dbg_attn_args, out32)
  P(lk_dbg_attn_args, mass) P(lk_dbg_attn_args, ws_bytes)
  P(lk_store_snapshot, cfg) P(lk_store_snapshot, lazy) P(lk_store_snapshot, batch)
  P(lk_store_snapshot, prefilled) P(lk_store_snapshot, body_bytes)
  printf("magic %llu\n", (unsigned long long)LK_SNAPSHOT_MAGIC);
  printf("snapshot_version %d\n", (int)LK_SNAPSHOT_VERSION);
  P(lk_model_cfg, ffn_act) P(lk_model_cfg, rms_eps) P(lk_model_cfg, rope_theta)
  P(lk_lazy_cfg, rho) P(lk_lazy_cfg, top_s) P(lk_lazy_cfg, group) P(lk_lazy_cfg, stale_keys)
  P(lk_lazy_cfg, refresh_every) P(lk_lazy_cfg, diff_attn) P(lk_lazy_cfg, skip_tau)
  P(lk_weights, layers) P(lk_layer_weights, w_down)
  P(lk_store_view, slots) P(lk_store_view, n_selected) P(lk_store_view, res_row_bytes) P(lk_store_view, row_stride)
  P(lk_store_view, decode_cache) P(lk_store_view, ring_rows) P(lk_store_view, first_cached_loop)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "p.c")
        exe = os.path.join(d, "p")
        open(c, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(line.rsplit(" ", 1) for line in out.strip().splitlines())
    assert int(got.pop("magic")) == B.SNAPSHOT_MAGIC
    assert int(got.pop("snapshot_version")) == B.SNAPSHOT_VERSION
    assert B.SNAPSHOT_MAGIC.to_bytes(8, "little") == b"LKSNAP01"
    for name in ("lk_model_cfg", "lk_lazy_cfg", "lk_layer_weights", "lk_weights", "lk_store_view",
                 "lk_store_snapshot", "lk_dbg_attn_args"):
        assert int(got[name]) == ctypes.sizeof(getattr(B, name)), name
    for key, val in got.items():
        if "." in key:
            t, f = key.split(".")
            assert getattr(getattr(B, t), f).offset == int(val), key


def _handle(shape, lazy):
    cfg = B.model_cfg(shape)
    lz = B.lazy_cfg(lazy)
    n = shape.n_prelude + shape.n_shared + shape.n_coda
    lw = (B.lk_layer_weights * n)()
    for i in range(n):
        lw[i] = B.lk_layer_weights(16, 16, 16, 16, 16, 16)   # never dereferenced on the host
    w = B.lk_weights(16, 16, 16, lw)
    return B.lk_create(cfg, lz, w)


@pytest.mark.parametrize("name", list(I.WORKLOADS))
def test_store_size_query_matches_closed_form(name):
    wl = I.workload(name)
    for mode in ("per_loop", "last_loop", "lazy"):
        lz = I.Lazy(**{**wl.lazy.__dict__, "mode": mode})
        h = _handle(wl.shape, lz)
        try:
            T, Tm = min(wl.prompt, 4096), min(wl.prompt, 4096) + 64
            _, need = B.lk_kv_store_alloc(h, wl.batch, T, Tm)
            exp = accounting.kv_bytes(wl.shape, lz, wl.batch, T, Tm)["total"]
            # plus the lazy decode cache: float16 K and V rows of the stable columns
            # (rounded up to 128 per sequence and KV head) and of a window ring
            # (window + 16 rounded up to 128) for every loop k >= 2
            s = wl.shape
            if mode == "lazy" and s.n_loops >= 2:
                ncs = -(-min(lz.top_s, T) // 128) * 128
                wr = -(-(lz.window + 16) // 128) * 128
                exp += (s.n_loops - 1) * s.n_shared * 2 * wl.batch * s.n_kv_heads * (ncs + wr) * s.head_dim * 2
            assert exp <= need <= exp + 256 * 13, (mode, need, exp)
            assert B.lk_effective_depth(h) == accounting.effective_depth(wl.shape)
            ws1 = B.lk_workspace_bytes(h, wl.batch, 1)
            wsT = B.lk_workspace_bytes(h, wl.batch, T)
            assert 0 < ws1 <= wsT
        finally:
            B.lk_destroy(h)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, -2), ("n_kv_heads", 3, -1), ("n_shared", 0, -1), ("d_model", 100, -2),
    ("n_loops", 0, -1), ("n_loops", 18, -2), ("ffn_act", "relu", None),
])
def test_create_rejects_bad_model_configs(field, value, code):
    s = I.workload("tiny_1p2x2c1_t32").shape
    if value == "relu":
        with pytest.raises(KeyError):
            B.model_cfg(I.Shape(**{**s.__dict__, "ffn_act": "relu"}))
        return
    setattr(s, field, value)
    with pytest.raises(B.LKError) as e:
        _handle(s, I.Lazy(mode="per_loop"))
    assert e.value.code == code


@pytest.mark.parametrize("kw", [dict(rho=0.0), dict(rho=1.5), dict(window=0), dict(top_s=0),
                                dict(base_bits=4), dict(res_bits=2), dict(group=16), dict(stale_keys=2),
                                dict(refresh_every=-1), dict(diff_attn=2),
                                dict(skip_tau=-1.0), dict(skip_tau=float("nan"))])
def test_create_rejects_bad_lazy_configs(kw):
    s = I.workload("tiny_1p2x2c1_t32").shape
    lz = I.Lazy(mode="lazy", rho=0.5, top_s=8, window=4, base_bits=16, res_bits=8)
    for k, v in kw.items():
        setattr(lz, k, v)
    with pytest.raises(B.LKError) as e:
        _handle(s, lz)
    assert e.value.code in (-1, -2)


def test_alloc_and_workspace_argument_errors():
    wl = I.workload("tiny_1p2x2c1_t32")
    h = _handle(wl.shape, wl.lazy)
    try:
        for args in ((0, 8, 8), (1, 0, 8), (1, 9, 8)):
            with pytest.raises(B.LKError) as e:
                B.lk_kv_store_alloc(h, *args)
            assert e.value.code == -1
        _, need = B.lk_kv_store_alloc(h, 1, 8, 8)
        with pytest.raises(B.LKError) as e:   # buffer too small: refused before any launch
            B.lk_kv_store_alloc(h, 1, 8, 8, dev_buf=256, buf_bytes=need - 1)
        assert e.value.code == -3
        with pytest.raises(B.LKError):
            B.lk_workspace_bytes(h, 0, 1)
    finally:
        B.lk_destroy(h)


def test_null_arguments_are_errors():
    lib = B.lib()
    assert lib.lk_looped_prefill(None, None, None, 1, 1, None, None, 0, None) == -1
    assert lib.lk_looped_decode_step(None, None, None, None, None, 0, None) == -1
    assert lib.lk_dbg_topk(None, 1, 1, 1, None, None) == -1
    assert b"null" in lib.lk_last_error()


def test_snapshot_size_query_and_import_validation():
    """Snapshot header checks, all made on the host before any copy (a per_loop store
    is allocated without a launch, so a dummy device address serves)."""
    wl = I.workload("tiny_1p2x2c1_t32")
    lz = I.Lazy(mode="per_loop")
    h = _handle(wl.shape, lz)
    other = _handle(I.Shape(**{**wl.shape.__dict__, "input_reinject": True}), lz)
    try:
        _, need = B.lk_kv_store_alloc(h, 1, 8, 12)
        s, _ = B.lk_kv_store_alloc(h, 1, 8, 12, dev_buf=256, buf_bytes=need)
        hdr_bytes = ctypes.sizeof(B.lk_store_snapshot)
        n = ctypes.c_size_t()
        assert B.lib().lk_kv_store_export(s, None, 0, ctypes.byref(n), None) == 0
        body = n.value - hdr_bytes
        assert 0 < body <= need

        def header(**kw):
            hd = B.lk_store_snapshot(B.SNAPSHOT_MAGIC, hdr_bytes, B.SNAPSHOT_VERSION, B.model_cfg(wl.shape),
                                     B.lazy_cfg(lz), 1, 8, 12, wl.shape.n_loops, 10, 1, body)
            for k, v in kw.items():
                setattr(hd, k, v)
            return bytearray(bytes(hd)) + bytearray(body)

        import numpy as np
        cases = [
            ("short", header()[:hdr_bytes - 1]),
            ("magic", header(magic=B.SNAPSHOT_MAGIC + 1)),
            ("version", header(version=99)),
            ("config", header(cfg=B.model_cfg(I.Shape(**{**wl.shape.__dict__, "input_reinject": True})))),
            ("policy", header(lazy=B.lazy_cfg(I.Lazy(mode="last_loop")))),
            ("batch", header(batch=2)),
            ("capacity", header(max_tokens=13)),
            ("loops", header(loops=0)),
            ("loops", header(loops=wl.shape.n_loops + 1)),
            ("length", header(tokens=7)),
            ("length", header(tokens=13)),
            ("length", header(prefilled=0)),
            ("body", header(body_bytes=body + 256)),
            ("truncated", header()[:-1]),
        ]
        for what, buf in cases:
            a = np.frombuffer(bytes(buf), np.uint8)
            with pytest.raises(B.LKError) as e:
                B.lk_kv_store_import(s, a)
            assert e.value.code == -1, what
        assert B.lk_kv_store_length(s) == 0
        small = np.zeros(8, np.uint8)   # the snapshot buffer must hold header and body
        assert B.lib().lk_kv_store_export(s, small.ctypes.data, small.size, ctypes.byref(n), None) == -3
        for bad in (0, wl.shape.n_loops + 1):
            with pytest.raises(B.LKError):
                B.lk_kv_store_set_loops(s, bad)
        B.lk_kv_store_set_loops(s, 1)
        B.lk_kv_store_release(s)
    finally:
        B.lk_destroy(other)
        B.lk_destroy(h)


def test_debug_attention_argument_errors_and_size_query():
    """Host-side checks of lk_dbg_attention (nothing is launched): bad head counts and
    shapes are refused, and with no workspace the decode kinds report the bytes of
    their split partials (B * H * splits * (hd + 2) floats, splits as a decode step
    sizes them for the capacity tmax)."""
    a = B.lk_dbg_attn_args(kind=B.DBG_ATTN["decode"], B=8, H=16, Hkv=4, hd=128, kv_format=1, t=100,
                           tmax=33088, q=16, k=16, v=16, k_scales=16, v_scales=16, out=16)
    need = B.lk_dbg_attention(a)
    assert need > 0 and need % (8 * 16 * 130 * 4) == 0
    splits = need // (8 * 16 * 130 * 4)
    assert 1 <= splits <= 256 and splits * 768 >= (8 * 4 * 33088) // 768   # chunks >= 128 keys
    bad = B.lk_dbg_attn_args(kind=B.DBG_ATTN["decode"], B=8, H=12, Hkv=4, hd=128, kv_format=1, t=10, tmax=64,
                             q=16, k=16, v=16, k_scales=16, v_scales=16, out=16)
    with pytest.raises(B.LKError):
        B.lk_dbg_attention(bad)
    seg = B.lk_dbg_attn_args(kind=B.DBG_ATTN["decode_seg"], B=2, H=8, Hkv=2, hd=64, t=500, q=16, cols=16,
                             n_cols=100, window=40, s_k=16, s_v=16, s_cap=128, r_k=16, r_v=16, r_cap=128, out=16)
    assert B.lk_dbg_attention(seg) == 2 * 8 * 2 * 66 * 4      # 1 + 1 splits of 128 rows
    seg.s_cap = 64                                            # below n_cols and not a multiple of 128
    with pytest.raises(B.LKError):
        B.lk_dbg_attention(seg)
    sp = B.lk_dbg_attn_args(kind=B.DBG_ATTN["prefill_sparse"], B=1, H=8, Hkv=2, hd=64, T=100, q=16, cols=16,
                            n_cols=10, window=4, s_k=16, s_v=16, s_cap=16, r_k=16, r_v=16, r_cap=104, qpos=16,
                            n_rows=10, out=16)
    with pytest.raises(B.LKError) as e:
        B.lk_dbg_attention(sp)                                # head_dim 64 is not taken there
    assert e.value.code == -2
    with pytest.raises(B.LKError):
        B.lk_dbg_attention(B.lk_dbg_attn_args(kind=9, B=1, H=1, Hkv=1, hd=32, q=16, out=16))
