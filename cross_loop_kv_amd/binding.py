"""ctypes binding of ``liblooped_kv.so`` (the C ABI in include/looped_kv.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch provides device memory (``tensor.data_ptr()``) and the
stream.  If the library is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblooped_kv.so")

LK_OK = 0
LK_ERR = {-1: "LK_ERR_INVALID_ARG", -2: "LK_ERR_UNSUPPORTED", -3: "LK_ERR_CAPACITY",
          -4: "LK_ERR_HIP", -5: "LK_ERR_STATE"}
MODES = {"per_loop": 0, "last_loop": 1, "lazy": 2}
ACTS = {"gelu": 0, "swiglu": 1}


class LKError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{LK_ERR.get(code, code)}: {msg}")
        self.code = code


class lk_model_cfg(C.Structure):
    _fields_ = [("vocab", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("ffn_act", C.c_int32), ("n_prelude", C.c_int32), ("n_shared", C.c_int32),
                ("n_loops", C.c_int32), ("n_coda", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_float), ("input_reinject", C.c_int32)]


class lk_lazy_cfg(C.Structure):
    _fields_ = [("mode", C.c_int32), ("rho", C.c_double), ("top_s", C.c_int32),
                ("window", C.c_int32), ("base_bits", C.c_int32), ("res_bits", C.c_int32),
                ("group", C.c_int32), ("stale_keys", C.c_int32), ("refresh_every", C.c_int32),
                ("diff_attn", C.c_int32), ("skip_tau", C.c_float)]


class lk_layer_weights(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("wqkv", C.c_void_p), ("wo", C.c_void_p),
                ("ffn_norm", C.c_void_p), ("w_in", C.c_void_p), ("w_down", C.c_void_p)]


class lk_weights(C.Structure):
    _fields_ = [("tok_emb", C.c_void_p), ("loop_emb", C.c_void_p), ("final_norm", C.c_void_p),
                ("layers", C.POINTER(lk_layer_weights))]


class lk_store_view(C.Structure):
    _fields_ = [("dense", C.c_void_p), ("loop_rows", C.c_void_p), ("base_codes", C.c_void_p),
                ("base_scales", C.c_void_p), ("res_codes", C.c_void_p), ("res_scales", C.c_void_p),
                ("slot_maps", C.c_void_p), ("columns", C.c_void_p), ("slots", C.c_int64),
                ("n_selected", C.c_int32), ("n_columns", C.c_int32), ("res_row_bytes", C.c_int64),
                ("row_stride", C.c_int32), ("decode_cache", C.c_void_p), ("cache_rows", C.c_int32),
                ("ring_rows", C.c_int32), ("first_cached_loop", C.c_int32)]


class lk_dbg_attn_args(C.Structure):
    _fields_ = [("kind", C.c_int32), ("B", C.c_int32), ("H", C.c_int32), ("Hkv", C.c_int32), ("hd", C.c_int32),
                ("kv_format", C.c_int32), ("t", C.c_int32), ("T", C.c_int32), ("tmax", C.c_int32),
                ("q", C.c_void_p), ("q_half", C.c_int32), ("k", C.c_void_p), ("v", C.c_void_p),
                ("k_scales", C.c_void_p), ("v_scales", C.c_void_p), ("cols", C.c_void_p),
                ("n_cols", C.c_int32), ("window", C.c_int32), ("s_k", C.c_void_p), ("s_v", C.c_void_p),
                ("s_cap", C.c_int32), ("r_k", C.c_void_p), ("r_v", C.c_void_p), ("r_cap", C.c_int32),
                ("qpos", C.c_void_p), ("n_rows", C.c_int32), ("out", C.c_void_p), ("out32", C.c_void_p),
                ("lse", C.c_void_p), ("mass", C.c_void_p), ("ws", C.c_void_p), ("ws_bytes", C.c_size_t)]


DBG_ATTN = {"decode": 0, "decode_seg": 1, "prefill": 2, "mass": 3, "prefill_sparse": 4}

SNAPSHOT_MAGIC = 0x313050414E534B4C   # bytes "LKSNAP01"
SNAPSHOT_VERSION = 2


class lk_store_snapshot(C.Structure):
    """Header of a store snapshot; the body (the start of the store buffer) follows."""
    _fields_ = [("magic", C.c_uint64), ("header_bytes", C.c_uint32), ("version", C.c_uint32),
                ("cfg", lk_model_cfg), ("lazy", lk_lazy_cfg),
                ("batch", C.c_int32), ("prompt_tokens", C.c_int32), ("max_tokens", C.c_int32),
                ("loops", C.c_int32), ("tokens", C.c_int32), ("prefilled", C.c_int32),
                ("body_bytes", C.c_uint64)]


_SIGS = {
    "lk_create": (C.c_int, [C.POINTER(lk_model_cfg), C.POINTER(lk_lazy_cfg), C.POINTER(lk_weights),
                            C.POINTER(C.c_void_p)]),
    "lk_destroy": (None, [C.c_void_p]),
    "lk_kv_store_alloc": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                    C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p),
                                    C.POINTER(C.c_size_t)]),
    "lk_kv_store_release": (None, [C.c_void_p]),
    "lk_kv_store_bytes_used": (C.c_int, [C.c_void_p, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "lk_kv_store_cache_bytes": (C.c_int, [C.c_void_p, C.POINTER(C.c_size_t)]),
    "lk_kv_store_length": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32)]),
    "lk_kv_store_range_check": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.c_void_p]),
    "lk_kv_store_set_loops": (C.c_int, [C.c_void_p, C.c_int32]),
    "lk_kv_store_export": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.POINTER(C.c_size_t), C.c_void_p]),
    "lk_kv_store_import": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "lk_workspace_bytes": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_size_t)]),
    "lk_looped_prefill": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                    C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "lk_looped_decode_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_size_t, C.c_void_p]),
    "lk_looped_decode_step_static": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "lk_effective_depth": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32)]),
    "lk_last_error": (C.c_char_p, []),
    "lk_kv_store_view": (C.c_int, [C.c_void_p, C.POINTER(lk_store_view)]),
    "lk_kv_store_force_selection": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "lk_kv_store_keep_codes": (C.c_int, [C.c_void_p, C.c_int32]),
    "lk_timing_enable": (C.c_int, [C.c_void_p, C.c_char_p]),
    "lk_timing_sample": (C.c_int, [C.c_void_p, C.c_int32]),
    "lk_set_decode_graphs": (C.c_int, [C.c_void_p, C.c_int32]),
    "lk_decode_weight_bytes": (C.c_int, [C.c_void_p, C.POINTER(C.c_size_t)]),
    "lk_set_decode_weights": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "lk_timing_read": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_double)]),
    "lk_timing_read_class": (C.c_int, [C.c_void_p, C.c_char_p, C.POINTER(C.c_int32), C.POINTER(C.c_double)]),
    "lk_dbg_topk": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "lk_dbg_quantize": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                  C.c_void_p, C.c_void_p]),
    "lk_dbg_delta": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "lk_dbg_gemm": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                              C.c_void_p]),
    "lk_dbg_gemm_epi": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32,
                                  C.c_int32, C.c_int32, C.c_void_p]),
    "lk_dbg_attention": (C.c_int, [C.POINTER(lk_dbg_attn_args), C.POINTER(C.c_size_t), C.c_void_p]),
    "lk_dbg_kv_write": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p,
                                  C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]),
}

EXPORTED = tuple(_SIGS)
_lib = None


def lib() -> C.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with python -m cross_loop_kv_amd.build")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(code: int) -> None:
    if code != LK_OK:
        raise LKError(code, lib().lk_last_error().decode())


def _stream(stream=None) -> Optional[int]:
    """The caller's stream, or torch's current stream (None = the null stream)."""
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream or None
    return stream


# ---- same-name wrappers ----------------------------------------------------------
def lk_create(cfg: lk_model_cfg, lazy: lk_lazy_cfg, weights: lk_weights) -> int:
    h = C.c_void_p()
    _check(lib().lk_create(C.byref(cfg), C.byref(lazy), C.byref(weights), C.byref(h)))
    return h.value


def lk_destroy(h: int) -> None:
    lib().lk_destroy(h)


def lk_kv_store_alloc(h, batch, prompt_tokens, max_tokens, dev_buf=None, buf_bytes=0, stream=None):
    """Returns (store handle or None, need_bytes)."""
    need = C.c_size_t()
    out = C.c_void_p()
    _check(lib().lk_kv_store_alloc(h, batch, prompt_tokens, max_tokens, dev_buf, buf_bytes,
                                   _stream(stream) if dev_buf else None, C.byref(out), C.byref(need)))
    return (out.value if dev_buf else None), need.value


def lk_kv_store_release(s: int) -> None:
    lib().lk_kv_store_release(s)


def lk_kv_store_bytes_used(s: int) -> Tuple[int, int]:
    a, b = C.c_size_t(), C.c_size_t()
    _check(lib().lk_kv_store_bytes_used(s, C.byref(a), C.byref(b)))
    return a.value, b.value


def lk_kv_store_cache_bytes(s: int) -> int:
    n = C.c_size_t()
    _check(lib().lk_kv_store_cache_bytes(s, C.byref(n)))
    return n.value


def lk_kv_store_length(s: int) -> int:
    t = C.c_int32()
    _check(lib().lk_kv_store_length(s, C.byref(t)))
    return t.value


def lk_kv_store_range_check(s: int, clear: bool = False, stream=None) -> bool:
    flag = C.c_int32()
    _check(lib().lk_kv_store_range_check(s, 1 if clear else 0, C.byref(flag), _stream(stream)))
    return bool(flag.value)


def lk_kv_store_set_loops(s: int, n: int) -> None:
    _check(lib().lk_kv_store_set_loops(s, n))


def lk_kv_store_export(s: int, stream=None) -> np.ndarray:
    """The store's snapshot as a host uint8 array (header, then body)."""
    need = C.c_size_t()
    _check(lib().lk_kv_store_export(s, None, 0, C.byref(need), None))
    buf = np.empty(need.value, np.uint8)
    _check(lib().lk_kv_store_export(s, buf.ctypes.data, buf.size, C.byref(need), _stream(stream)))
    return buf


def lk_kv_store_import(s: int, snap: np.ndarray, stream=None) -> None:
    snap = np.ascontiguousarray(snap, dtype=np.uint8)
    _check(lib().lk_kv_store_import(s, snap.ctypes.data, snap.size, _stream(stream)))


def lk_workspace_bytes(h: int, batch: int, tokens: int) -> int:
    n = C.c_size_t()
    _check(lib().lk_workspace_bytes(h, batch, tokens, C.byref(n)))
    return n.value


def lk_looped_prefill(h, s, d_ids, B, T, d_out, d_ws, ws_bytes, stream=None) -> None:
    _check(lib().lk_looped_prefill(h, s, d_ids, B, T, d_out, d_ws, ws_bytes, _stream(stream)))


def lk_looped_decode_step(h, s, d_ids, d_out, d_ws, ws_bytes, stream=None) -> None:
    _check(lib().lk_looped_decode_step(h, s, d_ids, d_out, d_ws, ws_bytes, _stream(stream)))


def lk_looped_decode_step_static(h, s, d_ids, d_out, stream=None) -> None:
    _check(lib().lk_looped_decode_step_static(h, s, d_ids, d_out, _stream(stream)))


def lk_effective_depth(h: int) -> int:
    d = C.c_int32()
    _check(lib().lk_effective_depth(h, C.byref(d)))
    return d.value


def lk_kv_store_view(s: int) -> lk_store_view:
    v = lk_store_view()
    _check(lib().lk_kv_store_view(s, C.byref(v)))
    return v


def lk_kv_store_force_selection(s: int, d_tokens, d_columns) -> None:
    _check(lib().lk_kv_store_force_selection(s, d_tokens, d_columns))


def lk_kv_store_keep_codes(s: int, enable: bool) -> None:
    _check(lib().lk_kv_store_keep_codes(s, 1 if enable else 0))


def lk_set_decode_weights(h: int, d_buf, nbytes: int, stream=None) -> None:
    _check(lib().lk_set_decode_weights(h, d_buf, nbytes, _stream(stream)))


def lk_decode_weight_bytes(h: int) -> int:
    n = C.c_size_t()
    _check(lib().lk_decode_weight_bytes(h, C.byref(n)))
    return n.value


def lk_set_decode_graphs(h: int, enable: bool) -> None:
    _check(lib().lk_set_decode_graphs(h, 1 if enable else 0))


def lk_timing_sample(h: int, per_call: int) -> None:
    _check(lib().lk_timing_sample(h, per_call))


def lk_timing_enable(h: int, kernel_class: Optional[str]) -> None:
    _check(lib().lk_timing_enable(h, kernel_class.encode() if kernel_class else None))


def lk_timing_read(h: int) -> Tuple[int, float]:
    n, ms = C.c_int32(), C.c_double()
    _check(lib().lk_timing_read(h, C.byref(n), C.byref(ms)))
    return n.value, ms.value


def lk_timing_read_class(h: int, kernel_class: str) -> Tuple[int, float]:
    n, ms = C.c_int32(), C.c_double()
    _check(lib().lk_timing_read_class(h, kernel_class.encode(), C.byref(n), C.byref(ms)))
    return n.value, ms.value


def lk_dbg_topk(d_keys, rows, cols, n, d_idx, stream=None) -> None:
    _check(lib().lk_dbg_topk(d_keys, rows, cols, n, d_idx, _stream(stream)))


def lk_dbg_quantize(d_x, rows, hd, bits, d_codes, d_scales, stream=None) -> None:
    _check(lib().lk_dbg_quantize(d_x, rows, hd, bits, d_codes, d_scales, _stream(stream)))


def lk_dbg_delta(d_a, d_b, rows, d, d_key, stream=None) -> None:
    _check(lib().lk_dbg_delta(d_a, d_b, rows, d, d_key, _stream(stream)))


def lk_dbg_gemm(d_a, d_w, d_c, M, N, K, stream=None) -> None:
    _check(lib().lk_dbg_gemm(d_a, d_w, d_c, M, N, K, _stream(stream)))


def lk_dbg_gemm_epi(d_a, d_w, epi, d_c, d_out, M, N, K, stream=None) -> None:
    _check(lib().lk_dbg_gemm_epi(d_a, d_w, epi, d_c, d_out, M, N, K, _stream(stream)))


def lk_dbg_attention(args: lk_dbg_attn_args, stream=None) -> int:
    """Runs the kind's kernels (args.ws set) or returns the workspace bytes it needs
    (args.ws None)."""
    need = C.c_size_t()
    _check(lib().lk_dbg_attention(C.byref(args), C.byref(need), _stream(stream)))
    return need.value


def lk_dbg_kv_write(s, layer, loop, d_qkv, rows_per_seq, d_pos, d_q_out, q_half, d_ws=None, ws_bytes=0,
                    stream=None) -> None:
    _check(lib().lk_dbg_kv_write(s, layer, loop, d_qkv, rows_per_seq, d_pos, d_q_out, 1 if q_half else 0,
                                 d_ws, ws_bytes, _stream(stream)))


# ---- model / store objects (device memory from torch) ----------------------------------
def model_cfg(shape) -> lk_model_cfg:
    return lk_model_cfg(shape.vocab, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                        shape.ffn_dim, ACTS[shape.ffn_act], shape.n_prelude, shape.n_shared,
                        shape.n_loops, shape.n_coda, shape.rms_eps, shape.rope_theta,
                        int(getattr(shape, "input_reinject", False)))


def lazy_cfg(lz) -> lk_lazy_cfg:
    return lk_lazy_cfg(MODES[lz.mode], float(lz.rho), int(lz.top_s), int(lz.window),
                       int(lz.base_bits), int(lz.res_bits), int(lz.group), int(getattr(lz, "stale_keys", False)),
                       int(getattr(lz, "refresh_every", 0)), int(getattr(lz, "diff_attn", False)),
                       float(getattr(lz, "skip_tau", 0.0)))


def _aligned_bytes(nbytes: int, device):
    """A torch uint8 buffer of at least nbytes whose data pointer is 256-byte aligned."""
    import torch
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf, buf[off:off + nbytes]


class Store:
    def __init__(self, model: "LoopedModel", batch: int, prompt: int, max_tokens: int):
        self.model = model
        self.batch, self.prompt, self.max_tokens = batch, prompt, max_tokens
        _, need = lk_kv_store_alloc(model.h, batch, prompt, max_tokens)
        self._raw, self.buf = _aligned_bytes(max(need, 256), model.device)
        self.need = need
        self.s, _ = lk_kv_store_alloc(model.h, batch, prompt, max_tokens, self.buf.data_ptr(), need)

    def view(self) -> lk_store_view:
        return lk_kv_store_view(self.s)

    def bytes_used(self) -> Tuple[int, int]:
        return lk_kv_store_bytes_used(self.s)

    def length(self) -> int:
        return lk_kv_store_length(self.s)

    def out_of_f16_range(self, clear: bool = False) -> bool:
        """Whether the writer met a q/K/V element outside the float16 range."""
        return lk_kv_store_range_check(self.s, clear)

    def export(self) -> np.ndarray:
        """Snapshot of the store's state (host uint8 array)."""
        return lk_kv_store_export(self.s)

    def import_(self, snap: np.ndarray):
        """Replace the store's state with a snapshot (see lk_kv_store_import)."""
        lk_kv_store_import(self.s, snap)
        self.loops = lk_store_snapshot.from_buffer_copy(bytes(snap[:C.sizeof(lk_store_snapshot)])).loops

    def set_loops(self, n: int):
        """Loop count for the next prefill and its decode steps (1..the model's K)."""
        lk_kv_store_set_loops(self.s, n)
        self.loops = n

    def cache_bytes(self) -> int:
        return lk_kv_store_cache_bytes(self.s)

    def force_selection(self, tokens=None, columns=None):
        """tokens: int32 cuda [K-1, B, n]; columns: int32 cuda [R, B, Hkv, n_cols] (or None)."""
        self._forced = (tokens, columns)
        lk_kv_store_force_selection(self.s, tokens.data_ptr() if tokens is not None else None,
                                    columns.data_ptr() if columns is not None else None)

    def keep_codes(self, enable: bool = True):
        lk_kv_store_keep_codes(self.s, enable)

    def close(self):
        if getattr(self, "s", None):
            lk_kv_store_release(self.s)
            self.s = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LoopedModel:
    """Weights on the GPU in the library's packed bf16 layout plus a handle.

    Every prefill and decode call of a model uses the model's one workspace buffer, on
    the caller's current stream: calls issued on different streams must be ordered by
    the caller (torch's side streams do not wait for the null stream)."""

    def __init__(self, shape, lazy, weights: Iterable, device: str = "cuda"):
        import torch
        self.shape, self.lazy, self.device = shape, lazy, device
        bf = torch.bfloat16

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=torch.float32).to(bf)

        self.t: Dict = {}
        layers: Dict[int, Dict] = {}
        items = weights.items() if isinstance(weights, dict) else None
        if items is not None and "layers" in weights:
            self.t["tok_emb"] = dev(weights["tok_emb"])
            self.t["loop_emb"] = dev(weights["loop_emb"])
            self.t["final_norm"] = dev(weights["final_norm"])
            src_layers = list(enumerate(weights["layers"]))
        else:
            src_layers = []
            ones = np.ones(shape.d_model, np.float32)
            for name, li, arr in weights:
                if li < 0:
                    self.t[name] = dev(arr)
                else:
                    layers.setdefault(li, {"attn_norm": ones, "ffn_norm": ones})[name] = arr
                    if name == "w_down":
                        src_layers.append((li, layers.pop(li)))
            self.t["final_norm"] = dev(ones)
        self.layers = []
        for li, L in src_layers:
            packed = {
                "attn_norm": dev(L["attn_norm"]), "ffn_norm": dev(L["ffn_norm"]),
                "wqkv": torch.cat([dev(L["wq"]), dev(L["wk"]), dev(L["wv"])], 0).contiguous(),
                "wo": dev(L["wo"]),
                "w_in": (torch.cat([dev(L["w_gate"]), dev(L["w_up"])], 0).contiguous()
                         if shape.ffn_act == "swiglu" else dev(L["w_up"])),
                "w_down": dev(L["w_down"]),
            }
            self.layers.append(packed)
        n = len(self.layers)
        assert n == shape.n_prelude + shape.n_shared + shape.n_coda, "layer count mismatch"
        self._lw = (lk_layer_weights * n)()
        for i, L in enumerate(self.layers):
            self._lw[i] = lk_layer_weights(L["attn_norm"].data_ptr(), L["wqkv"].data_ptr(),
                                           L["wo"].data_ptr(), L["ffn_norm"].data_ptr(),
                                           L["w_in"].data_ptr(), L["w_down"].data_ptr())
        self._w = lk_weights(self.t["tok_emb"].data_ptr(), self.t["loop_emb"].data_ptr(),
                             self.t["final_norm"].data_ptr(), self._lw)
        self._cfg = model_cfg(shape)
        self._lz = lazy_cfg(lazy)
        self.h = lk_create(self._cfg, self._lz, self._w)
        self._ws = None
        self._ws_bytes = 0
        self._pk = None
        self.pack_decode_weights(True)

    def pack_decode_weights(self, enable: bool = True, share=None) -> None:
        """Give the handle the packed decode copy of the weights (a device buffer owned
        here, or `share`'s), or detach it (decode then uses the row-major weights)."""
        if not enable:
            lk_set_decode_weights(self.h, None, 0)
            self._pk = None
            return
        nbytes = lk_decode_weight_bytes(self.h)
        if nbytes == 0:
            return
        if share is not None and share._pk is not None:
            self._pk = share._pk
        elif self._pk is None:
            self._pk = _aligned_bytes(nbytes, self.device)
        lk_set_decode_weights(self.h, self._pk[1].data_ptr(), nbytes)

    def sibling(self, lazy) -> "LoopedModel":
        """A second handle over the same device weights with another lazy configuration
        (e.g. the dense per-loop reference of a lazy model).  Keeps this model alive."""
        m = object.__new__(LoopedModel)
        m.shape, m.lazy, m.device = self.shape, lazy, self.device
        m.t, m.layers, m._lw, m._w, m._cfg = self.t, self.layers, self._lw, self._w, self._cfg
        m._parent = self
        m._lz = lazy_cfg(lazy)
        m.h = lk_create(m._cfg, m._lz, m._w)
        m._ws = None
        m._ws_bytes = 0
        m._pk = None
        m.pack_decode_weights(True, share=self)
        return m

    def weight_bytes(self) -> int:
        tot = sum(t.numel() * t.element_size() for t in self.t.values())
        for L in self.layers:
            tot += sum(t.numel() * t.element_size() for t in L.values())
        return tot

    def effective_depth(self) -> int:
        return lk_effective_depth(self.h)

    def workspace(self, batch: int, tokens: int):
        need = lk_workspace_bytes(self.h, batch, tokens)
        if self._ws is None or self._ws_bytes < need:
            self._ws = None
            self._ws_raw, self._ws = _aligned_bytes(need, self.device)
            self._ws_bytes = need
        return self._ws, need

    def store(self, batch: int, prompt: int, max_tokens: int, loops: Optional[int] = None) -> Store:
        st = Store(self, batch, prompt, max_tokens)
        if loops is not None:
            st.set_loops(loops)
        return st

    def prefill(self, store: Store, ids, out=None):
        import torch
        B, T = ids.shape
        ids = ids.to(device=self.device, dtype=torch.int32).contiguous()
        if out is None:
            out = torch.empty(B, T, self.shape.d_model, dtype=torch.float32, device=self.device)
        ws, nbytes = self.workspace(B, T)
        lk_looped_prefill(self.h, store.s, ids.data_ptr(), B, T, out.data_ptr(), ws.data_ptr(), nbytes)
        return out

    def decode(self, store: Store, ids, out=None):
        import torch
        ids = ids.to(device=self.device, dtype=torch.int32).contiguous().view(-1)
        B = ids.shape[0]
        if out is None:
            out = torch.empty(B, self.shape.d_model, dtype=torch.float32, device=self.device)
        ws, nbytes = self.workspace(B, 1)
        lk_looped_decode_step(self.h, store.s, ids.data_ptr(), out.data_ptr(), ws.data_ptr(), nbytes)
        return out

    def close(self):
        if getattr(self, "h", None):
            lk_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
