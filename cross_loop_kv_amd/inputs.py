"""Seeded synthetic inputs for looped-Transformer inference.

This module only *generates* inputs: weight tensors, token ids and the named
workload shapes.  It holds none of the method's arithmetic, so both the HIP
path and the CPU oracle may take their inputs from here.

Conventions (fixed so that both sides see identical tensors):

* weights: ``numpy.random.default_rng(seed)``, ``standard_normal(float32) * 0.02``
  drawn tensor by tensor in this order: token embedding, then for every layer
  (prelude layers, shared-block layers, coda layers) q, k, v, o, gate (SwiGLU
  only), up, down, then the loop-embedding table.  Norm gains are ones.  Every
  weight is then rounded to bfloat16 (round to nearest even) and kept as the
  float32 value of that bfloat16, because the GPU path stores its weights in
  bfloat16 and both sides must start from the same numbers.
* prompt ids: seed 1, uniform on [0, vocab); decode ids: seed 2.

The model structure (P prelude layers, R shared layers applied K times, Q coda
layers; effective depth P + R*K + Q) is the sandwich layout of the FlashLoop
walk-through (discosf.com FlashLoop article, section 3.1).
"""
from __future__ import annotations

import copy
from dataclasses import dataclass, field, asdict
from typing import Dict, Iterator, List, Tuple

import numpy as np

WEIGHT_STD = 0.02
SEED_WEIGHTS = 0
SEED_PROMPT = 1
SEED_DECODE = 2


@dataclass
class Shape:
    """Model shape of a looped Transformer (sandwich P + R x K + Q)."""
    vocab: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    ffn_act: str            # "gelu" (exact erf) or "swiglu"
    n_prelude: int
    n_shared: int
    n_loops: int
    n_coda: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    input_reinject: bool = False  # the prelude output is fed into every loop k >= 2

    @property
    def n_layers_stored(self) -> int:
        return self.n_prelude + self.n_shared + self.n_coda


@dataclass
class Lazy:
    """Inference-time cache/update policy."""
    mode: str = "lazy"      # "per_loop" | "last_loop" | "lazy"
    rho: float = 1.0        # kept-token fraction at loops k >= 2
    top_s: int = 0          # stable key columns
    window: int = 1         # recent-window length (>= 1)
    base_bits: int = 16     # loop-1 KV: 16 (working precision) or 8 (int8, group 32)
    res_bits: int = 16      # loop-k residual: 16, 8 or 4
    group: int = 32
    stale_keys: bool = False  # carried tokens keep their last measured change (else 0)
    refresh_every: int = 0    # p > 0: loops k >= 2 with (k - 1) % p == 0 recompute every token
    diff_attn: bool = False   # loops k >= 2: sparse term plus the row's loop-1 (dense - sparse)
    skip_tau: float = 0.0     # decode: a token leaves the loops once its state change is below this


@dataclass
class Workload:
    name: str
    shape: Shape
    lazy: Lazy
    batch: int
    prompt: int
    decode_steps: int
    dtype: str              # nominal model precision of the workload
    note: str = ""

    def replace(self, **kw) -> "Workload":
        w = copy.deepcopy(self)
        for k, v in kw.items():
            if hasattr(w.shape, k):
                setattr(w.shape, k, v)
            elif hasattr(w.lazy, k):
                setattr(w.lazy, k, v)
            else:
                setattr(w, k, v)
        return w


def _swiglu(vocab, d, h, hkv, f, p, r, k, q):
    return Shape(vocab=vocab, d_model=d, n_heads=h, n_kv_heads=hkv, head_dim=128,
                 ffn_dim=f, ffn_act="swiglu", n_prelude=p, n_shared=r, n_loops=k, n_coda=q)


# Named workloads.  Vocab 32000 where none is given, MHA where GQA is not given.
WORKLOADS: Dict[str, Workload] = {
    "tiny_1p2x2c1_t32": Workload(
        name="tiny_1p2x2c1_t32",
        shape=Shape(vocab=256, d_model=64, n_heads=2, n_kv_heads=2, head_dim=32, ffn_dim=256,
                    ffn_act="gelu", n_prelude=1, n_shared=2, n_loops=2, n_coda=1),
        lazy=Lazy(mode="lazy", rho=0.5, top_s=8, window=4, base_bits=16, res_bits=8),
        batch=1, prompt=32, decode_steps=8, dtype="fp32"),
    "prefill_2p4x4c2_b4_t4096": Workload(
        name="prefill_2p4x4c2_b4_t4096",
        shape=_swiglu(32000, 2048, 16, 16, 5632, 2, 4, 4, 2),
        lazy=Lazy(mode="lazy", rho=0.25, top_s=256, window=128, base_bits=16, res_bits=4),
        batch=4, prompt=4096, decode_steps=0, dtype="bf16"),
    "twopass_22x2_b16_ctx8k": Workload(
        name="twopass_22x2_b16_ctx8k",
        shape=_swiglu(32000, 2048, 16, 4, 5632, 0, 22, 2, 0),
        lazy=Lazy(mode="lazy", rho=0.2, top_s=512, window=256, base_bits=16, res_bits=4),
        batch=16, prompt=8192, decode_steps=512, dtype="bf16"),
    "deep_48x4_b8_ctx32k": Workload(
        name="deep_48x4_b8_ctx32k",
        shape=_swiglu(32000, 2048, 16, 4, 5632, 0, 48, 4, 0),
        lazy=Lazy(mode="lazy", rho=0.1, top_s=1024, window=512, base_bits=8, res_bits=4),
        batch=8, prompt=32768, decode_steps=256, dtype="bf16"),
    "long_4p8x8c4_ctx64k": Workload(
        name="long_4p8x8c4_ctx64k",
        shape=_swiglu(32000, 4096, 32, 8, 11008, 4, 8, 8, 4),
        lazy=Lazy(mode="lazy", rho=0.1, top_s=2048, window=1024, base_bits=16, res_bits=4),
        batch=1, prompt=65536, decode_steps=256, dtype="bf16"),
}


def workload(name: str) -> Workload:
    return copy.deepcopy(WORKLOADS[name])


# ----------------------------------------------------------------------------
# bfloat16 helpers (input preparation only)
# ----------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 result."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bfloat16-representable float32 values (the bf16 encoding)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# Weights
# ----------------------------------------------------------------------------

def layer_tensor_shapes(s: Shape) -> List[Tuple[str, Tuple[int, int]]]:
    hd = s.head_dim
    out = [("wq", (s.n_heads * hd, s.d_model)),
           ("wk", (s.n_kv_heads * hd, s.d_model)),
           ("wv", (s.n_kv_heads * hd, s.d_model)),
           ("wo", (s.d_model, s.n_heads * hd))]
    if s.ffn_act == "swiglu":
        out.append(("w_gate", (s.ffn_dim, s.d_model)))
    out.append(("w_up", (s.ffn_dim, s.d_model)))
    out.append(("w_down", (s.d_model, s.ffn_dim)))
    return out


def iter_weights(s: Shape, seed: int = SEED_WEIGHTS, bf16: bool = True
                 ) -> Iterator[Tuple[str, int, np.ndarray]]:
    """Yield (name, layer_index or -1, float32 array) in the fixed draw order."""
    rng = np.random.default_rng(seed)

    def draw(shape):
        a = rng.standard_normal(shape, dtype=np.float32)
        a *= np.float32(WEIGHT_STD)
        return round_to_bf16(a) if bf16 else a

    yield "tok_emb", -1, draw((s.vocab, s.d_model))
    for li in range(s.n_layers_stored):
        for name, shp in layer_tensor_shapes(s):
            yield name, li, draw(shp)
    yield "loop_emb", -1, draw((s.n_loops, s.d_model))


def gen_weights(s: Shape, seed: int = SEED_WEIGHTS, bf16: bool = True) -> Dict:
    """All weights as a nested dict of float32 numpy arrays.

    ``{"tok_emb", "loop_emb", "final_norm", "layers": [ {attn_norm, wq, wk, wv, wo,
    ffn_norm, [w_gate], w_up, w_down}, ... ]}`` with layers ordered prelude,
    shared block, coda.
    """
    layers = [dict(attn_norm=np.ones(s.d_model, np.float32),
                   ffn_norm=np.ones(s.d_model, np.float32))
              for _ in range(s.n_layers_stored)]
    w: Dict = {"layers": layers, "final_norm": np.ones(s.d_model, np.float32)}
    for name, li, arr in iter_weights(s, seed, bf16):
        if li < 0:
            w[name] = arr
        else:
            layers[li][name] = arr
    return w


def gen_prompt_ids(s: Shape, batch: int, tokens: int, seed: int = SEED_PROMPT) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, s.vocab, size=(batch, tokens), dtype=np.int64).astype(np.int32)


def gen_decode_ids(s: Shape, batch: int, steps: int, seed: int = SEED_DECODE) -> np.ndarray:
    """[steps, batch] teacher-forced decode tokens."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, s.vocab, size=(steps, batch), dtype=np.int64).astype(np.int32)


def shape_dict(s: Shape) -> dict:
    return asdict(s)
