"""Independent float64 reference Transformer built from PyTorch library routines.

Used only to pin the oracle: ``torch.nn.functional.rms_norm``,
``scaled_dot_product_attention`` (causal or with an explicit boolean mask),
``silu`` / ``gelu`` and rotary embedding written as complex multiplication
(the textbook form of RoPE: the pair (x_i, x_{i+hd/2}) is the complex number
x_i + j x_{i+hd/2}, multiplied by exp(j * pos * theta^(-2i/hd))).
"""
import numpy as np
import torch
import torch.nn.functional as F

D = torch.float64


def _t(a):
    return torch.as_tensor(np.asarray(a), dtype=D)


def rope_complex(x, pos, theta):
    """x [T, heads, hd] -> rotated, via complex multiplication."""
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=D) / hd)
    ang = torch.as_tensor(pos, dtype=D)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def layer(W, x, shape, mask=None):
    """One pre-norm layer on a full sequence x [T, d] (causal unless mask given)."""
    T = x.shape[0]
    H, Hkv, hd = shape.n_heads, shape.n_kv_heads, shape.head_dim
    a = F.rms_norm(x, (x.shape[-1],), weight=_t(W["attn_norm"]), eps=shape.rms_eps)
    q = (a @ _t(W["wq"]).T).view(T, H, hd)
    k = (a @ _t(W["wk"]).T).view(T, Hkv, hd)
    v = (a @ _t(W["wv"]).T).view(T, Hkv, hd)
    pos = np.arange(T)
    q = rope_complex(q, pos, shape.rope_theta)
    k = rope_complex(k, pos, shape.rope_theta)
    rep = H // Hkv
    k = k.repeat_interleave(rep, dim=1)
    v = v.repeat_interleave(rep, dim=1)
    if mask is None:
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                           is_causal=True)
    else:
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                           attn_mask=mask)
    o = o.transpose(0, 1).reshape(T, H * hd)
    x = x + o @ _t(W["wo"]).T
    b = F.rms_norm(x, (x.shape[-1],), weight=_t(W["ffn_norm"]), eps=shape.rms_eps)
    if shape.ffn_act == "swiglu":
        f = F.silu(b @ _t(W["w_gate"]).T) * (b @ _t(W["w_up"]).T)
    else:
        f = F.gelu(b @ _t(W["w_up"]).T, approximate="none")
    return x + f @ _t(W["w_down"]).T


def unrolled_forward(weights, shape, ids, loops=None, loop_emb=True, reinject=False):
    """Standard Transformer over the unrolled weight-tied stack.

    Layer sequence: prelude layers, then for each loop k (with ``reinject``, the
    prelude output is first added back to the state for k >= 2) the loop embedding
    row k-1 is added and the shared layers are applied, then the coda layers, then
    the final RMSNorm.  ``ids`` is one sequence [T]; returns float64 [T, d].
    """
    K = shape.n_loops if loops is None else loops
    L = weights["layers"]
    x = _t(weights["tok_emb"])[torch.as_tensor(np.asarray(ids), dtype=torch.long)]
    P, R = shape.n_prelude, shape.n_shared
    for li in range(P):
        x = layer(L[li], x, shape)
    e = x
    for k in range(K):
        if reinject and k >= 1:
            x = x + e
        if loop_emb:
            x = x + _t(weights["loop_emb"][k])
        for r in range(R):
            x = layer(L[P + r], x, shape)
    for j in range(shape.n_coda):
        x = layer(L[P + R + j], x, shape)
    return F.rms_norm(x, (x.shape[-1],), weight=_t(weights["final_norm"]), eps=shape.rms_eps)
