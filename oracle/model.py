"""Looped-Transformer forward, dense and lazy (oracle; test infrastructure only).

Plain float32 NumPy; each sequence of a batch is processed on its own (the
method couples nothing across sequences).  Sources, by page:

* discosf.com FlashLoop walk-through: sandwich P + R x K + Q and effective
  depth P + R*K + Q (section 3.1); learned loop embedding added to the loop
  input, RoPE inside the block, residual state passing (section 3.2);
  inference flow embed -> prelude -> loop state = prelude output -> for each
  loop add the loop embedding and run the R shared layers -> coda -> head
  (section 4.1); one KV cache per loop, projections shared (section 5.2);
  pre-LN (section 8).
* aiboss88.com tutorial: shared stack kept once outside the loop (step 1);
  per_loop is the default KV mode, last_loop overwrites the previous pass's
  KV in every recurrent attention layer (step 4).
* arxivdaily.com FlashLoop abstract: token-sparse updates, sparse attention
  over a stable subset of key columns, KV-residual quantization.

Readings where the pages leave a step open (the rules of the lazy method are
not given on any page):

* layer: x += Wo . attn(RoPE(Wq a), RoPE(Wk a), Wv a) with a = rmsnorm(x) g1;
  x += FFN(rmsnorm(x) g2); FFN = Wd (silu(Wg b) * Wu b) or W2 gelu_erf(W1 b);
  no biases; RMSNorm eps 1e-5; RoPE rotate-half, theta 1e4; scale 1/sqrt(hd);
  KV head of query head h is h * Hkv // H.  The "output = body(input) +
  input" of the walk-through is the per-layer residual (no extra outer skip).
* loop k adds loop_emb[k-1] to the state, which stays in the residual stream;
  in lazy mode only the recomputed rows receive it.
* lazy loop 1 is dense.  Column mass of KV head g at shared layer r is the sum
  over all prompt queries and over the query heads of g of the loop-1
  softmax probabilities; S = the top_s columns by mass (all columns if
  T <= top_s), reused at every later loop and decode step.
* lazy loop k >= 2: key_i = ||h_{k-1,i} - h_{k-2,i}||^2 (h_0 = prelude output;
  carried rows have key 0, or with ``lazy.stale_keys`` keep the key they had at
  loop k-1, i.e. the change measured when they were last recomputed); the n
  largest keys are recomputed, the rest carry forward unchanged.  A recomputed query i attends over
  (S intersect [0, i]) union [max(0, i-w+1), i] of the loop-k reconstruction.
* difference-corrected sparse attention (``lazy.diff_attn``; the FlashLoop abstract,
  arxivdaily.com: the attention-output *differences* between loops come from a sparse,
  stable set of key columns): a recomputed row's attention output at loop k >= 2 is its
  previous output plus the change of its sparse term, o_k = o_{k'} + (a_k - a_{k'}),
  where a_j is the softmax over the row's sparse column set of loop j's query and
  reconstruction and k' the loop that last computed the row.  Since loop 1 computes
  every row densely, o_k = a_k + (o_1 - a_1) exactly: the oracle keeps D = o_1 - a_1
  per (shared layer, token) from loop 1 and adds it to the sparse output.  A decode
  token's D comes from its own loop 1 (dense output minus the sparse one over the
  loop-1 reconstruction).  Off, o_k = a_k.
* decode-time loop skipping (``lazy.skip_tau`` = tau > 0; the FlashLoop abstract: state
  changes concentrate on fewer tokens as the loops proceed, carried into decode): a
  decode token enters loop k >= 2 only if the squared change of its state over loop
  k-1, ||h_{k-1} - h_{k-2}||^2 (the selection key; h_0 = the prelude output), is at
  least tau.  Otherwise it leaves the loops with the state h_{k-1}, which goes to the
  coda; it stores no row for loops k..K, so its loop-j reconstruction stays its
  loop-(k-1) one (the lazy store's rule for carried rows).  tau = 0: never skipped.
* periodic refresh (``lazy.refresh_every`` = p > 0): a loop k >= 2 with (k - 1) % p
  == 0 recomputes every token instead of the top n (the token set is refreshed; the
  attention stays the sparse one and the residual rows are stored for every token).
* input re-injection (aiboss88.com tutorial, step 3: a structure that passes the
  input representation into every loop): with ``shape.input_reinject`` the prelude
  output e is added to the state before every loop k >= 2 (loop 1 starts from e), as
  (state + e) + loop_emb[k-1]; in lazy mode only the recomputed rows receive it, like
  the loop embedding.
* loop count (aiboss88.com tutorial, step 3: n_recurrent_loops picked by the caller
  with the same checkpoint): ``n_loops`` (default shape.n_loops) runs loops 1..n_loops
  of a store laid out for shape.n_loops loops; prefill and decode use the same count.
* KV store: loop 1 is the base (working precision, or int8 groups with a zero
  previous reconstruction); loop k >= 2 stores, for recomputed rows only,
  r = KV_k - recon_{k-1} quantized (16 bits: the full KV_k row instead), so
  recon_k = recon_{k-1} + dequant(r) on those rows and recon_{k-1} elsewhere.
  Residual rows live in compact slots addressed by a per-(loop, sequence) slot
  map.  A decode token runs every loop and is always stored.

Every tensor is float32; the GPU path's own roundings are its business and are
held to the parity bound by the tests, not modelled here.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf

from . import quant
from .select import n_selected, top_n_ascending

F32 = np.float32


# ----------------------------------------------------------------------------
# Building blocks
# ----------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=F32)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    return (x / np.sqrt(ms + F32(eps))) * gain


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float):
    """Rotary angles computed in float64, returned as float32 [n, hd/2]."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on x [n, heads, hd] with cos/sin [n, hd/2]."""
    half = x.shape[-1] // 2
    x1 = x[..., :half]
    x2 = x[..., half:]
    c = cos[:, None, :]
    s = sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1).astype(F32)


def gelu_erf(x: np.ndarray) -> np.ndarray:
    return (F32(0.5) * x * (F32(1.0) + _erf(x / F32(np.sqrt(2.0))).astype(F32))).astype(F32)


def silu(x: np.ndarray) -> np.ndarray:
    return (x / (F32(1.0) + np.exp(-x))).astype(F32)


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, cols_of, mass=None):
    """Softmax attention of each query row over its own key columns.

    q [n, H, hd]; keys/vals [Hkv, Tc, hd]; ``cols_of(i, g)`` gives the ascending
    key positions that row i attends to through KV head g.  Query head h reads
    KV head h // (H // Hkv).  If ``mass`` [Hkv, Tc] is given, each row's
    probabilities, summed over the query heads of each KV head, are added to it.
    """
    n, H, hd = q.shape
    Hkv = keys.shape[0]
    G = H // Hkv
    scale = F32(1.0 / np.sqrt(hd))
    out = np.empty((n, H, hd), dtype=F32)
    for i in range(n):
        for g in range(Hkv):
            cols = cols_of(i, g)
            kk = keys[g, cols, :]                      # [c, hd]
            vv = vals[g, cols, :]
            s = (q[i, g * G:(g + 1) * G] @ kk.T) * scale   # [G, c]
            m = np.max(s, axis=-1, keepdims=True)
            p = np.exp(s - m)
            p = p / np.sum(p, axis=-1, keepdims=True, dtype=F32)
            out[i, g * G:(g + 1) * G] = p @ vv
            if mass is not None:
                mass[g, cols] += np.sum(p, axis=0, dtype=F32)
    return out


def attend_masked(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, pos: np.ndarray, allowed,
                  mass=None, block: int = 256):
    """``attend`` written as a masked softmax: query row i (at position pos[i], pos
    ascending) over the key columns c <= max(pos) with ``allowed(p, c, g)`` true,
    where p is a block of row positions [nb], c the column indices [nc] and the
    result a boolean [nb, nc] (the row's column set as a mask; columns outside it
    get score -inf, so probability 0).  Rows are taken ``block`` at a time as one
    score matrix per KV head; per row this is the same softmax and products as
    ``attend`` over the gathered columns, up to the summation order inside the
    matrix products.  The block arithmetic runs as float32 PyTorch CPU operations
    (multithreaded), which is what makes a 32k-token prompt affordable.  ``mass`` as
    in ``attend``."""
    import torch
    n, H, hd = q.shape
    Hkv = keys.shape[0]
    G = H // Hkv
    pos = np.asarray(pos, np.int64)
    scale = float(F32(1.0 / np.sqrt(hd)))
    out = np.empty((n, H, hd), dtype=F32)
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=F32))
    kt = torch.from_numpy(np.ascontiguousarray(keys, dtype=F32))
    vt = torch.from_numpy(np.ascontiguousarray(vals, dtype=F32))
    for g in range(Hkv):
        for i0 in range(0, n, block):
            i1 = min(n, i0 + block)
            pb = pos[i0:i1]
            nc = int(pb[-1]) + 1
            ok = torch.from_numpy(np.ascontiguousarray(allowed(pb, np.arange(nc), g)))   # [nb, nc]
            qb = qt[i0:i1, g * G:(g + 1) * G, :].reshape(-1, hd)                        # [nb*G, hd]
            sc = (qb @ kt[g, :nc, :].T) * scale
            sc = sc.view(i1 - i0, G, nc).masked_fill(~ok[:, None, :], float("-inf"))
            m = sc.amax(dim=-1, keepdim=True)
            p = torch.exp(sc - m)
            p = p / p.sum(dim=-1, keepdim=True)
            out[i0:i1, g * G:(g + 1) * G] = (p.view(-1, nc) @ vt[g, :nc, :]).view(i1 - i0, G, hd).numpy()
            if mass is not None:
                mass[g, :nc] += p.sum(dim=(0, 1)).numpy()
    return out


def causal_mask(p: np.ndarray, c: np.ndarray, g: int) -> np.ndarray:
    """Column c is visible from position p when c <= p."""
    return c[None, :] <= p[:, None]


def sparse_mask(S: np.ndarray, window: int):
    """Mask form of ``sparse_cols``: (S intersect [0, p]) union [p - window + 1, p]."""
    def allowed(p, c, g):
        inS = np.zeros(c.shape[0], bool)
        s_g = S[g]
        inS[s_g[s_g < c.shape[0]]] = True
        return (c[None, :] <= p[:, None]) & (inS[None, :] | (c[None, :] > p[:, None] - window))
    return allowed


def causal_cols(i: int) -> np.ndarray:
    return np.arange(i + 1)


def sparse_cols(i: int, S: np.ndarray, window: int) -> np.ndarray:
    """(S intersect [0, i]) union [max(0, i - window + 1), i], ascending, no duplicates."""
    lo = max(0, i - window + 1)
    return np.union1d(S[S <= i], np.arange(lo, i + 1))


# ----------------------------------------------------------------------------
# Model
# ----------------------------------------------------------------------------

class LoopedOracle:
    """Looped Transformer with a per_loop, last_loop or lazy KV store.

    ``prefill(ids[B, T])`` returns the final-normed hidden states [B, T, d];
    ``decode(ids[B])`` appends one token per sequence and returns [B, d].
    """

    def __init__(self, shape, lazy, weights, batch: int, max_tokens: int, n_loops=None):
        self.K = shape.n_loops if n_loops is None else int(n_loops)
        if not 1 <= self.K <= shape.n_loops:
            raise ValueError("n_loops must be in [1, shape.n_loops]")
        self.inject = bool(getattr(shape, "input_reinject", False))
        self.s = shape
        self.lz = lazy
        self.w = weights
        self.B = batch
        self.Tmax = max_tokens
        if lazy.mode not in ("per_loop", "last_loop", "lazy"):
            raise ValueError("mode must be per_loop, last_loop or lazy")
        if shape.n_heads % shape.n_kv_heads:
            raise ValueError("n_heads must be a multiple of n_kv_heads")
        if lazy.mode == "lazy":
            if lazy.window < 1:
                raise ValueError("window must be >= 1")
            if lazy.base_bits not in (16, 8) or lazy.res_bits not in (16, 8, 4):
                raise ValueError("unsupported bit width")
            if shape.head_dim % lazy.group:
                raise ValueError("head_dim must be a multiple of the group")
            if int(getattr(lazy, "refresh_every", 0)) < 0:
                raise ValueError("refresh_every must be >= 0")
        self.diff = lazy.mode == "lazy" and bool(getattr(lazy, "diff_attn", False))
        self.tau = F32(getattr(lazy, "skip_tau", 0.0)) if lazy.mode == "lazy" else F32(0)
        if self.tau < 0:
            raise ValueError("skip_tau must be >= 0")
        self.decode_keys = {}        # (k, b, t) -> a decode token's key at loop k >= 2
        self.decode_loops = {}       # (b, t) -> loops a decode token ran
        self.D = {}                  # diff_attn: (r, b) -> o_1 - a_1 [T, H, hd] of the prompt
        self.depth = 0           # layer applications in the last call
        self.forced_codes_from = None  # another LoopedOracle whose quantized codes are reused
        self.forced_tokens = None    # {(k, b): kept indices} overrides selection
        self.forced_S = None         # [r][b][g] column lists override top-s
        self.mass = {}               # (r, b) -> loop-1 column mass [Hkv, T]
        self.keys = {}               # (k, b) -> delta keys [T]
        self.T = None            # prompt length
        self.t = 0               # tokens held per sequence
        self._alloc()

    # ---------------------------------------------------------------- store
    def _alloc(self):
        s, B, Tm = self.s, self.B, self.Tmax
        Hkv, hd = s.n_kv_heads, s.head_dim
        kv = lambda: np.zeros((B, Hkv, Tm, hd), F32)
        self.dense_k = [kv() for _ in range(s.n_prelude + s.n_coda)]
        self.dense_v = [kv() for _ in range(s.n_prelude + s.n_coda)]
        R, K = s.n_shared, s.n_loops
        if self.lz.mode == "per_loop":
            self.loop_k = [[kv() for _ in range(R)] for _ in range(K)]
            self.loop_v = [[kv() for _ in range(R)] for _ in range(K)]
        elif self.lz.mode == "last_loop":
            self.last_k = [kv() for _ in range(R)]
            self.last_v = [kv() for _ in range(R)]
        else:
            ng = hd // self.lz.group
            if self.lz.base_bits == 16:
                self.base = [[kv(), kv()] for _ in range(R)]          # [r][K/V] fp32
            else:
                self.base = [[(np.zeros((B, Hkv, Tm, hd), np.int8),
                               np.zeros((B, Hkv, Tm, ng), np.float16)) for _ in range(2)]
                             for _ in range(R)]
            self.slot = np.full((K, B, Tm), -1, np.int32)   # slot[k-1]; k = 2..K used
            self.res = None          # allocated at prefill (needs the slot count)
            self.S = None            # [R][B][Hkv] arrays of columns
            self.sel = {}            # (k, b) -> kept indices at loop k

    def _alloc_residuals(self, n_slots: int):
        s, B = self.s, self.B
        Hkv, hd, R, K = s.n_kv_heads, s.head_dim, s.n_shared, s.n_loops
        ng = hd // self.lz.group
        self.n_slots = n_slots
        self.res = {}
        for k in range(2, K + 1):
            for r in range(R):
                for kv in range(2):
                    if self.lz.res_bits == 16:
                        self.res[(k, r, kv)] = np.zeros((B, Hkv, n_slots, hd), F32)
                    else:
                        self.res[(k, r, kv)] = (np.zeros((B, Hkv, n_slots, hd), np.int8),
                                                np.zeros((B, Hkv, n_slots, ng), np.float16))

    # base write / read for lazy stores -----------------------------------
    def _base_write(self, r, b, rows, kvals, vvals):
        """kvals/vvals [Hkv, n, hd] for positions ``rows``."""
        for kv, x in ((0, kvals), (1, vvals)):
            if self.lz.base_bits == 16:
                self.base[r][kv][b][:, rows, :] = x
            else:
                if self.forced_codes_from is not None:
                    src = self.forced_codes_from.base[r][kv]
                    codes, sc = src[0][b][:, rows, :], src[1][b][:, rows, :]
                else:
                    codes, sc = quant.quantize(x, 8, self.lz.group)   # residual vs zero
                self.base[r][kv][0][b][:, rows, :] = codes
                self.base[r][kv][1][b][:, rows, :] = sc

    def recon(self, k: int, r: int, b: int, kv: int, cols: np.ndarray) -> np.ndarray:
        """Loop-k reconstruction of K (kv=0) or V (kv=1) rows ``cols``: [Hkv, c, hd]."""
        if self.lz.base_bits == 16:
            x = self.base[r][kv][b][:, cols, :].copy()
        else:
            codes, sc = self.base[r][kv]
            x = quant.dequantize(codes[b][:, cols, :], sc[b][:, cols, :], self.lz.group)
        for kk in range(2, k + 1):
            sl = self.slot[kk - 1, b, cols]
            have = np.nonzero(sl >= 0)[0]
            if have.size == 0:
                continue
            store = self.res[(kk, r, kv)]
            if self.lz.res_bits == 16:
                x[:, have, :] = store[b][:, sl[have], :]
            else:
                codes, sc = store
                d = quant.dequantize(codes[b][:, sl[have], :], sc[b][:, sl[have], :],
                                     self.lz.group)
                x[:, have, :] = x[:, have, :] + d
        return x

    def _res_write(self, k, r, b, rows, slots, kvals, vvals):
        """Store the loop-k entries of positions ``rows`` (new KV [Hkv, n, hd])."""
        for kv, x in ((0, kvals), (1, vvals)):
            store = self.res[(k, r, kv)]
            if self.lz.res_bits == 16:
                store[b][:, slots, :] = x
            elif self.forced_codes_from is not None:
                src = self.forced_codes_from.res[(k, r, kv)]
                codes, sc = src[0][b][:, slots, :], src[1][b][:, slots, :]
                store[0][b][:, slots, :] = codes
                store[1][b][:, slots, :] = sc
            else:
                prev = self.recon(k - 1, r, b, kv, rows)
                codes, sc = quant.quantize(x - prev, self.lz.res_bits, self.lz.group)
                store[0][b][:, slots, :] = codes
                store[1][b][:, slots, :] = sc

    # ---------------------------------------------------------------- layer
    def _qkv(self, li, x, pos):
        s, W = self.s, self.w["layers"][li]
        n = x.shape[0]
        a = rmsnorm(x, W["attn_norm"], s.rms_eps)
        q = (a @ W["wq"].T).reshape(n, s.n_heads, s.head_dim)
        k = (a @ W["wk"].T).reshape(n, s.n_kv_heads, s.head_dim)
        v = (a @ W["wv"].T).reshape(n, s.n_kv_heads, s.head_dim)
        cos, sin = rope_cos_sin(pos, s.head_dim, s.rope_theta)
        return apply_rope(q, cos, sin), apply_rope(k, cos, sin), v.astype(F32)

    def _out_ffn(self, li, x, o):
        s, W = self.s, self.w["layers"][li]
        n = x.shape[0]
        x = (x + o.reshape(n, -1) @ W["wo"].T).astype(F32)
        b = rmsnorm(x, W["ffn_norm"], s.rms_eps)
        if s.ffn_act == "swiglu":
            f = silu(b @ W["w_gate"].T) * (b @ W["w_up"].T)
        else:
            f = gelu_erf(b @ W["w_up"].T)
        return (x + f.astype(F32) @ W["w_down"].T).astype(F32)

    def _refresh(self, k: int) -> bool:
        """Loop k >= 2 recomputes every token (the refresh period divides k - 1)."""
        p = int(getattr(self.lz, "refresh_every", 0))
        return p > 0 and (k - 1) % p == 0

    def _loop_rows(self, T: int) -> dict:
        """Tokens each loop k >= 2 of the model recomputes: all at refresh loops, else n."""
        n = n_selected(self.lz.rho, T)
        return {k: (T if self._refresh(k) else n) for k in range(2, self.s.n_loops + 1)}

    # -------------------------------------------------------------- prefill
    def prefill(self, ids: np.ndarray) -> np.ndarray:
        ids = np.asarray(ids)
        B, T = ids.shape
        if B != self.B or T > self.Tmax or T < 1:
            raise ValueError("bad prompt shape")
        self.T, self.t = T, T
        if self.lz.mode == "lazy":
            self.n_sel = n_selected(self.lz.rho, T)
            self.n_k = self._loop_rows(T)
            self._alloc_residuals(max(self.n_k.values(), default=0) + (self.Tmax - T))
            self.S = [[None] * B for _ in range(self.s.n_shared)]
        out = np.empty((B, T, self.s.d_model), F32)
        self.depth = 0
        for b in range(B):
            self.depth = 0
            out[b] = self._prefill_one(b, ids[b])
        return out

    def _coda(self, b, h, pos):
        s = self.s
        for j in range(s.n_coda):
            h = self._dense_layer_idx(s.n_prelude + s.n_shared + j, s.n_prelude + j, h, pos, b)
        return rmsnorm(h, self.w["final_norm"], s.rms_eps)

    def _dense_layer_idx(self, li, ci, h, pos, b):
        """Prelude/coda layer ``li`` using dense cache ``ci``."""
        return self._shared_dense(li, h, pos, self.dense_k[ci], self.dense_v[ci], b)

    def _prelude_idx(self, b, h, pos):
        for li in range(self.s.n_prelude):
            h = self._dense_layer_idx(li, li, h, pos, b)
        return h

    def _prefill_one(self, b, ids_b):
        s = self.s
        T = ids_b.shape[0]
        pos = np.arange(T)
        h = self.w["tok_emb"][ids_b].astype(F32)
        h = self._prelude_idx(b, h, pos)
        e = h.copy()
        P = s.n_prelude
        if self.lz.mode == "per_loop":
            for k in range(1, self.K + 1):
                h = self._loop_input(h, e, k)
                for r in range(s.n_shared):
                    h = self._shared_dense(P + r, h, pos, self.loop_k[k - 1][r],
                                           self.loop_v[k - 1][r], b)
        elif self.lz.mode == "last_loop":
            for k in range(1, self.K + 1):
                h = self._loop_input(h, e, k)
                for r in range(s.n_shared):
                    h = self._shared_dense(P + r, h, pos, self.last_k[r], self.last_v[r], b)
        else:
            h = self._lazy_prefill_loops(b, h, pos)
        return self._coda(b, h, pos)

    def _loop_input(self, h, e, k):
        """State entering loop k: (h + e if re-injecting and k >= 2) + loop_emb[k-1]."""
        if self.inject and k >= 2:
            h = (h + e).astype(F32)
        return (h + self.w["loop_emb"][k - 1]).astype(F32)

    def _shared_dense(self, li, h, pos, kc, vc, b):
        q, k, v = self._qkv(li, h, pos)
        kc[b][:, pos, :] = k.transpose(1, 0, 2)
        vc[b][:, pos, :] = v.transpose(1, 0, 2)
        hi = int(pos.max()) + 1
        o = attend_masked(q, kc[b][:, :hi], vc[b][:, :hi], pos, causal_mask)
        self.depth += 1
        return self._out_ffn(li, h, o)

    def _lazy_prefill_loops(self, b, h0, pos):
        s, lz = self.s, self.lz
        P, R, K, T = s.n_prelude, s.n_shared, self.K, pos.shape[0]
        allc = np.arange(T)
        # loop 1: dense, writes the base, accumulates the column mass, picks S.
        x = (h0 + self.w["loop_emb"][0]).astype(F32)
        for r in range(R):
            q, k, v = self._qkv(P + r, x, pos)
            self._base_write(r, b, pos, k.transpose(1, 0, 2), v.transpose(1, 0, 2))
            kr = self.recon(1, r, b, 0, allc)
            vr = self.recon(1, r, b, 1, allc)
            mass = np.zeros((s.n_kv_heads, T), F32)
            o = attend_masked(q, kr, vr, pos, causal_mask, mass=mass)
            if self.forced_S is not None:
                self.S[r][b] = [np.asarray(c, np.int32) for c in self.forced_S[r][b]]
            else:
                self.S[r][b] = [allc.astype(np.int32) if T <= lz.top_s
                                else top_n_ascending(mass[g], lz.top_s)
                                for g in range(s.n_kv_heads)]
            self.mass[(r, b)] = mass
            if self.diff and K >= 2:
                # the loop-1 sparse term of every token over the loop-1 reconstruction
                self.D[(r, b)] = (o - self._attend_sparse(q, kr, vr, pos, r, b)).astype(F32)
            self.depth += 1
            x = self._out_ffn(P + r, x, o)
        h_prev2, h_prev = h0, x
        stale = bool(getattr(lz, "stale_keys", False))
        for k in range(2, K + 1):
            n = self.n_k[k]
            key = np.sum((h_prev - h_prev2) ** 2, axis=-1, dtype=F32)
            if stale and k >= 3:
                # a token carried through loop k-1 keeps the change measured when it
                # was last recomputed
                carried = np.ones(key.shape[0], bool)
                carried[self.sel[(k - 1, b)]] = False
                key = np.where(carried, self.keys[(k - 1, b)], key).astype(F32)
            self.keys[(k, b)] = key
            if self._refresh(k):
                I = np.arange(T)
            elif self.forced_tokens is not None:
                I = self.forced_tokens[(k, b)]
            else:
                I = top_n_ascending(key, n)
            I = np.asarray(I, dtype=np.int64)
            self.sel[(k, b)] = I.astype(np.int32)
            self.slot[k - 1, b, I] = np.arange(n, dtype=np.int32)
            xs = self._loop_input(h_prev[I], h0[I], k)
            for r in range(R):
                q, kk, vv = self._qkv(P + r, xs, I)
                self._res_write(k, r, b, I, np.arange(n), kk.transpose(1, 0, 2),
                                vv.transpose(1, 0, 2))
                kr = self.recon(k, r, b, 0, allc)
                vr = self.recon(k, r, b, 1, allc)
                # each KV head has its own S: attend head-group by head-group.
                o = self._attend_sparse(q, kr, vr, I, r, b)
                if self.diff:
                    o = (o + self.D[(r, b)][I]).astype(F32)
                self.depth += 1
                xs = self._out_ffn(P + r, xs, o)
            h_new = h_prev.copy()
            h_new[I] = xs
            h_prev2, h_prev = h_prev, h_new
        return h_prev

    def _attend_sparse(self, q, kr, vr, rows, r, b):
        """Rows ``rows`` attend over their sparse column sets (each KV head has its own S)."""
        S, w = self.S[r][b], self.lz.window
        return attend_masked(q, kr, vr, rows, sparse_mask(S, w))

    def start_from_state(self, T: int, base, res, slot, S, dense_kv=None):
        """Take a lazy store state as a prefill of T tokens would leave it, built
        elsewhere, and continue with decode from there.

        base[r][kv]: (int8 codes [B, Hkv, Tmax, hd], float16 scales [B, Hkv, Tmax,
        hd/group]) for 8-bit bases, else float32 rows [B, Hkv, Tmax, hd];
        res[(k, r, kv)] for k = 2..shape.n_loops: the same forms over
        the most tokens a loop recomputes (n_selected(rho, T), or T with refresh loops)
        + Tmax - T slots (int8 codes hold the int4 values too);
        slot [shape.n_loops, B, Tmax] int32, row k-1 the slot of each position at
        loop k (-1: not stored); S[r][b][g] ascending int32 column arrays;
        dense_kv[i] = (K rows, V rows) float32 [B, Hkv, Tmax, hd] of prelude/coda
        layer i when there are any.  The arrays are used as given, not copied."""
        s, lz = self.s, self.lz
        if lz.mode != "lazy":
            raise ValueError("a store state exists in lazy mode only")
        if not 1 <= T <= self.Tmax:
            raise ValueError("bad prompt length")
        n_dense = s.n_prelude + s.n_coda
        if n_dense and (dense_kv is None or len(dense_kv) != n_dense):
            raise ValueError("prelude/coda rows are needed")
        n = n_selected(lz.rho, T)
        n_k = self._loop_rows(T)
        n_max = max(n_k.values(), default=0)
        if slot.shape != (s.n_loops, self.B, self.Tmax):
            raise ValueError("slot map shape")
        for (k, r, kv), x in res.items():
            a = x if lz.res_bits == 16 else x[0]
            if a.shape[2] != n_max + self.Tmax - T:
                raise ValueError("residual slot count")
        self.T, self.t, self.n_sel, self.n_k = T, T, n, n_k
        self.n_slots = n_max + self.Tmax - T
        self.base, self.res, self.slot, self.S = base, res, slot, S
        for i in range(n_dense):
            self.dense_k[i], self.dense_v[i] = dense_kv[i]
        self.sel = {(k, b): np.nonzero(slot[k - 1, b, :T] >= 0)[0].astype(np.int32)
                    for k in range(2, self.K + 1) for b in range(self.B)}

    # --------------------------------------------------------------- decode
    def decode(self, ids: np.ndarray) -> np.ndarray:
        ids = np.asarray(ids).reshape(-1)
        if self.T is None:
            raise RuntimeError("decode before prefill")
        if ids.shape[0] != self.B:
            raise ValueError("one token per sequence")
        if self.t >= self.Tmax:
            raise ValueError("store capacity exceeded")
        out = np.empty((self.B, self.s.d_model), F32)
        t = self.t
        for b in range(self.B):
            self.depth = 0
            out[b] = self._decode_one(b, int(ids[b]), t)
        self.t = t + 1
        return out

    def _decode_one(self, b, tok, t):
        s, lz = self.s, self.lz
        P, R, K = s.n_prelude, s.n_shared, self.K
        pos = np.array([t])
        h = self.w["tok_emb"][tok][None, :].astype(F32)
        h = self._prelude_idx(b, h, pos)
        e = h.copy()
        if lz.mode in ("per_loop", "last_loop"):
            for k in range(1, K + 1):
                h = self._loop_input(h, e, k)
                for r in range(R):
                    if lz.mode == "per_loop":
                        kc, vc = self.loop_k[k - 1][r], self.loop_v[k - 1][r]
                    else:
                        kc, vc = self.last_k[r], self.last_v[r]
                    h = self._shared_dense(P + r, h, pos, kc, vc, b)
        else:
            allc = np.arange(t + 1)
            D = {}           # diff_attn: shared layer -> this token's o_1 - a_1 [1, H, hd]
            h_prev2 = e      # h_{k-2} at loop k (h_0: the prelude output)
            ran = K
            for k in range(1, K + 1):
                if k >= 2 and self.tau > 0:
                    key = np.sum((h - h_prev2) ** 2, axis=-1, dtype=F32)[0]
                    self.decode_keys[(k, b, t)] = key
                    if key < self.tau:   # leaves the loops with h_{k-1}
                        ran = k - 1
                        break
                    h_prev2 = h
                h = self._loop_input(h, e, k)
                if k >= 2:
                    slot = self.n_k[k] + (t - self.T)
                    self.slot[k - 1, b, t] = slot
                for r in range(R):
                    q, kk, vv = self._qkv(P + r, h, pos)
                    kt, vt = kk.transpose(1, 0, 2), vv.transpose(1, 0, 2)
                    if k == 1:
                        self._base_write(r, b, pos, kt, vt)
                        kr = self.recon(1, r, b, 0, allc)
                        vr = self.recon(1, r, b, 1, allc)
                        o = attend_masked(q, kr, vr, pos, causal_mask)
                        if self.diff and K >= 2:
                            D[r] = (o - self._attend_sparse(q, kr, vr, pos, r, b)).astype(F32)
                    else:
                        self._res_write(k, r, b, pos, np.array([slot]), kt, vt)
                        kr = self.recon(k, r, b, 0, allc)
                        vr = self.recon(k, r, b, 1, allc)
                        o = self._attend_sparse(q, kr, vr, pos, r, b)
                        if self.diff:
                            o = (o + D[r]).astype(F32)
                    self.depth += 1
                    h = self._out_ffn(P + r, h, o)
            self.decode_loops[(b, t)] = ran
        # coda
        for j in range(s.n_coda):
            h = self._dense_layer_idx(P + R + j, P + j, h, pos, b)
        return rmsnorm(h, self.w["final_norm"], s.rms_eps)[0]
