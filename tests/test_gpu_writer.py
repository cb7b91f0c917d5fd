"""The KV-store writer against the oracle's quantizer, bit for bit, on identical float32
projections (lk_dbg_kv_write through the C ABI; no codes injected).

The writer rotates q and K by RoPE at the row's position (the rotate-half formula,
each product rounded before the sum), and stores loop 1 as the base (int8 codes with
float16 scales against a zero reconstruction, or bf16 rows) and loop k >= 2 as the
quantized difference to the loop-(k-1) reconstruction (int4 codes packed two per
byte, int8 codes, or bf16 rows), with the loop's slot map (the FlashLoop abstract's
KV-residual quantization, in the store format the library documents).  Expected
values: oracle.model.apply_rope / rope_cos_sin for the rotation, oracle.quant for
codes, scales, dequantization and int4 packing, the store layout for addresses.
Everything integer (codes, scales, packed bytes, slot maps) and every rotated q / K
value must match exactly.

Two call patterns are covered: the prefill pattern (many rows per sequence at given
positions, residuals in consecutive slots) and the decode pattern the throughput
figure's decode step runs (one row per sequence at the store length, the previous
loop's reconstruction carried in float32 from loop to loop, the float16 window-ring
row written alongside).  A last test covers the store's float16-range flag."""
import numpy as np
import pytest
import torch

from cross_loop_kv_amd import binding as B
from cross_loop_kv_amd import inputs as I
from oracle import quant
from oracle.model import apply_rope, rope_cos_sin
from oracle.select import n_selected
from tests.gpu_util import log, store_region

pytestmark = pytest.mark.gpu


def _shape(n_loops=4):
    return I.Shape(vocab=256, d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, ffn_dim=512, ffn_act="swiglu",
                   n_prelude=0, n_shared=2, n_loops=n_loops, n_coda=0)


def _f32_to_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


class StoreReader:
    """The lazy store's regions as numpy arrays in the oracle's [b][g][pos][...] order."""

    def __init__(self, store, shape, lz):
        torch.cuda.synchronize()
        self.st, self.s, self.lz = store, shape, lz
        self.v = store.view()
        self.Bn = store.batch
        self.Tp = self.v.row_stride

    def _deinterleave(self, a):
        """[B, Hkv, Tp/8, X, 8] -> [B, Hkv, Tp, X]."""
        b, h, t8, x, _ = a.shape
        return a.transpose(0, 1, 2, 4, 3).reshape(b, h, t8 * 8, x)

    def base(self, r, kv):
        s, Bn, Tp, hd, Hkv = self.s, self.Bn, self.Tp, self.s.head_dim, self.s.n_kv_heads
        n = Bn * Hkv * Tp * hd
        if self.lz.base_bits == 16:
            raw = store_region(self.st, self.v.base_codes + (2 * r + kv) * n * 2, n * 2, torch.int16)
            x = raw.cpu().numpy().view(np.uint16)
            x = x.reshape(Bn, Hkv, Tp, hd) if kv == 0 else self._deinterleave(x.reshape(Bn, Hkv, Tp // 8, hd, 8))
            return x, None
        c = store_region(self.st, self.v.base_codes + (2 * r + kv) * n, n, torch.int8).cpu().numpy()
        ns = Bn * Hkv * Tp * (hd // 32)
        sc = store_region(self.st, self.v.base_scales + (2 * r + kv) * ns * 2, ns * 2, torch.int16).cpu().numpy() \
            .view(np.uint16)
        if kv == 0:
            return c.reshape(Bn, Hkv, Tp, hd), sc.reshape(Bn, Hkv, Tp, hd // 32)
        return (self._deinterleave(c.reshape(Bn, Hkv, Tp // 8, hd, 8)),
                self._deinterleave(sc.reshape(Bn, Hkv, Tp // 8, hd // 32, 8)))

    def res(self, k, r, kv):
        s, Bn, hd, Hkv = self.s, self.Bn, self.s.head_dim, self.s.n_kv_heads
        R, slots, rb = s.n_shared, self.v.slots, self.v.res_row_bytes
        reg = ((k - 2) * R + r) * 2 + kv
        rows = Bn * Hkv * slots
        codes = store_region(self.st, self.v.res_codes + reg * rows * rb, rows * rb, torch.uint8).cpu().numpy()
        codes = codes.reshape(Bn, Hkv, slots, rb)
        if self.lz.res_bits == 16:
            return codes.view(np.uint16), None
        sc = store_region(self.st, self.v.res_scales + reg * rows * (hd // 32) * 2, rows * (hd // 32) * 2,
                          torch.int16).cpu().numpy().view(np.uint16).reshape(Bn, Hkv, slots, hd // 32)
        return codes, sc

    def slot_map(self, k):
        K = self.s.n_loops
        sm = store_region(self.st, self.v.slot_maps, (K - 1) * self.Bn * self.Tp * 4, torch.int32).cpu().numpy()
        return sm.reshape(K - 1, self.Bn, self.Tp)[k - 2]

    def ring(self, k, r, kv):
        """The float16 window ring of (loop k, layer r): [B, Hkv, ring_rows, hd]."""
        v, s, Bn, hd, Hkv = self.v, self.s, self.Bn, self.s.head_dim, self.s.n_kv_heads
        R, K, k0 = s.n_shared, s.n_loops, v.first_cached_loop
        one_s = Bn * Hkv * v.cache_rows * hd * 2
        one_r = Bn * Hkv * v.ring_rows * hd * 2
        off = (K + 1 - k0) * R * 2 * one_s + ((k - k0) * R + r) * 2 * one_r + kv * one_r
        x = store_region(self.st, v.decode_cache + off, one_r, torch.int16).cpu().numpy().view(np.float16)
        if kv == 0:
            return x.reshape(Bn, Hkv, v.ring_rows, hd)
        return self._deinterleave(x.reshape(Bn, Hkv, v.ring_rows // 8, hd, 8))


def _split(qkv, s):
    """float32 projections [rows, (H + 2 Hkv) hd] -> q [rows, H, hd], k, v [rows, Hkv, hd]."""
    H, Hkv, hd = s.n_heads, s.n_kv_heads, s.head_dim
    q = qkv[:, :H * hd].reshape(-1, H, hd)
    k = qkv[:, H * hd:(H + Hkv) * hd].reshape(-1, Hkv, hd)
    v = qkv[:, (H + Hkv) * hd:].reshape(-1, Hkv, hd)
    return q, k, v


def _codes_expected(x, bits):
    """oracle.quant codes of [..., hd] rows in the store's byte form, and scale bits."""
    c, sc = quant.quantize(x, bits)
    cb = quant.pack_int4(c) if bits == 4 else c.view(np.uint8)
    return cb, sc.view(np.uint16), quant.dequantize(c, sc)


def _projections(rng, rows, s, scale_spread=True):
    H, Hkv, hd = s.n_heads, s.n_kv_heads, s.head_dim
    x = rng.standard_normal((rows, (H + 2 * Hkv) * hd)).astype(np.float32)
    if scale_spread:   # row magnitudes over several binades
        x *= (2.0 ** rng.integers(-6, 5, (rows, 1))).astype(np.float32)
    return x


@pytest.mark.parametrize("base_bits,res_bits", [(8, 4), (8, 8), (16, 16), (16, 4)])
def test_prefill_pattern_writer_is_bit_exact(base_bits, res_bits):
    """Loop 1 writes 200 positions of 2 sequences; loops 2, 3, 4 each write the
    residuals of 60 kept positions (a random subset each loop, so some positions are
    stored at loop 2 and 4 but not 3) against the reconstruction the store holds.
    Codes, scales, int4 packing, slot maps, 16-bit rows and the rotated q (bf16 at
    loop 1, float16 at loop 2) must equal the oracle's exactly."""
    s = _shape()
    lz = I.Lazy(mode="lazy", rho=0.3, top_s=16, window=8, base_bits=base_bits, res_bits=res_bits)
    Bn, T = 2, 200
    n = n_selected(lz.rho, T)
    rng = np.random.default_rng(7 + base_bits + res_bits)
    model = B.LoopedModel(s, lz, I.gen_weights(s, seed=1))
    st = model.store(Bn, T, T + 4)
    H, Hkv, hd, R = s.n_heads, s.n_kv_heads, s.head_dim, s.n_shared
    r = 1
    recon = {0: np.zeros((Bn, Hkv, T, hd), np.float32), 1: np.zeros((Bn, Hkv, T, hd), np.float32)}
    sel = {}
    for k in range(1, s.n_loops + 1):
        rows_per = T if k == 1 else n
        pos = np.stack([np.arange(T) if k == 1 else np.sort(rng.choice(T, n, replace=False)) for _ in range(Bn)])
        sel[k] = pos
        qkv = _projections(rng, Bn * rows_per, s)
        q_half = k == 2
        q_out = torch.zeros(Bn * rows_per, H * hd, dtype=torch.int16, device="cuda")
        B.lk_dbg_kv_write(st.s, r, k, torch.from_numpy(qkv).cuda().data_ptr(), rows_per,
                          torch.from_numpy(pos.reshape(-1).astype(np.int32)).cuda().data_ptr(), q_out.data_ptr(),
                          q_half)
        torch.cuda.synchronize()
        q, kk, vv = _split(qkv, s)
        cos, sin = rope_cos_sin(pos.reshape(-1), hd, s.rope_theta)
        qr, kr = apply_rope(q, cos, sin), apply_rope(kk, cos, sin)
        gq = q_out.cpu().numpy().view(np.uint16).reshape(-1, H, hd)
        eq = qr.astype(np.float16).view(np.uint16) if q_half else _f32_to_bf16_bits(qr)
        assert np.array_equal(gq, eq), f"loop {k}: rotated q"
        rd = StoreReader(st, s, lz)
        for kv, x in ((0, kr), (1, vv)):
            x = x.reshape(Bn, rows_per, Hkv, hd).transpose(0, 2, 1, 3)     # [b, g, row, hd]
            if k == 1:
                gc, gs = rd.base(r, kv)
                if base_bits == 16:
                    assert np.array_equal(gc[:, :, :T], _f32_to_bf16_bits(x)), f"bf16 base kv={kv}"
                    recon[kv] = _f32_to_bf16_bits(x).astype(np.uint32).__lshift__(16).view(np.float32)
                else:
                    ec, es, deq = _codes_expected(x, 8)
                    assert np.array_equal(gc[:, :, :T].view(np.uint8), ec), f"int8 base codes kv={kv}"
                    assert np.array_equal(gs[:, :, :T], es), f"int8 base scales kv={kv}"
                    recon[kv] = deq
                continue
            prev = np.stack([recon[kv][b][:, pos[b]] for b in range(Bn)])   # [b, g, n, hd]
            gc, gs = rd.res(k, r, kv)
            if res_bits == 16:
                eb = _f32_to_bf16_bits(x)
                assert np.array_equal(gc[:, :, :n], eb), f"loop {k} bf16 rows kv={kv}"
                new = eb.astype(np.uint32).__lshift__(16).view(np.float32)
            else:
                ec, es, deq = _codes_expected(x - prev, res_bits)
                assert np.array_equal(gc[:, :, :n], ec), f"loop {k} codes kv={kv}"
                assert np.array_equal(gs[:, :, :n], es), f"loop {k} scales kv={kv}"
                new = prev + deq
            for b in range(Bn):
                recon[kv][b][:, pos[b]] = new[b]
        sm = rd.slot_map(k) if k >= 2 else None
        if sm is not None:
            for b in range(Bn):
                exp = np.full(T, -1, np.int32)
                exp[pos[b]] = np.arange(n)
                assert np.array_equal(sm[b, :T], exp), f"loop {k} slot map"
    log(f"  prefill writer base {base_bits} / residual {res_bits}: bit-exact over {s.n_loops} loops")


def test_decode_pattern_writer_is_bit_exact():
    """After a prefill of 2 x 96 tokens (int8 base, int4 residuals, 4 loops), one
    decode token's loops 1..4 are written as a decode step writes them (position =
    the store length, slot = n + 0, the previous loop's reconstruction carried in
    float32): base codes and scales, residual codes, scales and int4 bytes, slot-map
    entries, the float16 window-ring rows and the rotated q must equal the oracle's."""
    s = _shape()
    lz = I.Lazy(mode="lazy", rho=0.3, top_s=16, window=8, base_bits=8, res_bits=4)
    Bn, T = 2, 96
    n = n_selected(lz.rho, T)
    rng = np.random.default_rng(17)
    model = B.LoopedModel(s, lz, I.gen_weights(s, seed=2))
    st = model.store(Bn, T, T + 4)
    model.prefill(st, torch.from_numpy(I.gen_prompt_ids(s, Bn, T)))
    ws, nbytes = model.workspace(Bn, 1)
    H, Hkv, hd = s.n_heads, s.n_kv_heads, s.head_dim
    t = T
    cos, sin = rope_cos_sin(np.full(Bn, t), hd, s.rope_theta)
    for r in range(s.n_shared):
        prev = {}
        for k in range(1, s.n_loops + 1):
            qkv = _projections(rng, Bn, s)
            q_out = torch.zeros(Bn, H * hd, dtype=torch.int16, device="cuda")
            B.lk_dbg_kv_write(st.s, r, k, torch.from_numpy(qkv).cuda().data_ptr(), 1, None, q_out.data_ptr(),
                              k == 1, ws.data_ptr(), nbytes)
            torch.cuda.synchronize()
            q, kk, vv = _split(qkv, s)
            qr, kr = apply_rope(q, cos, sin), apply_rope(kk, cos, sin)
            gq = q_out.cpu().numpy().view(np.uint16).reshape(Bn, H, hd)
            eq = qr.astype(np.float16).view(np.uint16) if k == 1 else _f32_to_bf16_bits(qr)
            assert np.array_equal(gq, eq), f"layer {r} loop {k}: rotated q"
            rd = StoreReader(st, s, lz)
            for kv, x in ((0, kr), (1, vv)):
                if k == 1:
                    ec, es, deq = _codes_expected(x, 8)                     # [b, g, hd]
                    gc, gs = rd.base(r, kv)
                    assert np.array_equal(gc[:, :, t].view(np.uint8), ec), f"layer {r} base codes kv={kv}"
                    assert np.array_equal(gs[:, :, t], es), f"layer {r} base scales kv={kv}"
                    prev[kv] = deq
                    continue
                ec, es, deq = _codes_expected(x - prev[kv], 4)
                gc, gs = rd.res(k, r, kv)
                assert np.array_equal(gc[:, :, n], ec), f"layer {r} loop {k} codes kv={kv}"
                assert np.array_equal(gs[:, :, n], es), f"layer {r} loop {k} scales kv={kv}"
                prev[kv] = prev[kv] + deq
                ring = rd.ring(k, r, kv)[:, :, t % rd.v.ring_rows]
                assert np.array_equal(ring.view(np.uint16), prev[kv].astype(np.float16).view(np.uint16)), \
                    f"layer {r} loop {k} ring row kv={kv}"
            if k >= 2:
                assert np.all(rd.slot_map(k)[:, t] == n), f"loop {k} slot map"
    assert st.length() == T
    log("  decode writer: bit-exact over 2 layers x 4 loops")


def test_writer_flags_elements_outside_float16_range():
    """The store's float16-range flag (lk_kv_store_range_check): raised when a rotated q,
    a rotated K or a V element that the writer handles is not finite or exceeds 65504 in
    magnitude (the int8-base attention operands, the decode caches and q are float16,
    where such an element is inf); not raised by in-range rows or by +-65504 itself;
    lowered by a clearing read.  The element under test sits in the row at position 0,
    whose rotation angle is 0, so the rotated value is the projection itself."""
    s = _shape()
    lz = I.Lazy(mode="lazy", rho=0.3, top_s=16, window=8, base_bits=8, res_bits=4)
    Bn, T = 1, 32
    rng = np.random.default_rng(11)
    model = B.LoopedModel(s, lz, I.gen_weights(s, seed=1))
    st = model.store(Bn, T, T + 4)
    H, Hkv, hd = s.n_heads, s.n_kv_heads, s.head_dim
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    q_out = torch.zeros(Bn * T, H * hd, dtype=torch.int16, device="cuda")

    def write(qkv):
        d = torch.from_numpy(qkv).cuda()
        B.lk_dbg_kv_write(st.s, 0, 1, d.data_ptr(), T, pos.data_ptr(), q_out.data_ptr(), 0)
        torch.cuda.synchronize()
        return st.out_of_f16_range(clear=True)

    assert not st.out_of_f16_range(), "a new store"
    base = _projections(rng, Bn * T, s)
    assert not write(base), "in-range rows"
    qcol, kcol, vcol = 17, H * hd + hd + 3, (H + Hkv) * hd + 5
    cases = [("V at 65504", vcol, 65504.0, False), ("V at -65504", vcol, -65504.0, False),
             ("K at 65504", kcol, 65504.0, False), ("V above", vcol, 65520.0, True),
             ("K above", kcol, -7.0e4, True), ("q above", qcol, 1.0e5, True),
             ("V NaN", vcol, np.nan, True), ("K inf", kcol, np.inf, True)]
    for name, col, val, flagged in cases:
        x = base.copy()
        x[0, col] = val
        log(f"  range flag: {name}")
        assert write(x) == flagged, name
    assert not st.out_of_f16_range(), "the clearing reads left the flag lowered"


def test_decode_flags_a_loop_two_query_outside_float16_range():
    """The range flag in a decode step's loops >= 2, where the attention launch rotates q
    itself (its new-key split checks every rotated q element of its KV-head group).
    One shared-layer weight W_q[i, j] = 8000 and a loop-2 embedding of 1000 in model
    dimension j: at loop 1 RMSNorm keeps that input near 1 in magnitude (q_i about
    8000 · |a_j|, inside the float16 range); at loop 2 the embedding dominates the row,
    a_j is about sqrt(d) and q_i about 1.8e5, whose rotation leaves at least
    1.8e5 / sqrt(2) in one of the pair's two elements.  K and V stay small, and so does
    the residual stream: the decode products take it times the norm gain in float16, so
    an element above 65504 there (an embedding of 1e6, say) makes K and V non-finite,
    which raises the flag on its own.  The prefill's loop 2 raises the flag through the
    store writer; after it is cleared, one decode step must raise it again.  The same
    model without the large weight leaves it lowered."""
    s = _shape(n_loops=2)
    lz = I.Lazy(mode="lazy", rho=0.3, top_s=16, window=8, base_bits=8, res_bits=4)
    Bn, T, j, i = 2, 32, 5, 3
    ids = torch.from_numpy(I.gen_prompt_ids(s, Bn, T))
    dec = torch.from_numpy(I.gen_decode_ids(s, Bn, 1))
    for big_q in (True, False):
        W = I.gen_weights(s, seed=1)
        W["loop_emb"][1, j] = 1000.0
        if big_q:
            W["layers"][0]["wq"][i, j] = 8000.0
        model = B.LoopedModel(s, lz, W)
        st = model.store(Bn, T, T + 4)
        model.prefill(st, ids)
        torch.cuda.synchronize()
        assert st.out_of_f16_range(clear=True) == big_q, "prefill loop 2"
        assert not st.out_of_f16_range(), "the clearing read left the flag lowered"
        model.decode(st, dec[0])
        torch.cuda.synchronize()
        log(f"  decode range flag with W_q[{i}, {j}] {'= 8000' if big_q else 'unchanged'}")
        assert st.out_of_f16_range() == big_q, "decode loop 2"
        st = None
        model.close()
