"""Attention kernels, one by one, against the oracle's attention on identical inputs
(lk_dbg_attention through the C ABI), at the full context of the decode workload the
throughput figure is quoted on (a 32768-token prompt; 8 sequences, 16 query and 4 KV
heads of 128, top-s 1024, window 512) and at the prefill workload's shape.

Both sides read the same numbers: int8 codes with float16 scales (dequantized in
float32 by the oracle), or bf16 / float16 rows, and a q that is exactly
representable in the kernel's operand type.  The oracle is oracle.model.attend
(the row-by-row gathered softmax; every query's key set written out) or its masked
form attend_masked (pinned to attend on the CPU), in float32.

Bounds (max|gpu - oracle| / max|oracle| unless stated), from the roundings each
kernel makes on identical inputs:
* float16 MFMA kernels (int8 decode, two-segment decode, sparse prefill rows):
  code * scale products and probabilities rounded to float16 (2^-11 relative),
  float32 accumulation: 3e-3 on the float32 output; the sparse prefill rows write
  bf16 (2^-9 of each element): 6e-3.
* bf16 kernels (bf16 decode rows, flash prefill over bf16 rows): probabilities
  rounded to bf16 (2^-9) and a bf16 output: 1e-2.  The flash prefill over int8 rows
  takes float16 operands (code * scale and probabilities to 2^-11) and writes bf16:
  1e-2 as well.
* log-sum-exp: 2e-3 absolute (log2 units; each score from float16 K carries about
  2^-11 of its size); column mass: 2e-3 relative per column (the same probabilities,
  summed in another order), and the top-s columns picked from the kernel's mass are a
  valid top-s of the oracle's mass.
"""
import numpy as np
import pytest
import torch

from cross_loop_kv_amd import binding as B
from oracle.model import attend, attend_masked, causal_mask, sparse_cols
from oracle.select import top_n_ascending
from tests.gpu_util import log, max_abs_rel

pytestmark = pytest.mark.gpu

DEC = dict(B=8, H=16, Hkv=4, hd=128, T=32768, tmax=33088, top_s=1024, window=512)


# ---------------------------------------------------------------- layouts (store order)
def v_interleave(a):
    """[B, Hkv, tmax, X] -> [B, Hkv, tmax/8, X, 8] (8 positions interleaved per element)."""
    b, h, t, x = a.shape
    return np.ascontiguousarray(a.reshape(b, h, t // 8, 8, x).transpose(0, 1, 2, 4, 3))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def int8_rows(rng, Bn, Hkv, tmax, hd, n_valid, std):
    """int8 codes uniform on +-127 and float16 group scales for a spread of about std;
    rows at or past n_valid are zero.  Returns codes, scales, float32 values."""
    codes = np.zeros((Bn, Hkv, tmax, hd), np.int8)
    codes[:, :, :n_valid] = rng.integers(-127, 128, (Bn, Hkv, n_valid, hd), dtype=np.int8)
    sc = np.zeros((Bn, Hkv, tmax, hd // 32), np.float16)
    sc[:, :, :n_valid] = (std * np.sqrt(3.0) / 127 * rng.uniform(0.5, 1.5, (Bn, Hkv, n_valid, hd // 32)))
    val = (codes.astype(np.float32).reshape(Bn, Hkv, tmax, hd // 32, 32) *
           sc.astype(np.float32)[..., None]).reshape(Bn, Hkv, tmax, hd)
    return codes, sc, val


def f16_vals(rng, shape, std):
    return (rng.standard_normal(shape) * std).astype(np.float16)


def bf16_vals(rng, shape, std):
    x = torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16)
    return x, x.float().numpy()


def run(args, keep):
    """Size query, then the call with a workspace; keep holds the device tensors alive."""
    need = B.lk_dbg_attention(args)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    args.ws, args.ws_bytes = ws.data_ptr(), ws.numel()
    keep.append(ws)
    B.lk_dbg_attention(args)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- decode, loop 1
@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", ["int8", "bf16"])
def test_decode_split_attention_and_merge_at_full_context(fmt):
    """One query per sequence at position t = 32768 + 40 over keys [0, t] of int8 rows
    (the lazy loop-1 base; q float16) or bf16 rows (the dense per-loop / last-loop
    baselines; q bf16), split over the 33088-row capacity exactly as a decode step
    splits it and merged by the combine kernel."""
    p = DEC
    rng = np.random.default_rng(101 if fmt == "int8" else 102)
    Bn, H, Hkv, hd, tmax = p["B"], p["H"], p["Hkv"], p["hd"], p["tmax"]
    t = p["T"] + 40
    keep = []
    if fmt == "int8":
        kc, ks, kval = int8_rows(rng, Bn, Hkv, tmax, hd, t + 1, 2.0)
        vc, vs, vval = int8_rows(rng, Bn, Hkv, tmax, hd, t + 1, 1.0)
        k_d, v_d = dev(kc), dev(v_interleave(vc))
        ks_d, vs_d = dev(ks.view(np.uint16)), dev(v_interleave(vs.view(np.uint16)))
        q16 = f16_vals(rng, (Bn, H * hd), 1.0)
        q_d, qf = dev(q16.view(np.uint16)), q16.astype(np.float32)
        kvfmt, q_half = 1, 1
        keep += [ks_d, vs_d]
    else:
        kb, kval = bf16_vals(rng, (Bn, Hkv, tmax, hd), 2.0)
        vb, vval = bf16_vals(rng, (Bn, Hkv, tmax, hd), 1.0)
        kval[:, :, t + 1:] = 0
        vval[:, :, t + 1:] = 0
        k_d = kb.view(torch.int16).cuda()
        v_d = dev(v_interleave(vb.view(torch.int16).numpy()))
        ks_d = vs_d = None
        qb, qf = bf16_vals(rng, (Bn, H * hd), 1.0)
        q_d = qb.view(torch.int16).cuda()
        kvfmt, q_half = 0, 0
    out = torch.zeros(Bn, H * hd, dtype=torch.int16, device="cuda")
    out32 = torch.zeros(Bn, H * hd, dtype=torch.float32, device="cuda")
    keep += [k_d, v_d, q_d]
    a = B.lk_dbg_attn_args(kind=B.DBG_ATTN["decode"], B=Bn, H=H, Hkv=Hkv, hd=hd, kv_format=kvfmt, t=t, tmax=tmax,
                           q=q_d.data_ptr(), q_half=q_half, k=k_d.data_ptr(), v=v_d.data_ptr(),
                           k_scales=ks_d.data_ptr() if ks_d is not None else None,
                           v_scales=vs_d.data_ptr() if vs_d is not None else None,
                           out=out.data_ptr(), out32=out32.data_ptr())
    run(a, keep)
    g = out32.cpu().numpy()
    gb = out.cpu().view(torch.bfloat16).float().numpy()
    errs = []
    for b in range(Bn):
        o = attend(qf[b].reshape(1, H, hd), kval[b, :, :t + 1], vval[b, :, :t + 1],
                   lambda i, gg: np.arange(t + 1))[0].reshape(-1)
        errs.append(max_abs_rel(g[b], o))
        assert max_abs_rel(gb[b], o) < 1e-2
    bound = 3e-3 if fmt == "int8" else 1e-2
    log(f"  decode {fmt} over {t + 1} keys: max-abs-rel per sequence max {max(errs):.2e} (bound {bound:.0e})")
    assert max(errs) < bound


# ---------------------------------------------------------------- decode, loops >= 2
@pytest.mark.timeout(600)
@pytest.mark.parametrize("t_off", [5, 300])
def test_decode_two_segment_attention_at_full_context(t_off):
    """One query per sequence at t = 32768 + t_off over (S intersect [0, t - 512]) union
    [t - 511, t], S 1024 ascending prompt columns per (sequence, KV head): the stable
    columns from the float16 cache (row i = column S[i]), the window from the float16
    ring of 640 rows (position p at row p % 640).  At t_off 5 the window's ring rows
    wrap past the ring's end; a fifth of S lies inside the window, so those columns
    are read once, through the ring."""
    p = DEC
    rng = np.random.default_rng(200 + t_off)
    Bn, H, Hkv, hd, s, w = p["B"], p["H"], p["Hkv"], p["hd"], p["top_s"], p["window"]
    t = p["T"] + t_off
    s_cap, r_cap = 1024, 640
    assert (t - w + 1) % r_cap > t % r_cap or t_off != 5          # the window wraps the ring
    K = f16_vals(rng, (Bn, Hkv, t + 1, hd), 2.0)
    V = f16_vals(rng, (Bn, Hkv, t + 1, hd), 1.0)
    S = np.zeros((Bn, Hkv, s), np.int32)
    for b in range(Bn):
        for g in range(Hkv):
            inside = rng.choice(np.arange(t - w + 1, p["T"]), s // 5, replace=False) if t - w + 1 < p["T"] else []
            S[b, g] = np.sort(np.concatenate([rng.choice(t - w + 1, s - len(inside), replace=False), inside]))
    sk = np.zeros((Bn, Hkv, s_cap, hd), np.float16)
    sv = np.zeros((Bn, Hkv, s_cap, hd), np.float16)
    rk = np.zeros((Bn, Hkv, r_cap, hd), np.float16)
    rv = np.zeros((Bn, Hkv, r_cap, hd), np.float16)
    for b in range(Bn):
        for g in range(Hkv):
            sk[b, g, :s] = K[b, g, S[b, g]]
            sv[b, g, :s] = V[b, g, S[b, g]]
            lo = max(0, t - w + 1) & ~7
            for pp in range(lo, t + 1):
                rk[b, g, pp % r_cap] = K[b, g, pp]
                rv[b, g, pp % r_cap] = V[b, g, pp]
    q16 = f16_vals(rng, (Bn, H * hd), 1.0)
    keep = [dev(q16.view(np.uint16)), dev(S), dev(sk.view(np.uint16)), dev(v_interleave(sv).view(np.uint16)),
            dev(rk.view(np.uint16)), dev(v_interleave(rv).view(np.uint16))]
    out = torch.zeros(Bn, H * hd, dtype=torch.int16, device="cuda")
    out32 = torch.zeros(Bn, H * hd, dtype=torch.float32, device="cuda")
    a = B.lk_dbg_attn_args(kind=B.DBG_ATTN["decode_seg"], B=Bn, H=H, Hkv=Hkv, hd=hd, t=t, q=keep[0].data_ptr(),
                           q_half=1, cols=keep[1].data_ptr(), n_cols=s, window=w, s_k=keep[2].data_ptr(),
                           s_v=keep[3].data_ptr(), s_cap=s_cap, r_k=keep[4].data_ptr(), r_v=keep[5].data_ptr(),
                           r_cap=r_cap, out=out.data_ptr(), out32=out32.data_ptr())
    run(a, keep)
    g = out32.cpu().numpy()
    qf = q16.astype(np.float32)
    errs = []
    for b in range(Bn):
        o = attend(qf[b].reshape(1, H, hd), K[b].astype(np.float32), V[b].astype(np.float32),
                   lambda i, gg: sparse_cols(t, S[b, gg], w))[0].reshape(-1)
        errs.append(max_abs_rel(g[b], o))
    log(f"  two-segment decode at t={t}: max-abs-rel per sequence max {max(errs):.2e}")
    assert max(errs) < 3e-3


# ---------------------------------------------------------------- prefill, loop 1
@pytest.mark.timeout(900)
def test_flash_prefill_lse_and_column_mass_at_full_context():
    """Causal attention of a 32768-token prompt over int8 rows (the lazy loop-1 base),
    4 query heads on one KV head: every output row and its log-sum-exp against the
    oracle, then the column mass the kernel derives from that log-sum-exp against the
    oracle's mass (summed over all 32768 queries and the 4 heads), and the top-1024
    columns picked from the kernel's mass (lk_dbg_topk, the selector prefill uses) are
    a top-1024 of the oracle's mass up to its float32 rounding."""
    rng = np.random.default_rng(301)
    T, H, Hkv, hd, s = 32768, 4, 1, 128, 1024
    kc, ks, kval = int8_rows(rng, 1, Hkv, T, hd, T, 1.5)
    vc, vs, vval = int8_rows(rng, 1, Hkv, T, hd, T, 1.0)
    qb, qf = bf16_vals(rng, (T, H * hd), 1.0)
    keep = [qb.view(torch.int16).cuda(), dev(kc), dev(v_interleave(vc)), dev(ks.view(np.uint16)),
            dev(v_interleave(vs.view(np.uint16)))]
    out = torch.zeros(T, H * hd, dtype=torch.int16, device="cuda")
    lse = torch.zeros(H, T, dtype=torch.float32, device="cuda")
    mass = torch.zeros(Hkv, T, dtype=torch.float32, device="cuda")
    common = dict(B=1, H=H, Hkv=Hkv, hd=hd, kv_format=1, T=T, tmax=T, q=keep[0].data_ptr(), k=keep[1].data_ptr(),
                  v=keep[2].data_ptr(), k_scales=keep[3].data_ptr(), v_scales=keep[4].data_ptr(),
                  out=out.data_ptr(), lse=lse.data_ptr(), mass=mass.data_ptr())
    run(B.lk_dbg_attn_args(kind=B.DBG_ATTN["prefill"], **common), keep)
    run(B.lk_dbg_attn_args(kind=B.DBG_ATTN["mass"], **common), keep)
    idx = torch.zeros(Hkv, s, dtype=torch.int32, device="cuda")
    B.lk_dbg_topk(mass.data_ptr(), Hkv, T, s, idx.data_ptr())
    torch.cuda.synchronize()
    log("  oracle: causal attention over 32768 positions ...")
    om = np.zeros((Hkv, T), np.float32)
    o = attend_masked(qf.reshape(T, H, hd), kval[0], vval[0], np.arange(T), causal_mask, mass=om)
    g = out.cpu().view(torch.bfloat16).float().numpy().reshape(T, H, hd)
    e_out = max_abs_rel(g, o)
    worst_row = float(np.max(np.max(np.abs(g - o), axis=(1, 2)) / np.max(np.abs(o), axis=(1, 2))))
    # log-sum-exp of sampled rows in float64 (log2 units of the scaled scores)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, T // 2, T - 1], rng.integers(0, T, 56)]))
    gl = lse.cpu().numpy()
    e_lse = 0.0
    for i in rows:
        sc = (qf.reshape(T, H, hd)[i].astype(np.float64) @ kval[0, 0, :i + 1].astype(np.float64).T) / np.sqrt(hd)
        mx = sc.max(axis=1, keepdims=True)
        ref = (mx[:, 0] + np.log(np.exp(sc - mx).sum(axis=1))) / np.log(2.0)
        e_lse = max(e_lse, float(np.max(np.abs(gl[:, i] - ref))))
    gm = mass.cpu().numpy()
    e_mass = float(np.max(np.abs(gm - om) / np.maximum(om, 1e-3 * om.max())))
    tot = float(gm.sum())
    log(f"  flash prefill T={T}: out {e_out:.2e} (worst row {worst_row:.2e}), lse {e_lse:.2e}, "
        f"mass {e_mass:.2e}, mass total {tot:.1f} (= H/Hkv * T = {H // Hkv * T})")
    assert e_out < 1e-2 and e_lse < 2e-3 and e_mass < 2e-3
    assert abs(tot - H // Hkv * T) < 1e-3 * T
    # the kernel's top-s: every picked column's oracle mass is at least the oracle's
    # s-th largest, less the float32 rounding of the masses
    gi = np.sort(idx.cpu().numpy()[0])
    oi = top_n_ascending(om[0], s)
    thr = np.sort(om[0])[::-1][s - 1]
    tol = 2e-3 * thr
    assert len(set(gi.tolist())) == s
    assert np.all(om[0][gi] >= thr - tol)
    differ = np.setxor1d(gi, oi)
    assert np.all(np.abs(om[0][differ] - thr) <= tol), "columns swapped outside a near-tie"
    log(f"  top-{s} columns: {len(differ) // 2} swapped in near-ties, rest identical")


@pytest.mark.timeout(600)
def test_flash_prefill_bf16_rows_at_prefill_shape():
    """Causal attention of a 4096-token prompt over bf16 rows, 16 heads with their own
    KV head each (the prefill workload's 16 x 128 MHA), all rows against the oracle."""
    rng = np.random.default_rng(302)
    T, H, Hkv, hd = 4096, 16, 16, 128
    kb, kval = bf16_vals(rng, (1, Hkv, T, hd), 1.0)
    vb, vval = bf16_vals(rng, (1, Hkv, T, hd), 1.0)
    qb, qf = bf16_vals(rng, (T, H * hd), 1.0)
    keep = [qb.view(torch.int16).cuda(), kb.view(torch.int16).cuda(), dev(v_interleave(vb.view(torch.int16).numpy()))]
    out = torch.zeros(T, H * hd, dtype=torch.int16, device="cuda")
    lse = torch.zeros(H, T, dtype=torch.float32, device="cuda")
    run(B.lk_dbg_attn_args(kind=B.DBG_ATTN["prefill"], B=1, H=H, Hkv=Hkv, hd=hd, kv_format=0, T=T, tmax=T,
                           q=keep[0].data_ptr(), k=keep[1].data_ptr(), v=keep[2].data_ptr(), out=out.data_ptr(),
                           lse=lse.data_ptr()), keep)
    o = attend_masked(qf.reshape(T, H, hd), kval[0], vval[0], np.arange(T), causal_mask)
    g = out.cpu().view(torch.bfloat16).float().numpy().reshape(T, H, hd)
    e = max_abs_rel(g, o)
    log(f"  flash prefill bf16 T={T} H={H}: {e:.2e}")
    assert e < 1e-2


# ---------------------------------------------------------------- prefill, loops >= 2
@pytest.mark.timeout(600)
def test_sparse_prefill_rows_at_full_context():
    """The 3277 kept rows of a 32768-token prompt (rho 0.1), each over (S intersect
    [0, i - 512]) union [i - 511, i], S 1024 columns per KV head, 16 query heads on 4 KV
    heads: stable columns from the float16 cache, the window from float16 rows at every
    position, every row against the oracle."""
    rng = np.random.default_rng(401)
    T, H, Hkv, hd, s, w, n = 32768, 16, 4, 128, 1024, 512, 3277
    K = f16_vals(rng, (Hkv, T, hd), 1.5)
    V = f16_vals(rng, (Hkv, T, hd), 1.0)
    S = np.stack([np.sort(rng.choice(T, s, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    rows = np.sort(rng.choice(T, n, replace=False)).astype(np.int32)
    sk = np.stack([K[g, S[g]] for g in range(Hkv)])[None]
    sv = np.stack([V[g, S[g]] for g in range(Hkv)])[None]
    qb, qf = bf16_vals(rng, (n, H * hd), 1.0)
    keep = [qb.view(torch.int16).cuda(), dev(rows), dev(S), dev(sk.view(np.uint16)),
            dev(v_interleave(sv).view(np.uint16)), dev(K[None].view(np.uint16)),
            dev(v_interleave(V[None]).view(np.uint16))]
    out = torch.zeros(n, H * hd, dtype=torch.int16, device="cuda")
    run(B.lk_dbg_attn_args(kind=B.DBG_ATTN["prefill_sparse"], B=1, H=H, Hkv=Hkv, hd=hd, T=T, q=keep[0].data_ptr(),
                           qpos=keep[1].data_ptr(), n_rows=n, cols=keep[2].data_ptr(), n_cols=s, window=w,
                           s_k=keep[3].data_ptr(), s_v=keep[4].data_ptr(), s_cap=s, r_k=keep[5].data_ptr(),
                           r_v=keep[6].data_ptr(), r_cap=T, out=out.data_ptr()), keep)
    o = attend(qf.reshape(n, H, hd), K.astype(np.float32), V.astype(np.float32),
               lambda i, g: sparse_cols(int(rows[i]), S[g], w))
    g = out.cpu().view(torch.bfloat16).float().numpy().reshape(n, H, hd)
    e = max_abs_rel(g, o)
    log(f"  sparse prefill rows: {n} rows over s={s} + w={w}: {e:.2e}")
    assert e < 6e-3
