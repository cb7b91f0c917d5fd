"""Kernel-level GPU tests through the C ABI.

Bit-exact: the top-n selector (indices) and the residual quantizer (codes and
float16 scales) against the oracle on identical float32 inputs.  Tolerance:
delta keys and the bf16 GEMM against float32/float64 references.
"""
import math

import numpy as np
import scipy.special
import pytest
import torch

from cross_loop_kv_amd import binding as B
from oracle import quant
from oracle.select import top_n_ascending
from tests.gpu_util import log, max_abs_rel

pytestmark = pytest.mark.gpu


def _keys(rng, rows, cols, kind):
    if kind == "ties":
        return (rng.integers(0, 5, size=(rows, cols)) * 0.25).astype(np.float32)
    if kind == "zeros":
        k = np.zeros((rows, cols), np.float32)
        k[:, ::7] = rng.random((rows, (cols + 6) // 7)).astype(np.float32)
        return k
    if kind == "equal":
        return np.full((rows, cols), 3.0, np.float32)
    return (rng.random((rows, cols)) * 10 ** rng.uniform(-3, 3)).astype(np.float32)


@pytest.mark.parametrize("cols", [1, 7, 256, 1000, 4097, 32768])
@pytest.mark.parametrize("kind", ["random", "ties", "zeros", "equal"])
def test_topk_bit_exact(cols, kind):
    rng = np.random.default_rng(cols)
    rows = 3
    keys = _keys(rng, rows, cols, kind)
    for n in sorted({1, max(1, cols // 10), max(1, cols // 2), cols}):
        log(f"topk cols={cols} kind={kind} n={n}")
        d_k = torch.from_numpy(keys).cuda()
        d_i = torch.full((rows, n), -1, dtype=torch.int32, device="cuda")
        B.lk_dbg_topk(d_k.data_ptr(), rows, cols, n, d_i.data_ptr())
        got = d_i.cpu().numpy()
        for r in range(rows):
            np.testing.assert_array_equal(got[r], top_n_ascending(keys[r], n))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("hd", [32, 128])
def test_quantizer_bit_exact(bits, hd):
    rng = np.random.default_rng(bits * 1000 + hd)
    rows = 4096
    mags = np.float32(10.0) ** rng.uniform(-9, 5.5, size=(rows, 1)).astype(np.float32)
    x = (rng.standard_normal((rows, hd)).astype(np.float32) * mags).astype(np.float32)
    x[::17] = 0.0                                   # zero groups
    x[5, :32] = np.float32(7.0 * (1 + 2 ** -11))    # fp16 tie in the scale (int4)
    x[6, :32] = 1e6                                 # saturating scale
    log(f"quantize bits={bits} hd={hd}")
    d_x = torch.from_numpy(x).cuda()
    nb = hd * bits // 8
    d_c = torch.zeros((rows, nb), dtype=torch.uint8, device="cuda")
    d_s = torch.zeros((rows, hd // 32), dtype=torch.int16, device="cuda")
    B.lk_dbg_quantize(d_x.data_ptr(), rows, hd, bits, d_c.data_ptr(), d_s.data_ptr())
    codes, s16 = quant.quantize(x, bits)
    exp_c = quant.pack_int4(codes) if bits == 4 else codes.view(np.uint8)
    np.testing.assert_array_equal(d_c.cpu().numpy(), exp_c)
    np.testing.assert_array_equal(d_s.cpu().numpy().view(np.uint16), s16.view(np.uint16))


def test_delta_keys():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((300, 2048)).astype(np.float32)
    b = a + rng.standard_normal((300, 2048)).astype(np.float32) * np.float32(0.01)
    d_k = torch.empty(300, dtype=torch.float32, device="cuda")
    d_a, d_b = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()   # keep both alive
    B.lk_dbg_delta(d_a.data_ptr(), d_b.data_ptr(), 300, 2048, d_k.data_ptr())
    torch.cuda.synchronize()
    ref = ((a.astype(np.float64) - b) ** 2).sum(1)
    np.testing.assert_allclose(d_k.cpu().numpy(), ref, rtol=1e-5)


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (8, 3072, 2048), (16, 192, 64), (17, 64, 64),
                                   (300, 192, 64), (1000, 3072, 2048), (257, 2048, 5632)])
def test_gemm_against_float64(M, N, K):
    rng = np.random.default_rng(M * 7 + N)
    a = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    log(f"gemm M={M} N={N} K={K}")
    d_a, d_w = a.cuda(), w.cuda()   # keep both alive until the kernel has run
    B.lk_dbg_gemm(d_a.data_ptr(), d_w.data_ptr(), c.data_ptr(), M, N, K)
    torch.cuda.synchronize()
    ref = a.double() @ w.double().T
    assert max_abs_rel(c.cpu().numpy(), ref.numpy()) < 1e-4


@pytest.mark.parametrize("epi", [0, 1, 2, 3])
@pytest.mark.parametrize("M,N,K", [(513, 1024, 2048), (256, 256, 5632), (4100, 4096, 128), (300, 192, 64),
                                   (8, 256, 128)])
def test_gemm_epilogues_against_float64(epi, M, N, K):
    """Fused epilogues (store, residual add, SwiGLU, exact-erf GELU) on the big-tile path
    (M >= 256, K % 128 == 0; at 4100 x 4096 there are more tiles than workgroups, so a
    workgroup runs several), the tiled path and the decode path, against float64."""
    rng = np.random.default_rng(epi * 131 + M + N)
    rows = 2 * N if epi == 2 else N
    a = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((rows, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    c0 = rng.standard_normal((M, N)).astype(np.float32)
    log(f"gemm epi={epi} M={M} N={N} K={K}")
    d_a, d_w = a.cuda(), w.cuda()
    d_c = torch.from_numpy(c0).cuda()
    d_o = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    B.lk_dbg_gemm_epi(d_a.data_ptr(), d_w.data_ptr(), epi, d_c.data_ptr(), d_o.data_ptr(), M, N, K)
    torch.cuda.synchronize()
    p = a.double() @ w.double().T
    if epi == 0:
        assert max_abs_rel(d_c.cpu().numpy(), p.numpy()) < 1e-4
    elif epi == 1:
        ref = c0.astype(np.float64) + p.numpy()
        assert max_abs_rel(d_c.cpu().numpy(), ref) < 1e-4
    else:
        if epi == 2:
            g, u = p[:, :N].numpy(), p[:, N:].numpy()
            ref = g / (1.0 + np.exp(-g)) * u
        else:
            x = p.numpy()
            ref = 0.5 * x * (1.0 + scipy.special.erf(x / math.sqrt(2.0)))
        out = d_o.float().cpu().numpy().astype(np.float64)
        # bf16 output: half an ulp (2^-9 relative) plus the fp32 accumulation error
        assert np.all(np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())


def test_entry_points_reject_bad_sizes():
    with pytest.raises(B.LKError):
        B.lk_dbg_topk(1, 1, 4, 5, 1)          # n > cols, refused before launch
    with pytest.raises(B.LKError):
        B.lk_dbg_quantize(1, 1, 48, 4, 1, 1)  # hd not a multiple of 32
    with pytest.raises(B.LKError):
        B.lk_dbg_gemm(1, 1, 1, 4, 20, 64)     # N not a multiple of 16
