"""lk_looped_decode_step_static (the decode step for callers that cannot allocate: its
workspace is the library's static per-GPU array) against lk_looped_decode_step with a
caller workspace, through the C ABI: twin stores prefilled alike, decoded step by step,
one through each entry point; the outputs and the stores' state must be equal bit for
bit.  Two calls in a row on one GPU, the second with a smaller batch (the array keeps
the first call's contents)."""
import numpy as np
import pytest
import torch

from cross_loop_kv_amd import binding as B
from cross_loop_kv_amd import inputs as I
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _shape():
    return I.Shape(vocab=512, d_model=256, n_heads=8, n_kv_heads=2, head_dim=64, ffn_dim=512, ffn_act="swiglu",
                   n_prelude=1, n_shared=2, n_loops=3, n_coda=1)


def _twin_steps(model, Bsz, T, steps, seed):
    ids = torch.from_numpy(I.gen_prompt_ids(model.shape, Bsz, T, seed=seed))
    dec = torch.from_numpy(I.gen_decode_ids(model.shape, Bsz, steps, seed=seed + 1)).cuda()
    a, b = model.store(Bsz, T, T + steps), model.store(Bsz, T, T + steps)
    a.buf.zero_()      # the snapshots below also hold the never-written parts of each buffer
    b.buf.zero_()
    model.prefill(a, ids)
    model.prefill(b, ids)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for i in range(steps):
        oa = torch.empty(Bsz, model.shape.d_model, dtype=torch.float32, device="cuda")
        with torch.cuda.stream(side):
            ref = model.decode(a, dec[i]).clone()                      # caller workspace, graph replay
            d = dec[i].to(torch.int32).contiguous()
            B.lk_looped_decode_step_static(model.h, b.s, d.data_ptr(), oa.data_ptr())
        side.synchronize()
        assert torch.equal(oa, ref), f"batch {Bsz} step {i}"
    assert a.length() == b.length() == T + steps
    sa, sb = a.export(), b.export()
    assert np.array_equal(sa, sb), "store state differs"


def test_static_scratch_decode_matches_workspace_decode():
    s = _shape()
    lz = I.Lazy(mode="lazy", rho=0.3, top_s=24, window=16, base_bits=8, res_bits=4)
    model = B.LoopedModel(s, lz, I.gen_weights(s, seed=41))
    _twin_steps(model, 6, 120, 3, seed=43)
    _twin_steps(model, 2, 90, 2, seed=47)     # a smaller batch on the same array
    log("  static-scratch decode equals the workspace decode bit for bit (batch 6, then 2)")
