#!/usr/bin/env python3
"""Lazy looped-Transformer decode benchmark on one MI355X.

Workload (default): 48 shared layers x 4 loops (192 layer applications per
token), d_model 2048, 16 query / 4 KV heads of 128, SwiGLU FFN 5632, batch 8,
32768-token seeded random prompt; lazy cache with rho 0.1, 1024 stable columns
+ 512-token window, int8 base and int4 residuals (group 32, float16 scales).
Weights are seeded N(0, 0.02) rounded to bf16; data is synthetic.

A step is one decode step: every sequence appends one token that runs the whole
looped stack through the library's C ABI.  The prompt is prefilled once (timed
separately).  Prints one JSON line with decode tokens/s, KV bytes per token, the
roofline of the dominant kernel (decode attention over the base KV, timed live
with HIP events on the library's stream) and the CPU oracle timed on a bounded
sample of the same workload.
"""
import argparse
import copy
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "looped-decode tokens/s + KV bytes/token at K=4, 32k ctx; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="deep_48x4_b8_ctx32k")
    ap.add_argument("--mode", default=None, choices=["per_loop", "last_loop", "lazy"])
    ap.add_argument("--prompt", type=int, default=None, help="override the prompt length")
    ap.add_argument("--base-bits", type=int, default=None)
    ap.add_argument("--diff-attn", action="store_true",
                    help="difference-corrected sparse attention (lazy mode)")
    ap.add_argument("--skip-tau", type=float, default=0.0,
                    help="decode-time loop skipping threshold (lazy mode; 0: off)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timer", action="store_true",
                    help="replay the decode step as one graph with no timed kernel class")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 2 GiB device copy (HBM counter calibration)")
    ap.add_argument("--no-drift", action="store_true",
                    help="skip the lazy-versus-dense drift comparison")
    ap.add_argument("--drift-batch", type=int, default=2,
                    help="sequences of the prompt compared lazy versus dense (full context)")
    ap.add_argument("--drift-steps", type=int, default=8)
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the dense per-loop, last-loop and bf16-base decode baselines")
    ap.add_argument("--baseline-steps", type=int, default=32)
    ap.add_argument("--sweep", action="store_true",
                    help="only the rho x residual-bits frontier of the long-context workload: one JSON "
                         "line per point (tokens/s, KV bytes/token, drift against dense per-loop)")
    ap.add_argument("--sweep-steps", type=int, default=64)
    ap.add_argument("--gemm-shapes", action="store_true",
                    help="only time the prefill projection GEMMs of the workload, per shape, next to "
                         "torch.matmul (hipBLASLt, bf16 output) as a reference; one JSON line per shape")
    ap.add_argument("--gemm-filter", default=None, help="with --gemm-shapes: only shapes whose name contains this")
    ap.add_argument("--gemm-reps", type=int, default=10)
    ap.add_argument("--gemm-rows", default="all", choices=["all", "loop1", "lazy"],
                    help="with --gemm-shapes: the loop-1 row count B*T, the lazy-loop one B*n, or both")
    return ap.parse_args()


MFMA_BF16_PEAK_TFLOPS = 2500.0


# warm-up steps of each dense / bf16-base baseline decode
BASELINE_WARMUP = 8


def decode_tokens_needed(warmup, steps, baseline_steps, baselines=True):
    """Decode steps the seeded token draw has to cover: the timed run's warm-up and
    timed steps and, with the baselines, each baseline's warm-up and timed steps."""
    n = warmup + steps
    return max(n, BASELINE_WARMUP + baseline_steps) if baselines else n


def kept_rows(rho, T):
    """Tokens recomputed per sequence at loops k >= 2: ceil(rho T) clamped to [1, T]."""
    return max(1, min(T, math.ceil(rho * T - 1e-9)))


def prefill_gemm_flops(shape, lazy, batch, T):
    """Algorithmic flops of the projection GEMMs (QKV, O, FFN in and out) of one prefill:
    every layer application multiplies its rows by the four weight matrices; prelude,
    coda and dense loops run all B*T rows, lazy loops k >= 2 only the kept rows."""
    s = shape
    qkv_w = (s.n_heads + 2 * s.n_kv_heads) * s.head_dim
    fin = 2 if s.ffn_act == "swiglu" else 1
    per_row = 2 * (qkv_w * s.d_model + s.d_model * s.n_heads * s.head_dim
                   + fin * s.ffn_dim * s.d_model + s.d_model * s.ffn_dim)
    if lazy.mode == "lazy":
        dense_apps = s.n_prelude + s.n_coda + s.n_shared
        sparse_rows = batch * kept_rows(lazy.rho, T) * s.n_shared * (s.n_loops - 1)
    else:
        dense_apps = s.n_prelude + s.n_coda + s.n_shared * s.n_loops
        sparse_rows = 0
    return per_row * (batch * T * dense_apps + sparse_rows)


def prefill_attention_flops(shape, lazy, batch, T):
    """Algorithmic flops of one prefill's dense causal attention launches (prelude, coda
    and loop 1; every loop in the dense modes): Q K^T and P V over the causal half,
    2 hd flops per (query, key <= query, head) each; and of its column-mass launches
    (lazy loop 1): one more Q K^T over the causal half."""
    s = shape
    pairs = T * (T + 1) / 2.0
    dense_layers = s.n_prelude + s.n_coda + (s.n_shared if lazy.mode == "lazy" else s.n_shared * s.n_loops)
    attn = 4.0 * s.head_dim * s.n_heads * pairs * batch * dense_layers
    mass = 2.0 * s.head_dim * s.n_heads * pairs * batch * (s.n_shared if lazy.mode == "lazy" else 0)
    return attn, mass


def decode_run(model, store, dec, warmup, steps, timer=None):
    """Decode `warmup` then `steps` timed steps on a dedicated stream (graph replay);
    returns (seconds of the timed steps, last output)."""
    import torch
    from cross_loop_kv_amd import binding as B
    dout = torch.empty(store.batch, model.shape.d_model, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    B.lk_timing_enable(model.h, timer)
    B.lk_timing_sample(model.h, 1)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            model.decode(store, dec[i], out=dout)
    torch.cuda.synchronize()
    B.lk_timing_read(model.h)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(steps):
            model.decode(store, dec[warmup + i], out=dout)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, dout


def decode_baseline(model, wl, lazy, ids, dec, warmup, steps):
    """Decode throughput of another cache policy over the same device weights (a sibling
    handle): its own prefill of the same prompt (untimed), then timed decode steps."""
    import torch
    Bsz, T = ids.shape
    sib = model.sibling(lazy)
    st = sib.store(Bsz, T, T + warmup + steps)
    t0 = time.time()
    sib.prefill(st, ids)
    torch.cuda.synchronize()
    prefill_s = time.time() - t0
    el, dout = decode_run(sib, st, dec, warmup, steps)
    assert torch.isfinite(dout).all().item()
    shared, _ = st.bytes_used()
    cache = st.cache_bytes()
    t_now = st.length()
    res = {"mode": lazy.mode, "tokens_per_s": round(Bsz * steps / el, 2), "ms_per_step": round(el * 1e3 / steps, 3),
           "steps": steps, "prefill_s": round(prefill_s, 2),
           "kv_bytes_per_token_store_only": round(shared / (Bsz * t_now), 1),
           "kv_bytes_per_token": round((shared + cache) / (Bsz * t_now), 1)}
    if lazy.mode == "lazy":
        res["base_bits"] = lazy.base_bits
        res["res_bits"] = lazy.res_bits
    del st
    sib.close()
    del sib
    torch.cuda.empty_cache()
    log(f"baseline {res}")
    return res


def frontier_sweep(args):
    """The long-context workload's speed / KV-memory / drift frontier: for rho in
    {1, .5, .25, .1} and residual bits in {16, 8, 4}, a lazy prefill of the 65536-token
    prompt and timed decode steps, against dense per-loop inference over the same
    weights, prompt and decode tokens (drift of the prefill outputs and of every
    decode step's output).  One JSON line per point."""
    import torch
    from cross_loop_kv_amd import binding as B
    from cross_loop_kv_amd import inputs as I
    wl = I.workload("long_4p8x8c4_ctx64k")
    s, Bsz, T = wl.shape, wl.batch, wl.prompt
    warm, steps = 8, args.sweep_steps
    ids = torch.from_numpy(I.gen_prompt_ids(s, Bsz, T)).cuda()
    dec = torch.from_numpy(I.gen_decode_ids(s, Bsz, warm + steps)).cuda()
    dense_lz = I.Lazy(mode="per_loop")
    model = B.LoopedModel(s, dense_lz, I.iter_weights(s))

    def run(m, lz):
        st = m.store(Bsz, T, T + warm + steps)
        t0 = time.time()
        p = m.prefill(st, ids)
        torch.cuda.synchronize()
        pf = time.time() - t0
        outs, t_dec = [], 0.0
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for i in range(warm + steps):
                if i == warm:
                    stream.synchronize()
                    t0 = time.perf_counter()
                outs.append(m.decode(st, dec[i]).clone())
        stream.synchronize()
        t_dec = time.perf_counter() - t0
        shared, _ = st.bytes_used()
        cache = st.cache_bytes()
        t_now = st.length()
        info = {"prefill_s": round(pf, 2), "tokens_per_s": round(Bsz * steps / t_dec, 2),
                "kv_bytes_per_token_store_only": round(shared / (Bsz * t_now), 1),
                "kv_bytes_per_token": round((shared + cache) / (Bsz * t_now), 1)}
        del st
        torch.cuda.empty_cache()
        return p, torch.stack(outs[warm:], 0), info

    dp, dd, dinfo = run(model, dense_lz)
    log(f"dense per-loop: {dinfo}")
    E = 2 * s.n_kv_heads * s.head_dim
    dense_tok = 2 * s.n_shared * s.n_loops * E
    for rho in (1.0, 0.5, 0.25, 0.1):
        for bits in (16, 8, 4):
            lz = copy.deepcopy(wl.lazy)
            lz.rho, lz.res_bits = rho, bits
            sib = model.sibling(lz)
            p, d, info = run(sib, lz)
            sib.close()
            del sib
            point = {"sweep": "long_4p8x8c4_ctx64k", "rho": rho, "res_bits": bits, "base_bits": lz.base_bits,
                     "top_s": lz.top_s, "window": lz.window, "decode_steps": steps, **info,
                     "kv_reduction_store_only": round(dense_tok / info["kv_bytes_per_token_store_only"], 3),
                     "dense_per_loop_tokens_per_s": dinfo["tokens_per_s"],
                     "speedup_vs_dense": round(info["tokens_per_s"] / dinfo["tokens_per_s"], 3),
                     "drift_prefill": drift_stats(p, dp), "drift_decode": drift_stats(d, dd)}
            print(json.dumps(point), flush=True)
            del p, d
            torch.cuda.empty_cache()


def gemm_shapes(args):
    """Per-shape timing of the prefill projection GEMMs (library kernel with its fused
    epilogue) at the workload's loop-1 rows (B*T) and lazy-loop rows (B*n)."""
    import torch
    from cross_loop_kv_amd import binding as B
    from cross_loop_kv_amd import inputs as I
    wl = I.workload(args.workload)
    s, lz = wl.shape, wl.lazy
    qkv_w = (s.n_heads + 2 * s.n_kv_heads) * s.head_dim
    hhd = s.n_heads * s.head_dim
    act = 2 if s.ffn_act == "swiglu" else 3
    fin = 2 if s.ffn_act == "swiglu" else 1
    rows = [wl.batch * wl.prompt] if args.gemm_rows != "lazy" else []
    if lz.mode == "lazy" and s.n_loops > 1 and args.gemm_rows != "loop1":
        rows.append(wl.batch * kept_rows(lz.rho, wl.prompt))
    projs = [("qkv", qkv_w, s.d_model, 0), ("o", s.d_model, hhd, 1), ("ffn_in", s.ffn_dim, s.d_model, act),
             ("down", s.d_model, s.ffn_dim, 1)]

    def timeit(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for M in rows:
        for name, N, K, epi in projs:
            if args.gemm_filter and args.gemm_filter not in name:
                continue
            wrows = fin * N if name == "ffn_in" else N
            gen = torch.Generator(device="cuda").manual_seed(M + N)
            a = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
            w = (torch.randn(wrows, K, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
            c = torch.zeros(M, N, device="cuda", dtype=torch.float32)
            o = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
            flops = 2.0 * M * wrows * K
            t_lib = timeit(lambda: B.lk_dbg_gemm_epi(a.data_ptr(), w.data_ptr(), epi, c.data_ptr(), o.data_ptr(),
                                                     M, N, K), args.gemm_reps)
            wt = w.t()
            t_ref = timeit(lambda: torch.matmul(a, wt), args.gemm_reps)
            print(json.dumps({"gemm": name, "M": M, "N": wrows, "K": K, "epilogue": ["store", "add", "swiglu", "gelu"][epi],
                              "ms": round(t_lib, 4), "tflops": round(flops / t_lib / 1e9, 1),
                              "frac": round(flops / t_lib / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                              "ref_hipblaslt_ms": round(t_ref, 4),
                              "ref_frac": round(flops / t_ref / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}), flush=True)
            del a, w, c, o, wt
            torch.cuda.empty_cache()


def drift_stats(a, b):
    """Lazy output a against the dense reference b (final-normed hidden states, last dim
    d): max |a - b| / max |b|, mean per-token cosine similarity, relative L2."""
    import torch
    a64, b64 = a.double(), b.double()
    d = a64.shape[-1]
    cos = torch.nn.functional.cosine_similarity(a64.reshape(-1, d), b64.reshape(-1, d), dim=1)
    return {"max_abs_rel": float((a64 - b64).abs().max() / b64.abs().max()),
            "mean_cos": float(cos.mean()),
            "rel_l2": float((a64 - b64).norm() / b64.norm())}


def measure_drift(model, wl, ids, dec, nb, steps):
    """Prefill the first nb sequences of the prompt at full context and decode `steps`
    tokens, once with the lazy model and once with the dense per-loop model over the same
    weights; compare the outputs."""
    import torch
    from cross_loop_kv_amd import inputs as I
    T = ids.shape[1]
    dense = model.sibling(I.Lazy(mode="per_loop"))
    outs = {}
    for name, m in (("lazy", model), ("dense", dense)):
        st = m.store(nb, T, T + steps)
        p = m.prefill(st, ids[:nb])
        d = [m.decode(st, dec[i][:nb]).clone() for i in range(steps)]
        torch.cuda.synchronize()
        outs[name] = (p, torch.stack(d, 1) if d else None)
        del st
    dense.close()
    res = {"vs": "per_loop (dense looped inference over the same weights)", "batch": nb, "context": T,
           "decode_steps": steps, "prefill_out": drift_stats(outs["lazy"][0], outs["dense"][0])}
    if steps:
        res["decode_out"] = drift_stats(outs["lazy"][1], outs["dense"][1])
    return res


def decode_attention_bytes(shape, lazy, batch, t):
    """Algorithmic bytes of one loop-1 decode-attention launch at context length t+1:
    K and V rows of every (sequence, KV head) read once, q read, partials written."""
    hd, Hkv, H = shape.head_dim, shape.n_kv_heads, shape.n_heads
    if lazy.mode == "lazy" and lazy.base_bits == 8:
        per_elem = 1.0 + 2.0 / 32
    else:
        per_elem = 2.0
    kv = batch * Hkv * (t + 1) * 2 * hd * per_elem
    return kv + batch * H * hd * 2


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_decode_dense_i8_deep_48x4_b8_ctx32k_traffic.md")


def kernel_source_hash():
    """Hash of the source the loop-1 decode-attention kernel is built from: the
    attention file's helpers (up to the flash prefill section) and its dense decode
    section (up to the sparse-gather section), the KV-store address arithmetic of
    the common header, and the new token's K/V writer of the kernel header."""
    import hashlib
    att = open(os.path.join(ROOT, "cross_loop_kv_amd", "csrc", "k_attn.hip")).read()
    com = open(os.path.join(ROOT, "cross_loop_kv_amd", "csrc", "lk_common.h")).read()
    ker = open(os.path.join(ROOT, "cross_loop_kv_amd", "csrc", "lk_kernels.h")).read()
    mark = "// ---------------------------------------------------------------- "
    a = att.index("typedef _Float16 half8")
    a2 = att.index(mark + "flash prefill")
    d = att.index(mark + "dense decode (MFMA)")
    b = att.index(mark + "sparse decode: gather")
    c = com.index(mark + "KV store views")
    k0 = ker.index("// Element e of one token's K")
    k1 = ker.index("// ---- GEMM")
    return hashlib.sha256((att[a:a2] + att[d:b] + com[c:] + ker[k0:k1]).encode()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the loop-1 int8 decode attention from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (copy-calibrated), or None when the
    summary is for another workload or the kernel source changed since it was taken."""
    import re
    if workload != "deep_48x4_b8_ctx32k" or not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    sha = re.search(r"^kernel_source_hash: ([0-9a-f]+)$", txt, re.M)
    val = re.search(r"^traffic_bytes_per_launch: (\d+)$", txt, re.M)
    if not (sha and val):
        return None
    return int(val.group(1)) if kernel_source_hash() == sha.group(1) else None


def cpu_baseline(wl, n_steps=8, rng_seed=3):
    """The oracle on a bounded sample: ``n_steps`` decode steps of the full batch at
    the full context through ONE shared layer x K loops, on a synthetic store state
    (what a prefill leaves: base, kept-row residuals, slot maps, column sets),
    scaled to the R shared layers of the workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from cross_loop_kv_amd import inputs as I
    from oracle.model import LoopedOracle
    from oracle.select import n_selected

    s1 = copy.deepcopy(wl.shape)
    s1.n_shared = 1
    R_full = wl.shape.n_shared
    W = I.gen_weights(s1)
    B, T, lz = wl.batch, wl.prompt, wl.lazy
    Tm = T + n_steps
    m = LoopedOracle(s1, lz, W, B, Tm)
    rng = np.random.default_rng(rng_seed)
    Hkv, hd, K = s1.n_kv_heads, s1.head_dim, s1.n_loops
    if lz.mode == "lazy":
        # a synthetic prefill state: base rows, kept-row residuals, slot maps, column sets
        n = n_selected(lz.rho, T)
        ng = hd // lz.group

        def rows(n_rows, qmax, scale):
            if qmax is None:
                return rng.standard_normal((B, Hkv, n_rows, hd), np.float32)
            return (rng.integers(-qmax, qmax + 1, (B, Hkv, n_rows, hd), dtype=np.int8),
                    np.full((B, Hkv, n_rows, ng), scale, np.float16))

        base = [[rows(Tm, None if lz.base_bits == 16 else 127, 0.01) for _ in range(2)]]
        qres = None if lz.res_bits == 16 else 2 ** (lz.res_bits - 1) - 1
        res = {(k, 0, kv): rows(n + n_steps, qres, 0.001) for k in range(2, K + 1) for kv in range(2)}
        slot = np.full((K, B, Tm), -1, np.int32)
        for k in range(2, K + 1):
            for b in range(B):
                slot[k - 1, b, np.sort(rng.choice(T, n, replace=False))] = np.arange(n, dtype=np.int32)
        ncols = min(lz.top_s, T)
        S = [[[np.sort(rng.choice(T, ncols, replace=False)).astype(np.int32) for _ in range(Hkv)]
              for _ in range(B)]]
        m.start_from_state(T, base, res, slot, S)
    else:
        m.T = m.t = T   # dense rows of a T-token prompt, left at zero
    ids = I.gen_decode_ids(s1, B, n_steps)
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    with threadpool_limits(limits=cores):
        t0 = time.time()
        for i in range(n_steps):
            m.decode(ids[i])
        dt = time.time() - t0
    step_s = dt / n_steps * R_full
    return {"value": B / step_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"{n_steps} decode steps of batch {B} at context {T + 1}..{T + n_steps} through 1 shared "
                       f"layer x {s1.n_loops} loops ({s1.n_loops} layer applications each) on a synthetic store, "
                       f"{dt:.1f} s, scaled x{R_full} to the {R_full}-layer stack")}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the path runs on a single MI355X and has no multi-GPU "
              "mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from cross_loop_kv_amd import binding as B
    from cross_loop_kv_amd import inputs as I

    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)
    if args.gemm_shapes:
        gemm_shapes(args)
        return
    if args.sweep:
        frontier_sweep(args)
        return
    wl = I.workload(args.workload)
    if args.prompt:
        wl.prompt = args.prompt
    if args.mode:
        wl.lazy.mode = args.mode
    if args.base_bits:
        wl.lazy.base_bits = args.base_bits
    if args.diff_attn:
        wl.lazy.diff_attn = True
    if args.skip_tau:
        wl.lazy.skip_tau = args.skip_tau
    s, lz = wl.shape, wl.lazy
    Bsz, T = wl.batch, wl.prompt
    total_tokens = T + args.warmup + args.steps

    t0 = time.time()
    model = B.LoopedModel(s, lz, I.iter_weights(s))
    torch.cuda.synchronize()
    log(f"weights: {model.weight_bytes() / 1e9:.2f} GB in {time.time() - t0:.1f}s")
    store = model.store(Bsz, T, total_tokens)
    log(f"store: {store.need / 1e9:.2f} GB allocated for {total_tokens} tokens")
    ids = torch.from_numpy(I.gen_prompt_ids(s, Bsz, T)).cuda()
    # decode tokens for the timed run and for the baselines
    n_dec = decode_tokens_needed(args.warmup, args.steps, args.baseline_steps, not args.no_baselines)
    dec = torch.from_numpy(I.gen_decode_ids(s, Bsz, n_dec)).cuda()
    torch.cuda.synchronize()
    # every projection GEMM, dense attention and column-mass launch of the prefill runs
    # between two HIP events
    B.lk_timing_enable(model.h, "gemm_prefill,attn_prefill,column_mass")
    B.lk_timing_sample(model.h, 0)
    t0 = time.time()
    out = model.prefill(store, ids)
    torch.cuda.synchronize()
    prefill_s = time.time() - t0
    g_launches, g_ms = B.lk_timing_read_class(model.h, "gemm_prefill")
    a_launches, a_ms = B.lk_timing_read_class(model.h, "attn_prefill")
    m_launches, m_ms = B.lk_timing_read_class(model.h, "column_mass")
    B.lk_timing_read(model.h)
    assert torch.isfinite(out).all().item(), "non-finite prefill output"
    del out
    log(f"prefill {Bsz}x{T}: {prefill_s:.2f}s (projection GEMMs {g_ms / 1e3:.2f}s over {g_launches} launches)")
    g_flops = prefill_gemm_flops(s, lz, Bsz, T)
    g_tflops = g_flops / (g_ms * 1e-3) / 1e12 if g_ms > 0 else 0.0

    dout = torch.empty(Bsz, s.d_model, dtype=torch.float32, device="cuda")
    # Decode runs on a dedicated stream (default priority): the library captures the
    # step as HIP graphs there during warmup and replays them, launching the timed
    # attention kernel (one launch per step) directly between two events.  The timer
    # is on from the start; the read after warmup clears the warmup launches.
    stream = torch.cuda.Stream()
    B.lk_timing_enable(model.h, None if args.no_kernel_timer else "attn_decode_dense")
    # time the first loop-1 attention launch of every step: every launch of a step has
    # the same size, and one timed launch keeps the replayed step in two graphs
    B.lk_timing_sample(model.h, 1)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            model.decode(store, dec[i], out=dout)
    torch.cuda.synchronize()
    B.lk_timing_read(model.h)
    t_first = store.length()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            model.decode(store, dec[args.warmup + i], out=dout)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launches, kern_ms = B.lk_timing_read(model.h)
    B.lk_timing_enable(model.h, None)
    assert torch.isfinite(dout).all().item(), "non-finite decode output"
    ms_per_step = elapsed * 1e3 / args.steps
    value = Bsz * args.steps / elapsed

    # roofline of the dominant kernel: loop-1 (dense) decode attention
    n_class = s.n_prelude + s.n_coda + (s.n_shared if lz.mode == "lazy" else s.n_shared * s.n_loops)
    per_step_launches = launches / args.steps if args.steps else 0
    bytes_tot = sum(decode_attention_bytes(s, lz, Bsz, t_first + i) for i in range(args.steps)) \
        * per_step_launches
    avg_ms = kern_ms / max(launches, 1)
    bytes_per_launch = bytes_tot / max(launches, 1)
    achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9 if launches else 0.0

    shared, total = store.bytes_used()
    cache = store.cache_bytes()
    t_now = store.length()
    kv_tok_shared = shared / (Bsz * t_now)
    kv_tok_resident = (shared + cache) / (Bsz * t_now)
    E = 2 * s.n_kv_heads * s.head_dim
    dense_per_loop = 2 * s.n_shared * s.n_loops * E
    if args.calibrate_copy:
        x = torch.empty(2 ** 29, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random ids, seeded N(0,0.02) bf16 weights)",
        "config": {"workload": args.workload, "batch": Bsz, "context": T,
                   "shared_layers": s.n_shared, "loops": s.n_loops, "prelude": s.n_prelude,
                   "coda": s.n_coda, "d_model": s.d_model, "heads": s.n_heads,
                   "kv_heads": s.n_kv_heads, "ffn": s.ffn_dim, "mode": lz.mode, "rho": lz.rho,
                   "top_s": lz.top_s, "window": lz.window, "base_bits": lz.base_bits,
                   "res_bits": lz.res_bits, "layer_applications": model.effective_depth(),
                   **({"diff_attn": True} if getattr(lz, "diff_attn", False) else {}),
                   **({"skip_tau": lz.skip_tau} if getattr(lz, "skip_tau", 0.0) else {})},
        "kv_bytes_per_token": round(kv_tok_resident, 1),
        "kv_bytes_per_token_dense_per_loop": dense_per_loop,
        "kv_reduction_vs_dense_per_loop": round(dense_per_loop / kv_tok_resident, 3),
        "kv_bytes_per_token_store_only": round(kv_tok_shared, 1),
        "kv_reduction_store_only": round(dense_per_loop / kv_tok_shared, 3),
        "decode_cache_bytes": cache,
        "kv_bytes_total_per_token": round(total / (Bsz * t_now), 1),
        "prefill_s": round(prefill_s, 3),
        "prefill_tokens_per_s": round(Bsz * T / prefill_s, 1),
        "roofline": {"kernel": "attn_decode_dense_kernel (decode attention over the loop-1 base)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload) if lz.mode == "lazy" and lz.base_bits == 8 else None,
                     "launches_timed": launches, "launches_per_step": n_class,
                     "avg_launch_us": round(avg_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": int(bytes_per_launch),
                     "share_of_step": round(avg_ms * n_class / ms_per_step, 4)},
    }
    res["roofline_gemm"] = {
        "kernel": "gemm_big_kernel (prefill QKV, O, gate/up, down)", "bound": "mfma",
        "achieved": round(g_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(g_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "launches_timed": g_launches,
        "algorithmic_flops": int(g_flops), "time_ms": round(g_ms, 2)}
    if getattr(lz, "skip_tau", 0.0) and lz.mode == "lazy" and s.n_loops > 1:
        # share of the decode tokens' loop-k rows (k >= 2) that were stored, from the slot maps
        v = store.view()
        off = int(v.slot_maps) - store.buf.data_ptr()
        sm = store.buf[off:off + (s.n_loops - 1) * Bsz * v.row_stride * 4].view(torch.int32)
        sm = sm.view(s.n_loops - 1, Bsz, v.row_stride)[:, :, T:t_now]
        res["skip"] = {"tau": lz.skip_tau, "decode_loop_rows_stored_frac": round(float((sm >= 0).float().mean()), 4)}
    a_flops, m_flops = prefill_attention_flops(s, lz, Bsz, T)
    res["roofline_prefill_attention"] = {
        "kernel": "attn_prefill_fa_kernel (loop-1 causal attention over the prompt)", "bound": "mfma",
        "achieved": round(a_flops / (a_ms * 1e-3) / 1e12, 1) if a_ms > 0 else None,
        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(a_flops / (a_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4) if a_ms > 0 else None,
        "launches_timed": a_launches, "algorithmic_flops": int(a_flops), "time_ms": round(a_ms, 2),
        "column_mass": {"achieved": round(m_flops / (m_ms * 1e-3) / 1e12, 1) if m_ms > 0 else None,
                        "frac": round(m_flops / (m_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4) if m_ms > 0 else None,
                        "launches_timed": m_launches, "algorithmic_flops": int(m_flops),
                        "time_ms": round(m_ms, 2)}}
    if not args.no_baselines and lz.mode == "lazy":
        # the same workload under the dense per-loop cache, the last-loop-only cache and a
        # bf16 loop-1 base, on the same weights, prompt and decode tokens
        del store
        torch.cuda.empty_cache()
        base = []
        for blz in (I.Lazy(mode="per_loop"), I.Lazy(mode="last_loop"),
                    I.Lazy(**{**lz.__dict__, "base_bits": 16})):
            base.append(decode_baseline(model, wl, blz, ids, dec, BASELINE_WARMUP, args.baseline_steps))
        res["baselines"] = {b["mode"] + ("_bf16_base" if b.get("base_bits") == 16 else ""): b for b in base}
        res["baselines"]["lazy_speedup_vs_per_loop"] = round(value / base[0]["tokens_per_s"], 3)
        store = None
    if not args.no_drift:
        del store
        log(f"drift: lazy vs dense per-loop, {args.drift_batch} sequences at context {T}...")
        res["drift"] = measure_drift(model, wl, ids, dec, min(args.drift_batch, Bsz), args.drift_steps)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)...")
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
