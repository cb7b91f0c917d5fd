"""Host-side logic of bench.py (no GPU): the decode-token draw covers every decode run
that indexes it."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.mark.parametrize("warmup,steps,baseline_steps", [(5, 20, 32), (64, 256, 32), (0, 1, 32), (8, 4, 100)])
def test_decode_tokens_cover_the_timed_run_and_the_baselines(warmup, steps, baseline_steps):
    """decode_run reads rows 0 .. warmup + steps - 1 of the draw; each baseline reads rows
    0 .. BASELINE_WARMUP + baseline_steps - 1 of the same draw.  A short timed run
    (the driver's --steps 20 --warmup 5) once indexed past a draw sized for itself alone."""
    b = _bench()
    n = b.decode_tokens_needed(warmup, steps, baseline_steps)
    assert n >= warmup + steps
    assert n >= b.BASELINE_WARMUP + baseline_steps
    assert b.decode_tokens_needed(warmup, steps, baseline_steps, baselines=False) == warmup + steps


def test_committed_traffic_summary_is_of_the_current_kernel_source():
    """The bench line's roofline traffic comes from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of the loop-1 decode attention, which records a hash of the
    source that kernel is built from; the summary must be of the current source (else
    the bench reports the traffic as null until the counters are taken again)."""
    b = _bench()
    t = b.measured_traffic("deep_48x4_b8_ctx32k")
    assert t is not None, "re-take the counters: the kernel source changed since they were taken"
    # within 2 % of the algorithmic bytes at the summary's context (8 x 4 x 32771 x 272 + q)
    alg = 8 * 4 * 32771 * 272 + 8 * 16 * 128 * 2
    assert alg <= t <= 1.02 * alg
