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
