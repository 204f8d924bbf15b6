"""Seeded random small workloads, bit-exact against the oracle through the
single-call and the split entry points.  Each seed draws its own shape (hot
slots S, top-k width k, requests, layers, page size and resident tail,
padding rows, step count) and per-step mix (kept, recent and uniform
positions, growth), so combinations the hand-picked cases do not reach still
meet the oracle: k = 1, ragged S, batches on both sides of the fused
instance's threshold, fast-path and LRU rows together."""
import numpy as np
import pytest

from tests.harness import run_parity
from workloads import synth

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    S = int(rng.choice([48, 64, 96, 128, 200, 256, 333, 512, 1024, 2048]))
    k = int(rng.integers(1, S + 1))
    R = int(rng.integers(2, 13))
    nb = int(rng.integers(1, R + 1))
    L = int(rng.choice([1, 1, 2, 3]))
    P = int(rng.choice([0, 0, 8, 16]))
    tail = int(rng.choice([0, 2, 4])) * P if P else 0
    n0 = [int(v) for v in rng.integers(1, 6 * S, size=nb)]
    grow = int(rng.choice([0, 1, 5]))
    keep = int(rng.integers(0, k + 1))
    window = int(rng.integers(1, min(n0) + 1))              # the generator needs window <= seq_len
    recent = int(rng.integers(0, min(k - keep, window) + 1))  # and keep + recent <= k
    pad = int(rng.integers(0, 3))
    steps = int(rng.integers(2, 6))
    return dict(R=R, S=S, k=k, steps=steps, n0=n0, L=L, grow=grow, keep=keep, recent=recent,
                recent_window=window, P=P, resident_tail=tail, padding_rows=pad)


@pytest.mark.parametrize("mode", ["resolve", "split"])
@pytest.mark.parametrize("seed", range(64))
def test_random_small_workload_vs_oracle(seed, mode):
    spec = _draw(seed)
    print("[random %s seed %d] S=%d k=%d R=%d L=%d P=%d tail=%d pad=%d steps=%d"
          % (mode, seed, spec["S"], spec["k"], spec["R"], spec["L"], spec["P"],
             spec["resident_tail"], spec["padding_rows"], spec["steps"]), flush=True)
    w = synth("random%d" % seed, 2000 + seed, **spec)
    run_parity(w, mode=mode)
