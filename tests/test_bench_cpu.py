"""bench.py's CPU-baseline leg on the tiny shape (no GPU): the oracle
comparison it reports counts exactly what it says.

The "GPU" logits here are the oracle's own rows of a verify window, then
copies with one row's argmax moved far away (a mismatch outside a near tie)
or with the top two ids of a row made to tie (a flagged near tie that
flips, when the oracle's top-2 gap is under the tolerance)."""
import numpy as np

import bench
from oracle import Fp64Model, forward_cacheless
from seeded_inputs import generate_weights, get_config, prompt_ids


def _oracle_rows(w, seq, first):
    return list(forward_cacheless(Fp64Model(w, cache=False), seq, positions=np.arange(first, len(seq))))


def test_cpu_baseline_oracle_comparison_counts():
    cfg = get_config("tiny")
    w = generate_weights(cfg)
    ids = prompt_ids(cfg.seed, 0, 6, cfg.vocab).tolist()
    rows = _oracle_rows(w, ids, 3)                 # a 3-row "verify window" at contexts 4..6
    steps = [(4, 1, 10), (4, 0, 12)]
    tol = 3e-2

    exact = bench.cpu_baseline(w, ids, 3, steps, tol, (ids, 3, [r.copy() for r in rows]))
    assert exact["oracle_rows"] == 3 and exact["oracle_max_abs_dlogit"] == 0.0
    assert exact["oracle_argmax_mismatches"] == 0 and exact["near_tie_flips"] == 0
    assert exact["kind"] == "oracle" and exact["value"] > 0
    assert exact["oracle_rows_at"] == "one verify window, contexts 4..6"
    # committed tokens / ((k+1) decodes per verify x s per decode)
    assert np.isclose(exact["value"], 3 / (10 * exact["s_per_decode"]))

    moved = [r.copy() for r in rows]
    a = int(np.argmax(moved[1]))
    b = (a + 1) % cfg.vocab
    moved[1][b] = moved[1][a] + 10.0          # far from any near tie
    r = bench.cpu_baseline(w, ids, 3, steps, tol, (ids, 3, moved))
    assert r["oracle_argmax_mismatches"] == 1 and np.isclose(r["oracle_max_abs_dlogit"], 10.0 + moved[1][a] - rows[1][b])

    # near ties are gaps strictly under tol: a tolerance just above oracle row
    # 2's top-two gap flags it, and a GPU row preferring the runner-up is a
    # flip, not a mismatch; a tolerance equal to the gap does not flag it
    o = rows[2]
    lo, hi = np.argsort(o)[-2:]
    gap = float(o[hi] - o[lo])
    tied = [x.copy() for x in rows]
    tied[2][lo] = o[hi] + 1e-9
    t = bench.cpu_baseline(w, ids, 3, steps, 1.01 * gap, (ids, 3, tied))
    assert t["near_tie_flags"] >= 1 and t["near_tie_flips"] == 1 and t["oracle_argmax_mismatches"] == 0
    t = bench.cpu_baseline(w, ids, 3, steps, gap, (ids, 3, tied))
    assert t["near_tie_flips"] == 0 and t["oracle_argmax_mismatches"] == 1


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2 and "one GPU only" in r.stdout + r.stderr and r.stdout.strip() == ""
