"""Batched greedy block verify (several sequences in one forward), through the C ABI.

Rows of different sequences meet only in the weight GEMMs, whose per-row
arithmetic ignores the other rows, and each row attends to its own
sequence's cache; so every context must end exactly as sv_verify on it
alone leaves it -- (n, next), observer logits bits, argmax, history and KV
bits -- whatever else the batch holds and in whatever order:
* tiny: 6 sequences of different lengths, window sizes 0..8 and draft
  patterns, against one-at-a-time verifies; the same batch reversed and
  regrouped; a batch of 9 sequences (81 rows) through the row-tiled kernels;
  argument errors that leave every context untouched; in both batches every
  row's logits also against the fp64 oracle's cacheless recompute of its
  own sequence (|dlogit| <= 3e-2, argmax equal away from flagged near ties),
  the equality with the plain greedy computation that "Phase 23:
  Speculative Verify Parity", section 3, reports as matched;
* 8B shape: 8 sequences x K = 4 (40 rows) against one-at-a-time verifies;
* Gemma-style int4 layers (GeGLU, 6 q heads per KV head): 4 sequences,
  19 rows, against one-at-a-time verifies;
* tiny, seeded: 10 rounds over 4 sequences with random rollbacks, a random
  subset and order of sequences per batch and random window sizes 0..8,
  against mirror contexts verified one at a time.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


@pytest.fixture(scope="module")
def tiny():
    import torch
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights, get_config
    assert torch.cuda.is_available()
    cfg = get_config("tiny")
    w = generate_weights(cfg)
    return DeviceModel(w), w, cfg


def _ids(n, idx, vocab, seed=21):
    from seeded_inputs import prompt_ids
    return prompt_ids(seed, idx, n, vocab).tolist()


def _contexts(dm, cfg, lens, seed=21, **kw):
    """Sessions prefilled with prompts of the given lengths, and their snapshots."""
    from greedy_block_verification_amd.session import Session
    ss, snaps = [], []
    for i, n in enumerate(lens):
        s = Session(dm, cfg=cfg, **(kw if i == 0 else {}))
        s.prefill(_ids(n, i, cfg.vocab, seed))
        s.set_debug(True)
        ss.append(s)
        snaps.append(s.snapshot())
    return ss, snaps


def _truth(dm, cfg, snap, k):
    """The greedy continuation after a snapshot's prefix (next_id first)."""
    from greedy_block_verification_amd.session import Session
    s = Session(dm, cfg=cfg)
    s.restore(snap)
    out = [s.next_id]
    for _ in range(k):
        out.append(s.decode_step(out[-1]))
    s.close()
    return out


def _drafts(dm, cfg, snaps, ks, seed):
    """Per sequence: a window that matches the greedy continuation up to a
    random point and is random after it."""
    rng = np.random.default_rng(seed)
    out = []
    for snap, k in zip(snaps, ks):
        if k == 0:
            out.append([])
            continue
        t = _truth(dm, cfg, snap, k)
        cut = int(rng.integers(0, k + 1))
        d = t[1:cut + 1] + rng.integers(0, cfg.vocab, k - cut).tolist()
        out.append(d)
    return out


def _alone(dm, cfg, snap, drafts):
    """sv_verify on one context restored from snap: (n, next), logits bits,
    argmax, history, KV bits of the window's positions."""
    from greedy_block_verification_amd.session import Session
    s = Session(dm, cfg=cfg)
    s.restore(snap)
    s.set_debug(True)
    kv0 = s.kv_len
    n, nx = s.verify(drafts)
    res = dict(n=n, nx=nx, arg=s.last_argmax(), logits=[_bits(s.logits(r)) for r in range(len(drafts) + 1)],
               hist=s.history(), kv=s.kv_positions(s.kv_len, kv0), kv_len=s.kv_len)
    s.close()
    return res


def _check(s, got, ref, m):
    assert got == (ref["n"], ref["nx"])
    assert s.kv_len == ref["kv_len"] and s.next_id == ref["nx"]
    assert s.last_argmax() == ref["arg"]
    for r in range(m):
        np.testing.assert_array_equal(_bits(s.logits(r)), ref["logits"][r])
    assert s.history() == ref["hist"]
    np.testing.assert_array_equal(s.kv_positions(ref["kv_len"], ref["kv_len"] - ref["n"] - 1), ref["kv"])


def _check_oracle(w, cfg, ss, lens, drafts, seed, label):
    """Teacher-forced: row r of sequence i scores prompt_i + next_i +
    drafts_i[:r] in the fp64 oracle (forward_cacheless of that sequence)."""
    from oracle import Fp64Model, forward_cacheless
    from oracle.spec import greedy_id, top2_margin
    tol = 3e-2
    m = Fp64Model(w)
    worst, flips, rows = 0.0, 0, 0
    for i, (s, n, d) in enumerate(zip(ss, lens, drafts)):
        hist = s.history(n)
        seq = _ids(n, i, cfg.vocab, seed) + [hist[n - 1]] + list(d)
        ref = forward_cacheless(m, seq, positions=np.arange(n, n + len(d) + 1))
        for r in range(len(d) + 1):
            lg = s.logits(r).astype(np.float64)
            worst = max(worst, float(np.max(np.abs(lg - ref[r]))))
            if int(np.argmax(lg)) != greedy_id(ref[r]):
                assert top2_margin(ref[r]) < tol, f"{label}: sequence {i} row {r} flips away from a near tie"
                flips += 1
            rows += 1
    print(f"{label}: {rows} batched rows vs the oracle, max|dlogit| {worst:.3e}, flagged flips {flips}")
    assert worst <= tol


def _run_batch(ss, snaps, drafts):
    from greedy_block_verification_amd import binding as B
    for s, snap in zip(ss, snaps):
        s.restore(snap)
    return B.sv_verify_batch([s.ctx for s in ss], [s.kv_len for s in ss], drafts)


def test_batch_equals_one_at_a_time(tiny):
    dm, w, cfg = tiny
    lens = [32, 5, 77, 40, 1, 120]
    ks = [4, 0, 8, 3, 8, 1]
    ss, snaps = _contexts(dm, cfg, lens)
    drafts = _drafts(dm, cfg, snaps, ks, seed=1)
    refs = [_alone(dm, cfg, snap, d) for snap, d in zip(snaps, drafts)]
    got = _run_batch(ss, snaps, drafts)
    for s, g, ref, k in zip(ss, got, refs, ks):
        _check(s, g, ref, k + 1)
    _check_oracle(w, cfg, ss, lens, drafts, 21, "tiny batch of 6")
    # reversed, and regrouped into two batches: the same bits
    order = list(reversed(range(len(ss))))
    got = _run_batch([ss[i] for i in order], [snaps[i] for i in order], [drafts[i] for i in order])
    for j, i in enumerate(order):
        _check(ss[i], got[j], refs[i], ks[i] + 1)
    for grp in ([0, 2, 4], [5, 3, 1]):
        got = _run_batch([ss[i] for i in grp], [snaps[i] for i in grp], [drafts[i] for i in grp])
        for j, i in enumerate(grp):
            _check(ss[i], got[j], refs[i], ks[i] + 1)
    for s in ss:
        s.close()


def test_batch_through_row_tiled_kernels(tiny):
    """9 sequences x 9 rows = 81 rows: more than one weight-streaming forward
    holds, so ctxs[0] (max_prefill_rows 128) runs the row-tiled kernels."""
    dm, w, cfg = tiny
    lens = [10 + 13 * i for i in range(9)]
    ks = [8] * 9
    ss, snaps = _contexts(dm, cfg, lens, seed=22, prefill_rows=128)
    drafts = _drafts(dm, cfg, snaps, ks, seed=2)
    refs = [_alone(dm, cfg, snap, d) for snap, d in zip(snaps, drafts)]
    got = _run_batch(ss, snaps, drafts)
    for s, g, ref in zip(ss, got, refs):
        _check(s, g, ref, 9)
    _check_oracle(w, cfg, ss, lens, drafts, 22, "tiny row-tiled batch of 9")
    for s in ss:
        s.close()


def test_batch_argument_errors_leave_contexts_untouched(tiny):
    from greedy_block_verification_amd import binding as B
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import get_config
    dm, w, cfg = tiny
    ss, snaps = _contexts(dm, cfg, [20, 30])
    before = [(s.kv_len, s.next_id, s.history()) for s in ss]
    ctx = [s.ctx for s in ss]
    lens = [s.kv_len for s in ss]
    bad = [
        (ctx, [lens[0], lens[1] + 1], [[1], [2]]),          # prefix length mismatch
        ([ctx[0], ctx[0]], [lens[0], lens[0]], [[1], [2]]),  # the same context twice
        (ctx, lens, [[1], [cfg.vocab]]),                    # id out of range
        (ctx, lens, [[1] * (cfg.max_k + 1), [2]]),          # window too long
    ]
    for c, pl, d in bad:
        with pytest.raises(B.SvError):
            B.sv_verify_batch(c, pl, d)
    other = Session(dm, cfg=get_config("tiny", max_ctx=512))
    other.prefill([1, 2, 3])
    with pytest.raises(B.SvError):                          # different capacity
        B.sv_verify_batch([ctx[0], other.ctx], [lens[0], 3], [[1], [2]])
    assert [(s.kv_len, s.next_id, s.history()) for s in ss] == before
    other.close()
    for s in ss:
        s.close()


def test_q8b_batch_of_8_equals_one_at_a_time(q8b_device):
    from seeded_inputs import get_config
    dev, w = q8b_device
    cfg = get_config("q8b")
    lens = [128, 150, 97, 128, 200, 64, 133, 180]
    ks = [4] * 8
    ss, snaps = _contexts(dev, cfg, lens, seed=23)
    drafts = _drafts(dev, cfg, snaps, ks, seed=3)
    refs = [_alone(dev, cfg, snap, d) for snap, d in zip(snaps, drafts)]
    got = _run_batch(ss, snaps, drafts)
    for s, g, ref in zip(ss, got, refs):
        _check(s, g, ref, 5)
    for s in ss:
        s.close()


def test_int4_gemma_layers_batch_equals_one_at_a_time():
    import torch
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights
    from seeded_inputs.configs import layer_variant
    assert torch.cuda.is_available()
    cfg = layer_variant("gemma_int4", n_layers=3, vocab=1024)
    dm = DeviceModel(generate_weights(cfg))
    lens = [87, 40, 12, 66]
    ks = [4, 3, 2, 6]
    ss, snaps = _contexts(dm, cfg, lens, seed=24)
    drafts = _drafts(dm, cfg, snaps, ks, seed=4)
    refs = [_alone(dm, cfg, snap, d) for snap, d in zip(snaps, drafts)]
    got = _run_batch(ss, snaps, drafts)
    for s, g, ref, k in zip(ss, got, refs, ks):
        _check(s, g, ref, k + 1)
    for s in ss:
        s.close()


def test_random_batches_with_rollbacks_track_one_at_a_time(tiny):
    """Seeded rounds: a random subset of four sequences, in random order and
    with random window sizes (0..8) and drafts right up to a random point, is
    verified in one batch while mirror contexts verify the same windows one
    at a time; random rollbacks of single sequences come in between.  After
    every round each batched context equals its mirror: (n, next), kv_len,
    next_id, history, the logits rows of its window and its KV bits."""
    from greedy_block_verification_amd import binding as B
    dm, w, cfg = tiny
    rng = np.random.default_rng(31)
    lens = [20, 33, 7, 61]
    ss, _ = _contexts(dm, cfg, lens, seed=23)
    ms, _ = _contexts(dm, cfg, lens, seed=23)
    for rnd in range(10):
        if rnd % 3 == 2:   # roll one sequence (and its mirror) back
            i = int(rng.integers(0, 4))
            if ss[i].kv_len > 1:
                n = int(rng.integers(1, ss[i].kv_len))
                ss[i].truncate(n)
                ms[i].truncate(n)
        pick = [int(x) for x in rng.permutation(4)[:int(rng.integers(1, 5))]]
        ks = [int(rng.integers(0, cfg.max_k + 1)) for _ in pick]
        pick_ks = [(i, k) for i, k in zip(pick, ks) if ss[i].kv_len + k + 1 <= cfg.max_ctx]
        if not pick_ks:
            continue
        drafts = _drafts(dm, cfg, [ss[i].snapshot() for i, _ in pick_ks], [k for _, k in pick_ks], seed=100 + rnd)
        got = B.sv_verify_batch([ss[i].ctx for i, _ in pick_ks], [ss[i].kv_len for i, _ in pick_ks], drafts)
        for (i, k), d, g in zip(pick_ks, drafts, got):
            kv0 = ms[i].kv_len
            ref = ms[i].verify(d)
            assert tuple(g) == tuple(ref)
            s, m = ss[i], ms[i]
            assert (s.kv_len, s.next_id) == (m.kv_len, m.next_id) and s.history() == m.history()
            for r in range(k + 1):
                np.testing.assert_array_equal(_bits(s.logits(r)), _bits(m.logits(r)))
            np.testing.assert_array_equal(s.kv_positions(s.kv_len), m.kv_positions(m.kv_len))
    for s in ss + ms:
        s.close()
