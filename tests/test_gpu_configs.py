"""GPU parity at the full model sizes, through the C ABI.

* 0.6B-shaped (bf16): teacher-forced verify rows vs the fp64 oracle
  (|dlogit| <= 3e-2, argmax equal away from near-ties); verify == decode bit
  for bit for K in {1, 2, 4, 8}; the speculative loop with 40 % draft
  corruption commits exactly the GPU's own greedy decode.
* Gemma-style int4: oracle rows within 6e-2; the 87-id prefix built three
  ways (one-token commits, 9-row block commits, one prefill) gives identical
  KV bits, and K = 8 / 16 verifies match across histories and match per-row
  one-token decodes.
* 8B-shaped (bf16): sampled oracle rows (the oracle scores them one forward
  at a time) and verify == decode for K = 4.
The oracle runs on this host; its inputs are the same seeded weights.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TOL = {"bf16": 3e-2, "int4": 6e-2}


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _check_rows_vs_oracle(sess, weights, prefix, drafts, label):
    from oracle import Fp64Model, forward_cacheless
    from oracle.spec import greedy_id, top2_margin
    cfg = weights.cfg
    tol = TOL[cfg.weight_fmt]
    sess.set_debug(True)
    nx = sess.prefill(prefix)
    sess.verify(drafts)
    seq = list(prefix) + [nx] + list(drafts)
    P = len(prefix)
    ref = forward_cacheless(Fp64Model(weights, cache=False), seq, positions=np.arange(P, P + len(drafts) + 1))
    worst, flips = 0.0, 0
    for r in range(len(drafts) + 1):
        lg = sess.logits(r).astype(np.float64)
        worst = max(worst, float(np.max(np.abs(lg - ref[r]))))
        if int(np.argmax(lg)) != greedy_id(ref[r]):
            assert top2_margin(ref[r]) < tol, f"{label}: argmax flip at row {r} away from a near-tie"
            flips += 1
    print(f"{label}: max|dlogit| {worst:.3e} over {len(drafts) + 1} rows, flagged flips {flips}")
    assert worst <= tol


def _verify_vs_decode(dev, snap, drafts, cfg=None):
    from greedy_block_verification_amd.session import Session
    a, b = Session(dev, cfg=cfg), Session(dev, cfg=cfg)
    a.restore(snap)
    b.restore(snap)
    a.set_debug(True)
    b.set_debug(True)
    rows = [a.next_id] + list(drafts)
    dec, dec_arg = [], []
    for t in rows:
        dec_arg.append(a.decode_step(t))
        dec.append(a.logits(0))
    n, nxt = b.verify(drafts)
    assert b.last_argmax() == dec_arg
    for r in range(len(rows)):
        np.testing.assert_array_equal(_bits(b.logits(r)), _bits(dec[r]))
    exp_n = 0
    while exp_n < len(drafts) and drafts[exp_n] == dec_arg[exp_n]:
        exp_n += 1
    assert (n, nxt) == (exp_n, dec_arg[exp_n])
    a.close()
    b.close()


# ------------------------------------------------------------------ 0.6B shape
@pytest.fixture(scope="module")
def q06b():
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights, get_config
    w = generate_weights(get_config("q06b"))
    return DeviceModel(w), w


def test_q06b_rows_match_oracle(q06b):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = q06b
    ids = prompt_ids(w.cfg.seed, 7, 24, w.cfg.vocab).tolist()
    _check_rows_vs_oracle(Session(dev), w, ids[:19], ids[19:23], "q06b")


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_q06b_verify_equals_decode(q06b, k):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = q06b
    s = Session(dev)
    s.prefill(prompt_ids(w.cfg.seed, 0, 512, w.cfg.vocab).tolist())
    snap = s.snapshot()
    rng = np.random.default_rng(50 + k)
    _verify_vs_decode(dev, snap, rng.integers(0, w.cfg.vocab, k).tolist())


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_q06b_spec_loop_commits_greedy_decode(q06b, k):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import DraftSource, prompt_ids
    dev, w = q06b
    ids = prompt_ids(w.cfg.seed, 1, 512, w.cfg.vocab).tolist()
    s = Session(dev)
    nx = s.prefill(ids)
    truth = [nx]
    for _ in range(128):
        truth.append(s.decode_step(truth[-1]))
    s.truncate(512)
    src = DraftSource(w.cfg.seed, 1, w.cfg.vocab, p_correct=0.60)
    out, acc, prop, steps = [], 0, 0, 0
    while len(out) < 128:
        k_eff = min(k, 128 - len(out) - 1)
        c = len(out)
        drafts = src.window(truth[c + 1: c + 1 + k_eff], k_eff) if k_eff else []
        cur = s.next_id
        n, _ = s.verify(drafts)
        out += [cur] + drafts[:n]
        acc, prop, steps = acc + n, prop + k_eff, steps + 1
    assert out == truth[:128]
    assert s.kv_len == 512 + 128
    print(f"q06b K={k}: {steps} verifies, acceptance {acc / max(1, prop):.3f}, tokens/verify {128 / steps:.2f}")


# ------------------------------------------------------------------ Gemma-style int4
@pytest.fixture(scope="module")
def gemma():
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights, get_config
    w = generate_weights(get_config("gemma_int4"))
    return DeviceModel(w), w


def test_gemma_int4_rows_match_oracle(gemma):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = gemma
    ids = prompt_ids(w.cfg.seed, 3, 24, w.cfg.vocab).tolist()
    _check_rows_vs_oracle(Session(dev), w, ids[:15], ids[15:23], "gemma_int4")


def test_gemma_int4_seventeen_rows_match_oracle(gemma):
    """17 rows: the int4 register-operand kernel's two-row-tile form."""
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = gemma
    ids = prompt_ids(w.cfg.seed, 4, 24, w.cfg.vocab).tolist()
    _check_rows_vs_oracle(Session(dev), w, ids[:8], ids[8:24], "gemma_int4 17 rows")


def test_gemma_int4_cache_histories_and_row_decode(gemma):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = gemma
    ids = prompt_ids(w.cfg.seed, 0, 87, w.cfg.vocab).tolist()
    s1, s2, s3 = Session(dev), Session(dev), Session(dev)
    for t in ids:
        nx1 = s1.decode_step(t)
    for i in range(0, 87, 9):
        nx2 = s2.prefill(ids[i:i + 9])
    nx3 = s3.prefill(ids)
    assert nx1 == nx2 == nx3
    kv = s1.kv_positions(87)
    np.testing.assert_array_equal(kv, s2.kv_positions(87))
    np.testing.assert_array_equal(kv, s3.kv_positions(87))
    rng = np.random.default_rng(87)
    for k in (8, 16):
        drafts = rng.integers(0, w.cfg.vocab, k).tolist()
        snaps = [s.snapshot() for s in (s1, s2, s3)]
        outs = []
        for snap in snaps:
            v = Session(dev)
            v.restore(snap)
            v.set_debug(True)
            res = v.verify(drafts)
            outs.append((res, [_bits(v.logits(r)) for r in range(k + 1)]))
            v.close()
        for res, rows in outs[1:]:
            assert res == outs[0][0]
            for r in range(k + 1):
                np.testing.assert_array_equal(rows[r], outs[0][1][r])
        # every row of the verify equals a one-token decode of the same prefix
        _verify_vs_decode(dev, snaps[0], drafts)


# ------------------------------------------------------------------ 8B shape
@pytest.fixture(scope="module")
def q8b(q8b_device):
    return q8b_device


def test_q8b_rows_match_oracle(q8b):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = q8b
    ids = prompt_ids(w.cfg.seed, 9, 12, w.cfg.vocab).tolist()
    _check_rows_vs_oracle(Session(dev), w, ids[:6], ids[6:10], "q8b")


def test_q8b_thirteen_rows_match_oracle(q8b):
    """13 rows: the activation planes of 9-16 rows outgrow one LDS stage, so
    these forwards run the register-operand ring kernel."""
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = q8b
    ids = prompt_ids(w.cfg.seed, 10, 18, w.cfg.vocab).tolist()
    _check_rows_vs_oracle(Session(dev), w, ids[:6], ids[6:18], "q8b 13 rows")


def test_q8b_seventeen_rows_match_oracle(q8b):
    """17 rows: the register-operand ring with row 16 staged in LDS."""
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = q8b
    ids = prompt_ids(w.cfg.seed, 11, 22, w.cfg.vocab).tolist()
    _check_rows_vs_oracle(Session(dev), w, ids[:6], ids[6:22], "q8b 17 rows")


def test_q8b_verify_equals_decode(q8b):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = q8b
    s = Session(dev)
    s.prefill(prompt_ids(w.cfg.seed, 0, 128, w.cfg.vocab).tolist())
    snap = s.snapshot()
    s.close()
    rng = np.random.default_rng(8)
    for k in (4, 16):
        _verify_vs_decode(dev, snap, rng.integers(0, w.cfg.vocab, k).tolist())


def test_q06b_random_operation_sequence(q06b):
    """At the 0.6B shape and contexts of 480-600 positions (8-10 attention
    splits, so the split + combine path): a seeded random sequence of
    verifies (random K, drafts right up to a random index), rollbacks and
    decodes; after each, kv_len, next_id, history, the last forward's
    committed logits rows and every committed position's KV bits equal those
    of a context rebuilt from one-token decodes alone."""
    import numpy as np
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = q06b
    cfg = w.cfg
    rng = np.random.default_rng(7)
    ids = prompt_ids(cfg.seed, 11, 480, cfg.vocab).tolist()
    s = Session(dev)
    s.set_debug(True)
    s.prefill(ids)
    committed = list(ids)
    bits = lambda a: np.asarray(a, dtype=np.float32).view(np.uint32)

    def rebuilt(n):
        r = Session(dev)
        r.set_debug(True)
        logits = []
        for t in committed[:n]:
            r.decode_step(t)
            logits.append(r.logits(0))
        return r, logits

    for _ in range(8):
        op = rng.choice(["verify", "verify", "verify", "truncate", "decode"])
        kv0 = s.kv_len
        if op == "verify":
            k = int(rng.integers(1, cfg.max_k + 1))
            probe, _ = rebuilt(kv0)
            truth, t = [], s.next_id
            for _ in range(k):
                t = probe.decode_step(t)
                truth.append(t)
            probe.close()
            wrong_at = int(rng.integers(0, k + 1))
            drafts = truth[:wrong_at] + [(x + 1) % cfg.vocab for x in truth[wrong_at:]]
            rows = [s.next_id] + drafts
            n, _ = s.verify(drafts)
            assert n == wrong_at
            committed[kv0:] = rows[:n + 1]
            fresh = n + 1
        elif op == "truncate" and kv0 > 461:
            s.truncate(int(rng.integers(460, kv0)))
            del committed[s.kv_len:]
            fresh = 0
        else:
            t = s.next_id
            s.decode_step(t)
            committed[kv0:] = [t]
            fresh = 1
        ref, logits = rebuilt(s.kv_len)
        assert (s.kv_len, s.next_id) == (ref.kv_len, ref.next_id) and s.history() == ref.history()
        np.testing.assert_array_equal(s.kv_positions(s.kv_len), ref.kv_positions(ref.kv_len))
        for r in range(fresh):
            np.testing.assert_array_equal(bits(s.logits(r)), bits(logits[kv0 + r]))
        ref.close()
    s.close()


def test_q8b_random_operation_sequence(q8b):
    """The headline shape under a seeded random sequence of verifies (K up to
    16), rollbacks and decodes: each state equals a context rebuilt from
    one-token decodes alone (kv_len, next_id, history, committed logits rows,
    KV bits)."""
    import numpy as np
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = q8b
    cfg = w.cfg
    rng = np.random.default_rng(8)
    ids = prompt_ids(cfg.seed, 12, 150, cfg.vocab).tolist()
    s = Session(dev)
    s.set_debug(True)
    s.prefill(ids)
    committed = list(ids)
    bits = lambda a: np.asarray(a, dtype=np.float32).view(np.uint32)

    def rebuilt(n):
        r = Session(dev)
        r.set_debug(True)
        logits = []
        for t in committed[:n]:
            r.decode_step(t)
            logits.append(r.logits(0))
        return r, logits

    for _ in range(6):
        op = rng.choice(["verify", "verify", "verify", "truncate", "decode"])
        kv0 = s.kv_len
        if op == "verify":
            k = int(rng.integers(1, cfg.max_k + 1))
            probe, _ = rebuilt(kv0)
            truth, t = [], s.next_id
            for _ in range(k):
                t = probe.decode_step(t)
                truth.append(t)
            probe.close()
            wrong_at = int(rng.integers(0, k + 1))
            drafts = truth[:wrong_at] + [(x + 1) % cfg.vocab for x in truth[wrong_at:]]
            rows = [s.next_id] + drafts
            n, _ = s.verify(drafts)
            assert n == wrong_at
            committed[kv0:] = rows[:n + 1]
            fresh = n + 1
        elif op == "truncate" and kv0 > 141:
            s.truncate(int(rng.integers(140, kv0)))
            del committed[s.kv_len:]
            fresh = 0
        else:
            t = s.next_id
            s.decode_step(t)
            committed[kv0:] = [t]
            fresh = 1
        ref, logits = rebuilt(s.kv_len)
        assert (s.kv_len, s.next_id) == (ref.kv_len, ref.next_id) and s.history() == ref.history()
        np.testing.assert_array_equal(s.kv_positions(s.kv_len), ref.kv_positions(ref.kv_len))
        for r in range(fresh):
            np.testing.assert_array_equal(bits(s.logits(r)), bits(logits[kv0 + r]))
        ref.close()
    s.close()


def test_gemma_int4_random_operation_sequence(gemma):
    """The int4 GeGLU shape (2 KV heads, groups of 6 q heads) under a seeded
    random sequence of verifies (K up to 16), rollbacks and decodes: each
    state equals a context rebuilt from one-token decodes alone."""
    import numpy as np
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = gemma
    cfg = w.cfg
    rng = np.random.default_rng(9)
    ids = prompt_ids(cfg.seed, 13, 87, cfg.vocab).tolist()
    s = Session(dev)
    s.set_debug(True)
    s.prefill(ids)
    committed = list(ids)
    bits = lambda a: np.asarray(a, dtype=np.float32).view(np.uint32)

    def rebuilt(n):
        r = Session(dev)
        r.set_debug(True)
        logits = []
        for t in committed[:n]:
            r.decode_step(t)
            logits.append(r.logits(0))
        return r, logits

    for _ in range(6):
        op = rng.choice(["verify", "verify", "verify", "truncate", "decode"])
        kv0 = s.kv_len
        if op == "verify":
            k = int(rng.integers(1, cfg.max_k + 1))
            probe, _ = rebuilt(kv0)
            truth, t = [], s.next_id
            for _ in range(k):
                t = probe.decode_step(t)
                truth.append(t)
            probe.close()
            wrong_at = int(rng.integers(0, k + 1))
            drafts = truth[:wrong_at] + [(x + 1) % cfg.vocab for x in truth[wrong_at:]]
            rows = [s.next_id] + drafts
            n, _ = s.verify(drafts)
            assert n == wrong_at
            committed[kv0:] = rows[:n + 1]
            fresh = n + 1
        elif op == "truncate" and kv0 > 81:
            s.truncate(int(rng.integers(80, kv0)))
            del committed[s.kv_len:]
            fresh = 0
        else:
            t = s.next_id
            s.decode_step(t)
            committed[kv0:] = [t]
            fresh = 1
        ref, logits = rebuilt(s.kv_len)
        assert (s.kv_len, s.next_id) == (ref.kv_len, ref.next_id) and s.history() == ref.history()
        np.testing.assert_array_equal(s.kv_positions(s.kv_len), ref.kv_positions(ref.kv_len))
        for r in range(fresh):
            np.testing.assert_array_equal(bits(s.logits(r)), bits(logits[kv0 + r]))
        ref.close()
    s.close()
