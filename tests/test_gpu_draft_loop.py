"""Draft model in the loop (draft-then-verify with two contexts), through the C ABI.

* A tiny-shaped draft with its own weights proposes for the tiny target:
  the committed ids equal the target's plain greedy continuation, and the
  draft context's KV bits equal a fresh draft context that decoded the
  committed sequence one id at a time (its rollbacks leave nothing behind).
* The target as its own draft: every window is accepted (the draft's
  catch-up decode after a full acceptance is exercised every round).
* Seeded synthetic proposals: the draft still decodes them; commits match.
* In every loop the committed stream is also checked against the fp64
  oracle, teacher-forced: each committed id is the oracle's greedy id after
  the prompt and the ids committed before it, except where the oracle's
  top-2 gap is under 3e-2 (a flagged near tie, counted) -- the equality with
  plain greedy decoding that "Phase 23: Speculative Verify Parity",
  section 3, reports as matched.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def models():
    import torch
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights, get_config
    assert torch.cuda.is_available()
    tw = generate_weights(get_config("tiny"))
    dw = generate_weights(get_config("tiny", seed=9))
    return DeviceModel(tw), DeviceModel(dw), get_config("tiny")


@pytest.fixture(scope="module")
def target_oracle():
    from oracle import Fp64Model
    from seeded_inputs import generate_weights, get_config
    return Fp64Model(generate_weights(get_config("tiny")))


def _check_oracle(orc, ids, committed, label):
    from oracle import TokenDecoder
    from oracle.spec import greedy_id, top2_margin
    od = TokenDecoder(orc)
    prev = None
    for t in ids:
        prev = od.decode(t)
    flips = 0
    for tok in committed:
        if tok != greedy_id(prev):
            assert top2_margin(prev) < 3e-2, f"{label}: committed id {tok} is not the oracle's greedy id"
            flips += 1
        prev = od.decode(tok)
    print(f"{label}: {len(committed)} committed ids vs the oracle, flagged flips {flips}")


def _truth(dm, ids, n):
    from greedy_block_verification_amd.session import Session
    s = Session(dm)
    out = [s.prefill(ids)]
    for _ in range(n - 1):
        out.append(s.decode_step(out[-1]))
    s.close()
    return out


def _run(target_dm, draft_dm, ids, k, n_commit, proposer=None):
    from greedy_block_verification_amd.draft_loop import DraftLoop, prefill_pair
    from greedy_block_verification_amd.session import Session
    t, d = Session(target_dm), Session(draft_dm)
    prefill_pair(t, d, ids)
    loop = DraftLoop(t, d, proposer)
    got = []
    while len(got) < n_commit:
        got += loop.step(k)
    return t, d, loop, got


@pytest.mark.parametrize("k", [0, 1, 3, 4])
def test_draft_model_loop_commits_greedy_and_keeps_draft_cache_exact(models, target_oracle, k):
    from greedy_block_verification_amd.session import Session
    tm, dm, cfg = models
    from seeded_inputs import prompt_ids
    ids = prompt_ids(31, k, 32, cfg.vocab).tolist()
    t, d, loop, got = _run(tm, dm, ids, k, 40)
    truth = _truth(tm, ids, len(got))
    assert got == truth
    _check_oracle(target_oracle, ids, got, f"draft loop K={k}")
    fresh = Session(dm)
    fresh.prefill(ids)
    for x in got:
        fresh.decode_step(x)
    L = d.kv_len
    assert fresh.kv_len == L
    np.testing.assert_array_equal(d.kv_positions(L), fresh.kv_positions(L))
    for s in (t, d, fresh):
        s.close()


def test_target_as_its_own_draft_accepts_every_window(models, target_oracle):
    tm, dm, cfg = models
    from seeded_inputs import prompt_ids
    ids = prompt_ids(32, 0, 20, cfg.vocab).tolist()
    t, d, loop, got = _run(tm, tm, ids, 4, 30)
    assert loop.accepted == loop.proposed == 4 * loop.steps
    assert got == _truth(tm, ids, len(got))
    _check_oracle(target_oracle, ids, got, "target as its own draft")
    t.close()
    d.close()


def test_synthetic_proposals_still_run_the_draft(models, target_oracle):
    from seeded_inputs import DraftSource, prompt_ids
    tm, dm, cfg = models
    ids = prompt_ids(33, 0, 24, cfg.vocab).tolist()
    truth = _truth(tm, ids, 80)
    src = DraftSource(33, 0, cfg.vocab, p_correct=0.7)
    state = {}

    def proposer(k):
        c = state["t"].kv_len - len(ids)          # committed ids so far
        return src.window(truth[c + 1: c + 1 + k], k)

    from greedy_block_verification_amd.draft_loop import DraftLoop, prefill_pair
    from greedy_block_verification_amd.session import Session
    t, d = Session(tm), Session(dm)
    state["t"] = t
    prefill_pair(t, d, ids)
    loop = DraftLoop(t, d, proposer)
    got = []
    while len(got) < 60:
        got += loop.step(4)
    assert got == truth[:len(got)]
    _check_oracle(target_oracle, ids, got, "synthetic proposals")
    assert 0 < loop.accepted < loop.proposed
    assert d.kv_len == t.kv_len
    t.close()
    d.close()
