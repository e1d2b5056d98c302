"""Pins of the fp64 oracle against things other than itself (CPU only)."""
import copy
import math

import numpy as np
import pytest

from seeded_inputs import (PATTERNS, DraftSource, generate_weights, get_config,
                           layer_variant, prompt_ids)
from oracle import Fp64Model, TokenDecoder, forward_cacheless
from oracle import model as om
from oracle.spec import (block_verify, greedy_generate, greedy_id, prefill,
                         spec_generate, top2_margin)

import _torch_formulation as tf


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


# ------------------------------------------------ brute force: cacheless recompute
@pytest.mark.parametrize("variant", ["tiny", "q06b", "gemma_int4", "q8b"])
def test_cached_decoder_matches_cacheless(variant):
    if variant == "tiny":
        cfg = get_config("tiny", gain_std=0.1)
        T = 24
    else:
        cfg = layer_variant(variant, n_layers=2, vocab=512, gain_std=0.1, max_ctx=64)
        T = 10
    w = generate_weights(cfg)
    m = Fp64Model(w)
    ids = prompt_ids(cfg.seed, 0, T, cfg.vocab)
    dec = TokenDecoder(m)
    cached = np.stack([dec.decode(int(t)) for t in ids])
    brute = forward_cacheless(m, list(ids))
    assert _rel(cached, brute) < 1e-12


# ------------------------------------------------ second formulation on torch library routines
@pytest.mark.parametrize("gain_std", [0.0, 0.1])
def test_torch_library_formulation_tiny(gain_std):
    cfg = get_config("tiny", gain_std=gain_std)
    w = generate_weights(cfg)
    ids = prompt_ids(cfg.seed, 3, 20, cfg.vocab)
    dec = TokenDecoder(Fp64Model(w))
    ours = np.stack([dec.decode(int(t)) for t in ids])
    ref = tf.forward(w, ids)
    assert np.max(np.abs(ours - ref)) < 1e-10


def test_torch_library_formulation_geglu_int4():
    cfg = layer_variant("gemma_int4", n_layers=2, vocab=512, gain_std=0.1, max_ctx=64)
    w = generate_weights(cfg)
    ids = prompt_ids(cfg.seed, 1, 8, cfg.vocab)
    dec = TokenDecoder(Fp64Model(w))
    ours = np.stack([dec.decode(int(t)) for t in ids])
    assert np.max(np.abs(ours - tf.forward(w, ids))) < 1e-10


# ------------------------------------------------ closed forms
def test_attention_one_position_returns_v():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 64))
    K = rng.standard_normal((1, 2, 64))
    V = rng.standard_normal((1, 2, 64))
    o = om.attend_one(q, K, V, group=2)
    np.testing.assert_array_equal(o, V[0, [0, 0, 1, 1], :])


def test_attention_zero_query_is_mean_of_v():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((7, 2, 64))
    V = rng.standard_normal((7, 2, 64))
    o = om.attend_one(np.zeros((4, 64)), K, V, group=2)
    np.testing.assert_allclose(o, V.mean(axis=0)[[0, 0, 1, 1]], rtol=0, atol=1e-14)


def test_uniform_attention_in_model_when_wq_wk_zero(tiny_weights):
    # With Wq = Wk = 0 every score is 0, so each head averages the cached v.
    w = copy.deepcopy(tiny_weights)
    for L in w.layers:
        L["wq"][:] = 0
        L["wk"][:] = 0
    m = Fp64Model(w)
    cfg = w.cfg
    dec = TokenDecoder(m)
    ids = prompt_ids(cfg.seed, 5, 6, cfg.vocab)
    for t in ids[:-1]:
        dec.decode(int(t))
    seen = {}
    orig = om.attend_one

    def spy(q, K, V, group):
        out = orig(q, K, V, group)
        seen.setdefault("first", (out, V))
        return out
    om.attend_one = spy
    try:
        dec.decode(int(ids[-1]))
    finally:
        om.attend_one = orig
    out, V = seen["first"]
    np.testing.assert_allclose(out, V.mean(axis=0)[[j // cfg.group for j in range(cfg.n_q_heads)]],
                               rtol=0, atol=1e-14)


def test_rope_position_zero_is_identity_and_preserves_norm():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((3, 128))
    np.testing.assert_array_equal(om.rope(u, om.rope_angles(0, 128, 1e4)), u)
    r = om.rope(u, om.rope_angles(12345, 128, 1e4))
    pair = lambda z: z[:, :64] ** 2 + z[:, 64:] ** 2
    np.testing.assert_allclose(pair(r), pair(u), rtol=1e-13, atol=1e-13)


def test_rope_basis_vectors_closed_form():
    # dh = 4, theta = 1e4: pair 0 = (u0, u2) turns by p, pair 1 = (u1, u3) by p / 100.
    for p in (1, 7, 250):
        ang = om.rope_angles(p, 4, 1e4)
        e0 = om.rope(np.array([[1.0, 0, 0, 0]]), ang)[0]
        e1 = om.rope(np.array([[0, 1.0, 0, 0]]), ang)[0]
        e2 = om.rope(np.array([[0, 0, 1.0, 0]]), ang)[0]
        np.testing.assert_allclose(e0, [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
        np.testing.assert_allclose(e1, [0, math.cos(p / 100), 0, math.sin(p / 100)], atol=1e-15)
        np.testing.assert_allclose(e2, [-math.sin(p), 0, math.cos(p), 0], atol=1e-15)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 128))
    k = rng.standard_normal((1, 128))
    def score(pq, pk):
        return float(om.rope(q, om.rope_angles(pq, 128, 1e4))[0] @ om.rope(k, om.rope_angles(pk, 128, 1e4))[0])
    for c in (1, 17, 1000):
        assert abs(score(40, 13) - score(40 + c, 13 + c)) < 1e-12 * max(1.0, abs(score(40, 13)))


@pytest.mark.parametrize("c", [3.0, -0.25, 1e-4])
def test_rmsnorm_of_constant_vector(c):
    eps = 1e-6
    out = om.rmsnorm(np.full(256, c), np.ones(256), eps)
    np.testing.assert_allclose(out, math.copysign(1.0, c) / math.sqrt(1.0 + eps / (c * c)), rtol=1e-15)


def test_zero_residual_model_scores_its_own_embedding(tiny_weights):
    # Wo = Wd = 0 leaves x = E[t], so logits = rmsnorm(E[t]) . E^T and the
    # greedy id repeats the last token (its self-dot dominates at d = 256).
    w = copy.deepcopy(tiny_weights)
    for L in w.layers:
        L["wo"][:] = 0
        L["wd"][:] = 0
    m = Fp64Model(w)
    cfg = w.cfg
    ids = prompt_ids(cfg.seed, 7, 12, cfg.vocab)
    dec = TokenDecoder(m)
    E = m.embed_rows(np.arange(cfg.vocab))
    for t in ids:
        lg = dec.decode(int(t))
        e = E[int(t)]
        expect = E @ (e / math.sqrt(np.mean(e * e) + cfg.rms_eps))
        np.testing.assert_allclose(lg, expect, rtol=0, atol=1e-12)
        assert greedy_id(lg) == int(t)


# ------------------------------------------------ argmax convention
def test_greedy_ties_go_to_lowest_id():
    v = np.zeros(100)
    v[[17, 42, 99]] = 5.0
    assert greedy_id(v) == 17
    v[17] = np.nextafter(5.0, 0)
    assert greedy_id(v) == 42
    v = np.array([0.0, -0.0, -1.0])
    assert greedy_id(v) == 0 and greedy_id(v[::-1].copy()) == 1
    assert top2_margin(np.array([1.0, 3.0, 3.0])) == 0.0


def test_planted_identical_lm_rows_pick_lowest_id(tiny_weights):
    w = copy.deepcopy(tiny_weights)
    m0 = Fp64Model(tiny_weights)
    cfg = w.cfg
    ids = prompt_ids(cfg.seed, 9, 6, cfg.vocab)
    d0 = TokenDecoder(m0)
    a = greedy_id([d0.decode(int(t)) for t in ids][-1])
    b = next(x for x in range(a) if x not in set(ids.tolist())) if a > 0 else None
    assert b is not None
    w.embed[b] = w.embed[a]
    dec = TokenDecoder(Fp64Model(w))
    lg = [dec.decode(int(t)) for t in ids][-1]
    assert lg[a] == lg[b]
    assert greedy_id(lg) == b


# ------------------------------------------------ spec-loop integer invariants
def _truth_fn(truth):
    # Drafts proposed from a known greedy continuation: position i of the
    # window after committing `out` proposes truth[len(out) + 1 + i].
    def f(pattern_src):
        def draft(out, cur, k):
            return pattern_src.window(truth[len(out) + 1: len(out) + 1 + k], k)
        return draft
    return f


@pytest.mark.parametrize("pattern", PATTERNS)
def test_spec_loop_commits_greedy_continuation(tiny_model, pattern):
    cfg = tiny_model.cfg
    ids = prompt_ids(cfg.seed, 0, 32, cfg.vocab)
    dec = TokenDecoder(tiny_model)
    nx = prefill(dec, ids)
    base = dec.length
    truth = greedy_generate(dec, nx, 64 + 8)
    dec.truncate(base)
    src = DraftSource(cfg.seed, 0, cfg.vocab, pattern=pattern)
    out, steps = spec_generate(dec, nx, 64, 4, _truth_fn(truth)(src))
    assert out == truth[:64]
    assert sum(n + 1 for _, n in steps) == 64
    assert dec.length == base + 64
    planted = {"all_accept": 4, "mismatch_at_2": 2, "mismatch_at_0": 0}[pattern]
    for k_eff, n in steps:
        assert n == min(planted, k_eff)


def test_spec_loop_random_corruption(tiny_model):
    cfg = tiny_model.cfg
    ids = prompt_ids(cfg.seed, 1, 32, cfg.vocab)
    dec = TokenDecoder(tiny_model)
    nx = prefill(dec, ids)
    truth = greedy_generate(dec, nx, 72)
    dec.truncate(32)
    src = DraftSource(cfg.seed, 1, cfg.vocab, p_correct=0.6)
    out, steps = spec_generate(dec, nx, 64, 4, _truth_fn(truth)(src))
    assert out == truth[:64]
    assert sum(n + 1 for _, n in steps) == 64


def test_verify_with_no_drafts_is_one_decode(tiny_model):
    cfg = tiny_model.cfg
    ids = prompt_ids(cfg.seed, 2, 16, cfg.vocab)
    d1, d2 = TokenDecoder(tiny_model), TokenDecoder(tiny_model)
    nx = prefill(d1, ids)
    prefill(d2, ids)
    r = block_verify(d1, nx, [], keep_logits=True)
    lg = d2.decode(nx)
    assert r.n_accepted == 0 and r.next_id == greedy_id(lg)
    np.testing.assert_array_equal(r.row_logits[0], lg)


def test_changed_future_drafts_leave_earlier_rows_unchanged(tiny_model):
    cfg = tiny_model.cfg
    ids = prompt_ids(cfg.seed, 4, 20, cfg.vocab)
    rng = np.random.default_rng(5)
    base_d = TokenDecoder(tiny_model)
    nx = prefill(base_d, ids)
    drafts = rng.integers(0, cfg.vocab, 8).tolist()
    ref = block_verify(copy.deepcopy(base_d), nx, drafts, keep_logits=True)
    for r in range(8):
        changed = drafts[:r] + rng.integers(0, cfg.vocab, 8 - r).tolist()
        got = block_verify(copy.deepcopy(base_d), nx, changed, keep_logits=True)
        for row in range(r + 1):
            np.testing.assert_array_equal(got.row_logits[row], ref.row_logits[row])
            assert got.row_argmax[row] == ref.row_argmax[row]


@pytest.mark.parametrize("reject_at", range(6))
def test_rollback_restores_one_token_state_exactly(tiny_model, reject_at):
    cfg = tiny_model.cfg
    ids = prompt_ids(cfg.seed, 6, 24, cfg.vocab)
    dec = TokenDecoder(tiny_model)
    nx = prefill(dec, ids)
    truth = greedy_generate(copy.deepcopy(dec), nx, 8)
    wrong = (truth[reject_at + 1] + 1) % cfg.vocab
    drafts = truth[1:7]
    drafts[reject_at] = wrong
    r = block_verify(dec, nx, drafts)
    assert r.n_accepted == reject_at
    assert r.next_id == truth[reject_at + 1]
    ref = TokenDecoder(tiny_model)
    prefill(ref, ids)
    for t in truth[:reject_at + 1]:
        ref.decode(t)
    got, want = dec.state(), ref.state()
    assert got[0] == want[0]
    for a, b in zip(got[1] + got[2], want[1] + want[2]):
        np.testing.assert_array_equal(a, b)
