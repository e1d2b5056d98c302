"""Planted mistakes in the oracle must each fail at least one pin.

Each mutation replaces one oracle primitive (on the CPU, via monkeypatch) by a
plausible wrong variant; the check re-runs the independent pins (torch library
formulation, closed forms, spec invariants, page tie examples) and asserts
that they now disagree.
"""
import copy
import json
import math
import os

import numpy as np
import pytest

from seeded_inputs import DraftSource, generate_weights, get_config, prompt_ids
from oracle import Fp64Model, TokenDecoder
from oracle import model as om
from oracle import spec as osp

import _torch_formulation as tf

CFG = get_config("tiny", gain_std=0.1)


def _pin_torch_formulation():
    w = generate_weights(CFG)
    ids = prompt_ids(CFG.seed, 3, 12, CFG.vocab)
    dec = TokenDecoder(Fp64Model(w))
    ours = np.stack([dec.decode(int(t)) for t in ids])
    return np.max(np.abs(ours - tf.forward(w, ids))) < 1e-10


def _wrong_rmsnorm_no_eps(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * g


def _wrong_rmsnorm_no_gain(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _wrong_rope_sign(u, ang):
    half = u.shape[-1] // 2
    c, s = np.cos(ang)[..., None, :], np.sin(ang)[..., None, :]
    u1, u2 = u[..., :half], u[..., half:]
    return np.concatenate([u1 * c + u2 * s, u2 * c - u1 * s], axis=-1)


def _wrong_rope_interleaved(u, ang):
    c, s = np.cos(ang)[..., None, :], np.sin(ang)[..., None, :]
    u1, u2 = u[..., 0::2], u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = u1 * c - u2 * s
    out[..., 1::2] = u2 * c + u1 * s
    return out


def _wrong_rope_angles(pos, head_dim, theta):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.multiply.outer(np.asarray(pos, dtype=np.float64), theta ** (-i / head_dim))


def _wrong_attend_gqa_modulo(q, K, V, group):
    nq, dh = q.shape
    nkv = K.shape[1]
    out = np.empty_like(q)
    for j in range(nq):
        s = K[:, j % nkv, :] @ q[j] / math.sqrt(dh)
        out[j] = om.softmax(s) @ V[:, j % nkv, :]
    return out


def _wrong_attend_no_scale(q, K, V, group):
    return om.attend_one.__wrapped__(q * math.sqrt(q.shape[1]), K, V, group)


def _wrong_mlp_swapped(h, wg, wu, wd, act):
    return (om.ACTS[act](h @ wu.T) * (h @ wg.T)) @ wd.T


def _wrong_softmax_no_shift_and_sum(s):
    e = np.exp(s)
    return e / np.sum(e) ** 0.5


MODEL_MUTATIONS = {
    "rmsnorm_no_eps": ("rmsnorm", _wrong_rmsnorm_no_eps),
    "rmsnorm_no_gain": ("rmsnorm", _wrong_rmsnorm_no_gain),
    "rope_sign": ("rope", _wrong_rope_sign),
    "rope_interleaved_pairs": ("rope", _wrong_rope_interleaved),
    "rope_frequency": ("rope_angles", _wrong_rope_angles),
    "gqa_modulo": ("attend_one", _wrong_attend_gqa_modulo),
    "attention_no_scale": ("attend_one", _wrong_attend_no_scale),
    "mlp_gate_up_swapped": ("mlp", _wrong_mlp_swapped),
    "softmax_bad_normaliser": ("softmax", _wrong_softmax_no_shift_and_sum),
}


@pytest.mark.parametrize("name", sorted(MODEL_MUTATIONS))
def test_model_mutation_is_caught(monkeypatch, name):
    attr, fn = MODEL_MUTATIONS[name]
    if name == "attention_no_scale":
        orig = om.attend_one
        fn = lambda q, K, V, group: orig(q * math.sqrt(q.shape[1]), K, V, group)  # noqa: E731
    assert _pin_torch_formulation()
    monkeypatch.setattr(om, attr, fn)
    assert not _pin_torch_formulation()


def test_tie_break_to_highest_id_is_caught(monkeypatch):
    monkeypatch.setattr(osp, "greedy_id", lambda lg: int(len(lg) - 1 - np.argmax(lg[::-1])))
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_ties.json")))["cases"]
    wrong = 0
    for c in cases:
        v = np.full(262144, -1e9)
        for tok, val in c["logits"].items():
            v[int(tok)] = val
        wrong += osp.greedy_id(v) != c["greedy"]
    assert wrong > 0


def _spec_pin(model):
    ids = prompt_ids(1, 0, 32, model.cfg.vocab)
    dec = TokenDecoder(model)
    nx = osp.prefill(dec, ids)
    truth = osp.greedy_generate(dec, nx, 40)
    dec.truncate(32)
    src = DraftSource(1, 0, model.cfg.vocab, pattern="mismatch_at_2")
    def draft(out, cur, k):
        return src.window(truth[len(out) + 1: len(out) + 1 + k], k)
    out, steps = osp.spec_generate(dec, nx, 32, 4, draft)
    return out == truth[:32] and all(n == min(2, k) for k, n in steps)


def test_acceptance_off_by_one_is_caught(monkeypatch, tiny_model):
    assert _spec_pin(tiny_model)
    orig = osp.block_verify

    def wrong(dec, next_id, drafts, keep_logits=False):
        base = dec.length
        r = orig(dec, next_id, drafts, keep_logits)
        if r.n_accepted < len(drafts):   # accepts the first mismatching draft too
            dec.truncate(base)
            for t in [next_id] + list(drafts[:r.n_accepted + 1]):
                dec.decode(t)
            r.n_accepted += 1
            r.next_id = r.row_argmax[r.n_accepted]
        return r
    monkeypatch.setattr(osp, "block_verify", wrong)
    assert not _spec_pin(tiny_model)


def _rollback_pin(model):
    ids = prompt_ids(1, 6, 24, model.cfg.vocab)
    dec = TokenDecoder(model)
    nx = osp.prefill(dec, ids)
    truth = osp.greedy_generate(copy.deepcopy(dec), nx, 8)
    drafts = truth[1:7]
    drafts[2] = (truth[3] + 1) % model.cfg.vocab
    r = osp.block_verify(dec, nx, drafts)
    ref = TokenDecoder(model)
    osp.prefill(ref, ids)
    for t in truth[:r.n_accepted + 1]:
        ref.decode(t)
    got, want = dec.state(), ref.state()
    return got[0] == want[0] and all(a.shape == b.shape and np.array_equal(a, b)
                                     for a, b in zip(got[1] + got[2], want[1] + want[2]))


def test_truncate_keeps_one_stale_position_is_caught(monkeypatch, tiny_model):
    assert _rollback_pin(tiny_model)
    orig = TokenDecoder.truncate

    def leaky(self, new_len):
        orig(self, min(self.length, new_len + 1))
    monkeypatch.setattr(TokenDecoder, "truncate", leaky)
    assert not _rollback_pin(tiny_model)
