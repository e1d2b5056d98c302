"""The seeded input generator: bf16 rounding, int4 format, determinism."""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

from seeded_inputs import (DraftSource, generate_weights, get_config, prompt_ids,
                           quantize_int4_g64)
from seeded_inputs.weights import bf16_bits_from_f32, f32_from_bf16_bits

G = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 0.02,
        rng.standard_normal(1000).astype(np.float32) * 1e30,
        # exact halfway cases: ties to even in both directions
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00008000, 0x7F7F8000], dtype=np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, -2.5], dtype=np.float32),
    ])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(f32_from_bf16_bits(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_int4_quantizer_properties():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[3, 64:128] = 0.0                       # an all-zero group
    q, sb = quantize_int4_g64(w)
    s = f32_from_bf16_bits(sb).astype(np.float64)
    assert q.dtype == np.int8 and q.min() >= -8 and q.max() <= 7
    assert s[3, 1] == 0 and np.all(q[3, 64:128] == 0)
    # scale = bf16(max|w| / 7)
    amax = np.abs(w.reshape(64, 8, 64)).max(-1)
    np.testing.assert_array_equal(sb, bf16_bits_from_f32(amax / np.float32(7)))
    deq = q.astype(np.float64).reshape(64, 8, 64) * s[..., None]
    err = np.abs(deq - w.reshape(64, 8, 64))
    unclamped = (np.abs(w.reshape(64, 8, 64) / np.where(s == 0, 1, s)[..., None]) <= 7.5)
    assert np.all(err[unclamped] <= s[..., None].repeat(64, -1)[unclamped] / 2 * (1 + 1e-6))
    # re-quantising q*s gives back q and s when the group reaches code +-7
    q2, sb2 = quantize_int4_g64(deq.reshape(64, 512).astype(np.float32))
    full = np.abs(q.reshape(64, 8, 64)).max(-1) == 7
    np.testing.assert_array_equal(sb2[full], sb[full])
    np.testing.assert_array_equal(q2.reshape(64, 8, 64)[full], q.reshape(64, 8, 64)[full])


def _digest(w):
    h = hashlib.sha256()
    h.update(w.embed.tobytes())
    h.update(w.g_final.tobytes())
    for L in w.layers:
        for k in sorted(L):
            h.update(k.encode())
            h.update(np.ascontiguousarray(L[k]).tobytes())
    return h.hexdigest()


def test_generator_is_deterministic_and_matches_recorded_digest():
    cfg = get_config("tiny")
    a, b = generate_weights(cfg, threads=1), generate_weights(cfg, threads=4)
    assert _digest(a) == _digest(b)
    rec = json.load(open(os.path.join(G, "input_digests.json")))
    assert _digest(a) == rec["tiny_weights_sha256"]
    assert prompt_ids(1, 0, 32, 2048).tolist() == rec["tiny_prompt0"]


def test_weight_statistics():
    w = generate_weights(get_config("tiny"))
    x = f32_from_bf16_bits(w.layers[0]["wg"]).astype(np.float64)
    assert abs(x.mean()) < 1e-3 and abs(x.std() - 0.02) < 5e-4
    assert np.all(w.layers[0]["g_attn"] == 0x3F80)


def test_draft_source_patterns_and_rate():
    truth = list(range(100, 108))
    for pat, bad in (("all_accept", None), ("mismatch_at_2", 2), ("mismatch_at_0", 0)):
        d = DraftSource(1, 0, 2048, pattern=pat).window(truth, 8)
        for i in range(8):
            assert (d[i] != truth[i]) == (i == bad)
    src = DraftSource(4, 0, 151936, p_correct=0.66)
    hits = sum(x == t for _ in range(2000) for x, t in zip(src.window(truth, 8), truth))
    assert abs(hits / 16000 - 0.66) < 0.02
