"""Row-tiled prefill (forwards of more than 64 rows), through the C ABI.

The tiled GEMMs and the many-row attention run the same per-row arithmetic
as the weight-streaming kernels of decode and verify, so a prefill through
them must give every row the bits a one-token decode gives it:
* tiny config: each row of one 200-row tiled forward vs the one-token decode
  of that row (logits bits, argmax) and every position's KV bits; the rows
  of a 130-row tiled forward vs the fp64 oracle within 3e-2;
* tiny config: chunkings 128 + 128 + 44 (tiled, tiled, weight-streaming) and
  64-row forwards only give the same history, KV bits and next logits;
* 8B shape: a 700-id prefill in tiled chunks (512 + 188) vs 64-row chunks:
  equal history, equal KV bits at sampled positions of every layer, equal
  logits of the last 60 rows, and an identical decode step afterwards;
* Gemma-style int4 layers (int4 tiled GEMM, GeGLU, 6 q heads per KV head):
  every row of a 150-row tiled forward vs the one-token decode of that row.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TOL = 3e-2


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


@pytest.fixture(scope="module")
def tiny():
    import torch
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights, get_config
    assert torch.cuda.is_available()
    cfg = get_config("tiny", max_ctx=1024)
    w = generate_weights(get_config("tiny"))
    return DeviceModel(w), w, cfg


def _ids(n, idx, vocab, seed=11):
    from seeded_inputs import prompt_ids
    return prompt_ids(seed, idx, n, vocab).tolist()


def test_tiled_prefill_rows_equal_decode_rows(tiny):
    from greedy_block_verification_amd.session import Session
    dm, w, cfg = tiny
    ids = _ids(200, 0, cfg.vocab)
    a = Session(dm, cfg=cfg, prefill_rows=256)
    a.set_debug(True)
    nxt = a.prefill(ids)
    arg = a.last_argmax()
    assert len(arg) == 200 and arg[-1] == nxt
    got = [_bits(a.logits(r)) for r in range(200)]
    b = Session(dm, cfg=cfg)
    b.set_debug(True)
    for r, t in enumerate(ids):
        assert b.decode_step(t) == arg[r]
        np.testing.assert_array_equal(got[r], _bits(b.logits(0)))
    np.testing.assert_array_equal(a.kv_positions(200), b.kv_positions(200))
    assert a.history() == b.history()
    a.close()
    b.close()


def test_tiled_prefill_matches_oracle(tiny):
    from greedy_block_verification_amd.session import Session
    from oracle import Fp64Model, forward_cacheless
    from oracle.spec import top2_margin
    dm, w, cfg = tiny
    ids = _ids(130, 1, cfg.vocab)
    a = Session(dm, cfg=cfg, prefill_rows=256)
    a.set_debug(True)
    a.prefill(ids)                       # one tiled forward of 130 rows (a ragged second row block)
    ref = forward_cacheless(Fp64Model(w), ids)
    flagged = 0
    for r in range(130):
        lg = a.logits(r).astype(np.float64)
        assert np.max(np.abs(lg - ref[r])) <= TOL, r
        if int(np.argmax(lg)) != int(np.argmax(ref[r])):
            assert top2_margin(ref[r]) < TOL
            flagged += 1
    assert flagged <= 2
    a.close()


@pytest.mark.parametrize("rows", [128, 256])
def test_tiled_chunkings_equal_small_forwards(tiny, rows):
    from greedy_block_verification_amd.session import Session
    dm, w, cfg = tiny
    ids = _ids(300, 2, cfg.vocab)
    a = Session(dm, cfg=cfg, prefill_rows=rows)
    b = Session(dm, cfg=cfg)
    assert a.prefill(ids) == b.prefill(ids)
    assert a.history() == b.history()
    np.testing.assert_array_equal(a.kv_positions(300), b.kv_positions(300))
    a.set_debug(True)
    b.set_debug(True)
    assert a.decode_step(ids[0]) == b.decode_step(ids[0])
    np.testing.assert_array_equal(_bits(a.logits(0)), _bits(b.logits(0)))
    # a block commit of 70 ids after a prefix goes through the tiled path too
    more = _ids(70, 3, cfg.vocab)
    assert a.prefill(more) == b.prefill(more)
    np.testing.assert_array_equal(a.kv_positions(371, 290), b.kv_positions(371, 290))
    a.close()
    b.close()


def test_q8b_tiled_prefill_equals_small_forwards(q8b_device):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import get_config
    dev, w = q8b_device
    cfg = get_config("q8b")
    ids = _ids(700, 4, cfg.vocab)
    a = Session(dev, cfg=cfg, prefill_rows=512)
    b = Session(dev, cfg=cfg)
    a.set_debug(True)
    b.set_debug(True)
    assert a.prefill(ids) == b.prefill(ids)
    assert a.history() == b.history()
    # last forwards: a = rows 512..699 (tiled), b = rows 640..699 (64-row)
    for r in range(60):
        np.testing.assert_array_equal(_bits(a.logits(128 + r)), _bits(b.logits(r)))
    rng = np.random.default_rng(5)
    for p in sorted(rng.choice(700, 24, replace=False).tolist()) + [0, 511, 512, 699]:
        np.testing.assert_array_equal(a.kv_positions(p + 1, p), b.kv_positions(p + 1, p))
    t = int(rng.integers(0, cfg.vocab))
    assert a.decode_step(t) == b.decode_step(t)
    np.testing.assert_array_equal(_bits(a.logits(0)), _bits(b.logits(0)))
    a.close()
    b.close()


def test_int4_tiled_prefill_rows_equal_decode_rows():
    import torch
    from greedy_block_verification_amd.session import DeviceModel, Session
    from seeded_inputs import generate_weights
    from seeded_inputs.configs import layer_variant
    assert torch.cuda.is_available()
    cfg = layer_variant("gemma_int4", n_layers=3, vocab=1024)
    dm = DeviceModel(generate_weights(cfg))
    ids = _ids(150, 5, cfg.vocab)
    a = Session(dm, cfg=cfg, prefill_rows=256)
    a.set_debug(True)
    nxt = a.prefill(ids)
    arg = a.last_argmax()
    assert len(arg) == 150 and arg[-1] == nxt
    got = [_bits(a.logits(r)) for r in range(150)]
    b = Session(dm, cfg=cfg)
    b.set_debug(True)
    for r, t in enumerate(ids):
        assert b.decode_step(t) == arg[r]
        np.testing.assert_array_equal(got[r], _bits(b.logits(0)))
    np.testing.assert_array_equal(a.kv_positions(150), b.kv_positions(150))
    a.close()
    b.close()
