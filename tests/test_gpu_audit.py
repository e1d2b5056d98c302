"""Audit mode (top-k dumps, selected-logit reads, state clone, sampled decode
audit), through the C ABI.

* sv_topk equals the host sort of the stored row by (logit descending, id
  ascending), bits and ids, and its first id is the row's argmax; planted
  exact ties come out lowest id first.
* sv_selected_logits equals the stored row at the chosen ids, and reading
  logits never changes the argmax.
* sv_clone_state copies the committed KV bits, history and next_id; the
  clone then decodes exactly as the source does.
* DecodeAudit over a speculative stream finds no disagreement on the real
  path, and reports every row (with both sides' top-k) when the shadow runs
  a different model.
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
    return DeviceModel(generate_weights(cfg)), cfg


def _ids(n, idx, vocab):
    from seeded_inputs import prompt_ids
    return prompt_ids(41, idx, n, vocab).tolist()


def test_topk_and_selected_logits_match_the_stored_row(tiny):
    from greedy_block_verification_amd import binding as B
    from greedy_block_verification_amd.session import Session
    dm, cfg = tiny
    s = Session(dm)
    s.set_debug(True)
    s.prefill(_ids(40, 0, cfg.vocab))
    arg = s.last_argmax()
    for r in (0, 17, 39):
        row = s.logits(r)
        order = sorted(range(cfg.vocab), key=lambda i: (-float(row[i]), i))   # -0.0 ties +0.0
        for k in (1, 8, 64):
            got = B.sv_topk(s.ctx, r, k)
            assert [i for i, _ in got] == order[:k]
            np.testing.assert_array_equal(_bits([v for _, v in got]), _bits(row[order[:k]]))
        assert B.sv_topk(s.ctx, r, 1)[0][0] == arg[r]
        sel = np.random.default_rng(r).integers(0, cfg.vocab, 300).tolist()
        np.testing.assert_array_equal(_bits(B.sv_selected_logits(s.ctx, r, sel)), _bits(row[sel]))
    assert s.last_argmax() == arg
    with pytest.raises(B.SvError):
        B.sv_topk(s.ctx, 40, 4)
    with pytest.raises(B.SvError):
        B.sv_selected_logits(s.ctx, 0, [cfg.vocab])
    s.close()


def test_topk_orders_exact_ties_lowest_id_first(tiny):
    """Planted exact copies of an LM-head row tie bit for bit with it."""
    from greedy_block_verification_amd import binding as B
    from greedy_block_verification_amd.session import DeviceModel, Session
    from seeded_inputs.weights import ModelWeights
    from seeded_inputs import generate_weights
    dm, cfg = tiny
    w = generate_weights(cfg)
    s = Session(dm)
    s.set_debug(True)
    ids = _ids(12, 1, cfg.vocab)
    s.prefill(ids)
    a = s.last_argmax()[-1]
    s.close()
    copies = sorted({(a + 5) % cfg.vocab, (a + 700) % cfg.vocab} - set(ids))
    emb = w.embed.copy()
    for c in copies:
        emb[c] = emb[a]
    planted = DeviceModel(ModelWeights(w.cfg, emb, w.g_final, w.layers), share_layers_with=dm)
    p = Session(planted)
    p.set_debug(True)
    p.prefill(ids)
    top = B.sv_topk(p.ctx, len(ids) - 1, 1 + len(copies))
    group = sorted([a] + copies)
    assert [i for i, _ in top] == group
    assert len({float(v) for _, v in top}) == 1
    p.close()


def test_clone_state_copies_the_committed_cache(tiny):
    from greedy_block_verification_amd import binding as B
    from greedy_block_verification_amd.session import Session
    dm, cfg = tiny
    perm = np.random.default_rng(3).permutation(cfg.max_ctx // 16)
    src, dst = Session(dm), Session(dm, page_perm=perm, poison=True)
    src.prefill(_ids(70, 2, cfg.vocab))
    B.sv_clone_state(dst.ctx, src.ctx)
    assert (dst.kv_len, dst.next_id, dst.history()) == (src.kv_len, src.next_id, src.history())
    np.testing.assert_array_equal(dst.kv_positions(70), src.kv_positions(70))
    src.set_debug(True)
    dst.set_debug(True)
    assert src.decode_step(5) == dst.decode_step(5)
    np.testing.assert_array_equal(_bits(src.logits(0)), _bits(dst.logits(0)))
    with pytest.raises(B.SvError):
        B.sv_clone_state(src.ctx, src.ctx)
    src.close()
    dst.close()


def test_sampled_decode_audit(tiny):
    from greedy_block_verification_amd.audit import DecodeAudit
    from greedy_block_verification_amd.session import DeviceModel, Session
    from seeded_inputs import DraftSource, generate_weights, get_config
    dm, cfg = tiny
    ids = _ids(30, 3, cfg.vocab)
    ref = Session(dm)
    truth = [ref.prefill(ids)]
    for _ in range(60):
        truth.append(ref.decode_step(truth[-1]))
    ref.close()

    def run(shadow_model, every):
        s, sh = Session(dm), Session(shadow_model)
        s.prefill(ids)
        audit = DecodeAudit(s, sh, every=every, topk=5)
        src = DraftSource(41, 0, cfg.vocab, p_correct=0.7)
        c = 0
        while c < 48:
            k = min(4, 60 - c - 1)
            n, _ = audit.verify(src.window(truth[c + 1: c + 1 + k], k))
            c += n + 1
        s.close()
        sh.close()
        return audit

    clean = run(dm, 2)
    assert clean.audited >= 5 and clean.rows_checked > clean.audited and clean.mismatches == []
    other = DeviceModel(generate_weights(get_config("tiny", seed=9)))
    bad = run(other, 3)
    assert bad.audited >= 3 and len(bad.mismatches) == bad.rows_checked
    m = bad.mismatches[0]
    assert len(m["topk_verify"]) == 5 and len(m["topk_decode"]) == 5
    assert m["topk_verify"][0][0] == m["argmax_verify"] and m["topk_decode"][0][0] == m["argmax_decode"]
    assert m["differing_logits"] > 0
