"""8B-shaped stress case at a 32768-position context, through the C ABI.

The committed prefix of 32704 positions is a synthetic, seeded KV cache
(random fp16 K and V in every layer and head) restored into the context with
sv_restore; the oracle cannot score 32K positions, so these checks are
GPU-vs-GPU properties that hold at any size:
* verify == one-token decode bit for bit for K in {1, 2, 4, 8, 16, 32};
* rollback after a reject at every index 0..K-1 (K = 32), then a re-verify,
  equals the state built by one-token commits (logits and KV bits);
* planted near-ties in the LM head (a row copied exactly, and a row one
  bf16 ulp away) resolve identically in verify and decode, and an exact tie
  goes to the lower id;
* rows straddling a change of the attention split plan, and a 32640-id
  prompt prefilled through the row-tiled kernels, verify == decode bitwise.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

PREFIX = 32704


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


@pytest.fixture(scope="module")
def stress(q8b_device):
    import torch
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import get_config
    dev, w = q8b_device
    cfg = get_config("q8b_stress")
    s = Session(dev, cfg=cfg)
    n_pages = cfg.max_ctx // cfg.page_size
    pool = s.kv.view(cfg.n_layers, n_pages, -1)
    g = torch.Generator(device=s.kv.device)
    g.manual_seed(cfg.seed + 300)
    used = PREFIX // cfg.page_size
    for l in range(cfg.n_layers):
        vals = torch.randn((used, pool.shape[2]), generator=g, device=s.kv.device, dtype=torch.float32)
        pool[l, :used] = vals.to(torch.float16).view(torch.int16)
    torch.cuda.synchronize()
    hist = np.random.default_rng(cfg.seed + 301).integers(0, cfg.vocab, PREFIX).tolist()
    from greedy_block_verification_amd import binding as B
    B.sv_restore(s.ctx, PREFIX, hist)
    snap = s.snapshot()
    s.close()
    return dev, w, cfg, snap


def _sess(dev, cfg, snap, debug=True):
    from greedy_block_verification_amd.session import Session
    s = Session(dev, cfg=cfg)
    s.restore(snap)
    s.set_debug(debug)
    return s


@pytest.mark.parametrize("k", [1, 2, 4, 8, 16, 32])
def test_stress_verify_equals_decode(stress, k):
    dev, w, cfg, snap = stress
    rng = np.random.default_rng(1000 + k)
    drafts = rng.integers(0, cfg.vocab, k).tolist()
    a, b = _sess(dev, cfg, snap), _sess(dev, cfg, snap)
    rows = [a.next_id] + drafts
    dec, arg = [], []
    for t in rows:
        arg.append(a.decode_step(t))
        dec.append(a.logits(0))
    n, nxt = b.verify(drafts)
    assert b.last_argmax() == arg
    for r in range(k + 1):
        np.testing.assert_array_equal(_bits(b.logits(r)), _bits(dec[r]))
    assert b.kv_len == PREFIX + n + 1
    a.close()
    b.close()


@pytest.mark.parametrize("kv_len", [184, 1020, 8180])
def test_stress_verify_equals_decode_across_split_plan_changes(stress, kv_len):
    """Rows of one verify that straddle a change of the attention launch or
    split plan: around ctx 192 (3 splits folded in the workgroup vs 4 folded
    by the combine pass, chosen by the verify's longest row), around ctx 1024
    (16 vs 17 splits) and around ctx 8192 (one block per split vs two)."""
    dev, w, cfg, snap = stress
    k = 16
    rng = np.random.default_rng(2000 + kv_len)
    drafts = rng.integers(0, cfg.vocab, k).tolist()
    a, b = _sess(dev, cfg, snap), _sess(dev, cfg, snap)
    a.truncate(kv_len)
    b.truncate(kv_len)
    rows = [a.next_id] + drafts
    dec = []
    for t in rows:
        a.decode_step(t)
        dec.append(a.logits(0))
    b.verify(drafts)
    for r in range(k + 1):
        np.testing.assert_array_equal(_bits(b.logits(r)), _bits(dec[r]))
    np.testing.assert_array_equal(a.kv_positions(kv_len + 1, kv_len - 4), b.kv_positions(kv_len + 1, kv_len - 4))
    a.close()
    b.close()


def test_stress_prefilled_32k_context_verify_equals_decode(q8b_device):
    """A 32640-id prompt prefilled through the row-tiled kernels (2048-row
    forwards), then a K = 8 verify at that context: bit-identical to one-token
    decodes of the same rows."""
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import get_config, prompt_ids
    dev, w = q8b_device
    cfg = get_config("q8b_stress")
    ids = prompt_ids(cfg.seed, 900, 32640, cfg.vocab).tolist()
    a = Session(dev, cfg=cfg, prefill_rows=2048)
    nx = a.prefill(ids)
    assert a.kv_len == 32640 and a.next_id == nx
    snap = a.snapshot()
    a.close()
    drafts = np.random.default_rng(9).integers(0, cfg.vocab, 8).tolist()
    b, c = _sess(dev, cfg, snap), _sess(dev, cfg, snap)
    dec = []
    for t in [b.next_id] + drafts:
        b.decode_step(t)
        dec.append((b.last_argmax()[0], b.logits(0)))
    c.verify(drafts)
    for r in range(9):
        assert c.last_argmax()[r] == dec[r][0]
        np.testing.assert_array_equal(_bits(c.logits(r)), _bits(dec[r][1]))
    b.close()
    c.close()


def test_stress_rollback_at_every_index(stress):
    dev, w, cfg, snap = stress
    K = 32
    ref = _sess(dev, cfg, snap, debug=False)
    truth = [ref.next_id]
    for _ in range(K + 6):
        truth.append(ref.decode_step(truth[-1]))
    ref.close()
    # truth[i + 1] is the greedy id after the prefix + truth[0..i]
    for j in range(K):
        s = _sess(dev, cfg, snap)
        drafts = truth[1:K + 1]
        drafts[j] = (truth[j + 1] + 1) % cfg.vocab
        n, nxt = s.verify(drafts)
        assert (n, nxt) == (j, truth[j + 1])
        dr2 = truth[j + 2: j + 6]
        n2, _ = s.verify(dr2)
        assert n2 == 4
        got = [_bits(s.logits(r)) for r in range(5)]
        chk = _sess(dev, cfg, snap)
        for t in truth[:j + 1]:
            chk.decode_step(t)
        for r, t in enumerate([truth[j + 1]] + dr2):
            chk.decode_step(t)
            np.testing.assert_array_equal(_bits(chk.logits(0)), got[r])
        lo = PREFIX - 16
        np.testing.assert_array_equal(chk.kv_positions(chk.kv_len, lo), s.kv_positions(s.kv_len, lo))
        s.close()
        chk.close()


def test_stress_planted_near_ties(stress):
    from greedy_block_verification_amd.session import DeviceModel, Session
    from seeded_inputs.weights import ModelWeights
    dev, w, cfg, snap = stress
    rng = np.random.default_rng(77)
    drafts = rng.integers(1000, cfg.vocab, 4).tolist()
    base = _sess(dev, cfg, snap)
    base.verify(drafts)
    a = base.last_argmax()[0]
    base.close()
    # plant: c = an exact copy of LM-head row a with c < a (exact tie -> lower id),
    #        b = row a with one element moved by one bf16 ulp (a 1-ulp near-tie)
    c = a - 1 if a > 0 else a + 1
    b = a - 2 if a > 1 else a + 2
    emb = w.embed.copy()
    emb[c] = emb[a]
    emb[b] = emb[a]
    emb[b, 0] = np.uint16(int(emb[a, 0]) + 1)
    planted = DeviceModel(ModelWeights(w.cfg, emb, w.g_final, w.layers), share_layers_with=dev)
    p1, p2 = _sess(planted, cfg, snap), _sess(planted, cfg, snap)
    rows = [p1.next_id] + drafts
    dec = []
    for t in rows:
        p1.decode_step(t)
        dec.append((p1.last_argmax()[0], p1.logits(0)))
    p2.verify(drafts)
    for r in range(5):
        np.testing.assert_array_equal(_bits(p2.logits(r)), _bits(dec[r][1]))
        assert p2.last_argmax()[r] == dec[r][0]
    lg = p2.logits(0)
    assert lg[c] == lg[a]                       # exact copy -> exactly equal logits
    win = p2.last_argmax()[0]
    top = lg.max()
    assert lg[win] == top and win == int(np.flatnonzero(lg == top)[0])   # lowest id among the maxima
    if lg[a] == top:
        assert win == min(a, c, b if lg[b] == top else a)
    print(f"planted: a={a} c={c} b={b}; logits a {lg[a]!r} c {lg[c]!r} b {lg[b]!r}; argmax {win}")
    p1.close()
    p2.close()
