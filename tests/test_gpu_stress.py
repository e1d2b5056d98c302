"""8B-shaped stress case at a 32768-position context, through the C ABI.

The committed prefix of 32704 positions is a synthetic, seeded KV cache
(random fp16 K and V in every layer and head) restored into the context with
sv_restore; the oracle cannot score 32K positions, so these checks are
GPU-vs-GPU properties that hold at any size:
* verify == one-token decode bit for bit for K in {1, 2, 4, 8, 16, 32};
* rollback after a reject at every index 0..K-1 (K = 32), then a re-verify,
  equals the state built by one-token commits (logits and KV bits);
* planted near-ties in the LM head (a row copied exactly, and rows one bf16
  ulp away at the largest and the smallest |h_j| of the final hidden vector,
  below and above the argmax id) resolve identically in verify and decode,
  every other logit keeps its bits, and the lowest id wins among equal
  maxima;
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


@pytest.mark.parametrize("kv_len,k", [(184, 16), (1020, 16), (4084, 16), (8180, 16), (4094, 4), (8190, 4)])
def test_stress_verify_equals_decode_across_split_plan_changes(stress, kv_len, k):
    """Rows of one verify that straddle a change of the attention launch or
    split plan: around ctx 192 (3 splits folded in the workgroup vs 4 folded
    by the combine pass, chosen by the verify's longest row), around ctx 1024
    (16 vs 17 splits), around ctx 4096 (one block per split vs two) and
    around ctx 8192 (two blocks per split vs three).  K = 16 runs the
    two-waves-per-SIMD block walk; K = 4 (two q tiles) the pipelined one,
    whose first-block guess (from the first row) misses for the rows past
    the change; one-token decodes run the pipelined walk."""
    dev, w, cfg, snap = stress
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


def test_stress_one_session_across_blocks_per_split(stress):
    """One context verifies K = 4 windows at 32K, 8186 and 4090 positions in
    turn: the same row and split counts (64 splits) at 8, 2 and 1 blocks per
    split.  The forward's captured graphs carry the split kernel's
    blocks-per-split guess, so each window runs with its own; every window's
    rows must equal one-token decodes of the same rows bit for bit."""
    dev, w, cfg, snap = stress
    b = _sess(dev, cfg, snap)
    for kv_len in (PREFIX, 8186, 4090):
        if kv_len < b.kv_len:
            b.truncate(kv_len)
        drafts = np.random.default_rng(3000 + kv_len).integers(0, cfg.vocab, 4).tolist()
        a = _sess(dev, cfg, snap)
        if kv_len < a.kv_len:
            a.truncate(kv_len)
        dec = []
        for t in [a.next_id] + drafts:
            a.decode_step(t)
            dec.append(a.logits(0))
        a.close()
        b.verify(drafts)
        for r in range(5):
            np.testing.assert_array_equal(_bits(b.logits(r)), _bits(dec[r]))
        b.truncate(kv_len)
    b.close()


@pytest.mark.parametrize("lens", [(PREFIX, 8186, 4090), (8186,), (1500, 600)])
def test_stress_long_context_batch_equals_one_at_a_time(stress, lens):
    """Batched verify at long contexts: each sequence's rows equal its own
    verify's bit for bit.  Three sequences (6 q tiles) run the two-waves-per-
    SIMD block walk, one sequence (2 q tiles) the pipelined one, both with
    the sequence table (page numbers and context lengths per tile) and the
    batch's first-block guess of one block per split, which misses at 8 and
    2 blocks per split; 1500 and 600 positions (24 and 10 one-block splits)
    run the split kernel that requests its block ahead of q, with the
    sequence table."""
    from greedy_block_verification_amd import binding as B
    dev, w, cfg, snap = stress
    drafts = [np.random.default_rng(4000 + n).integers(0, cfg.vocab, 4).tolist() for n in lens]
    ref = []
    for n, d in zip(lens, drafts):
        a = _sess(dev, cfg, snap)
        if n < a.kv_len:
            a.truncate(n)
        got = a.verify(d)
        ref.append((got, [_bits(a.logits(r)) for r in range(5)]))
        a.close()
    ss = [_sess(dev, cfg, snap) for _ in lens]
    for s, n in zip(ss, lens):
        if n < s.kv_len:
            s.truncate(n)
    got = B.sv_verify_batch([s.ctx for s in ss], [s.kv_len for s in ss], drafts)
    for s, g, (g_ref, lg_ref) in zip(ss, got, ref):
        assert tuple(g) == tuple(g_ref)
        for r in range(5):
            np.testing.assert_array_equal(_bits(s.logits(r)), lg_ref[r])
    for s in ss:
        s.close()


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


def _planted_model(dev, w, rows):
    """A device model sharing dev's layer weights whose tied embedding / LM
    head has the given rows replaced ({id: bf16 row bits})."""
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs.weights import ModelWeights
    emb = w.embed.copy()
    for i, r in rows.items():
        emb[i] = r
    return DeviceModel(ModelWeights(w.cfg, emb, w.g_final, w.layers), share_layers_with=dev)


def _rows_and_logits(model, cfg, snap, drafts):
    """(verify logits and argmax, one-token decode logits and argmax) of the window."""
    p1, p2 = _sess(model, cfg, snap), _sess(model, cfg, snap)
    dec = []
    for t in [p1.next_id] + drafts:
        p1.decode_step(t)
        dec.append((p1.last_argmax()[0], p1.logits(0)))
    p2.verify(drafts)
    ver = [(p2.last_argmax()[r], p2.logits(r)) for r in range(len(drafts) + 1)]
    p1.close()
    p2.close()
    return ver, dec


def test_stress_planted_near_ties(stress):
    """Near ties planted in the LM head as the measurement plan describes:
    with a the unplanted argmax of row 0, row c is an exact copy of row a,
    and rows b1..b4 are row a with one element moved by one bf16 ulp -- at
    the largest |h_j| of the row's final normalised hidden vector (a gap
    fp32 resolves) and at the smallest (a gap at fp32 rounding level), each
    once with b below a and once above it.  No planted id is among the
    window's ids (the head is tied, so planting also changes those ids'
    embeddings).  h is read through a probe head whose rows 'base + j' are
    the unit vectors e_j, so that logit = h_j.  Checked unconditionally:
    verify == decode bits and argmax on every row; every logit of an
    unplanted id equals the unplanted model's bit for bit; c ties a
    exactly; the winner of row 0 is the lowest id among its maxima and is
    one of a, c, b1..b4; at the largest |h_j| each gap has the sign of
    (row change) x h_j."""
    from seeded_inputs.weights import f32_from_bf16_bits
    dev, w, cfg, snap = stress
    rng = np.random.default_rng(77)
    drafts = rng.integers(1000, 90000, 4).tolist()
    base = _sess(dev, cfg, snap)
    rows = [base.next_id] + drafts
    base.verify(drafts)
    a = base.last_argmax()[0]
    lg0 = base.logits(0)
    base.close()
    d = cfg.d_model
    # probe: unit rows at ids [pb, pb + d), away from the window's ids and from a
    pb = next(x for x in (100000, 110000, 120000, 130000, 140000)
              if all(not x <= t < x + d for t in rows + [a]))
    unit = {pb + j: np.zeros(d, dtype=np.uint16) for j in range(d)}
    for j in range(d):
        unit[pb + j][j] = 0x3F80                       # bf16 1.0
    probe = _planted_model(dev, w, unit)
    pv, _ = _rows_and_logits(probe, cfg, snap, drafts)
    del probe
    h = pv[0][1][pb:pb + d].astype(np.float64)         # row 0's final hidden vector, h_j = logit of e_j
    ea = w.embed[a]
    ea_f = f32_from_bf16_bits(ea).astype(np.float64)
    # largest |h_j| where row a's element is at least 2^-7 in magnitude (one
    # bf16 ulp there is at least 2^-14, so the gap clears fp32 rounding of
    # the logit); smallest |h_j| anywhere
    big_ok = np.abs(ea_f) >= 2.0 ** -7
    j_big = int(np.argmax(np.where(big_ok, np.abs(h), -1.0)))
    j_small = int(np.argmin(np.abs(h)))
    # plant: ids around a (two below, three above; none among the window's ids)
    taken = set(rows)
    below = [x for x in range(a - 1, -1, -1) if x not in taken][:2]
    above = [x for x in range(a + 1, cfg.vocab) if x not in taken][:3]
    assert len(below) == 2 and len(above) == 3, "a sits too close to an end of the vocabulary"
    c = above[2]
    plan = {below[0]: j_big, above[0]: j_big, below[1]: j_small, above[1]: j_small}
    planted_rows = {c: ea.copy()}
    for b, j in plan.items():
        r = ea.copy()
        r[j] = np.uint16(int(ea[j]) + 1)               # one ulp further from zero
        planted_rows[b] = r
    assert not set(planted_rows) & set(rows)
    model = _planted_model(dev, w, planted_rows)
    ver, dec = _rows_and_logits(model, cfg, snap, drafts)
    for r in range(5):
        np.testing.assert_array_equal(_bits(ver[r][1]), _bits(dec[r][1]))
        assert ver[r][0] == dec[r][0]
        lg = ver[r][1]
        top = lg.max()
        assert ver[r][0] == int(np.flatnonzero(lg == top)[0])   # lowest id among the maxima
    lg = ver[0][1]
    others = np.ones(cfg.vocab, dtype=bool)
    others[list(planted_rows)] = False
    np.testing.assert_array_equal(_bits(lg[others]), _bits(lg0[others]))
    assert _bits(lg[c]) == _bits(lg[a])
    top = lg.max()
    cands = [a, c] + list(plan)
    assert lg[a] == lg0[a] and top == max(lg[x] for x in cands)
    assert ver[0][0] == min(x for x in cands if lg[x] == top)
    # the direction of each resolvable gap: row change (one ulp away from zero) times h_j
    for b in (below[0], above[0]):
        delta = float(f32_from_bf16_bits(planted_rows[b][j_big:j_big + 1])[0]) - float(ea_f[j_big])
        gap = float(lg[b]) - float(lg[a])
        assert gap != 0.0 and np.sign(gap) == np.sign(delta * h[j_big])
    print(f"planted: a={a} c={c} |h| max {abs(h[j_big]):.3g} at {j_big}, min {abs(h[j_small]):.3g} at {j_small}; "
          + ", ".join(f"b={b} (j={j}) gap {float(lg[b]) - float(lg[a]):.3g}" for b, j in plan.items())
          + f"; row-0 argmax {ver[0][0]}")
