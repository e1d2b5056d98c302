"""GPU vs the fp64 oracle at the contexts the long-context attention paths run at.

The pages reject a fix unless every exact-parity workload passes, long
contexts and near ties included ("Shape and cache history in Gemma block
verification", section "Next discriminating tests").  The short-context
oracle checks elsewhere stop at contexts the single-workgroup fold serves;
here every row is scored against ``forward_cacheless`` (the brute-force
causal recompute) at contexts where the other attention paths run:

* 600-id prompt, K = 8 verify (contexts 577..609): more than three KV splits
  per row, so the split kernel writes global partials and the combine pass
  folds them; the last prefill forward's rows take the same path.
* 4090-id prompt, K = 8 verify (contexts 4091..4099): the split plan changes
  inside the window, from 64 splits of one 64-position block (context up to
  4096) to 33 splits of two blocks (4097 on), where the split kernel walks
  several blocks per unit.
* 8186-id prompt, K = 8 verify (contexts 8187..8195): the split plan changes
  inside the window, from 64 splits of two blocks (context up to 8192) to 43
  splits of three (8193 on); page addressing runs past page 512.
* Both prompts also go through the row-tiled prefill (forwards of more than
  64 rows, whose attention walks each row's splits in one wave); its rows
  and the verify after it must equal the 64-row path bit for bit.
* The Gemma-style int4 GeGLU layer shape (6 q heads per KV head) at the
  600-id context.
* The tiny shape (head_dim 64) at the 4090- and 8186-id prompts: the 64-wide
  instances of the same attention paths; the Gemma shape at the 4090-id
  prompt as well.

Models are 2-layer variants of the full layer shapes with a 512-id
vocabulary and norm gains bf16(1 + 0.1 N(0,1)), so the oracle finishes in
seconds to tens of seconds.  Tolerances: |dlogit| <= 3e-2 (bf16 weights),
<= 6e-2 (int4); an argmax may differ from the oracle's only where the
oracle's top-2 gap is under that tolerance (a flagged near tie).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TOL = {"bf16": 3e-2, "int4": 6e-2}


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _model(name, max_ctx):
    import torch
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights
    from seeded_inputs.configs import layer_variant
    assert torch.cuda.is_available()
    cfg = layer_variant(name, 2, 512, max_ctx=max_ctx, gain_std=0.1)
    w = generate_weights(cfg)
    return DeviceModel(w), w


@pytest.fixture(scope="module")
def q06b_l2():
    return _model("q06b", 8448)


@pytest.fixture(scope="module")
def gemma_l2():
    return _model("gemma_int4", 4352)


@pytest.fixture(scope="module")
def tiny_long():
    return _model("tiny", 8448)


def _oracle_rows(weights, seq, lo, hi):
    from oracle import Fp64Model, forward_cacheless
    return forward_cacheless(Fp64Model(weights), seq, positions=np.arange(lo, hi))


def _compare(label, got, ref, tol):
    """Every row within tol of the oracle; argmax flips only at flagged near ties."""
    from oracle.spec import greedy_id, top2_margin
    worst, flags, flips = 0.0, 0, 0
    for r, (g, o) in enumerate(zip(got, ref)):
        g = np.asarray(g, dtype=np.float64)
        worst = max(worst, float(np.max(np.abs(g - o))))
        near = top2_margin(o) < tol
        flags += int(near)
        if int(np.argmax(g)) != greedy_id(o):
            assert near, f"{label}: argmax differs from the oracle at row {r} away from a near tie"
            flips += 1
    print(f"{label}: {len(got)} rows, max|dlogit| {worst:.3e}, near ties {flags}, flipped {flips}", flush=True)
    assert worst <= tol, f"{label}: max|dlogit| {worst} above {tol}"
    return worst


def _run(dev, w, n_prompt, prompt_idx, rows_per_forward):
    """Prefill n_prompt ids (64-row forwards, or row-tiled forwards of up to
    rows_per_forward rows), keep the last prefill forward's logits, then
    verify 8 drafts.  Returns (next id, first position of the last prefill
    forward, its logits rows, drafts, verify logits rows, argmax rows)."""
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    cfg = w.cfg
    ids = prompt_ids(cfg.seed, prompt_idx, n_prompt, cfg.vocab).tolist()
    s = Session(dev, prefill_rows=rows_per_forward)
    s.set_debug(True)
    nx = s.prefill(ids)
    rows = s.last_argmax()
    last_n = len(rows)
    first = n_prompt - last_n
    pref = [s.logits(r) for r in range(last_n)]
    drafts = np.random.default_rng(prompt_idx).integers(0, cfg.vocab, 8).tolist()
    s.verify(drafts)
    ver = [s.logits(r) for r in range(9)]
    arg = s.last_argmax()
    s.close()
    return ids, nx, first, pref, drafts, ver, arg


def _long_context_case(dev, w, n_prompt, prompt_idx, tiled_rows, label):
    tol = TOL[w.cfg.weight_fmt]
    ids, nx, first, pref, drafts, ver, arg = _run(dev, w, n_prompt, prompt_idx, 0)
    print(f"{label}: 64-row prefill, last forward rows {first}..{n_prompt - 1}; verify contexts "
          f"{n_prompt + 1}..{n_prompt + 9}", flush=True)
    # the row-tiled prefill: the same rows' bits, and the same verify after it
    ids2, nx2, first2, pref2, drafts2, ver2, arg2 = _run(dev, w, n_prompt, prompt_idx, tiled_rows)
    assert ids2 == ids and nx2 == nx and drafts2 == drafts
    assert first2 <= first
    for r in range(len(pref)):
        np.testing.assert_array_equal(_bits(pref2[first - first2 + r]), _bits(pref[r]))
    for r in range(9):
        np.testing.assert_array_equal(_bits(ver2[r]), _bits(ver[r]))
    assert arg2 == arg
    # one oracle recompute scores the verify rows, the 64-row path's last
    # prefill forward and up to 64 earlier rows of the row-tiled forward
    lo = max(first2, first - 64)
    seq = ids + [nx] + drafts
    ref = _oracle_rows(w, seq, lo, n_prompt + 9)
    off = first - lo
    _compare(f"{label} verify rows", ver, ref[off + len(pref):], tol)
    _compare(f"{label} prefill rows {first}..{n_prompt - 1}", pref, ref[off:off + len(pref)], tol)
    if lo < first:
        _compare(f"{label} row-tiled prefill rows {lo}..{first - 1}", pref2[lo - first2:first - first2],
                 ref[:off], tol)


def test_combine_path_context_600_matches_oracle(q06b_l2):
    dev, w = q06b_l2
    _long_context_case(dev, w, 600, 500, 512, "q06b L2 ctx 600")


def test_split_plan_change_at_4096_matches_oracle(q06b_l2):
    dev, w = q06b_l2
    _long_context_case(dev, w, 4090, 503, 2048, "q06b L2 ctx 4090")


def test_split_plan_change_at_8192_matches_oracle(q06b_l2):
    dev, w = q06b_l2
    _long_context_case(dev, w, 8186, 501, 4096, "q06b L2 ctx 8186")


def test_int4_geglu_context_600_matches_oracle(gemma_l2):
    dev, w = gemma_l2
    _long_context_case(dev, w, 600, 502, 512, "gemma int4 L2 ctx 600")


@pytest.mark.parametrize("n_prompt,tiled", [(4090, 2048), (8186, 4096)])
def test_head_dim_64_split_plan_changes_match_oracle(tiny_long, n_prompt, tiled):
    """The 64-wide head instances of the long-context attention paths (the
    tiny shape: 4 q heads, 2 KV heads, head_dim 64) across the plan changes
    at 4096 and 8192 positions, against the oracle."""
    dev, w = tiny_long
    _long_context_case(dev, w, n_prompt, 504, tiled, f"tiny L2 ctx {n_prompt}")


def test_int4_geglu_split_plan_change_at_4096_matches_oracle(gemma_l2):
    """6 q heads per KV head (54 q-rows of a K = 8 window over 4 q tiles)
    across the plan change at 4096 positions, int4 weights."""
    dev, w = gemma_l2
    _long_context_case(dev, w, 4090, 505, 2048, "gemma int4 L2 ctx 4090")
