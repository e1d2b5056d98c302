"""QKV item plans of the one-workgroup-per-CU GEMM, through the C ABI.

When the fused QKV matrix has r = n_items % grid > 0 leftover 16-column
items and 2 r <= grid, the last round's items are split into 8-column halves
(rows i and i ^ 4 of a QKV tile are a RoPE pair, so each half holds whole
pairs).  The 8B shape takes the case 2 r == grid; these small shapes take
the ragged case (only some workgroups get a half) and the full case, and
check oracle rows and verify == one-token decode bit for bit at K = 1, 4, 8.
"""
from dataclasses import replace

import numpy as np
import pytest

from test_gpu_configs import _check_rows_vs_oracle, _verify_vs_decode

pytestmark = pytest.mark.gpu

# (q heads, KV heads) at head_dim 64: QKV outputs (nq + 2 nkv) * 64
SHAPES = {
    "ragged": (48, 12),   # 288 items: on 256 CUs, 32 leftover items -> 64 halves
    "full": (64, 16),     # 384 items: 128 leftover items -> 256 halves
}


def _cfg(kind):
    from seeded_inputs.configs import PRESETS
    nq, nkv = SHAPES[kind]
    return replace(PRESETS["tiny"], name=f"qkv_split_{kind}", n_layers=2, d_model=512, n_q_heads=nq,
                   n_kv_heads=nkv, head_dim=64, d_ff=1024, vocab=512, max_ctx=256, max_k=8, seed=11)


@pytest.fixture(scope="module", params=sorted(SHAPES))
def model(request):
    import torch
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights
    cfg = _cfg(request.param)
    n_items = cfg.qkv_dim // 16
    grid = min(n_items, torch.cuda.get_device_properties(0).multi_processor_count)
    r = n_items % grid
    print(f"{cfg.name}: {n_items} QKV items on {grid} workgroups, {r} split into {2 * r} halves"
          if 0 < 2 * r <= grid else f"{cfg.name}: {n_items} QKV items on {grid} workgroups, no split")
    w = generate_weights(cfg)
    return DeviceModel(w), w


def test_split_qkv_rows_match_oracle(model):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = model
    ids = prompt_ids(w.cfg.seed, 3, 30, w.cfg.vocab).tolist()
    _check_rows_vs_oracle(Session(dev), w, ids[:22], ids[22:30], w.cfg.name)


@pytest.mark.parametrize("k", [1, 4, 8])
def test_split_qkv_verify_equals_decode(model, k):
    from greedy_block_verification_amd.session import Session
    from seeded_inputs import prompt_ids
    dev, w = model
    s = Session(dev)
    s.prefill(prompt_ids(w.cfg.seed, 0, 90, w.cfg.vocab).tolist())
    snap = s.snapshot()
    rng = np.random.default_rng(70 + k)
    _verify_vs_decode(dev, snap, rng.integers(0, w.cfg.vocab, k).tolist())
