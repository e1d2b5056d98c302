"""Values printed on the pages, stored under tests/golden with their citations."""
import json
import os

import numpy as np

from oracle.spec import greedy_id
from seeded_inputs.weights import bf16_bits_from_f32, f32_from_bf16_bits
from greedy_block_verification_amd import metrics

G = os.path.join(os.path.dirname(__file__), "golden")


def test_page_tie_examples_follow_lowest_id_rule():
    cases = json.load(open(os.path.join(G, "page_ties.json")))["cases"]
    assert len(cases) == 8
    for c in cases:
        v = np.full(262144, -1e9)
        for tok, val in c["logits"].items():
            v[int(tok)] = val
            # the printed logits are bf16-granular
            f = np.float32(val)
            assert f32_from_bf16_bits(bf16_bits_from_f32(np.array([f])))[0] == f
        assert greedy_id(v) == c["greedy"], c["cite"]


def test_xserv_counter_arithmetic():
    g = json.load(open(os.path.join(G, "xserv_counters.json")))
    assert round(metrics.acceptance_rate(g["accepted"], g["proposed"]), 4) == g["acceptance_rate"]
    steps = metrics.target_steps(g["verify_steps"], g["commit_decode_steps"], g["correction_steps"],
                                 g["mirror_decode_steps"])
    assert steps == g["target_steps"]
    assert round(metrics.tokens_per_target_step(g["tokens"], steps), 4) == g["tokens_per_target_step"]
    for pre in ("baseline_e2e", "spec_e2e", "baseline_decode", "spec_decode"):
        assert abs(metrics.tok_s_from_tpot_ms(g[pre + "_tpot_ms"]) - g[pre + "_tok_s"]) < 2e-3
    assert round(metrics.speedup(g["spec_e2e_tok_s"], g["baseline_e2e_tok_s"]), 4) == g["speedup_e2e"]
    assert round(metrics.speedup(g["spec_decode_tok_s"], g["baseline_decode_tok_s"]), 4) == g["speedup_decode"]
