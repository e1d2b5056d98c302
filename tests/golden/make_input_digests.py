"""Writes input_digests.json: a regression digest of the seeded input generator.

Run from the repository root: python tests/golden/make_input_digests.py
It calls only ``seeded_inputs`` (no GPU code, no oracle arithmetic).
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from seeded_inputs import generate_weights, get_config, prompt_ids  # noqa: E402
from test_inputs import _digest  # noqa: E402

out = {
    "tiny_weights_sha256": _digest(generate_weights(get_config("tiny"), threads=1)),
    "tiny_prompt0": prompt_ids(1, 0, 32, 2048).tolist(),
}
json.dump(out, open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_digests.json"), "w"), indent=1)
print(out["tiny_weights_sha256"])
