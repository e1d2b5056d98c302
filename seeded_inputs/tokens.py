"""Seeded prompt ids and draft windows.

Prompts are ``integers(0, V)`` from ``SeedSequence([seed + 100, prompt_index])``.
Draft windows are derived from the target's true greedy continuation (computed
by whichever side runs the workload) and a seeded generator
``SeedSequence([seed + 200, stream, step])``: each window position is the true
token with probability ``p_correct``, otherwise a uniformly random *wrong* id.
Fixed patterns (all-accept, wrong at index 2, wrong at index 0) put a random
wrong id at the named index and the true tokens elsewhere.
"""
from __future__ import annotations

import numpy as np

PATTERNS = ("all_accept", "mismatch_at_2", "mismatch_at_0")


def prompt_ids(seed: int, index: int, length: int, vocab: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed + 100, index])))
    return g.integers(0, vocab, size=length, dtype=np.int64).astype(np.int32)


def _wrong_id(g: np.random.Generator, true_id: int, vocab: int) -> int:
    x = int(g.integers(0, vocab - 1))
    return x + 1 if x >= true_id else x


def draft_window(truth, k: int, vocab: int, rng: np.random.Generator,
                 p_correct: float | None = None, pattern: str | None = None) -> list:
    """k draft ids proposing ``truth[0:k]`` with seeded corruption."""
    truth = [int(t) for t in truth[:k]]
    assert len(truth) == k
    out = []
    for i, t in enumerate(truth):
        if pattern is not None:
            wrong = (pattern == "mismatch_at_2" and i == 2) or (pattern == "mismatch_at_0" and i == 0)
        else:
            wrong = bool(rng.random() >= p_correct)
        out.append(_wrong_id(rng, t, vocab) if wrong else t)
    return out


class DraftSource:
    """Stateful seeded draft generator for one generation stream."""

    def __init__(self, seed: int, stream: int, vocab: int,
                 p_correct: float | None = None, pattern: str | None = None):
        assert (p_correct is None) != (pattern is None)
        self.rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed + 200, stream])))
        self.vocab, self.p, self.pattern = vocab, p_correct, pattern

    def window(self, truth, k: int) -> list:
        return draft_window(truth, k, self.vocab, self.rng, self.p, self.pattern)
