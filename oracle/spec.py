"""Greedy block verification by its plain definition -- test infrastructure only.

Acceptance rule ("Shape and cache history in Gemma block verification",
section "Mechanism and failure"): a draft token is accepted only if it equals
the target's greedy token after the same preceding ids; a causal block forward
merely computes all those decisions at once.  Here every decision is taken by
the per-token decoder, one position per call -- never by a block forward.

Window of one verify at committed prefix T (kv_len = len(T)) whose pending
greedy token is ``next`` (decided, not yet in the cache), with drafts
d_0..d_{K-1}:

  rows   w_0 = next, w_r = d_{r-1}             (K + 1 rows)
  a_r    = greedy(T + w_0..w_r)                 (row r's greedy id)
  n      = number of leading i with d_i == a_i  (0 <= n <= K)
  commit T + w_0..w_n ; new next = a_n          (the correction, or the bonus
                                                  token when every draft holds)

Rollback ("Phase 23: Speculative Verify Parity", section 2, steps 4-5): when all
drafts are accepted the written KV is kept; otherwise the cache is truncated to
the accepted prefix.  Ties in the argmax go to the lowest id.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .model import TokenDecoder


def greedy_id(logits: np.ndarray) -> int:
    """Largest logit; among equal maxima the lowest token id."""
    m = np.max(logits)
    return int(np.flatnonzero(logits == m)[0])


def top2_margin(logits: np.ndarray) -> float:
    """top1 - top2 of a logit vector (0 for an exact tie)."""
    part = np.partition(logits, -2)[-2:]
    return float(part[1] - part[0])


@dataclass
class VerifyResult:
    n_accepted: int
    next_id: int
    row_argmax: list        # a_0..a_K
    row_logits: list        # fp64 logits of every row


def block_verify(dec: TokenDecoder, next_id: int, drafts, keep_logits: bool = False) -> VerifyResult:
    """One verify window on ``dec`` (whose length is the committed prefix)."""
    base = dec.length
    rows = [int(next_id)] + [int(d) for d in drafts]
    a, logits = [], []
    for tok in rows:
        lg = dec.decode(tok)
        a.append(greedy_id(lg))
        if keep_logits:
            logits.append(lg)
    n = 0
    while n < len(drafts) and int(drafts[n]) == a[n]:
        n += 1
    dec.truncate(base + n + 1)
    return VerifyResult(n, a[n], a, logits)


def prefill(dec: TokenDecoder, ids) -> int:
    """Feed ``ids`` one by one; return the greedy id after them."""
    lg = None
    for t in ids:
        lg = dec.decode(int(t))
    return greedy_id(lg)


def greedy_generate(dec: TokenDecoder, next_id: int, n: int) -> list:
    """Plain greedy decoding: commit ``next_id`` and the n-1 greedy ids after it."""
    out = []
    cur = int(next_id)
    for _ in range(n):
        out.append(cur)
        cur = greedy_id(dec.decode(cur))
    return out


def spec_generate(dec: TokenDecoder, next_id: int, n_gen: int, k: int, draft_fn):
    """Speculative greedy loop; returns (committed ids, per-verify (k_eff, n) list).

    ``draft_fn(committed_so_far, next_id, k_eff)`` proposes k_eff ids.  The
    window shrinks to ``min(k, remaining - 1)`` so exactly n_gen ids commit.
    """
    out, steps = [], []
    cur = int(next_id)
    while len(out) < n_gen:
        k_eff = min(k, n_gen - len(out) - 1)
        drafts = list(draft_fn(list(out), cur, k_eff)) if k_eff > 0 else []
        r = block_verify(dec, cur, drafts)
        out += [cur] + drafts[:r.n_accepted]
        steps.append((k_eff, r.n_accepted))
        cur = r.next_id
    return out, steps
