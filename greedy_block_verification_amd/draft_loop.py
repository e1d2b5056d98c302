"""Draft model in the loop: draft-then-verify speculative decoding with two
contexts on one GPU.

The setup of "Phase 23: Speculative Verify Parity", section 3 (a 0.6B-shaped
draft proposing for an 8B-shaped target, the committed-token throughput
measured end to end against plain target decoding) on this library's
calls:

* the draft context proposes K ids with K one-token decodes
  (``sv_decode_step``): the pending target token, then its own guesses;
* the target verifies them in one forward (``sv_verify``);
* the draft context rolls back to the committed prefix with
  ``sv_kv_truncate`` (O(1)), and when every draft was accepted it decodes
  the last draft so it has seen every committed position.

A round costs K (or K + 1) draft decodes and one target forward of K + 1
rows and commits n + 1 ids; DraftLoop keeps the draft and verify wall time
apart so the end-to-end rate and its split can be reported.

Both contexts then hold exactly the committed prefix, so the draft's cache is
the one a plain one-token decode of the committed sequence builds (tested).
``proposer`` may replace the draft model's own guesses -- random-init models
almost never agree, so measurements drive acceptance with seeded synthetic
windows while the draft's decodes still run and cost what they cost.
"""
from __future__ import annotations

import time

from . import binding as B


class DraftLoop:
    """One generation stream: a target session and a draft session over the
    same committed prefix (both prefilled with the same prompt)."""

    def __init__(self, target, draft, proposer=None):
        if target.kv_len != draft.kv_len:
            raise ValueError("target and draft contexts must hold the same committed prefix")
        self.t, self.d = target, draft
        self.proposer = proposer           # fn(k) -> k ids, or None for the draft's own guesses
        self.draft_s = self.verify_s = 0.0
        self.proposed = self.accepted = self.steps = 0

    def step(self, k: int):
        """One round: K draft decodes, one verify, the rollback.  Returns the
        committed ids (the pending token and the accepted drafts)."""
        t, d = self.t, self.d
        base = t.kv_len
        cur = t.next_id
        t0 = time.perf_counter()
        # the draft decodes the pending token, then d_0 .. d_{k-2}: positions base .. base + k - 1
        if self.proposer is None:
            drafts, x = [], cur
            for _ in range(k):
                x = d.decode_step(x)
                drafts.append(x)
        else:
            drafts = [int(v) for v in self.proposer(k)]
            for x in [cur] + drafts[:k - 1] if k > 0 else []:
                d.decode_step(x)
        t1 = time.perf_counter()
        n, nx = t.verify(drafts)
        t2 = time.perf_counter()
        keep = base + n + 1
        committed = [cur] + drafts[:n]
        if keep <= d.kv_len:
            d.truncate(keep)
        else:                               # every draft accepted (or k = 0): feed what the draft has not seen
            for x in committed[d.kv_len - base:]:
                d.decode_step(x)
        self.draft_s += (t1 - t0) + (time.perf_counter() - t2)
        self.verify_s += t2 - t1
        self.proposed += k
        self.accepted += n
        self.steps += 1
        assert d.kv_len == t.kv_len == keep
        return committed


def prefill_pair(target, draft, ids):
    """Prefill the same prompt into both contexts."""
    nt = B.sv_prefill(target.ctx, ids)
    B.sv_prefill(draft.ctx, ids)
    return nt
