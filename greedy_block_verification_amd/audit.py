"""Audit mode: sampled decode audit of a speculative stream, with top-k dumps.

"Phase 23: Speculative Verify Parity", section 4, leaves two diagnostics for
later: auditing sampled verify steps against plain one-token decode, and
dumping the top candidates where the two disagree.  DecodeAudit wraps one
context: every ``every``-th verify first clones the context's committed
state into a shadow context (``sv_clone_state``, on the device), runs the
verify with observer logits on, then replays the committed rows on the
shadow with one-token decodes and compares every row's logits bit for bit
and its argmax.  A disagreeing row is recorded with both sides' top-k
(``sv_topk``); the stream itself is never altered (observer mode does not
change the argmax).
"""
from __future__ import annotations

import numpy as np

from . import binding as B


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


class DecodeAudit:
    def __init__(self, session, shadow, every: int = 8, topk: int = 8):
        if every < 1 or not 1 <= topk <= 64:
            raise ValueError("every >= 1, 1 <= topk <= 64")
        self.s, self.shadow = session, shadow
        self.every, self.topk = every, topk
        self.steps = self.audited = self.rows_checked = 0
        self.mismatches = []

    def verify(self, drafts):
        s, sh = self.s, self.shadow
        self.steps += 1
        audit = self.steps % self.every == 0
        if not audit:
            return s.verify(drafts)
        B.sv_clone_state(sh.ctx, s.ctx)
        rows = [s.next_id] + [int(d) for d in drafts]
        s.set_debug(True)
        sh.set_debug(True)
        n, nx = s.verify(drafts)
        for r in range(n + 1):
            a_dec = sh.decode_step(rows[r])
            v, d = _bits(s.logits(r)), _bits(sh.logits(0))
            a_ver = s.last_argmax()[r]
            self.rows_checked += 1
            if a_ver != a_dec or not np.array_equal(v, d):
                self.mismatches.append({
                    "step": self.steps, "row": r, "position": sh.kv_len - 1,
                    "argmax_verify": a_ver, "argmax_decode": a_dec,
                    "differing_logits": int(np.count_nonzero(v != d)),
                    "topk_verify": B.sv_topk(s.ctx, r, self.topk),
                    "topk_decode": B.sv_topk(sh.ctx, 0, self.topk),
                })
        s.set_debug(False)
        sh.set_debug(False)
        self.audited += 1
        return n, nx
