"""fp64 CPU oracle for greedy block verification -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The HIP
path never routes through it, and it shares no code with the HIP path: its only
inputs are the seeded model data from ``seeded_inputs`` (shapes, bf16 / int4
weights, token ids).

What it computes (plain, slow, obviously correct definitions, fp64 throughout,
weights widened exactly from bf16 or from int4 codes times bf16 scales):

* ``model.TokenDecoder`` -- one-position-per-call decoder with a KV cache: the
  decoder-only forward of a pre-norm GQA transformer (RMSNorm, rotate-half RoPE,
  softmax attention, SwiGLU/GeGLU MLP, tied LM head).
* ``model.forward_cacheless`` -- the same model recomputed over a whole token
  sequence without a cache (brute force; also teacher-forced scoring).
* ``spec.greedy_id`` -- argmax with ties to the lowest token id.
* ``spec.block_verify`` -- the acceptance rule of greedy speculative decoding:
  a draft is accepted only while it equals the target's greedy token after the
  same preceding ids; the longest matching prefix is committed and the cache is
  truncated to it ("Shape and cache history in Gemma block verification",
  section "Mechanism and failure"; "Phase 23: Speculative Verify Parity",
  section 2 "Design", steps 4 and 5).
* ``spec.greedy_generate`` / ``spec.spec_generate`` -- plain greedy decoding and
  the speculative loop built on ``block_verify``.

Pins (CPU tests, ``-m "not gpu"``) tie it to things other than itself:
cacheless brute force, a torch-CPU second formulation built on library
routines, closed forms (one-position attention, uniform attention, RoPE
identity/norm/relative-shift, rmsnorm of a constant vector, the zero-residual
model), spec-loop integer invariants, causality under changed future drafts,
exact rollback restoration, planted ties, int4 properties, and the tie
examples printed on the pages (``tests/golden``).  Nothing here is
"parity unpinned".
"""
from .model import Fp64Model, TokenDecoder, forward_cacheless  # noqa: F401
from .spec import (  # noqa: F401
    greedy_id, top2_margin, block_verify, greedy_generate, spec_generate, VerifyResult,
)
