"""Counter formulas of a speculative-decoding run.

Names follow the counters of "Phase 23: Speculative Verify Parity", section 3
(Validation): acceptance is accepted / proposed drafts; tokens per target step
divides committed tokens by every target forward (verify, commit decode,
correction and mirror decode steps); a TPOT in milliseconds converts to tokens
per second as 1000 / TPOT; a speedup is the ratio of speculative to baseline
throughput.
"""


def acceptance_rate(accepted: int, proposed: int) -> float:
    return accepted / proposed if proposed else 0.0


def target_steps(verify: int, commit_decode: int = 0, correction: int = 0, mirror_decode: int = 0) -> int:
    return verify + commit_decode + correction + mirror_decode


def tokens_per_target_step(tokens: int, steps: int) -> float:
    return tokens / steps if steps else 0.0


def tok_s_from_tpot_ms(tpot_ms: float) -> float:
    return 1000.0 / tpot_ms


def speedup(spec_tok_s: float, baseline_tok_s: float) -> float:
    return spec_tok_s / baseline_tok_s


def verified_tok_s(committed_tokens: int, seconds: float) -> float:
    """Committed (verified) tokens per second of verify wall time."""
    return committed_tokens / seconds if seconds > 0 else 0.0
