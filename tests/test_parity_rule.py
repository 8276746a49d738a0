"""The parity driver's tolerances and token rule, exercised on the CPU with the oracle on both sides.

A second oracle instance stands in for the GPU; mistakes are planted in what it hands over (its logits
and tokens), never in the product.  These check that the driver accepts an exact match over the full
length, and rejects a logit error above tolerance, a token mismatch inside the first 32 steps, and a
later mismatch that is not a near-tie of the oracle.
"""
import numpy as np
import pytest

from persistent_decode_megakernel_02_amd import synth
from persistent_decode_megakernel_02_amd.configs import TINY
from tests.parity import GAP, STRICT_STEPS, compare_teacher_forced, oracle_for

N = 48


@pytest.fixture(scope="module")
def run():
    weights = synth.make_weights(TINY, seed=0)
    prompt = synth.make_sequences(TINY, 1, 12, 0, seed=0)["prompts"][0].numpy()
    ref = oracle_for(TINY, weights, max_seq=11 + N, n_seq=1)
    for t in prompt[:-1]:
        ref.step(0, int(t), want_logits=False)
    toks, logits, tok = [], [], int(prompt[-1])
    for _ in range(N):
        lo = ref.step(0, tok)
        tok = int(np.argmax(lo))
        toks.append(tok)
        logits.append(lo)
    ref.close()
    return weights, prompt, np.array(toks), np.stack(logits)


def check(run, toks, logits, n=N):
    weights, prompt, _, _ = run
    orc = oracle_for(TINY, weights, max_seq=11 + N, n_seq=1)
    try:
        for t in prompt[:-1]:
            orc.step(0, int(t), want_logits=False)
        return compare_teacher_forced(orc, 0, int(prompt[-1]), toks, logits, n_check=n, label="rule")
    finally:
        orc.close()


def test_exact_match_runs_the_full_length(run):
    rep = check(run, run[2], run[3])
    assert rep.steps == N and rep.max_abs == 0.0 and rep.first_divergence is None


def test_logit_error_above_tolerance_fails(run):
    logits = run[3].copy()
    logits[7, 100] += 0.031
    with pytest.raises(AssertionError, match="step 7: max"):
        check(run, run[2], logits)


def test_mean_error_above_tolerance_fails(run):
    logits = run[3].copy()
    logits[3] += 0.0031 * np.where(np.arange(logits.shape[1]) == run[2][3], 0, 1).astype(np.float32)
    with pytest.raises(AssertionError, match="step 3: max"):
        check(run, run[2], logits)


def _swap_token(run, i):
    """GPU tokens/logits where step i picks the oracle's second-best token (its logit raised by a hair)."""
    toks, logits = run[2].copy(), run[3].copy()
    second = int(np.argsort(logits[i])[-2])
    logits[i, second] = logits[i, toks[i]] + 1e-6
    toks[i] = second
    return toks, logits, float(run[3][i, run[2][i]] - run[3][i, second])


def _gap(run, j):
    s = np.sort(run[3][j])
    return float(s[-1] - s[-2])


def test_token_mismatch_inside_strict_steps_fails(run):
    # a step whose top-2 gap is within the logit tolerance, so only the token rule can reject the swap
    i = next(j for j in range(STRICT_STEPS) if _gap(run, j) < 0.02)
    toks, logits, _ = _swap_token(run, i)
    with pytest.raises(AssertionError, match=f"first {STRICT_STEPS} steps"):
        check(run, toks, logits, n=i + 1)


def test_late_mismatch_depends_on_the_oracle_gap(run):
    i = next(j for j in range(STRICT_STEPS, N) if _gap(run, j) < 0.02)
    toks, logits, gap = _swap_token(run, i)
    assert gap < GAP
    rep = check(run, toks, logits, n=i + 1)  # a near-tie: accepted, and the run goes on to the end
    assert rep.steps == i + 1 and rep.first_divergence == i
    # the same swap against a token far below the oracle's best is rejected
    # rejected: a token more than GAP below the oracle's best whose GPU logits stay within tolerance
    # (the GPU's best logit moved down and that token's moved up by about half the difference each)
    def third_gap(j):
        s3 = np.sort(run[3][j])
        return float(s3[-1] - s3[-3])
    j = next(j for j in range(STRICT_STEPS, N) if GAP < third_gap(j) < 0.058)
    toks2, logits2 = run[2].copy(), run[3].copy()
    third = int(np.argsort(logits2[j])[-3])
    half = third_gap(j) / 2
    logits2[j, toks2[j]] -= half
    logits2[j, third] += half + 2e-4
    assert int(np.argmax(logits2[j])) == third
    toks2[j] = third
    with pytest.raises(AssertionError, match="not a near-tie"):
        check(run, toks2, logits2, n=j + 1)


def test_asking_for_more_steps_than_produced_fails(run):
    with pytest.raises(AssertionError, match="asked for"):
        check(run, run[2][:5], run[3][:5], n=6)
