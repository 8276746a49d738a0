"""Error paths through the C ABI on the GPU (tiny model).

Argument, state and capacity errors are caught on the host, leave the context as it was, and
decoding can fill max_seq exactly. A poll budget of one poll per wait, set from the host,
makes the kernel's own bounded waits give up. The launch then ends with MK_ERR_TIMEOUT, and the
GPU goes on decoding correctly in a new context. Whether a wait exceeds that budget depends on
timing, so a run that never needs a second poll may also finish normally, with the same
tokens."""
import numpy as np
import pytest
import torch

from persistent_decode_megakernel_02_amd import binding as mk, synth
from persistent_decode_megakernel_02_amd.configs import TINY

pytestmark = pytest.mark.gpu

PROMPT = 20


def _inputs():
    weights = synth.make_weights(TINY, seed=5, device="cuda")
    prompt = synth.make_sequences(TINY, 1, PROMPT, 0, seed=5)["prompts"].numpy()
    return weights, prompt


def _code(call):
    with pytest.raises(mk.MkError) as e:
        call()
    return e.value.code


def _decode_fresh(weights, prompt, max_seq, n):
    eng = mk.Engine(TINY, batch=1, max_seq=max_seq)
    eng.load_weights(weights)
    eng.prefill(prompt)
    toks, logits = eng.decode(n)
    torch.cuda.synchronize()
    out = toks.cpu().numpy(), logits.cpu().numpy()
    eng.close()
    return out


def test_state_argument_and_capacity_errors_leave_the_context_usable():
    print("errors: state / argument / capacity", flush=True)
    weights, prompt = _inputs()
    max_seq = PROMPT - 1 + 11
    eng = mk.Engine(TINY, batch=1, max_seq=max_seq)
    assert _code(lambda: eng.decode(1)) == mk.MK_ERR_STATE  # no weights yet
    eng.load_weights(weights)
    bad = prompt.copy()
    bad[0, 3] = TINY.vocab
    assert _code(lambda: eng.prefill(bad)) == mk.MK_ERR_INVALID_ARG  # token id out of range
    assert _code(lambda: eng.prefill(np.zeros((1, max_seq + 1), np.int32))) == mk.MK_ERR_CAPACITY
    assert _code(lambda: eng.set_mode(7)) == mk.MK_ERR_INVALID_ARG
    eng.prefill(prompt)
    assert eng.state()[0] == PROMPT - 1
    assert _code(lambda: eng.decode(12)) == mk.MK_ERR_CAPACITY  # one step past max_seq
    assert eng.state()[0] == PROMPT - 1  # unchanged
    toks, logits = eng.decode(11)  # exactly to max_seq
    torch.cuda.synchronize()
    assert eng.state()[0] == max_seq
    assert _code(lambda: eng.decode(1)) == mk.MK_ERR_CAPACITY
    t_ref, l_ref = _decode_fresh(weights, prompt, max_seq, 11)
    assert np.array_equal(toks.cpu().numpy(), t_ref)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), l_ref.view(np.uint32))
    eng.close()


def test_exhausted_poll_budget_ends_the_launch_with_a_timeout():
    print("errors: poll budget of one", flush=True)
    weights, prompt = _inputs()
    max_seq, n = PROMPT - 1 + 32, 32
    t_ref, _ = _decode_fresh(weights, prompt, max_seq, n)
    eng = mk.Engine(TINY, batch=1, max_seq=max_seq, watchdog_polls=1)
    eng.load_weights(weights)
    eng.prefill(prompt)  # its attention merges poll with the same budget; a give-up there is reported by decode
    try:
        toks, _ = eng.decode(n)
        torch.cuda.synchronize()
        timed_out = False
    except mk.MkError as e:
        assert e.code == mk.MK_ERR_TIMEOUT, str(e)
        assert "watchdog" in str(e)
        timed_out = True
    print("timed out" if timed_out else "finished within the budget", flush=True)
    if not timed_out:
        assert np.array_equal(toks.cpu().numpy(), t_ref)
    eng.reset()
    eng.close()
    # the GPU keeps decoding correctly
    t_after, _ = _decode_fresh(weights, prompt, max_seq, n)
    assert np.array_equal(t_after, t_ref)


@pytest.mark.parametrize("batch,lora", [(1, 0), (4, 16), (16, 0)])
def test_nan_canaries_in_scratch_are_never_read(batch, lora):
    # Scratch filled with NaN (and tags no step uses) after the prefill: the decode writes every
    # activation and partial before reading it, so tokens and logits equal a clean context's.
    from dataclasses import replace
    from persistent_decode_megakernel_02_amd.configs import ModelShape
    shape = replace(TINY, lora_rank=lora) if batch < 8 else ModelShape(2, 512, 8, 2, 64, 1024, 1000)
    print(f"[case] NaN canaries batch={batch} lora={lora}", flush=True)
    weights = synth.make_weights(shape, seed=4, device="cuda")
    seqs = synth.make_sequences(shape, batch, 11, 0, seed=4)
    outs = []
    for poison in (False, True):
        eng = mk.Engine(shape, batch=batch, max_seq=10 + 8)
        try:
            eng.load_weights(weights)
            eng.prefill(seqs["prompts"].numpy())
            if poison:
                mk.mk_debug_poison(eng.ctx)
            toks, logits = eng.decode(8)
            torch.cuda.synchronize()
            outs.append((toks.cpu().numpy(), logits.cpu().numpy()))
        finally:
            eng.close()
    assert np.all(np.isfinite(outs[1][1]))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
