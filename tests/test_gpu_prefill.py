"""GPU parity of the megakernel prefill (MK_PREFILL_MEGAKERNEL).

The prompt runs through the persistent kernel, a chunk of C tokens per step as the columns of
every projection (C = 16 on the matrix cores where the shape allows, else 4), an append task per
KV-head group writing the chunk's keys and values, and each token attending up to its own
position.  Checked by decoding after it: against the CPU oracle (teacher-forced, 32 steps), and
against the per-operator prefill.  Every case prints its name before touching the GPU.
"""
from dataclasses import replace

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from persistent_decode_megakernel_02_amd import binding as mk  # noqa: E402
from persistent_decode_megakernel_02_amd import synth  # noqa: E402
from persistent_decode_megakernel_02_amd.configs import TINY, ModelShape  # noqa: E402
from tests.parity import compare_teacher_forced, oracle_for  # noqa: E402

pytestmark = pytest.mark.gpu

# hidden, ffn and Hq * D multiples of 512: 16-token chunks on the matrix cores
WIDE = ModelShape(n_layers=2, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=5632, vocab=3000,
                  rope_theta=500000.0)
TINY_QK = replace(TINY, n_kv_heads=4, qk_norm=True)


def say(msg):
    print(f"[case] {msg}", flush=True)


def run(shape, batch, prompt_len, n_steps, prefill, n_workers=0, split=0, seed=0):
    weights = synth.make_weights(shape, seed=seed, device="cuda")
    seqs = synth.make_sequences(shape, batch, prompt_len, 0, seed=seed)
    eng = mk.Engine(shape, batch=batch, max_seq=prompt_len - 1 + n_steps, n_workers=n_workers, split=split,
                    prefill=prefill)
    try:
        eng.load_weights(weights)
        eng.prefill(seqs["prompts"].numpy())
        pos, _ = eng.state()
        assert pos == prompt_len - 1
        toks, logits = eng.decode(n_steps)
        torch.cuda.synchronize()
        out = toks.cpu().numpy(), logits.cpu().numpy()
    finally:
        eng.close()
    return weights, seqs, out


def check(shape, weights, seqs, toks, logits, n_steps, label, n_threads=1):
    P = seqs["prompts"].shape[1]
    orc = oracle_for(shape, weights, max_seq=P - 1 + n_steps, n_seq=toks.shape[1], n_threads=n_threads)
    try:
        for b in range(toks.shape[1]):
            prompt = seqs["prompts"][b].numpy()
            for t in prompt[:-1]:
                orc.step(b, int(t), want_logits=False)
            rep = compare_teacher_forced(orc, b, int(prompt[-1]), toks[:, b], logits[:, b], n_check=n_steps,
                                         label=f"{label} seq {b}")
            assert rep.steps == n_steps
    finally:
        orc.close()


# prompt lengths: whole chunks, a ragged last chunk, shorter than one chunk, a single token
@pytest.mark.parametrize("shape,batch,prompt_len,n_workers,split", [
    (TINY, 1, 39, 0, 0), (TINY, 2, 17, 0, 0), (TINY, 4, 3, 8, 16), (TINY, 1, 2, 0, 0), (TINY, 1, 1, 0, 0),
    (TINY_QK, 1, 30, 37, 0), (TINY, 1, 40, 0, 4),
])
def test_megakernel_prefill_tiny_matches_oracle(shape, batch, prompt_len, n_workers, split):
    say(f"megakernel prefill tiny batch={batch} prompt={prompt_len} workers={n_workers} split={split}")
    w, s, (toks, logits) = run(shape, batch, prompt_len, 32, mk.MK_PREFILL_MEGAKERNEL, n_workers, split)
    check(shape, w, s, toks, logits, 32, "mk-prefill tiny")


@pytest.mark.parametrize("batch,prompt_len", [(1, 39), (2, 50), (1, 16)])
def test_megakernel_prefill_matrix_cores_matches_oracle(batch, prompt_len):
    say(f"megakernel prefill, 16-token chunks on the matrix cores, batch={batch} prompt={prompt_len}")
    w, s, (toks, logits) = run(WIDE, batch, prompt_len, 32, mk.MK_PREFILL_MEGAKERNEL)
    check(WIDE, w, s, toks, logits, 32, "mk-prefill wide", n_threads=8)


def test_megakernel_prefill_agrees_with_per_op_prefill():
    say("megakernel prefill vs per-operator prefill, tiny and wide")
    for shape in (TINY, WIDE):
        _, _, (t0, l0) = run(shape, 1, 39, 16, mk.MK_PREFILL_PER_OP)
        _, _, (t1, l1) = run(shape, 1, 39, 16, mk.MK_PREFILL_MEGAKERNEL)
        assert np.array_equal(t0, t1)
        assert np.abs(l0 - l1).max() < 1e-3


@pytest.mark.parametrize("shape", [TINY, WIDE, replace(TINY, lora_rank=16)])
def test_second_megakernel_prefill_on_one_context(shape):
    # a second prefill restarts the prefill graph's steps: its step-tagged words must not meet the
    # first prefill's (same tags); the result equals a fresh context's
    say(f"two megakernel prefills on one context, {shape.hidden}x{shape.n_layers} lora={shape.lora_rank}")
    weights = synth.make_weights(shape, seed=0, device="cuda")
    s1 = synth.make_sequences(shape, 1, 30, 0, seed=1)
    s2 = synth.make_sequences(shape, 1, 30, 0, seed=2)
    outs = []
    for prompts in ((s1, s2), (s2,)):
        eng = mk.Engine(shape, batch=1, max_seq=29 + 12, prefill=mk.MK_PREFILL_MEGAKERNEL)
        try:
            eng.load_weights(weights)
            for p in prompts:
                eng.prefill(p["prompts"].numpy())
                toks, logits = eng.decode(12)
            torch.cuda.synchronize()
            outs.append((toks.cpu().numpy(), logits.cpu().numpy()))
        finally:
            eng.close()
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
