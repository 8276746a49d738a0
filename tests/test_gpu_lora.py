"""GPU parity of the fused LoRA + Linear path (Mirage article, "Case 2: LoRA + Linear").

Every projection of every layer carries a rank-r adapter, and each GEMV tile computes its
operator's y = W x + B (A x) as the concatenated product (W|B)(x|A x).  Checked against the CPU
oracle (teacher-forced, 32 steps), between the megakernel and the per-operator launches (bit for
bit), and across schedules.  Every case prints its name before touching the GPU.
"""
from dataclasses import replace

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from persistent_decode_megakernel_02_amd import binding as mk  # noqa: E402
from persistent_decode_megakernel_02_amd import synth  # noqa: E402
from persistent_decode_megakernel_02_amd.configs import TINY  # noqa: E402
from tests.parity import compare_teacher_forced, oracle_for  # noqa: E402

pytestmark = pytest.mark.gpu

TINY_LORA = replace(TINY, lora_rank=16)
TINY_LORA64_QK = replace(TINY, n_kv_heads=4, qk_norm=True, lora_rank=64)


def say(msg):
    print(f"[case] {msg}", flush=True)


def run(shape, batch, prompt_len, n_steps, mode=mk.MK_MODE_MEGAKERNEL, split=0, n_workers=0, schedule=None,
        seed=0):
    weights = synth.make_weights(shape, seed=seed, device="cuda")
    seqs = synth.make_sequences(shape, batch, prompt_len, 0, seed=seed)
    eng = mk.Engine(shape, batch=batch, max_seq=prompt_len - 1 + n_steps, mode=mode, split=split,
                    n_workers=n_workers, schedule=schedule)
    try:
        eng.load_weights(weights)
        eng.prefill(seqs["prompts"].numpy())
        toks, logits = eng.decode(n_steps)
        torch.cuda.synchronize()
        out = toks.cpu().numpy(), logits.cpu().numpy()
    finally:
        eng.close()
    return weights, seqs, out


def check(shape, weights, seqs, toks, logits, n_steps, label):
    P = seqs["prompts"].shape[1]
    orc = oracle_for(shape, weights, max_seq=P - 1 + n_steps, n_seq=toks.shape[1])
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


@pytest.mark.parametrize("shape,batch,n_workers,split", [
    (TINY_LORA, 1, 0, 0), (TINY_LORA, 1, 8, 16), (TINY_LORA, 2, 37, 8), (TINY_LORA, 4, 0, 4),
    (TINY_LORA64_QK, 1, 0, 0), (TINY_LORA64_QK, 4, 8, 0),
])
def test_lora_megakernel_matches_oracle(shape, batch, n_workers, split):
    say(f"LoRA r={shape.lora_rank} batch={batch} workers={n_workers} split={split}")
    w, s, (toks, logits) = run(shape, batch, 39, 32, split=split, n_workers=n_workers)
    check(shape, w, s, toks, logits, 32, f"lora{shape.lora_rank}")


def test_lora_changes_the_result():
    # the adapters are not a no-op: the same weights without them give other logits
    say("LoRA vs the same base weights without adapters")
    w, s, (_, l1) = run(TINY_LORA, 1, 39, 4)
    n_base = len(synth.canonical_names(TINY))
    eng = mk.Engine(TINY, batch=1, max_seq=42)
    try:
        eng.load_weights(w[:n_base])
        eng.prefill(s["prompts"].numpy())
        _, l0 = eng.decode(4)
        torch.cuda.synchronize()
        l0 = l0.cpu().numpy()
    finally:
        eng.close()
    assert np.abs(l1 - l0).max() > 1e-2


@pytest.mark.parametrize("batch,n_workers,split,sched", [
    (1, 0, 0, dict(rotate=3, attn_offset=5)),
    (2, 8, 16, dict(qkv_tiles=3, wo_tiles=5, gu_tiles=7, down_tiles=6, lm_tiles=4)),
    (4, 37, 0, dict(wo_tiles=2, gu_tiles=30, rotate=36)),
])
def test_lora_per_op_and_schedules_are_bit_identical(batch, n_workers, split, sched):
    say(f"LoRA per-op and schedule {sched} batch={batch} workers={n_workers}")
    _, _, (t0, l0) = run(TINY_LORA, batch, 23, 20, split=split, n_workers=n_workers)
    _, _, (t1, l1) = run(TINY_LORA, batch, 23, 20, mode=mk.MK_MODE_PER_OP, split=split, n_workers=n_workers)
    _, _, (t2, l2) = run(TINY_LORA, batch, 23, 20, split=split, n_workers=n_workers, schedule=sched)
    for t, lg in ((t1, l1), (t2, l2)):
        assert np.array_equal(t0, t)
        assert np.array_equal(l0.view(np.uint32), lg.view(np.uint32))


def test_lora_errors():
    say("LoRA errors: batch 8, missing adapter tensor")
    with pytest.raises(mk.MkError) as e:
        mk.Engine(replace(TINY, hidden=512, ffn=1024, lora_rank=8), batch=8, max_seq=16)
    assert e.value.code == mk.MK_ERR_UNSUPPORTED
    eng = mk.Engine(TINY_LORA, batch=1, max_seq=16)
    try:
        w = synth.make_weights(TINY_LORA, seed=0, device="cuda")
        with pytest.raises(mk.MkError) as e:
            eng.load_weights([x for x in w if x[0] != "layers.1.lora_b.up"])
        assert e.value.code == mk.MK_ERR_INVALID_ARG
    finally:
        eng.close()
