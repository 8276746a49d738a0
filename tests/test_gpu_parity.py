"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from persistent_decode_megakernel_02_amd import binding as mk  # noqa: E402
from persistent_decode_megakernel_02_amd import synth  # noqa: E402
from persistent_decode_megakernel_02_amd.configs import TINY, ModelShape  # noqa: E402
from tests.parity import compare_teacher_forced, oracle_for  # noqa: E402

pytestmark = pytest.mark.gpu

TINY_MHA_QK = ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=688, vocab=512,
                         qk_norm=True)
# wide enough that at batch 8 and 16 the activations exceed the LDS staging area and every GEMV runs in
# K slices (the last one ragged)
WIDE = ModelShape(n_layers=2, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=5632, vocab=3000,
                  rope_theta=500000.0)
TINY_G4 = ModelShape(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1000, vocab=2000,
                     rope_theta=500000.0)


def say(msg):
    print(f"[case] {msg}", flush=True)


def run_prompt_case(shape, batch, prompt_len, n_steps, mode=mk.MK_MODE_MEGAKERNEL, split=0, n_workers=0, seed=0,
                    schedule=None):
    weights = synth.make_weights(shape, seed=seed, device="cuda")
    seqs = synth.make_sequences(shape, batch, prompt_len, 0, seed=seed)
    max_seq = prompt_len - 1 + n_steps
    eng = mk.Engine(shape, batch=batch, max_seq=max_seq, mode=mode, split=split, n_workers=n_workers,
                    schedule=schedule)
    eng.load_weights(weights)
    eng.prefill(seqs["prompts"].numpy())
    toks, logits = eng.decode(n_steps)
    torch.cuda.synchronize()
    out = toks.cpu().numpy(), logits.cpu().numpy()
    eng.close()
    return weights, seqs, out


def check_against_oracle(shape, weights, seqs, toks, logits, n_steps, label, n_threads=1):
    batch = toks.shape[1]
    P = seqs["prompts"].shape[1]
    orc = oracle_for(shape, weights, max_seq=P - 1 + n_steps, n_seq=batch, n_threads=n_threads)
    for b in range(batch):
        prompt = seqs["prompts"][b].numpy()
        for t in prompt[:-1]:
            orc.step(b, int(t), want_logits=False)
        rep = compare_teacher_forced(orc, b, int(prompt[-1]), toks[:, b], logits[:, b], n_check=n_steps,
                                     label=f"{label} seq {b}")
        assert rep.steps == n_steps
    orc.close()


# (8, 16): one merging split per head, listed after the others; (0, 0), (37, 32): every attention
# task on a worker of its own, one merging split; (0, 4): 10 to 18 active splits, each merging a
# slice of the outputs; (40, 8): 5 to 9 active splits, both merge forms
@pytest.mark.parametrize("n_workers,split", [(0, 0), (8, 16), (37, 32), (0, 4), (40, 8)])
def test_tiny_megakernel_matches_oracle(n_workers, split):
    say(f"tiny megakernel workers={n_workers} split={split}")
    w, s, (toks, logits) = run_prompt_case(TINY, 1, 39, 32, split=split, n_workers=n_workers)
    check_against_oracle(TINY, w, s, toks, logits, 32, "tiny")


@pytest.mark.parametrize("n_workers,split", [(8, 16), (0, 4)])
def test_tiny_per_op_is_bit_identical_to_megakernel(n_workers, split):
    say(f"tiny per-op vs megakernel workers={n_workers} split={split}")
    _, _, (t0, l0) = run_prompt_case(TINY, 1, 39, 32, mode=mk.MK_MODE_MEGAKERNEL, split=split, n_workers=n_workers)
    _, _, (t1, l1) = run_prompt_case(TINY, 1, 39, 32, mode=mk.MK_MODE_PER_OP, split=split, n_workers=n_workers)
    assert np.array_equal(t0, t1)
    assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32))


# A schedule moves tiles between workers and changes their sizes; every row's sum and every attention
# split is computed the same way wherever it runs, so the results are bit-identical to the plain
# schedule's, in both modes.
SCHEDULES = [
    (1, 0, 0, dict(rotate=1, attn_offset=3)),
    (1, 8, 0, dict(qkv_tiles=3, wo_tiles=5, gu_tiles=7, down_tiles=6, lm_tiles=4, rotate=5, attn_offset=2)),
    (2, 37, 8, dict(qkv_tiles=7, wo_tiles=37, gu_tiles=20, down_tiles=11, lm_tiles=37, rotate=36, attn_offset=30)),
    (4, 0, 0, dict(qkv_tiles=16, wo_tiles=128, gu_tiles=200, down_tiles=255, lm_tiles=64, rotate=77,
                   attn_offset=129)),
]


@pytest.mark.parametrize("batch,n_workers,split,sched", SCHEDULES)
def test_tiny_schedules_are_bit_identical(batch, n_workers, split, sched):
    say(f"tiny schedule batch={batch} workers={n_workers} split={split} {sched}")
    w, s, (t0, l0) = run_prompt_case(TINY, batch, 23, 24, split=split, n_workers=n_workers)
    _, _, (t1, l1) = run_prompt_case(TINY, batch, 23, 24, split=split, n_workers=n_workers, schedule=sched)
    _, _, (t2, l2) = run_prompt_case(TINY, batch, 23, 24, mode=mk.MK_MODE_PER_OP, split=split, n_workers=n_workers,
                                     schedule=sched)
    assert np.array_equal(t0, t1) and np.array_equal(t0, t2)
    assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32))
    assert np.array_equal(l0.view(np.uint32), l2.view(np.uint32))
    check_against_oracle(TINY, w, s, t1, l1, 24, "tiny scheduled")


def test_tiny_megakernel_deterministic_and_resumable():
    say("tiny determinism / split decode calls")
    shape = TINY
    weights = synth.make_weights(shape, seed=3, device="cuda")
    seqs = synth.make_sequences(shape, 1, 39, 0, seed=3)
    res = []
    for chunks in ([32], [32], [5, 27], [1, 1, 30]):
        eng = mk.Engine(shape, batch=1, max_seq=38 + 32)
        eng.load_weights(weights)
        eng.prefill(seqs["prompts"].numpy())
        ts, ls = [], []
        for n in chunks:
            t, l = eng.decode(n)
            ts.append(t.cpu().numpy())
            ls.append(l.cpu().numpy())
        pos, pend = eng.state()
        assert pos == 38 + 32
        res.append((np.concatenate(ts), np.concatenate(ls)))
        eng.close()
    for t, l in res[1:]:
        assert np.array_equal(t, res[0][0])
        assert np.array_equal(l.view(np.uint32), res[0][1].view(np.uint32))


def test_tiny_mha_qknorm_matches_oracle():
    say("tiny MHA + QK-norm")
    w, s, (toks, logits) = run_prompt_case(TINY_MHA_QK, 1, 20, 40, split=16, n_workers=64)
    check_against_oracle(TINY_MHA_QK, w, s, toks, logits, 40, "tiny-mha-qk")


def test_g4_head128_matches_oracle():
    say("G=4 head_dim=128 ragged ffn/vocab")
    w, s, (toks, logits) = run_prompt_case(TINY_G4, 1, 30, 36, split=32, n_workers=256)
    check_against_oracle(TINY_G4, w, s, toks, logits, 36, "g4")


@pytest.mark.parametrize("batch", [2, 4])
def test_batched_sequences_match_oracle(batch):
    say(f"tiny batch={batch}")
    w, s, (toks, logits) = run_prompt_case(TINY, batch, 17, 33, split=16, n_workers=128)
    check_against_oracle(TINY, w, s, toks, logits, 33, f"tiny-b{batch}")


def test_prefilled_kv_matches_oracle():
    say("tiny pre-filled KV")
    shape, B, n_pos, n_steps = TINY_G4, 2, 150, 34
    weights = synth.make_weights(shape, seed=5, device="cuda")
    seqs = synth.make_sequences(shape, B, 0, n_pos, seed=5, device="cuda")
    eng = mk.Engine(shape, batch=B, max_seq=n_pos + n_steps, split=32)
    eng.load_weights(weights)
    for b in range(B):
        eng.load_kv(b, seqs["k"][b], seqs["v"][b], int(seqs["pending"][b]))
    toks, logits = eng.decode(n_steps)
    toks, logits = toks.cpu().numpy(), logits.cpu().numpy()
    eng.close()
    orc = oracle_for(shape, weights, max_seq=n_pos + n_steps, n_seq=B)
    for b in range(B):
        orc.set_kv(b, synth.bf16_bits(seqs["k"][b]), synth.bf16_bits(seqs["v"][b]))
        rep = compare_teacher_forced(orc, b, int(seqs["pending"][b]), toks[:, b], logits[:, b], n_check=n_steps,
                                     label=f"kv seq {b}")
        assert rep.steps == n_steps


@pytest.mark.parametrize("batch,prompt,steps", [(8, 9, 24), (16, 5, 20)])
def test_k_sliced_batches_match_oracle(batch, prompt, steps):
    say(f"wide batch={batch}: K-sliced activation staging")
    w, s, (toks, logits) = run_prompt_case(WIDE, batch, prompt, steps)
    check_against_oracle(WIDE, w, s, toks, logits, steps, f"wide-b{batch}", n_threads=16)


# split-K of the O- and down-projection at batch >= 8: Hq D = 4096 gives WO two K slices of 2048,
# F = 7168 gives DOWN four (the last ragged); WIDE's F = 5632 splits its three slices as 1 + 2
WIDE_K = ModelShape(n_layers=2, hidden=1024, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=7168, vocab=3000,
                    rope_theta=500000.0)
# hidden 4096: the QKV tiles split too (the parts pass on their sums of squares for the RMSNorm)
WIDE_Q = ModelShape(n_layers=2, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=4608, vocab=3000,
                    rope_theta=500000.0)
SPLIT_K = [
    (WIDE_Q, 8, 5, 16, dict(qkv_ksplit=2)),
    (WIDE_Q, 16, 3, 12, dict(qkv_tiles=16, qkv_ksplit=2, wo_ksplit=1, rotate=3)),
    (WIDE_K, 8, 9, 24, dict(wo_ksplit=2, down_ksplit=4)),
    (WIDE, 16, 5, 20, dict(down_tiles=200, down_ksplit=2, rotate=7)),
    # the fp64 GEMV (batch <= 4): parts of whole 8-element chunks; at batch 4 the plain rule splits
    # WIDE's down-projection in two (5632 fp64 activations of 4 sequences exceed 128 KB)
    (WIDE, 4, 9, 16, {}),
    (WIDE_K, 2, 9, 16, dict(wo_ksplit=2, down_ksplit=8, down_tiles=200)),
]


@pytest.mark.parametrize("shape,batch,prompt,steps,sched", SPLIT_K)
def test_split_k_matches_oracle(shape, batch, prompt, steps, sched):
    say(f"split-K batch={batch} hidden={shape.hidden} ffn={shape.ffn} {sched}")
    w, s, (toks, logits) = run_prompt_case(shape, batch, prompt, steps, schedule=sched)
    check_against_oracle(shape, w, s, toks, logits, steps, f"split-K b{batch}", n_threads=16)


@pytest.mark.parametrize("shape,batch,sched", [(WIDE_K, 8, dict(wo_ksplit=2, down_ksplit=4)),
                                                (WIDE_K, 4, dict(wo_ksplit=2, down_ksplit=4)),
                                                (WIDE_Q, 8, dict(qkv_ksplit=2))])
def test_split_k_per_op_and_resumed_decode_are_bit_identical(shape, batch, sched):
    say(f"split-K: megakernel vs per-operator launches vs decode in three calls, batch={batch} "
        f"hidden={shape.hidden} {sched}")
    weights = synth.make_weights(shape, seed=5, device="cuda")
    seqs = synth.make_sequences(shape, batch, 7, 0, seed=5)
    res = []
    for mode, chunks in ((mk.MK_MODE_MEGAKERNEL, [12]), (mk.MK_MODE_PER_OP, [12]), (mk.MK_MODE_MEGAKERNEL, [1, 4, 7])):
        eng = mk.Engine(shape, batch=batch, max_seq=6 + 12, mode=mode, schedule=sched)
        eng.load_weights(weights)
        eng.prefill(seqs["prompts"].numpy())
        out = [eng.decode(n) for n in chunks]
        torch.cuda.synchronize()
        res.append((np.concatenate([t.cpu().numpy() for t, _ in out]),
                    np.concatenate([lg.cpu().numpy() for _, lg in out])))
        eng.close()
    for t, lg in res[1:]:
        assert np.array_equal(t, res[0][0])
        assert np.array_equal(lg.view(np.uint32), res[0][1].view(np.uint32))


@pytest.mark.parametrize("batch,shape", [(1, TINY), (4, TINY), (16, WIDE)])
def test_argmax_ties_go_to_the_lowest_index(batch, shape):
    # Two LM-head rows made identical and dominant: their logits are equal and the largest, so the
    # greedy token must be the lower row at every step, for every sequence.  The two rows sit in
    # different LM tiles (the tie crosses the per-tile partial maxima).
    say(f"argmax tie-break batch={batch}")
    weights = synth.make_weights(shape, seed=3, device="cuda")
    V = shape.vocab
    lo_row, hi_row = 5, V - 7
    named = dict(weights)
    lm = named["lm_head"].clone()
    lm[hi_row] = lm[lo_row] = (lm[lo_row].float() * 50.0).to(torch.bfloat16)
    weights = [(n, lm if n == "lm_head" else t) for n, t in weights]
    seqs = synth.make_sequences(shape, batch, 9, 0, seed=3)
    eng = mk.Engine(shape, batch=batch, max_seq=8 + 6)
    try:
        eng.load_weights(weights)
        eng.prefill(seqs["prompts"].numpy())
        toks, logits = eng.decode(6)
        torch.cuda.synchronize()
        toks, logits = toks.cpu().numpy(), logits.cpu().numpy()
    finally:
        eng.close()
    if batch < 8:  # one fp64 sum per row: identical rows give identical bits
        assert np.array_equal(logits[..., lo_row].view(np.uint32), logits[..., hi_row].view(np.uint32))
    top = logits.max(axis=-1)
    tied = (logits[..., lo_row] == top) & (logits[..., hi_row] == top)
    assert tied.any(), "the planted rows never held the maximum"
    assert np.all(toks[tied] == lo_row)
