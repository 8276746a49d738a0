"""Pins of the CPU oracle to facts outside itself.

Closed forms, invariants, special cases that reduce to a library routine,
and a float64 brute-force (non-cached, causal-mask) forward of whole tiny
decoders.  All CPU; none of these touches the GPU path.
"""
import math

import numpy as np
import pytest
import torch

from oracle import pyoracle as po
from persistent_decode_megakernel_02_amd import synth
from persistent_decode_megakernel_02_amd.configs import TINY, ModelShape
from tests.refmodel import bf16_bits_to_f64, forward_logits

U = 2.0 ** -53  # unit roundoff of the oracle's fp64 evaluation


def bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- bf16
def test_bf16_round_to_nearest_even_closed_forms():
    assert po.f32_to_bf16(1.0) == 0x3F80
    assert po.f32_to_bf16(1.0 + 2 ** -8) == 0x3F80          # tie -> even (down)
    assert po.f32_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert po.f32_to_bf16(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81
    assert po.f32_to_bf16(-2.0) == 0xC000
    assert po.bf16_to_f32(0x3FC0) == 1.5


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ours = np.array([po.f32_to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(ours, bits(x))


# ---------------------------------------------------------------- matvec
@pytest.mark.parametrize("rows,cols", [(7, 256), (37, 688), (64, 1000)])
def test_matvec_brute_force_within_higham_bound(rows, cols):
    rng = np.random.default_rng(rows * cols)
    W16 = bits(rng.standard_normal((rows, cols)) * 0.02)
    x = rng.standard_normal(cols)
    y = po.matvec(W16, x)
    W = bf16_bits_to_f64(W16)
    # exact in rational arithmetic would be best; fp64 BLAS is itself within the same bound
    exact = W @ x
    bound = 2 * (cols + 1) * U / (1 - (cols + 1) * U) * (np.abs(W) @ np.abs(x))
    assert np.all(np.abs(y - exact) <= bound * 1.0001)
    # every fp32 rounding of the result agrees with the rounding of the exact sum except at a
    # rounding boundary, which random data does not hit
    assert np.array_equal(y.astype(np.float32), exact.astype(np.float32))
    # row r of the output depends on row r of W only (no transposition)
    W16b = W16.copy()
    W16b[3] = bits(np.zeros(cols))
    y2 = po.matvec(W16b, x)
    assert y2[3] == 0.0 and np.array_equal(np.delete(y2, 3), np.delete(y, 3))


def test_matvec_is_the_sequential_fp64_sum_of_each_row():
    # every row is summed k = 0, 1, ... in fp64 with each product and each sum rounded once, whatever
    # the compiler's vectorisation across rows (rows 0-7 go in blocks of four, row 8 alone)
    rng = np.random.default_rng(11)
    rows, cols = 9, 300
    W16 = bits(rng.standard_normal((rows, cols)) * 0.02)
    x = rng.standard_normal(cols)
    W = bf16_bits_to_f64(W16)
    want = []
    for r in range(rows):
        acc = 0.0
        for k in range(cols):
            acc = acc + float(W[r, k]) * float(x[k])
        want.append(acc)
    assert np.array_equal(po.matvec(W16, x), np.array(want))


def test_matvec_threads_bit_identical():
    rng = np.random.default_rng(5)
    W16 = bits(rng.standard_normal((300, 512)) * 0.02)
    x = rng.standard_normal(512)
    assert np.array_equal(po.matvec(W16, x, 1), po.matvec(W16, x, 4))


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector_is_gamma():
    n, eps = 256, 1e-5
    ones = bits(np.ones(n))
    y = po.rmsnorm(np.ones(n, np.float32), ones, eps)
    e32 = float(np.float32(eps))  # eps is carried as an fp32 value
    assert np.allclose(y, 1.0 / math.sqrt(1.0 + e32), rtol=1e-15, atol=0)
    assert np.all(np.abs(y - 1.0) <= 5.1e-6)
    c = 3.0
    y = po.rmsnorm(np.full(n, c, np.float32), ones, eps)
    assert np.allclose(y, c / math.sqrt(c * c + e32), rtol=1e-15)


def test_rmsnorm_random_gamma_against_float64():
    rng = np.random.default_rng(2)
    n, eps = 4096, 1e-5
    x = rng.standard_normal(n).astype(np.float32)
    g16 = bits(rng.uniform(0.5, 1.5, n))
    y = po.rmsnorm(x, g16, eps)
    xd = x.astype(np.float64)
    ref = xd / np.sqrt(np.mean(xd * xd) + float(np.float32(eps))) * bf16_bits_to_f64(g16)
    assert np.allclose(y, ref, rtol=1e-13, atol=0)
    # scale invariance up to eps (|alpha x| >> eps): rmsnorm(8 x) = 8 x / sqrt(64 mean(x^2) + eps)
    y2 = po.rmsnorm((x * 8.0).astype(np.float32), g16, eps)
    assert np.allclose(y, y2, rtol=1e-5, atol=0)
    ref2 = 8 * xd / np.sqrt(64 * np.mean(xd * xd) + float(np.float32(eps))) * bf16_bits_to_f64(g16)
    assert np.allclose(y2, ref2, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- RoPE
def test_rope_identity_at_position_zero():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(128)
    assert np.array_equal(po.rope(x, 0, 500000.0), x)


def test_rope_pairing_and_frequency_closed_form():
    # d=4, theta=100: pair 1 is (1, 3) with frequency 100^(-1/2) = 0.1; at position 10 the angle is 1 rad
    y = po.rope(np.array([0, 1, 0, 0], np.float64), 10, 100.0)
    assert np.allclose(y, [0, math.cos(1.0), 0, math.sin(1.0)], atol=1e-15)
    # pair 0 is (0, 2) with frequency 1; at position 1 the angle is 1 rad
    y = po.rope(np.array([1, 0, 0, 0], np.float64), 1, 100.0)
    assert np.allclose(y, [math.cos(1.0), 0, math.sin(1.0), 0], atol=1e-15)
    y = po.rope(np.array([0, 0, 1, 0], np.float64), 1, 100.0)
    assert np.allclose(y, [-math.sin(1.0), 0, math.cos(1.0), 0], atol=1e-15)


def test_rope_preserves_pair_norms_and_relative_positions():
    rng = np.random.default_rng(4)
    d, theta = 128, 500000.0
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    for p in (1, 17, 4095):
        r = po.rope(q, p, theta)
        half = d // 2
        assert np.allclose(r[:half] ** 2 + r[half:] ** 2, q[:half] ** 2 + q[half:] ** 2, rtol=1e-13)
    a = float(np.dot(po.rope(q, 100, theta), po.rope(k, 37, theta)))
    b = float(np.dot(po.rope(q, 1100, theta), po.rope(k, 1037, theta)))
    assert abs(a - b) <= 1e-11 * (np.abs(q) @ np.abs(k))


# ---------------------------------------------------------------- attention
def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(6)
    d = 64
    K = bits(rng.standard_normal((1, d)))
    V = bits(rng.standard_normal((1, d)))
    o = po.attend(rng.standard_normal(d), K, V)
    assert np.array_equal(o, bf16_bits_to_f64(V[0]).astype(np.float32))


def test_attention_weights_are_softmax_of_scaled_scores_and_sum_to_one():
    rng = np.random.default_rng(7)
    n, d = 40, 64
    K16 = bits(rng.standard_normal((n, d)))
    V16 = bits(np.eye(n, d))        # one-hot values expose the softmax weights
    q = rng.standard_normal(d) * 0.5
    w = po.attend(q, K16, V16)[:n]
    assert abs(float(np.sum(w.astype(np.float64))) - 1.0) < 1e-6
    s = bf16_bits_to_f64(K16) @ q / math.sqrt(d)
    ref = torch.softmax(torch.from_numpy(s), dim=0).numpy()
    # the weights are fp64 values rounded once to fp32
    assert np.array_equal(w, ref.astype(np.float32))


def test_attention_zero_query_is_mean_of_values():
    rng = np.random.default_rng(8)
    n, d = 33, 128
    K16 = bits(rng.standard_normal((n, d)))
    V16 = bits(rng.standard_normal((n, d)))
    o = po.attend(np.zeros(d), K16, V16)
    assert np.array_equal(o, bf16_bits_to_f64(V16).mean(axis=0).astype(np.float32))


def test_attention_shift_invariance():
    rng = np.random.default_rng(9)
    n, d = 20, 64
    K = rng.standard_normal((n, d))
    K[:, 5] = 0.0
    K16 = bits(K)
    V16 = bits(rng.standard_normal((n, d)))
    q = rng.standard_normal(d)
    # adding the same vector c to every key adds q.c to every score, which the softmax ignores
    c = np.zeros(d)
    c[5] = 4.0
    K2 = bits(bf16_bits_to_f64(K16) + c)
    assert np.array_equal(bf16_bits_to_f64(K2), bf16_bits_to_f64(K16) + c)
    o1, o2 = po.attend(q, K16, V16), po.attend(q, K2, V16)
    assert np.allclose(o1, o2, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- SiLU / argmax
def test_silu_closed_forms():
    assert po.silu(0.0) == 0.0
    assert abs(po.silu(40.0) - 40.0) < 1e-14
    assert abs(po.silu(-40.0)) < 1e-15
    assert abs(po.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    for z in np.linspace(-8, 8, 33):
        assert abs(po.silu(float(z)) - z / (1 + math.exp(-z))) <= 1e-15 * max(1.0, abs(z))


def test_argmax_lowest_index_on_ties():
    assert po.argmax(np.array([1, 3, 2, 3], np.float32)) == 1
    assert po.argmax(np.array([-5, -5], np.float32)) == 0
    assert po.argmax(np.array([0, 0, 7], np.float32)) == 2


# ---------------------------------------------------------------- whole decoder
def _weights(shape, seed, gamma_random=True):
    ws = synth.make_weights(shape, seed=seed, device="cpu")
    rng = np.random.default_rng(seed + 100)
    out16, out64 = [], {}
    for name, t in ws:
        a = synth.bf16_bits(t)
        if name.endswith("norm") and gamma_random:
            a = bits(rng.uniform(0.6, 1.4, a.shape))   # non-unit gammas so a dropped gamma shows
        out16.append(a)
        out64[name] = bf16_bits_to_f64(a)
    return out16, out64


SHAPES = {
    "tiny_gqa": TINY,
    "tiny_mha_qknorm": ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=688,
                                  vocab=512, qk_norm=True),
    "tiny_g4": ModelShape(n_layers=1, hidden=128, n_q_heads=8, n_kv_heads=2, head_dim=32, ffn=200, vocab=300,
                          rope_theta=500000.0),
    "tiny_lora": ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688, vocab=512,
                            lora_rank=8),
    "tiny_lora_qknorm": ModelShape(n_layers=1, hidden=128, n_q_heads=4, n_kv_heads=4, head_dim=32, ffn=200,
                                   vocab=300, qk_norm=True, lora_rank=16),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_cached_decode_equals_float64_causal_forward(name):
    shape = SHAPES[name]
    w16, w64 = _weights(shape, seed=11)
    # scale up weights so that attention is far from uniform and errors would show
    rng = np.random.default_rng(12)
    tokens = rng.integers(0, shape.vocab, 12)
    orc = po.Oracle(shape, w16, max_seq=16)
    got = np.stack([orc.step(0, int(t)) for t in tokens])
    # same fp32 storage points: the two can differ only where an fp64 value sits within fp64 rounding of an
    # fp32 rounding boundary, which these inputs do not hit -- so the logits are bit-identical
    ref32 = forward_logits(shape, w64, tokens, store32=True)
    assert np.array_equal(got, ref32), np.abs(got - ref32).max()
    # and the plain float64 decoder, with no fp32 storage at all
    ref = forward_logits(shape, w64, tokens)
    assert np.abs(got - ref).max() <= 1e-4 * max(1.0, np.abs(ref).max())
    assert orc.pos() == len(tokens)


def test_cached_decode_with_prefilled_kv_equals_float64_forward():
    shape = SHAPES["tiny_gqa"]
    w16, w64 = _weights(shape, seed=13)
    rng = np.random.default_rng(14)
    P, KD = 9, shape.n_kv_heads * shape.head_dim
    k16 = bits(rng.standard_normal((shape.n_layers, P, KD)))
    v16 = bits(rng.standard_normal((shape.n_layers, P, KD)))
    tokens = rng.integers(0, shape.vocab, 5)
    orc = po.Oracle(shape, w16, max_seq=P + 5)
    orc.set_kv(0, k16, v16)
    got = np.stack([orc.step(0, int(t)) for t in tokens])
    pre = (bf16_bits_to_f64(k16), bf16_bits_to_f64(v16))
    ref32 = forward_logits(shape, w64, tokens, kv_prefix=pre, store32=True)
    assert np.array_equal(got, ref32), np.abs(got - ref32).max()
    ref = forward_logits(shape, w64, tokens, kv_prefix=pre)
    assert np.abs(got - ref).max() <= 1e-4 * max(1.0, np.abs(ref).max())


def test_zero_residual_branches_reduce_to_embedding_readout():
    # Wo = Wd = 0: every layer leaves x unchanged, so logits = W_lm . rmsnorm(E[tok]) . gamma_f
    shape = SHAPES["tiny_gqa"]
    w16, w64 = _weights(shape, seed=15)
    names = synth.canonical_names(shape)
    for i, n in enumerate(names):
        if n.endswith(".wo") or n.endswith(".w_down"):
            w16[i] = np.zeros_like(w16[i])
    orc = po.Oracle(shape, w16, max_seq=4)
    for tok in (3, 700, 1023):
        logits = orc.step(0, tok)
        e = w64["embed"][tok]
        h = e / np.sqrt(np.mean(e * e) + float(np.float32(shape.rms_eps))) * w64["final_norm"]
        ref = w64["lm_head"] @ h
        assert np.array_equal(logits, ref.astype(np.float32))
        assert po.argmax(logits) == int(np.argmax(ref))


def test_cache_capacity_and_token_range_errors():
    shape = SHAPES["tiny_g4"]
    w16, _ = _weights(shape, seed=16, gamma_random=False)
    orc = po.Oracle(shape, w16, max_seq=2)
    orc.step(0, 1, want_logits=False)
    with pytest.raises(ValueError):
        orc.step(0, shape.vocab)
    orc.step(0, 2, want_logits=False)
    with pytest.raises(ValueError):
        orc.step(0, 3)


# ---------------------------------------------------------------- LoRA + Linear
# Mirage article, "Case 2: LoRA + Linear": W x + B A x = (W|B)(x|A x).
def _lora_operands(rows, cols, r, seed):
    rng = np.random.default_rng(seed)
    W = bits(rng.standard_normal((rows, cols)) * 0.05)
    A = bits(rng.standard_normal((r, cols)) * 0.05)
    B = bits(rng.standard_normal((rows, r)) * 0.05)
    x = rng.standard_normal(cols)
    return W, A, B, x


@pytest.mark.parametrize("rows,cols,r", [(7, 300, 1), (33, 129, 8), (64, 512, 16)])
def test_lora_linear_is_the_concatenated_product(rows, cols, r):
    # the article's identity, with the concatenations made explicit: the plain (pinned) matvec of
    # [W | B] against [x | A x], A x materialised in fp32, gives the same bits
    W, A, B, x = _lora_operands(rows, cols, r, seed=rows + cols)
    u = po.matvec(A, x).astype(np.float32).astype(np.float64)
    ref = po.matvec(np.concatenate([W, B], axis=1), np.concatenate([x, u]))
    got = po.lora_linear(W, A, B, x)
    assert np.array_equal(got, ref)


def test_lora_linear_with_a_zero_adapter_is_the_plain_linear():
    W, A, B, x = _lora_operands(40, 256, 8, seed=3)
    plain = po.matvec(W, x)
    assert np.array_equal(po.lora_linear(W, A, np.zeros_like(B), x), plain)
    assert np.array_equal(po.lora_linear(W, np.zeros_like(A), B, x), plain)
    assert np.array_equal(po.lora_linear(W, None, None, x), plain)


def test_lora_linear_within_float64_bound_of_the_merged_weight():
    # (W + B A) x in float64 with A x exact: differs from the oracle only by the fp32 rounding of A x
    # (|u| 2^-24 relative, carried through B) and fp64 summation error
    W, A, B, x = _lora_operands(50, 400, 16, seed=5)
    Wf, Af, Bf = (bf16_bits_to_f64(a) for a in (W, A, B))
    ref = (Wf + Bf @ Af) @ x
    u = Af @ x
    bound = np.abs(Bf) @ (np.abs(u) * 2.0 ** -24) + 1e-12 * (np.abs(Wf) @ np.abs(x) + np.abs(Bf) @ np.abs(u))
    got = po.lora_linear(W, A, B, x)
    assert np.all(np.abs(got - ref) <= bound)
    assert np.abs(got - po.matvec(W, x)).max() > 1e-3   # the adapter is not a no-op here


def test_lora_decoder_with_zero_b_equals_the_base_decoder():
    # B = 0 on every adapter: the LoRA decoder's logits are bit-identical to the base model's
    shape = SHAPES["tiny_lora"]
    base = ModelShape(**{**shape.__dict__, "lora_rank": 0})
    w16, _ = _weights(shape, seed=17)
    names = synth.canonical_names(shape)
    for i, n in enumerate(names):
        if ".lora_b." in n:
            w16[i] = np.zeros_like(w16[i])
    n_base = len(synth.canonical_names(base))
    tokens = np.random.default_rng(18).integers(0, shape.vocab, 6)
    a, b = po.Oracle(shape, w16, max_seq=8), po.Oracle(base, w16[:n_base], max_seq=8)
    for t in tokens:
        assert np.array_equal(a.step(0, int(t)), b.step(0, int(t)))
