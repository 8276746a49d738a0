"""Float64 non-cached causal forward of the decoder, written in matrix form.

Used only to pin the CPU oracle: the oracle decodes token by token through a
bf16 KV cache; this reference recomputes every prefix from scratch with a
causal mask in float64, rounding K (after RoPE) and V to bf16 exactly where a
cache would hold them.  With store32=True it also rounds to fp32 where the
decoder stores an activation (raw q/k/v, rotated k, attention output,
residual stream after each sublayer, SwiGLU output, logits); with
store32=False everything else stays float64.  It shares no code with the
oracle.
"""
import numpy as np
import torch


def bf16_round(a: np.ndarray) -> np.ndarray:
    # torch's float32 -> bfloat16 cast rounds to nearest even
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope_rows(x, positions, theta):
    # x [..., T, D]; rotate-half pairing (i, i + D/2), freq theta^(-2i/D)
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def forward_logits(shape, w: dict, tokens, kv_prefix=None, store32=False):
    """Logits [T, V] for every position of `tokens` (all positions causal).

    w maps canonical names to float64 arrays.  kv_prefix optionally gives
    pre-filled (K, V) as float64 [L, P, Hkv*D] occupying positions 0..P-1.
    """
    st = f32 if store32 else (lambda a: a)
    H, D, Hq, Hkv = shape.hidden, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    G = Hq // Hkv
    eps = float(np.float32(shape.rms_eps))  # the decoder carries eps as an fp32 value
    T = len(tokens)
    P = 0 if kv_prefix is None else kv_prefix[0].shape[1]
    pos = np.arange(P, P + T)
    x = w["embed"][np.asarray(tokens)]
    lora = getattr(shape, "lora_rank", 0) > 0
    for layer in range(shape.n_layers):
        p = f"layers.{layer}."

        def lin(h, wname, t):
            # a linear layer, plus its LoRA update B (A h) with A h materialised (fp32 under store32)
            y = h @ w[p + wname].T
            if lora:
                y = y + st(h @ w[p + "lora_a." + t].T) @ w[p + "lora_b." + t].T
            return y

        h = rms(x, w[p + "attn_norm"], eps)
        q = st(lin(h, "wq", "q")).reshape(T, Hq, D).transpose(1, 0, 2)
        k = st(lin(h, "wk", "k")).reshape(T, Hkv, D).transpose(1, 0, 2)
        v = st(lin(h, "wv", "v")).reshape(T, Hkv, D).transpose(1, 0, 2)
        if shape.qk_norm:
            q = rms(q, w[p + "q_norm"], eps)
            k = rms(k, w[p + "k_norm"], eps)
        q = rope_rows(q, pos, shape.rope_theta)
        k = bf16_round(st(rope_rows(k, pos, shape.rope_theta)))
        v = bf16_round(v)
        if P:
            kp = kv_prefix[0][layer].reshape(P, Hkv, D).transpose(1, 0, 2)
            vp = kv_prefix[1][layer].reshape(P, Hkv, D).transpose(1, 0, 2)
            k = np.concatenate([kp, k], axis=1)
            v = np.concatenate([vp, v], axis=1)
        o = np.zeros((Hq, T, D))
        allpos = np.arange(P + T)
        mask = allpos[None, :] > pos[:, None]
        for hh in range(Hq):
            g = hh // G
            s = q[hh] @ k[g].T / np.sqrt(D)
            s = np.where(mask, -np.inf, s)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            o[hh] = st((e @ v[g]) / e.sum(axis=1, keepdims=True))
        x = st(x + lin(o.transpose(1, 0, 2).reshape(T, Hq * D), "wo", "o"))
        h2 = rms(x, w[p + "ffn_norm"], eps)
        gt = lin(h2, "w_gate", "gate")
        up = lin(h2, "w_up", "up")
        x = st(x + lin(st(gt / (1.0 + np.exp(-gt)) * up), "w_down", "down"))
    return st(rms(x, w["final_norm"], eps) @ w["lm_head"].T)
