"""Seeded synthetic inputs shared by the GPU path, the oracle and the benchmark.

This module holds no arithmetic of the decoder: it only draws random weights,
prompts and pre-filled KV caches with torch's seeded generators, so that both
sides of every parity check read the very same arrays.

* Weights: N(0, 0.02) drawn in fp32 and rounded to bf16; every RMSNorm gamma
  is 1.  One generator seeded with `seed` draws the tensors in canonical order.
  LoRA adapters (shapes with lora_rank > 0) follow the base tensors, per layer
  lora_a then lora_b of q, k, v, o, gate, up, down, drawn the same way (both
  non-zero, so that the adapters change every projection).
* Prompts, pending tokens and pre-filled K/V: a second generator seeded with
  `seed + 1`, drawn per sequence in the order prompt, then per layer K then V,
  then the pending token.  Pre-filled K/V are N(0, 1) rounded to bf16 and
  stand for already-rotated keys.
Draws depend on the device the generator runs on (CPU and GPU streams
differ); a parity check always hands one set of arrays to both sides.
"""
from __future__ import annotations

import torch

from .configs import ModelShape


def canonical_names(m: ModelShape) -> list[str]:
    names = ["embed"]
    for layer in range(m.n_layers):
        p = f"layers.{layer}."
        names += [p + "attn_norm", p + "wq", p + "wk", p + "wv", p + "wo"]
        if m.qk_norm:
            names += [p + "q_norm", p + "k_norm"]
        names += [p + "ffn_norm", p + "w_gate", p + "w_up", p + "w_down"]
    names += ["final_norm", "lm_head"]
    if getattr(m, "lora_rank", 0) > 0:
        for layer in range(m.n_layers):
            for t in LORA_TARGETS:
                names += [f"layers.{layer}.lora_a.{t}", f"layers.{layer}.lora_b.{t}"]
    return names


LORA_TARGETS = ("q", "k", "v", "o", "gate", "up", "down")


def canonical_shape(m: ModelShape, name: str) -> tuple[int, ...]:
    H, D, F, V = m.hidden, m.head_dim, m.ffn, m.vocab
    QD, KD = m.n_q_heads * D, m.n_kv_heads * D
    parts = name.split(".")
    if len(parts) == 4 and parts[2] in ("lora_a", "lora_b"):
        fan_in, fan_out = {"q": (H, QD), "k": (H, KD), "v": (H, KD), "o": (QD, H), "gate": (H, F), "up": (H, F),
                           "down": (F, H)}[parts[3]]
        return (m.lora_rank, fan_in) if parts[2] == "lora_a" else (fan_out, m.lora_rank)
    base = parts[-1]
    return {
        "embed": (V, H), "lm_head": (V, H), "final_norm": (H,),
        "attn_norm": (H,), "ffn_norm": (H,), "q_norm": (D,), "k_norm": (D,),
        "wq": (QD, H), "wk": (KD, H), "wv": (KD, H), "wo": (H, QD),
        "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
    }[base]


def make_weights(m: ModelShape, seed: int = 0, device: str | torch.device = "cpu") -> list[tuple[str, torch.Tensor]]:
    """Canonical-order list of (name, bf16 tensor) on `device`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for name in canonical_names(m):
        shape = canonical_shape(m, name)
        if name.endswith("norm"):
            t = torch.ones(shape, dtype=torch.bfloat16, device=device)
        else:
            t = (torch.randn(shape, generator=g, dtype=torch.float32, device=device) * 0.02).to(torch.bfloat16)
        out.append((name, t))
    return out


def make_sequences(m: ModelShape, batch: int, prompt_len: int, kv_prefill: int, seed: int = 0,
                   device: str | torch.device = "cpu") -> dict:
    """Per-sequence prompt ids, or pre-filled K/V with a pending token.

    Returns {"prompts": int32 [B, P] or None,
             "k": bf16 [B, L, n_pos, Hkv*D] or None, "v": same, "pending": int32 [B] or None}.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed + 1)
    KD = m.n_kv_heads * m.head_dim
    prompts, ks, vs, pend = [], [], [], []
    for _ in range(batch):
        if prompt_len > 0:
            prompts.append(torch.randint(0, m.vocab, (prompt_len,), generator=g, device=device, dtype=torch.int64))
        if kv_prefill > 0:
            k = torch.empty((m.n_layers, kv_prefill, KD), dtype=torch.bfloat16, device=device)
            v = torch.empty_like(k)
            for layer in range(m.n_layers):
                k[layer] = torch.randn((kv_prefill, KD), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
                v[layer] = torch.randn((kv_prefill, KD), generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
            ks.append(k)
            vs.append(v)
            pend.append(torch.randint(0, m.vocab, (1,), generator=g, device=device, dtype=torch.int64))
    return {
        "prompts": torch.stack(prompts).to(torch.int32) if prompts else None,
        "k": torch.stack(ks) if ks else None,
        "v": torch.stack(vs) if vs else None,
        "pending": torch.cat(pend).to(torch.int32) if pend else None,
    }


def bf16_bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 tensor's bit patterns (host copy)."""
    import numpy as np
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
