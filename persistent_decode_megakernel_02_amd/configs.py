"""Model shapes and decode workloads.

Each entry is a Llama-style decoder shape plus the decode run it is measured
on.  The 8B shape matches LLaMA-3-8B and the 7B MHA shape with QK-Norm matches
Chameleon-7B, the two models the Mirage article (iaiol.com, end-to-end latency
paragraph) times at batch 1 and 4K context; the 39-token prompt / 512-token
greedy decode is the workload of the MPK digest (fr.news.hada.io, "Valeur clé
de MPK").  Weights are random (no trained checkpoint is used anywhere).
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    qk_norm: bool = False
    lora_rank: int = 0  # > 0: a LoRA adapter of this rank on every projection of every layer


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int
    prompt_len: int      # > 0: prompt prefilled through mk_prefill
    kv_prefill: int      # > 0: KV cache pre-filled with N(0,1) bf16 values
    n_steps: int         # greedy decode steps
    seed: int = 0

    @property
    def start_pos(self) -> int:
        # prompt of P tokens: P-1 positions are prefilled, the last prompt
        # token is consumed by decode step 0 at position P-1.
        return self.prompt_len - 1 if self.prompt_len > 0 else self.kv_prefill

    @property
    def max_seq(self) -> int:
        return self.start_pos + self.n_steps


TINY = ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688, vocab=1024,
                  rope_theta=10000.0)
LLAMA8B = ModelShape(n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                     vocab=128256, rope_theta=500000.0)
LLAMA8B_LORA16 = replace(LLAMA8B, lora_rank=16)
CHAMELEON7B = ModelShape(n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=32, head_dim=128, ffn=11008,
                         vocab=65536, rope_theta=10000.0, qk_norm=True)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, batch=1, prompt_len=39, kv_prefill=0, n_steps=32),
    "llama8b_decode512": Workload("llama8b_decode512", LLAMA8B, batch=1, prompt_len=39, kv_prefill=0, n_steps=512),
    "llama8b_ctx4096": Workload("llama8b_ctx4096", LLAMA8B, batch=1, prompt_len=0, kv_prefill=4096, n_steps=128),
    "llama8b_b1_ctx1024": Workload("llama8b_b1_ctx1024", LLAMA8B, batch=1, prompt_len=0, kv_prefill=1024, n_steps=64),
    "llama8b_b4_ctx1024": Workload("llama8b_b4_ctx1024", LLAMA8B, batch=4, prompt_len=0, kv_prefill=1024, n_steps=64),
    "llama8b_b8_ctx1024": Workload("llama8b_b8_ctx1024", LLAMA8B, batch=8, prompt_len=0, kv_prefill=1024, n_steps=64),
    "llama8b_b16_ctx1024": Workload("llama8b_b16_ctx1024", LLAMA8B, batch=16, prompt_len=0, kv_prefill=1024, n_steps=64),
    "chameleon7b_ctx4096": Workload("chameleon7b_ctx4096", CHAMELEON7B, batch=1, prompt_len=0, kv_prefill=4096,
                                    n_steps=128),
    # the decode512 workload with a rank-16 LoRA adapter on every projection (Mirage article, "Case 2")
    "llama8b_lora16_decode512": Workload("llama8b_lora16_decode512", LLAMA8B_LORA16, batch=1, prompt_len=39,
                                         kv_prefill=0, n_steps=512),
}


def small_variant(w: Workload, **kw) -> Workload:
    return replace(w, **kw)


def weight_bytes(m: ModelShape) -> int:
    """bf16 bytes of every weight read in one decode step (one embedding row), adapters included."""
    H, D = m.hidden, m.head_dim
    per_layer = ((m.n_q_heads + 2 * m.n_kv_heads) * D * H + H * m.n_q_heads * D + 3 * m.ffn * H) * 2
    if m.lora_rank:  # A [r][in] and B [out][r] of q, k, v, o, gate, up, down
        QD, KD, F = m.n_q_heads * D, m.n_kv_heads * D, m.ffn
        ins = 3 * H + QD + 2 * H + F
        outs = QD + 2 * KD + H + 2 * F + H
        per_layer += m.lora_rank * (ins + outs) * 2
    norms = (2 * H + (2 * D if m.qk_norm else 0)) * 2
    return m.n_layers * (per_layer + norms) + (m.vocab * H + H + H) * 2


def kv_bytes_per_step(m: ModelShape, n_attended: int) -> int:
    """bf16 K and V bytes one sequence reads (n_attended positions) plus writes (one position)."""
    row = m.n_kv_heads * m.head_dim * 2 * 2  # K and V, bf16
    return m.n_layers * row * (n_attended + 1)
