"""Per-operator anatomy of one traced decode step.

The persistent kernel can stamp, for one decode step, four device wall-clock times per task of
every worker (mk_set_trace): task start, event seen, input staged (GEMV) or partial stored
(attention), task end.  This tool runs a workload, traces one step and reports per operator,
averaged over the middle layers, with times in microseconds measured from the producers' last
end (the end of the previous operator instance's last task):

    phase        last end of this operator instance
    det_first    first worker to see its event
    det_last     last worker to see its event
    late         workers that started the task after the producers' last end
    late_seen    for those, event seen minus task start (the detection round trip)
    stage        median, event seen to input staged (GEMV)
    work         median, event seen to task end
    crit_*       the worker that ends the operator last: start, seen, staged, end
    spread       median and 90th percentile of (producers' last end - each producer's end)

    python -m persistent_decode_megakernel_02_amd.trace_anatomy --workload llama8b_decode512 \\
        --steps 300 --step 250                                   # on the GPU
"""
from __future__ import annotations

import argparse

import numpy as np

NAMES = {1: "QKV", 2: "ATT", 3: "WO", 4: "GU", 5: "DN", 6: "LM"}


def trace_step(wname: str, steps: int, step: int):
    import torch

    from . import binding as mk
    from . import synth
    from .configs import WORKLOADS
    from .schedule_search import parse_graph

    w = WORKLOADS[wname]
    torch.cuda.set_device(0)
    weights = synth.make_weights(w.model, seed=w.seed, device="cuda")
    seqs = synth.make_sequences(w.model, w.batch, w.prompt_len, w.kv_prefill, seed=w.seed, device="cuda")
    eng = mk.Engine(w.model, batch=w.batch, max_seq=w.start_pos + steps)
    try:
        eng.load_weights(weights)

        def restore():
            if w.prompt_len > 0:
                eng.prefill(seqs["prompts"].cpu().numpy())
            else:
                for b in range(w.batch):
                    eng.load_kv(b, seqs["k"][b], seqs["v"][b], int(seqs["pending"][b]))

        toks = torch.empty((steps, w.batch), dtype=torch.int32, device="cuda")
        logits = torch.empty((steps, w.batch, w.model.vocab), dtype=torch.float32, device="cuda")
        restore()
        mk.mk_decode(eng.ctx, steps, toks, logits)
        restore()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mk.mk_decode(eng.ctx, steps, toks, logits)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        mk.mk_set_trace(eng.ctx, step)
        restore()
        mk.mk_decode(eng.ctx, steps, toks, logits)
        torch.cuda.synchronize()
        tr, khz = mk.mk_get_trace(eng.ctx)
        graph = parse_graph(mk.mk_get_graph(eng.ctx))
    finally:
        eng.close()
    return ms, tr, khz, graph


def anatomy(tr, khz, g):
    """Per-operator means over layers 2 .. L-3 of the quantities in the module docstring."""
    us = 1000.0 / khz
    inst = {}
    for wk in range(tr.shape[0]):
        for i, t in enumerate(g["lists"][wk]):
            r = tr[wk, i]
            if int(r[3]) == 0:
                continue
            op, layer = g["op"][t], g["layer"][t]
            key = (layer, op) if op != 6 else (g["L"], 6)
            inst.setdefault(key, []).append([float(x) for x in r])
    order = sorted(inst, key=lambda k: max(x[3] for x in inst[k]))
    rows, prev = {}, None
    for k in order:
        a = np.array(inst[k])
        last = a[:, 3].max()
        if prev is not None and 2 <= k[0] < g["L"] - 2 and k[1] in NAMES:
            P = prev
            start, seen, staged, end = a[:, 0], a[:, 1], a[:, 2], a[:, 3]
            ok = seen > 0
            crit = int(np.argmax(end))
            late = (start > P) & ok
            gemv = k[1] != 2
            spread = (last - end) * us
            rows.setdefault(NAMES[k[1]], []).append({
                "phase": (last - P) * us,
                "det_first": (seen[ok].min() - P) * us,
                "det_last": (seen[ok].max() - P) * us,
                "late": float(late.sum()),
                "late_seen": float(np.median((seen[late] - start[late]) * us)) if late.any() else 0.0,
                "stage": float(np.median((staged[ok] - seen[ok]) * us)) if gemv else 0.0,
                "work": float(np.median((end[ok] - seen[ok]) * us)),
                "crit_start": (start[crit] - P) * us, "crit_seen": (seen[crit] - P) * us,
                "crit_staged": (staged[crit] - P) * us if gemv else 0.0, "crit_end": (end[crit] - P) * us,
                "spread_p50": float(np.percentile(spread, 50)), "spread_p90": float(np.percentile(spread, 90)),
            })
        prev = last
    return {n: {q: float(np.mean([r[q] for r in v])) for q in v[0]} for n, v in rows.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama8b_decode512")
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--step", type=int, default=250, help="the traced decode step")
    a = ap.parse_args()
    ms, tr, khz, g = trace_step(a.workload, a.steps, a.step)
    print(f"{a.workload}: {ms:.4f} ms/token; step {a.step} traced")
    res = anatomy(tr, khz, g)
    cols = ["phase", "det_first", "det_last", "late", "late_seen", "stage", "work",
            "crit_start", "crit_seen", "crit_staged", "crit_end", "spread_p50", "spread_p90"]
    print("op   " + " ".join(f"{c:>11s}" for c in cols))
    for n in ["QKV", "ATT", "WO", "GU", "DN"]:
        if n in res:
            print(f"{n:4s} " + " ".join(f"{res[n][c]:11.2f}" for c in cols))


if __name__ == "__main__":
    main()
