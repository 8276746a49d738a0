"""Offline schedule search for the task graph.

Ada-MK (gist.science, "L'Itinéraire Pré-planifié") searches the schedule of its megakernel
offline, measures the candidates on the target GPU and then fixes the winner, so that nothing is
decided while the kernel runs.  This module does that for the graph builder's schedule
(csrc/graph.cpp): the attention split, the tile count of every GEMV operator, and where each
operator's tasks sit on the workers (a rotation per operator, an offset for the attention tasks).

A candidate is scored by the persistent kernel's own time on the workload (HIP events around one
mk_decode launch, median of several launches).  Each candidate must decode bit-identical tokens
and logits to the plain schedule: tiling and placement move work between workers but never
change how a row or an attention split is computed.  For the plain schedule and the winner it
also records the per-operator phase times from the kernel's trace (mk_set_trace), which is what
shows where a schedule gains or loses.

The search is coordinate descent from the plain schedule: for each field in turn, every listed
value is tried with the others at their current best, and a change is kept only if it is faster
by more than the noise margin.  Two sweeps.  The winner is then timed against the plain schedule
in interleaved pairs, and frozen only if it wins every pair.

    python -m persistent_decode_megakernel_02_amd.schedule_search --workload llama8b_decode512 \\
        --out results.json              # on the GPU
    python -m persistent_decode_megakernel_02_amd.schedule_search --freeze results.json [...]
                                        # writes csrc/schedule_table.inc from result files
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "schedule_table.inc")


def log(msg):
    print(f"[search] {msg}", file=sys.stderr, flush=True)


def candidates(shape, batch, workers, plain_split):
    """Values tried per field (0 = the plain rule)."""
    G = shape.n_q_heads // shape.n_kv_heads
    rg = (G + 2) * shape.head_dim
    tg = min(max(1, workers // shape.n_kv_heads), rg)
    splits = sorted({max(16, int(round(plain_split * f))) for f in (0.5, 0.75, 1.0, 1.25, 1.5, 2.0)})
    smax = (8 if G == 1 else 5) * 4096 // shape.head_dim
    splits = [s for s in splits if s <= smax]
    frac = lambda fs: sorted({max(1, int(workers * f)) for f in fs}, reverse=True)  # noqa: E731
    # split-K of WO / DOWN (matrix-core GEMV, batch >= 8): 2, 4, 8 parts up to the K slices of 2048
    ks = lambda k: [1] + [p for p in (2, 4, 8) if batch >= 8 and p <= -(-k // 2048)]  # noqa: E731
    return {
        "wo_ksplit": ks(shape.n_q_heads * shape.head_dim),
        "down_ksplit": ks(shape.ffn),
        "qkv_ksplit": ks(shape.hidden),
        "split": splits,
        "rotate": [0, 1, 2, 4, 8, 16, 32, 64, 128],
        "attn_offset": [0, 16, 64, 128, 192],
        "qkv_tiles": sorted({tg, max(1, tg * 3 // 4), max(1, tg // 2)}, reverse=True),
        "wo_tiles": frac((1.0, 0.9375, 0.875, 0.75, 0.5)),
        "gu_tiles": frac((1.0, 0.96875, 0.9375, 0.875)),
        "down_tiles": frac((1.0, 0.96875, 0.9375, 0.875)),
        "lm_tiles": frac((1.0, 0.875, 0.75, 0.5)),
    }


class Bench:
    """One workload on the GPU: weights and inputs made once, one context per candidate."""

    def __init__(self, wname, steps, warmup, reps):
        import torch

        from . import binding as mk
        from . import synth
        from .configs import WORKLOADS

        self.torch, self.mk = torch, mk
        self.w = w = WORKLOADS[wname]
        self.steps, self.warmup, self.reps = steps, warmup, reps
        self.max_seq = w.start_pos + max(steps, warmup)
        torch.cuda.set_device(0)
        log(f"{w.name}: generating weights")
        self.weights = synth.make_weights(w.model, seed=w.seed, device="cuda")
        self.seqs = synth.make_sequences(w.model, w.batch, w.prompt_len, w.kv_prefill, seed=w.seed, device="cuda")
        self.toks = torch.empty((max(steps, warmup), w.batch), dtype=torch.int32, device="cuda")
        self.logits = torch.empty((max(steps, warmup), w.batch, w.model.vocab), dtype=torch.float32, device="cuda")
        self.ref = None

    def _restore(self, eng):
        w = self.w
        if w.prompt_len > 0:
            eng.prefill(self.seqs["prompts"].cpu().numpy())
        else:
            for b in range(w.batch):
                eng.load_kv(b, self.seqs["k"][b], self.seqs["v"][b], int(self.seqs["pending"][b]))

    def run(self, split, sched, trace=False):
        """Median ms/token over reps launches; checks bit-identity with the first candidate run."""
        torch, mk, w = self.torch, self.mk, self.w
        eng = mk.Engine(w.model, batch=w.batch, max_seq=self.max_seq, split=split, schedule=sched)
        try:
            eng.load_weights(self.weights)
            times = []
            for r in range(self.reps + 1):
                self._restore(eng)
                n = self.warmup if r == 0 else self.steps
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                mk.mk_decode(eng.ctx, n, self.toks, self.logits)
                e1.record()
                torch.cuda.synchronize()
                if r > 0:
                    times.append(e0.elapsed_time(e1) / n)
            out = (self.toks[: self.steps].clone(), self.logits[: self.steps].clone())
            if self.ref is None:
                self.ref = {}
                self.first = out
            # tiling and placement change no bit; the attention split and split-K regroup sums (the
            # part counts as built, read back from the graph: 0 in a field takes the plain rule)
            graph = mk.mk_get_graph(eng.ctx)
            key = (split, graph_ksplits(graph))
            ref = self.ref.get(key)
            if ref is not None:  # same sums: tiling and placement must not change a single bit
                if not (torch.equal(out[0], ref[0]) and torch.equal(out[1].view(torch.int32), ref[1].view(torch.int32))):
                    raise RuntimeError(f"schedule {sched} split {split}: results differ from the same split's")
            else:  # other groupings of the same sums: same tokens, close logits
                d = (out[1] - self.first[1]).abs().max().item()
                if not torch.equal(out[0], self.first[0]) or d > 1e-3:
                    log(f"split {split}: tokens differ or max |d logit| {d} > 1e-3 (a near-tie): not a candidate")
                    times = [math.inf]
                self.ref[key] = out
            phases = self._phases(eng) if trace else None
        finally:
            eng.close()
        return statistics.median(times), times, phases, graph

    def _phases(self, eng):
        """Per-operator phase times (us) of one traced step: last end of an operator instance minus
        the last end of the one before it, averaged over layers."""
        import numpy as np

        mk = self.mk
        step = self.steps // 2
        mk.mk_set_trace(eng.ctx, step)
        self._restore(eng)
        mk.mk_decode(eng.ctx, self.steps, self.toks, self.logits)
        self.torch.cuda.synchronize()
        tr, khz = mk.mk_get_trace(eng.ctx)
        nw = tr.shape[0]
        mk.mk_set_trace(eng.ctx, -1)
        g = parse_graph(mk.mk_get_graph(eng.ctx))
        ends = {}
        lists = g["lists"]
        for wkr in range(nw):
            for i, t in enumerate(lists[wkr]):
                e = int(tr[wkr, i, 3])
                if e == 0:
                    continue
                op, layer = g["op"][t], g["layer"][t]
                key = (layer, op) if op != 6 else (g["L"], 6)
                ends[key] = max(ends.get(key, 0), e)
        order = sorted(ends, key=lambda k: ends[k])
        names = {1: "QKV", 2: "ATT", 3: "WO", 4: "GU", 5: "DN", 6: "LM"}
        acc = {}
        prev = None
        for k in order:
            if prev is not None:
                acc.setdefault(names[k[1]], []).append((ends[k] - ends[prev]) * 1000.0 / khz)
            prev = k
        return {n: round(float(np.mean(v)), 2) for n, v in acc.items()}


def parse_graph(raw: bytes):
    import struct

    w = struct.unpack(f"<{len(raw) // 4}I", raw)
    nw, nev, nt = w[2], w[5], w[6]
    base = 8 + 3 * nev
    op, layer, worker = [], [], []
    for i in range(nt):
        r = w[base + 17 * i: base + 17 * (i + 1)]
        op.append(r[1])
        layer.append(r[2])
        worker.append(r[11])
    lists = [[] for _ in range(nw)]
    for i in range(nt):
        lists[worker[i]].append(i)
    return {"op": op, "layer": layer, "lists": lists, "L": max(layer) + 1}


def graph_ksplits(raw: bytes):
    """Split-K part count of each operator (QKV, WO, DN) in a serialised graph."""
    import struct

    w = struct.unpack(f"<{len(raw) // 4}I", raw)
    nev, nt = w[5], w[6]
    base = 8 + 3 * nev
    ks = {}
    for i in range(nt):
        r = w[base + 17 * i: base + 17 * (i + 1)]
        ks[r[1]] = max(ks.get(r[1], 1), r[16])
    return tuple(ks.get(op, 1) for op in (1, 3, 5))


def plain_split(shape, batch, max_seq, workers):
    """The split the plain rule gives (read back from the built graph's header)."""
    import struct

    from . import binding as mk

    raw = mk.mk_build_graph(mk.make_cfg(shape, batch=batch, max_seq=max_seq, schedule={}), workers)
    return struct.unpack("<8I", raw[:32])[3]


def search(args):
    import torch

    from . import binding as mk

    b = Bench(args.workload, args.steps, args.warmup, args.reps)
    w = b.w
    workers = torch.cuda.get_device_properties(0).multi_processor_count
    s0 = plain_split(w.model, w.batch, b.max_seq, workers)
    space = candidates(w.model, w.batch, workers, s0)
    log(f"{w.name}: {workers} workers, plain split {s0}; space {space}")
    best = {"split": s0, **{k: 0 for k in space if k != "split"}}

    def sched_of(cfg):
        return {k: v for k, v in cfg.items() if k != "split"}

    t_plain, times, ph_plain, _ = b.run(s0, sched_of(best), trace=True)
    log(f"plain: {t_plain:.4f} ms/token {times} phases {ph_plain}")
    evals = [{"cfg": dict(best), "ms": t_plain, "times": times}]
    noise = max(args.margin, (max(times) - min(times)) / t_plain)
    t_best = t_plain
    for sweep in range(args.sweeps):
        for field, values in space.items():
            for v in values:
                cfg = dict(best)
                cfg[field] = v
                if any(e["cfg"] == cfg for e in evals):
                    continue
                try:
                    t, times, _, _ = b.run(cfg["split"], sched_of(cfg))
                except mk.MkError as e:  # e.g. a split-K that does not divide the tile count
                    log(f"sweep {sweep} {field}={v}: rejected ({e})")
                    continue
                evals.append({"cfg": cfg, "ms": t, "times": times})
                log(f"sweep {sweep} {field}={v}: {t:.4f} ms/token")
                if t < t_best * (1.0 - noise):
                    best, t_best = cfg, t
                    log(f"  -> new best {best} {t_best:.4f}")
    # confirm the winner against the plain schedule, interleaved
    conf = []
    for _ in range(args.confirm):
        tp, _, _, _ = b.run(s0, {k: 0 for k in space if k != "split"})
        tw, _, _, _ = b.run(best["split"], sched_of(best))
        conf.append((tp, tw))
    t_win, _, ph_win, graph = b.run(best["split"], sched_of(best), trace=True)
    res = {
        "workload": w.name, "shape": {k: getattr(w.model, k) for k in
                                      ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab")},
        "batch": w.batch, "max_seq": b.max_seq, "workers": workers, "steps": args.steps, "reps": args.reps,
        "plain": {"cfg": evals[0]["cfg"], "ms": t_plain, "phases_us": ph_plain},
        "winner": {"cfg": best, "ms": t_win, "phases_us": ph_win},
        "confirm_plain_vs_winner_ms": conf, "noise_margin": noise, "evaluations": evals,
        "device": torch.cuda.get_device_name(0), "time": time.strftime("%Y-%m-%d %H:%M:%S"),
    }
    with open(args.out, "w") as f:
        json.dump(res, f, indent=1)
    log(f"winner {best}: {t_win:.4f} ms/token (plain {t_plain:.4f}); confirm {conf}")


def measure(args):
    """Time the default (frozen) schedule with whatever library MK_LIBRARY selects."""
    b = Bench(args.workload, args.steps, args.warmup, args.reps)
    t, times, phases, _ = b.run(0, None, trace=True)
    res = {"workload": b.w.name, "library": os.environ.get("MK_LIBRARY", "libmk.so"), "ms": t, "times": times,
           "phases_us": phases}
    with open(args.out, "w") as f:
        json.dump(res, f)
    log(f"{res['library']}: {t:.4f} ms/token {times} phases {phases}")


def compare_variants(args):
    """Compile-time alternatives (build.VARIANTS, built beforehand) against the default library,
    one process each, interleaved default / variant, --confirm rounds."""
    import subprocess

    from .build import VARIANT_DIR

    names = args.variants.split(",")
    runs = {"default": []}
    for r in range(args.confirm):
        for name in names:
            for lib in ("default", name):
                env = dict(os.environ)
                env.pop("MK_LIBRARY", None)
                if lib != "default":
                    env["MK_LIBRARY"] = os.path.join(VARIANT_DIR, f"libmk_{lib}.so")
                    if not os.path.exists(env["MK_LIBRARY"]):
                        raise FileNotFoundError(env["MK_LIBRARY"] + " (build it with build.py --variants)")
                out = f"{args.out}.{lib}.{r}.json"
                cmd = [sys.executable, "-m", "persistent_decode_megakernel_02_amd.schedule_search", "--measure",
                       "--workload", args.workload, "--steps", str(args.steps), "--reps", str(args.reps),
                       "--out", out]
                subprocess.run(cmd, env=env, check=True)
                runs.setdefault(lib, []).append(json.load(open(out)))
    summary = {lib: {"ms": [x["ms"] for x in v], "phases_us": v[-1]["phases_us"]} for lib, v in runs.items()}
    with open(args.out, "w") as f:
        json.dump({"workload": args.workload, "steps": args.steps, "reps": args.reps, "runs": summary}, f, indent=1)
    for lib, v in summary.items():
        log(f"{lib}: {v['ms']}")


def seq_bucket(m):
    """The max_seq range a frozen entry covers: the power-of-two octave holding the searched max_seq."""
    lo = 1 << int(math.floor(math.log2(m)))
    return lo, 2 * lo - 1


def freeze(paths):
    """Write csrc/schedule_table.inc from search result files.  An entry is written only where the
    winner beat the plain schedule in every confirmation pair."""
    rows = []
    for p in paths:
        r = json.load(open(p))
        conf = r["confirm_plain_vs_winner_ms"]
        win = r["winner"]["cfg"]
        kept = bool(conf) and all(tw < tp for tp, tw in conf) and win != r["plain"]["cfg"]
        s = r["shape"]
        lo, hi = seq_bucket(r["max_seq"])
        gain = [round(1 - tw / tp, 4) for tp, tw in conf]
        rows.append((kept, f"    // {r['workload']}: plain {r['plain']['ms']:.4f} ms/token, winner "
                           f"{r['winner']['ms']:.4f}; paired gains {gain}" + ("" if kept else " (not kept)")))
        if kept:
            rows.append((True, "    {%d, %d, %d, %d, %d, %d, %d, %d, %d, %d, %d, {%d, %d, %d, %d, %d, %d, %d, %d, %d, %d, %d}},"
                         % (s["n_layers"], s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], s["ffn"],
                            s["vocab"], r["batch"], r["workers"], lo, hi, win["split"], win["qkv_tiles"],
                            win["wo_tiles"], win["gu_tiles"], win["down_tiles"], win["lm_tiles"], win["rotate"],
                            win["attn_offset"], win.get("wo_ksplit", 0), win.get("down_ksplit", 0),
                            win.get("qkv_ksplit", 0))))
    body = "\n".join(line for _, line in rows)
    text = f"""// schedule_table.inc -- schedules frozen by the offline search (schedule_search.py), one entry
// per (shape, batch, workers, max_seq range).  An entry overrides the plain rules of graph.cpp
// for that case; every other case keeps them.  Written by schedule_search.py --freeze from the
// search's result files; an entry is kept only where the winner beat the plain schedule in every
// interleaved confirmation pair.
struct FrozenSchedule {{
  int L, H, Hq, Hkv, D, F, V, B, workers, seq_lo, seq_hi;
  Schedule s;
}};
static const FrozenSchedule kFrozenSchedules[] = {{
    // L, H, Hq, Hkv, D, F, V, B, workers, max_seq range,
    //   {{split, qkv, wo, gu, down, lm tiles, rotate, attn_offset, wo_ksplit, down_ksplit, qkv_ksplit}}
{body}
    {{0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, {{}}}},  // end marker, matches nothing (empty max_seq range)
}};
"""
    with open(TABLE, "w") as f:
        f.write(text)
    print(text)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama8b_decode512")
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--sweeps", type=int, default=2)
    ap.add_argument("--confirm", type=int, default=5)
    ap.add_argument("--margin", type=float, default=0.001, help="smallest relative gain kept")
    ap.add_argument("--out", default="schedule_search.json")
    ap.add_argument("--freeze", nargs="*", help="result files to freeze into csrc/schedule_table.inc")
    ap.add_argument("--measure", action="store_true", help="time the default schedule only")
    ap.add_argument("--variants", default="", help="comma-separated build variants to compare with the default")
    args = ap.parse_args()
    if args.freeze:
        freeze(args.freeze)
    elif args.measure:
        measure(args)
    elif args.variants:
        compare_variants(args)
    else:
        search(args)


if __name__ == "__main__":
    main()
