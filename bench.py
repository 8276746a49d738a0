"""Benchmark: greedy decode of the Llama-3-8B-shaped decoder at batch 1.

Workload (the MPK digest's decode benchmark, fr.news.hada.io, "Valeur clé de
MPK"): a 39-token prompt, then 512 greedy decode steps, no speculative
decoding, on random bf16 weights of the 8B shape.  A "step" is one decode
step of the whole model (one token).  The timed region is ONE mk_decode
call, i.e. one persistent-kernel launch covering --steps steps, with the
prompt already prefilled and every input resident in HBM.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode ms/token (8B-shape, bs=1) + achieved HBM GB/s vs ~8 TB/s peak"
PEAK_GBS = 8000.0  # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(shape, batch, start_pos, n_steps):
    """Weights streamed once per step plus, per sequence, K/V of every attended position read and one written."""
    from persistent_decode_megakernel_02_amd.configs import kv_bytes_per_step, weight_bytes
    w = weight_bytes(shape) * n_steps
    kv = sum(kv_bytes_per_step(shape, start_pos + i + 1) for i in range(n_steps)) * batch
    return w + kv


def measured_traffic(workload, n_steps):
    """HBM bytes per launch from the committed counter summary, or None.

    The summary holds FETCH_SIZE + WRITE_SIZE of the persistent kernel per decode step, scaled by what the
    same counters read for the library's known-volume probes.  It counts only while the kernel source is the
    one it was taken on (sha256 prefix recorded beside the numbers); otherwise the figure is stale."""
    import hashlib
    f = os.path.join(ROOT, "profiles", f"mk_persistent_{workload}_hbm_traffic.json")
    src = os.path.join(ROOT, "persistent_decode_megakernel_02_amd", "csrc", "kernels.hip")
    if not os.path.exists(f):
        return None
    rec = json.load(open(f))
    if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != rec["kernel_sha256_prefix"]:
        return None
    return rec["traffic_bytes_per_step"] * n_steps


def host_info():
    """Core count, CPU model and RAM of the host the oracle runs on."""
    model, ram_gb = None, None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram_gb = round(int(line.split()[1]) / 2**20, 1)
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model, "host_ram_GiB": ram_gb}


def cpu_baseline(shape, host_weights, tokens, n_threads, budget_s=20.0, max_steps=8):
    """The oracle as it stands, on the full model of the workload, timed on this host.

    It decodes the workload's first tokens from an empty cache: one untimed step, then up to max_steps
    timed steps or about budget_s seconds, whichever comes first.  Attention over these few positions is a
    negligible share of a step at this shape (the weight matrices dominate), so the per-step time stands
    for the workload's steps.  Returns (ms per step, steps timed)."""
    from tests.parity import oracle_for

    orc = oracle_for(shape, host_weights, max_seq=max_steps + 1, n_seq=1, n_threads=n_threads)
    try:
        orc.step(0, int(tokens[0]))
        t0 = time.perf_counter()
        n = 0
        while n < max_steps and (time.perf_counter() - t0) < budget_s:
            orc.step(0, int(tokens[(n + 1) % len(tokens)]))
            n += 1
        dt = time.perf_counter() - t0
    finally:
        orc.close()
    return dt / n * 1000.0, n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="llama8b_decode512")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill timing")
    ap.add_argument("--split", type=int, default=0)
    ap.add_argument("--probe-gib", type=float, default=8.0, help="read-probe buffer (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding is a design, not a measured path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from persistent_decode_megakernel_02_amd import binding as mk
    from persistent_decode_megakernel_02_amd import synth
    from persistent_decode_megakernel_02_amd.configs import WORKLOADS

    w = WORKLOADS[args.workload]
    shape, B = w.model, w.batch
    K, W = args.steps, args.warmup
    max_seq = w.start_pos + max(K, W)
    torch.cuda.set_device(0)
    log(f"workload {w.name}: generating weights on cuda:0")
    weights = synth.make_weights(shape, seed=w.seed, device="cuda")
    seqs = synth.make_sequences(shape, B, w.prompt_len, w.kv_prefill, seed=w.seed, device="cuda")
    host_weights = None
    eng = None
    toks = logits = mega_toks = mega_logits = None
    out = None
    # Every device object is released on every path before the interpreter exits: the context is
    # destroyed (mk_destroy synchronises its stream and frees its memory) in the finally clause, not by
    # a finaliser during interpreter shutdown.
    try:
        # prompts are prefilled through the megakernel (one launch per sequence; untimed)
        eng = mk.Engine(shape, batch=B, max_seq=max_seq, split=args.split, prefill=mk.MK_PREFILL_MEGAKERNEL)
        eng.load_weights(weights)
        if not args.no_cpu:
            log("copying weights to host for the CPU baseline")
            host_weights = [(n, t.cpu()) for n, t in weights]
        del weights
        torch.cuda.empty_cache()

        def restore():
            if w.prompt_len > 0:
                eng.prefill(seqs["prompts"].cpu().numpy())
            else:
                for b in range(B):
                    eng.load_kv(b, seqs["k"][b], seqs["v"][b], int(seqs["pending"][b]))

        toks = torch.empty((max(K, W), B), dtype=torch.int32, device="cuda")
        logits = torch.empty((max(K, W), B, shape.vocab), dtype=torch.float32, device="cuda")

        def timed(mode, n):
            """HIP events on torch's current stream, which is the stream the library launches on."""
            eng.set_mode(mode)
            restore()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record()
            mk.mk_decode(eng.ctx, n, toks, logits)
            e1.record()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) * 1000.0
            return e0.elapsed_time(e1), eng.last_ms(), wall

        log(f"warmup: {W} steps (megakernel)")
        if W > 0:
            timed(mk.MK_MODE_MEGAKERNEL, W)
        log(f"timed: {K} steps in one persistent launch")
        ms_torch, ms_kernel, ms_wall = timed(mk.MK_MODE_MEGAKERNEL, K)
        first_tokens = toks[: min(K, 8), 0].cpu().tolist()
        mega_toks, mega_logits = toks[:K].clone(), logits[:K].clone()
        ms_per_step = ms_torch / K
        nbytes = algorithmic_bytes(shape, B, w.start_pos, K)
        # value and the roofline fraction come from the same timer (HIP events around the launch)
        achieved = nbytes / (ms_torch * 1e-3) / 1e9
        roofline_ms = nbytes / K / (PEAK_GBS * 1e9) * 1e3
        log(f"megakernel: {ms_per_step:.4f} ms/token ({ms_torch:.2f} ms events on the launch stream, "
            f"{ms_kernel:.2f} ms library events, {ms_wall:.2f} ms wall), {achieved:.1f} GB/s, "
            f"roofline {roofline_ms:.4f} ms/token, first tokens {first_tokens}")

        ablation, identical = None, None
        if not args.no_ablation:
            log(f"ablation: {K} steps, one launch per operator")
            a_torch, a_kernel, _ = timed(mk.MK_MODE_PER_OP, K)
            ablation = a_torch / K
            identical = bool(torch.equal(mega_toks, toks[:K]) and
                             torch.equal(mega_logits.view(torch.int32), logits[:K].view(torch.int32)))
            log(f"per-operator: {ablation:.4f} ms/token; bit-identical to the megakernel: {identical}")
            eng.set_mode(mk.MK_MODE_MEGAKERNEL)
        prompt_tokens = (seqs["prompts"][0].cpu().tolist() if w.prompt_len > 0 else first_tokens)

        prefill = None
        if w.prompt_len > 0 and not args.no_prefill:
            # prefill of the workload's prompt, per operator and through the megakernel (wall time of the
            # synchronous call, median of 3), and of a longer prompt that fits the context
            def time_prefill(mode, prompts):
                eng.set_prefill(mode)
                ts = []
                for _ in range(3):
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    eng.prefill(prompts)
                    ts.append((time.perf_counter() - t0) * 1000.0)
                return sorted(ts)[1]
            host_prompts = seqs["prompts"].cpu().numpy()
            long_len = min(max_seq, 513)
            long_prompts = np.random.default_rng(1).integers(0, shape.vocab, (B, long_len)).astype(np.int32)
            prefill = {}
            for name, pr in (("prompt", host_prompts), ("long", long_prompts)):
                ms_op = time_prefill(mk.MK_PREFILL_PER_OP, pr)
                ms_mk = time_prefill(mk.MK_PREFILL_MEGAKERNEL, pr)
                prefill[name] = {"positions": int(pr.shape[1] - 1), "per_op_ms": round(ms_op, 2),
                                 "megakernel_ms": round(ms_mk, 2)}
                log(f"prefill of {pr.shape[1] - 1} positions: per operator {ms_op:.2f} ms, megakernel {ms_mk:.2f} ms")
            eng.set_prefill(mk.MK_PREFILL_MEGAKERNEL)
        eng.close()
        eng = None
        del toks, logits, mega_toks, mega_logits, seqs
        toks = logits = mega_toks = mega_logits = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

        probe = None
        if args.probe_gib > 0:
            nb = int(args.probe_gib * (1 << 30))
            probe = {"read_GBps": round(mk.mk_read_bandwidth(nb, 3), 1),
                     "copy_GBps": round(mk.mk_copy_bandwidth(nb, 3), 1), "bytes": nb}
            log(f"plain read probe: {probe['read_GBps']} GB/s, copy probe: {probe['copy_GBps']} GB/s")

        cpu = None
        if host_weights is not None:
            info = host_info()
            threads = max(1, min(16, info["nproc"] or 1))
            log(f"CPU baseline: oracle, {threads} threads, full {w.name} model ({info['cpu_model']}, "
                f"nproc {info['nproc']})")
            ms_cpu, n_cpu = cpu_baseline(shape, host_weights, prompt_tokens, threads)
            host_weights = None
            cpu = {"value": round(ms_cpu, 1), "unit": "ms/token", "cores": threads, "kind": "oracle",
                   "sample": f"{n_cpu} decode steps of the full {w.name} model (batch 1, all {shape.n_layers} "
                             f"layers and the LM head) after one untimed step, from an empty cache; "
                             f"{threads} threads splitting each matrix's rows",
                   **info}
            log(f"CPU oracle: {ms_cpu:.1f} ms/token over {n_cpu} steps")

        traffic = measured_traffic(w.name, K)
        out = {
            "metric": METRIC,
            "value": round(ms_per_step, 5),
            "unit": "ms/token",
            "n_gpus": 1,
            "steps": K,
            "warmup": W,
            "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": False,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f64",
            "data": "synthetic",
            "config": {"workload": w.name, "batch": B, "prompt_tokens": w.prompt_len, "kv_prefill": w.kv_prefill,
                       "decode_steps": K, "weights": "bf16 N(0,0.02) seeded", "kv_cache": "bf16",
                       "activations": "f32 stored, f64 evaluation", "mode": "persistent megakernel, one launch"},
            "tokens_per_s": round(B * 1000.0 / ms_per_step, 2),
            "kernel_ms_library_events": round(ms_kernel, 3),
            "ablation_per_op_ms_per_step": round(ablation, 5) if ablation else None,
            "prefill_ms": prefill,
            "ablation_bit_identical": identical,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                         "roofline_ms_per_step": round(roofline_ms, 5), "algorithmic_bytes_per_launch": nbytes},
            "cpu_baseline": cpu,
            "stream_probe": probe,
            "frac_of_measured_read_peak": round(achieved / probe["read_GBps"], 4) if probe else None,
        }
    finally:
        if eng is not None:
            eng.close()
        del toks, logits, mega_toks, mega_logits
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
