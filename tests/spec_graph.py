"""Independent specification of the task-graph lowering, for the bit-exact test.

Re-derives, from the written rules alone, the canonical bytes that the C++
builder (libmk.so: mk_build_graph) emits.  Shares no code with it.

Rules (one decode step; the persistent kernel repeats it every step):
  * Operators per layer, in topological order: QKV, ATTN, WO, GU, DOWN; then LM.
  * GEMV tiling by output units; tile i of T over R units covers
    [floor(i R / T), floor((i+1) R / T)).  T = min(workers, R) for WO (R = H),
    GU (R = F row pairs), DOWN (R = H) and LM (R = V).  QKV is tiled inside each
    KV-head group of RG = (G + 2) D fused rows with TG = min(max(1, workers // Hkv), RG)
    tiles per group; group g's rows start at g * RG.
  * ATTN: one task per (split s, sequence b, KV head g), split-major, split s
    covering positions [s S, (s + 1) S), S from the default rule unless given, NS = ceil(max_seq / S).
    Default rule: S = min(Smax, max(32, ceil(max_seq / (workers // (B Hkv))))); when Smax caps it and
    the resulting tasks come to at most 3 per worker, S = max(32, ceil(max_seq / ns)) with ns the
    largest split count that keeps that per-worker count (and at least ceil(max_seq / Smax)).
  * Task number k of an operator runs on worker k mod workers.
  * Events per layer: Hkv QKV-group events, ATT, O, A, X; then one LM event.
    Fan-ins: TG, F_att, T_wo, T_gu, T_down, T_lm.  Slots are numbered
    consecutively in event order.  The attention tasks are "distributed" when
    NS*B*Hkv <= workers (each on a worker of its own); then F_att = NS*B*Hkv,
    else F_att = B*Hkv.
  * Waits: QKV(0) waits LM of the previous step (lag 1); QKV(l>0) waits X(l-1);
    ATTN waits its group's QKV event; WO waits ATT; GU waits O; DOWN waits A;
    LM waits X(L-1).  Signals: QKV tile i of group g -> QKV(l, g) slot i;
    ATTN task k = (s, b, g) -> ATT slot k when distributed (every split merges a slice
    and notifies; splits beyond the current length notify at once), else slot b*Hkv+g
    (only the split holding the current position merges and notifies);
    GEMV tile i -> its event, slot i.
"""
from __future__ import annotations

import struct
from dataclasses import dataclass

OP_QKV, OP_ATTN, OP_WO, OP_GU, OP_DOWN, OP_LM = 1, 2, 3, 4, 5, 6
EV_NONE = 0xFFFFFFFF


@dataclass
class Task:
    op: int
    layer: int
    tile: int
    a0: int
    a1: int
    wait_ev: int
    wait_lag: int
    sig_ev: int
    sig_slot: int
    worker: int


def spec_graph(L, H, Hq, Hkv, D, F, V, B, max_seq, workers, split=0):
    G = Hq // Hkv
    if split > 0:
        S = split
    else:  # splits of a full cache fill the workers once; 32 <= S <= Smax = 5 * 4096 / D (8 * 4096 / D when G = 1)
        per = max(1, B * Hkv)
        ns_target = max(1, workers // per)
        smax = (8 if G == 1 else 5) * 4096 // D
        S = min(smax, max(32, -(-max_seq // ns_target)))
        ns_min = -(-max_seq // smax)
        if ns_min > ns_target:  # capped: at most 3 tasks per worker -> as many splits as keep that count
            per_worker = -(-(ns_min * per) // workers)
            if per_worker <= 3:
                S = max(32, -(-max_seq // max(ns_min, per_worker * workers // per)))
    NS = -(-max_seq // S)
    RG = (G + 2) * D
    TG = min(max(1, workers // Hkv), RG)
    n_wo, n_gu, n_down, n_lm = min(workers, H), min(workers, F), min(workers, H), min(workers, V)
    per_layer = Hkv + 4
    dist = NS * B * Hkv <= workers

    def ev(layer, k):
        return layer * per_layer + k

    ev_lm = L * per_layer
    fanin = []
    for _ in range(L):
        fanin += [TG] * Hkv + [NS * B * Hkv if dist else B * Hkv, n_wo, n_gu, n_down]
    fanin.append(n_lm)

    def lo(i, R, T):
        return i * R // T

    tasks: list[Task] = []
    for layer in range(L):
        in_ev, lag = (ev_lm, 1) if layer == 0 else (ev(layer - 1, Hkv + 3), 0)
        for g in range(Hkv):
            for i in range(TG):
                t = g * TG + i
                tasks.append(Task(OP_QKV, layer, t, g * RG + lo(i, RG, TG), g * RG + lo(i + 1, RG, TG),
                                  in_ev, lag, ev(layer, g), i, t % workers))
        k = 0
        for s in range(NS):
            for b in range(B):
                for g in range(Hkv):
                    tasks.append(Task(OP_ATTN, layer, k, b * Hkv + g, s, ev(layer, g), 0, ev(layer, Hkv),
                                      k if dist else b * Hkv + g, k % workers))
                    k += 1
        for op, R, T, wait, sig in ((OP_WO, H, n_wo, Hkv, Hkv + 1), (OP_GU, F, n_gu, Hkv + 1, Hkv + 2),
                                    (OP_DOWN, H, n_down, Hkv + 2, Hkv + 3)):
            for i in range(T):
                tasks.append(Task(op, layer, i, lo(i, R, T), lo(i + 1, R, T), ev(layer, wait), 0, ev(layer, sig), i,
                                  i % workers))
    for i in range(n_lm):
        tasks.append(Task(OP_LM, 0, i, lo(i, V, n_lm), lo(i + 1, V, n_lm), ev(L - 1, Hkv + 3), 0, ev_lm, i,
                          i % workers))
    return {"split": S, "n_splits": NS, "fanin": fanin, "tasks": tasks}


def canonical_bytes(g, workers) -> bytes:
    fanin, tasks = g["fanin"], g["tasks"]
    slot0, acc = [], 0
    for f in fanin:
        slot0.append(acc)
        acc += f
    words = [0x31474B4D, 1, workers, g["split"], g["n_splits"], len(fanin), len(tasks), acc]
    for i, f in enumerate(fanin):
        words += [i, f, slot0[i]]
    for i, t in enumerate(tasks):
        wf = 0 if t.wait_ev == EV_NONE else fanin[t.wait_ev]
        words += [i, t.op, t.layer, t.tile, t.a0, t.a1, t.wait_ev, wf, t.wait_lag, t.sig_ev, t.sig_slot, t.worker]
    return struct.pack(f"<{len(words)}I", *words)
