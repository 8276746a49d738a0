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
  * Placement: tile i of the k-th GEMV operator of a layer (QKV 0, WO 1, GU 2, DOWN 3; the LM
    head 4) runs on worker (i + k * rotate) mod workers; attention task k on worker
    (k + attn_offset) mod workers.
  * A schedule may fix the tile counts: TG = min(qkv_tiles, RG) QKV tiles per group, and
    T = min(x_tiles, R) for the other GEMV operators (0 keeps the rules above).
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
  * LoRA (rank r > 0, a multiple of 8 up to 64): the GEMV operators QKV, WO, GU, DOWN have
    nA = 3r, r, r, r adapter A rows (units); with T tiles, q = ceil(nA / T) per tile: tile i holds
    [min(i q, nA), min((i+1) q, nA)).  One event per (layer, operator), appended after the LM event
    in layer-major order QKV, WO, GU, DOWN, with fan-in ceil(nA / q) (the holders).  Other tasks:
    la0 = la1 = 0, lora_ev = none.
  * Split-K (decode graphs of batch >= 2 without LoRA): ks = wo_ksplit (down_ksplit), 0 taking the plain rule.
    Batch >= 8: the first of 4, 2 that is at most ceil(K / 2048) and divides T, else 1.  Batch < 8:
    need = the first of 1, 2, 4 with ceil(K / p) * B * 8 <= 131072 (else 8), then the first of
    1, 2, 4, 8 at least need that divides T, else 1.  Always 1 in the prefill graph, with LoRA and at
    batch 1.
    QKV (qkv_ksplit, batch >= 8 only): 0 means none; a given 2, 4 or 8 must be at most ceil(H / 2048)
    and divide TG; the parts of a row tile lie inside one KV-head group (row tile r = i // ks of the
    group's TG tiles covers the group's rows [floor(r RG / (TG / ks)), ...)), fan-in TG / ks.
    With ks > 1 the T tasks of WO (DOWN)
    form T / ks row tiles of ks consecutive tasks; task i is part p = i mod ks of row tile r = i // ks,
    covering units [floor(r R / (T / ks)), floor((r+1) R / (T / ks))); only the last part (p = ks - 1)
    signals, slot r, so the event's fan-in is T / ks; the other parts signal none (slot 0).  Valid:
    ks in {1, 2, 4, 8}, ks | T, at batch >= 8 ks <= ceil(K / 2048) (K = Hq D for WO, F for DOWN).
  * Canonical bytes, version 3: each task row ends with la0, la1, lora_ev, kp, kn.
  * Prefill graph (chunk > 0): B = chunk virtual sequences, the given split, the plain tiling and
    placement; after each layer's QKV tasks one append task per KV-head group g (op 7, tile g,
    a0 = g, on the worker of the group's first QKV tile) waits QKV(l, g) and signals its own event
    (fan-in 1), numbered after the LM event and the LoRA events, layer-major; attention tasks wait
    on it instead of QKV(l, g); never "distributed"; no LM tasks (the LM event stays in the table);
    layer 0 waits X(L-1) of the previous step (lag 1).
"""
from __future__ import annotations

import struct
from dataclasses import dataclass

OP_QKV, OP_ATTN, OP_WO, OP_GU, OP_DOWN, OP_LM, OP_APPEND = 1, 2, 3, 4, 5, 6, 7
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
    la0: int = 0
    la1: int = 0
    lora_ev: int = EV_NONE
    kp: int = 0
    kn: int = 1


def spec_graph(L, H, Hq, Hkv, D, F, V, B, max_seq, workers, split=0, qkv_tiles=0, wo_tiles=0, gu_tiles=0,
               down_tiles=0, lm_tiles=0, rotate=0, attn_offset=0, lora_rank=0, chunk=0, wo_ksplit=0,
               down_ksplit=0, qkv_ksplit=0):
    G = Hq // Hkv
    if chunk:
        B = chunk
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
    TG = min(qkv_tiles or max(1, workers // Hkv), RG)
    n_wo, n_gu = min(wo_tiles or workers, H), min(gu_tiles or workers, F)
    n_down, n_lm = min(down_tiles or workers, H), min(lm_tiles or workers, V)
    rot, aoff = rotate % workers, attn_offset % workers
    ksplit = {OP_WO: wo_ksplit, OP_GU: 1, OP_DOWN: down_ksplit}
    splittable = not chunk and not lora_rank and B >= 2
    for op, T, K in ((OP_WO, n_wo, Hq * D), (OP_DOWN, n_down, F)):
        nsl = -(-K // 2048)
        if ksplit[op] == 0:  # the plain rule
            if not splittable:
                ksplit[op] = 1
            elif B >= 8:
                ksplit[op] = next((k for k in (4, 2) if k <= nsl and T % k == 0), 1)
            else:  # fewest parts whose fp64 staging of B sequences takes at most 128 KB
                need = next((p for p in (1, 2, 4) if -(-K // p) * B * 8 <= 131072), 8)
                ksplit[op] = next((p for p in (1, 2, 4, 8) if p >= need and T % p == 0), 1)
        ks = ksplit[op]
        if ks > 1 and (not splittable or ks not in (2, 4, 8) or T % ks or (B >= 8 and ks > nsl)):
            raise ValueError("invalid split-K")
    # QKV (batch >= 8): parts of a row tile within one KV-head group
    nslq = -(-H // 2048)
    qks = qkv_ksplit or 1  # the plain rule leaves QKV unsplit
    if qks > 1 and (not splittable or B < 8 or qks not in (2, 4, 8) or TG % qks or qks > nslq):
        raise ValueError("invalid QKV split-K")

    def place(k, i):
        return (i + k * rot) % workers
    per_layer = Hkv + 4
    dist = not chunk and NS * B * Hkv <= workers

    def ev(layer, k):
        return layer * per_layer + k

    ev_lm = L * per_layer
    fanin = []
    for _ in range(L):
        fanin += [TG // qks] * Hkv + [NS * B * Hkv if dist else B * Hkv, n_wo // ksplit[OP_WO], n_gu,
                               n_down // ksplit[OP_DOWN]]
    fanin.append(n_lm)
    # LoRA A-row events, after the LM event
    n_arows = {OP_QKV: 3 * lora_rank, OP_WO: lora_rank, OP_GU: lora_rank, OP_DOWN: lora_rank}
    tiles = {OP_QKV: TG * Hkv, OP_WO: n_wo, OP_GU: n_gu, OP_DOWN: n_down}
    q = {op: -(-n_arows[op] // tiles[op]) for op in n_arows} if lora_rank else {}
    kidx = {OP_QKV: 0, OP_WO: 1, OP_GU: 2, OP_DOWN: 3}
    if lora_rank:
        for _ in range(L):
            for op in (OP_QKV, OP_WO, OP_GU, OP_DOWN):
                fanin.append(-(-n_arows[op] // q[op]))

    ev_app0 = ev_lm + 1 + (4 * L if lora_rank else 0)
    if chunk:
        fanin += [1] * (L * Hkv)

    def lora_fields(op, layer, tile):
        if not lora_rank or op not in kidx:
            return {}
        n = n_arows[op]
        return dict(la0=min(tile * q[op], n), la1=min((tile + 1) * q[op], n),
                    lora_ev=ev_lm + 1 + 4 * layer + kidx[op])

    def lo(i, R, T):
        return i * R // T

    tasks: list[Task] = []
    for layer in range(L):
        if layer == 0:
            in_ev, lag = (ev(L - 1, Hkv + 3) if chunk else ev_lm), 1
        else:
            in_ev, lag = ev(layer - 1, Hkv + 3), 0
        for g in range(Hkv):
            for i in range(TG):
                t = g * TG + i
                r, p = divmod(i, qks)
                last = p == qks - 1
                tasks.append(Task(OP_QKV, layer, t, g * RG + lo(r, RG, TG // qks), g * RG + lo(r + 1, RG, TG // qks),
                                  in_ev, lag, ev(layer, g) if last else EV_NONE, r if last else 0, place(0, t),
                                  kp=p, kn=qks, **lora_fields(OP_QKV, layer, t)))
        if chunk:
            for g in range(Hkv):
                tasks.append(Task(OP_APPEND, layer, g, g, 0, ev(layer, g), 0, ev_app0 + layer * Hkv + g, 0,
                                  place(0, g * TG)))
        k = 0
        for s in range(NS):
            for b in range(B):
                for g in range(Hkv):
                    wait = ev_app0 + layer * Hkv + g if chunk else ev(layer, g)
                    tasks.append(Task(OP_ATTN, layer, k, b * Hkv + g, s, wait, 0, ev(layer, Hkv),
                                      k if dist else b * Hkv + g, (k + aoff) % workers))
                    k += 1
        for k, (op, R, T, wait, sig) in enumerate(((OP_WO, H, n_wo, Hkv, Hkv + 1), (OP_GU, F, n_gu, Hkv + 1, Hkv + 2),
                                                   (OP_DOWN, H, n_down, Hkv + 2, Hkv + 3)), start=1):
            ks = ksplit[op]
            for i in range(T):
                r, p = divmod(i, ks)
                last = p == ks - 1
                tasks.append(Task(op, layer, i, lo(r, R, T // ks), lo(r + 1, R, T // ks), ev(layer, wait), 0,
                                  ev(layer, sig) if last else EV_NONE, r if last else 0, place(k, i),
                                  kp=p, kn=ks, **lora_fields(op, layer, i)))
    for i in range(0 if chunk else n_lm):
        tasks.append(Task(OP_LM, 0, i, lo(i, V, n_lm), lo(i + 1, V, n_lm), ev(L - 1, Hkv + 3), 0, ev_lm, i,
                          place(4, i)))
    return {"split": S, "n_splits": NS, "fanin": fanin, "tasks": tasks}


def canonical_bytes(g, workers) -> bytes:
    fanin, tasks = g["fanin"], g["tasks"]
    slot0, acc = [], 0
    for f in fanin:
        slot0.append(acc)
        acc += f
    words = [0x31474B4D, 3, workers, g["split"], g["n_splits"], len(fanin), len(tasks), acc]
    for i, f in enumerate(fanin):
        words += [i, f, slot0[i]]
    for i, t in enumerate(tasks):
        wf = 0 if t.wait_ev == EV_NONE else fanin[t.wait_ev]
        words += [i, t.op, t.layer, t.tile, t.a0, t.a1, t.wait_ev, wf, t.wait_lag, t.sig_ev, t.sig_slot, t.worker,
                  t.la0, t.la1, t.lora_ev, t.kp, t.kn]
    return struct.pack(f"<{len(words)}I", *words)
