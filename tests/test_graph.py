"""Task-graph construction: bit-exact against an independent spec builder, plus invariants
and a randomized-interleaving simulation of the event protocol (CPU only)."""
import random
import struct
from dataclasses import replace

import pytest

from persistent_decode_megakernel_02_amd import binding as mk
from persistent_decode_megakernel_02_amd.configs import CHAMELEON7B, LLAMA8B, TINY, ModelShape
from tests.spec_graph import OP_ATTN, OP_DOWN, OP_GU, OP_LM, OP_QKV, OP_WO, canonical_bytes, spec_graph

CASES = [
    (TINY, 1, 71, 256, 0), (TINY, 1, 71, 8, 16), (TINY, 4, 50, 37, 32), (TINY, 16, 20, 256, 0),
    (LLAMA8B, 1, 550, 256, 0), (LLAMA8B, 1, 4224, 256, 128), (LLAMA8B, 16, 1088, 256, 0), (LLAMA8B, 8, 1088, 100, 64),
    (CHAMELEON7B, 1, 4224, 256, 128), (CHAMELEON7B, 2, 300, 64, 0),
    (ModelShape(3, 512, 8, 2, 128, 1000, 2000), 2, 100, 256, 32),
]


def cfg_of(shape, B, max_seq, split, schedule=None):
    return mk.make_cfg(shape, batch=B, max_seq=max_seq, split=split, schedule=schedule)


SPEC_ARGS = ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab")


def spec_bytes(shape, B, max_seq, workers, split, **sched):
    dims = [getattr(shape, a) for a in SPEC_ARGS]
    return canonical_bytes(spec_graph(*dims, B, max_seq, workers, split, lora_rank=shape.lora_rank, **sched), workers)


# LoRA: adapter A rows spread over the first tiles of every GEMV operator, one event per (layer, operator)
LORA_CASES = [
    (replace(TINY, lora_rank=8), 1, 71, 256, 0, None),
    (replace(TINY, lora_rank=64), 2, 40, 8, 16, None),       # 192 QKV A rows over 8 tiles: 24 each
    (replace(TINY, lora_rank=16), 4, 50, 37, 0, dict(qkv_tiles=3, wo_tiles=5, rotate=2)),
    (replace(LLAMA8B, lora_rank=16), 1, 550, 256, 0, None),
    (replace(LLAMA8B, lora_rank=64), 4, 1088, 256, 0, dict(gu_tiles=200, down_tiles=100)),
]


@pytest.mark.parametrize("shape,B,max_seq,workers,split,sched", LORA_CASES)
def test_lora_graph_bytes_equal_spec(shape, B, max_seq, workers, split, sched):
    got = mk.mk_build_graph(cfg_of(shape, B, max_seq, split, sched), workers)
    assert got == spec_bytes(shape, B, max_seq, workers, split, **(sched or {}))
    g = parse(got)
    n_plain = len(parse(mk.mk_build_graph(cfg_of(replace(shape, lora_rank=0), B, max_seq, split, sched),
                                          workers))["events"])
    assert len(g["events"]) == n_plain + 4 * shape.n_layers
    # every adapter row of every operator is held by exactly one tile, and the holders fill the event's slots
    for layer in range(shape.n_layers):
        for op, n_rows in ((OP_QKV, 3 * shape.lora_rank), (OP_WO, shape.lora_rank), (OP_GU, shape.lora_rank),
                           (OP_DOWN, shape.lora_rank)):
            ts = [t for t in g["tasks"] if t[1] == op and t[2] == layer]
            held = sorted(r for t in ts for r in range(t[12], t[13]))
            assert held == list(range(n_rows))
            evs = {t[14] for t in ts}
            assert len(evs) == 1
            (ev,) = evs
            holders = sorted(t[3] for t in ts if t[13] > t[12])
            assert holders == list(range(len(holders))) and g["events"][ev][1] == len(holders)
    assert all(t[14] == 0xFFFFFFFF for t in g["tasks"] if t[1] in (OP_ATTN, OP_LM))


# the megakernel prefill's graph: chunk virtual sequences, the decode graph's split, append tasks
PREFILL_CASES = [
    (TINY, 1, 71, 256, 4), (TINY, 2, 40, 37, 4), (replace(TINY, lora_rank=16), 1, 71, 8, 4),
    (LLAMA8B, 1, 550, 256, 16), (LLAMA8B, 4, 1088, 256, 16), (CHAMELEON7B, 1, 4224, 256, 16),
]


@pytest.mark.parametrize("shape,B,max_seq,workers,chunk", PREFILL_CASES)
def test_prefill_graph_bytes_equal_spec(shape, B, max_seq, workers, chunk):
    cfg = cfg_of(shape, B, max_seq, 0)
    split = struct.unpack("<8I", mk.mk_build_graph(cfg, workers)[:32])[3]  # the decode graph's
    got = mk.mk_build_prefill_graph(cfg, workers, chunk, split)
    dims = [getattr(shape, a) for a in SPEC_ARGS]
    spec = canonical_bytes(spec_graph(*dims, B, max_seq, workers, split, lora_rank=shape.lora_rank, chunk=chunk),
                           workers)
    assert got == spec
    g = parse(got)
    assert g["split"] == split
    ops = [t[1] for t in g["tasks"]]
    assert OP_LM not in ops and ops.count(7) == shape.n_layers * shape.n_kv_heads
    # per layer: QKV, then the appends, then attention
    for layer in range(shape.n_layers):
        idx = {op: [t[0] for t in g["tasks"] if t[1] == op and t[2] == layer] for op in (OP_QKV, 7, OP_ATTN)}
        assert max(idx[OP_QKV]) < min(idx[7]) and max(idx[7]) < min(idx[OP_ATTN])


def test_lora_rank_is_validated():
    for r in (4, 12, 72, -8):
        with pytest.raises(mk.MkError):
            mk.mk_build_graph(cfg_of(replace(TINY, lora_rank=r), 1, 40, 0), 256)


# schedules the offline search may give: tile counts below and at the worker count, rotations,
# attention offsets (some wrap past the worker count)
SCHEDULE_CASES = [
    (LLAMA8B, 1, 550, 256, 0, dict(rotate=1)),
    (LLAMA8B, 1, 550, 256, 0, dict(rotate=37, attn_offset=100)),
    (LLAMA8B, 1, 550, 256, 40, dict(qkv_tiles=16, wo_tiles=128, gu_tiles=200, down_tiles=255, lm_tiles=64)),
    (LLAMA8B, 4, 1088, 256, 0, dict(wo_tiles=192, rotate=64, attn_offset=300)),
    (LLAMA8B, 16, 1088, 256, 0, dict(gu_tiles=256, down_tiles=128, rotate=3, attn_offset=7)),
    (TINY, 2, 40, 37, 0, dict(qkv_tiles=5, wo_tiles=30, rotate=36, attn_offset=36)),
    (CHAMELEON7B, 1, 4224, 256, 0, dict(qkv_tiles=6, rotate=128, attn_offset=1)),
]


@pytest.mark.parametrize("shape,B,max_seq,workers,split,sched", SCHEDULE_CASES)
def test_given_schedule_bytes_equal_spec(shape, B, max_seq, workers, split, sched):
    got = mk.mk_build_graph(cfg_of(shape, B, max_seq, split, sched), workers)
    assert got == spec_bytes(shape, B, max_seq, workers, split, **sched)


def test_given_schedule_of_zeros_is_the_plain_rule():
    for shape, B, max_seq, workers, split in CASES[:6]:
        assert mk.mk_build_graph(cfg_of(shape, B, max_seq, split, {}), workers) == \
            spec_bytes(shape, B, max_seq, workers, split)


@pytest.mark.parametrize("bad", [dict(wo_tiles=257), dict(lm_tiles=-1), dict(rotate=-3), dict(qkv_tiles=33)])
def test_given_schedule_rejects_bad_fields(bad):
    with pytest.raises(mk.MkError) as e:
        mk.mk_build_graph(cfg_of(LLAMA8B, 1, 550, 0, bad), 256)
    assert e.value.code == mk.MK_ERR_INVALID_ARG or e.value.code == mk.MK_ERR_UNSUPPORTED


def parse(raw: bytes):
    w = struct.unpack(f"<{len(raw) // 4}I", raw)
    magic, ver, workers, split, ns, nev, nt, nslots = w[:8]
    ev = [w[8 + 3 * i: 11 + 3 * i] for i in range(nev)]
    base = 8 + 3 * nev
    tasks = [w[base + 17 * i: base + 17 * (i + 1)] for i in range(nt)]
    return dict(magic=magic, ver=ver, workers=workers, split=split, ns=ns, events=ev, tasks=tasks, nslots=nslots)


@pytest.mark.parametrize("shape,B,max_seq,workers,split", CASES)
def test_builder_bytes_equal_spec(shape, B, max_seq, workers, split):
    got = mk.mk_build_graph(cfg_of(shape, B, max_seq, split), workers)
    spec = canonical_bytes(spec_graph(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                                      shape.head_dim, shape.ffn, shape.vocab, B, max_seq, workers, split), workers)
    assert len(got) == len(spec)
    assert got == spec


@pytest.mark.parametrize("shape,B,max_seq,workers,split", CASES)
def test_graph_invariants(shape, B, max_seq, workers, split):
    g = parse(mk.mk_build_graph(cfg_of(shape, B, max_seq, split), workers))
    assert g["magic"] == 0x31474B4D and g["ver"] == 3
    tasks, events = g["tasks"], g["events"]
    # topological indices are consecutive; slots partition the flag array
    assert [t[0] for t in tasks] == list(range(len(tasks)))
    acc = 0
    for i, (eid, fanin, slot0) in enumerate(events):
        assert eid == i and slot0 == acc and fanin > 0
        acc += fanin
    assert acc == g["nslots"]
    # every event slot has a producer; GEMV/QKV slots exactly one
    producers = {}
    for t in tasks:
        producers.setdefault((t[9], t[10]), []).append(t)
    for e, (eid, fanin, _) in enumerate(events):
        for s in range(fanin):
            ps = producers.get((e, s), [])
            assert ps, f"event {e} slot {s} has no producer"
            if ps[0][1] != OP_ATTN:
                assert len(ps) == 1
    # waits refer to earlier producers in the same step (lag 0) or to the previous step (lag 1)
    first_index = {}
    for t in tasks:
        first_index.setdefault(t[9], t[0])
    last_index = {}
    for t in tasks:
        last_index[t[9]] = t[0]
    for t in tasks:
        if t[8] == 0:
            assert last_index[t[6]] < t[0], "wait on an event produced later in the step"
        else:
            assert t[1] == OP_QKV and t[2] == 0
        assert t[7] == events[t[6]][1]
    # each GEMV operator's tiles partition its output units (one writer per output row: with split-K
    # the last part of each row tile)
    H, F, V = shape.hidden, shape.ffn, shape.vocab
    RG = (shape.n_q_heads // shape.n_kv_heads + 2) * shape.head_dim
    for layer in range(shape.n_layers):
        for op, R in ((OP_QKV, shape.n_kv_heads * RG), (OP_WO, H), (OP_GU, F), (OP_DOWN, H)):
            rng = sorted((t[4], t[5]) for t in tasks if t[1] == op and t[2] == layer and t[15] == t[16] - 1)
            assert rng[0][0] == 0 and rng[-1][1] == R
            assert all(a[1] == b[0] for a, b in zip(rng, rng[1:])) and all(a < b for a, b in rng)
    rng = sorted((t[4], t[5]) for t in tasks if t[1] == OP_LM)
    assert rng[0][0] == 0 and rng[-1][1] == V and all(a[1] == b[0] for a, b in zip(rng, rng[1:]))
    # attention: one task per (split, sequence, KV head); splits cover max_seq
    att = [t for t in tasks if t[1] == OP_ATTN and t[2] == 0]
    assert len(att) == g["ns"] * B * shape.n_kv_heads
    assert g["ns"] == -(-max_seq // g["split"])
    # task k of an operator runs on worker k mod workers (the per-operator kernel steps by it)
    assert all(t[11] == t[3] % g["workers"] for t in tasks)
    # QKV tiles never straddle a KV-head group
    for t in tasks:
        if t[1] == OP_QKV:
            assert t[4] // RG == (t[5] - 1) // RG


def simulate(g, shape, B, steps, start_pos, seed, drop=None, early=None, violations=None):
    """Run every worker's list under random interleaving with the event rules, one flag per slot
    holding the number of steps its producer signalled; returns True if all steps complete, False
    on deadlock.  Attention splits beyond the current length do nothing.  A merging split stores
    its partial, stays on its worker until every active split of its head has stored, then
    signals; a split that does not merge stores and moves on without signalling.  The split
    holding the current position merges; with the attention tasks distributed (one slot per task)
    and more than 8 active splits, every active split merges a slice, and a wait on the attention
    event reads only the slots of the step's merging splits.

    Data check: a task's results count as written when it completes; a consumer that passes its
    wait records, in `violations`, every waited slot whose last signaller has not completed that
    step.  `early`: a task that signals before it completes (an early release), as two separate
    moves of its worker, so that consumers may run in between."""
    rnd = random.Random(seed)
    tasks, events = g["tasks"], g["events"]
    workers, S, Hkv = g["workers"], g["split"], shape.n_kv_heads
    per_layer = Hkv + 4
    dist = g["ns"] * B * Hkv <= workers
    lists = [[t for t in tasks if t[11] == w] for w in range(workers)]
    L = shape.n_layers
    kdone = {}                     # split-K (op, row tile, part) -> uses published (use u = step * L + layer)
    kread = {}                     # split-K (op, row tile) -> uses the last part has reduced
    flags = {}                     # (event, slot) -> steps signalled
    done_split = {}                # (step, layer, bg) -> active splits that stored their partial
    stored = [False] * workers     # a merging split has stored and waits for its head's others
    pos = [0] * workers            # (step * len(list) + index)
    total = [steps * len(lst) for lst in lists]
    completed = {}                 # topo index -> steps completed
    signaller = {}                 # (event, slot) -> topo index of the last task that signalled it
    released = [False] * workers   # the early-release task has signalled but not completed

    def n_active(step):
        return -(-(start_pos + step + 1) // S)

    def slots(ev, step):
        fanin = events[ev][1]
        if dist and ev < shape.n_layers * per_layer and ev % per_layer == Hkv:
            n_act = n_active(step)
            return range(n_act * B * Hkv) if n_act > 8 else range((n_act - 1) * B * Hkv, n_act * B * Hkv)
        return range(fanin)

    def merges(t, step):
        n_act = n_active(step)
        return t[5] == n_act - 1 or (dist and n_act > 8)

    def parts_ready(t, step):  # the last K part of a row tile reduces once the others have published
        kp, kn = t[15], t[16]
        if kn == 1 or kp < kn - 1:
            return True
        u = step * L + t[2]
        return all(kdone.get((t[1], t[3] // kn, p), 0) >= u + 1 for p in range(kn - 1))

    def finish(t, step):
        completed[t[0]] = step + 1
        kp, kn = t[15], t[16]
        if kn == 1:
            return
        key, u = (t[1], t[3] // kn), step * L + t[2]
        if kp < kn - 1:  # publishing overwrites the previous use's partials: it must have been reduced
            if violations is not None and kread.get(key, 0) < u:
                violations.append((t[0], "kpart", step))
            kdone[key + (kp,)] = u + 1
        else:
            kread[key] = u + 1

    while True:
        ready = []
        for w in range(workers):
            if pos[w] >= total[w]:
                continue
            step, i = divmod(pos[w], len(lists[w]))
            t = lists[w][i]
            if t[1] == OP_ATTN and t[5] >= n_active(step):
                ready.append(w)
            elif stored[w]:
                if done_split.get((step, t[2], t[4]), 0) == n_active(step):
                    ready.append(w)
            else:
                target = step + 1 - t[8]
                if (target <= 0 or all(flags.get((t[6], sl), 0) >= target for sl in slots(t[6], step - t[8]))) \
                        and parts_ready(t, step):
                    ready.append(w)
        if not ready:
            return all(pos[w] >= total[w] for w in range(workers))
        w = rnd.choice(ready)
        step, i = divmod(pos[w], len(lists[w]))
        t = lists[w][i]
        if released[w]:  # the early-release task completes now
            released[w] = False
            finish(t, step)
            pos[w] += 1
            continue
        if violations is not None and t[6] != 0xFFFFFFFF and not stored[w] and not (
                t[1] == OP_ATTN and t[5] >= n_active(step)):
            target = step + 1 - t[8]
            if target > 0:
                for sl in slots(t[6], step - t[8]):
                    src = signaller.get((t[6], sl))
                    if src is not None and completed.get(src, 0) < target:
                        violations.append((t[0], src, step))
        signal = t[9] != 0xFFFFFFFF  # a split-K part below the last signals nothing
        if t[1] == OP_ATTN:
            if t[5] >= n_active(step):
                signal = False
            elif not stored[w]:
                key = (step, t[2], t[4])
                done_split[key] = done_split.get(key, 0) + 1
                if merges(t, step):
                    stored[w] = True
                    continue
                signal = False
            else:
                stored[w] = False
        if early is not None and t[0] == early:  # signal now, complete on the worker's next move
            released[w] = True
        else:
            finish(t, step)
            pos[w] += 1
        if signal and not (drop is not None and t[0] == drop):
            assert flags.get((t[9], t[10]), 0) <= step, "slot signalled twice in a step"
            flags[(t[9], t[10])] = step + 1
            signaller[(t[9], t[10])] = t[0]


@pytest.mark.parametrize("workers,split,seed", [(8, 16, 0), (13, 8, 1), (37, 32, 2), (40, 8, 4), (20, 8, 5)])
def test_event_protocol_completes_under_random_interleavings(workers, split, seed):
    shape = ModelShape(2, 128, 4, 2, 64, 96, 100)
    g = parse(mk.mk_build_graph(cfg_of(shape, 2, 40, split), workers))
    assert simulate(g, shape, 2, steps=3, start_pos=5, seed=seed)


@pytest.mark.parametrize("steps,start_pos,seed", [(3, 12, 6), (4, 30, 7)])
def test_event_protocol_with_slice_merges(steps, start_pos, seed):
    # 2-position splits: 7 to 17 active splits per head, so both merge forms occur
    shape = ModelShape(2, 128, 4, 2, 64, 96, 100)
    g = parse(mk.mk_build_graph(cfg_of(shape, 2, 40, 2), 96))
    assert g["ns"] * 2 * shape.n_kv_heads <= 96
    assert simulate(g, shape, 2, steps=steps, start_pos=start_pos, seed=seed)


@pytest.mark.parametrize("seed", range(4))
def test_no_consumer_reads_unfinished_results_in_simulation(seed):
    shape = ModelShape(2, 128, 4, 2, 64, 96, 100)
    for workers, split in ((8, 16), (37, 8)):
        g = parse(mk.mk_build_graph(cfg_of(shape, 1, 40, split), workers))
        bad = []
        assert simulate(g, shape, 1, steps=3, start_pos=5, seed=seed, violations=bad)
        assert bad == []


def test_early_release_is_caught_in_simulation():
    # a GEMV tile that signals before its results are written: some interleaving lets a consumer
    # pass its wait in between, and the data check sees it
    shape = ModelShape(2, 128, 4, 2, 64, 96, 100)
    g = parse(mk.mk_build_graph(cfg_of(shape, 1, 40, 16), 8))
    victim = next(t[0] for t in g["tasks"] if t[1] == OP_WO and t[2] == 0)
    caught = 0
    for seed in range(20):
        bad = []
        assert simulate(g, shape, 1, steps=2, start_pos=5, seed=seed, early=victim, violations=bad)
        caught += any(src == victim for _, src, _ in bad)
    assert caught > 0


def test_dropped_signal_deadlocks_in_simulation():
    shape = ModelShape(2, 128, 4, 2, 64, 96, 100)
    g = parse(mk.mk_build_graph(cfg_of(shape, 1, 40, 16), 8))
    victim = next(t[0] for t in g["tasks"] if t[1] == OP_GU and t[2] == 1)
    assert not simulate(g, shape, 1, steps=2, start_pos=5, seed=3, drop=victim)


@pytest.mark.parametrize("bad", [dict(batch=3), dict(n_q_heads=6), dict(head_dim=96), dict(split=1000)])
def test_builder_rejects_unsupported_shapes(bad):
    base = dict(shape=TINY, B=1, max_seq=64, split=0)
    shape = TINY
    B = bad.get("batch", 1)
    if "n_q_heads" in bad:
        shape = ModelShape(2, 256, bad["n_q_heads"], 4, 64, 688, 1024)
    if "head_dim" in bad:
        shape = ModelShape(2, 256, 4, 2, bad["head_dim"], 688, 1024)
    split = bad.get("split", 0)
    del base
    with pytest.raises(mk.MkError):
        mk.mk_build_graph(cfg_of(shape, B, 64, split), 256)


# split-K of the O- and down-projection (batch >= 8): K >= 4096 for WO (Hq D) and DOWN (F)
KSHAPE = ModelShape(2, 128, 32, 8, 128, 8192, 100)
KSHAPE_Q = ModelShape(2, 4096, 32, 8, 128, 4096, 100)  # hidden 4096: QKV has two K slices
KSPLIT_CASES = [
    (KSHAPE, 8, 40, 24, 16, dict(wo_ksplit=2, down_ksplit=4)),
    (KSHAPE, 16, 40, 37, 8, dict(wo_tiles=36, down_tiles=32, wo_ksplit=2, down_ksplit=4, rotate=5)),
    (LLAMA8B, 8, 1088, 256, 0, dict(wo_ksplit=2, down_ksplit=4)),
    (LLAMA8B, 16, 1088, 256, 0, dict(down_tiles=192, down_ksplit=2, rotate=3)),
    (KSHAPE_Q, 8, 40, 32, 16, dict(qkv_ksplit=2, wo_ksplit=2, down_ksplit=2)),
    (KSHAPE_Q, 16, 40, 37, 8, dict(qkv_tiles=3, qkv_ksplit=1, down_tiles=36, down_ksplit=2)),
    (KSHAPE, 2, 40, 24, 16, dict(wo_ksplit=2, down_ksplit=8, rotate=1)),   # fp64 GEMV path
    (LLAMA8B, 4, 1088, 256, 0, {}),                                         # plain rule: DOWN in 4
    (LLAMA8B, 4, 1088, 100, 0, dict(down_tiles=98)),                        # 4 does not divide 98: none
]


def plain_ks(B, K, T):
    """Written out from the rule: at batch >= 8, the first of 4, 2 within K's slices of 2048 that
    divides T; below, the first of 1, 2, 4, 8 dividing T from the fewest parts whose fp64 staging of
    B sequences fits 128 KB."""
    if B == 1:
        return 1
    if B >= 8:
        for k in (4, 2):
            if k * 2048 < K + 2048 and T % k == 0:
                return k
        return 1
    need = 1
    while need < 8 and (K + need - 1) // need * B * 8 > 128 * 1024:
        need *= 2
    for k in (1, 2, 4, 8):
        if k >= need and T % k == 0:
            return k
    return 1


def test_split_k_plain_rule():
    ks = lambda g, op: {t[16] for t in g["tasks"] if t[1] == op}  # noqa: E731
    for B, wo, down, qkv in ((1, 1, 1, 1), (2, 1, 2, 1), (4, 1, 4, 1), (8, 2, 4, 1), (16, 2, 4, 1)):
        g = parse(mk.mk_build_graph(cfg_of(LLAMA8B, B, 1088, 0), 256))
        assert ks(g, OP_WO) == {wo} and ks(g, OP_DOWN) == {down} and ks(g, OP_QKV) == {qkv}
    # 1 turns it off; tile counts that 4 does not divide take 2, or none
    g = parse(mk.mk_build_graph(cfg_of(LLAMA8B, 8, 1088, 0, dict(wo_ksplit=1, down_ksplit=1, qkv_ksplit=1)), 256))
    assert ks(g, OP_WO) == {1} and ks(g, OP_DOWN) == {1} and ks(g, OP_QKV) == {1}
    g = parse(mk.mk_build_graph(cfg_of(LLAMA8B, 8, 1088, 0, dict(wo_tiles=255, down_tiles=250)), 256))
    assert ks(g, OP_WO) == {1} and ks(g, OP_DOWN) == {2}
    # QKV splits only when asked
    g = parse(mk.mk_build_graph(cfg_of(LLAMA8B, 16, 1088, 0, dict(qkv_tiles=6, qkv_ksplit=2)), 256))
    assert ks(g, OP_QKV) == {2}
    # the prefill graph never splits
    g = parse(mk.mk_build_prefill_graph(cfg_of(LLAMA8B, 8, 1088, 0), 256, 16, 64))
    assert ks(g, OP_WO) == {1} and ks(g, OP_DOWN) == {1} and ks(g, OP_QKV) == {1}


@pytest.mark.parametrize("shape,B,max_seq,workers,split,sched", KSPLIT_CASES)
def test_split_k_graph_bytes_equal_spec(shape, B, max_seq, workers, split, sched):
    got = mk.mk_build_graph(cfg_of(shape, B, max_seq, split, sched), workers)
    assert got == spec_bytes(shape, B, max_seq, workers, split, **sched)
    g = parse(got)
    # a part count not given takes the plain rule
    wo_ks = sched.get("wo_ksplit") or plain_ks(B, shape.n_q_heads * shape.head_dim, sched.get("wo_tiles") or workers)
    down_ks = sched.get("down_ksplit") or plain_ks(B, shape.ffn, sched.get("down_tiles") or workers)
    # QKV: row tiles of ks parts inside each KV-head group (plain rule: 2 with hidden's two K slices)
    tg = len([t for t in g["tasks"] if t[1] == OP_QKV and t[2] == 0]) // shape.n_kv_heads
    qks = sched.get("qkv_ksplit") or 1
    rg = (shape.n_q_heads // shape.n_kv_heads + 2) * shape.head_dim
    for layer in range(shape.n_layers):
        for grp in range(shape.n_kv_heads):
            ts = [t for t in g["tasks"] if t[1] == OP_QKV and t[2] == layer and t[3] // tg == grp]
            assert [(t[15], t[16]) for t in ts] == [(i % qks, qks) for i in range(tg)]
            assert all(ts[i][4:6] == ts[i - i % qks + qks - 1][4:6] for i in range(tg))
            rows = [(t[4], t[5]) for t in ts[qks - 1::qks]]
            assert rows[0][0] == grp * rg and rows[-1][1] == (grp + 1) * rg
            sig = [t for t in ts if t[9] != 0xFFFFFFFF]
            assert sig == ts[qks - 1::qks] and [t[10] for t in sig] == list(range(tg // qks))
    for op, ks in ((OP_WO, wo_ks), (OP_DOWN, down_ks)):
        for layer in range(shape.n_layers):
            ts = [t for t in g["tasks"] if t[1] == op and t[2] == layer]
            assert [(t[15], t[16]) for t in ts] == [(i % ks, ks) for i in range(len(ts))]
            # the parts of a row tile share its rows; the row tiles cover the output once
            rows = [(t[4], t[5]) for t in ts[ks - 1::ks]]
            assert all(ts[i][4:6] == ts[i - i % ks + ks - 1][4:6] for i in range(len(ts)))
            assert rows[0][0] == 0 and rows[-1][1] == shape.hidden
            assert all(a[1] == b[0] for a, b in zip(rows, rows[1:]))
            # only last parts signal, one slot per row tile
            sig = [t for t in ts if t[9] != 0xFFFFFFFF]
            assert sig == ts[ks - 1::ks] and [t[10] for t in sig] == list(range(len(sig)))
            assert g["events"][sig[0][9]][1] == len(sig)


@pytest.mark.parametrize("bad", [
    (replace(KSHAPE, lora_rank=8), 4, dict(wo_ksplit=2)),  # not with adapters
    (KSHAPE, 1, dict(down_ksplit=2)),                     # not for one sequence
    (LLAMA8B, 4, dict(qkv_ksplit=2)),                     # QKV: matrix-core GEMV only
    (LLAMA8B, 8, dict(qkv_ksplit=4)),                     # more parts than hidden's two K slices
    (LLAMA8B, 8, dict(qkv_tiles=5, qkv_ksplit=2)),        # does not divide the tiles per group
    (KSHAPE, 8, dict(down_ksplit=3)),                     # not 2, 4 or 8
    (KSHAPE, 8, dict(wo_ksplit=4)),                       # more parts than WO's two K slices
    (KSHAPE, 8, dict(down_tiles=30, down_ksplit=4)),      # does not divide the tile count
    (LLAMA8B, 8, dict(down_ksplit=8)),                    # 14336 has 7 K slices
    (KSHAPE, 8, dict(wo_ksplit=-2)),
])
def test_split_k_is_validated(bad):
    shape, B, sched = bad
    with pytest.raises(mk.MkError):
        mk.mk_build_graph(cfg_of(shape, B, 40, 0, sched), 24)


@pytest.mark.parametrize("case,seed", [(0, 0), (0, 1), (1, 2), (1, 3), (6, 4), (6, 5), (4, 6), (4, 7)])
def test_split_k_protocol_completes_without_stale_partials(case, seed):
    shape, B, max_seq, workers, split, sched = KSPLIT_CASES[case]
    g = parse(mk.mk_build_graph(cfg_of(shape, B, max_seq, split, sched), workers))
    bad = []
    assert simulate(g, shape, B, steps=3, start_pos=5, seed=seed, violations=bad)
    assert bad == []


def test_split_k_simulation_catches_a_reordered_list():
    # control for the simulator: the four parts of one down-projection row tile moved onto one worker
    # in reverse order put the reducing part ahead of parts it polls for, which must deadlock
    shape, B, max_seq, workers, split, sched = KSPLIT_CASES[0]
    g = parse(mk.mk_build_graph(cfg_of(shape, B, max_seq, split, dict(sched, down_tiles=4)), workers))
    assert simulate(g, shape, B, steps=2, start_pos=5, seed=0)
    idx = [i for i, t in enumerate(g["tasks"]) if t[1] == OP_DOWN and t[2] == 0]
    assert len(idx) == 4
    w0 = g["tasks"][idx[0]][11]
    moved = [g["tasks"][i][:11] + (w0,) + g["tasks"][i][12:] for i in reversed(idx)]
    tasks = list(g["tasks"])
    for i, t in zip(idx, moved):
        tasks[i] = t
    assert not simulate(dict(g, tasks=tasks), shape, B, steps=2, start_pos=5, seed=0)
