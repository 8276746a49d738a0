"""Task-graph construction: bit-exact against an independent spec builder, plus invariants
and a randomized-interleaving simulation of the event protocol (CPU only)."""
import random
import struct

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


def cfg_of(shape, B, max_seq, split):
    return mk.make_cfg(shape, batch=B, max_seq=max_seq, split=split)


def parse(raw: bytes):
    w = struct.unpack(f"<{len(raw) // 4}I", raw)
    magic, ver, workers, split, ns, nev, nt, nslots = w[:8]
    ev = [w[8 + 3 * i: 11 + 3 * i] for i in range(nev)]
    base = 8 + 3 * nev
    tasks = [w[base + 12 * i: base + 12 * (i + 1)] for i in range(nt)]
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
    assert g["magic"] == 0x31474B4D and g["ver"] == 1
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
    # each GEMV operator's tiles partition its output units (one writer per output row)
    H, F, V = shape.hidden, shape.ffn, shape.vocab
    RG = (shape.n_q_heads // shape.n_kv_heads + 2) * shape.head_dim
    for layer in range(shape.n_layers):
        for op, R in ((OP_QKV, shape.n_kv_heads * RG), (OP_WO, H), (OP_GU, F), (OP_DOWN, H)):
            rng = sorted((t[4], t[5]) for t in tasks if t[1] == op and t[2] == layer)
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


def simulate(g, shape, B, steps, start_pos, seed, drop=None):
    """Run every worker's list under random interleaving with the event rules, one flag per slot
    holding the number of steps its producer signalled; returns True if all steps complete, False
    on deadlock.  Attention splits beyond the current length do nothing.  A merging split stores
    its partial, stays on its worker until every active split of its head has stored, then
    signals; a split that does not merge stores and moves on without signalling.  The split
    holding the current position merges; with the attention tasks distributed (one slot per task)
    and more than 8 active splits, every active split merges a slice, and a wait on the attention
    event reads only the slots of the step's merging splits."""
    rnd = random.Random(seed)
    tasks, events = g["tasks"], g["events"]
    workers, S, Hkv = g["workers"], g["split"], shape.n_kv_heads
    per_layer = Hkv + 4
    dist = g["ns"] * B * Hkv <= workers
    lists = [[t for t in tasks if t[11] == w] for w in range(workers)]
    flags = {}                     # (event, slot) -> steps signalled
    done_split = {}                # (step, layer, bg) -> active splits that stored their partial
    stored = [False] * workers     # a merging split has stored and waits for its head's others
    pos = [0] * workers            # (step * len(list) + index)
    total = [steps * len(lst) for lst in lists]

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
                if target <= 0 or all(flags.get((t[6], sl), 0) >= target for sl in slots(t[6], step - t[8])):
                    ready.append(w)
        if not ready:
            return all(pos[w] >= total[w] for w in range(workers))
        w = rnd.choice(ready)
        step, i = divmod(pos[w], len(lists[w]))
        t = lists[w][i]
        signal = True
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
        pos[w] += 1
        if signal and not (drop is not None and t[0] == drop):
            assert flags.get((t[9], t[10]), 0) <= step, "slot signalled twice in a step"
            flags[(t[9], t[10])] = step + 1


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
