"""Host logic of the trace anatomy tool on a synthetic trace with known answers."""
import numpy as np

from persistent_decode_megakernel_02_amd.trace_anatomy import anatomy


def test_anatomy_of_a_synthetic_trace():
    # 5 layers, each one GEMV instance (op 4, gate/up) and one attention instance (op 2), two
    # workers with one task each per instance; clock 1 MHz, so one tick is 1 us
    L, khz = 5, 1000
    op, layer, lists = [], [], [[], []]
    tr = np.zeros((2, 2 * L, 4), dtype=np.uint64)
    t0 = 100.0
    for l in range(L):
        for o in (2, 4):
            for wk in range(2):
                i = len(op)
                op.append(o)
                layer.append(l)
                lists[wk].append(i)
            # worker 0 ends first, worker 1 last; both start before the previous end (P = t0)
            for wk, (st, se, sg, en) in enumerate([(t0 - 1, t0 + 2, t0 + 3, t0 + 10), (t0 + 1, t0 + 4, t0 + 6, t0 + 12)]):
                tr[wk, len(lists[wk]) - 1] = [st, se, sg, en]
            t0 += 12
    g = {"op": op, "layer": layer, "lists": lists, "L": L}
    res = anatomy(tr, khz, g)
    gu = res["GU"]
    assert gu["phase"] == 12 and gu["det_first"] == 2 and gu["det_last"] == 4
    assert gu["late"] == 1 and gu["late_seen"] == 3            # worker 1 started at +1, saw at +4
    assert gu["stage"] == 1.5 and gu["work"] == 8              # medians of (1, 2) and (8, 8)
    assert (gu["crit_start"], gu["crit_seen"], gu["crit_staged"], gu["crit_end"]) == (1, 4, 6, 12)
    assert gu["spread_p50"] == 1 and abs(gu["spread_p90"] - 1.8) < 1e-9
    assert res["ATT"]["stage"] == 0.0
