"""mk_prefill_noalloc (static token staging, no allocation) against mk_prefill, through the C ABI.

Two calls in a row on one context, the second with a shorter prompt set: after each, the decode that
follows must be bit-identical to the decode after mk_prefill of the same prompts on a second context.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from persistent_decode_megakernel_02_amd import binding as mk  # noqa: E402
from persistent_decode_megakernel_02_amd import synth  # noqa: E402
from persistent_decode_megakernel_02_amd.configs import TINY  # noqa: E402

pytestmark = pytest.mark.gpu


def _decode(eng, n):
    toks, logits = eng.decode(n)
    torch.cuda.synchronize()
    return toks.cpu().numpy(), logits.cpu().numpy()


def test_prefill_noalloc_matches_prefill_twice_second_shorter():
    print("[case] mk_prefill_noalloc vs mk_prefill, tiny batch 2, prompts of 23 then 9 tokens", flush=True)
    B, n = 2, 12
    weights = synth.make_weights(TINY, seed=7, device="cuda")
    long_p = synth.make_sequences(TINY, B, 23, 0, seed=7)["prompts"].numpy()
    short_p = synth.make_sequences(TINY, B, 9, 0, seed=8)["prompts"].numpy()
    ref = mk.Engine(TINY, batch=B, max_seq=22 + n)
    ref.load_weights(weights)
    na = mk.Engine(TINY, batch=B, max_seq=22 + n)
    na.load_weights(weights)
    try:
        for prompts in (long_p, short_p):
            ref.prefill(prompts)
            t_ref, l_ref = _decode(ref, n)
            mk.mk_prefill_noalloc(na.ctx, prompts)
            assert na.state()[0] == prompts.shape[1] - 1
            t_na, l_na = _decode(na, n)
            assert np.array_equal(t_na, t_ref)
            assert np.array_equal(l_na.view(np.uint32), l_ref.view(np.uint32))
        # beyond the static array's capacity: a clear error, nothing run
        big = mk.Engine(TINY, batch=4, max_seq=16400)
        try:
            big.load_weights(weights)
            with pytest.raises(mk.MkError) as e:
                mk.mk_prefill_noalloc(big.ctx, np.zeros((4, 16390), np.int32))  # 4 * 16389 staged tokens
        finally:
            big.close()
        assert e.value.code == mk.MK_ERR_CAPACITY and "at most 65536" in str(e.value)
    finally:
        ref.close()
        na.close()
