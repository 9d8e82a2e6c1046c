"""The entry point that allocates nothing (mla_prolog_run_noalloc), through
the C ABI, against mla_prolog_run of a handle on the same inputs, at the
parity tolerances: two calls in a row, the second with fewer tokens, so that
what the first left in the shared workspace cannot pass for the second's.

The two entry points may take different kernels for the same token count
(the handle's small-T runs hand data across blocks; the no-allocation call
never does), so the outputs are compared at the parity tolerances, and the
cache slots not named by cacheIndex bit for bit.
"""
import sys

import numpy as np
import pytest

import synth
from synth import device as dev
from synth.generate import Dims, custom_workload
from parity import assert_bf16_close, assert_int8_close, assert_scales_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import head_latent_attention_amd as mla  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def outputs(t):
    return {k: dev.bits(v) for k, v in t.items()
            if k in ("query_out", "query_rope_out", "dequant_scale_q_nope", "kv_cache", "kr_cache")}


def compare(inp, got, ref):
    """got (no-allocation call) against ref (handle), both full runs."""
    T = int(inp["T"])
    q8 = ref.get("dequant_scale_q_nope") is not None
    if ref.get("query_rope_out") is not None:
        assert_bf16_close(got["query_rope_out"], ref["query_rope_out"], "query_rope_out")
    if q8:
        assert_int8_close(got["query_out"], ref["query_out"], "query_out (int8)")
        assert_scales_close(got["dequant_scale_q_nope"], ref["dequant_scale_q_nope"], "dequant_scale_q_nope")
    else:
        assert_bf16_close(got["query_out"], ref["query_out"], "query_out")
    n = int(inp["block_num"]) * int(inp["block_size"])
    idx = np.asarray(inp["cache_index"], dtype=np.int64)[:T]
    named = np.zeros(n, dtype=bool)
    named[idx[(idx >= 0) & (idx < n)]] = True
    for k in ("kv_cache", "kr_cache"):
        if ref.get(k) is None:
            continue
        a, b = np.asarray(got[k]).reshape(n, -1), np.asarray(ref[k]).reshape(n, -1)
        assert np.array_equal(a[~named], b[~named]), f"{k} differs outside the named slots"
        if a.dtype == np.uint16:
            assert_bf16_close(a[named], b[named], k)
        else:
            assert np.abs(a[named].astype(np.int32) - b[named].astype(np.int32)).max(initial=0) <= 1, k


CASES = {
    # model head dims: the handle takes the one-launch kernel at 32 and 5
    # tokens, the no-allocation call the four stream-ordered kernels
    "bf16_t32_then_t5": (custom_workload("na_bf16", T=32, dims=Dims(He=512, Hcq=256, Hckv=512, N=8, D=128, Dr=64),
                                         block_num=4, block_size=16, seed=301), 5),
    # int8 full quantisation with the int8 query: tiled, then small-T
    "int8_t130_then_t37": (custom_workload("na_q8", T=130, dims=Dims(He=1024, Hcq=192, Hckv=512, N=3, D=128, Dr=64),
                                           block_num=16, block_size=16, quant=True, seed=302), 37),
    # the static scenario, concatenated layout, transposed weights
    "static_t70_then_t9": (custom_workload("na_pre", T=70, dims=Dims(He=1024, Hcq=256, Hckv=512, N=4, D=128, Dr=64),
                                           block_num=8, block_size=16, preprocess=True, concat=True, weight_nk=True,
                                           seed=303), 9),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_the_handle(name):
    wl, t_small = CASES[name]
    big = synth.make_inputs(wl)
    small = synth.make_inputs(wl, T=t_small)
    desc = mla.make_desc(**dev.desc_args(big))
    # the packed weights come from a handle's one-time conversion
    tw = dev.upload(big)
    with mla.MlaProlog(desc) as h:
        packed = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
        h.pack_weights(tw, packed)
        torch.cuda.synchronize()
        for inp in (big, small):
            T = int(inp["T"])
            say(f"case no-allocation call {name} T={T}")
            ta, tb = dev.upload(inp), dev.upload(inp)
            ta["packed_weights"] = tb["packed_weights"] = packed
            mla.run_noalloc(desc, ta, T)
            h.run(tb, T)
            torch.cuda.synchronize()
            h.check()
            compare(inp, outputs(ta), outputs(tb))
