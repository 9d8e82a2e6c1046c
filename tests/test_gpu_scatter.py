"""Cache slot writes, bit for bit, on the HIP path alone.

The prolog page ("Parameters", cacheIndex, kvCacheRef, krCacheRef) writes
each token's c^KV and k^R rows to the slot cacheIndex names, in place, and
nothing else.  Against the double-precision oracle the row values can only
match to the bf16 bound (the device sums in fp32), so placement is pinned
here without the oracle:

- the same tokens run twice on fresh caches, with cacheIndex A and then an
  unrelated set of slots B: the row at slot A[t] of the first run equals the
  row at B[t] of the second, bit for bit, and every other slot keeps the
  sentinel;
- two tokens with identical inputs (x, sin/cos, and the per-token scale of
  int8 x) give bitwise identical cache rows and query rows.

The cases take the execution paths that write cache rows: the one-launch
small-T kernel, the paired kernel, the tiled medium and large paths, the
row-major kernels, int8 caches, the concatenated layout and fp16 tensors.  The debugging
check of cacheIndex (check_index) is covered at the end.
"""
import sys

import numpy as np
import pytest

import synth
from synth import device as dev
from synth.generate import Dims, custom_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import head_latent_attention_amd as mla  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = {
    "one_launch_t16": (custom_workload("sc_fused_t16", T=16, dims=Dims(He=384, Hcq=128, Hckv=512, N=16, D=128,
                                                                        Dr=64), block_num=4, block_size=16,
                                       seed=201), True, {}),
    "paired_t16": (custom_workload("sc_pair_t16", T=16, dims=Dims(He=384, Hcq=128, Hckv=512, N=16, D=128, Dr=64),
                                   block_num=4, block_size=16, seed=202), True, {"MLA_PROLOG_FUSED": "0"}),
    "tiled_t70": (custom_workload("sc_tiled_t70", T=70, dims=Dims(He=1024, Hcq=256, Hckv=512, N=4, D=128, Dr=64),
                                  block_num=8, block_size=16, seed=203), True, {}),
    "tiled_large_t2100": (custom_workload("sc_large_t2100", T=2100, dims=Dims(He=264, Hcq=72, Hckv=40, N=3, D=24,
                                                                           Dr=16), block_num=160, block_size=16,
                                          seed=204), True, {}),
    "row_major_t37": (custom_workload("sc_rm_t37", T=37, dims=Dims(He=264, Hcq=72, Hckv=40, N=3, D=24, Dr=16),
                                      block_num=4, block_size=16, seed=205), False, {}),
    "int8_kvq_t130": (custom_workload("sc_kvq_t130", T=130, dims=Dims(He=1024, Hcq=192, Hckv=512, N=3, D=128,
                                                                     Dr=64), block_num=16, block_size=16,
                                      quant=True, kv_quant=True, seed=206), True, {}),
    "partial_kvq_t5": (custom_workload("sc_pkvq_t5", T=5, dims=Dims(He=512, Hcq=256, Hckv=128, N=4, D=128, Dr=64),
                                       block_num=2, block_size=16, partial=True, smooth=True, kv_quant=True,
                                       seed=207), True, {}),
    "static_concat_t37": (custom_workload("sc_pre_t37", T=37, dims=Dims(He=272, Hcq=80, Hckv=48, N=3, D=32, Dr=16),
                                          block_num=4, block_size=16, preprocess=True, concat=True,
                                          weight_nk=True, seed=208), True, {}),
    "static_fp16_t70": (custom_workload("sc_pre16_t70", T=70, dims=Dims(He=1024, Hcq=256, Hckv=512, N=4, D=128,
                                                                      Dr=64), block_num=8, block_size=16,
                                        preprocess=True, weight_nk=True, fp16=True, seed=209), True, {}),
}


def run(inp, packed, cache_index=None):
    """One run on fresh sentinel caches; host copies of every output."""
    t = dev.upload(inp)
    if cache_index is not None:
        t["cache_index"] = torch.from_numpy(np.asarray(cache_index, dtype=np.int64)).to("cuda")
    desc = mla.make_desc(**dev.desc_args(inp))
    with mla.MlaProlog(desc) as h:
        if packed:
            buf = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
            h.pack_weights(t, buf)
            t["packed_weights"] = buf
        h.run(t, int(inp["T"]))
        torch.cuda.synchronize()
    return {k: dev.bits(v) for k, v in t.items()
            if k in ("query_out", "query_rope_out", "dequant_scale_q_nope", "kv_cache", "kr_cache")}


def slot_rows(inp, got):
    """The caches as (slots, row) arrays: kv (with k^R after c^KV in the
    concatenated layout), and kr when separate."""
    n = int(inp["block_num"]) * int(inp["block_size"])
    out = [np.asarray(got["kv_cache"]).reshape(n, -1)]
    if got.get("kr_cache") is not None:
        out.append(np.asarray(got["kr_cache"]).reshape(n, -1))
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_slot_placement_is_bit_exact(name, monkeypatch):
    wl, packed, env = CASES[name]
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    inp = synth.make_inputs(wl)
    T = int(inp["T"])
    n = int(inp["block_num"]) * int(inp["block_size"])
    a = np.asarray(inp["cache_index"], dtype=np.int64)
    # B: distinct slots drawn apart from A's order
    b = np.random.default_rng(1000 + T).permutation(n)[:T].astype(np.int64)
    say(f"case slot placement {name} T={T} slots={n} packed={packed}")
    ga, gb = run(inp, packed), run(inp, packed, cache_index=b)
    sentinel = [slot_rows(inp, {k: inp[k] for k in ("kv_cache", "kr_cache") if inp.get(k) is not None})]
    for ca, cb, c0 in zip(slot_rows(inp, ga), slot_rows(inp, gb), sentinel[0]):
        # the named slots hold the same bits in both runs
        assert np.array_equal(ca[a], cb[b]), "a token's row differs between its two slots"
        # and every other slot still holds the sentinel
        keep_a = np.ones(n, dtype=bool); keep_a[a] = False
        keep_b = np.ones(n, dtype=bool); keep_b[b] = False
        assert np.array_equal(ca[keep_a], c0[keep_a]), "run A wrote outside its slots"
        assert np.array_equal(cb[keep_b], c0[keep_b]), "run B wrote outside its slots"
        # every named slot was written (the row differs from the sentinel row)
        assert not np.all(ca[a] == c0[a], axis=1).any(), "a named slot kept the sentinel"
    # the queries do not depend on the slots
    for k in ("query_out", "query_rope_out", "dequant_scale_q_nope"):
        if ga.get(k) is not None:
            assert np.array_equal(ga[k], gb[k]), k


@pytest.mark.parametrize("name", list(CASES))
def test_identical_tokens_give_identical_rows(name, monkeypatch):
    wl, packed, env = CASES[name]
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    inp = synth.make_inputs(wl)
    T = int(inp["T"])
    last = T - 1
    for k in ("token_x", "rope_sin", "rope_cos", "dequant_scale_x"):
        if inp.get(k) is not None:
            arr = np.array(inp[k])
            arr[last] = arr[0]
            inp[k] = arr
    say(f"case identical tokens 0 and {last}: {name}")
    got = run(inp, packed)
    idx = np.asarray(inp["cache_index"], dtype=np.int64)
    for rows in slot_rows(inp, got):
        assert np.array_equal(rows[idx[0]], rows[idx[last]]), "identical tokens wrote different cache rows"
    for k in ("query_out", "query_rope_out", "dequant_scale_q_nope"):
        if got.get(k) is not None:
            assert np.array_equal(got[k][0], got[k][last]), k


def test_check_index_refuses_out_of_range_slots():
    # the debugging check: a run whose cacheIndex leaves [0, slots) returns
    # 161002 and enqueues nothing; a valid one runs as usual
    wl, packed, _ = CASES["tiled_t70"]
    inp = synth.make_inputs(wl)
    T = int(inp["T"])
    n = int(inp["block_num"]) * int(inp["block_size"])
    say("case check_index")
    t = dev.upload(inp)
    desc = mla.make_desc(**dev.desc_args(inp), check_index=1)
    with mla.MlaProlog(desc) as h:
        for bad in (-1, n, n + 5):
            idx = np.array(inp["cache_index"], dtype=np.int64)
            idx[T // 2] = bad
            with pytest.raises(mla.MlaError) as e:
                h.run(dict(t, cache_index=torch.from_numpy(idx).to("cuda")), T)
            assert e.value.status == mla.MLA_ERR_PARAM_INVALID
        torch.cuda.synchronize()
        assert not dev.bits(t["query_out"]).any(), "a refused run wrote queryOut"
        assert np.array_equal(dev.bits(t["kv_cache"]), np.asarray(inp["kv_cache"])), "a refused run wrote the cache"
        h.run(t, T)
        torch.cuda.synchronize()
    # the same path without the check gives the same bits
    ref = run(inp, packed=False)
    for k in ("query_out", "query_rope_out", "kv_cache", "kr_cache"):
        assert np.array_equal(dev.bits(t[k]), ref[k]), k
