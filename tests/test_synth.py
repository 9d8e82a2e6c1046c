"""The seeded input generator: determinism, shapes, and the cache-slot recipes."""
import numpy as np

import synth


def test_deterministic_and_prefix():
    wl = synth.workload("tiny_t4")
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    for k, v in a.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b[k]), k
    c = synth.make_inputs(wl, T=2)
    assert np.array_equal(c["token_x"], a["token_x"][:2])
    assert np.array_equal(c["cache_index"], a["cache_index"][:2])


def test_shapes_and_distinct_slots():
    a = synth.make_inputs(synth.workload("tiny_t4"))
    d = a["dims"]
    assert a["token_x"].shape == (4, d.He) and a["token_x"].dtype == np.uint16
    assert a["weight_uq_qr"].shape == (d.Hcq, d.N * (d.D + d.Dr))
    assert a["weight_dkv_kr"].shape == (d.He, d.Hckv + d.Dr)
    assert a["weight_uk"].shape == (d.N, d.D, d.Hckv)
    assert a["kv_cache"].shape == (4, 16, 1, d.Hckv)
    idx = a["cache_index"]
    assert len(set(idx.tolist())) == len(idx) and idx.min() >= 0 and idx.max() < 64
    assert np.all(a["kv_cache"] == synth.SENTINEL_BF16)


def test_prefill_slots_fill_blocks_contiguously():
    from synth.generate import custom_workload, MODEL
    wl = custom_workload("p", T=2 * 300, dims=MODEL, block_num=16, block_size=128,
                         positions="prefill:2x300")
    pos, slots = synth.generate._positions_and_slots(wl)
    assert np.array_equal(pos[:300], np.arange(300)) and np.array_equal(pos[300:], np.arange(300))
    assert len(set(slots.tolist())) == 600
    # within a block, consecutive positions land in consecutive slots
    assert np.all(np.diff(slots[:128]) == 1) and slots[0] % 128 == 0


def test_int8_workload_ranges():
    from synth.generate import custom_workload, Dims
    wl = custom_workload("q", T=8, dims=Dims(64, 32, 16, 2, 8, 8), block_num=2, block_size=16,
                         quant=True)
    a = synth.make_inputs(wl)
    assert a["token_x"].dtype == np.int8 and a["token_x"].min() >= -127
    assert np.all((a["dequant_scale_x"] > 0.005) & (a["dequant_scale_x"] < 0.02))
    assert np.all((a["dequant_scale_w_dq"] >= 0.001) & (a["dequant_scale_w_dq"] <= 0.01))
