"""Tolerances of the GPU-vs-oracle comparison, and the comparison itself.

bf16 outputs: |gpu - ref| <= 1e-2 + 1e-2 |ref| per element.  int8 q^N: at most
1 LSB apart, on at most 0.1% of the elements.  Dequantisation scales: relative
error <= 1e-2.  Cache slots: every slot not named by cacheIndex keeps its bits
exactly; named slots hold the row within the bf16 tolerance.
"""
import numpy as np

BF16_ATOL = 1e-2
BF16_RTOL = 1e-2
INT8_MAX_LSB = 1
INT8_MAX_FRAC = 1e-3
SCALE_RTOL = 1e-2


def bf16_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def assert_bf16_close(got_bits, ref_bits, what):
    g, r = bf16_f64(got_bits), bf16_f64(ref_bits)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    bad = ~(np.abs(g - r) <= BF16_ATOL + BF16_RTOL * np.abs(r))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; "
                             f"first at {tuple(i)}: gpu {g[tuple(i)]} ref {r[tuple(i)]}")


def assert_int8_close(got, ref, what):
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert diff.max(initial=0) <= INT8_MAX_LSB, f"{what}: max int8 difference {diff.max()}"
    frac = np.count_nonzero(diff) / max(1, diff.size)
    assert frac <= INT8_MAX_FRAC, f"{what}: {frac:.2e} of elements differ"
    return frac


def assert_scales_close(got, ref, what):
    g, r = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rel = np.abs(g - r) / np.maximum(np.abs(r), 1e-30)
    ok = (rel <= SCALE_RTOL) | ((g == 0) & (r == 0))
    assert ok.all(), f"{what}: worst relative error {rel[~ok].max()}"


def check_queries(got, ref, rows, int8_query):
    """got: host arrays of the full run; ref: oracle outputs for ``rows``."""
    assert_bf16_close(got["query_rope_out"][rows], ref["query_rope_out"], "query_rope_out")
    if int8_query:
        assert_int8_close(got["query_out"][rows], ref["query_out"], "query_out (int8)")
        assert_scales_close(got["dequant_scale_q_nope"][rows], ref["dequant_scale_q_nope"],
                            "dequant_scale_q_nope")
    else:
        assert_bf16_close(got["query_out"][rows], ref["query_out"], "query_out")


def check_caches(inp, kv_after, kr_after, ref, rows):
    """Untouched slots bit-exact; slots of ``rows`` within tolerance of the
    oracle's rows; every in-range named slot written."""
    d = inp["dims"]
    nslots = int(inp["block_num"]) * int(inp["block_size"])
    kv0 = np.asarray(inp["kv_cache"]).reshape(nslots, d.Hckv)
    kr0 = np.asarray(inp["kr_cache"]).reshape(nslots, d.Dr)
    kv1 = np.asarray(kv_after).reshape(nslots, d.Hckv)
    kr1 = np.asarray(kr_after).reshape(nslots, d.Dr)
    idx = np.asarray(inp["cache_index"], dtype=np.int64)
    named = np.zeros(nslots, dtype=bool)
    valid = idx[(idx >= 0) & (idx < nslots)]
    named[valid] = True
    assert np.array_equal(kv1[~named], kv0[~named]), "kv cache changed outside the named slots"
    assert np.array_equal(kr1[~named], kr0[~named]), "kr cache changed outside the named slots"
    for r, t in enumerate(rows):
        s = int(idx[t])
        if 0 <= s < nslots:
            assert_bf16_close(kv1[s], ref["kv_rows"][r], f"kv cache slot {s} (token {t})")
            assert_bf16_close(kr1[s], ref["kr_rows"][r], f"kr cache slot {s} (token {t})")
    if valid.size:
        assert not np.all(kv1[valid] == kv0[valid], axis=1).any(), "a named kv slot was not written"
