"""Tolerances of the GPU-vs-oracle comparison, and the comparison itself.

bf16 outputs: |gpu - ref| <= 1e-2 + 1e-2 |ref| per element.  int8 q^N: at most
1 LSB apart, on at most 0.1% of the elements.  Dequantisation scales: relative
error <= 1e-2.  Cache slots: every slot not named by cacheIndex keeps its bits
exactly; named slots hold the row within the bf16 tolerance.  int8 (quantised)
cache rows: every code equals the oracle's, except that a value v * scale
within TIE_BAND of a rounding tie may round either way (the same reasoning as
for c^Q below: y's summation order is not fixed).

An int8 c^Q taken from a floating-point down-projection (partial
quantisation) is decided from y summed in fp32 on the device and in double
in the oracle; a code at a rounding tie may then go either way, and both are
results of the method (its summation order is not fixed).  A code whose
oracle value lies within TIE_BAND code units of a tie counts as ambiguous,
and the queries of its token may move, beyond the bf16 tolerance, by what
rounding those codes the other way changes: s_cq |W8[k, n]| s_w[n] per code
in u, carried through RoPE (q^R) and through bf16(q^C) W^UK (q^N).

q^C = bf16(u) (fp16 in the FLOAT16 scenario) is itself a rounding point
whose input carries the same freedom: u's last bits follow y's summation
order, through c^Q or through c^Q's int8 scale.  An element of u whose oracle
value lies within QC_TIE_BAND steps of a rounding midpoint may land one step
to either side; queryOut (bf16 / fp16) of its token and head may then move by
that step times |W^UK[h][j, :]| on top of the tolerance.
"""
import numpy as np

BF16_ATOL = 1e-2
BF16_RTOL = 1e-2
INT8_MAX_LSB = 1
INT8_MAX_FRAC = 1e-3
SCALE_RTOL = 1e-2
#: code units: the fp32 summation error of y, carried to c^Q * m / s_cq, is
#: about 1e-4 at the model sizes (sqrt(K) fp32 half-ulps of y's typical size,
#: times |gamma m| / (rms s_cq)); the band leaves a 10x margin
TIE_BAND = 1e-3
#: steps of q^C's format: u's relative error from y's summation order is a
#: few fp32 ulps (2^-22 or so), 2^-14 of a bf16 step; the band leaves a wide
#: margin and still flags only about one element in a thousand
QC_TIE_BAND = 1e-3


#: fp16 outputs (the static scenario's FLOAT16 variant) take the bf16 bound
#: above, which holds the int8 decisions on x and c^Q that fp32 and double may
#: take apart; that the outputs carry fp16's precision and not less is checked
#: on top: the median relative error stays below 2^-11, one fp16 half-step at
#: the bottom of a binade, where rounding to bf16 anywhere on the way would
#: put the median near 2^-10
FP16_MEDIAN_REL = 2.0 ** -11


def bf16_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp16_f64(bits) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.float16).astype(np.float64)


def half_f64(bits, fp16=False) -> np.ndarray:
    return fp16_f64(bits) if fp16 else bf16_f64(bits)


def assert_fp16_precision(g, r, what):
    m = np.abs(r) > 1e-3
    if m.sum() < 64:
        return
    rel = float(np.median(np.abs(g[m] - r[m]) / np.abs(r[m])))
    assert rel < FP16_MEDIAN_REL, f"{what}: median relative error {rel:.3e} is not fp16's"


def assert_bf16_close(got_bits, ref_bits, what, extra=None, fp16=False):
    """``extra``: an allowance per element on top of the tolerance.  With
    ``fp16`` both sides are fp16 bit patterns (see FP16_MEDIAN_REL)."""
    g, r = half_f64(got_bits, fp16), half_f64(ref_bits, fp16)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if fp16:
        assert_fp16_precision(g, r, what)
    tol = BF16_ATOL + BF16_RTOL * np.abs(r)
    if extra is not None:
        tol = tol + extra
    bad = ~(np.abs(g - r) <= tol)
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


def tie_allowance(inp, ref, rows):
    """Allowances for queryRopeOut and queryOut (bf16) of ``rows`` when c^Q's
    int8 codes come from a floating-point y: see the module text.  ``ref``
    holds the oracle's intermediates (c_q, u) for the rows.  Returns
    (allow_qr, allow_qn, number of ambiguous codes)."""
    d = inp["dims"]
    n = len(rows)
    w8 = np.asarray(inp["weight_uq_qr"])
    sw = np.asarray(inp["dequant_scale_w_uq_qr"], np.float64)
    m = inp.get("smooth_scales_cq")
    m = np.ones(d.Hcq) if m is None else np.asarray(m, np.float64)
    wuk = bf16_f64(inp["weight_uk"]).reshape(d.N, d.D, d.Hckv)
    cos = bf16_f64(inp["rope_cos"])
    sin = bf16_f64(inp["rope_sin"])
    half = d.Dr // 2
    allow_qr = np.zeros((n, d.N, d.Dr))
    allow_qn = np.zeros((n, d.N, d.Hckv))
    namb = 0
    for r, t in enumerate(rows):
        cm = ref["c_q"][r] * m
        amax = np.max(np.abs(cm))
        if amax == 0:
            continue
        s = amax / 127
        v = np.abs(cm) / s
        amb = np.abs(v - np.floor(v) - 0.5) < TIE_BAND
        if not amb.any():
            continue
        namb += int(amb.sum())
        du = (s * np.abs(w8[amb].astype(np.float64)).sum(axis=0) * sw).reshape(d.N, d.D + d.Dr)
        dr = du[:, d.D:]
        allow_qr[r, :, :half] = dr[:, :half] * np.abs(cos[t, :half]) + dr[:, half:] * np.abs(sin[t, :half])
        allow_qr[r, :, half:] = dr[:, half:] * np.abs(cos[t, half:]) + dr[:, :half] * np.abs(sin[t, half:])
        # bf16(q^C) moves by du plus one bf16 step of |u| + du
        u = np.abs(ref["u"][r].reshape(d.N, d.D + d.Dr)[:, :d.D]) + du[:, :d.D]
        step = 2.0 ** (np.floor(np.log2(np.maximum(u, 1e-300))) - 7)
        dqc = du[:, :d.D] + step * (du[:, :d.D] > 0)
        for h in range(d.N):
            allow_qn[r, h] = dqc[h] @ np.abs(wuk[h])
    return allow_qr, allow_qn, namb


def qc_tie_allowance(inp, ref, fp16=False):
    """Allowance for queryOut (bf16 or fp16) of the rows in ``ref``, which
    holds the oracle's u: for every element of u's nope columns within
    QC_TIE_BAND steps of a rounding midpoint of q^C's format, one step of
    q^C times |W^UK[h][j, :]|."""
    d = inp["dims"]
    u = np.asarray(ref["u"], np.float64).reshape(-1, d.N, d.D + d.Dr)[:, :, :d.D]
    a = np.abs(u)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    step = 2.0 ** (np.maximum(e, -14) - 10) if fp16 else 2.0 ** (e - 7)
    pos = a / step
    amb = (a > 0) & (np.abs(pos - np.floor(pos) - 0.5) < QC_TIE_BAND)
    wuk = np.abs(half_f64(inp["weight_uk"], fp16).reshape(d.N, d.D, d.Hckv))
    allow = np.zeros((u.shape[0], d.N, d.Hckv))
    for r, h, j in zip(*np.nonzero(amb)):
        allow[r, h] += step[r, h, j] * wuk[h, j]
    return allow


def check_queries(got, ref, rows, int8_query, allow=None, fp16=False, inp=None):
    """got: host arrays of the full run; ref: oracle outputs for ``rows``;
    allow: None, or the (queryRopeOut, queryOut) allowances of tie_allowance;
    fp16: the outputs are fp16 bit patterns; inp: the inputs, to add the
    q^C rounding allowance (``ref`` then holds the oracle's u)."""
    allow_qr, allow_qn = (None, None) if allow is None else allow
    if inp is not None and not int8_query:
        qc = qc_tie_allowance(inp, ref, fp16)
        allow_qn = qc if allow_qn is None else allow_qn + qc
    assert_bf16_close(got["query_rope_out"][rows], ref["query_rope_out"], "query_rope_out", allow_qr, fp16)
    if int8_query:
        assert_int8_close(got["query_out"][rows], ref["query_out"], "query_out (int8)")
        assert_scales_close(got["dequant_scale_q_nope"][rows], ref["dequant_scale_q_nope"],
                            "dequant_scale_q_nope")
    else:
        assert_bf16_close(got["query_out"][rows], ref["query_out"], "query_out", allow_qn, fp16)


def assert_cache_codes(got, ref_codes, v, scale, what):
    """int8 cache codes against the oracle's: equal, or one apart where the
    float32 value v * scale lies within TIE_BAND of a rounding tie."""
    g = np.asarray(got).astype(np.int32)
    r = np.asarray(ref_codes).astype(np.int32)
    x = np.abs(np.asarray(v, np.float64).astype(np.float32) * np.asarray(scale, np.float32)).astype(np.float64)
    tie = np.abs(x - np.floor(x) - 0.5) < TIE_BAND
    ok = (g == r) | (tie & (np.abs(g - r) == 1))
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} of {ok.size} codes differ; first at {tuple(i)}: "
                             f"gpu {g[tuple(i)]} ref {r[tuple(i)]}")


def check_caches(inp, kv_after, kr_after, ref, rows):
    """Untouched slots bit-exact; slots of ``rows`` within tolerance of the
    oracle's rows (int8 rows: assert_cache_codes, with the oracle's c_kv and
    k_r intermediates in ``ref``); every in-range named slot written."""
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
    kv8 = bool(inp.get("kv_quant", False))
    f16 = bool(inp.get("fp16", False))
    kr8 = kv8 and bool(inp.get("partial", False))
    for r, t in enumerate(rows):
        s = int(idx[t])
        if 0 <= s < nslots:
            if kv8:
                assert_cache_codes(kv1[s], ref["kv_rows"][r], ref["c_kv"][r], inp["quant_scale_ckv"],
                                   f"kv cache slot {s} (token {t})")
            else:
                assert_bf16_close(kv1[s], ref["kv_rows"][r], f"kv cache slot {s} (token {t})", fp16=f16)
            if kr8:
                assert_cache_codes(kr1[s], ref["kr_rows"][r], ref["k_r"][r], inp["quant_scale_ckr"],
                                   f"kr cache slot {s} (token {t})")
            else:
                assert_bf16_close(kr1[s], ref["kr_rows"][r], f"kr cache slot {s} (token {t})", fp16=f16)
    if valid.size:
        assert not np.all(kv1[valid] == kv0[valid], axis=1).any(), "a named kv slot was not written"
