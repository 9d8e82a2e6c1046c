"""The comparison rules of tests/parity.py on the CPU, with the oracle on both
sides: the allowances for int8 c^Q codes at a rounding tie and for q^C at a
rounding midpoint cover a value rounded the other way and nothing more."""
import numpy as np
import pytest

import oracle
import synth
from synth.generate import Dims, custom_workload
from parity import check_queries, qc_tie_allowance, tie_allowance

# token 35 of this workload has a c^Q * m code exactly at a tie in fp32
WL = custom_workload("partial_t37", T=37, dims=Dims(He=264, Hcq=80, Hckv=40, N=3, D=32, Dr=16),
                     block_num=4, block_size=16, seed=81, partial=True, smooth=True)
TIED_TOKEN = 35


def _tied_code(inp, ref, t):
    m = inp["smooth_scales_cq"].astype(np.float64)
    cm = ref["c_q"][t] * m
    v = np.abs(cm) / (np.max(np.abs(cm)) / 127)
    return int(np.argmin(np.abs(v - np.floor(v) - 0.5)))


def test_allowance_covers_a_tie_rounded_the_other_way():
    inp = synth.make_inputs(WL)
    rows = np.arange(inp["T"])
    ref = oracle.run(inp, intermediates=True)
    k = _tied_code(inp, ref, TIED_TOKEN)
    # nudge the tied code's smoothing factor so that the oracle itself rounds
    # it up instead of to even; no other code moves
    m = inp["smooth_scales_cq"].copy()
    m[k] = np.float32(m[k] * np.float32(1 + 2 ** -20))
    flipped = oracle.run(dict(inp, smooth_scales_cq=m))
    aqr, aqn, namb = tie_allowance(inp, ref, rows)
    assert namb >= 1 and aqr[TIED_TOKEN].max() > 0
    with pytest.raises(AssertionError):
        check_queries(flipped, ref, rows, False)          # the plain tolerance is too tight
    check_queries(flipped, ref, rows, False, (aqr, aqn))  # the allowance covers the flip


@pytest.mark.parametrize("mutation", [6, 7], ids=["smooth_divided", "smooth_ignored"])
def test_allowance_does_not_hide_a_planted_mistake(mutation):
    inp = synth.make_inputs(WL)
    rows = np.arange(inp["T"])
    ref = oracle.run(inp, intermediates=True)
    bad = oracle.run(inp, mutation=mutation)
    with pytest.raises(AssertionError):
        check_queries(bad, ref, rows, False, tie_allowance(inp, ref, rows)[:2])


def _bf16_round_as_fp16(bits):
    # fp16 values rounded to bf16 (nearest even), then written back as fp16
    v = np.ascontiguousarray(np.asarray(bits, np.uint16)).view(np.float16).astype(np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float16).view(np.uint16)


def test_fp16_outputs_must_carry_fp16_precision():
    # the oracle's own fp16 outputs pass; the same values rounded through
    # bf16 stay inside the bf16 bound but fail the fp16 precision check
    inp = synth.make_inputs(synth.workload("tiny_pre_f16_t4"))
    ref = oracle.run(inp, caches=False)
    if inp.get("concat", False):
        d = inp["dims"]
        q = np.asarray(ref["query_out"])
        ref = dict(ref, query_out=q[..., :d.Hckv], query_rope_out=q[..., d.Hckv:])
    rows = np.arange(int(inp["T"]))
    check_queries(ref, ref, rows, False, fp16=True)
    bad = dict(ref, query_out=_bf16_round_as_fp16(ref["query_out"]))
    with pytest.raises(AssertionError, match="not fp16's"):
        check_queries(bad, ref, rows, False, fp16=True)


# token 209 of this workload has u (head 2, nope column 70) within 1e-5 of a
# bf16 step of a rounding midpoint: q^C = bf16(u) may round either way
QC_WL = custom_workload("ring_partial_n3_d96_t256", T=256, dims=Dims(He=512, Hcq=192, Hckv=128, N=3, D=96, Dr=64),
                        block_num=17, block_size=16, partial=True, smooth=True, seed=386)
QC_TOKEN, QC_HEAD, QC_COL = 209, 2, 70


def _qc_case():
    inp = synth.make_inputs(QC_WL)
    rows = [QC_TOKEN]
    ref = oracle.run(inp, tokens=rows, caches=False, intermediates=True)
    d = inp["dims"]
    # nudge that column's dequantisation scale so that the oracle's u crosses
    # the midpoint; no other element of u moves
    col = QC_HEAD * (d.D + d.Dr) + QC_COL
    sw = inp["dequant_scale_w_uq_qr"].copy()
    sw[col] = np.float32(sw[col] * np.float32(1 + 2 ** -20))
    flipped = oracle.run(dict(inp, dequant_scale_w_uq_qr=sw), tokens=rows, caches=False, intermediates=True)
    return inp, ref, flipped


def test_qc_allowance_covers_a_midpoint_rounded_the_other_way():
    inp, ref, flipped = _qc_case()
    d = inp["dims"]
    u0 = ref["u"].reshape(d.N, d.D + d.Dr)
    u1 = flipped["u"].reshape(d.N, d.D + d.Dr)
    moved = np.argwhere(u0 != u1)
    assert moved.tolist() == [[QC_HEAD, QC_COL]]
    assert abs(u1[QC_HEAD, QC_COL] / u0[QC_HEAD, QC_COL] - 1) < 2e-6
    allow = qc_tie_allowance(inp, ref)
    assert allow[0, QC_HEAD].max() > 0 and allow[0, :QC_HEAD].max() == 0
    rows = np.array([0])
    with pytest.raises(AssertionError):
        check_queries(flipped, ref, rows, False)             # the plain tolerance is too tight
    check_queries(flipped, ref, rows, False, inp=inp)         # the allowance covers the other rounding


def test_qc_allowance_does_not_hide_a_planted_mistake():
    inp, ref, _ = _qc_case()
    bad = oracle.run(inp, tokens=[QC_TOKEN], caches=False, mutation=4)   # W^UK read transposed
    with pytest.raises(AssertionError):
        check_queries(bad, ref, np.array([0]), False, inp=inp)
