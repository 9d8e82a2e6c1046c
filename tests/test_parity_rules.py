"""The comparison rules of tests/parity.py on the CPU, with the oracle on both
sides: the allowance for int8 c^Q codes at a rounding tie covers a code
rounded the other way and nothing more."""
import numpy as np
import pytest

import oracle
import synth
from synth.generate import Dims, custom_workload
from parity import check_queries, tie_allowance

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
