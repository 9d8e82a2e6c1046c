"""Pins of the CPU oracle against what the MLA prolog page and the mathematics
fix, independent of the oracle's own code (aclnnMlaPrologV2WeightNz,
"Function" formulas; aclnnMlaPreprocess, rope-mode constraint).

No page prints a worked numeric example, so the pins are closed forms,
invariants, special cases that reduce to a library routine, hand-worked tiny
cases, brute force on tiny shapes, and planted mistakes that must fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.generate import Dims, custom_workload


def lib_bf16_to_f64(bits):
    """bf16 bits -> float64 through torch's own bf16 type (a library routine)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


# ---------------------------------------------------------------------------
# bf16 codec
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.1, 0x3DCD), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0 + 2.0 ** -8, 0x3F80),             # tie between 1 and 1+2^-7 -> even (1)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),         # tie between 1+2^-7 and 1+2^-6 -> even
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie -> up
    (2.0 ** -133, 0x0001),                 # smallest subnormal
    (2.0 ** -134, 0x0000),                 # half of it: tie -> even (zero)
    (3.0 * 2.0 ** -134, 0x0002),           # 1.5 subnormal ulps: tie -> even (2)
    (3.5e38, 0x7F80), (-3.5e38, 0xFF80), (float("inf"), 0x7F80),
])
def test_bf16_encode_known_values(value, bits):
    assert int(oracle.bf16_bits([value])[0]) == bits


def test_bf16_encode_matches_library_on_float32_values():
    # for values already representable in binary32, nearest-even to bf16 is
    # what torch's float32 -> bfloat16 conversion does
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_decode_matches_library_on_all_finite_patterns():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint32).astype(np.uint16)
    e = (bits >> 7) & 0xFF
    bits = bits[e != 0xFF]
    assert np.array_equal(oracle.bf16_value(bits), lib_bf16_to_f64(bits))


def test_bf16_round_is_nearest():
    # the rounded value is never farther than half a bf16 step
    rng = np.random.default_rng(2)
    v = rng.standard_normal(5000) * 100
    r = oracle.bf16_value(oracle.bf16_bits(v))
    e = np.floor(np.log2(np.abs(v)))
    assert np.all(np.abs(r - v) <= 2.0 ** (e - 8) * (1 + 1e-12))


# ---------------------------------------------------------------------------
# fp16 codec (the preprocess page's FLOAT16 input)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3C00), (-2.0, 0xC000), (0.1, 0x2E66), (0.0, 0x0000), (-0.0, 0x8000),
    (65504.0, 0x7BFF),                      # largest finite
    (65519.99, 0x7BFF), (65520.0, 0x7C00),  # below / at the rounding tie to infinity
    (1.0 + 2.0 ** -11, 0x3C00),             # tie between 1 and 1+2^-10 -> even (1)
    (1.0 + 3 * 2.0 ** -11, 0x3C02),         # tie between 1+2^-10 and 1+2^-9 -> even
    (1.0 + 2.0 ** -11 + 2.0 ** -40, 0x3C01),  # just above the tie -> up
    (2.0 ** -14, 0x0400),                   # smallest normal
    (2.0 ** -24, 0x0001),                   # smallest subnormal
    (2.0 ** -25, 0x0000),                   # half of it: tie -> even (zero)
    (3.0 * 2.0 ** -25, 0x0002),             # 1.5 subnormal steps: tie -> even (2)
    (1023 * 2.0 ** -24 + 2.0 ** -25, 0x0400),  # the last subnormal tie carries into the normals
    (1e6, 0x7C00), (-1e6, 0xFC00), (float("inf"), 0x7C00),
])
def test_f16_encode_known_values(value, bits):
    assert int(oracle.f16_bits([value])[0]) == bits


def test_f16_encode_matches_library():
    # numpy's float64 -> float16 conversion rounds to nearest even directly
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 17, 20000),
                        rng.integers(-70000, 70000, 2000).astype(np.float64)])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_bits(v), ref)


def test_f16_decode_matches_library_on_all_finite_patterns():
    bits = np.arange(0, 1 << 16, 3, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 10) & 0x1F) != 0x1F]
    assert np.array_equal(oracle.f16_value(bits), lib_f16_to_f64(bits))


# ---------------------------------------------------------------------------
# RmsNorm (aclnnMlaPrologV2WeightNz, "RmsNorm formula")
# ---------------------------------------------------------------------------
def test_rmsnorm_hand_worked():
    # v = (3, 4): mean square 12.5; with eps = 0 the output is v / sqrt(12.5)
    out = oracle.rmsnorm([3.0, 4.0], [1.0, 1.0], 0.0)
    assert np.allclose(out, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    # gamma scales each element; eps = 0.5 sits inside the root: sqrt(13)
    out = oracle.rmsnorm([3.0, 4.0], [2.0, -1.0], 0.5)
    assert np.allclose(out, [6 / math.sqrt(13.0), -4 / math.sqrt(13.0)], rtol=0, atol=1e-15)


@pytest.mark.parametrize("n,eps", [(64, 1e-6), (1536, 1e-6), (512, 1e-5), (7, 0.3)])
def test_rmsnorm_unit_gamma_closed_form(n, eps):
    rng = np.random.default_rng(n)
    v = rng.standard_normal(n) * rng.uniform(0.01, 10)
    out = oracle.rmsnorm(v, np.ones(n), eps)
    ms = np.mean(v * v)
    assert abs(math.sqrt(np.mean(out * out)) - math.sqrt(ms / (ms + eps))) < 1e-12


def test_rmsnorm_scale_invariant_without_eps_and_linear_in_gamma():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(100)
    g = rng.uniform(0.5, 1.5, 100)
    a = oracle.rmsnorm(v, g, 0.0)
    assert np.allclose(oracle.rmsnorm(37.5 * v, g, 0.0), a, rtol=1e-13, atol=0)
    assert np.allclose(a, g * oracle.rmsnorm(v, np.ones(100), 0.0), rtol=1e-13, atol=0)


# ---------------------------------------------------------------------------
# RoPE, rotate-half (aclnnMlaPreprocess, rope-mode constraint)
# ---------------------------------------------------------------------------
def test_rope_identity_at_zero_angle():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(64)
    assert np.array_equal(oracle.rope(v, np.ones(64), np.zeros(64)), v)


def test_rope_is_complex_rotation_of_half_pairs():
    rng = np.random.default_rng(5)
    Dr, h = 64, 32
    v = rng.standard_normal(Dr)
    theta = rng.uniform(-10, 10, h)
    cos = np.concatenate([np.cos(theta)] * 2)
    sin = np.concatenate([np.sin(theta)] * 2)
    out = oracle.rope(v, cos, sin)
    z = (v[:h] + 1j * v[h:]) * np.exp(1j * theta)
    assert np.allclose(out[:h], z.real, rtol=0, atol=1e-14)
    assert np.allclose(out[h:], z.imag, rtol=0, atol=1e-14)
    # pair norms preserved
    assert np.allclose(out[:h] ** 2 + out[h:] ** 2, v[:h] ** 2 + v[h:] ** 2, rtol=1e-13)


def test_rope_hand_worked_quarter_turn():
    # Dr = 2, angle 90 degrees: (a, b) -> (-b, a)
    out = oracle.rope([3.0, 5.0], [0.0, 0.0], [1.0, 1.0])
    assert np.array_equal(out, [-5.0, 3.0])


def test_rope_angles_add():
    rng = np.random.default_rng(6)
    v = rng.standard_normal(16)
    t1, t2 = rng.uniform(-3, 3, 8), rng.uniform(-3, 3, 8)
    c = lambda t: np.concatenate([np.cos(t)] * 2)
    s = lambda t: np.concatenate([np.sin(t)] * 2)
    two = oracle.rope(oracle.rope(v, c(t1), s(t1)), c(t2), s(t2))
    assert np.allclose(two, oracle.rope(v, c(t1 + t2), s(t1 + t2)), rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# dynamic int8 ("Dequant Scale Query Nope calculation formula")
# ---------------------------------------------------------------------------
def test_quant_hand_worked():
    # max 1.0 -> scale 1/127; -0.5*127 = -63.5 ties to even (-64); 0.25*127 = 31.75 -> 32
    q, s = oracle.quant_int8([1.0, -0.5, 0.25, 0.0])
    assert s == np.float32(1.0) / np.float32(127.0)
    assert q.tolist() == [127, -64, 32, 0]


def test_quant_round_trip_bound_and_range():
    rng = np.random.default_rng(7)
    for _ in range(50):
        v = rng.standard_normal(512) * rng.uniform(1e-3, 1e3)
        q, s = oracle.quant_int8(v)
        v32 = v.astype(np.float32).astype(np.float64)
        assert np.all(np.abs(q.astype(np.int32)) <= 127)
        assert np.all(np.abs(v32 - s * q) <= s / 2 * (1 + 1e-6))
        i = int(np.argmax(np.abs(v)))
        assert abs(int(q[i])) == 127 and np.sign(q[i]) == np.sign(v[i])
        assert s == np.float32(np.max(np.abs(v32))) / np.float32(127)


def test_quant_zero_row():
    q, s = oracle.quant_int8(np.zeros(16))
    assert s == 0.0 and not q.any()


# ---------------------------------------------------------------------------
# the whole prolog
# ---------------------------------------------------------------------------
TINY = synth.workload("tiny_t4")
RAGGED = custom_workload("ragged", T=5, dims=Dims(He=40, Hcq=24, Hckv=12, N=3, D=6, Dr=4),
                         block_num=3, block_size=16, seed=11)
RAGGED_Q8 = custom_workload("ragged_q8", T=6, dims=Dims(He=48, Hcq=16, Hckv=8, N=2, D=4, Dr=6),
                            block_num=2, block_size=16, quant=True, seed=12)


def lib_f16_to_f64(bits):
    """fp16 bits -> float64 through numpy's own half type (a library routine)."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def values(inp, key):
    a = np.asarray(inp[key])
    if a.dtype == np.int8:
        return a.astype(np.float64)
    return lib_f16_to_f64(a) if inp.get("fp16") else lib_bf16_to_f64(a)


def brute_force(inp, cos_sin=None):
    """Scalar Python loops over the formulas, written without the oracle:
    returns y, c_q, c_kv, k_r, u (per head nope | rope), q_r, q_n, all float64,
    with no intermediate rounding.  Weights come unpacked (W^UQ, W^QR, W^DKV,
    W^KR taken on their own)."""
    d = inp["dims"]
    T = inp["T"]
    x = values(inp, "token_x").tolist()
    wdq = values(inp, "weight_dq").tolist()
    wuq = values(inp, "weight_uq").tolist()
    wqr = values(inp, "weight_qr").tolist()
    wdkv = values(inp, "weight_dkv").tolist()
    wkr = values(inp, "weight_kr").tolist()
    wuk = values(inp, "weight_uk").tolist()
    gcq = values(inp, "rmsnorm_gamma_cq").tolist()
    gckv = values(inp, "rmsnorm_gamma_ckv").tolist()
    cos = values(inp, "rope_cos").tolist()
    sin = values(inp, "rope_sin").tolist()
    quant = inp["quant"]
    res = {k: [] for k in ("y_q", "c_q", "c_kv", "k_r", "u_nope", "q_r", "q_n")}
    half = d.Dr // 2

    def mm(row, w, ncol):
        return [sum(row[k] * w[k][n] for k in range(len(row))) for n in range(ncol)]

    def norm(v, g, eps):
        r = math.sqrt(sum(a * a for a in v) / len(v) + eps)
        return [g[i] * v[i] / r for i in range(len(v))]

    def rot(v, c, s):
        return ([v[i] * c[i] - v[i + half] * s[i] for i in range(half)]
                + [v[i + half] * c[i + half] + v[i] * s[i + half] for i in range(half)])

    for t in range(T):
        yq, ykv, ykr = mm(x[t], wdq, d.Hcq), mm(x[t], wdkv, d.Hckv), mm(x[t], wkr, d.Dr)
        if quant:
            sx = float(inp["dequant_scale_x"][t])
            swq = inp["dequant_scale_w_dq"].astype(np.float64)
            swk = inp["dequant_scale_w_dkv_kr"].astype(np.float64)
            yq = [yq[n] * sx * swq[n] for n in range(d.Hcq)]
            ykv = [ykv[n] * sx * swk[n] for n in range(d.Hckv)]
            ykr = [ykr[n] * sx * swk[d.Hckv + n] for n in range(d.Dr)]
        cq = norm(yq, gcq, inp["eps_cq"])
        res["y_q"].append(yq)
        res["c_q"].append(cq)
        res["c_kv"].append(norm(ykv, gckv, inp["eps_ckv"]))
        res["k_r"].append(rot(ykr, cos[t], sin[t]))
        unope = mm(cq, wuq, d.N * d.D)
        urope = mm(cq, wqr, d.N * d.Dr)
        res["u_nope"].append(unope)
        res["q_r"].append([rot(urope[h * d.Dr:(h + 1) * d.Dr], cos[t], sin[t]) for h in range(d.N)])
        res["q_n"].append([[sum(unope[h * d.D + j] * wuk[h][j][c] for j in range(d.D))
                            for c in range(d.Hckv)] for h in range(d.N)])
    return {k: np.array(v) for k, v in res.items()}


def near_bf16(bits, ref):
    """Each bf16 value is within half a bf16 step of the float64 reference."""
    got = lib_bf16_to_f64(bits)
    ref = np.asarray(ref, dtype=np.float64)
    return np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)


def near_f16(bits, ref):
    """Each fp16 value is within half an fp16 step of the float64 reference
    (2^-11 relative for normal values, 2^-25 absolute below them)."""
    got = lib_f16_to_f64(bits)
    ref = np.asarray(ref, dtype=np.float64)
    return np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -11 + 2.0 ** -25)


@pytest.mark.parametrize("wl", [TINY, RAGGED], ids=["tiny_t4", "ragged"])
def test_whole_oracle_matches_brute_force(wl):
    inp = synth.make_inputs(wl, unpacked=True)
    d = inp["dims"]
    o = oracle.run(inp, round_intermediates=False, intermediates=True)
    bf = brute_force(inp)
    T = inp["T"]
    assert np.allclose(o["y"][:, :d.Hcq], bf["y_q"], rtol=1e-12, atol=1e-12)
    assert np.allclose(o["c_q"], bf["c_q"], rtol=1e-12, atol=1e-12)
    u = o["u"].reshape(T, d.N, d.D + d.Dr)
    assert np.allclose(u[:, :, :d.D].reshape(T, -1), bf["u_nope"], rtol=1e-12, atol=1e-12)
    assert np.allclose(o["q_n"], bf["q_n"], rtol=1e-11, atol=1e-12)
    assert near_bf16(o["kv_rows"], bf["c_kv"])
    assert near_bf16(o["kr_rows"], bf["k_r"])
    assert near_bf16(o["query_rope_out"], bf["q_r"])
    assert near_bf16(o["query_out"], bf["q_n"])


def test_int8_inputs_match_brute_force():
    inp = synth.make_inputs(RAGGED_Q8, unpacked=True)
    d = inp["dims"]
    o = oracle.run(inp, intermediates=True, query_int8=False)
    bf = brute_force(inp)
    assert np.allclose(o["y"][:, :d.Hcq], bf["y_q"], rtol=1e-13, atol=0)
    assert np.allclose(o["c_q"], bf["c_q"], rtol=1e-12, atol=1e-12)
    assert near_bf16(o["kv_rows"], bf["c_kv"])
    assert near_bf16(o["kr_rows"], bf["k_r"])
    # the up-projection runs on the per-token int8 image of c^Q (R3'):
    # u = (c8 . W8) * s_cq * s_w exactly, with c8, s_cq the pinned quantiser's
    w8 = np.asarray(inp["weight_uq_qr"]).astype(np.int64)
    sw = inp["dequant_scale_w_uq_qr"].astype(np.float64)
    for t in range(inp["T"]):
        c8, s = oracle.quant_int8(o["c_q"][t])
        u = (c8.astype(np.int64) @ w8).astype(np.float64) * float(s) * sw
        assert np.allclose(o["u"][t], u, rtol=1e-13, atol=0)


def test_composition_of_the_two_up_projections():
    # without R3/R5, q^N[t,h] = c^Q[t] (W^UQ_h W^UK_h): the product of the
    # per-head column block of W^UQ with that head's W^UK
    inp = synth.make_inputs(TINY, unpacked=True)
    d = inp["dims"]
    o = oracle.run(inp, round_intermediates=False, intermediates=True)
    wuq = values(inp, "weight_uq")
    wuk = values(inp, "weight_uk")
    for h in range(d.N):
        comp = wuq[:, h * d.D:(h + 1) * d.D] @ wuk[h]
        assert np.allclose(o["q_n"][:, h, :], o["c_q"] @ comp, rtol=1e-10, atol=1e-12)


def test_query_rope_at_zero_angle_is_the_qr_projection():
    # with cos = 1, sin = 0, q^R[t,h] = bf16(bf16(c^Q[t]) W^QR_h)
    inp = synth.make_inputs(TINY, unpacked=True)
    d = inp["dims"]
    inp["rope_cos"] = np.full_like(inp["rope_cos"], 0x3F80)
    inp["rope_sin"] = np.zeros_like(inp["rope_sin"])
    o = oracle.run(inp, intermediates=True)
    cq = oracle.bf16_value(oracle.bf16_bits(o["c_q"]))
    ref = cq @ values(inp, "weight_qr")
    assert near_bf16(o["query_rope_out"].reshape(inp["T"], -1), ref)
    # and the key rope is x W^KR
    assert near_bf16(o["kr_rows"], values(inp, "token_x") @ values(inp, "weight_kr"))


def test_rounding_points_feed_the_next_product():
    # with R3/R5 on, u = bf16(c^Q) W^UqQr and q^N = bf16(q^C) W^UK exactly
    inp = synth.make_inputs(TINY, unpacked=True)
    d = inp["dims"]
    T = inp["T"]
    o = oracle.run(inp, intermediates=True)
    cq = oracle.bf16_value(oracle.bf16_bits(o["c_q"]))
    assert np.allclose(o["u"], cq @ values(inp, "weight_uq_qr"), rtol=1e-12, atol=1e-13)
    qc = oracle.bf16_value(oracle.bf16_bits(o["u"].reshape(T, d.N, -1)[:, :, :d.D]))
    wuk = values(inp, "weight_uk")
    for h in range(d.N):
        assert np.allclose(o["q_n"][:, h], qc[:, h] @ wuk[h], rtol=1e-12, atol=1e-13)
    assert np.array_equal(o["query_out"], oracle.bf16_bits(o["q_n"]))


def test_int8_query_output():
    inp = synth.make_inputs(TINY)
    o = oracle.run(inp, intermediates=True, query_int8=True)
    q, s, qn = o["query_out"], o["dequant_scale_q_nope"], o["q_n"]
    for t in range(inp["T"]):
        for h in range(inp["dims"].N):
            q_ref, s_ref = oracle.quant_int8(qn[t, h])
            assert s[t, h] == np.float32(s_ref) and np.array_equal(q[t, h], q_ref)
            assert np.all(np.abs(qn[t, h] - s[t, h] * q[t, h]) <= s[t, h] / 2 * (1 + 1e-6))


def test_only_named_slots_change():
    inp = synth.make_inputs(RAGGED)
    o = oracle.run(inp)
    kv, kr = o["kv_cache"], o["kr_cache"]
    bs = inp["block_size"]
    touched = np.zeros(kv.shape[0] * bs, dtype=bool)
    for t, s in enumerate(inp["cache_index"]):
        touched[s] = True
        assert np.array_equal(kv[s // bs, s % bs, 0], o["kv_rows"][t])
        assert np.array_equal(kr[s // bs, s % bs, 0], o["kr_rows"][t])
    flat_kv = kv.reshape(-1, kv.shape[-1])
    flat_kr = kr.reshape(-1, kr.shape[-1])
    assert np.all(flat_kv[~touched] == synth.SENTINEL_BF16)
    assert np.all(flat_kr[~touched] == synth.SENTINEL_BF16)


def test_out_of_range_slots_are_skipped():
    inp = synth.make_inputs(RAGGED)
    n = inp["block_num"] * inp["block_size"]
    inp["cache_index"] = np.array([-1, n, n + 5, 0, 1], dtype=np.int64)
    o = oracle.run(inp)
    flat_kv = o["kv_cache"].reshape(-1, inp["dims"].Hckv)
    assert np.array_equal(flat_kv[0], o["kv_rows"][3])
    assert np.array_equal(flat_kv[1], o["kv_rows"][4])
    assert np.all(flat_kv[2:] == synth.SENTINEL_BF16)


def test_token_permutation_and_subsets():
    inp = synth.make_inputs(RAGGED)
    full = oracle.run(inp)
    perm = np.array([3, 0, 4, 2, 1])
    pin = dict(inp)
    for k in ("token_x", "rope_sin", "rope_cos", "cache_index"):
        pin[k] = np.ascontiguousarray(np.asarray(inp[k])[perm])
    p = oracle.run(pin)
    for k in ("query_out", "query_rope_out", "kv_rows", "kr_rows"):
        assert np.array_equal(p[k], full[k][perm])
    assert np.array_equal(p["kv_cache"], full["kv_cache"])
    sub = oracle.run(inp, tokens=[4, 1])
    assert np.array_equal(sub["query_out"], full["query_out"][[4, 1]])
    assert np.array_equal(sub["query_rope_out"], full["query_rope_out"][[4, 1]])


def test_thread_count_does_not_change_results():
    inp = synth.make_inputs(RAGGED_Q8)
    a = oracle.run(inp, nthreads=1)
    b = oracle.run(inp, nthreads=5)
    for k in a:
        assert np.array_equal(a[k], b[k])


# ---------------------------------------------------------------------------
# partial quantisation (int8 weightUqQr only) and smoothScalesCq
# ---------------------------------------------------------------------------
PARTIAL = synth.workload("tiny_partial_t4")
RAGGED_PARTIAL = custom_workload("ragged_partial", T=5, dims=Dims(He=40, Hcq=24, Hckv=12, N=3, D=6, Dr=4),
                                 block_num=3, block_size=16, seed=13, partial=True, smooth=True)
RAGGED_Q8_SMOOTH = custom_workload("ragged_q8_smooth", T=6, dims=Dims(He=48, Hcq=16, Hckv=8, N=2, D=4, Dr=6),
                                   block_num=2, block_size=16, quant=True, seed=14, smooth=True)


def _with(inp, **kw):
    out = dict(inp)
    out.update(kw)
    return out


@pytest.mark.parametrize("wl", [PARTIAL, RAGGED_PARTIAL], ids=["tiny_partial", "ragged_partial"])
def test_partial_scenario_keeps_the_bf16_cache_path(wl):
    # only weightUqQr is int8: y, c^Q and the cache rows are those of the
    # scalar formulas on the bf16 inputs, whatever weightUqQr holds
    inp = synth.make_inputs(wl, unpacked=True)
    d = inp["dims"]
    o = oracle.run(inp, intermediates=True)
    bf = brute_force(inp)
    assert np.allclose(o["y"][:, :d.Hcq], bf["y_q"], rtol=1e-12, atol=1e-12)
    assert np.allclose(o["c_q"], bf["c_q"], rtol=1e-12, atol=1e-12)
    assert near_bf16(o["kv_rows"], bf["c_kv"])
    assert near_bf16(o["kr_rows"], bf["k_r"])
    other = oracle.run(_with(inp, weight_uq_qr=np.zeros_like(inp["weight_uq_qr"])))
    assert np.array_equal(other["kv_cache"], o["kv_cache"])
    assert np.array_equal(other["kr_cache"], o["kr_cache"])


def _smooth_bound_holds(inp, o):
    """u = c8 W8 s_cq s_w approximates (c^Q * m) W8 s_w within the int8
    rounding of c^Q * m: each code is off by at most half a step s_cq (plus
    the float32 rounding of c^Q * m before the decision)."""
    w8 = np.asarray(inp["weight_uq_qr"]).astype(np.float64)
    sw = inp["dequant_scale_w_uq_qr"].astype(np.float64)
    m = inp.get("smooth_scales_cq")
    m = np.ones(inp["dims"].Hcq) if m is None else m.astype(np.float64)
    for t in range(inp["T"]):
        cm = o["c_q"][t] * m
        s = np.max(np.abs(cm)) / 127 * (1 + 1e-6)
        ref = (cm @ w8) * sw
        err = ((s / 2 + np.abs(cm) * 2.0 ** -24) @ np.abs(w8)) * sw
        if not np.all(np.abs(o["u"][t] - ref) <= err * (1 + 1e-9) + 1e-300):
            return False
    return True


@pytest.mark.parametrize("wl", [PARTIAL, RAGGED_PARTIAL, RAGGED_Q8_SMOOTH],
                         ids=["tiny_partial", "ragged_partial", "ragged_q8_smooth"])
def test_smoothed_up_projection_within_the_quantisation_bound(wl):
    inp = synth.make_inputs(wl)
    o = oracle.run(inp, intermediates=True, query_int8=False)
    assert _smooth_bound_holds(inp, o)
    # the smoothing is not a no-op on these inputs: the same bound around the
    # unsmoothed product fails
    assert not _smooth_bound_holds(_with(inp, smooth_scales_cq=None), o)


@pytest.mark.parametrize("wl", [PARTIAL, RAGGED_Q8_SMOOTH], ids=["tiny_partial", "ragged_q8_smooth"])
def test_unit_smoothing_is_no_smoothing(wl):
    inp = synth.make_inputs(wl)
    a = oracle.run(_with(inp, smooth_scales_cq=np.ones(inp["dims"].Hcq, dtype=np.float32)))
    b = oracle.run(_with(inp, smooth_scales_cq=None))
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("wl", [PARTIAL, RAGGED_Q8_SMOOTH], ids=["tiny_partial", "ragged_q8_smooth"])
def test_power_of_two_smoothing_scales_the_product_exactly(wl):
    # m = 4 everywhere: c^Q * 4 has the same int8 codes with a 4x scale, so
    # u is exactly 4x the unsmoothed u (every rounding commutes with 4)
    inp = synth.make_inputs(wl)
    d = inp["dims"]
    four = oracle.run(_with(inp, smooth_scales_cq=np.full(d.Hcq, 4.0, dtype=np.float32)),
                      intermediates=True, query_int8=False)
    one = oracle.run(_with(inp, smooth_scales_cq=None), intermediates=True, query_int8=False)
    assert np.array_equal(four["u"], 4.0 * one["u"])
    assert np.array_equal(four["c_q"], one["c_q"])


# ---------------------------------------------------------------------------
# KV-cache quantisation (quantScaleCkv / quantScaleCkr): R1', R2'
# ---------------------------------------------------------------------------
KVQ_PARTIAL = custom_workload("kvq_partial", T=5, dims=Dims(He=40, Hcq=32, Hckv=24, N=3, D=16, Dr=16),
                              block_num=3, block_size=16, seed=15, partial=True, smooth=True, kv_quant=True)
KVQ_FULL = custom_workload("kvq_full", T=6, dims=Dims(He=48, Hcq=16, Hckv=16, N=2, D=16, Dr=16),
                           block_num=2, block_size=16, quant=True, seed=16, kv_quant=True)


def _codes_within_half_step(codes, v, scale):
    """Each code is v * scale to within half a step (plus the float32
    roundings of v and of the product), or the saturated end of the int8
    range on the side v * scale lies."""
    x = np.asarray(v, np.float64) * np.asarray(scale, np.float64)
    c = np.asarray(codes).astype(np.float64)
    slack = 0.5 + np.abs(x) * 2.0 ** -22
    inner = (c > -128) & (c < 127)
    ok = np.where(inner, np.abs(c - x) <= slack, False)
    ok |= (c == 127) & (x >= 126.5 - np.abs(x) * 2.0 ** -22)
    ok |= (c == -128) & (x <= -127.5 + np.abs(x) * 2.0 ** -22)
    return bool(ok.all())


def _kvq_pins_hold(wl, mutation=0):
    try:
        inp = synth.make_inputs(wl)
        o = oracle.run(inp, intermediates=True, mutation=mutation, query_int8=False)
        ok = _codes_within_half_step(o["kv_rows"], o["c_kv"], inp["quant_scale_ckv"])
        # the same codes from the bf16 rows of the unquantised cache path
        plain = oracle.run(dict(inp, kv_quant=False, kv_cache=None, kr_cache=None), caches=False,
                           query_int8=False, mutation=mutation)
        bf = lib_bf16_to_f64(plain["kv_rows"])
        x = bf * inp["quant_scale_ckv"].astype(np.float64)
        inner = (o["kv_rows"] > -128) & (o["kv_rows"] < 127)
        ok = ok and bool(np.all(np.abs(o["kv_rows"][inner] - x[inner]) <= 0.5 + np.abs(x[inner]) * 2.0 ** -8))
        if wl.partial:
            ok = ok and _codes_within_half_step(o["kr_rows"], o["k_r"], inp["quant_scale_ckr"])
        return ok
    except Exception:
        return False


@pytest.mark.parametrize("wl", [KVQ_PARTIAL, KVQ_FULL], ids=["partial", "full"])
def test_cache_codes_are_the_scaled_rows(wl):
    assert _kvq_pins_hold(wl)


def test_cache_codes_saturate():
    inp = synth.make_inputs(KVQ_PARTIAL)
    big = dict(inp, quant_scale_ckv=np.full(inp["dims"].Hckv, 1e4, np.float32),
               quant_scale_ckr=np.full(inp["dims"].Dr, 1e4, np.float32))
    o = oracle.run(big, intermediates=True)
    for codes, v in ((o["kv_rows"], o["c_kv"]), (o["kr_rows"], o["k_r"])):
        x = v * 1e4
        out = np.abs(x) >= 128          # beyond the int8 range: saturated on its side
        assert out.mean() > 0.9
        assert np.all(np.where(x[out] > 0, codes[out] == 127, codes[out] == -128))


@pytest.mark.parametrize("wl", [KVQ_PARTIAL, KVQ_FULL], ids=["partial", "full"])
def test_cache_quantisation_leaves_the_queries_alone(wl):
    inp = synth.make_inputs(wl)
    a = oracle.run(inp)
    b = oracle.run(dict(inp, kv_quant=False, kv_cache=None, kr_cache=None), caches=False)
    for k in ("query_out", "query_rope_out"):
        assert np.array_equal(a[k], b[k])
    if not wl.partial:   # full quantisation keeps a bf16 kr cache
        assert a["kr_rows"].dtype == np.uint16 and np.array_equal(a["kr_rows"], b["kr_rows"])
    else:
        assert a["kr_rows"].dtype == np.int8
    # the int8 caches change only at the named slots
    kv = a["kv_cache"].reshape(-1, inp["dims"].Hckv)
    named = np.zeros(kv.shape[0], bool)
    named[inp["cache_index"]] = True
    assert np.all(kv[~named] == synth.SENTINEL_I8)
    assert np.array_equal(kv[inp["cache_index"]], a["kv_rows"])


def _whole_pins_hold(mutation):
    """All whole-prolog pins above, as one predicate, for the planted mistakes."""
    try:
        inp = synth.make_inputs(TINY, unpacked=True)
        d = inp["dims"]
        o = oracle.run(inp, round_intermediates=False, intermediates=True, mutation=mutation)
        bf = brute_force(inp)
        ok = (np.allclose(o["c_q"], bf["c_q"], rtol=1e-12, atol=1e-12)
              and np.allclose(o["q_n"], bf["q_n"], rtol=1e-11, atol=1e-12)
              and near_bf16(o["kv_rows"], bf["c_kv"]) and near_bf16(o["kr_rows"], bf["k_r"])
              and near_bf16(o["query_rope_out"], bf["q_r"])
              and near_bf16(o["query_out"], bf["q_n"]))
        return bool(ok)
    except Exception:
        return False


def test_pins_hold_without_planted_mistake():
    assert _whole_pins_hold(0)


def _smooth_pins_hold(mutation):
    try:
        ok = True
        for wl in (PARTIAL, RAGGED_Q8_SMOOTH):
            inp = synth.make_inputs(wl)
            o = oracle.run(inp, intermediates=True, query_int8=False, mutation=mutation)
            ok = ok and _smooth_bound_holds(inp, o)
        return bool(ok)
    except Exception:
        return False


def test_smooth_pins_hold_without_planted_mistake():
    assert _smooth_pins_hold(0)


@pytest.mark.parametrize("mutation", [6, 7], ids=["smooth_divided", "smooth_ignored"])
def test_planted_smoothing_mistakes_fail_a_pin(mutation):
    assert not _smooth_pins_hold(mutation)


def test_planted_cache_scale_mistake_fails_a_pin():
    # planted mistake 8: the cache value divided by its scale instead of multiplied
    assert _kvq_pins_hold(KVQ_PARTIAL) and _kvq_pins_hold(KVQ_FULL)
    assert not _kvq_pins_hold(KVQ_PARTIAL, mutation=8)
    assert not _kvq_pins_hold(KVQ_FULL, mutation=8)


@pytest.mark.parametrize("mutation", [1, 2, 3, 4, 5],
                         ids=["rope_sign", "eps_outside_root", "uq_qr_blocked", "wuk_transposed",
                              "gamma_dropped"])
def test_planted_mistakes_fail_a_pin(mutation):
    assert not _whole_pins_hold(mutation)


# ---------------------------------------------------------------------------
# the MLA preprocess page's static scenario (aclnnMlaPreprocess, "Function"
# formulas and parameter table, quantMode 0) and its concatenated layout
# ---------------------------------------------------------------------------
PRE = synth.workload("tiny_pre_t4")
RAGGED_PRE = custom_workload("ragged_pre", T=5, dims=Dims(He=48, Hcq=32, Hckv=16, N=3, D=16, Dr=16),
                             block_num=2, block_size=16, seed=14, preprocess=True)


def test_static_quant_hand_worked():
    # round-half-even(v * 4) + 3, saturated to [-128, 127]
    v = [0.25, -0.3, 10.0, -10.0, 0.125, 0.625, 0.875, 100.0, -100.0, -31.5]
    want = [4, 2, 43, -37, 3, 5, 7, 127, -128, -123]
    assert oracle.quant_static_asym(v, 4.0, 3).tolist() == want
    # without an offset the codes are the symmetric rounding, clipped to -128
    assert oracle.quant_static_asym([-40.0, 40.0, 0.375], 4.0, 0).tolist() == [-128, 127, 2]


def _kn(inp, key):
    """A weight as (k, n), whichever way the inputs hold it."""
    w = np.asarray(inp[key]).astype(np.int64)
    return w.T if inp.get("weight_nk") else w


def _codes(v, scale_bits, offset, fp16=False):
    """Static codes written with numpy: float32 product, rint (half to even)."""
    dec = lib_f16_to_f64 if fp16 else lib_bf16_to_f64
    s = np.float32(dec(np.asarray(scale_bits))[0])
    r = np.rint(np.asarray(v, np.float64).astype(np.float32) * s).astype(np.float64) + int(offset[0])
    return np.clip(r, -128, 127).astype(np.int64)


def brute_force_static(inp):
    """The static scenario with numpy in float64 (decisions in float32), written
    without the oracle: returns y, c_q (the norm before beta1), u, c_kv, k_r,
    q_r and q_n, the last four before their bf16 rounding."""
    d = inp["dims"]
    T, half = inp["T"], d.Dr // 2
    h16 = bool(inp.get("fp16"))
    x = values(inp, "token_x")
    if inp.get("x_norm", True):
        rms = np.sqrt((x * x).mean(axis=1, keepdims=True) + inp["eps_x"])
        v = values(inp, "rmsnorm_gamma_x") * x / rms + values(inp, "rmsnorm_beta_x")
    else:
        v = x
    x8 = _codes(v, inp["quant_scale_x"], inp["quant_offset_x"], h16)
    wcat = np.concatenate([_kn(inp, "weight_dq"), _kn(inp, "weight_dkv_kr")], axis=1)
    ds = np.concatenate([inp["dequant_scale_w_dq"], inp["dequant_scale_w_dkv_kr"]]).astype(np.float64)
    y = (x8 @ wcat + np.asarray(inp["bias_dqkv"], np.int64)).astype(np.float64) * ds
    yq, ykv, ykr = y[:, :d.Hcq], y[:, d.Hcq:d.Hcq + d.Hckv], y[:, d.Hcq + d.Hckv:]

    def norm(a, g, eps):
        return g * a / np.sqrt((a * a).mean(axis=1, keepdims=True) + eps)

    def rot(a, c, s):
        lo, hi = a[..., :half], a[..., half:]
        return np.concatenate([lo * c[..., :half] - hi * s[..., :half],
                               hi * c[..., half:] + lo * s[..., half:]], axis=-1)

    cq = norm(yq, values(inp, "rmsnorm_gamma_cq"), inp["eps_cq"])
    c8 = _codes(cq + values(inp, "rmsnorm_beta_cq"), inp["quant_scale_cq"], inp["quant_offset_cq"], h16)
    u = ((c8 @ _kn(inp, "weight_uq_qr") + np.asarray(inp["bias_uq_qr"], np.int64)).astype(np.float64)
         * inp["dequant_scale_w_uq_qr"].astype(np.float64))
    cos, sin = values(inp, "rope_cos"), values(inp, "rope_sin")
    uh = u.reshape(T, d.N, d.D + d.Dr)
    q_r = rot(uh[:, :, d.D:], cos[:, None, :], sin[:, None, :])
    # R5: q^C rounded to the 16-bit format (numpy's own half rounding for fp16)
    qc = (uh[:, :, :d.D].astype(np.float16).astype(np.float64) if h16
          else lib_bf16_to_f64(oracle.bf16_bits(uh[:, :, :d.D])))
    q_n = np.einsum("thd,hdc->thc", qc, values(inp, "weight_uk"))
    return {"y": y, "c_q": cq, "u": u, "c_kv": norm(ykv, values(inp, "rmsnorm_gamma_ckv"), inp["eps_ckv"]),
            "k_r": rot(ykr, cos, sin), "q_r": q_r, "q_n": q_n}


def _static_pins_hold(inp, mutation=0):
    d = inp["dims"]
    o = oracle.run(inp, intermediates=True, mutation=mutation)
    bf = brute_force_static(inp)
    q = o["query_out"]
    qn, qr = (q[..., :d.Hckv], q[..., d.Hckv:]) if inp.get("concat") else (q, o["query_rope_out"])
    near = near_f16 if inp.get("fp16") else near_bf16
    return bool(np.allclose(o["y"], bf["y"], rtol=1e-15, atol=0)
                and np.allclose(o["c_q"], bf["c_q"], rtol=1e-13, atol=1e-14)
                and np.allclose(o["u"], bf["u"], rtol=1e-15, atol=0)
                and near(o["kv_rows"], bf["c_kv"]) and near(o["kr_rows"], bf["k_r"])
                and near(qr, bf["q_r"]) and near(qn, bf["q_n"]))


PRE_F16 = synth.workload("tiny_pre_f16_t4")
RAGGED_PRE_F16 = custom_workload("ragged_pre_f16", T=5, dims=Dims(He=48, Hcq=32, Hckv=16, N=3, D=16, Dr=16),
                                 block_num=2, block_size=16, seed=15, preprocess=True, fp16=True)


@pytest.mark.parametrize("wl", [PRE, RAGGED_PRE, PRE_F16, RAGGED_PRE_F16],
                         ids=["tiny_pre", "ragged_pre", "tiny_pre_f16", "ragged_pre_f16"])
def test_static_scenario_matches_brute_force(wl):
    assert _static_pins_hold(synth.make_inputs(wl))


def test_fp16_outputs_are_fp16_roundings():
    # the FLOAT16 input: every 16-bit output is the fp16 rounding of its
    # double value (half an fp16 step), which a bf16 rounding misses by far
    inp = synth.make_inputs(RAGGED_PRE_F16)
    d = inp["dims"]
    o = oracle.run(inp, intermediates=True)
    bf = brute_force_static(inp)
    assert not inp["concat"]
    assert near_f16(o["query_out"], bf["q_n"]) and near_f16(o["query_rope_out"], bf["q_r"])
    assert near_f16(o["kv_rows"], bf["c_kv"]) and near_f16(o["kr_rows"], bf["k_r"])
    # the same bits read as bf16 are not near the references
    assert not near_bf16(o["query_out"], bf["q_n"])


@pytest.mark.parametrize("mutation", [1, 2, 4, 9, 10, 11],
                         ids=["rope_sign", "eps_outside", "wuk_transposed", "offset_ignored", "beta_dropped",
                              "bias_subtracted"])
def test_planted_mistakes_fail_the_fp16_static_pin(mutation):
    inp = synth.make_inputs(RAGGED_PRE_F16)
    try:
        held = _static_pins_hold(inp, mutation)
    except Exception:
        held = False
    assert not held


def test_fp16_static_pin_holds_without_planted_mistake():
    assert _static_pins_hold(synth.make_inputs(RAGGED_PRE_F16))


def test_static_scenario_without_the_input_norm():
    # doRmsNorm false: x is quantised as it is
    inp = synth.make_inputs(RAGGED_PRE)
    inp["x_norm"] = False
    assert _static_pins_hold(inp)
    a = oracle.run(synth.make_inputs(RAGGED_PRE), intermediates=True)
    assert not np.allclose(oracle.run(inp, intermediates=True)["y"], a["y"])


def test_bias_carries_the_offset():
    # with bias = -offset * sum_k W[k, n] + e, the codes' offset cancels
    # exactly: the result equals offset 0 with bias e, as long as no code
    # saturates (a small quantScale keeps the codes within +-60)
    base = synth.make_inputs(RAGGED_PRE)
    for k in ("quant_scale_x", "quant_scale_cq"):
        base[k] = oracle.bf16_bits(np.array([8.0]))
    zero = dict(base)
    for off, b, w in (("quant_offset_x", "bias_dqkv", None), ("quant_offset_cq", "bias_uq_qr", "weight_uq_qr")):
        o = int(base[off][0])
        assert o != 0
        wkn = (np.concatenate([_kn(base, "weight_dq"), _kn(base, "weight_dkv_kr")], axis=1) if w is None
               else _kn(base, w))
        zero[off] = np.zeros(1, np.int8)
        zero[b] = (np.asarray(base[b], np.int64) + o * wkn.sum(axis=0)).astype(np.int32)
    a = oracle.run(base, intermediates=True)
    z = oracle.run(zero, intermediates=True)
    assert np.array_equal(a["y"], z["y"]) and np.array_equal(a["u"], z["u"])
    assert np.array_equal(a["query_out"], z["query_out"])


def test_concatenated_layout_is_the_split_layout_side_by_side():
    inp = synth.make_inputs(PRE)
    d = inp["dims"]
    assert inp["concat"]
    c = oracle.run(inp)
    split = dict(inp, concat=False)
    split["kv_cache"] = np.full((inp["block_num"], inp["block_size"], 1, d.Hckv), synth.SENTINEL_BF16, np.uint16)
    split["kr_cache"] = np.full((inp["block_num"], inp["block_size"], 1, d.Dr), synth.SENTINEL_BF16, np.uint16)
    s = oracle.run(split)
    assert np.array_equal(c["query_out"], np.concatenate([s["query_out"], s["query_rope_out"]], axis=2))
    assert np.array_equal(c["kv_cache"], np.concatenate([s["kv_cache"], s["kr_cache"]], axis=3))
    assert "query_rope_out" not in c and "kr_cache" not in c


@pytest.mark.parametrize("wl", [PRE, RAGGED_Q8, TINY], ids=["tiny_pre", "ragged_q8", "tiny_bf16"])
def test_transposed_weights_give_the_same_result(wl):
    inp = synth.make_inputs(wl)
    flip = dict(inp, weight_nk=not inp.get("weight_nk", False))
    for k in ("weight_dq", "weight_uq_qr", "weight_dkv_kr"):
        flip[k] = np.ascontiguousarray(np.asarray(inp[k]).T)
    a, b = oracle.run(inp), oracle.run(flip)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_static_pins_hold_without_planted_mistake():
    assert _static_pins_hold(synth.make_inputs(RAGGED_PRE))


@pytest.mark.parametrize("mutation", [9, 10, 11], ids=["offset_ignored", "beta_dropped", "bias_subtracted"])
def test_planted_static_mistakes_fail_a_pin(mutation):
    inp = synth.make_inputs(RAGGED_PRE)
    try:
        held = _static_pins_hold(inp, mutation)
    except Exception:
        held = False
    assert not held
