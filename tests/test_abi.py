"""The C ABI on the host: the library loads, exports every symbol the header
declares, and its pure-host validation returns the page's status classes
(aclnnMlaPrologV2WeightNz, "Return Value").  No device is touched."""
import ctypes
import os
import re

import pytest

import head_latent_attention_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\w[\w\s\*]*?\b(mla_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_exports_every_declared_symbol():
    declared = header_functions()
    assert set(declared) == set(mla.EXPORTS), declared
    L = mla.lib()
    for name in declared:
        assert hasattr(L, name), name


def model_desc(**kw):
    a = dict(He=7168, Hcq=1536, Hckv=512, N=128, D=128, Dr=64, block_num=1024, block_size=128,
             max_tokens=256, eps_cq=1e-6, eps_ckv=1e-6)
    a.update(kw)
    return mla.make_desc(**a)


FAKE = 1 << 40   # an aligned address; validate never dereferences it


STATIC_ONLY = ("gamma_x", "beta_x", "quant_scale_x", "quant_offset_x", "bias_dqkv", "beta_cq",
               "quant_scale_cq", "quant_offset_cq", "bias_uq_qr")


def fake_tensors(q8=False, in8=False, partial=False, smooth=False, kvq=False, static=False,
                 concat=False):
    t = {f: FAKE for f in mla.TENSOR_FIELDS}
    if not static:
        for f in STATIC_ONLY:
            t[f] = None
    else:
        t["scale_x"] = None
    if concat:
        t["query_rope_out"] = None
        t["kr_cache"] = None
    if not kvq:
        t["quant_scale_ckv"] = None
    if not (kvq and partial):
        t["quant_scale_ckr"] = None
    if not (in8 or static):
        for f in ("scale_x", "scale_w_dq", "scale_w_dkv_kr"):
            t[f] = None
        if not partial:
            t["scale_w_uq_qr"] = None
    elif not in8:
        t["scale_x"] = None
    if not q8:
        t["dequant_scale_q_nope"] = None
    if not smooth:
        t["smooth_scales_cq"] = None
    return t


def test_valid_descriptions():
    assert mla.validate(model_desc()) == mla.MLA_OK
    assert mla.validate(model_desc(), fake_tensors(), 32) == mla.MLA_OK
    assert mla.validate(model_desc(in_dtype=1, query_dtype=1), fake_tensors(True, True), 128) == mla.MLA_OK
    assert mla.validate(model_desc(in_dtype=1), fake_tensors(in8=True, smooth=True), 128) == mla.MLA_OK
    part = model_desc(in_dtype=mla.MLA_INT8_PARTIAL)
    assert mla.validate(part, fake_tensors(partial=True), 32) == mla.MLA_OK
    assert mla.validate(part, fake_tensors(partial=True, smooth=True), 32) == mla.MLA_OK
    # quantised caches: kv (full quantisation), kv and kr (partial)
    assert mla.validate(model_desc(in_dtype=1, query_dtype=1, cache_dtype=1),
                        fake_tensors(True, True, kvq=True), 128) == mla.MLA_OK
    assert mla.validate(model_desc(in_dtype=2, cache_dtype=1),
                        fake_tensors(partial=True, kvq=True), 32) == mla.MLA_OK
    # the bf16 down-projection of partial quantisation keeps the bf16 size rules
    assert mla.validate(model_desc(in_dtype=mla.MLA_INT8_PARTIAL, He=7176, Hckv=504)) == mla.MLA_OK
    # the preprocess page's static scenario, its concatenated layout and
    # transposed weights (which need the packed copy)
    st = model_desc(in_dtype=mla.MLA_INT8_STATIC, concat=1, weights_nk=1)
    assert mla.validate(st, fake_tensors(static=True, concat=True), 32) == mla.MLA_OK
    t = fake_tensors(static=True); t["bias_dqkv"] = None; t["bias_uq_qr"] = None   # biases optional
    assert mla.validate(model_desc(in_dtype=3), t, 32) == mla.MLA_OK
    t = fake_tensors(static=True); t["gamma_x"] = None; t["beta_x"] = None
    assert mla.validate(model_desc(in_dtype=3, x_quant_only=1), t, 32) == mla.MLA_OK
    assert mla.validate(model_desc(concat=1), fake_tensors(concat=True), 32) == mla.MLA_OK
    # the static scenario's FLOAT16 input, split and concatenated
    assert mla.validate(model_desc(in_dtype=3, float_dtype=mla.MLA_FP16), fake_tensors(static=True), 32) == mla.MLA_OK
    assert mla.validate(model_desc(in_dtype=3, concat=1, weights_nk=1, float_dtype=mla.MLA_FP16),
                        fake_tensors(static=True, concat=True), 32) == mla.MLA_OK
    tiny = mla.make_desc(256, 64, 32, 2, 16, 8, 4, 16, 4)
    assert mla.validate(tiny, fake_tensors(), 4) == mla.MLA_OK
    assert mla.workspace_bytes(model_desc()) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(He=0), mla.MLA_ERR_PARAM_INVALID),
    (dict(N=-2), mla.MLA_ERR_PARAM_INVALID),
    (dict(block_size=24), mla.MLA_ERR_PARAM_INVALID),
    (dict(block_num=-1), mla.MLA_ERR_PARAM_INVALID),
    (dict(eps_cq=-1.0), mla.MLA_ERR_PARAM_INVALID),
    (dict(in_dtype=4), mla.MLA_ERR_PARAM_INVALID),
    (dict(in_dtype=3, query_dtype=1), mla.MLA_ERR_PARAM_INVALID),   # the static scenario: bf16 queryOut
    (dict(in_dtype=3, cache_dtype=1), mla.MLA_ERR_PARAM_INVALID),   # and bf16 caches
    (dict(in_dtype=3, Hcq=1544), mla.MLA_ERR_UNSUPPORTED),          # int8 size rules
    (dict(in_dtype=3, eps_x=-1.0), mla.MLA_ERR_PARAM_INVALID),
    (dict(x_quant_only=1), mla.MLA_ERR_PARAM_INVALID),              # the static scenario's option
    (dict(concat=2), mla.MLA_ERR_PARAM_INVALID),
    (dict(weights_nk=-1), mla.MLA_ERR_PARAM_INVALID),
    (dict(concat=1, in_dtype=1, query_dtype=1), mla.MLA_ERR_PARAM_INVALID),  # concatenated rows are bf16
    (dict(concat=1, in_dtype=2, cache_dtype=1), mla.MLA_ERR_PARAM_INVALID),
    (dict(query_dtype=1), mla.MLA_ERR_PARAM_INVALID),   # int8 q^N needs int8 inputs
    (dict(He=7164), mla.MLA_ERR_UNSUPPORTED),
    (dict(Dr=128), mla.MLA_ERR_UNSUPPORTED),
    (dict(Hckv=1024), mla.MLA_ERR_UNSUPPORTED),
    (dict(in_dtype=1, Hcq=1544), mla.MLA_ERR_UNSUPPORTED),
    (dict(in_dtype=1, Hckv=504), mla.MLA_ERR_UNSUPPORTED),
    (dict(in_dtype=1, Dr=56), mla.MLA_ERR_UNSUPPORTED),
    (dict(in_dtype=2, query_dtype=1), mla.MLA_ERR_PARAM_INVALID),   # int8 q^N: full quantisation only
    (dict(in_dtype=2, Hcq=1544), mla.MLA_ERR_UNSUPPORTED),
    (dict(in_dtype=2, D=120), mla.MLA_ERR_UNSUPPORTED),
    (dict(float_dtype=mla.MLA_FP16), mla.MLA_ERR_PARAM_INVALID),        # fp16: the static scenario only
    (dict(in_dtype=1, float_dtype=mla.MLA_FP16), mla.MLA_ERR_PARAM_INVALID),
    (dict(in_dtype=2, float_dtype=mla.MLA_FP16), mla.MLA_ERR_PARAM_INVALID),
    (dict(in_dtype=3, float_dtype=1), mla.MLA_ERR_PARAM_INVALID),
    (dict(in_dtype=3, float_dtype=5), mla.MLA_ERR_PARAM_INVALID),
    (dict(in_dtype=3, float_dtype=-1), mla.MLA_ERR_PARAM_INVALID),
    (dict(cache_dtype=1), mla.MLA_ERR_PARAM_INVALID),             # quantised caches: int8 scenarios only
    (dict(in_dtype=1, cache_dtype=2), mla.MLA_ERR_PARAM_INVALID),
])
def test_bad_descriptions(kw, code):
    assert mla.validate(model_desc(**kw)) == code
    assert mla.workspace_bytes(model_desc(**kw)) == 0


def test_bad_run_arguments():
    d = model_desc()
    assert mla.validate(d, fake_tensors(), 257) == mla.MLA_ERR_PARAM_INVALID   # T > max_tokens
    assert mla.validate(d, fake_tensors(), -1) == mla.MLA_ERR_PARAM_INVALID
    t = fake_tensors(); t["weight_uk"] = None; t["packed_weights"] = None
    assert mla.validate(d, t, 8) == mla.MLA_ERR_NULLPTR
    t = fake_tensors(); t["kv_cache"] = None
    assert mla.validate(d, t, 8) == mla.MLA_ERR_NULLPTR
    t = fake_tensors(); t["token_x"] = FAKE + 2
    assert mla.validate(d, t, 8) == mla.MLA_ERR_PARAM_INVALID                  # misaligned
    t = fake_tensors(); t["scale_x"] = FAKE
    assert mla.validate(d, t, 8) == mla.MLA_ERR_PARAM_INVALID                  # scale in bf16 mode
    d8 = model_desc(in_dtype=1, query_dtype=1)
    assert mla.validate(d8, fake_tensors(q8=False, in8=True), 8) == mla.MLA_ERR_NULLPTR
    assert mla.validate(d8, fake_tensors(q8=True, in8=False), 8) == mla.MLA_ERR_NULLPTR
    # smoothScalesCq belongs to the int8 weightUqQr scenarios
    assert mla.validate(d, fake_tensors(smooth=True), 8) == mla.MLA_ERR_PARAM_INVALID
    t = fake_tensors(q8=True, in8=True, smooth=True); t["smooth_scales_cq"] = FAKE + 2
    assert mla.validate(d8, t, 8) == mla.MLA_ERR_PARAM_INVALID                 # misaligned
    # partial quantisation: the weightUqQr scale alone
    dp = model_desc(in_dtype=mla.MLA_INT8_PARTIAL)
    t = fake_tensors(partial=True); t["scale_w_uq_qr"] = None
    assert mla.validate(dp, t, 8) == mla.MLA_ERR_NULLPTR
    t = fake_tensors(partial=True); t["scale_x"] = FAKE
    assert mla.validate(dp, t, 8) == mla.MLA_ERR_PARAM_INVALID
    # cache scales: exactly those of the int8 caches
    dk = model_desc(in_dtype=1, cache_dtype=1)
    assert mla.validate(dk, fake_tensors(in8=True), 8) == mla.MLA_ERR_NULLPTR          # no quantScaleCkv
    t = fake_tensors(in8=True, kvq=True); t["quant_scale_ckr"] = FAKE                 # kr stays bf16 here
    assert mla.validate(dk, t, 8) == mla.MLA_ERR_PARAM_INVALID
    dpk = model_desc(in_dtype=2, cache_dtype=1)
    t = fake_tensors(partial=True, kvq=True); t["quant_scale_ckr"] = None
    assert mla.validate(dpk, t, 8) == mla.MLA_ERR_NULLPTR
    t = fake_tensors(partial=True); t["quant_scale_ckv"] = FAKE                       # bf16 caches
    assert mla.validate(dp, t, 8) == mla.MLA_ERR_PARAM_INVALID
    # every tensor 16-byte aligned: the per-channel vectors are read in
    # 16-byte chunks, so a 4-byte aligned scale is refused too
    for f in ("scale_x", "scale_w_dq", "scale_w_uq_qr", "scale_w_dkv_kr", "smooth_scales_cq"):
        t = fake_tensors(q8=True, in8=True, smooth=True); t[f] = FAKE + 4
        assert mla.validate(d8, t, 8) == mla.MLA_ERR_PARAM_INVALID, f
    t = fake_tensors(True, True, kvq=True); t["quant_scale_ckv"] = FAKE + 4
    assert mla.validate(model_desc(in_dtype=1, query_dtype=1, cache_dtype=1), t, 8) == mla.MLA_ERR_PARAM_INVALID


def test_bad_static_and_concat_arguments():
    st = model_desc(in_dtype=mla.MLA_INT8_STATIC)
    for f in ("quant_scale_x", "quant_offset_x", "beta_cq", "quant_scale_cq", "quant_offset_cq", "gamma_x",
              "beta_x", "scale_w_dq", "scale_w_uq_qr", "scale_w_dkv_kr"):
        t = fake_tensors(static=True); t[f] = None
        assert mla.validate(st, t, 8) == mla.MLA_ERR_NULLPTR, f
    t = fake_tensors(static=True); t["scale_x"] = FAKE                            # x is quantised here
    assert mla.validate(st, t, 8) == mla.MLA_ERR_PARAM_INVALID
    t = fake_tensors(static=True, smooth=True)
    assert mla.validate(st, t, 8) == mla.MLA_ERR_PARAM_INVALID
    t = fake_tensors(static=True)                                                 # gamma0 without the norm
    assert mla.validate(model_desc(in_dtype=3, x_quant_only=1), t, 8) == mla.MLA_ERR_PARAM_INVALID
    for f in ("bias_dqkv", "bias_uq_qr", "beta_cq", "quant_scale_x", "quant_offset_cq"):
        t = fake_tensors(static=True); t[f] = FAKE + 4
        assert mla.validate(st, t, 8) == mla.MLA_ERR_PARAM_INVALID, f
    t = fake_tensors(static=True); t["gamma_x"] = FAKE + 8                        # read in 16-byte chunks
    assert mla.validate(st, t, 8) == mla.MLA_ERR_PARAM_INVALID
    for f in STATIC_ONLY:                                                         # other scenarios
        t = fake_tensors(); t[f] = FAKE
        assert mla.validate(model_desc(), t, 8) == mla.MLA_ERR_PARAM_INVALID, f
    # the concatenated layout has no q^R output or kr cache of its own
    dc = model_desc(concat=1)
    for f in ("query_rope_out", "kr_cache"):
        t = fake_tensors(concat=True); t[f] = FAKE
        assert mla.validate(dc, t, 8) == mla.MLA_ERR_PARAM_INVALID, f
    t = fake_tensors(concat=True); t["kv_cache"] = None
    assert mla.validate(dc, t, 8) == mla.MLA_ERR_NULLPTR
    t = fake_tensors(); t["query_rope_out"] = None
    assert mla.validate(model_desc(), t, 8) == mla.MLA_ERR_NULLPTR
    # transposed weights need the packed copy
    t = fake_tensors(); t["packed_weights"] = None
    assert mla.validate(model_desc(weights_nk=1), t, 8) == mla.MLA_ERR_UNSUPPORTED
    assert mla.validate(model_desc(), t, 8) == mla.MLA_OK
    # with the packed copy, the unpacked weights are optional
    for f in ("weight_dq", "weight_uq_qr", "weight_uk", "weight_dkv_kr"):
        t = fake_tensors(); t[f] = None
        assert mla.validate(model_desc(), t, 8) == mla.MLA_OK, f
        t["packed_weights"] = None
        assert mla.validate(model_desc(), t, 8) == mla.MLA_ERR_NULLPTR, f
        t = fake_tensors(); t[f] = FAKE + 4
        assert mla.validate(model_desc(), t, 8) == mla.MLA_ERR_PARAM_INVALID, f
    # and so do fp16 tensors
    t = fake_tensors(static=True); t["packed_weights"] = None
    assert mla.validate(model_desc(in_dtype=3, float_dtype=mla.MLA_FP16), t, 8) == mla.MLA_ERR_UNSUPPORTED
    assert mla.validate(model_desc(in_dtype=3), t, 8) == mla.MLA_OK
    # the reserved word must be zero
    d = model_desc(in_dtype=3)
    d.reserved = 1
    assert mla.validate(d) == mla.MLA_ERR_PARAM_INVALID


def test_empty_run_needs_no_tensors():
    # T = 0: empty tensors are allowed, nothing is checked or launched
    assert mla.validate(model_desc(), {}, 0) == mla.MLA_OK


def test_no_cache_blocks_needs_no_caches():
    t = fake_tensors(); t["kv_cache"] = None; t["kr_cache"] = None
    assert mla.validate(model_desc(block_num=0), t, 8) == mla.MLA_OK


def test_status_strings():
    for code in (0, 161001, 161002, 361001, 561002):
        assert mla.status_string(code) != "unknown status"


# ---- sparse flash attention over the caches --------------------------------
def sfa_desc(**kw):
    a = dict(N=128, D=512, Dr=64, block_num=4096, block_size=128, max_blocks=256, sparse_size=2048,
             sparse_block_size=1, max_tokens=32, scale=1 / 24)
    a.update(kw)
    return mla.make_sfa_desc(**a)


def sfa_tensors(concat=False, lse=True):
    t = {f: FAKE for f in mla.SFA_TENSOR_FIELDS}
    if concat:
        t["kr_cache"] = None
    if not lse:
        t["softmax_max"] = t["softmax_sum"] = None
    return t


def test_sfa_valid():
    assert mla.sfa_validate(sfa_desc()) == mla.MLA_OK
    assert mla.sfa_validate(sfa_desc(), sfa_tensors(), 32) == mla.MLA_OK
    assert mla.sfa_validate(sfa_desc(concat=1), sfa_tensors(concat=True, lse=False), 32) == mla.MLA_OK
    assert mla.sfa_validate(sfa_desc(N=3, D=64, Dr=32, sparse_block_size=4), sfa_tensors(), 1) == mla.MLA_OK
    assert mla.sfa_validate(sfa_desc(), {}, 0) == mla.MLA_OK


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), mla.MLA_ERR_PARAM_INVALID),
    (dict(block_size=0), mla.MLA_ERR_PARAM_INVALID),
    (dict(sparse_size=0), mla.MLA_ERR_PARAM_INVALID),
    (dict(concat=2), mla.MLA_ERR_PARAM_INVALID),
    (dict(scale=float("nan")), mla.MLA_ERR_PARAM_INVALID),
    (dict(D=520), mla.MLA_ERR_UNSUPPORTED),
    (dict(D=48), mla.MLA_ERR_UNSUPPORTED),
    (dict(Dr=16), mla.MLA_ERR_UNSUPPORTED),
    (dict(Dr=96), mla.MLA_ERR_UNSUPPORTED),
    (dict(N=129), mla.MLA_ERR_UNSUPPORTED),
    (dict(block_num=1 << 24, block_size=1024), mla.MLA_ERR_UNSUPPORTED),
])
def test_sfa_bad_descriptions(kw, code):
    assert mla.sfa_validate(sfa_desc(**kw)) == code


def test_sfa_bad_run_arguments():
    d = sfa_desc()
    assert mla.sfa_validate(d, sfa_tensors(), 33) == mla.MLA_ERR_PARAM_INVALID
    for f in ("query", "query_rope", "kv_cache", "kr_cache", "sparse_indices", "block_table", "seq_lens_kv",
              "attention_out"):
        t = sfa_tensors(); t[f] = None
        assert mla.sfa_validate(d, t, 8) == mla.MLA_ERR_NULLPTR, f
    t = sfa_tensors(); t["query"] = FAKE + 8
    assert mla.sfa_validate(d, t, 8) == mla.MLA_ERR_PARAM_INVALID
    assert mla.sfa_validate(sfa_desc(concat=1), sfa_tensors(), 8) == mla.MLA_ERR_PARAM_INVALID   # kr given


@pytest.mark.parametrize("value", ["0", "-3", "abc", "12x", "", str((1 << 20) + 1)])
def test_bad_poll_limit_is_refused(value, monkeypatch):
    # create reads MLA_PROLOG_FUSED_SPIN before it touches a device, and
    # refuses any value that is not a whole number in [1, 2^20]
    monkeypatch.setenv("MLA_PROLOG_FUSED_SPIN", value)
    h = ctypes.c_void_p()
    assert mla.lib().mla_prolog_create(ctypes.byref(model_desc()), ctypes.byref(h)) == mla.MLA_ERR_PARAM_INVALID
    assert not h.value


def test_poll_limit_setter_needs_a_handle():
    assert mla.lib().mla_prolog_set_poll_limit(None, 5) == mla.MLA_ERR_NULLPTR


def test_noalloc_refuses_what_it_cannot_take():
    # host-side refusals come before any device call: a workspace beyond the
    # 64 MiB array, the debugging check of cacheIndex, the usual validation
    L = mla.lib()
    t = mla.make_tensors(fake_tensors())
    big = model_desc(max_tokens=4096)
    assert L.mla_prolog_run_noalloc(ctypes.byref(big), ctypes.byref(t), 4096, None) == mla.MLA_ERR_PARAM_INVALID
    chk = model_desc(check_index=1)
    assert L.mla_prolog_run_noalloc(ctypes.byref(chk), ctypes.byref(t), 32, None) == mla.MLA_ERR_PARAM_INVALID
    assert L.mla_prolog_run_noalloc(ctypes.byref(model_desc()), ctypes.byref(t), 257, None) == mla.MLA_ERR_PARAM_INVALID
    assert L.mla_prolog_run_noalloc(ctypes.byref(model_desc()), None, 32, None) == mla.MLA_ERR_NULLPTR
    assert L.mla_prolog_run_noalloc(ctypes.byref(model_desc()), ctypes.byref(t), 0, None) == mla.MLA_OK
