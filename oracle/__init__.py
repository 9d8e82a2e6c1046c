"""CPU oracle of the MLA prolog (aclnnMlaPrologV2WeightNz, "Function",
formulas) -- TEST INFRASTRUCTURE ONLY.

The arithmetic lives in ``mla_oracle.cpp`` (plain loops, double precision,
explicit rounding points); this module only loads it with ctypes and marshals
numpy arrays.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it; the HIP library and its binding never do.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "mla_oracle.cpp")
#: the built oracle; MLA_ORACLE_LIBRARY names another build of the same
#: source (the sanitizer test builds one with AddressSanitizer and UBSan)
LIBRARY = os.environ.get("MLA_ORACLE_LIBRARY") or os.path.join(HERE, "libmla_oracle.so")
BUILD_CMD = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-shared",
             "-fPIC", "-pthread", SOURCE, "-o", LIBRARY]


def build() -> str:
    """Compile the oracle with the host compiler (always recompiles)."""
    subprocess.run(BUILD_CMD, check=True)
    return LIBRARY


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class Problem(ctypes.Structure):
    _fields_ = [
        ("T", _I64), ("He", _I64), ("Hcq", _I64), ("Hckv", _I64), ("N", _I64), ("D", _I64),
        ("Dr", _I64), ("block_num", _I64), ("block_size", _I64),
        ("eps_cq", ctypes.c_double), ("eps_ckv", ctypes.c_double),
        ("quant_in", ctypes.c_int32), ("query_int8", ctypes.c_int32),
        ("round_intermediates", ctypes.c_int32), ("mutation", ctypes.c_int32),
        ("quant_uq", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("x", _P), ("w_dq", _P), ("w_uq_qr", _P), ("w_uk", _P), ("w_dkv_kr", _P),
        ("gamma_cq", _P), ("gamma_ckv", _P), ("rope_sin", _P), ("rope_cos", _P),
        ("cache_index", _P), ("kv_cache", _P), ("kr_cache", _P),
        ("scale_x", _P), ("scale_w_dq", _P), ("scale_w_uq_qr", _P), ("scale_w_dkv_kr", _P),
        ("smooth_cq", _P), ("tokens", _P), ("n_tokens", _I64),
        ("query_out", _P), ("query_rope_out", _P), ("dequant_scale_q_nope", _P),
        ("kv_rows", _P), ("kr_rows", _P),
        ("y_out", _P), ("cq_out", _P), ("u_out", _P), ("qn_out", _P),
        ("kv_int8", ctypes.c_int32), ("kr_int8", ctypes.c_int32),
        ("quant_scale_ckv", _P), ("quant_scale_ckr", _P), ("ckv_out", _P), ("kr_out", _P),
        ("static_quant", ctypes.c_int32), ("x_norm", ctypes.c_int32), ("concat", ctypes.c_int32),
        ("weight_nk", ctypes.c_int32), ("eps_x", ctypes.c_double),
        ("gamma_x", _P), ("beta_x", _P), ("quant_scale_x", _P), ("quant_offset_x", _P),
        ("bias_dqkv", _P), ("beta_cq", _P), ("quant_scale_cq", _P), ("quant_offset_cq", _P),
        ("bias_uq_qr", _P),
        ("fp16", ctypes.c_int32), ("pad2_", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        L = ctypes.CDLL(LIBRARY)
        L.mla_oracle_run.argtypes = [ctypes.POINTER(Problem), ctypes.c_int]
        L.mla_oracle_run.restype = ctypes.c_int
        L.mla_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.mla_oracle_bf16_value.restype = ctypes.c_double
        L.mla_oracle_bf16_bits.argtypes = [ctypes.c_double]
        L.mla_oracle_bf16_bits.restype = ctypes.c_uint16
        L.mla_oracle_f16_value.argtypes = [ctypes.c_uint16]
        L.mla_oracle_f16_value.restype = ctypes.c_double
        L.mla_oracle_f16_bits.argtypes = [ctypes.c_double]
        L.mla_oracle_f16_bits.restype = ctypes.c_uint16
        L.mla_oracle_rmsnorm.argtypes = [_P, _P, _I64, ctypes.c_double, _P]
        L.mla_oracle_rope.argtypes = [_P, _P, _P, _I64, _P]
        L.mla_oracle_quant_int8.argtypes = [_P, _I64, _P, _P]
        L.mla_oracle_quant_static_asym.argtypes = [_P, _I64, ctypes.c_float, ctypes.c_int, _P]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# ---- single building blocks (for the pins) ---------------------------------
def bf16_value(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    L = lib()
    return np.array([L.mla_oracle_bf16_value(int(v)) for v in b.ravel()]).reshape(b.shape)


def bf16_bits(values) -> np.ndarray:
    v = np.asarray(values, dtype=np.float64)
    L = lib()
    return np.array([L.mla_oracle_bf16_bits(float(x)) for x in v.ravel()],
                    dtype=np.uint16).reshape(v.shape)


def f16_value(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    L = lib()
    return np.array([L.mla_oracle_f16_value(int(v)) for v in b.ravel()]).reshape(b.shape)


def f16_bits(values) -> np.ndarray:
    v = np.asarray(values, dtype=np.float64)
    L = lib()
    return np.array([L.mla_oracle_f16_bits(float(x)) for x in v.ravel()],
                    dtype=np.uint16).reshape(v.shape)


def rmsnorm(v, gamma, eps: float) -> np.ndarray:
    v, g = _f64(v), _f64(gamma)
    out = np.empty_like(v)
    lib().mla_oracle_rmsnorm(_ptr(v), _ptr(g), v.size, float(eps), _ptr(out))
    return out


def rope(v, cos, sin) -> np.ndarray:
    v, c, s = _f64(v), _f64(cos), _f64(sin)
    out = np.empty_like(v)
    lib().mla_oracle_rope(_ptr(v), _ptr(c), _ptr(s), v.size, _ptr(out))
    return out


def quant_int8(v):
    v = _f64(v)
    q = np.empty(v.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().mla_oracle_quant_int8(_ptr(v), v.size, _ptr(q), _ptr(s))
    return q, float(s[0])


def quant_static_asym(v, scale: float, offset: int) -> np.ndarray:
    """The preprocess page's static asymmetric int8 codes of v."""
    v = _f64(v)
    q = np.empty(v.size, dtype=np.int8)
    lib().mla_oracle_quant_static_asym(_ptr(v), v.size, float(scale), int(offset), _ptr(q))
    return q.reshape(v.shape)


# ---- the whole prolog ---------------------------------------------------------
def run(inp: Dict[str, object], tokens: Optional[Sequence[int]] = None,
        round_intermediates: bool = True, query_int8: Optional[bool] = None,
        mutation: int = 0, intermediates: bool = False, caches: bool = True,
        nthreads: int = 0) -> Dict[str, np.ndarray]:
    """Run the oracle on the host arrays of ``synth.make_inputs``.

    ``inp["quant"]`` is the int8 full-quantisation scenario, ``inp["partial"]``
    the partial one (only weightUqQr int8); ``inp["smooth_scales_cq"]``, when
    present, is smoothScalesCq; ``inp["kv_quant"]`` quantises the kv cache
    (and, with partial quantisation, the kr cache) with quantScaleCkv /
    quantScaleCkr.  ``inp["preprocess"]`` is the MLA preprocess page's static
    scenario (bf16 x quantised by RmsNormQuant, int8 weights with deScale and
    bias, c^Q quantised the same way; ``inp["x_norm"]`` False quantises x
    without its norm); ``inp["concat"]`` its concatenated layout (queryOut
    rows q^N | q^R, kvCache rows c^KV | k^R, no query_rope_out / kr_cache);
    ``inp["weight_nk"]`` weights given (n, k); ``inp["fp16"]`` (static scenario
    only) its FLOAT16 input, every 16-bit float tensor and rounding fp16.  ``tokens`` selects the rows to compute (tokens are independent); row r of
    every output holds token ``tokens[r]``.  With ``caches`` the returned
    ``kv_cache``/``kr_cache`` are copies of the input caches with the computed
    rows written at their cacheIndex slots.
    """
    d = inp["dims"]
    T = int(inp["T"])
    quant = bool(inp["quant"])
    static = bool(inp.get("preprocess", False))
    concat = bool(inp.get("concat", False))
    quant_uq = quant or bool(inp.get("partial", False))
    q8 = quant if query_int8 is None else bool(query_int8)
    kv8 = bool(inp.get("kv_quant", False))
    kr8 = kv8 and not quant
    keep = []

    def arr(a, dtype):
        a = np.ascontiguousarray(a, dtype=dtype)
        keep.append(a)
        return a

    x = arr(inp["token_x"], np.int8 if quant else np.uint16)
    wdq = arr(inp["weight_dq"], np.int8 if quant or static else np.uint16)
    wuq = arr(inp["weight_uq_qr"], np.int8 if quant_uq or static else np.uint16)
    wdkv = arr(inp["weight_dkv_kr"], np.int8 if quant or static else np.uint16)
    wuk = arr(inp["weight_uk"], np.uint16)
    gcq = arr(inp["rmsnorm_gamma_cq"], np.uint16)
    gckv = arr(inp["rmsnorm_gamma_ckv"], np.uint16)
    sin = arr(inp["rope_sin"], np.uint16)
    cos = arr(inp["rope_cos"], np.uint16)
    idx = arr(inp["cache_index"], np.int64)
    if tokens is None:
        rows = None
        n = T
    else:
        rows = arr(np.asarray(tokens), np.int64)
        n = rows.size
    N, Hckv, Dr, Hcq, D = d.N, d.Hckv, d.Dr, d.Hcq, d.D
    out = {
        "query_out": np.zeros((n, N, Hckv + Dr if concat else Hckv), dtype=np.int8 if q8 else np.uint16),
        "kv_rows": np.zeros((n, Hckv), dtype=np.int8 if kv8 else np.uint16),
        "kr_rows": np.zeros((n, Dr), dtype=np.int8 if kr8 else np.uint16),
    }
    if not concat:
        out["query_rope_out"] = np.zeros((n, N, Dr), dtype=np.uint16)
    if q8:
        out["dequant_scale_q_nope"] = np.zeros((n, N), dtype=np.float32)
    if intermediates:
        out["y"] = np.zeros((n, Hcq + Hckv + Dr))
        out["c_q"] = np.zeros((n, Hcq))
        out["u"] = np.zeros((n, N * (D + Dr)))
        out["q_n"] = np.zeros((n, N, Hckv))
        out["c_kv"] = np.zeros((n, Hckv))
        out["k_r"] = np.zeros((n, Dr))
    kv = kr = None
    if caches and "kv_cache" in inp:
        kv = np.array(inp["kv_cache"], dtype=np.int8 if kv8 else np.uint16, copy=True)
        kr = None if concat else np.array(inp["kr_cache"], dtype=np.int8 if kr8 else np.uint16, copy=True)

    p = Problem()
    p.T, p.He, p.Hcq, p.Hckv, p.N, p.D, p.Dr = T, d.He, Hcq, Hckv, N, D, Dr
    p.block_num, p.block_size = int(inp["block_num"]), int(inp["block_size"])
    p.eps_cq, p.eps_ckv = float(inp["eps_cq"]), float(inp["eps_ckv"])
    p.quant_in, p.query_int8, p.quant_uq = int(quant), int(q8), int(quant_uq)
    p.round_intermediates, p.mutation = int(bool(round_intermediates)), int(mutation)
    p.x, p.w_dq, p.w_uq_qr, p.w_uk, p.w_dkv_kr = _ptr(x), _ptr(wdq), _ptr(wuq), _ptr(wuk), _ptr(wdkv)
    p.gamma_cq, p.gamma_ckv, p.rope_sin, p.rope_cos = _ptr(gcq), _ptr(gckv), _ptr(sin), _ptr(cos)
    p.cache_index, p.kv_cache, p.kr_cache = _ptr(idx), _ptr(kv), _ptr(kr)
    if quant:
        p.scale_x = _ptr(arr(inp["dequant_scale_x"], np.float32))
        p.scale_w_dq = _ptr(arr(inp["dequant_scale_w_dq"], np.float32))
        p.scale_w_uq_qr = _ptr(arr(inp["dequant_scale_w_uq_qr"], np.float32))
        p.scale_w_dkv_kr = _ptr(arr(inp["dequant_scale_w_dkv_kr"], np.float32))
    elif quant_uq or static:
        p.scale_w_uq_qr = _ptr(arr(inp["dequant_scale_w_uq_qr"], np.float32))
    if static:
        p.static_quant, p.x_norm = 1, int(bool(inp.get("x_norm", True)))
        p.scale_w_dq = _ptr(arr(inp["dequant_scale_w_dq"], np.float32))
        p.scale_w_dkv_kr = _ptr(arr(inp["dequant_scale_w_dkv_kr"], np.float32))
        p.eps_x = float(inp["eps_x"])
        for f, key, dt in (("gamma_x", "rmsnorm_gamma_x", np.uint16), ("beta_x", "rmsnorm_beta_x", np.uint16),
                           ("quant_scale_x", "quant_scale_x", np.uint16),
                           ("quant_offset_x", "quant_offset_x", np.int8),
                           ("bias_dqkv", "bias_dqkv", np.int32), ("beta_cq", "rmsnorm_beta_cq", np.uint16),
                           ("quant_scale_cq", "quant_scale_cq", np.uint16),
                           ("quant_offset_cq", "quant_offset_cq", np.int8),
                           ("bias_uq_qr", "bias_uq_qr", np.int32)):
            if inp.get(key) is not None:
                setattr(p, f, _ptr(arr(inp[key], dt)))
    p.concat, p.weight_nk = int(concat), int(bool(inp.get("weight_nk", False)))
    p.fp16 = int(bool(inp.get("fp16", False)))
    if inp.get("smooth_scales_cq") is not None:
        p.smooth_cq = _ptr(arr(inp["smooth_scales_cq"], np.float32))
    p.kv_int8, p.kr_int8 = int(kv8), int(kr8)
    if kv8:
        p.quant_scale_ckv = _ptr(arr(inp["quant_scale_ckv"], np.float32))
    if kr8:
        p.quant_scale_ckr = _ptr(arr(inp["quant_scale_ckr"], np.float32))
    p.tokens, p.n_tokens = _ptr(rows), n
    p.query_out, p.query_rope_out = _ptr(out["query_out"]), _ptr(out.get("query_rope_out"))
    p.dequant_scale_q_nope = _ptr(out.get("dequant_scale_q_nope"))
    p.kv_rows, p.kr_rows = _ptr(out["kv_rows"]), _ptr(out["kr_rows"])
    if intermediates:
        p.y_out, p.cq_out, p.u_out, p.qn_out = (_ptr(out["y"]), _ptr(out["c_q"]),
                                                _ptr(out["u"]), _ptr(out["q_n"]))
        p.ckv_out, p.kr_out = _ptr(out["c_kv"]), _ptr(out["k_r"])
    rc = lib().mla_oracle_run(ctypes.byref(p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    if kv is not None:
        out["kv_cache"] = kv
        if kr is not None:
            out["kr_cache"] = kr
    return out


# ---- the sparse flash attention consumer of the caches ---------------------
class SfaProblem(ctypes.Structure):
    _fields_ = [
        ("T", _I64), ("N", _I64), ("D", _I64), ("Dr", _I64), ("block_num", _I64), ("block_size", _I64),
        ("K", _I64), ("sparse_block_size", _I64), ("max_blocks", _I64), ("scale", ctypes.c_double),
        ("concat", ctypes.c_int32), ("mutation", ctypes.c_int32),
        ("query", _P), ("query_rope", _P), ("kv", _P), ("kr", _P), ("indices", _P),
        ("block_table", _P), ("seq_lens", _P), ("out", _P), ("softmax_max", _P), ("softmax_sum", _P),
        ("out_f64", _P), ("tokens", _P), ("n_tokens", _I64),
    ]


def sfa(inp: Dict[str, object], tokens: Optional[Sequence[int]] = None, mutation: int = 0,
        nthreads: int = 0) -> Dict[str, np.ndarray]:
    """Sparse flash attention (MLA-absorb, one decode query per batch) on the
    host arrays of ``synth.sfa.make_sfa_inputs``: attention_out (bf16 bits),
    softmax_max, softmax_sum and the unrounded out_f64 of the selected rows."""
    L = lib()
    if not getattr(L, "_sfa_ready", False):
        L.mla_oracle_sfa.argtypes = [ctypes.POINTER(SfaProblem), ctypes.c_int]
        L.mla_oracle_sfa.restype = ctypes.c_int
        L._sfa_ready = True
    keep = []

    def arr(a, dtype):
        a = np.ascontiguousarray(a, dtype=dtype)
        keep.append(a)
        return a

    T, N, D, Dr = int(inp["T"]), int(inp["N"]), int(inp["D"]), int(inp["Dr"])
    rows = None if tokens is None else arr(np.asarray(tokens), np.int64)
    n = T if rows is None else rows.size
    out = {"attention_out": np.zeros((n, N, D), np.uint16), "softmax_max": np.zeros((n, N), np.float32),
           "softmax_sum": np.zeros((n, N), np.float32), "out_f64": np.zeros((n, N, D))}
    p = SfaProblem()
    p.T, p.N, p.D, p.Dr = T, N, D, Dr
    p.block_num, p.block_size = int(inp["block_num"]), int(inp["block_size"])
    p.K, p.sparse_block_size, p.max_blocks = int(inp["K"]), int(inp["sparse_block_size"]), int(inp["max_blocks"])
    p.scale, p.concat, p.mutation = float(inp["scale"]), int(bool(inp["concat"])), int(mutation)
    p.query, p.query_rope = _ptr(arr(inp["query"], np.uint16)), _ptr(arr(inp["query_rope"], np.uint16))
    p.kv = _ptr(arr(inp["kv_cache"], np.uint16))
    if not inp["concat"]:
        p.kr = _ptr(arr(inp["kr_cache"], np.uint16))
    p.indices, p.block_table = _ptr(arr(inp["indices"], np.int32)), _ptr(arr(inp["block_table"], np.int32))
    p.seq_lens = _ptr(arr(inp["seq_lens"], np.int32))
    p.out, p.softmax_max, p.softmax_sum = (_ptr(out["attention_out"]), _ptr(out["softmax_max"]),
                                           _ptr(out["softmax_sum"]))
    p.out_f64 = _ptr(out["out_f64"])
    p.tokens, p.n_tokens = _ptr(rows), n
    if L.mla_oracle_sfa(ctypes.byref(p), int(nthreads)) != 0:
        raise ValueError("oracle rejected the problem")
    return out
