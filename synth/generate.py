"""Counter-based, platform-independent synthetic inputs for the MLA prolog.

Every value is a pure function of (seed, tensor id, element index): element i of
tensor stream k is ``splitmix64_mix(key_k + (i + 1) * GOLDEN)`` with
``key_k = splitmix64_mix((seed << 16) | k)``.  Normals use Box-Muller on the
uniforms of counters 2i and 2i+1; ``N(0, 1/sqrt(K))`` is read as standard
deviation ``1/sqrt(K)`` with K the reduction length of that weight.  bf16
tensors are returned as their uint16 bit patterns (rounded to nearest even from
the drawn value), int8 tensors as int8, scales as float32.

The shapes, distributions and cache geometry are those of the MLA prolog
operator's parameter table (aclnnMlaPrologV2WeightNz, "Parameters" and
"Constraints"): tokenX (T, He), weightDq (He, Hcq), weightUqQr
(Hcq, N*(D+Dr)), weightUk (N, D, Hckv), weightDkvKr (He, Hckv+Dr), gammas,
ropeSin/ropeCos (T, Dr), cacheIndex (T) int64, caches
(BlockNum, BlockSize, 1, Hckv|Dr).

weightUqQr is packed head-interleaved: column h*(D+Dr)+j holds W^UQ column
h*D+j for j < D and W^QR column h*Dr+(j-D) otherwise.  weightDkvKr holds W^DKV
in columns [0, Hckv) and W^KR in [Hckv, Hckv+Dr).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 20

#: bf16 bit pattern every cache slot starts with (a quiet NaN whose payload no
#: arithmetic produces), so that untouched slots can be checked bitwise.
SENTINEL_BF16 = np.uint16(0x7FA5)
#: the byte an int8 (quantised) cache slot starts with
SENTINEL_I8 = np.int8(-77)
#: fp16 bit pattern an fp16 cache slot starts with (a quiet NaN with a payload)
SENTINEL_F16 = np.uint16(0x7E55)

# one random stream per tensor
_STREAM = {
    "x": 1, "w_dq": 2, "w_uq": 3, "w_qr": 4, "w_uk": 5, "w_dkv": 6, "w_kr": 7,
    "gamma_cq": 8, "gamma_ckv": 9, "pos": 10, "slots": 11, "sx": 12,
    "sw_dq": 13, "sw_uq_qr": 14, "sw_dkv_kr": 15, "blocks": 16, "smooth_cq": 17,
    "qs_ckv": 18, "qs_ckr": 19, "gamma_x": 20, "beta_x": 21, "qs_x": 22, "qo_x": 23,
    "bias_dqkv": 24, "beta_cq": 25, "qs_cq": 26, "qo_cq": 27, "bias_uq": 28,
    # the sparse attention consumer
    "sfa_q": 40, "sfa_qr": 41, "sfa_kv": 42, "sfa_kr": 43, "sfa_len": 44, "sfa_blocks": 45,
    "sfa_idx": 46,
}


def _mix(z: np.ndarray) -> np.ndarray:
    """splitmix64 finaliser, in place on a uint64 array."""
    t = np.empty_like(z)
    with np.errstate(over="ignore"):
        np.right_shift(z, np.uint64(30), out=t); np.bitwise_xor(z, t, out=z); np.multiply(z, _M1, out=z)
        np.right_shift(z, np.uint64(27), out=t); np.bitwise_xor(z, t, out=z); np.multiply(z, _M2, out=z)
        np.right_shift(z, np.uint64(31), out=t); np.bitwise_xor(z, t, out=z)
    return z


def _key(seed: int, stream: str) -> np.uint64:
    return _mix(np.array([(int(seed) << 16) | _STREAM[stream]], dtype=np.uint64))[0]


def _bits(seed: int, stream: str, start: int, n: int) -> np.ndarray:
    """Raw 64-bit draws for counters [start, start+n) of one stream."""
    key = _key(seed, stream)
    z = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        np.multiply(z, GOLDEN, out=z)
        np.add(z, key, out=z)
    return _mix(z)


def _uniform(seed: int, stream: str, n: int, start: int = 0) -> np.ndarray:
    """U[0,1) in float64 with 53 random bits."""
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        b = _bits(seed, stream, start + s, m)
        np.right_shift(b, np.uint64(11), out=b)
        np.multiply(b, 2.0 ** -53, out=out[s:s + m], casting="unsafe")
    return out


def _normal(seed: int, stream: str, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        b = _bits(seed, stream, 2 * s, 2 * m)
        np.right_shift(b, np.uint64(11), out=b)
        u = b.astype(np.float64)
        u1 = u[0::2]
        u1 += 1.0
        u1 *= 2.0 ** -53                      # (0, 1]
        u2 = u[1::2]
        u2 *= 2.0 * np.pi * 2.0 ** -53        # [0, 2pi)
        np.log(u1, out=u1)
        u1 *= -2.0
        np.sqrt(u1, out=u1)
        np.cos(u2, out=u2)
        np.multiply(u1, u2, out=out[s:s + m])
    return out


def _int8_uniform(seed: int, stream: str, n: int) -> np.ndarray:
    """Integers uniform on [-127, 127]."""
    out = np.empty(n, dtype=np.int8)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        u = _uniform(seed, stream, m, start=s)
        u *= 255.0
        np.floor(u, out=u)
        u -= 127.0
        out[s:s + m] = u.astype(np.int8)
    return out


def _to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round drawn float64 values to bf16 bit patterns (via float32, nearest even).

    The drawn values are finite, so the uint32 sums below cannot overflow."""
    flat = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    for s in range(0, flat.size, _CHUNK):
        b = flat[s:s + _CHUNK].view(np.uint32)
        lsb = np.right_shift(b, np.uint32(16))
        np.bitwise_and(lsb, np.uint32(1), out=lsb)
        lsb += b
        lsb += np.uint32(0x7FFF)
        np.right_shift(lsb, np.uint32(16), out=lsb)
        out[s:s + _CHUNK] = lsb
    return out.reshape(np.shape(v))


def _to_f16_bits(v: np.ndarray) -> np.ndarray:
    """Round drawn float64 values to fp16 bit patterns (nearest even, directly
    from float64)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


@dataclass(frozen=True)
class Dims:
    """Model sizes in the pages' notation."""
    He: int
    Hcq: int
    Hckv: int
    N: int
    D: int
    Dr: int


MODEL = Dims(He=7168, Hcq=1536, Hckv=512, N=128, D=128, Dr=64)
TINY = Dims(He=256, Hcq=64, Hckv=32, N=2, D=16, Dr=8)
# the tiny shape with Dr = 16: an int8 weightUqQr moves in 16-column chunks
TINY_Q = Dims(He=256, Hcq=64, Hckv=32, N=2, D=16, Dr=16)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    dims: Dims
    block_num: int
    block_size: int
    quant: bool           # int8 full-quant inputs and an int8 q^N output
    positions: str        # "uniform:<P>" or "prefill:<seqs>x<len>"
    seed: int
    eps: float = 1e-6
    partial: bool = False  # partial quantisation: only weightUqQr int8 (+ its scale)
    smooth: bool = False   # draw smoothScalesCq (int8 weightUqQr scenarios only)
    kv_quant: bool = False  # int8 kv cache (and, partially quantised, int8 kr cache)
    # the MLA preprocess page's static scenario: bf16 x quantised by
    # RmsNormQuant (x_norm False: quantised as is), int8 weights with
    # per-channel deScale and int32 bias, c^Q quantised the same way
    preprocess: bool = False
    x_norm: bool = True
    concat: bool = False     # cacheMode 0: queryOut q^N | q^R, kvCache c^KV | k^R
    weight_nk: bool = False  # weights given transposed, (n, k) row-major
    fp16: bool = False       # static scenario: FLOAT16 input (every 16-bit float tensor fp16)

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=T)


WORKLOADS: Dict[str, Workload] = {
    "tiny_t4": Workload("tiny_t4", 4, TINY, 4, 16, False, "uniform:64", 20260),
    "decode_t32": Workload("decode_t32", 32, MODEL, 1024, 128, False, "uniform:32768", 20261),
    "decode_t256": Workload("decode_t256", 256, MODEL, 4096, 128, False, "uniform:32768", 20262),
    "prefill_t8192": Workload("prefill_t8192", 8192, MODEL, 1024, 128, False, "prefill:2x4096", 20263),
    "int8_decode_t128": Workload("int8_decode_t128", 128, MODEL, 1024, 128, True, "uniform:32768", 20264),
    "tiny_partial_t4": Workload("tiny_partial_t4", 4, TINY_Q, 4, 16, False, "uniform:64", 20265,
                                partial=True, smooth=True),
    "partial_decode_t32": Workload("partial_decode_t32", 32, MODEL, 1024, 128, False, "uniform:32768",
                                   20266, partial=True, smooth=True),
    "int8_kvq_decode_t128": Workload("int8_kvq_decode_t128", 128, MODEL, 1024, 128, True, "uniform:32768",
                                     20267, kv_quant=True),
    "tiny_pre_t4": Workload("tiny_pre_t4", 4, TINY_Q, 4, 16, False, "uniform:64", 20268,
                            preprocess=True, concat=True, weight_nk=True),
    "pre_decode_t32": Workload("pre_decode_t32", 32, MODEL, 1024, 128, False, "uniform:32768", 20269,
                               preprocess=True, concat=True, weight_nk=True),
    # the static scenario with the preprocess page's FLOAT16 input
    "tiny_pre_f16_t4": Workload("tiny_pre_f16_t4", 4, TINY_Q, 4, 16, False, "uniform:64", 20270,
                                preprocess=True, concat=True, weight_nk=True, fp16=True),
    "pre_f16_decode_t32": Workload("pre_f16_decode_t32", 32, MODEL, 1024, 128, False, "uniform:32768", 20271,
                                   preprocess=True, concat=True, weight_nk=True, fp16=True),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _positions_and_slots(wl: Workload):
    T, nslots = wl.T, wl.block_num * wl.block_size
    kind, arg = wl.positions.split(":")
    if kind == "uniform":
        P = int(arg)
        pos = np.floor(_uniform(wl.seed, "pos", T) * P).astype(np.int64)
        if T > nslots:
            raise ValueError("more tokens than cache slots")
        order = np.argsort(_bits(wl.seed, "slots", 0, nslots), kind="stable")
        slots = order[:T].astype(np.int64)
        return pos, slots
    # prefill: sequences of consecutive positions 0..L-1, each given distinct
    # random blocks and filling them slot by slot
    nseq, L = (int(v) for v in arg.split("x"))
    if nseq * L != T:
        raise ValueError("prefill layout does not match T")
    per_seq = -(-L // wl.block_size)
    if nseq * per_seq > wl.block_num:
        raise ValueError("cache too small for the prefill layout")
    blocks = np.argsort(_bits(wl.seed, "blocks", 0, wl.block_num), kind="stable")
    blocks = blocks[:nseq * per_seq].reshape(nseq, per_seq)
    p = np.arange(L, dtype=np.int64)
    pos = np.tile(p, nseq)
    slots = np.concatenate([blocks[s][p // wl.block_size] * wl.block_size + p % wl.block_size
                            for s in range(nseq)]).astype(np.int64)
    return pos, slots


def rope_tables(pos: np.ndarray, Dr: int, base: float = 10000.0, fp16: bool = False):
    """Rotate-half sin/cos tables (bf16 bits, or fp16), one row per token:
    angle pos * base^(-2i/Dr) for i < Dr/2, repeated for the second half."""
    half = Dr // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / Dr)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    to = _to_f16_bits if fp16 else _to_bf16_bits
    return to(np.sin(ang)), to(np.cos(ang))


def make_inputs(wl: Workload, T: Optional[int] = None, with_caches: bool = True,
                unpacked: bool = False) -> Dict[str, object]:
    """All operator inputs for workload ``wl`` (optionally with T overridden).

    Token-dependent tensors are drawn for the workload's own T and then cut to
    the requested T, so a smaller T is a prefix of the full workload.  With
    ``unpacked`` the four weights that the operator takes packed in pairs are
    also returned on their own (weight_uq, weight_qr, weight_dkv, weight_kr).
    """
    d = wl.dims
    full_T = wl.T
    T = full_T if T is None else int(T)
    if T > full_T:
        wl = wl.with_tokens(T)
        full_T = T
    s = wl.seed
    He, Hcq, Hckv, N, D, Dr = d.He, d.Hcq, d.Hckv, d.N, d.D, d.Dr
    out: Dict[str, object] = {"workload": wl.name, "T": T, "dims": d,
                              "block_num": wl.block_num, "block_size": wl.block_size,
                              "quant": wl.quant, "partial": wl.partial, "kv_quant": wl.kv_quant,
                              "preprocess": wl.preprocess, "x_norm": wl.x_norm, "concat": wl.concat,
                              "weight_nk": wl.weight_nk, "fp16": wl.fp16,
                              "eps_cq": wl.eps, "eps_ckv": wl.eps, "eps_x": wl.eps}
    if wl.partial and wl.quant:
        raise ValueError("a workload is either fully or partially quantised")
    if wl.smooth and not (wl.quant or wl.partial):
        raise ValueError("smoothScalesCq belongs to the int8 weightUqQr scenarios")
    if wl.kv_quant and not (wl.quant or wl.partial):
        raise ValueError("cache quantisation belongs to the int8 scenarios")
    if wl.preprocess and (wl.quant or wl.partial or wl.smooth or wl.kv_quant):
        raise ValueError("the static scenario has its own quantisation")
    if wl.concat and (wl.quant or wl.kv_quant):
        raise ValueError("the concatenated layout holds bf16 rows")
    if wl.fp16 and not wl.preprocess:
        raise ValueError("the FLOAT16 input belongs to the static scenario")
    # the 16-bit float format of x, the gammas, betas and quant scales, the
    # rope tables, W^UK and the caches
    fbits = _to_f16_bits if wl.fp16 else _to_bf16_bits

    pos, slots = _positions_and_slots(wl)
    pos, slots = pos[:T], slots[:T]
    out["positions"] = pos
    out["cache_index"] = np.ascontiguousarray(slots, dtype=np.int64)
    out["rope_sin"], out["rope_cos"] = rope_tables(pos, Dr, fp16=wl.fp16)

    def gamma(stream, n):
        return fbits(0.5 + _uniform(s, stream, n))

    out["rmsnorm_gamma_cq"] = gamma("gamma_cq", Hcq)
    out["rmsnorm_gamma_ckv"] = gamma("gamma_ckv", Hckv)

    def head_interleave(wuq, wqr):
        a = wuq.reshape(Hcq, N, D)
        b = wqr.reshape(Hcq, N, Dr)
        return np.ascontiguousarray(np.concatenate([a, b], axis=2).reshape(Hcq, N * (D + Dr)))

    def static_scale(stream):
        # one bf16 quantScale in [12, 24): the normalised values are O(1), so
        # codes reach about +-100 and the largest saturate
        return fbits(12.0 + 12.0 * _uniform(s, stream, 1))

    def static_offset(stream):
        return np.floor(-4.0 + 9.0 * _uniform(s, stream, 1)).astype(np.int8)

    def descale(stream, n, K):
        # y = (acc + bias) * deScale is O(1): the codes are ~18 rms, the
        # weights ~73, so acc is about sqrt(K) * 1300
        return ((0.5 + _uniform(s, stream, n)) / (np.sqrt(K) * 1300.0)).astype(np.float32)

    def bias(stream, w_kn, offset):
        # the offset's share, -offset * sum_k W[k, n], plus a small term
        comp = -int(offset[0]) * w_kn.astype(np.int64).sum(axis=0)
        extra = np.floor(-2000.0 + 4000.0 * _uniform(s, stream, w_kn.shape[1])).astype(np.int64)
        return (comp + extra).astype(np.int32)

    if wl.preprocess:
        out["token_x"] = fbits(_normal(s, "x", full_T * He)[:T * He]).reshape(T, He)
        out["rmsnorm_gamma_x"] = gamma("gamma_x", He)
        out["rmsnorm_beta_x"] = fbits(-0.1 + 0.2 * _uniform(s, "beta_x", He))
        out["quant_scale_x"] = static_scale("qs_x")
        out["quant_offset_x"] = static_offset("qo_x")
        out["rmsnorm_beta_cq"] = fbits(-0.1 + 0.2 * _uniform(s, "beta_cq", Hcq))
        out["quant_scale_cq"] = static_scale("qs_cq")
        out["quant_offset_cq"] = static_offset("qo_cq")
        w_dq = _int8_uniform(s, "w_dq", He * Hcq).reshape(He, Hcq)
        w_uq = _int8_uniform(s, "w_uq", Hcq * N * D).reshape(Hcq, N * D)
        w_qr = _int8_uniform(s, "w_qr", Hcq * N * Dr).reshape(Hcq, N * Dr)
        w_dkv = _int8_uniform(s, "w_dkv", He * Hckv).reshape(He, Hckv)
        w_kr = _int8_uniform(s, "w_kr", He * Dr).reshape(He, Dr)
        out["dequant_scale_w_dq"] = descale("sw_dq", Hcq, He)
        out["dequant_scale_w_dkv_kr"] = descale("sw_dkv_kr", Hckv + Dr, He)
        out["dequant_scale_w_uq_qr"] = descale("sw_uq_qr", N * (D + Dr), Hcq)
        w_cat = np.concatenate([w_dq, w_dkv, w_kr], axis=1)
        out["bias_dqkv"] = bias("bias_dqkv", w_cat, out["quant_offset_x"])
        out["bias_uq_qr"] = bias("bias_uq", head_interleave(w_uq, w_qr), out["quant_offset_cq"])
    elif not wl.quant:
        out["token_x"] = _to_bf16_bits(_normal(s, "x", full_T * He)[:T * He]).reshape(T, He)
        w_dq = _to_bf16_bits(_normal(s, "w_dq", He * Hcq) / np.sqrt(He)).reshape(He, Hcq)
        if wl.partial:
            w_uq = _int8_uniform(s, "w_uq", Hcq * N * D).reshape(Hcq, N * D)
            w_qr = _int8_uniform(s, "w_qr", Hcq * N * Dr).reshape(Hcq, N * Dr)
            out["dequant_scale_w_uq_qr"] = (0.001 + 0.009 * _uniform(s, "sw_uq_qr", N * (D + Dr))).astype(np.float32)
        else:
            w_uq = _to_bf16_bits(_normal(s, "w_uq", Hcq * N * D) / np.sqrt(Hcq)).reshape(Hcq, N * D)
            w_qr = _to_bf16_bits(_normal(s, "w_qr", Hcq * N * Dr) / np.sqrt(Hcq)).reshape(Hcq, N * Dr)
        w_dkv = _to_bf16_bits(_normal(s, "w_dkv", He * Hckv) / np.sqrt(He)).reshape(He, Hckv)
        w_kr = _to_bf16_bits(_normal(s, "w_kr", He * Dr) / np.sqrt(He)).reshape(He, Dr)
    else:
        out["token_x"] = _int8_uniform(s, "x", full_T * He)[:T * He].reshape(T, He)
        out["dequant_scale_x"] = (0.005 + 0.015 * _uniform(s, "sx", full_T)[:T]).astype(np.float32)
        w_dq = _int8_uniform(s, "w_dq", He * Hcq).reshape(He, Hcq)
        w_uq = _int8_uniform(s, "w_uq", Hcq * N * D).reshape(Hcq, N * D)
        w_qr = _int8_uniform(s, "w_qr", Hcq * N * Dr).reshape(Hcq, N * Dr)
        w_dkv = _int8_uniform(s, "w_dkv", He * Hckv).reshape(He, Hckv)
        w_kr = _int8_uniform(s, "w_kr", He * Dr).reshape(He, Dr)
        out["dequant_scale_w_dq"] = (0.001 + 0.009 * _uniform(s, "sw_dq", Hcq)).astype(np.float32)
        out["dequant_scale_w_uq_qr"] = (0.001 + 0.009 * _uniform(s, "sw_uq_qr", N * (D + Dr))).astype(np.float32)
        out["dequant_scale_w_dkv_kr"] = (0.001 + 0.009 * _uniform(s, "sw_dkv_kr", Hckv + Dr)).astype(np.float32)
    if wl.smooth:
        # per-channel smoothing factors in [0.5, 2)
        out["smooth_scales_cq"] = (0.5 + 1.5 * _uniform(s, "smooth_cq", Hcq)).astype(np.float32)
    out["weight_dq"] = np.ascontiguousarray(w_dq)
    out["weight_uq_qr"] = head_interleave(w_uq, w_qr)
    out["weight_dkv_kr"] = np.ascontiguousarray(np.concatenate([w_dkv, w_kr], axis=1))
    if wl.weight_nk:
        for k in ("weight_dq", "weight_uq_qr", "weight_dkv_kr"):
            out[k] = np.ascontiguousarray(out[k].T)
    if unpacked:
        out["weight_uq"], out["weight_qr"] = w_uq, w_qr
        out["weight_dkv"], out["weight_kr"] = w_dkv, w_kr
    out["weight_uk"] = fbits(_normal(s, "w_uk", N * D * Hckv) / np.sqrt(D)).reshape(N, D, Hckv)

    kr8 = wl.kv_quant and wl.partial
    if wl.kv_quant:
        # per-channel quantScaleCkv in [16, 48): c^KV is O(1), so codes spread
        # over the int8 range and the largest saturate
        out["quant_scale_ckv"] = (16.0 + 32.0 * _uniform(s, "qs_ckv", Hckv)).astype(np.float32)
    if kr8:
        out["quant_scale_ckr"] = (16.0 + 32.0 * _uniform(s, "qs_ckr", Dr)).astype(np.float32)
    out["kv_cache_shape"] = (wl.block_num, wl.block_size, 1, Hckv + Dr if wl.concat else Hckv)
    out["kr_cache_shape"] = (wl.block_num, wl.block_size, 1, Dr)
    sent16 = SENTINEL_F16 if wl.fp16 else SENTINEL_BF16
    if with_caches and wl.concat:
        out["kv_cache"] = np.full(out["kv_cache_shape"], sent16, dtype=np.uint16)
    elif with_caches:
        out["kv_cache"] = (np.full(out["kv_cache_shape"], SENTINEL_I8, dtype=np.int8) if wl.kv_quant
                           else np.full(out["kv_cache_shape"], sent16, dtype=np.uint16))
        out["kr_cache"] = (np.full(out["kr_cache_shape"], SENTINEL_I8, dtype=np.int8) if kr8
                           else np.full(out["kr_cache_shape"], sent16, dtype=np.uint16))
    return out


def custom_workload(name: str, T: int, dims: Dims, block_num: int, block_size: int,
                    quant: bool = False, seed: int = 7, positions: str = "uniform:4096",
                    eps: float = 1e-6, partial: bool = False, smooth: bool = False,
                    kv_quant: bool = False, preprocess: bool = False, x_norm: bool = True,
                    concat: bool = False, weight_nk: bool = False, fp16: bool = False) -> Workload:
    """A workload with arbitrary (small) sizes for tests of ragged shapes."""
    return Workload(name, T, dims, block_num, block_size, quant, positions, seed, eps, partial, smooth,
                    kv_quant, preprocess, x_norm, concat, weight_nk, fp16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """View bf16 bit patterns as float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
