"""Python binding of libmla_prolog.so, the MI355X MLA prolog library.

Argument marshalling only: every step of the prolog runs in the library's HIP
kernels.  Tensors are passed as device pointers (``tensor.data_ptr()`` or
plain ints) and streams as ``hipStream_t`` handles; PyTorch is used by the
callers for device memory and streams, never for the computation.  Importing
this module does not need a GPU; creating a handle or running does, and fails
loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "csrc", "mla_prolog.hip")
#: every HIP source of the library: the prolog and its cache consumer
SOURCES = (SOURCE, os.path.join(HERE, "csrc", "mla_sfa.hip"))
#: the built library; MLA_PROLOG_LIBRARY names another build of the same
#: sources (the sanitizer test builds one whose host code carries AddressSanitizer
#: and UBSan)
LIBRARY = os.environ.get("MLA_PROLOG_LIBRARY") or os.path.join(HERE, "libmla_prolog.so")
# MFMA accumulators in VGPRs: with the default AGPR form the register
# allocator rotates the accumulators of the software-pipelined loops through
# copies on every iteration.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form=1"]

MLA_OK = 0
MLA_ERR_NULLPTR = 161001
MLA_ERR_PARAM_INVALID = 161002
MLA_ERR_RUNTIME = 361001
MLA_ERR_UNSUPPORTED = 561002
MLA_BF16 = 0
MLA_INT8 = 1
MLA_INT8_PARTIAL = 2   # in_dtype only: int8 weightUqQr, every other input bf16
MLA_INT8_STATIC = 3    # in_dtype only: the preprocess page's static int8 scenario
MLA_FP16 = 4           # float_dtype only: fp16 tensors in the static scenario

#: the symbols include/mla_prolog.h declares
EXPORTS = ("mla_prolog_validate", "mla_prolog_workspace_bytes", "mla_prolog_packed_weights_bytes",
           "mla_prolog_pack_weights", "mla_prolog_create",
           "mla_prolog_run", "mla_prolog_run_noalloc", "mla_prolog_destroy", "mla_prolog_profile_enable",
           "mla_prolog_profile_read", "mla_prolog_check", "mla_prolog_set_poll_limit",
           "mla_prolog_status_string",
           "mla_sfa_validate", "mla_sfa_create", "mla_sfa_run", "mla_sfa_destroy")
#: kernel order of mla_prolog_profile_read
KERNELS = ("down_proj", "norm_rope_cache", "up_proj", "uk")


def build() -> str:
    """Compile the HIP library for gfx950 with hipcc (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "hipcc")
    subprocess.run([hipcc, *HIPCC_FLAGS, "-o", LIBRARY, *SOURCES], check=True)
    return LIBRARY


class Desc(ctypes.Structure):
    _fields_ = [("He", ctypes.c_int64), ("Hcq", ctypes.c_int64), ("Hckv", ctypes.c_int64),
                ("N", ctypes.c_int64), ("D", ctypes.c_int64), ("Dr", ctypes.c_int64),
                ("block_num", ctypes.c_int64), ("block_size", ctypes.c_int64),
                ("max_tokens", ctypes.c_int64),
                ("eps_cq", ctypes.c_double), ("eps_ckv", ctypes.c_double),
                ("in_dtype", ctypes.c_int32), ("query_dtype", ctypes.c_int32),
                ("device", ctypes.c_int32), ("cache_dtype", ctypes.c_int32),
                ("concat", ctypes.c_int32), ("weights_nk", ctypes.c_int32),
                ("x_quant_only", ctypes.c_int32), ("check_index", ctypes.c_int32),
                ("eps_x", ctypes.c_double), ("float_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


TENSOR_FIELDS = ("token_x", "weight_dq", "weight_uq_qr", "weight_uk", "weight_dkv_kr",
                 "gamma_cq", "gamma_ckv", "rope_sin", "rope_cos", "cache_index",
                 "kv_cache", "kr_cache", "scale_x", "scale_w_dq", "scale_w_uq_qr",
                 "scale_w_dkv_kr", "query_out", "query_rope_out", "dequant_scale_q_nope",
                 "packed_weights", "smooth_scales_cq", "quant_scale_ckv", "quant_scale_ckr",
                 "gamma_x", "beta_x", "quant_scale_x", "quant_offset_x", "bias_dqkv", "beta_cq",
                 "quant_scale_cq", "quant_offset_cq", "bias_uq_qr")


class Tensors(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in TENSOR_FIELDS]


_lib: Optional[ctypes.CDLL] = None


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIBRARY)
        L.mla_prolog_validate.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Tensors), ctypes.c_int64]
        L.mla_prolog_validate.restype = ctypes.c_int
        L.mla_prolog_workspace_bytes.argtypes = [ctypes.POINTER(Desc)]
        L.mla_prolog_workspace_bytes.restype = ctypes.c_size_t
        L.mla_prolog_packed_weights_bytes.argtypes = [ctypes.POINTER(Desc)]
        L.mla_prolog_packed_weights_bytes.restype = ctypes.c_size_t
        L.mla_prolog_pack_weights.argtypes = [ctypes.c_void_p, ctypes.POINTER(Tensors), ctypes.c_void_p,
                                              ctypes.c_void_p]
        L.mla_prolog_pack_weights.restype = ctypes.c_int
        L.mla_prolog_create.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_void_p)]
        L.mla_prolog_create.restype = ctypes.c_int
        L.mla_prolog_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(Tensors), ctypes.c_int64,
                                     ctypes.c_void_p]
        L.mla_prolog_run.restype = ctypes.c_int
        L.mla_prolog_run_noalloc.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Tensors), ctypes.c_int64,
                                             ctypes.c_void_p]
        L.mla_prolog_run_noalloc.restype = ctypes.c_int
        L.mla_prolog_destroy.argtypes = [ctypes.c_void_p]
        L.mla_prolog_destroy.restype = ctypes.c_int
        L.mla_prolog_profile_enable.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.mla_prolog_profile_enable.restype = ctypes.c_int
        L.mla_prolog_profile_read.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(ctypes.c_int64)]
        L.mla_prolog_profile_read.restype = ctypes.c_int
        L.mla_prolog_check.argtypes = [ctypes.c_void_p]
        L.mla_prolog_check.restype = ctypes.c_int
        L.mla_prolog_set_poll_limit.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.mla_prolog_set_poll_limit.restype = ctypes.c_int
        L.mla_prolog_status_string.argtypes = [ctypes.c_int]
        L.mla_prolog_status_string.restype = ctypes.c_char_p
        L.mla_sfa_validate.argtypes = [ctypes.POINTER(SfaDesc), ctypes.POINTER(SfaTensors), ctypes.c_int64]
        L.mla_sfa_validate.restype = ctypes.c_int
        L.mla_sfa_create.argtypes = [ctypes.POINTER(SfaDesc), ctypes.POINTER(ctypes.c_void_p)]
        L.mla_sfa_create.restype = ctypes.c_int
        L.mla_sfa_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(SfaTensors), ctypes.c_int64, ctypes.c_void_p]
        L.mla_sfa_run.restype = ctypes.c_int
        L.mla_sfa_destroy.argtypes = [ctypes.c_void_p]
        L.mla_sfa_destroy.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_prolog_status_string(int(status)).decode()


def make_desc(He, Hcq, Hckv, N, D, Dr, block_num, block_size, max_tokens, eps_cq=1e-5,
              eps_ckv=1e-5, in_dtype=MLA_BF16, query_dtype=MLA_BF16, device=0,
              cache_dtype=MLA_BF16, concat=0, weights_nk=0, x_quant_only=0, eps_x=1e-5,
              check_index=0, float_dtype=MLA_BF16) -> Desc:
    return Desc(He, Hcq, Hckv, N, D, Dr, block_num, block_size, max_tokens, eps_cq, eps_ckv,
                in_dtype, query_dtype, device, cache_dtype, int(concat), int(weights_nk),
                int(x_quant_only), int(check_index), eps_x, int(float_dtype), 0)


def _address(v) -> Optional[int]:
    if v is None:
        return None
    if isinstance(v, int):
        return v
    return int(v.data_ptr())


def make_tensors(tensors: Dict[str, object]) -> Tensors:
    """Tensors struct from a dict of torch tensors / device addresses (missing = NULL)."""
    unknown = set(tensors) - set(TENSOR_FIELDS)
    if unknown:
        raise KeyError(f"unknown tensor names {sorted(unknown)}")
    return Tensors(*[_address(tensors.get(f)) for f in TENSOR_FIELDS])


def validate(desc: Desc, tensors: Optional[Dict[str, object]] = None, T: int = 0) -> int:
    t = make_tensors(tensors) if tensors is not None else None
    return lib().mla_prolog_validate(ctypes.byref(desc), ctypes.byref(t) if t is not None else None,
                                     int(T))


def workspace_bytes(desc: Desc) -> int:
    return int(lib().mla_prolog_workspace_bytes(ctypes.byref(desc)))


def packed_weights_bytes(desc: Desc) -> int:
    return int(lib().mla_prolog_packed_weights_bytes(ctypes.byref(desc)))


def run_noalloc(desc: Desc, tensors: Dict[str, object], T: int, stream=None) -> None:
    """One prolog with no handle and no allocation: the library's static
    per-device workspace (mla_prolog_run_noalloc)."""
    t = make_tensors(tensors)
    st = lib().mla_prolog_run_noalloc(ctypes.byref(desc), ctypes.byref(t), int(T),
                                      ctypes.c_void_p(_stream_handle(stream)))
    if st != MLA_OK:
        raise MlaError(st, "mla_prolog_run_noalloc")


def _stream_handle(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


class MlaProlog:
    """A library handle: ``MlaProlog(desc)``, then ``run(tensors, T, stream)``."""

    def __init__(self, desc: Desc):
        self.desc = desc
        h = ctypes.c_void_p()
        st = lib().mla_prolog_create(ctypes.byref(desc), ctypes.byref(h))
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_create")
        self._h = h

    def run(self, tensors: Dict[str, object], T: int, stream=None) -> None:
        """Enqueue one prolog over T tokens on ``stream`` (a torch stream, a
        raw hipStream_t address, or None for the current torch stream)."""
        t = make_tensors(tensors)
        st = lib().mla_prolog_run(self._h, ctypes.byref(t), int(T),
                                  ctypes.c_void_p(_stream_handle(stream)))
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_run")

    def pack_weights(self, tensors: Dict[str, object], packed, stream=None) -> None:
        """Enqueue the conversion of the four weights of ``tensors`` into
        ``packed`` (a device buffer of ``packed_weights_bytes(desc)`` bytes)."""
        t = make_tensors(tensors)
        st = lib().mla_prolog_pack_weights(self._h, ctypes.byref(t), ctypes.c_void_p(_address(packed)),
                                           ctypes.c_void_p(_stream_handle(stream)))
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_pack_weights")

    def profile(self, enable: bool = True) -> None:
        """Start (or stop) recording per-kernel HIP events on every run."""
        st = lib().mla_prolog_profile_enable(self._h, int(bool(enable)))
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_profile_enable")

    def profile_read(self):
        """(milliseconds per kernel summed over the runs since the last read,
        number of runs), kernels in the order of ``KERNELS``."""
        ms = (ctypes.c_double * 4)()
        n = ctypes.c_int64()
        st = lib().mla_prolog_profile_read(self._h, ms, ctypes.byref(n))
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_profile_read")
        return dict(zip(KERNELS, list(ms))), int(n.value)

    def check(self) -> None:
        """Wait for the device and raise if an earlier run of this handle gave
        up waiting for another block of its launch (its outputs are then not
        to be trusted)."""
        st = lib().mla_prolog_check(self._h)
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_check")

    def set_poll_limit(self, steps: int) -> None:
        """Poll steps after which a bounded wait of the small-T kernels gives
        up, from the next run on (0 = the default)."""
        st = lib().mla_prolog_set_poll_limit(self._h, int(steps))
        if st != MLA_OK:
            raise MlaError(st, "mla_prolog_set_poll_limit")

    def close(self) -> None:
        """check(), then free the handle."""
        if self._h:
            chk = lib().mla_prolog_check(self._h)
            st = lib().mla_prolog_destroy(self._h)
            self._h = None
            if chk != MLA_OK:
                raise MlaError(chk, "mla_prolog_check")
            if st != MLA_OK:
                raise MlaError(st, "mla_prolog_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- sparse flash attention over the caches (include/mla_sfa.h) ------------
class SfaDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("D", ctypes.c_int64), ("Dr", ctypes.c_int64),
                ("block_num", ctypes.c_int64), ("block_size", ctypes.c_int64), ("max_blocks", ctypes.c_int64),
                ("sparse_size", ctypes.c_int64), ("sparse_block_size", ctypes.c_int64),
                ("max_tokens", ctypes.c_int64), ("scale", ctypes.c_double),
                ("concat", ctypes.c_int32), ("device", ctypes.c_int32)]


SFA_TENSOR_FIELDS = ("query", "query_rope", "kv_cache", "kr_cache", "sparse_indices", "block_table",
                     "seq_lens_kv", "attention_out", "softmax_max", "softmax_sum")


class SfaTensors(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in SFA_TENSOR_FIELDS]


def make_sfa_desc(N, D, Dr, block_num, block_size, max_blocks, sparse_size, sparse_block_size, max_tokens,
                  scale, concat=0, device=0) -> SfaDesc:
    return SfaDesc(N, D, Dr, block_num, block_size, max_blocks, sparse_size, sparse_block_size, max_tokens,
                   float(scale), int(concat), device)


def make_sfa_tensors(tensors: Dict[str, object]) -> SfaTensors:
    unknown = set(tensors) - set(SFA_TENSOR_FIELDS)
    if unknown:
        raise KeyError(f"unknown tensor names {sorted(unknown)}")
    return SfaTensors(*[_address(tensors.get(f)) for f in SFA_TENSOR_FIELDS])


def sfa_validate(desc: SfaDesc, tensors: Optional[Dict[str, object]] = None, T: int = 0) -> int:
    t = make_sfa_tensors(tensors) if tensors is not None else None
    return lib().mla_sfa_validate(ctypes.byref(desc), ctypes.byref(t) if t is not None else None, int(T))


class MlaSfa:
    """Sparse flash attention handle: ``MlaSfa(desc)``, then ``run(tensors, T, stream)``."""

    def __init__(self, desc: SfaDesc):
        self.desc = desc
        h = ctypes.c_void_p()
        st = lib().mla_sfa_create(ctypes.byref(desc), ctypes.byref(h))
        if st != MLA_OK:
            raise MlaError(st, "mla_sfa_create")
        self._h = h

    def run(self, tensors: Dict[str, object], T: int, stream=None) -> None:
        t = make_sfa_tensors(tensors)
        st = lib().mla_sfa_run(self._h, ctypes.byref(t), int(T), ctypes.c_void_p(_stream_handle(stream)))
        if st != MLA_OK:
            raise MlaError(st, "mla_sfa_run")

    def close(self) -> None:
        if self._h:
            st = lib().mla_sfa_destroy(self._h)
            self._h = None
            if st != MLA_OK:
                raise MlaError(st, "mla_sfa_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
