"""Copies of the generated inputs in device memory (torch tensors), plus the
output buffers a run writes, keyed by the library's tensor names.  Data
movement only: nothing here computes any part of the prolog."""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch


def _tensor(a: np.ndarray, device, half=torch.bfloat16) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:          # bf16 (or fp16) bit patterns
        return torch.from_numpy(a.view(np.int16)).to(device).view(half)
    return torch.from_numpy(a).to(device)


def upload(inp: Dict[str, object], device="cuda:0", query_int8=None) -> Dict[str, torch.Tensor]:
    """Device tensors for every input of ``inp`` and zeroed outputs."""
    quant = bool(inp["quant"])
    q8 = quant if query_int8 is None else bool(query_int8)
    d = inp["dims"]
    T = int(inp["T"])
    names = {"token_x": "token_x", "weight_dq": "weight_dq", "weight_uq_qr": "weight_uq_qr",
             "weight_uk": "weight_uk", "weight_dkv_kr": "weight_dkv_kr",
             "rmsnorm_gamma_cq": "gamma_cq", "rmsnorm_gamma_ckv": "gamma_ckv",
             "rope_sin": "rope_sin", "rope_cos": "rope_cos", "cache_index": "cache_index",
             "kv_cache": "kv_cache", "kr_cache": "kr_cache"}
    if quant:
        names.update({"dequant_scale_x": "scale_x", "dequant_scale_w_dq": "scale_w_dq",
                      "dequant_scale_w_uq_qr": "scale_w_uq_qr",
                      "dequant_scale_w_dkv_kr": "scale_w_dkv_kr"})
    elif inp.get("partial", False):
        names["dequant_scale_w_uq_qr"] = "scale_w_uq_qr"
    elif inp.get("preprocess", False):
        names.update({"dequant_scale_w_dq": "scale_w_dq", "dequant_scale_w_uq_qr": "scale_w_uq_qr",
                      "dequant_scale_w_dkv_kr": "scale_w_dkv_kr", "rmsnorm_beta_cq": "beta_cq",
                      "quant_scale_x": "quant_scale_x", "quant_offset_x": "quant_offset_x",
                      "bias_dqkv": "bias_dqkv", "quant_scale_cq": "quant_scale_cq",
                      "quant_offset_cq": "quant_offset_cq", "bias_uq_qr": "bias_uq_qr"})
        if inp.get("x_norm", True):
            names.update({"rmsnorm_gamma_x": "gamma_x", "rmsnorm_beta_x": "beta_x"})
    if inp.get("smooth_scales_cq") is not None:
        names["smooth_scales_cq"] = "smooth_scales_cq"
    for k in ("quant_scale_ckv", "quant_scale_ckr"):
        if inp.get(k) is not None:
            names[k] = k
    # the 16-bit float tensors are fp16 in the static scenario's FLOAT16
    # variant, bf16 otherwise
    half = torch.float16 if inp.get("fp16", False) else torch.bfloat16
    out = {lib_name: _tensor(np.asarray(inp[key]), device, half) for key, lib_name in names.items()
           if key in inp}
    concat = bool(inp.get("concat", False))
    out["query_out"] = torch.zeros((T, d.N, d.Hckv + d.Dr if concat else d.Hckv),
                                   dtype=torch.int8 if q8 else half, device=device)
    if not concat:
        out["query_rope_out"] = torch.zeros((T, d.N, d.Dr), dtype=half, device=device)
    if q8:
        out["dequant_scale_q_nope"] = torch.zeros((T, d.N), dtype=torch.float32, device=device)
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a device tensor; bf16 and fp16 as uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def desc_args(inp: Dict[str, object], max_tokens=None, query_int8=None) -> Dict[str, object]:
    """Keyword arguments of ``make_desc`` for these inputs (in_dtype 0 bf16,
    1 int8 full quantisation, 2 partial quantisation, 3 the static scenario;
    float_dtype 4 for its fp16 tensors)."""
    d = inp["dims"]
    quant = bool(inp["quant"])
    q8 = quant if query_int8 is None else bool(query_int8)
    return dict(He=d.He, Hcq=d.Hcq, Hckv=d.Hckv, N=d.N, D=d.D, Dr=d.Dr,
                block_num=int(inp["block_num"]), block_size=int(inp["block_size"]),
                max_tokens=int(inp["T"]) if max_tokens is None else int(max_tokens),
                eps_cq=float(inp["eps_cq"]), eps_ckv=float(inp["eps_ckv"]),
                in_dtype=(2 if inp.get("partial", False) else 3 if inp.get("preprocess", False)
                          else int(quant)),
                query_dtype=int(q8), cache_dtype=int(bool(inp.get("kv_quant", False))),
                concat=int(bool(inp.get("concat", False))), weights_nk=int(bool(inp.get("weight_nk", False))),
                x_quant_only=int(not inp.get("x_norm", True)) if inp.get("preprocess", False) else 0,
                eps_x=float(inp.get("eps_x", 1e-5)), float_dtype=4 if inp.get("fp16", False) else 0)
