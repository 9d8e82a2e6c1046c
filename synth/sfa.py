"""Seeded synthetic inputs for the sparse flash attention consumer of the MLA
caches (aclnnSparseFlashAttention, parameter table, attentionMode 2): one
decode query per batch, paged caches (PA_BSND) with per-batch block tables.

Draws random numbers into the operator's shapes and dtypes; none of the
operator's arithmetic happens here.
  query (T, N, D) and queryRope (T, N, Dr): N(0, 1), bf16
  kv cache (block_num, block_size, 1, D) and kr cache (.., Dr): N(0, 1),
    bf16 (or one cache of D + Dr with concat)
  actualSeqLengthsKv (T): uniform on [len_lo, len_hi]
  blockTable (T, max_blocks): each batch's ceil(len / block_size) blocks
    are distinct random blocks of the pool; unused entries are -1
  sparseIndices (T, K): distinct random sparse-block ids below
    ceil(len / sparse_block_size), valid ones first, -1 after
  scaleValue: 1 / sqrt(D + Dr)
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

from .generate import _bits, _normal, _to_bf16_bits, _uniform


@dataclass(frozen=True)
class SfaWorkload:
    name: str
    T: int
    N: int
    D: int
    Dr: int
    block_size: int
    K: int                  # sparse_size
    sparse_block_size: int
    len_lo: int
    len_hi: int
    seed: int
    concat: bool = False
    spare_blocks: int = 3   # pool blocks no batch uses

    def with_tokens(self, T: int) -> "SfaWorkload":
        return replace(self, T=T)


SFA_WORKLOADS: Dict[str, SfaWorkload] = {
    "sfa_tiny_t3": SfaWorkload("sfa_tiny_t3", 3, 2, 32, 32, 16, 8, 1, 20, 60, 20300),
    # decode at the model's head count and widths: 2048 selected tokens
    "sfa_decode_t32": SfaWorkload("sfa_decode_t32", 32, 128, 512, 64, 128, 2048, 1, 12288, 20480, 20301),
}


def sfa_workload(name: str) -> SfaWorkload:
    return SFA_WORKLOADS[name]


def make_sfa_inputs(wl: SfaWorkload, caches: bool = True) -> Dict[str, object]:
    """Host arrays of every input (bf16 as uint16 bit patterns).  Without
    ``caches`` the cache contents are left out (their shapes are given)."""
    s = wl.seed
    T, N, D, Dr, bs = wl.T, wl.N, wl.D, wl.Dr, wl.block_size
    out: Dict[str, object] = {"workload": wl.name, "T": T, "N": N, "D": D, "Dr": Dr, "block_size": bs,
                              "K": wl.K, "sparse_block_size": wl.sparse_block_size, "concat": wl.concat,
                              "scale": 1.0 / np.sqrt(D + Dr)}
    lens = wl.len_lo + np.floor(_uniform(s, "sfa_len", T) * (wl.len_hi - wl.len_lo + 1)).astype(np.int64)
    nblk = -(-lens // bs)
    max_blocks = -(-wl.len_hi // bs)
    block_num = int(nblk.sum()) + wl.spare_blocks
    perm = np.argsort(_bits(s, "sfa_blocks", 0, block_num), kind="stable")
    table = np.full((T, max_blocks), -1, dtype=np.int32)
    used = 0
    for t in range(T):
        table[t, :nblk[t]] = perm[used:used + nblk[t]]
        used += int(nblk[t])
    idx = np.full((T, wl.K), -1, dtype=np.int32)
    for t in range(T):
        n_units = -(-int(lens[t]) // wl.sparse_block_size)
        order = np.argsort(_bits(s, "sfa_idx", t * (1 << 20), n_units), kind="stable")
        k = min(wl.K, n_units)
        idx[t, :k] = order[:k]
    out.update(seq_lens=lens.astype(np.int32), block_table=table, indices=idx, block_num=block_num,
               max_blocks=max_blocks)
    out["query"] = _to_bf16_bits(_normal(s, "sfa_q", T * N * D)).reshape(T, N, D)
    out["query_rope"] = _to_bf16_bits(_normal(s, "sfa_qr", T * N * Dr)).reshape(T, N, Dr)
    row = D + Dr if wl.concat else D
    out["kv_cache_shape"] = (block_num, bs, 1, row)
    out["kr_cache_shape"] = (block_num, bs, 1, Dr)
    if caches:
        kv = _to_bf16_bits(_normal(s, "sfa_kv", block_num * bs * D)).reshape(block_num, bs, 1, D)
        kr = _to_bf16_bits(_normal(s, "sfa_kr", block_num * bs * Dr)).reshape(block_num, bs, 1, Dr)
        if wl.concat:
            out["kv_cache"] = np.ascontiguousarray(np.concatenate([kv, kr], axis=3))
        else:
            out["kv_cache"], out["kr_cache"] = kv, kr
    return out


def custom_sfa_workload(name: str, T: int, N: int, D: int, Dr: int, block_size: int, K: int,
                        sparse_block_size: int = 1, len_lo: int = 1, len_hi: int = 256, seed: int = 9,
                        concat: bool = False) -> SfaWorkload:
    return SfaWorkload(name, T, N, D, Dr, block_size, K, sparse_block_size, len_lo, len_hi, seed, concat)
