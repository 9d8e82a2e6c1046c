"""Pins of the sparse flash attention oracle (aclnnSparseFlashAttention,
"Function" formula and parameter table, attentionMode 2 = MLA-absorb) against
what the formula and the mathematics fix, independent of the oracle's code:
an independent numpy formulation, closed forms (one selected row, zero
scale, no selected row), invariances (index order, padding, rows past the kv
length, block-wise against token-wise selection, the concatenated cache),
and planted mistakes that must fail a pin."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from synth.sfa import custom_sfa_workload, make_sfa_inputs, sfa_workload


def bf16(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


TINY = sfa_workload("sfa_tiny_t3")
RAGGED = custom_sfa_workload("ragged", T=4, N=3, D=24, Dr=8, block_size=16, K=11, len_lo=5, len_hi=70, seed=3)
BLOCKWISE = custom_sfa_workload("blockwise", T=3, N=2, D=16, Dr=8, block_size=16, K=5, sparse_block_size=4,
                                len_lo=9, len_hi=60, seed=4)


def numpy_attention(inp):
    """softmax(scale [q | q_r] . [kv | kr]^T) kv over the gathered rows, in
    float64 with numpy; returns out, max, sum."""
    T, N, D, Dr, bs, sbs = (inp[k] for k in ("T", "N", "D", "Dr", "block_size", "sparse_block_size"))
    kv = bf16(inp["kv_cache"]).reshape(-1, inp["kv_cache"].shape[-1])
    kr = kv[:, D:] if inp["concat"] else bf16(inp["kr_cache"]).reshape(-1, Dr)
    kv = kv[:, :D]
    q, qr = bf16(inp["query"]), bf16(inp["query_rope"])
    out = np.zeros((T, N, D))
    mx = np.full((T, N), -np.inf)
    sm = np.zeros((T, N))
    for t in range(T):
        pos = [i * sbs + u for i in inp["indices"][t] if i >= 0 for u in range(sbs)]
        pos = [p for p in pos if p < inp["seq_lens"][t]]
        slots = np.array([inp["block_table"][t][p // bs] * bs + p % bs for p in pos], dtype=np.int64)
        if slots.size == 0:
            continue
        s = inp["scale"] * (q[t] @ kv[slots].T + qr[t] @ kr[slots].T)       # (N, rows)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[t] = (w @ kv[slots]) / w.sum(axis=1, keepdims=True)
        mx[t], sm[t] = m[:, 0], w.sum(axis=1)
    return out, mx, sm


def _matches(inp, o):
    out, mx, sm = numpy_attention(inp)
    return bool(np.allclose(o["out_f64"], out, rtol=1e-12, atol=1e-13)
                and np.allclose(o["softmax_max"], mx.astype(np.float32), rtol=1e-6, atol=0)
                and np.allclose(o["softmax_sum"], sm.astype(np.float32), rtol=1e-6, atol=0)
                and np.array_equal(bf16(o["attention_out"]), bf16(oracle.bf16_bits(o["out_f64"]))))


@pytest.mark.parametrize("wl", [TINY, RAGGED, BLOCKWISE], ids=["tiny", "ragged", "blockwise"])
def test_matches_numpy_formulation(wl):
    inp = make_sfa_inputs(wl)
    assert _matches(inp, oracle.sfa(inp))


def test_one_selected_row_is_that_row():
    inp = make_sfa_inputs(TINY)
    inp["indices"] = np.full_like(inp["indices"], -1)
    inp["indices"][:, 0] = 3
    o = oracle.sfa(inp)
    for t in range(inp["T"]):
        slot = inp["block_table"][t][0] * inp["block_size"] + 3
        row = inp["kv_cache"].reshape(-1, inp["D"])[slot]
        for h in range(inp["N"]):
            assert np.array_equal(o["attention_out"][t, h], row)
    assert np.all(o["softmax_sum"] == 1.0)


def test_zero_scale_averages_the_rows():
    inp = make_sfa_inputs(RAGGED)
    inp["scale"] = 0.0
    o = oracle.sfa(inp)
    kv = bf16(inp["kv_cache"]).reshape(-1, inp["D"])
    bs = inp["block_size"]
    for t in range(inp["T"]):
        pos = [int(i) for i in inp["indices"][t] if 0 <= i < inp["seq_lens"][t]]
        mean = kv[[inp["block_table"][t][p // bs] * bs + p % bs for p in pos]].mean(axis=0)
        assert np.allclose(o["out_f64"][t], mean[None, :], rtol=1e-13, atol=1e-15)
        assert np.all(o["softmax_max"][t] == 0.0) and np.all(o["softmax_sum"][t] == len(pos))


def test_no_selected_row():
    inp = make_sfa_inputs(TINY)
    inp["indices"][1] = -1
    o = oracle.sfa(inp)
    assert not o["attention_out"][1].any()
    assert np.all(np.isneginf(o["softmax_max"][1])) and not o["softmax_sum"][1].any()
    assert o["attention_out"][0].any()


def test_index_order_padding_and_rows_past_the_length():
    inp = make_sfa_inputs(RAGGED)
    a = oracle.sfa(inp)
    shuf = dict(inp)
    rng = np.random.default_rng(0)
    idx = inp["indices"].copy()
    for t in range(inp["T"]):
        valid = idx[t][idx[t] >= 0]
        extra = [-1, inp["seq_lens"][t] + 3]          # padding and a position past the length
        row = np.concatenate([rng.permutation(valid), extra])
        idx[t] = row[:idx.shape[1]] if row.size >= idx.shape[1] else np.pad(row, (0, idx.shape[1] - row.size),
                                                                              constant_values=-1)
    shuf["indices"] = np.ascontiguousarray(np.concatenate([idx, np.full((inp["T"], 2), -1, np.int32)], axis=1))
    shuf["K"] = shuf["indices"].shape[1]
    shuf["indices"][:, -1] = inp["seq_lens"] + 1
    b = oracle.sfa(shuf)
    assert np.allclose(a["out_f64"], b["out_f64"], rtol=1e-13, atol=1e-15)


def test_blockwise_selection_is_the_expanded_tokenwise_one():
    inp = make_sfa_inputs(BLOCKWISE)
    sbs = inp["sparse_block_size"]
    tok = dict(inp, sparse_block_size=1, K=inp["K"] * sbs)
    idx = inp["indices"]
    tok["indices"] = np.where(idx[:, :, None] >= 0, idx[:, :, None] * sbs + np.arange(sbs), -1).reshape(
        inp["T"], -1).astype(np.int32)
    a, b = oracle.sfa(inp), oracle.sfa(tok)
    assert np.allclose(a["out_f64"], b["out_f64"], rtol=1e-13, atol=1e-15)


def test_concatenated_cache_is_the_separate_caches_side_by_side():
    inp = make_sfa_inputs(RAGGED)
    cat = make_sfa_inputs(replace(RAGGED, concat=True))
    assert np.array_equal(cat["kv_cache"], np.concatenate([inp["kv_cache"], inp["kr_cache"]], axis=3))
    a, b = oracle.sfa(inp), oracle.sfa(cat)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_token_subsets():
    inp = make_sfa_inputs(RAGGED)
    a = oracle.sfa(inp)
    b = oracle.sfa(inp, tokens=[3, 1])
    assert np.array_equal(b["attention_out"], a["attention_out"][[3, 1]])


@pytest.mark.parametrize("mutation", [21, 22, 23], ids=["rope_dropped", "scale_squared", "table_ignored"])
def test_planted_mistakes_fail_a_pin(mutation):
    inp = make_sfa_inputs(RAGGED)
    assert _matches(inp, oracle.sfa(inp))
    assert not _matches(inp, oracle.sfa(inp, mutation=mutation))
