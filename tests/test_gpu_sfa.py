"""GPU parity of the sparse flash attention consumer (aclnnSparseFlashAttention,
MLA-absorb decode) through its C ABI against the CPU oracle, on seeded
synthetic caches, indices and block tables.

attention_out (bf16): |gpu - ref| <= 2^-8 (sum_j p_j |v_j| / sum_j p_j + |ref|)
per element: the device rounds the softmax weights to bf16 for the P V
product, which moves an element by at most 2^-9 of that weighted mean of |v|;
both sides round the output to bf16.
softmax_max: within 1e-4 + 1e-5 |ref| (fp32 scores of bf16 products);
softmax_sum: relative 1e-3.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest

import oracle
from synth.sfa import custom_sfa_workload, make_sfa_inputs, sfa_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import head_latent_attention_amd as mla  # noqa: E402
from synth import device as dev  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def weighted_abs(inp, rows):
    """sum_j p_j |v_j[d]| / sum_j p_j per (token, head, column), in float64:
    how far the device's bf16 softmax weights (2^-9 relative each) can move
    an output element."""
    N, D, Dr, bs, sbs = (int(inp[k]) for k in ("N", "D", "Dr", "block_size", "sparse_block_size"))
    kvall = bf16(inp["kv_cache"]).reshape(-1, inp["kv_cache"].shape[-1])
    krall = kvall[:, D:] if inp["concat"] else bf16(inp["kr_cache"]).reshape(-1, Dr)
    out = np.zeros((len(rows), N, D))
    for r, t in enumerate(rows):
        pos = [int(i) * sbs + u for i in inp["indices"][t] if i >= 0 for u in range(sbs)]
        slots = []
        for p in pos:
            if p < inp["seq_lens"][t] and p // bs < inp["max_blocks"]:
                blk = int(inp["block_table"][t][p // bs])
                if 0 <= blk < inp["block_num"]:
                    slots.append(blk * bs + p % bs)
        if not slots:
            continue
        kv, kr = kvall[slots][:, :D], krall[slots]
        sc = inp["scale"] * (bf16(inp["query"][t]) @ kv.T + bf16(inp["query_rope"][t]) @ kr.T)
        w = np.exp(sc - sc.max(axis=1, keepdims=True))
        out[r] = (w @ np.abs(kv)) / w.sum(axis=1, keepdims=True)
    return out


def bf16(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # unwritten cache slots hold a NaN sentinel
        return b.view(np.float32).astype(np.float64)


def run_gpu(inp, lse=True, repeat=1, T=None):
    T = int(inp["T"]) if T is None else T
    t = {"query": inp["query"], "query_rope": inp["query_rope"], "kv_cache": inp["kv_cache"],
         "sparse_indices": inp["indices"], "block_table": inp["block_table"], "seq_lens_kv": inp["seq_lens"]}
    if not inp["concat"]:
        t["kr_cache"] = inp["kr_cache"]
    g = {k: dev._tensor(np.asarray(v), "cuda:0") for k, v in t.items()}
    N, D = int(inp["N"]), int(inp["D"])
    g["attention_out"] = torch.zeros((int(inp["T"]), N, D), dtype=torch.bfloat16, device="cuda:0")
    if lse:
        g["softmax_max"] = torch.zeros((int(inp["T"]), N), dtype=torch.float32, device="cuda:0")
        g["softmax_sum"] = torch.zeros((int(inp["T"]), N), dtype=torch.float32, device="cuda:0")
    desc = mla.make_sfa_desc(N=N, D=D, Dr=int(inp["Dr"]), block_num=int(inp["block_num"]),
                             block_size=int(inp["block_size"]), max_blocks=int(inp["max_blocks"]),
                             sparse_size=int(inp["K"]), sparse_block_size=int(inp["sparse_block_size"]),
                             max_tokens=int(inp["T"]), scale=float(inp["scale"]), concat=int(bool(inp["concat"])))
    with mla.MlaSfa(desc) as h:
        for _ in range(repeat):
            h.run(g, T)
        torch.cuda.synchronize()
    return {k: dev.bits(v) for k, v in g.items() if k in ("attention_out", "softmax_max", "softmax_sum")}


def check(inp, rows=None, lse=True):
    T = int(inp["T"])
    rows = np.arange(T) if rows is None else np.asarray(rows)
    say(f"case {inp['workload']} T={T} N={inp['N']} D={inp['D']} Dr={inp['Dr']} K={inp['K']} "
        f"sbs={inp['sparse_block_size']} concat={inp['concat']} rows={len(rows)}")
    got = run_gpu(inp, lse=lse)
    ref = oracle.sfa(inp, tokens=rows)
    g, r = bf16(got["attention_out"][rows]), bf16(ref["attention_out"])
    err = np.abs(g - r)
    say(f"  attention_out: |ref| mean {np.abs(r).mean():.3g}, max error {err.max():.3g}, "
        f"max error / (|ref| + 1e-2) {(err / (np.abs(r) + 1e-2)).max():.3g}")
    # twice the weights' rounding bound, plus two bf16 steps of the output
    tol = 2.0 ** -8 * (weighted_abs(inp, rows) + np.abs(r)) + 1e-6
    say(f"  worst error / tolerance {(err / tol).max():.3g}")
    bad = ~(err <= tol)
    assert not bad.any(), f"attention_out: {bad.sum()} of {bad.size} out of tolerance, first {np.argwhere(bad)[0]}"
    if lse:
        gm, rm = got["softmax_max"][rows].astype(np.float64), ref["softmax_max"].astype(np.float64)
        same_inf = np.isneginf(gm) & np.isneginf(rm)
        with np.errstate(invalid="ignore"):
            close = np.abs(gm - rm) <= 1e-4 + 1e-5 * np.abs(rm)
        assert np.all(same_inf | close), "softmax_max"
        gs, rs = got["softmax_sum"][rows].astype(np.float64), ref["softmax_sum"].astype(np.float64)
        assert np.all(np.abs(gs - rs) <= 1e-3 * np.abs(rs)), "softmax_sum"
    return got


SMALL = {
    "tiny_t3": sfa_workload("sfa_tiny_t3"),
    "ragged_t5": custom_sfa_workload("ragged_t5", T=5, N=3, D=64, Dr=32, block_size=16, K=40, len_lo=5,
                                     len_hi=300, seed=51),
    "heads80_t4": custom_sfa_workload("heads80_t4", T=4, N=80, D=128, Dr=64, block_size=32, K=100, len_lo=50,
                                      len_hi=900, seed=52),
    "blockwise_t4": custom_sfa_workload("blockwise_t4", T=4, N=16, D=96, Dr=32, block_size=16, K=12,
                                        sparse_block_size=4, len_lo=20, len_hi=200, seed=53),
    "one_split_t300": custom_sfa_workload("one_split_t300", T=300, N=8, D=64, Dr=32, block_size=16, K=70,
                                          len_lo=40, len_hi=120, seed=54),
    "long_t1": custom_sfa_workload("long_t1", T=1, N=16, D=128, Dr=64, block_size=64, K=5000, len_lo=6000,
                                   len_hi=7000, seed=55),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small(name):
    check(make_sfa_inputs(SMALL[name]))


def wide_spread_inputs():
    """8 tokens x 8 heads over 4096 selected rows (32 splits of four 32-row
    tiles each), scale 3 over 96 dimensions: scores spread by ~30."""
    inp = make_sfa_inputs(custom_sfa_workload("wide_t8", T=8, N=8, D=64, Dr=32, block_size=64, K=4096,
                                              len_lo=4200, len_hi=5000, seed=56))
    inp["scale"] = 3.0
    return inp


def tile_jumps(inp, rows=128):
    """How often, over the first `rows` selected rows of each (token, head),
    a 32-row tile's maximum score passes the running maximum of the tiles
    before it by more than 8 (float64)."""
    D, Dr, bs = int(inp["D"]), int(inp["Dr"]), int(inp["block_size"])
    kvall, krall = bf16(inp["kv_cache"]).reshape(-1, D), bf16(inp["kr_cache"]).reshape(-1, Dr)
    jumps = 0
    for t in range(int(inp["T"])):
        slots = [int(inp["block_table"][t][p // bs]) * bs + int(p) % bs for p in inp["indices"][t][:rows]]
        sc = inp["scale"] * (bf16(inp["query"][t]) @ kvall[slots].T + bf16(inp["query_rope"][t]) @ krall[slots].T)
        tmax = sc.reshape(sc.shape[0], rows // 32, 32).max(axis=2)
        run = np.maximum.accumulate(tmax, axis=1)
        jumps += int((tmax[:, 1:] > run[:, :-1] + 8.0).sum())
    return jumps


def test_wide_score_spread():
    """The attention kernel takes its exponentials against a reference that
    lags the running maximum by up to 8 and rescales O only when a tile
    passes it by more.  With scores spread this widely later tiles do, so the
    rescale runs after the first tile too; softmax_max and softmax_sum (the
    sum referred back to the true maximum) are compared as well."""
    inp = wide_spread_inputs()
    assert tile_jumps(inp) > 0
    check(inp)


@pytest.mark.parametrize("name", ["ragged_t5", "heads80_t4"])
def test_concatenated_cache(name):
    check(make_sfa_inputs(replace(SMALL[name], concat=True)))


def test_without_softmax_outputs():
    check(make_sfa_inputs(SMALL["ragged_t5"]), lse=False)


def test_empty_and_out_of_range_selections():
    inp = make_sfa_inputs(SMALL["ragged_t5"])
    inp["indices"][1] = -1                                   # nothing selected
    inp["indices"][2, ::3] = inp["seq_lens"][2] + 5          # past the kv length
    inp["block_table"][3, 1] = inp["block_num"] + 7          # a table entry out of range
    inp["block_table"][4, 0] = -1
    got = check(inp)
    assert not got["attention_out"][1].any() and np.all(np.isneginf(got["softmax_max"][1]))


def test_deterministic():
    inp = make_sfa_inputs(SMALL["heads80_t4"])
    say("case determinism heads80_t4")
    a, b = run_gpu(inp), run_gpu(inp, repeat=2)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_model_decode_t32():
    inp = make_sfa_inputs(sfa_workload("sfa_decode_t32"))
    check(inp, rows=[0, 5, 13, 31])


def test_model_concatenated_t4():
    wl = replace(sfa_workload("sfa_decode_t32"), name="sfa_decode_t4_concat", T=4, concat=True, len_lo=2500,
                 len_hi=5000)
    check(make_sfa_inputs(wl))


def test_consumes_the_prolog_caches():
    """The prolog writes two sequences' rows into the paged caches; the
    attention then reads them back through block tables rebuilt from the
    prolog's cacheIndex, with the prolog's own queries of each sequence's
    last token.  The oracle runs on host copies of the same device data."""
    from synth.generate import Dims, custom_workload
    import synth
    L, bs = 64, 16
    wl = custom_workload("prolog_for_sfa", T=2 * L, dims=Dims(He=256, Hcq=64, Hckv=64, N=4, D=32, Dr=32),
                         block_num=16, block_size=bs, seed=61, positions=f"prefill:2x{L}")
    pin = synth.make_inputs(wl)
    say("case the prolog's caches and queries read by the attention")
    t = dev.upload(pin)
    with mla.MlaProlog(mla.make_desc(**dev.desc_args(pin))) as h:
        h.run(t, 2 * L)
        torch.cuda.synchronize()
    d = pin["dims"]
    last = [L - 1, 2 * L - 1]
    idx = np.asarray(pin["cache_index"])
    table = np.stack([idx[s * L:(s + 1) * L:bs] // bs for s in range(2)]).astype(np.int32)
    rng = np.random.default_rng(5)
    inp = {"workload": "prolog_for_sfa", "T": 2, "N": d.N, "D": d.Hckv, "Dr": d.Dr, "block_size": bs, "K": 40,
           "sparse_block_size": 1, "concat": False, "scale": 1.0 / np.sqrt(d.Hckv + d.Dr),
           "seq_lens": np.array([L, L], np.int32), "block_table": table, "max_blocks": table.shape[1],
           "block_num": int(pin["block_num"]),
           "indices": np.stack([rng.permutation(L)[:40] for _ in range(2)]).astype(np.int32),
           "query": dev.bits(t["query_out"])[last], "query_rope": dev.bits(t["query_rope_out"])[last],
           "kv_cache": dev.bits(t["kv_cache"]), "kr_cache": dev.bits(t["kr_cache"])}
    check(inp)


def test_smaller_run_than_max_tokens():
    # the handle's split workspace is sized for 40 tokens; a run of 7 uses the
    # first tokens' rows only
    inp = make_sfa_inputs(SMALL["ragged_t5"])
    wl = replace(SMALL["ragged_t5"], T=40)
    big = make_sfa_inputs(wl)
    say("case sparse attention T=7 of max 40")
    t = {"query": big["query"], "query_rope": big["query_rope"], "kv_cache": big["kv_cache"],
         "kr_cache": big["kr_cache"], "sparse_indices": big["indices"], "block_table": big["block_table"],
         "seq_lens_kv": big["seq_lens"]}
    g = {k: dev._tensor(np.asarray(v), "cuda:0") for k, v in t.items()}
    N, D = int(big["N"]), int(big["D"])
    g["attention_out"] = torch.zeros((40, N, D), dtype=torch.bfloat16, device="cuda:0")
    desc = mla.make_sfa_desc(N=N, D=D, Dr=int(big["Dr"]), block_num=int(big["block_num"]),
                             block_size=int(big["block_size"]), max_blocks=int(big["max_blocks"]),
                             sparse_size=int(big["K"]), sparse_block_size=1, max_tokens=40,
                             scale=float(big["scale"]))
    with mla.MlaSfa(desc) as h:
        h.run(g, 7)
        torch.cuda.synchronize()
    out = dev.bits(g["attention_out"])
    ref = oracle.sfa(big, tokens=list(range(7)))
    g7, r7 = bf16(out[:7]), bf16(ref["attention_out"])
    tol = 2.0 ** -8 * (weighted_abs(big, list(range(7))) + np.abs(r7)) + 1e-6
    assert np.all(np.abs(g7 - r7) <= tol)
    assert not out[7:].any(), "rows past T were written"
    del inp
