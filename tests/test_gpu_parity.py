"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs, at the tolerances of tests/parity.py.

Small shapes are compared element by element over every token; the full
model-size workloads are compared on sampled tokens (all of their queries and
cache rows), plus a bitwise scan of every untouched cache slot.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from synth import device as dev
from synth.generate import Dims, custom_workload
from parity import check_caches, check_queries, tie_allowance

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import head_latent_attention_amd as mla  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


WEIGHTS = ("weight_dq", "weight_uq_qr", "weight_uk", "weight_dkv_kr")


def run_gpu(inp, query_int8=None, max_tokens=None, T=None, repeat=1, packed=False, prerun_negated=False,
            drop_unpacked=False):
    """Upload, run through the C ABI, download.  Returns host arrays.  With
    ``packed`` the weights are first converted by mla_prolog_pack_weights
    and the run reads the packed copy (with ``drop_unpacked`` the runs get
    no unpacked weights at all).  With ``prerun_negated`` the handle first
    runs once on -x (every intermediate differs), so that a result left in
    the workspace by an earlier run cannot pass for this one's."""
    T = int(inp["T"]) if T is None else T
    t = dev.upload(inp, query_int8=query_int8)
    desc = mla.make_desc(**dev.desc_args(inp, max_tokens=max_tokens, query_int8=query_int8))
    with mla.MlaProlog(desc) as h:
        if packed:
            buf = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
            h.pack_weights(t, buf)
            t["packed_weights"] = buf
            if drop_unpacked:
                for k in WEIGHTS:
                    del t[k]
                torch.cuda.synchronize()
        if prerun_negated:
            h.run(dict(t, token_x=-t["token_x"]), T)
        for _ in range(repeat):
            h.run(t, T)
        torch.cuda.synchronize()
    return {k: dev.bits(v) for k, v in t.items()
            if k in ("query_out", "query_rope_out", "dequant_scale_q_nope", "kv_cache", "kr_cache")}


def split_concat(inp, arrays):
    """queryOut and kvCache of the concatenated layout as the separate
    outputs (q^N | q^R and c^KV | k^R side by side)."""
    d = inp["dims"]
    out = dict(arrays)
    if arrays.get("query_out") is not None:
        q = np.asarray(arrays["query_out"])
        out["query_out"], out["query_rope_out"] = q[..., :d.Hckv], q[..., d.Hckv:]
    if arrays.get("kv_cache") is not None:
        kv = np.asarray(arrays["kv_cache"])
        out["kv_cache"], out["kr_cache"] = kv[..., :d.Hckv], kv[..., d.Hckv:]
    return out


def full_check(inp, query_int8=None, rows=None, packed=False, repeat=1, prerun_negated=False, drop_unpacked=False):
    q8 = bool(inp["quant"]) if query_int8 is None else bool(query_int8)
    rows = np.arange(int(inp["T"])) if rows is None else np.asarray(rows)
    say(f"case {inp['workload']} T={inp['T']} dims={inp['dims']} q8={q8} rows={len(rows)} packed={packed} "
        f"static={inp.get('preprocess', False)} concat={inp.get('concat', False)} nk={inp.get('weight_nk', False)}")
    got = run_gpu(inp, query_int8=query_int8, packed=packed, repeat=repeat, prerun_negated=prerun_negated,
                  drop_unpacked=drop_unpacked)
    partial = bool(inp.get("partial", False))
    ref = oracle.run(inp, tokens=rows, query_int8=query_int8, caches=False, intermediates=True)
    if inp.get("concat", False):
        got, ref, inp = split_concat(inp, got), split_concat(inp, ref), split_concat(inp, inp)
    allow = None
    if partial:
        # int8 c^Q from a float y: codes at a rounding tie may go either way
        aqr, aqn, namb = tie_allowance(inp, ref, rows)
        allow = (aqr, aqn)
        say(f"  c^Q codes within the tie band: {namb}")
    check_queries(got, ref, rows, q8, allow, fp16=bool(inp.get("fp16", False)), inp=inp)
    check_caches(inp, got["kv_cache"], got["kr_cache"], ref, rows)
    return got


SMALL = {
    "tiny_t4": synth.workload("tiny_t4"),
    "ragged_t37": custom_workload("ragged_t37", T=37, dims=Dims(He=264, Hcq=72, Hckv=40, N=3, D=24, Dr=16),
                                  block_num=4, block_size=16, seed=31),
    "ragged_t5_wide": custom_workload("ragged_t5_wide", T=5, dims=Dims(He=520, Hcq=200, Hckv=136, N=5, D=136, Dr=64),
                                      block_num=2, block_size=32, seed=32),
    "mid_t70": custom_workload("mid_t70", T=70, dims=Dims(He=1024, Hcq=256, Hckv=512, N=4, D=128, Dr=64),
                               block_num=8, block_size=16, seed=33),
    "t300_split1": custom_workload("t300", T=600, dims=Dims(He=512, Hcq=128, Hckv=64, N=2, D=32, Dr=16),
                                   block_num=40, block_size=16, seed=34),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_bf16(name):
    full_check(synth.make_inputs(SMALL[name]))


INT8_SMALL = {
    "q8_t9": custom_workload("q8_t9", T=9, dims=Dims(He=256, Hcq=64, Hckv=32, N=2, D=16, Dr=16),
                             block_num=2, block_size=16, quant=True, seed=41),
    "q8_t130": custom_workload("q8_t130", T=130, dims=Dims(He=1024, Hcq=192, Hckv=512, N=3, D=128, Dr=64),
                               block_num=16, block_size=16, quant=True, seed=42),
}


@pytest.mark.parametrize("name", list(INT8_SMALL))
def test_small_int8(name):
    full_check(synth.make_inputs(INT8_SMALL[name]))


def test_int8_inputs_bf16_query():
    full_check(synth.make_inputs(INT8_SMALL["q8_t130"]), query_int8=False)


def test_deterministic():
    inp = synth.make_inputs(SMALL["mid_t70"])
    say("case determinism mid_t70")
    a = run_gpu(inp)
    b = run_gpu(inp, repeat=2)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_zero_tokens_is_a_no_op():
    inp = synth.make_inputs(SMALL["tiny_t4"])
    say("case T=0")
    got = run_gpu(inp, T=0)
    assert np.all(got["kv_cache"] == synth.SENTINEL_BF16)
    assert not np.asarray(got["query_out"]).any()


def test_no_cache_blocks_still_computes_queries():
    wl = custom_workload("nocache", T=6, dims=Dims(He=256, Hcq=64, Hckv=32, N=2, D=16, Dr=8),
                         block_num=1, block_size=16, seed=51)
    inp = synth.make_inputs(wl)
    say("case block_num=0")
    t = dev.upload(inp)
    t.pop("kv_cache"), t.pop("kr_cache")
    args = dev.desc_args(inp)
    args["block_num"] = 0
    with mla.MlaProlog(mla.make_desc(**args)) as h:
        h.run(t, 6)
        torch.cuda.synchronize()
    ref = oracle.run(inp, caches=False, intermediates=True)
    got = {k: dev.bits(v) for k, v in t.items()}
    check_queries(got, ref, np.arange(6), False, inp=inp)


def test_out_of_range_slots_are_skipped():
    inp = synth.make_inputs(SMALL["ragged_t37"])
    n = inp["block_num"] * inp["block_size"]
    idx = np.array(inp["cache_index"])
    idx[:3] = [-5, n, n + 1000]
    inp["cache_index"] = idx
    full_check(inp)


def test_smaller_run_than_max_tokens():
    inp = synth.make_inputs(SMALL["mid_t70"])
    say("case T=19 of max 70")
    small = synth.make_inputs(SMALL["mid_t70"], T=19)
    got = run_gpu(small, max_tokens=70)
    ref = oracle.run(small, caches=False, intermediates=True)
    check_queries(got, ref, np.arange(19), False, inp=small)
    check_caches(small, got["kv_cache"], got["kr_cache"], ref, np.arange(19))


# ---- the model-size workloads, sampled ---------------------------------------
FULL = ["decode_t32", "decode_t256", "int8_decode_t128", "prefill_t8192"]


def check_rows(inp, seed=0):
    """The rows a full-size workload is compared on: every token up to 256
    tokens; above, one random row of every 64-token tile (the largest token
    tile of any launch shape) plus the first and last token of every
    sequence (where the positions restart at 0) and of the run."""
    T = int(inp["T"])
    if T <= 256:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    rows = {0, T - 1}
    for t0 in range(0, T, 64):
        rows.add(int(rng.integers(t0, min(T, t0 + 64))))
    pos = np.asarray(inp.get("positions", np.arange(T)))
    for s in np.flatnonzero(pos == 0):
        rows |= {int(s), max(0, int(s) - 1)}
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    inp = synth.make_inputs(synth.workload(name))
    full_check(inp, rows=check_rows(inp))


# ---- packed weights -----------------------------------------------------------
def packed_reference(inp):
    """The packed layout restated with numpy: per matrix, 64-column windows,
    each as k-stages of 4 column tiles x 64 lanes x 16 bytes; lane l of tile
    ct holds rows KL*(l//16)+i of column 16*ct + l%16."""
    d = inp["dims"]
    i8 = bool(inp["quant"]) or bool(inp.get("preprocess", False))   # W^DQ, W^DkvKr
    i8u = i8 or bool(inp.get("partial", False))                      # W^UqQr

    def kn(key):   # a weight as (k, n)
        w = np.asarray(inp[key])
        return w.T if inp.get("weight_nk", False) else w

    def windows_of(W, cols, K, kl):
        out = []
        ks = 4 * kl
        nst = -(-K // ks)
        for col0, width in cols:
            blk = np.zeros((nst * ks, 64), dtype=W.dtype)
            blk[:K, :width] = W[:, col0:col0 + width]
            st = blk.reshape(nst, 4, kl, 64)                    # stage, lane group, i, column
            st = st.reshape(nst, 4, kl, 4, 16)                  # .., column tile, column in tile
            st = st.transpose(0, 3, 1, 4, 2)                    # stage, ct, group, col, i
            out.append(np.ascontiguousarray(st).view(np.uint8).ravel())
        return out

    kl = 16 if i8 else 8
    klu = 16 if i8u else 8
    parts = []
    wdq = kn("weight_dq")
    parts += windows_of(wdq, [(c, min(64, d.Hcq - c)) for c in range(0, d.Hcq, 64)], d.He, kl)
    wkr = kn("weight_dkv_kr")
    nkr = d.Hckv + d.Dr
    parts += windows_of(wkr, [(c, min(64, nkr - c)) for c in range(0, nkr, 64)], d.He, kl)
    wuq = kn("weight_uq_qr")
    cols = []
    for h in range(d.N):
        base = h * (d.D + d.Dr)
        cols += [(base + c, min(64, d.D - c)) for c in range(0, d.D, 64)] + [(base + d.D, d.Dr)]
    parts += windows_of(wuq, cols, d.Hcq, klu)
    wuk = np.asarray(inp["weight_uk"])
    for h in range(d.N):
        parts += windows_of(wuk[h], [(c, min(64, d.Hckv - c)) for c in range(0, d.Hckv, 64)], d.D, 8)
    return np.concatenate(parts)


@pytest.mark.parametrize("name", ["tiny_t4", "ragged_t5_wide", "partial_t37", "tiny_pre_t4"])
def test_packed_layout(name):
    inp = synth.make_inputs(SMALL[name] if name in SMALL else PARTIAL[name] if name in PARTIAL
                            else synth.workload(name))
    say(f"case pack layout {name}")
    t = dev.upload(inp)
    desc = mla.make_desc(**dev.desc_args(inp))
    with mla.MlaProlog(desc) as h:
        buf = torch.zeros(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
        h.pack_weights(t, buf)
        torch.cuda.synchronize()
    ref = packed_reference(inp)
    assert buf.numel() == ref.size
    assert np.array_equal(buf.cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["tiny_t4", "ragged_t5_wide"])
def test_small_bf16_packed(name):
    full_check(synth.make_inputs(SMALL[name]), packed=True)


def test_small_int8_packed():
    full_check(synth.make_inputs(INT8_SMALL["q8_t9"]), packed=True)
    full_check(synth.make_inputs(INT8_SMALL["q8_t9"]), query_int8=False, packed=True)


def test_full_size_decode_packed():
    inp = synth.make_inputs(synth.workload("decode_t32"))
    full_check(inp, packed=True)


def test_int8_decode_t32_packed():
    # the int8 decode workload at 32 tokens runs on the packed small-T kernels
    inp = synth.make_inputs(synth.workload("int8_decode_t128"), T=32)
    full_check(inp, packed=True)


# ---- packed weights, two blocks per head (two nope windows, Dr = 64) ---------
# The halves of a head trade q^C (and, for the int8 query, the row maxima)
# through flags that every run must leave at zero: each case runs on -x
# first and then three times on x, on one handle.  Head counts with N % 8 == 0 and without take the two
# block-to-head mappings; Hckv = 320 leaves the second half one W^UK window
# short; D = 96 leaves the second nope window half empty.
PAIR = {
    "pair_t5_n4": custom_workload("pair_t5_n4", T=5, dims=Dims(He=512, Hcq=256, Hckv=128, N=4, D=128, Dr=64),
                                  block_num=2, block_size=16, seed=70),
    "pair_t32_n8": custom_workload("pair_t32_n8", T=32, dims=Dims(He=256, Hcq=192, Hckv=320, N=8, D=96, Dr=64),
                                   block_num=4, block_size=16, seed=71),
    "pair_t16_n16": custom_workload("pair_t16_n16", T=16, dims=Dims(He=384, Hcq=128, Hckv=512, N=16, D=128, Dr=64),
                                    block_num=2, block_size=16, seed=72),
    "pair_t27_n3": custom_workload("pair_t27_n3", T=27, dims=Dims(He=256, Hcq=160, Hckv=64, N=3, D=72, Dr=64),
                                   block_num=3, block_size=16, seed=73),
}
PAIR_INT8 = {
    "pair_q8_t17_n16": custom_workload("pair_q8_t17_n16", T=17, dims=Dims(He=512, Hcq=256, Hckv=256, N=16, D=128, Dr=64),
                                       block_num=2, block_size=16, seed=74, quant=True),
    "pair_q8_t3_n3": custom_workload("pair_q8_t3_n3", T=3, dims=Dims(He=256, Hcq=128, Hckv=320, N=3, D=96, Dr=64),
                                     block_num=1, block_size=16, seed=75, quant=True),
}


@pytest.mark.parametrize("name", list(PAIR))
def test_pair_bf16_packed(name):
    full_check(synth.make_inputs(PAIR[name]), packed=True, repeat=3, prerun_negated=True)


@pytest.mark.parametrize("name", ["pair_t5_n4", "pair_t32_n8"])
def test_pair_bf16_packed_unfused(name, monkeypatch):
    # the bf16 cases above run on the one-kernel path; this keeps the paired
    # kernel that serves when not all blocks of that launch fit on the device
    monkeypatch.setenv("MLA_PROLOG_FUSED", "0")
    full_check(synth.make_inputs(PAIR[name]), packed=True, repeat=2, prerun_negated=True)


def test_fused_mixed_token_counts():
    # one handle, runs of 32, 7, 16 and 32 tokens: the one-kernel path's
    # counters only grow, and each run must wait for its own arrivals
    wl = PAIR["pair_t32_n8"]
    desc_inp = synth.make_inputs(wl)
    desc = mla.make_desc(**dev.desc_args(desc_inp))
    with mla.MlaProlog(desc) as h:
        t0 = dev.upload(desc_inp)
        buf = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
        h.pack_weights(t0, buf)
        for T in (32, 7, 16, 32):
            inp = synth.make_inputs(wl, T=T)
            say(f"case fused mixed T={T}")
            t = dev.upload(inp)
            t["packed_weights"] = buf
            h.run(t, T)
            torch.cuda.synchronize()
            h.check()
            got = {k: dev.bits(v) for k, v in t.items() if k != "packed_weights"}
            ref = oracle.run(inp, caches=False, intermediates=True)
            check_queries(got, ref, np.arange(T), False, inp=inp)
            check_caches(inp, got["kv_cache"], got["kr_cache"], ref, np.arange(T))


def test_fused_gave_up_is_reported(monkeypatch):
    # a poll limit of one step makes the one-kernel path's waits give up
    # (every access stays in bounds and the kernel ends normally); the
    # handle must report it, and a fresh handle must not
    inp = synth.make_inputs(PAIR["pair_t16_n16"])
    say("case fused wait gives up")
    monkeypatch.setenv("MLA_PROLOG_FUSED_SPIN", "1")
    t = dev.upload(inp)
    desc = mla.make_desc(**dev.desc_args(inp))
    h = mla.MlaProlog(desc)
    buf = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
    h.pack_weights(t, buf)
    t["packed_weights"] = buf
    h.run(t, int(inp["T"]))
    torch.cuda.synchronize()
    # the give-up is visible to the host: the next run is refused, nothing
    # enqueued, until check() has reported it
    with pytest.raises(mla.MlaError) as e:
        h.run(t, int(inp["T"]))
    assert e.value.status == mla.MLA_ERR_RUNTIME
    with pytest.raises(mla.MlaError):
        h.check()
    h.check()   # the record was cleared
    h.set_poll_limit(0)
    h.run(t, int(inp["T"]))   # accepted again
    h.check()
    h.close()
    monkeypatch.delenv("MLA_PROLOG_FUSED_SPIN")
    full_check(inp, packed=True)


@pytest.mark.parametrize("path", ["one_launch", "paired"])
def test_run_after_a_wait_gave_up_is_correct(path, monkeypatch):
    # One handle: runs whose bounded waits are capped at one poll step (the
    # blocks waited for are often not there yet, so waits give up and leave
    # flags and tags of those runs behind; every access stays in bounds and
    # the kernels end normally), check() reports it; then the default limit,
    # and the next runs on the same workspace must match the oracle.  The
    # one-launch path waits on every block of the launch, so its runs give up
    # every time, and its q^C trade between a head's two blocks uses the
    # same exchange flags as the paired path.  In the paired path the two
    # blocks of a head reach their trade together (q^C, and with the int8
    # query the row maxima), so a one-step poll may or may not give up.
    if path == "paired":
        monkeypatch.setenv("MLA_PROLOG_FUSED", "0")
        inp = synth.make_inputs(PAIR_INT8["pair_q8_t17_n16"])
    else:
        inp = synth.make_inputs(PAIR["pair_t16_n16"])
    say(f"case wait gave up, then normal runs ({path})")
    T = int(inp["T"])
    q8 = bool(inp["quant"])
    t = dev.upload(inp)
    desc = mla.make_desc(**dev.desc_args(inp))
    with mla.MlaProlog(desc) as h:
        buf = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
        h.pack_weights(t, buf)
        t["packed_weights"] = buf
        h.set_poll_limit(1)
        gave_up = 0
        for _ in range(8):
            h.run(dict(t, token_x=-t["token_x"]), T)   # refused only after a give-up that check() clears
            try:
                h.check()
            except mla.MlaError:
                gave_up += 1
        say(f"  runs that gave up: {gave_up} of 8")
        if path == "one_launch":
            assert gave_up > 0
        h.set_poll_limit(0)
        for _ in range(2):
            h.run(t, T)
            torch.cuda.synchronize()
            h.check()
            got = {k: dev.bits(v) for k, v in t.items() if k != "packed_weights"}
            ref = oracle.run(inp, caches=False, intermediates=True)
            check_queries(got, ref, np.arange(T), q8, inp=inp)
            check_caches(inp, got["kv_cache"], got["kr_cache"], ref, np.arange(T))


@pytest.mark.parametrize("name", list(PAIR_INT8))
def test_pair_int8_packed(name):
    inp = synth.make_inputs(PAIR_INT8[name])
    full_check(inp, packed=True, repeat=3, prerun_negated=True)
    full_check(inp, query_int8=False, packed=True, repeat=3, prerun_negated=True)


# ---- packed weights, tiled kernels (token counts above 32) -------------------
TILED = {
    "ragged_t37": SMALL["ragged_t37"],
    "mid_t70": SMALL["mid_t70"],
    "ragged_t150_wide": custom_workload("ragged_t150_wide", T=150,
                                        dims=Dims(He=520, Hcq=200, Hckv=136, N=5, D=136, Dr=64),
                                        block_num=16, block_size=16, seed=35),
    "t600": SMALL["t300_split1"],
    "t2100_large": custom_workload("t2100_large", T=2100,
                                   dims=Dims(He=264, Hcq=72, Hckv=40, N=3, D=24, Dr=16),
                                   block_num=160, block_size=16, seed=36),
    # the long-run kernels at Dr = 64: a ragged last token tile, a ragged
    # last window group (15 windows), a half-empty second nope window (D = 96)
    # and an odd k-stage count (Hcq = 200)
    "t2100_wide": custom_workload("t2100_wide", T=2100,
                                  dims=Dims(He=520, Hcq=200, Hckv=136, N=5, D=96, Dr=64),
                                  block_num=160, block_size=16, seed=38),
}


@pytest.mark.parametrize("name", list(TILED))
def test_tiled_bf16_packed(name):
    full_check(synth.make_inputs(TILED[name]), packed=True)


def test_tiled_int8_packed():
    inp = synth.make_inputs(INT8_SMALL["q8_t130"])
    full_check(inp, packed=True)
    full_check(inp, query_int8=False, packed=True)


def test_tiled_int8_large_packed():
    wl = custom_workload("q8_t2100", T=2100, dims=Dims(He=512, Hcq=128, Hckv=96, N=3, D=32, Dr=32),
                         block_num=160, block_size=16, seed=37, quant=True)
    full_check(synth.make_inputs(wl), packed=True)


@pytest.mark.parametrize("name", ["decode_t256", "int8_decode_t128", "prefill_t8192"])
def test_full_size_tiled_packed(name):
    inp = synth.make_inputs(synth.workload(name))
    full_check(inp, rows=check_rows(inp), packed=True)


# model shapes at medium token counts past the ring kernel, where the launch
# mixes medium and large kernel shapes: 300 (the 256 x 256 up-projection),
# 1000 (also the long-run W^UK kernel), 1900 (also the 256 x 256
# down-projection)
MODEL_DIMS = Dims(He=7168, Hcq=1536, Hckv=512, N=128, D=128, Dr=64)


# the long-run int8-query W^UK kernel (whole 512-column rows per wave) from
# 448 tokens on: model shapes, and small dims with a half-width last window
# (Hckv 96) and a ragged token tail
def test_full_size_int8_query_long_run_packed():
    wl = custom_workload("model_q8_t900", T=900, dims=MODEL_DIMS, block_num=10, block_size=128, quant=True, seed=611)
    inp = synth.make_inputs(wl)
    full_check(inp, rows=check_rows(inp), packed=True)


def test_int8_query_long_run_ragged_packed():
    wl = custom_workload("q8_t780", T=780, dims=Dims(He=512, Hcq=128, Hckv=96, N=3, D=32, Dr=32),
                         block_num=50, block_size=16, seed=612, quant=True)
    full_check(synth.make_inputs(wl), packed=True)


@pytest.mark.parametrize("T", [300, 1000, 1900])
def test_full_size_medium_mixed_packed(T):
    wl = custom_workload(f"model_t{T}", T=T, dims=MODEL_DIMS, block_num=(T + 127) // 128 + 2, block_size=128,
                         seed=500 + T)
    inp = synth.make_inputs(wl)
    full_check(inp, rows=check_rows(inp), packed=True)


# ---- the medium-T up-projection in (head, half) blocks (two nope windows,
# Dr = 64): D = 96 leaves the second nope window half empty, N = 3 takes the
# other block-to-head mapping, 33 / 128 / 129 / 256 tokens the ends of its
# two token-tile counts
RING_DIMS = {"n3_d96": Dims(He=512, Hcq=192, Hckv=128, N=3, D=96, Dr=64),
             "n8_d128": Dims(He=256, Hcq=128, Hckv=320, N=8, D=128, Dr=64)}


@pytest.mark.parametrize("T", [33, 128, 129, 256])
@pytest.mark.parametrize("dims", list(RING_DIMS))
@pytest.mark.parametrize("mode", ["bf16", "int8", "partial"])
def test_ring_up_projection_packed(mode, dims, T):
    wl = custom_workload(f"ring_{mode}_{dims}_t{T}", T=T, dims=RING_DIMS[dims], block_num=(T + 15) // 16 + 1,
                         block_size=16, quant=mode == "int8", partial=mode == "partial",
                         smooth=mode == "partial", seed=130 + T)
    full_check(synth.make_inputs(wl), packed=True, repeat=2, prerun_negated=True)


# ---- the token counts where the launch shapes change --------------------------
BOUNDARY_DIMS = Dims(He=512, Hcq=128, Hckv=64, N=2, D=32, Dr=16)


@pytest.mark.parametrize("T", [32, 33, 64, 65, 128, 129, 256, 257, 2047, 2048])
def test_shape_boundaries_bf16_packed(T):
    wl = custom_workload(f"boundary_t{T}", T=T, dims=BOUNDARY_DIMS, block_num=(T + 15) // 16 + 1,
                         block_size=16, seed=50 + T)
    full_check(synth.make_inputs(wl), packed=True)


@pytest.mark.parametrize("T", [32, 33, 64, 65, 100, 128, 129])
def test_shape_boundaries_int8_packed(T):
    wl = custom_workload(f"boundary_q8_t{T}", T=T, dims=Dims(He=512, Hcq=128, Hckv=96, N=2, D=32, Dr=32),
                         block_num=(T + 15) // 16 + 1, block_size=16, quant=True, seed=60 + T)
    full_check(synth.make_inputs(wl), packed=True)


# ---- partial quantisation (int8 weightUqQr only) and smoothScalesCq -----------
# The down-projection, norms and caches run the bf16 kernels; c^Q is quantised
# per token (times the smoothing factors) for the int8 up-projection kernels.
PARTIAL = {
    "tiny_partial_t4": synth.workload("tiny_partial_t4"),
    "partial_t37": custom_workload("partial_t37", T=37, dims=Dims(He=264, Hcq=80, Hckv=40, N=3, D=32, Dr=16),
                                   block_num=4, block_size=16, seed=81, partial=True, smooth=True),
    "partial_t6_nosmooth": custom_workload("partial_t6", T=6, dims=Dims(He=264, Hcq=64, Hckv=40, N=2, D=16, Dr=16),
                                           block_num=2, block_size=16, seed=82, partial=True),
    "pair_partial_t5_n4": custom_workload("pair_partial_t5_n4", T=5,
                                          dims=Dims(He=512, Hcq=256, Hckv=128, N=4, D=128, Dr=64),
                                          block_num=2, block_size=16, seed=83, partial=True, smooth=True),
    "pair_partial_t32_n8": custom_workload("pair_partial_t32_n8", T=32,
                                           dims=Dims(He=264, Hcq=192, Hckv=320, N=8, D=96, Dr=64),
                                           block_num=4, block_size=16, seed=84, partial=True, smooth=True),
    "partial_t130": custom_workload("partial_t130", T=130, dims=Dims(He=1032, Hcq=192, Hckv=504, N=3, D=128, Dr=64),
                                    block_num=16, block_size=16, seed=85, partial=True, smooth=True),
    "partial_t300": custom_workload("partial_t300", T=300, dims=Dims(He=520, Hcq=128, Hckv=64, N=2, D=32, Dr=16),
                                    block_num=20, block_size=16, seed=86, partial=True, smooth=True),
    "partial_t2100_large": custom_workload("partial_t2100", T=2100,
                                           dims=Dims(He=264, Hcq=64, Hckv=40, N=3, D=32, Dr=16),
                                           block_num=160, block_size=16, seed=87, partial=True, smooth=True),
}


@pytest.mark.parametrize("name", ["tiny_partial_t4", "partial_t37", "partial_t6_nosmooth"])
def test_partial_row_major(name):
    full_check(synth.make_inputs(PARTIAL[name]))


@pytest.mark.parametrize("name", list(PARTIAL))
def test_partial_packed(name):
    inp = synth.make_inputs(PARTIAL[name])
    full_check(inp, packed=True, repeat=2, prerun_negated=True)


@pytest.mark.parametrize("name", ["pair_partial_t5_n4", "pair_partial_t32_n8"])
def test_partial_packed_unfused(name, monkeypatch):
    # up to 32 tokens these run in one launch; this keeps the down-projection,
    # norm and paired int8 kernels that serve when not all of that launch's
    # blocks fit on the device
    monkeypatch.setenv("MLA_PROLOG_FUSED", "0")
    full_check(synth.make_inputs(PARTIAL[name]), packed=True, repeat=2, prerun_negated=True)


@pytest.mark.parametrize("T", [32, 33, 64, 65, 100, 128, 129])
def test_shape_boundaries_partial_packed(T):
    wl = custom_workload(f"boundary_partial_t{T}", T=T, dims=Dims(He=520, Hcq=128, Hckv=88, N=2, D=32, Dr=32),
                         block_num=(T + 15) // 16 + 1, block_size=16, partial=True, smooth=True, seed=90 + T)
    full_check(synth.make_inputs(wl), packed=True)


def test_full_size_partial_decode_packed():
    inp = synth.make_inputs(synth.workload("partial_decode_t32"))
    full_check(inp, packed=True)


SMOOTH_Q8 = {
    "q8_smooth_t9": custom_workload("q8_smooth_t9", T=9, dims=Dims(He=256, Hcq=64, Hckv=32, N=2, D=16, Dr=16),
                                    block_num=2, block_size=16, quant=True, smooth=True, seed=95),
    "q8_smooth_pair_t16": custom_workload("q8_smooth_pair_t16", T=16,
                                          dims=Dims(He=512, Hcq=256, Hckv=128, N=4, D=128, Dr=64),
                                          block_num=2, block_size=16, quant=True, smooth=True, seed=96),
    "q8_smooth_t130": custom_workload("q8_smooth_t130", T=130, dims=Dims(He=1024, Hcq=192, Hckv=512, N=3, D=128, Dr=64),
                                      block_num=16, block_size=16, quant=True, smooth=True, seed=97),
}


@pytest.mark.parametrize("name", list(SMOOTH_Q8))
def test_int8_smoothed(name):
    inp = synth.make_inputs(SMOOTH_Q8[name])
    full_check(inp)
    full_check(inp, packed=True)
    full_check(inp, query_int8=False, packed=True)


# ---- KV-cache quantisation (quantScaleCkv / quantScaleCkr) --------------------
# int8 kv cache in full quantisation (kr stays bf16); int8 kv and kr caches in
# partial quantisation.  The cache rows are written by the norm kernel on
# every path; the cases cover the row-major, paired, tiled medium and tiled
# large launches, empty caches and skipped slots.
KVQ = {
    "kvq_full_t9": custom_workload("kvq_full_t9", T=9, dims=Dims(He=256, Hcq=64, Hckv=32, N=2, D=16, Dr=16),
                                   block_num=2, block_size=16, quant=True, kv_quant=True, seed=101),
    "kvq_full_pair_t16": custom_workload("kvq_full_pair_t16", T=16,
                                         dims=Dims(He=512, Hcq=256, Hckv=128, N=4, D=128, Dr=64),
                                         block_num=2, block_size=16, quant=True, kv_quant=True, seed=102),
    "kvq_full_t130": custom_workload("kvq_full_t130", T=130,
                                     dims=Dims(He=1024, Hcq=192, Hckv=512, N=3, D=128, Dr=64),
                                     block_num=16, block_size=16, quant=True, kv_quant=True, smooth=True, seed=103),
    "kvq_partial_t5": custom_workload("kvq_partial_t5", T=5, dims=Dims(He=512, Hcq=256, Hckv=128, N=4, D=128, Dr=64),
                                      block_num=2, block_size=16, partial=True, smooth=True, kv_quant=True, seed=104),
    "kvq_partial_t37": custom_workload("kvq_partial_t37", T=37, dims=Dims(He=264, Hcq=80, Hckv=40, N=3, D=32, Dr=16),
                                       block_num=4, block_size=16, partial=True, kv_quant=True, seed=105),
    "kvq_partial_t300": custom_workload("kvq_partial_t300", T=300, dims=Dims(He=520, Hcq=128, Hckv=64, N=2, D=32, Dr=16),
                                        block_num=20, block_size=16, partial=True, smooth=True, kv_quant=True, seed=106),
    "kvq_partial_t2100": custom_workload("kvq_partial_t2100", T=2100,
                                         dims=Dims(He=264, Hcq=64, Hckv=40, N=3, D=32, Dr=16),
                                         block_num=160, block_size=16, partial=True, kv_quant=True, seed=107),
}


@pytest.mark.parametrize("name", ["kvq_full_t9", "kvq_partial_t37"])
def test_quantised_cache_row_major(name):
    full_check(synth.make_inputs(KVQ[name]))


@pytest.mark.parametrize("name", list(KVQ))
def test_quantised_cache_packed(name):
    inp = synth.make_inputs(KVQ[name])
    full_check(inp, packed=True, repeat=2, prerun_negated=True)


def test_quantised_cache_skipped_slots_and_no_blocks():
    inp = synth.make_inputs(KVQ["kvq_partial_t5"])
    n = inp["block_num"] * inp["block_size"]
    inp["cache_index"] = np.array([-1, n, 0, n + 3, 1], dtype=np.int64)
    full_check(inp, packed=True)
    # no cache blocks: the queries are still computed and nothing is written
    wl = custom_workload("kvq_noblocks", T=5, dims=Dims(He=512, Hcq=256, Hckv=128, N=4, D=128, Dr=64),
                         block_num=1, block_size=16, partial=True, kv_quant=True, seed=108)
    inp0 = synth.make_inputs(wl)
    say("case kvq block_num=0")
    t = dev.upload(inp0)
    t.pop("kv_cache"), t.pop("kr_cache")
    args = dev.desc_args(inp0)
    args["block_num"] = 0
    with mla.MlaProlog(mla.make_desc(**args)) as h:
        h.run(t, 5)
        torch.cuda.synchronize()
    ref = oracle.run(inp0, caches=False, intermediates=True)
    rows = np.arange(5)
    check_queries({k: dev.bits(v) for k, v in t.items()}, ref, rows, False, tie_allowance(inp0, ref, rows)[:2],
                  inp=inp0)


def test_full_size_int8_quantised_cache_packed():
    inp = synth.make_inputs(synth.workload("int8_kvq_decode_t128"))
    full_check(inp, rows=check_rows(inp), packed=True)


# ---- the largest head dimensions the library takes (D = Hckv = 512, Dr = 64) --
# At small T these shapes run the per-window up-projection and W^UK kernels
# (16 D-stages, eight 64-column windows per head); above 32 tokens the tiled
# kernels.
MAXD = Dims(He=256, Hcq=128, Hckv=512, N=2, D=512, Dr=64)


@pytest.mark.parametrize("T", [5, 40])
def test_max_head_dims_bf16(T):
    wl = custom_workload(f"maxd_t{T}", T=T, dims=MAXD, block_num=4, block_size=16, seed=110 + T)
    inp = synth.make_inputs(wl)
    full_check(inp)
    full_check(inp, packed=True)


@pytest.mark.parametrize("T", [5, 40])
def test_max_head_dims_int8(T):
    wl = custom_workload(f"maxd_q8_t{T}", T=T, dims=MAXD, block_num=4, block_size=16, quant=True,
                         kv_quant=True, seed=120 + T)
    inp = synth.make_inputs(wl)
    full_check(inp, packed=True)
    full_check(inp, query_int8=False, packed=True)


# ---- the MLA preprocess page's static int8 scenario (quantMode 0), its
# concatenated layout (cacheMode 0) and transposed weights ------------------
def _pre(name, T, dims, seed, **kw):
    kw.setdefault("preprocess", True)
    kw.setdefault("concat", True)
    kw.setdefault("weight_nk", True)
    return custom_workload(name, T=T, dims=dims, block_num=max(2, -(-T // 16) + 1), block_size=16,
                           seed=seed, **kw)


MID = Dims(He=1024, Hcq=256, Hckv=512, N=4, D=128, Dr=64)
STATIC = {
    "pre_t4": synth.workload("tiny_pre_t4"),
    "pre_t37": _pre("pre_t37", 37, Dims(He=272, Hcq=80, Hckv=48, N=3, D=32, Dr=16), 91),
    "pre_t17_pair": _pre("pre_t17_pair", 17, Dims(He=512, Hcq=256, Hckv=256, N=8, D=128, Dr=64), 92),
    "pre_t9_pair": _pre("pre_t9_pair", 9, Dims(He=528, Hcq=320, Hckv=192, N=8, D=128, Dr=64), 99),
    "pre_t70": _pre("pre_t70", 70, MID, 93),
    "pre_t130": _pre("pre_t130", 130, Dims(He=1024, Hcq=192, Hckv=512, N=3, D=128, Dr=64), 94),
    "pre_t600": _pre("pre_t600", 600, Dims(He=512, Hcq=128, Hckv=64, N=2, D=32, Dr=16), 95),
    "pre_t2048": _pre("pre_t2048", 2048, Dims(He=512, Hcq=128, Hckv=64, N=2, D=32, Dr=16), 96),
}


@pytest.mark.parametrize("name", list(STATIC))
def test_static_packed(name):
    full_check(synth.make_inputs(STATIC[name]), packed=True, repeat=2, prerun_negated=True)


@pytest.mark.parametrize("name", ["pre_t9_pair", "pre_t17_pair"])
def test_static_packed_unfused(name, monkeypatch):
    # up to 32 tokens these run in one launch after the x quantiser; this
    # keeps the down-projection, norm and paired int8 kernels that serve when
    # not all of that launch's blocks fit on the device
    monkeypatch.setenv("MLA_PROLOG_FUSED", "0")
    full_check(synth.make_inputs(STATIC[name]), packed=True, repeat=2, prerun_negated=True)


def test_static_without_input_norm_packed():
    full_check(synth.make_inputs(_pre("pre_xq_t37", 37, Dims(He=272, Hcq=80, Hckv=48, N=3, D=32, Dr=16), 97,
                                      x_norm=False)), packed=True)


@pytest.mark.parametrize("concat", [False, True], ids=["split", "concat"])
def test_static_row_major(concat):
    # the unpacked kernels take (k, n) weights
    full_check(synth.make_inputs(_pre("pre_rm_t9", 9, Dims(He=256, Hcq=64, Hckv=32, N=2, D=16, Dr=16), 98,
                                      concat=concat, weight_nk=False)))


def test_full_size_static_decode_packed():
    inp = synth.make_inputs(synth.workload("pre_decode_t32"))
    full_check(inp, rows=np.arange(32), packed=True)


# the same scenario with the page's FLOAT16 input: every 16-bit float tensor,
# and the outputs, fp16; the tiled kernels at every T
STATIC_F16 = {
    "pre_f16_t4": synth.workload("tiny_pre_f16_t4"),
    "pre_f16_t37": _pre("pre_f16_t37", 37, Dims(He=272, Hcq=80, Hckv=48, N=3, D=32, Dr=16), 191, fp16=True),
    "pre_f16_t17_split": _pre("pre_f16_t17_split", 17, Dims(He=512, Hcq=256, Hckv=256, N=8, D=128, Dr=64), 192,
                              fp16=True, concat=False),
    "pre_f16_t70": _pre("pre_f16_t70", 70, MID, 193, fp16=True),
    "pre_f16_t130_split": _pre("pre_f16_t130_split", 130, Dims(He=1024, Hcq=192, Hckv=512, N=3, D=128, Dr=64),
                               194, fp16=True, concat=False),
    "pre_f16_t600": _pre("pre_f16_t600", 600, Dims(He=512, Hcq=128, Hckv=64, N=2, D=32, Dr=16), 195, fp16=True),
    "pre_f16_t2100": _pre("pre_f16_t2100", 2100, Dims(He=512, Hcq=128, Hckv=64, N=2, D=32, Dr=16), 196,
                          fp16=True),
    # a small-T run on the tiled down-projection with more He splits than
    # the small-T plans take (the workspace holds the partials of every
    # down-projection a run may take)
    "pre_f16_t17_he2048": _pre("pre_f16_t17_he2048", 17, Dims(He=2048, Hcq=1536, Hckv=512, N=2, D=128, Dr=64),
                               198, fp16=True),
}


@pytest.mark.parametrize("name", list(STATIC_F16))
def test_static_fp16_packed(name):
    full_check(synth.make_inputs(STATIC_F16[name]), packed=True, repeat=2, prerun_negated=True)


def test_static_fp16_without_input_norm_packed():
    full_check(synth.make_inputs(_pre("pre_f16_xq_t37", 37, Dims(He=272, Hcq=80, Hckv=48, N=3, D=32, Dr=16), 197,
                                      x_norm=False, fp16=True)), packed=True)


def test_full_size_static_fp16_decode_packed():
    inp = synth.make_inputs(synth.workload("pre_f16_decode_t32"))
    full_check(inp, rows=np.arange(32), packed=True)


def test_static_fp16_needs_packed_weights():
    inp = synth.make_inputs(STATIC_F16["pre_f16_t37"])
    say("case static fp16 without packed weights")
    t = dev.upload(inp)
    with mla.MlaProlog(mla.make_desc(**dev.desc_args(inp))) as h:
        with pytest.raises(mla.MlaError) as e:
            h.run(t, int(inp["T"]))
    assert e.value.status == mla.MLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["bf16_t16_one_launch", "bf16_t37", "int8_t130_ring", "static_t600",
                                  "static_fp16_t70", "bf16_t2100_large"])
def test_packed_runs_without_unpacked_weights(name):
    # with the packed copy given, a run reads no unpacked weight: the four
    # tensors are freed before it
    wl = {"bf16_t16_one_launch": custom_workload("nw_t16", T=16, dims=Dims(He=384, Hcq=128, Hckv=512, N=16, D=128,
                                                                          Dr=64), block_num=4, block_size=16,
                                                 seed=301),
          "bf16_t37": SMALL["ragged_t37"],
          "int8_t130_ring": INT8_SMALL["q8_t130"],
          "static_t600": STATIC["pre_t600"],
          "static_fp16_t70": STATIC_F16["pre_f16_t70"],
          "bf16_t2100_large": custom_workload("nw_t2100", T=2100, dims=Dims(He=264, Hcq=72, Hckv=40, N=3, D=24,
                                                                            Dr=16), block_num=160, block_size=16,
                                              seed=302)}[name]
    full_check(synth.make_inputs(wl), packed=True, drop_unpacked=True)


@pytest.mark.parametrize("name", ["bf16_t16_one_launch", "int8_t17_paired", "int8_q8_t130_ring", "bf16_t2100_large",
                                  "static_t37"])
def test_zero_tokens(name, monkeypatch):
    # tokens whose x is all zeros: y = 0, c^Q = 0 (eps keeps the norm
    # finite), the dynamic int8 scales of c^Q and q^N are 0 with codes 0
    wl = {"bf16_t16_one_launch": custom_workload("z_t16", T=16, dims=Dims(He=384, Hcq=128, Hckv=512, N=16, D=128,
                                                                         Dr=64), block_num=4, block_size=16, seed=311),
          "int8_t17_paired": PAIR_INT8["pair_q8_t17_n16"],
          "int8_q8_t130_ring": INT8_SMALL["q8_t130"],
          "bf16_t2100_large": custom_workload("z_t2100", T=2100, dims=Dims(He=264, Hcq=72, Hckv=40, N=3, D=24,
                                                                           Dr=16), block_num=160, block_size=16,
                                              seed=312),
          "static_t37": STATIC["pre_t37"]}[name]
    inp = synth.make_inputs(wl)
    T = int(inp["T"])
    x = np.array(inp["token_x"])
    for t in (0, T // 2, T - 1):
        x[t] = 0
    inp["token_x"] = x
    if name == "int8_t17_paired":
        monkeypatch.setenv("MLA_PROLOG_FUSED", "0")
    got = full_check(inp, packed=True)
    if inp["quant"]:
        # the zero tokens' int8 q^N is all zeros with scale 0
        for t in (0, T // 2, T - 1):
            assert not np.asarray(got["query_out"][t]).any()
            assert not np.asarray(got["dequant_scale_q_nope"][t]).any()


CONCAT_BF16 = {
    "cat_t5": _pre("cat_t5", 5, Dims(He=264, Hcq=72, Hckv=40, N=3, D=24, Dr=16), 101, preprocess=False),
    "cat_t32_pair": _pre("cat_t32_pair", 32, Dims(He=256, Hcq=192, Hckv=320, N=8, D=96, Dr=64), 102,
                         preprocess=False),
    "cat_t70": _pre("cat_t70", 70, MID, 103, preprocess=False),
    "cat_t2048": _pre("cat_t2048", 2048, Dims(He=512, Hcq=128, Hckv=64, N=2, D=32, Dr=16), 104,
                      preprocess=False),
}


@pytest.mark.parametrize("name", list(CONCAT_BF16))
def test_concat_bf16_packed(name):
    # cat_t32_pair runs on the one-kernel path
    full_check(synth.make_inputs(CONCAT_BF16[name]), packed=True, repeat=2, prerun_negated=True)


def test_concat_bf16_packed_unfused(monkeypatch):
    monkeypatch.setenv("MLA_PROLOG_FUSED", "0")
    full_check(synth.make_inputs(CONCAT_BF16["cat_t32_pair"]), packed=True)


def test_concat_bf16_row_major():
    wl = _pre("cat_rm_t37", 37, Dims(He=264, Hcq=72, Hckv=40, N=3, D=24, Dr=16), 105, preprocess=False,
              weight_nk=False)
    full_check(synth.make_inputs(wl))


def test_full_size_concat_decode_packed():
    from dataclasses import replace
    wl = replace(synth.workload("decode_t32"), name="decode_t32_concat", concat=True, weight_nk=True)
    full_check(synth.make_inputs(wl), rows=np.arange(32), packed=True)


@pytest.mark.parametrize("name", ["pre_t37", "cat_t32_pair"])
def test_concat_out_of_range_slots_are_skipped(name):
    # the concatenated rows are written whole or not at all
    wl = STATIC.get(name) or CONCAT_BF16[name]
    inp = synth.make_inputs(wl)
    n = inp["block_num"] * inp["block_size"]
    idx = np.array(inp["cache_index"])
    idx[:3] = [-1, n, n + 77]
    inp["cache_index"] = idx
    full_check(inp, packed=True)


def test_static_no_cache_blocks_still_computes_queries():
    inp = synth.make_inputs(STATIC["pre_t37"])
    say("case static, concatenated, block_num=0")
    t = dev.upload(inp)
    t.pop("kv_cache")
    args = dev.desc_args(inp)
    args["block_num"] = 0
    desc = mla.make_desc(**args)
    with mla.MlaProlog(desc) as h:
        buf = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
        h.pack_weights(t, buf)
        t["packed_weights"] = buf
        h.run(t, int(inp["T"]))
        torch.cuda.synchronize()
    ref = split_concat(inp, oracle.run(inp, caches=False, intermediates=True))
    got = split_concat(inp, {"query_out": dev.bits(t["query_out"])})
    check_queries(got, ref, np.arange(int(inp["T"])), False, inp=inp)


def test_static_smaller_run_than_max_tokens():
    say("case static T=23 of max 130")
    small = synth.make_inputs(STATIC["pre_t130"], T=23)
    d = small["dims"]
    t = dev.upload(small)
    desc = mla.make_desc(**dev.desc_args(small, max_tokens=130))
    with mla.MlaProlog(desc) as h:
        buf = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
        h.pack_weights(t, buf)
        t["packed_weights"] = buf
        h.run(t, 23)
        torch.cuda.synchronize()
    got = split_concat(small, {k: dev.bits(v) for k, v in t.items() if k in ("query_out", "kv_cache")})
    ref = split_concat(small, oracle.run(small, caches=False, intermediates=True))
    check_queries(got, ref, np.arange(23), False, inp=small)
    check_caches(split_concat(small, small), got["kv_cache"], got["kr_cache"], ref, np.arange(23))
