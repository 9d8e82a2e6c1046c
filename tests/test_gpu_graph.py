"""mla_prolog_run captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed, through the C ABI.

A captured run takes the kernels that hand no data across blocks, the same
selection as mla_prolog_run_noalloc, so every replay is compared bit for bit
with a no-allocation call on the same inputs.  Between replays the test
changes the contents of token_x in place, runs the no-allocation reference
and synchronises, as a serving loop would; a handle run after the replays
checks that eager runs of the same handle still agree.  The attention
consumer's run (mla_sfa_run) is captured and replayed the same way, each
replay compared bit for bit with an eager run.
"""
import sys

import numpy as np
import pytest

import synth
from synth import device as dev
from synth.generate import Dims, custom_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import head_latent_attention_amd as mla  # noqa: E402
from test_zz_no_alloc import compare, outputs  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = {
    # eagerly the one-launch kernel; captured, the stream-ordered kernels
    "bf16_t32": custom_workload("graph_bf16", T=32, dims=Dims(He=512, Hcq=256, Hckv=512, N=8, D=128, Dr=64),
                                block_num=4, block_size=16, seed=401),
    # eagerly the ring kernel with the W^UK product and its trades between
    # a head's blocks; captured, the ring kernel alone and the int8-query
    # W^UK kernel
    "int8_q8_t130": custom_workload("graph_q8", T=130, dims=Dims(He=1024, Hcq=192, Hckv=512, N=3, D=128, Dr=64),
                                    block_num=16, block_size=16, quant=True, seed=402),
    # the mixed medium kernels (the 256 x 256 up-projection, the long-run
    # W^UK kernels) and the long-run path, bf16 and the int8 query
    "bf16_t900": custom_workload("graph_t900", T=900, dims=Dims(He=520, Hcq=200, Hckv=136, N=5, D=96, Dr=64),
                                 block_num=64, block_size=16, seed=403),
    "int8_q8_t2100": custom_workload("graph_q8_t2100", T=2100, dims=Dims(He=512, Hcq=128, Hckv=96, N=3, D=32,
                                                                          Dr=32),
                                     block_num=140, block_size=16, quant=True, seed=404),
}


def other_x(x, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    if x.dtype == torch.int8:
        v = torch.randint(-127, 128, tuple(x.shape), generator=g, dtype=torch.int32).to(torch.int8)
    else:
        v = torch.randn(tuple(x.shape), generator=g).to(x.dtype)
    return v.to(x.device)


@pytest.mark.parametrize("name", list(CASES))
def test_captured_run_replays(name):
    inp = synth.make_inputs(CASES[name])
    T = int(inp["T"])
    desc = mla.make_desc(**dev.desc_args(inp))
    with mla.MlaProlog(desc) as h:
        tg = dev.upload(inp)
        packed = torch.empty(mla.packed_weights_bytes(desc), dtype=torch.uint8, device="cuda")
        h.pack_weights(tg, packed)
        tg["packed_weights"] = packed
        torch.cuda.synchronize()
        xs = [tg["token_x"].clone(), other_x(tg["token_x"], 7), tg["token_x"].clone()]
        say(f"case graph capture {name} T={T}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            h.run(tg, T)
        torch.cuda.synchronize()
        for i, x in enumerate(xs):
            say(f"case graph replay {name} #{i}")
            tg["token_x"].copy_(x)
            ref = dev.upload(inp)
            ref["packed_weights"] = packed
            ref["token_x"].copy_(x)
            mla.run_noalloc(desc, ref, T)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got, want = outputs(tg), outputs(ref)
            for k in want:
                assert np.array_equal(got[k], want[k]), f"replay {i}: {k} differs from the no-allocation call"
        h.check()
        # an eager run of the handle after the replays (its own kernels)
        say(f"case graph eager-after {name}")
        te = dev.upload(inp)
        te["packed_weights"] = packed
        te["token_x"].copy_(xs[1])
        h.run(te, T)
        torch.cuda.synchronize()
        h.check()
        ref = dev.upload(inp)
        ref["packed_weights"] = packed
        ref["token_x"].copy_(xs[1])
        mla.run_noalloc(desc, ref, T)
        torch.cuda.synchronize()
        compare(inp, outputs(te), outputs(ref))


def test_captured_run_refuses_the_index_check():
    inp = synth.make_inputs(CASES["bf16_t32"])
    T = int(inp["T"])
    desc = mla.make_desc(**dev.desc_args(inp), check_index=1)
    with mla.MlaProlog(desc) as h:
        tg = dev.upload(inp)
        torch.cuda.synchronize()
        say("case graph capture with the index check")
        g = torch.cuda.CUDAGraph()
        with pytest.raises(mla.MlaError) as e:
            with torch.cuda.graph(g):
                h.run(tg, T)
        assert e.value.status == mla.MLA_ERR_PARAM_INVALID
        torch.cuda.synchronize()


# ---- the attention consumer (mla_sfa_run): no data crosses blocks there, so
# a captured run replays as the eager one; split rows go through the combine
# kernel (long_t1) or not (heads80_t4)
SFA_CASES = ["heads80_t4", "long_t1"]


@pytest.mark.parametrize("name", SFA_CASES)
def test_captured_attention_replays(name):
    from synth.sfa import make_sfa_inputs
    from test_gpu_sfa import SMALL
    inp = make_sfa_inputs(SMALL[name])
    T, N, D = int(inp["T"]), int(inp["N"]), int(inp["D"])
    t = {"query": inp["query"], "query_rope": inp["query_rope"], "kv_cache": inp["kv_cache"],
         "kr_cache": inp["kr_cache"], "sparse_indices": inp["indices"], "block_table": inp["block_table"],
         "seq_lens_kv": inp["seq_lens"]}

    def tensors():
        g = {k: dev._tensor(np.asarray(v), "cuda:0") for k, v in t.items()}
        g["attention_out"] = torch.zeros((T, N, D), dtype=torch.bfloat16, device="cuda:0")
        g["softmax_max"] = torch.zeros((T, N), dtype=torch.float32, device="cuda:0")
        g["softmax_sum"] = torch.zeros((T, N), dtype=torch.float32, device="cuda:0")
        return g

    desc = mla.make_sfa_desc(N=N, D=D, Dr=int(inp["Dr"]), block_num=int(inp["block_num"]),
                             block_size=int(inp["block_size"]), max_blocks=int(inp["max_blocks"]),
                             sparse_size=int(inp["K"]), sparse_block_size=int(inp["sparse_block_size"]),
                             max_tokens=T, scale=float(inp["scale"]), concat=0)
    with mla.MlaSfa(desc) as h:
        gt = tensors()
        torch.cuda.synchronize()
        qs = [gt["query"].clone(), other_x(gt["query"], 11), gt["query"].clone()]
        say(f"case attention graph capture {name} T={T}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            h.run(gt, T)
        torch.cuda.synchronize()
        for i, q in enumerate(qs):
            say(f"case attention graph replay {name} #{i}")
            gt["query"].copy_(q)
            ref = tensors()
            ref["query"].copy_(q)
            h.run(ref, T)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k in ("attention_out", "softmax_max", "softmax_sum"):
                assert np.array_equal(dev.bits(gt[k]), dev.bits(ref[k])), f"replay {i}: {k} differs from the eager run"
