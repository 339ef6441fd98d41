"""The verify step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.  The
library allocates nothing, synchronises nothing and records no memset, so spec_verify with
a caller workspace, spec_verify_noalloc and spec_verify_philox capture as they are.  Each
replay runs on new inputs copied into the captured buffers, with eager work and a
synchronisation between replays, and equals an eager call on the same inputs bit for bit
(the kernels are deterministic)."""
import os

import numpy as np
import pytest
import torch

import speculative_decoding_verification_03_amd as sv
from speculative_decoding_verification_03_amd import workloads as W
from parity_util import to_host

pytestmark = pytest.mark.gpu

SEED = 1003


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(sv.lib_path), "libspecverify.so is not built"
    return torch.device("cuda:0")


def new_out(B, K, dev):
    return dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                p=torch.empty((B, K), dtype=torch.float32, device=dev),
                q=torch.empty((B, K), dtype=torch.float32, device=dev),
                status=torch.empty((B,), dtype=torch.int32, device=dev),
                uniforms=torch.empty((B, K + 1), dtype=torch.float32, device=dev))


def assert_same(got, ref, what):
    for k in ("tokens", "accept_len", "status"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{what}: {k}")
    for k in ("p", "q"):
        np.testing.assert_array_equal(np.isnan(got[k]), np.isnan(ref[k]), err_msg=f"{what}: {k} NaN")
        np.testing.assert_array_equal(np.nan_to_num(got[k]), np.nan_to_num(ref[k]), err_msg=f"{what}: {k}")


@pytest.mark.parametrize("entry", ["spec_verify", "spec_verify_noalloc", "spec_verify_philox"])
def test_graph_replays_equal_eager(dev, entry):
    cfg, step_philox = 3, 7
    say(f"graph capture of {entry}: {W.describe(cfg)}")
    x0 = W.make_inputs(cfg, step=0, device=dev)
    B, K = x0["B"], x0["K"]
    static = {k: x0[k].clone() for k in ("target", "draft", "tokens", "temperature")}
    u_static = torch.empty((B, K + 1), dtype=torch.float32, device=dev)
    sv.sv_fill_uniforms(SEED, 0, 0, B, K, out=u_static)
    ws = sv.Workspace(dev)
    out = new_out(B, K, dev)

    def call(o, inp, u, workspace):
        if entry == "spec_verify":
            sv.spec_verify(inp["target"], inp["draft"], inp["tokens"], u, inp["temperature"], out=o,
                           workspace=workspace)
        elif entry == "spec_verify_noalloc":
            sv.spec_verify_noalloc(inp["target"], inp["draft"], inp["tokens"], u, inp["temperature"],
                                   out=o)
        else:
            sv.spec_verify_philox(inp["target"], inp["draft"], inp["tokens"], inp["temperature"],
                                  SEED, 0, step_philox, out=o, workspace=workspace)

    # warm-up outside the capture (sizes the workspace, caches the library's per-device
    # lookups), on a side stream as torch's capture recipe asks
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, static, u_static, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, static, u_static, ws)
    torch.cuda.synchronize()

    ref_ws = sv.Workspace(dev)
    for step in range(1, 5):
        x = W.make_inputs(cfg, step=step, device=dev)
        for k in static:
            static[k].copy_(x[k])
        sv.sv_fill_uniforms(SEED, 0, step, B, K, out=u_static)
        junk = torch.randn((512, 512), device=dev) @ torch.randn((512, 512), device=dev)
        g.replay()
        torch.cuda.synchronize()
        got = to_host(out)
        ref = new_out(B, K, dev)
        if entry == "spec_verify_philox":
            sv.spec_verify_philox(x["target"], x["draft"], x["tokens"], x["temperature"], SEED, 0,
                                  step_philox, out=ref, workspace=ref_ws)
        else:
            u = torch.empty((B, K + 1), dtype=torch.float32, device=dev)
            sv.sv_fill_uniforms(SEED, 0, step, B, K, out=u)
            sv.spec_verify(x["target"], x["draft"], x["tokens"], u, x["temperature"], out=ref,
                           workspace=ref_ws)
        torch.cuda.synchronize()
        del junk
        assert_same(got, to_host(ref), f"{entry}, replay {step}")
        say(f"   replay {step}: {int((got['status'] != 0).sum())} flagged, mean accept "
            f"{float(got['accept_len'].mean()):.2f}")


@pytest.mark.parametrize("entry", ["spec_verify_greedy", "sv_sample"])
def test_graph_replays_equal_eager_greedy_and_sampler(dev, entry):
    cfg = 4
    x0 = W.make_inputs(cfg, step=0, device=dev, B=64)
    B, K = x0["B"], x0["K"]
    say(f"graph capture of {entry}: B={B} K={K} V={x0['V']}")
    if entry == "sv_sample":
        static = dict(rows=x0["draft"][:, 0].contiguous(), temperature=x0["temperature"].clone())
        u = torch.empty((B,), dtype=torch.float32, device=dev)
        out = dict(tokens=torch.empty((B,), dtype=torch.int32, device=dev),
                   status=torch.empty((B,), dtype=torch.int32, device=dev))
    else:
        static = dict(target=x0["target"].clone(), tokens=x0["tokens"].clone())
        out = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                   accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                   status=torch.empty((B,), dtype=torch.int32, device=dev))
    ws = sv.Workspace(dev)

    def call(o, inp):
        if entry == "sv_sample":
            sv.sv_sample(inp["rows"], u, inp["temperature"], out=o, workspace=ws)
        else:
            sv.spec_verify_greedy(inp["target"], inp["tokens"], out=o, workspace=ws)

    if entry == "sv_sample":
        sv.sv_fill_uniforms(SEED, 1, 0, B, 0, out=u.view(B, 1))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, static)
    torch.cuda.synchronize()
    for step in range(1, 4):
        x = W.make_inputs(cfg, step=step, device=dev, B=64)
        fresh = (dict(rows=x["draft"][:, 0].contiguous(), temperature=x["temperature"])
                 if entry == "sv_sample" else dict(target=x["target"], tokens=x["tokens"]))
        for k in static:
            static[k].copy_(fresh[k])
        if entry == "sv_sample":
            sv.sv_fill_uniforms(SEED, 1, step, B, 0, out=u.view(B, 1))
        junk = torch.randn((512, 512), device=dev) @ torch.randn((512, 512), device=dev)
        g.replay()
        torch.cuda.synchronize()
        got = to_host(out)
        if entry == "sv_sample":
            ref = to_host(sv.sv_sample(fresh["rows"], u, fresh["temperature"], workspace=sv.Workspace(dev)))
        else:
            ref = to_host(sv.spec_verify_greedy(fresh["target"], fresh["tokens"], workspace=sv.Workspace(dev)))
        torch.cuda.synchronize()
        del junk
        for k in got:
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{entry}, replay {step}: {k}")
