"""spec_verify_noalloc (the entry point whose workspace is the library's static scratch
array) through the C ABI, against spec_verify with a workspace of its own: the same
outputs bit for bit, on two calls in a row, the second with a smaller batch (the array
keeps the first call's contents)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import speculative_decoding_verification_03_amd as sv
from speculative_decoding_verification_03_amd import workloads as W
from parity_util import host_uniforms, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(sv.lib_path), "libspecverify.so is not built"
    return torch.device("cuda:0")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _outputs(B, K, dev):
    return dict(tokens=torch.full((B, K + 1), -7, dtype=torch.int32, device=dev),
                accept_len=torch.full((B,), -7, dtype=torch.int32, device=dev),
                p=torch.full((B, K), 7.0, dtype=torch.float32, device=dev),
                q=torch.full((B, K), 7.0, dtype=torch.float32, device=dev),
                status=torch.full((B,), -7, dtype=torch.int32, device=dev))


def test_noalloc_equals_spec_verify(dev):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for cfg, B, step in ((4, None, 31), (3, 24, 32)):
        inp = W.make_inputs(cfg, step=step, device=dev, B=B)
        Bn, K, V = inp["B"], inp["K"], inp["V"]
        print(f"noalloc: workload {cfg} B={Bn} K={K} V={V}", flush=True)
        assert sv.sv_workspace_bytes(Bn, K, V) <= sv.SV_NOALLOC_SCRATCH_BYTES
        u = torch.from_numpy(host_uniforms(1000 + cfg, 0, step, Bn, K)).to(dev)
        out = _outputs(Bn, K, dev)
        code = sv.SV_DTYPE_BF16 if inp["target"].dtype == torch.bfloat16 else sv.SV_DTYPE_F32
        st = sv.lib().spec_verify_noalloc(
            _ptr(inp["target"]), _ptr(inp["draft"]), code, _ptr(inp["tokens"]), _ptr(u),
            _ptr(inp["temperature"]), Bn, K, V, _ptr(out["tokens"]), _ptr(out["accept_len"]),
            _ptr(out["p"]), _ptr(out["q"]), _ptr(out["status"]), stream)
        assert st == sv.SV_OK
        ref = sv.spec_verify(inp["target"], inp["draft"], inp["tokens"], u, inp["temperature"],
                             workspace=sv.Workspace(dev))
        torch.cuda.synchronize()
        got, ref = to_host(out), to_host(ref)
        for k in ("tokens", "accept_len", "status"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        for k in ("p", "q"):
            np.testing.assert_array_equal(got[k].view(np.uint32), ref[k].view(np.uint32), err_msg=k)
        assert (got["status"] & ~16 == 0).all()
