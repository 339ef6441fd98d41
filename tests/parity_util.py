"""Helpers of the GPU parity tests: the near-tie comparison (oracle/parity.py), the
uniforms of the oracle's side, host copies of device results.

Uniforms: both sides take the array that the counter generator names for (seed, domain,
step).  The oracle's side always computes it with oracle/philox.py (``host_uniforms``);
the HIP side either gets that array copied in, or generates it with its own generator,
whose output tests compare with the host array bit for bit.
"""
import numpy as np

from oracle import philox
from oracle.parity import (NEAR_TIE, NEAR_TIE_BUDGET, PROB_ATOL_TINY, PROB_RTOL,  # noqa: F401
                           PROB_TINY, Tally, compare)

# (name, tally) pairs that the session prints at its end (tests/conftest.py)
REPORT = []


def host_uniforms(seed, domain, step, B, K):
    """u[B][K+1] fp32 named by (seed, domain, step), from the oracle's generator."""
    return philox.uniforms_array(seed, domain, step, B, K)


def host_uniforms_packed(seed, domain, step, cu, total):
    """The packed layout (ragged batches), from the oracle's generator."""
    return philox.uniforms_packed(seed, domain, step, cu, total)


def early_exit_expected(orc, gpu, temperature, K):
    """The oracle's results as spec_verify_early_exit reports them: p and q only up to and
    including the first rejection n, NaN after it (every position when all K drafts are
    accepted).  n is the HIP side's own: a near-tie may move it, and compare() then
    excuses the draw."""
    exp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in orc.items()}
    for b in range(len(gpu["accept_len"])):
        T = float(temperature[b])
        n = int(gpu["accept_len"][b])
        if T != 0.0 and 0 <= n < K:
            exp["p"][b, n + 1:] = np.nan
            exp["q"][b, n + 1:] = np.nan
    return exp


def to_host(out):
    return {k: (None if v is None else v.detach().cpu().numpy()) for k, v in out.items()}


def logits_to_host(x):
    """Device logits -> host array the oracle decodes (uint16 bit patterns for bf16)."""
    import torch
    x = x.detach().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()
