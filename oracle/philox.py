"""Counter-based uniform generator of the oracle (test infrastructure only).

This module is part of the CPU oracle.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does.  It shares no code with the HIP library, which implements the same published
generator on its own.

Why a generator at all: the exact rule ("Quy tắc chính xác" on the lesson page
"Việc giải mã giả định và Eagle"; "A Regra de Exatidão" on "Decodificação
Especulativa e EAGLE") draws one r ~ Uniform(0, 1) per drafted token, and the
build-it pseudocode on both pages draws a fresh one for the final categorical
sample.  The verify step takes those draws as an input array ``u[B][K+1]``; this
module defines which array a (seed, domain, step) triple names, so that a GPU run
and the oracle can agree on it bit for bit.

Generator: Philox4x64-10, as published by Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11).  State: a 4x64-bit
counter and a 2x64-bit key.  Each of the 10 rounds multiplies counter words 0 and
2 by two fixed 64-bit constants, keeps the 128-bit products as (hi, lo) pairs and
permutes: (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key
is bumped by two Weyl constants between rounds.

Uniform contract (ours):
    key     = (seed, domain)
    counter = (t, b, step, 0)
    u       = (word0 >> 40) * 2**-24            (a value in {0, 2^-24, ..., 1 - 2^-24})
so every u is exactly representable in fp32 and fp64, and 0 <= u < 1.
"""

MASK64 = (1 << 64) - 1

# Round multipliers and Weyl key increments of Philox4x64 (SC'11, Table 2 and
# the key schedule of the Philox family).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15  # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B  # sqrt(3) - 1
PHILOX_ROUNDS = 10


def philox4x64(counter, key, rounds=PHILOX_ROUNDS):
    """Philox4x64-R block function on Python integers (exact 128-bit products).

    counter: 4 unsigned 64-bit ints; key: 2 unsigned 64-bit ints.
    Returns the 4 output words.
    """
    c0, c1, c2, c3 = (int(v) & MASK64 for v in counter)
    k0, k1 = (int(v) & MASK64 for v in key)
    for r in range(rounds):
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        if r + 1 < rounds:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
    return c0, c1, c2, c3


def uniform(seed, domain, step, b, t):
    """One draw of the contract above, as a Python float."""
    w0 = philox4x64((t, b, step, 0), (seed, domain))[0]
    return (w0 >> 40) * 2.0 ** -24


def uniforms(seed, domain, step, B, K):
    """The array u[B][K+1] named by (seed, domain, step), as nested lists of floats.

    Slot t < K drives the ratio test of drafted token t; slot K drives the final
    categorical sample (replacement or bonus).
    """
    return [[uniform(seed, domain, step, b, t) for t in range(K + 1)] for b in range(B)]


def uniforms_array(seed, domain, step, B, K):
    """uniforms() as a float32 numpy array [B][K+1] (every value is exact in fp32)."""
    import numpy as np
    return np.array(uniforms(seed, domain, step, B, K), dtype=np.float32).reshape(B, K + 1)


def uniforms_packed(seed, domain, step, cu, total):
    """The packed layout of a ragged batch, float32 [total + B]: sequence b's K_b + 1
    uniforms (the dense array's first K_b + 1 of row b) at cu[b] + b; the slots of a
    sequence with invalid offsets stay 0."""
    import numpy as np
    cu = [int(v) for v in cu]
    B = len(cu) - 1
    out = np.zeros(total + B, dtype=np.float32)
    for b in range(B):
        k = cu[b + 1] - cu[b]
        if cu[b] < 0 or k < 0 or cu[b + 1] > total:
            continue
        out[cu[b] + b:cu[b] + b + k + 1] = [uniform(seed, domain, step, b, t) for t in range(k + 1)]
    return out
