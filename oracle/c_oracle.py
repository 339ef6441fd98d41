"""Python side of the plain-C fp64 oracle (verify_oracle.c).

TEST INFRASTRUCTURE ONLY, like the numpy oracle: only tests/, __graft_entry__.smoke()
and bench.py's cpu_baseline leg may use it.  It computes what
``spec_verify_oracle.verify`` computes (same arguments, same result dict), one C call
per sequence; the C call runs without Python's interpreter lock, so ``threads > 1``
spreads sequences over host cores with no copies.

``build()`` compiles verify_oracle.c with the host C compiler into
libverify_oracle.so next to it (plain -O2, no fast-math, no contraction).
"""
import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "verify_oracle.c")
LIB = os.path.join(HERE, "libverify_oracle.so")
DRAW_KINDS = ("test", "residual", "bonus")

_lib = None


def build():
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.oracle_verify_sequence.restype = i32
        L.oracle_verify_sequence.argtypes = [vp, vp, i32, i32, i32, vp, vp, f64, vp, vp, vp, vp,
                                             vp, vp, vp, vp]
        L.oracle_abi_version.restype = i32
        _lib = L
    return _lib


def _dtype_code(a):
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.float64:
        return 2
    raise TypeError(f"logit rows must be uint16 (bf16 bits), float32 or float64, got {a.dtype}")


def verify_sequence(zt, zd, x, u, T):
    """One sequence; arguments and result as spec_verify_oracle.verify_sequence."""
    zt = np.ascontiguousarray(zt)
    K = zt.shape[0] - 1
    V = zt.shape[1]
    code = _dtype_code(zt)
    T = float(T)
    if zd is not None:
        zd = np.ascontiguousarray(zd)
        if zd.dtype != zt.dtype and zd.size == 0:
            zd = zd.astype(zt.dtype)
        if zd.dtype != zt.dtype or zd.shape != (K, V):
            raise ValueError("draft rows must match the target rows' dtype and [K][V] shape")
    elif T != 0.0 and K > 0:
        raise ValueError("sampled sequences need draft rows")
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(K))
    ua = None if u is None else np.ascontiguousarray(np.asarray(u, dtype=np.float64).reshape(K + 1))
    if ua is None and T != 0.0:
        raise ValueError("sampled sequences need uniforms")
    tokens = np.empty(K + 1, dtype=np.int32)
    n = np.empty(1, dtype=np.int32)
    p = np.empty(max(K, 1), dtype=np.float64)
    q = np.empty(max(K, 1), dtype=np.float64)
    kind = np.empty(K + 1, dtype=np.int32)
    tpos = np.empty(K + 1, dtype=np.int32)
    margin = np.empty(K + 1, dtype=np.float64)
    nd = np.empty(1, dtype=np.int32)
    st = lib().oracle_verify_sequence(
        zt.ctypes.data, None if zd is None else zd.ctypes.data, code, K, V, xa.ctypes.data,
        None if ua is None else ua.ctypes.data, T, tokens.ctypes.data, n.ctypes.data,
        p.ctypes.data, q.ctypes.data, kind.ctypes.data, tpos.ctypes.data, margin.ctypes.data,
        nd.ctypes.data)
    if st < 0:
        raise MemoryError("oracle_verify_sequence: out of memory")
    draws = [(DRAW_KINDS[kind[i]], int(tpos[i]), float(margin[i])) for i in range(int(nd[0]))]
    return dict(tokens=[int(v) for v in tokens], n=int(n[0]), p=[float(v) for v in p[:K]],
                q=[float(v) for v in q[:K]], status=int(st), draws=draws)


def verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, seqs=None,
           threads=1):
    """Batched verify; arguments and result as spec_verify_oracle.verify.  threads > 1
    runs the sequences on a thread pool."""
    target_logits = np.asarray(target_logits)
    B, K1, V = target_logits.shape
    K = K1 - 1
    out_tokens = np.full((B, K + 1), -1, dtype=np.int32)
    out_n = np.full(B, -1, dtype=np.int32)
    out_p = np.full((B, K), np.nan, dtype=np.float32)
    out_q = np.full((B, K), np.nan, dtype=np.float32)
    out_status = np.full(B, -1, dtype=np.int32)
    draws = {}

    def one(b):
        T = float(np.float32(temperature[b]))
        zd = None if (draft_logits is None or T == 0.0) else draft_logits[b]
        return b, verify_sequence(target_logits[b], zd, draft_tokens[b],
                                  None if uniforms is None else uniforms[b], T)

    todo = list(range(B) if seqs is None else seqs)
    if threads > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            results = list(ex.map(one, todo))
    else:
        results = [one(b) for b in todo]
    for b, r in results:
        out_tokens[b] = r["tokens"]
        out_n[b] = r["n"]
        if K:
            out_p[b] = np.asarray(r["p"], dtype=np.float64).astype(np.float32)
            out_q[b] = np.asarray(r["q"], dtype=np.float64).astype(np.float32)
        out_status[b] = r["status"]
        draws[b] = r["draws"]
    return dict(tokens=out_tokens, accept_len=out_n, p=out_p, q=out_q, status=out_status,
                draws=draws)


def verify_greedy(target_logits, draft_tokens, seqs=None, threads=1):
    target_logits = np.asarray(target_logits)
    B = target_logits.shape[0]
    r = verify(target_logits, None, draft_tokens, None, np.zeros(B, dtype=np.float32), seqs,
               threads)
    return dict(tokens=r["tokens"], accept_len=r["accept_len"], status=r["status"])

