"""Python binding of libspecverify (the batched speculative-sampling verify step on MI355X).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI of
include/spec_verify.h.  PyTorch provides device memory and the stream; nothing here
computes.  The functions carry the C names.  If the library is not built, importing
works but every call raises ``LibraryMissing``: there is no fallback path.
"""
import ctypes
import os

__all__ = [
    "LibraryMissing", "SpecVerifyError", "lib", "lib_path",
    "sv_abi_version", "sv_status_string", "sv_workspace_bytes",
    "spec_verify", "spec_verify_greedy", "sv_fill_uniforms", "Workspace", "spec_verify_philox",
    "spec_verify_early_exit", "spec_verify_noalloc", "SV_NOALLOC_SCRATCH_BYTES",
    "spec_verify_ragged", "spec_verify_greedy_ragged", "sv_fill_uniforms_ragged", "sv_sample",
    "spec_verify_tree_greedy", "sv_tree_attention_mask", "SV_TREE_MAX_NODES",
    "sv_profile_begin", "sv_profile_end",
    "SV_OK", "SV_ERR_ARG", "SV_ERR_DTYPE", "SV_ERR_WORKSPACE", "SV_ERR_HIP", "SV_ERR_SCRATCH",
    "SV_DTYPE_F32", "SV_DTYPE_BF16",
    "SV_SEQ_ERR_TOKEN", "SV_SEQ_ERR_LOGIT", "SV_SEQ_ERR_TEMPERATURE", "SV_SEQ_ERR_UNIFORM",
    "SV_SEQ_NOTE_FALLBACK", "SV_SEQ_ERR_OFFSETS", "SV_SEQ_ERR_TREE",
]

SV_OK, SV_ERR_ARG, SV_ERR_DTYPE, SV_ERR_WORKSPACE, SV_ERR_HIP, SV_ERR_SCRATCH = 0, 1, 2, 3, 4, 5
SV_NOALLOC_SCRATCH_BYTES = 64 << 20
SV_DTYPE_F32, SV_DTYPE_BF16 = 0, 1
SV_SEQ_ERR_TOKEN, SV_SEQ_ERR_LOGIT, SV_SEQ_ERR_TEMPERATURE, SV_SEQ_ERR_UNIFORM = 1, 2, 4, 8
SV_SEQ_NOTE_FALLBACK = 16
SV_SEQ_ERR_OFFSETS = 32
SV_SEQ_ERR_TREE = 64
SV_TREE_MAX_NODES = 1024

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libspecverify.so")


class LibraryMissing(RuntimeError):
    pass


class SpecVerifyError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {sv_status_string(status)} (status {status})")


_lib = None


def lib():
    """The loaded ctypes library (loaded on first use)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise LibraryMissing(
            f"{lib_path} is not built; run `python -m speculative_decoding_verification_03_amd.build`")
    L = ctypes.CDLL(lib_path)
    vp, i32, u64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_size_t
    L.sv_abi_version.restype = i32
    L.sv_abi_version.argtypes = []
    L.sv_status_string.restype = ctypes.c_char_p
    L.sv_status_string.argtypes = [i32]
    L.sv_workspace_bytes.restype = i32
    L.sv_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
    L.spec_verify.restype = i32
    L.spec_verify.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32,
                              vp, vp, vp, vp, vp, vp, sz, vp]
    L.spec_verify_early_exit.restype = i32
    L.spec_verify_early_exit.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32,
                                         vp, vp, vp, vp, vp, vp, sz, vp]
    L.spec_verify_noalloc.restype = i32
    L.spec_verify_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32,
                                      vp, vp, vp, vp, vp, vp]
    L.spec_verify_philox.restype = i32
    L.spec_verify_philox.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, u64, u64, u64, vp,
                                     vp, vp, vp, vp, vp, vp, sz, vp]
    L.spec_verify_greedy.restype = i32
    L.spec_verify_greedy.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.sv_fill_uniforms.restype = i32
    L.sv_fill_uniforms.argtypes = [u64, u64, u64, i32, i32, vp, vp]
    L.spec_verify_ragged.restype = i32
    L.spec_verify_ragged.argtypes = [vp, vp, i32, vp, i32, i32, vp, vp, vp, i32, i32,
                                     vp, vp, vp, vp, vp, vp, sz, vp]
    L.spec_verify_greedy_ragged.restype = i32
    L.spec_verify_greedy_ragged.argtypes = [vp, i32, vp, i32, i32, vp, i32, i32,
                                            vp, vp, vp, vp, sz, vp]
    L.sv_sample.restype = i32
    L.sv_sample.argtypes = [vp, i32, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    L.spec_verify_tree_greedy.restype = i32
    L.spec_verify_tree_greedy.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.sv_tree_attention_mask.restype = i32
    L.sv_tree_attention_mask.argtypes = [vp, i32, i32, vp, vp, vp, vp]
    L.sv_fill_uniforms_ragged.restype = i32
    L.sv_fill_uniforms_ragged.argtypes = [u64, u64, u64, i32, vp, i32, i32, vp, vp]
    L.sv_profile_begin.restype = i32
    L.sv_profile_begin.argtypes = []
    L.sv_profile_end.restype = i32
    L.sv_profile_end.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double)]
    _lib = L
    return L


# --------------------------------------------------------------------------------------
# thin wrappers over the C names
# --------------------------------------------------------------------------------------

def sv_abi_version():
    return lib().sv_abi_version()


def sv_status_string(status):
    return lib().sv_status_string(int(status)).decode()


def sv_workspace_bytes(B, K, V):
    n = ctypes.c_size_t(0)
    st = lib().sv_workspace_bytes(int(B), int(K), int(V), ctypes.byref(n))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_workspace_bytes")
    return n.value


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _record(stream, *tensors):
    """Kernels on a stream other than the current one use these tensors (allocated on the
    current stream): tell the caching allocator, so that their memory is not handed to
    other work before that stream has finished with it."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, dtype=None, shape=None):
    torch = _torch()
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    del torch


class Workspace:
    """Device workspace for spec_verify / spec_verify_greedy, grown on demand.  Every call
    that uses it on a stream other than the current one records the buffer on that stream,
    so a buffer dropped when the workspace grows is not reused while work on that stream
    may still touch it."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, B, K, V):
        need = sv_workspace_bytes(B, K, V)
        if self.buf is None or self.buf.numel() < need:
            torch = _torch()
            self.buf = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def _workspace(ws, device, stream, B, K, V):
    """The caller's Workspace, else a default one per (device, stream): calls that share a
    workspace must not overlap, and calls on one stream never do."""
    if ws is None:
        key = (str(device), _stream(stream).value)
        ws = _default_ws.setdefault(key, Workspace(device))
    buf = ws.get(B, K, V)
    _record(stream, buf)
    return buf


def spec_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature,
                out=None, with_probs=True, workspace=None, stream=None, _entry="spec_verify"):
    """Sampled verify (greedy rule where temperature == 0).

    target_logits [B][K+1][V], draft_logits [B][K][V] (bf16 or fp32, same dtype),
    draft_tokens [B][K] int32, uniforms [B][K+1] fp32, temperature [B] fp32.
    Returns dict(tokens [B][K+1] int32, accept_len [B] int32, p, q [B][K] fp32 or None,
    status [B] int32).  Asynchronous on the stream; outputs stay on the device.
    """
    torch = _torch()
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits")
    _check(draft_logits, "draft_logits", target_logits.dtype, (B, K, V))
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    _check(uniforms, "uniforms", torch.float32, (B, K + 1))
    _check(temperature, "temperature", torch.float32, (B,))
    dev = target_logits.device
    if out is None:
        out = dict(
            tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
            accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
            p=torch.empty((B, K), dtype=torch.float32, device=dev) if with_probs else None,
            q=torch.empty((B, K), dtype=torch.float32, device=dev) if with_probs else None,
            status=torch.empty((B,), dtype=torch.int32, device=dev),
        )
    ws = _workspace(workspace, dev, stream, B, K, V)
    st = getattr(lib(), _entry)(
        _ptr(target_logits), _ptr(draft_logits), code, _ptr(draft_tokens), _ptr(uniforms),
        _ptr(temperature), B, K, V, _ptr(out["tokens"]), _ptr(out["accept_len"]),
        _ptr(out["p"]), _ptr(out["q"]), _ptr(out["status"]),
        _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, _entry)
    _record(stream, *out.values())
    return out


def spec_verify_early_exit(target_logits, draft_logits, draft_tokens, uniforms, temperature,
                           out=None, with_probs=True, workspace=None, stream=None):
    """spec_verify reading rows only up to each sequence's first rejection (see
    include/spec_verify.h): same tokens and accept lengths; p, q NaN where not read."""
    return spec_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, out=out,
                       with_probs=with_probs, workspace=workspace, stream=stream,
                       _entry="spec_verify_early_exit")


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, uniforms, temperature, out,
                        stream=None):
    """spec_verify with the library's static scratch array as its workspace (for callers
    that cannot allocate, e.g. under graph capture): `out` (tokens, accept_len, p, q,
    status; p and q may be None) must be given.  Same outputs as spec_verify."""
    torch = _torch()
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits")
    _check(draft_logits, "draft_logits", target_logits.dtype, (B, K, V))
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    _check(uniforms, "uniforms", torch.float32, (B, K + 1))
    _check(temperature, "temperature", torch.float32, (B,))
    st = lib().spec_verify_noalloc(
        _ptr(target_logits), _ptr(draft_logits), code, _ptr(draft_tokens), _ptr(uniforms),
        _ptr(temperature), B, K, V, _ptr(out["tokens"]), _ptr(out["accept_len"]),
        _ptr(out.get("p")), _ptr(out.get("q")), _ptr(out["status"]), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_noalloc")
    _record(stream, *[t for t in out.values() if t is not None])
    return out


def spec_verify_philox(target_logits, draft_logits, draft_tokens, temperature, seed, domain, step,
                       out=None, with_probs=True, workspace=None, stream=None):
    """spec_verify with uniforms from the counter generator (seed, domain, step), written to
    out["uniforms"] [B][K+1] by the call itself.  Same outputs as sv_fill_uniforms followed
    by spec_verify."""
    torch = _torch()
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits")
    _check(draft_logits, "draft_logits", target_logits.dtype, (B, K, V))
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    _check(temperature, "temperature", torch.float32, (B,))
    dev = target_logits.device
    if out is None:
        out = dict(
            tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
            accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
            p=torch.empty((B, K), dtype=torch.float32, device=dev) if with_probs else None,
            q=torch.empty((B, K), dtype=torch.float32, device=dev) if with_probs else None,
            status=torch.empty((B,), dtype=torch.int32, device=dev),
            uniforms=torch.empty((B, K + 1), dtype=torch.float32, device=dev),
        )
    _check(out["uniforms"], "uniforms", torch.float32, (B, K + 1))
    ws = _workspace(workspace, dev, stream, B, K, V)
    st = lib().spec_verify_philox(
        _ptr(target_logits), _ptr(draft_logits), code, _ptr(draft_tokens), _ptr(temperature),
        B, K, V, int(seed), int(domain), int(step), _ptr(out["uniforms"]), _ptr(out["tokens"]),
        _ptr(out["accept_len"]), _ptr(out["p"]), _ptr(out["q"]), _ptr(out["status"]),
        _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_philox")
    _record(stream, *out.values())
    return out


def spec_verify_greedy(target_logits, draft_tokens, out=None, workspace=None, stream=None):
    """Greedy verify: target_logits [B][K+1][V], draft_tokens [B][K] int32."""
    torch = _torch()
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits")
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    dev = target_logits.device
    if out is None:
        out = dict(
            tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
            accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
            status=torch.empty((B,), dtype=torch.int32, device=dev),
        )
    ws = _workspace(workspace, dev, stream, B, K, V)
    st = lib().spec_verify_greedy(
        _ptr(target_logits), code, _ptr(draft_tokens), B, K, V, _ptr(out["tokens"]),
        _ptr(out["accept_len"]), _ptr(out["status"]), _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_greedy")
    _record(stream, *out.values())
    return out


def spec_verify_ragged(target_logits, draft_logits, cu_drafts, draft_tokens, uniforms,
                       temperature, K_max, out=None, with_probs=True, workspace=None,
                       stream=None):
    """Ragged verify (packed layout, K_b = cu[b+1] - cu[b] drafts for sequence b).

    target_logits [total+B][V], draft_logits [total][V] (same dtype), cu_drafts [B+1] int32,
    draft_tokens [total] int32, uniforms [total+B] fp32, temperature [B] fp32, K_max a host
    bound on every K_b.  total = draft_tokens.shape[0].  Returns dict(tokens [total+B],
    accept_len [B], p, q [total] or None, status [B]).
    """
    torch = _torch()
    total = int(draft_tokens.shape[0])
    B = int(cu_drafts.shape[0]) - 1
    V = int(target_logits.shape[-1])
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits", None, (total + B, V))
    _check(draft_logits, "draft_logits", target_logits.dtype, (total, V))
    _check(cu_drafts, "cu_drafts", torch.int32, (B + 1,))
    _check(draft_tokens, "draft_tokens", torch.int32, (total,))
    _check(uniforms, "uniforms", torch.float32, (total + B,))
    _check(temperature, "temperature", torch.float32, (B,))
    dev = target_logits.device
    if out is None:
        out = dict(
            tokens=torch.empty((total + B,), dtype=torch.int32, device=dev),
            accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
            p=torch.empty((total,), dtype=torch.float32, device=dev) if with_probs else None,
            q=torch.empty((total,), dtype=torch.float32, device=dev) if with_probs else None,
            status=torch.empty((B,), dtype=torch.int32, device=dev),
        )
    ws = _workspace(workspace, dev, stream, B, K_max, V)
    st = lib().spec_verify_ragged(
        _ptr(target_logits), _ptr(draft_logits), code, _ptr(cu_drafts), total, int(K_max),
        _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature), B, V, _ptr(out["tokens"]),
        _ptr(out["accept_len"]), _ptr(out["p"]), _ptr(out["q"]), _ptr(out["status"]),
        _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_ragged")
    _record(stream, *out.values())
    return out


def spec_verify_greedy_ragged(target_logits, cu_drafts, draft_tokens, K_max, out=None,
                              workspace=None, stream=None):
    """Greedy verify in the packed layout of spec_verify_ragged."""
    torch = _torch()
    total = int(draft_tokens.shape[0])
    B = int(cu_drafts.shape[0]) - 1
    V = int(target_logits.shape[-1])
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits", None, (total + B, V))
    _check(cu_drafts, "cu_drafts", torch.int32, (B + 1,))
    _check(draft_tokens, "draft_tokens", torch.int32, (total,))
    dev = target_logits.device
    if out is None:
        out = dict(
            tokens=torch.empty((total + B,), dtype=torch.int32, device=dev),
            accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
            status=torch.empty((B,), dtype=torch.int32, device=dev),
        )
    ws = _workspace(workspace, dev, stream, B, K_max, V)
    st = lib().spec_verify_greedy_ragged(
        _ptr(target_logits), code, _ptr(cu_drafts), total, int(K_max), _ptr(draft_tokens), B, V,
        _ptr(out["tokens"]), _ptr(out["accept_len"]), _ptr(out["status"]), _ptr(ws),
        ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_greedy_ragged")
    _record(stream, *out.values())
    return out


def sv_sample(logits, uniforms, temperature, out=None, workspace=None, stream=None):
    """Draft-side sampler: logits [B][V], uniforms [B], temperature [B] -> dict(tokens, status)."""
    torch = _torch()
    B, V = logits.shape
    code = _dtype_code(logits)
    _check(logits, "logits")
    _check(uniforms, "uniforms", torch.float32, (B,))
    _check(temperature, "temperature", torch.float32, (B,))
    dev = logits.device
    if out is None:
        out = dict(tokens=torch.empty((B,), dtype=torch.int32, device=dev),
                   status=torch.empty((B,), dtype=torch.int32, device=dev))
    ws = _workspace(workspace, dev, stream, B, 0, V)
    st = lib().sv_sample(_ptr(logits), code, _ptr(uniforms), _ptr(temperature), B, V,
                         _ptr(out["tokens"]), _ptr(out["status"]), _ptr(ws), ws.numel(),
                         _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_sample")
    _record(stream, *out.values())
    return out


def spec_verify_tree_greedy(target_logits, parents, node_tokens, out=None, with_nodes=True,
                            workspace=None, stream=None):
    """Greedy verification of draft token trees: target_logits [B][N][V] (row j = logits
    after node j's path), parents [B][N] int32 (-1 for the root, else an earlier node),
    node_tokens [B][N] int32.  Returns dict(tokens [B][N], nodes [B][N] or None,
    accept_len [B], status [B])."""
    torch = _torch()
    B, N, V = target_logits.shape
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits")
    _check(parents, "parents", torch.int32, (B, N))
    _check(node_tokens, "node_tokens", torch.int32, (B, N))
    dev = target_logits.device
    if out is None:
        out = dict(tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
                   nodes=torch.empty((B, N), dtype=torch.int32, device=dev) if with_nodes else None,
                   accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                   status=torch.empty((B,), dtype=torch.int32, device=dev))
    ws = _workspace(workspace, dev, stream, B, max(N - 1, 0), V)
    st = lib().spec_verify_tree_greedy(
        _ptr(target_logits), code, _ptr(parents), _ptr(node_tokens), B, N, V, _ptr(out["tokens"]),
        _ptr(out["nodes"]), _ptr(out["accept_len"]), _ptr(out["status"]), _ptr(ws), ws.numel(),
        _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_tree_greedy")
    _record(stream, *out.values())
    return out


def sv_tree_attention_mask(parents, out=None, with_depth=True, stream=None):
    """Tree attention mask [B][N][N] uint8 (1: column node is the row node or an ancestor),
    depths [B][N] and status [B] of the trees given by parents [B][N] int32."""
    torch = _torch()
    B, N = parents.shape
    _check(parents, "parents", torch.int32, (B, N))
    dev = parents.device
    if out is None:
        out = dict(mask=torch.empty((B, N, N), dtype=torch.uint8, device=dev),
                   depth=torch.empty((B, N), dtype=torch.int32, device=dev) if with_depth else None,
                   status=torch.empty((B,), dtype=torch.int32, device=dev))
    st = lib().sv_tree_attention_mask(_ptr(parents), B, N, _ptr(out["mask"]), _ptr(out["depth"]),
                                      _ptr(out["status"]), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_tree_attention_mask")
    _record(stream, *out.values())
    return out


def sv_fill_uniforms_ragged(seed, domain, step, cu_drafts, total, K_max, out=None,
                            stream=None):
    """uniforms [total+B] fp32 in the packed layout (see include/spec_verify.h)."""
    torch = _torch()
    B = int(cu_drafts.shape[0]) - 1
    _check(cu_drafts, "cu_drafts", torch.int32, (B + 1,))
    if out is None:
        out = torch.empty((total + B,), dtype=torch.float32, device=cu_drafts.device)
    _check(out, "uniforms", torch.float32, (total + B,))
    st = lib().sv_fill_uniforms_ragged(int(seed), int(domain), int(step), B, _ptr(cu_drafts),
                                       int(total), int(K_max), _ptr(out), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_fill_uniforms_ragged")
    _record(stream, out)
    return out


def sv_fill_uniforms(seed, domain, step, B, K, out=None, device="cuda", stream=None):
    """uniforms [B][K+1] fp32 from the counter generator (see include/spec_verify.h)."""
    torch = _torch()
    if out is None:
        out = torch.empty((B, K + 1), dtype=torch.float32, device=device)
    _check(out, "uniforms", torch.float32, (B, K + 1))
    st = lib().sv_fill_uniforms(int(seed), int(domain), int(step), int(B), int(K),
                                _ptr(out), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_fill_uniforms")
    _record(stream, out)
    return out


def sv_profile_begin():
    """Start recording per-kernel HIP events in later calls (benchmark timing)."""
    st = lib().sv_profile_begin()
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_profile_begin")


def sv_profile_end():
    """Stop recording; returns (calls, ms of pass 1 summed, ms of pass 2 summed)."""
    calls = ctypes.c_int(0)
    t1 = ctypes.c_double(0.0)
    t2 = ctypes.c_double(0.0)
    st = lib().sv_profile_end(ctypes.byref(calls), ctypes.byref(t1), ctypes.byref(t2))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_profile_end")
    return calls.value, t1.value, t2.value
