"""Speculative-decoding verify step on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libspecverify.so`` (C ABI declared in
``include/specverify.h``).  The functions here only marshal arguments:
torch tensors provide device pointers and the current HIP stream, every step
of the verify path runs in the library's HIP kernels.  There is no fallback:
if the library is missing, :func:`load` raises.

    verify_attn(q, k_cache, v_cache, block_table, kv_len, ...)
        window-causal GQA of the K+1 verify positions over a paged KV cache
    reject_sample(target, draft, draft_tokens, uniforms, temperature, kv_len, ...)
        lossless verifier over the full vocabulary + KV-length commit
    verify_attn_tree(..., anc) / reject_sample_tree(..., parent, ...)
        the same two steps over a flattened draft tree
    verify_attn_window(q, k_new, v_new, k_cache, v_cache, ..., mode)
        attention with the window's K/V from the projection output, stored
        into the cache in the same kernel (append) or not (scratch)
    kv_commit(...), PagePool
        the accepted rows into their committed positions; host page list
"""

import ctypes
import os

__all__ = ["load", "lib_path", "exported_symbols", "verify_attn", "verify_attn_tree",
           "verify_attn_window", "kv_commit", "PagePool", "DraftLengthBandit", "accept_stats", "read_probe", "SV_WINDOW_READ", "SV_WINDOW_APPEND",
           "reject_sample", "reject_sample_noalloc", "reject_sample_tree",
           "verify_attn_workspace_bytes", "NOALLOC_SCRATCH_BYTES",
           "reject_sample_workspace_bytes", "reject_sample_tree_workspace_bytes",
           "reject_sample_filtered_workspace_bytes", "reject_sample_tree_filtered_workspace_bytes",
           "SpecVerifyError", "SV_F32", "SV_BF16", "STATUS", "EXPORTS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

SV_F32, SV_BF16 = 0, 1
SV_WINDOW_READ, SV_WINDOW_APPEND = 0, 1
NOALLOC_SCRATCH_BYTES = 16 << 20     # SV_NOALLOC_SCRATCH_BYTES
STATUS = {0: "SV_OK", -1: "SV_ERR_INVALID_ARG", -2: "SV_ERR_UNSUPPORTED",
          -3: "SV_ERR_WORKSPACE", -4: "SV_ERR_HIP", -5: "SV_ERR_NO_PAGES",
          -6: "SV_ERR_BAD_INPUT"}
EXPORTS = ("spec_verify_attn", "spec_verify_attn_workspace_bytes", "spec_verify_attn_tree",
           "spec_verify_attn_window", "spec_kv_commit",
           "spec_reject_sample", "spec_reject_sample_workspace_bytes", "spec_reject_sample_noalloc",
           "spec_reject_sample_filtered", "spec_reject_sample_filtered_workspace_bytes",
           "spec_reject_sample_tree", "spec_reject_sample_tree_workspace_bytes",
           "spec_reject_sample_tree_filtered_workspace_bytes",
           "spec_reject_sample_tree_filtered", "spec_reject_sample_trees",
           "spec_pages_create", "spec_pages_destroy", "spec_pages_reserve", "spec_pages_commit",
           "spec_pages_release", "spec_pages_free_count", "spec_pages_seq_blocks",
           "spec_pages_block_table", "spec_pages_check",
           "spec_bandit_create", "spec_bandit_destroy", "spec_bandit_select",
           "spec_bandit_update", "spec_bandit_stats", "spec_accept_stats",
           "spec_read_probe", "spec_status_string", "spec_version")


class SpecVerifyError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s returned %d (%s)" % (fn, status, STATUS.get(status, "?")))


def lib_path():
    return os.path.join(_HERE, "libspecverify.so")


def load():
    """Load the in-tree HIP library (raises OSError when it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise OSError("libspecverify.so not built at %s: run "
                      "python -m speculative_decoding_verification_verify_amd.build" % path)
    lib = ctypes.CDLL(path)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.spec_verify_attn.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     i32, i32, f32, i32, vp, sz, vp]
    lib.spec_verify_attn.restype = i32
    lib.spec_verify_attn_tree.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          i32, i32, i32, f32, i32, vp, sz, vp]
    lib.spec_verify_attn_tree.restype = i32
    lib.spec_verify_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.spec_verify_attn_workspace_bytes.restype = sz
    lib.spec_reject_sample.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                       vp, sz, vp]
    lib.spec_reject_sample.restype = i32
    lib.spec_reject_sample_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                               i32, vp]
    lib.spec_reject_sample_noalloc.restype = i32
    lib.spec_reject_sample_filtered.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                i32, i32, vp, sz, vp]
    lib.spec_reject_sample_filtered.restype = i32
    lib.spec_reject_sample_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_reject_sample_workspace_bytes.restype = sz
    lib.spec_reject_sample_tree.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                            i32, i32, vp, sz, vp]
    lib.spec_reject_sample_tree.restype = i32
    lib.spec_reject_sample_tree_filtered.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                     vp, i32, i32, i32, i32, vp, sz, vp]
    lib.spec_reject_sample_tree_filtered.restype = i32
    lib.spec_reject_sample_trees.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             i32, i32, i32, i32, vp, sz, vp]
    lib.spec_reject_sample_trees.restype = i32
    lib.spec_reject_sample_tree_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_reject_sample_tree_workspace_bytes.restype = sz
    for fn in ("spec_reject_sample_filtered_workspace_bytes",
               "spec_reject_sample_tree_filtered_workspace_bytes"):
        getattr(lib, fn).argtypes = [i32, i32, i32]
        getattr(lib, fn).restype = sz
    lib.spec_verify_attn_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                            i32, i32, i32, i32, i32, f32, i32, i32, vp, sz, vp]
    lib.spec_verify_attn_window.restype = i32
    lib.spec_kv_commit.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                   i32, i32, vp]
    lib.spec_kv_commit.restype = i32
    lib.spec_pages_create.argtypes = [i32, i32, i32]
    lib.spec_pages_create.restype = vp
    lib.spec_pages_destroy.argtypes = [vp]
    lib.spec_pages_destroy.restype = None
    for fn in ("spec_pages_reserve", "spec_pages_commit"):
        getattr(lib, fn).argtypes = [vp, i32, i32]
        getattr(lib, fn).restype = i32
    lib.spec_pages_release.argtypes = [vp, i32]
    lib.spec_pages_release.restype = i32
    lib.spec_pages_free_count.argtypes = [vp]
    lib.spec_pages_free_count.restype = i32
    lib.spec_pages_seq_blocks.argtypes = [vp, i32]
    lib.spec_pages_seq_blocks.restype = i32
    lib.spec_pages_block_table.argtypes = [vp]
    lib.spec_pages_block_table.restype = ctypes.POINTER(ctypes.c_int32)
    lib.spec_pages_check.argtypes = [vp]
    lib.spec_pages_check.restype = i32
    f64, i64p = ctypes.c_double, ctypes.POINTER(ctypes.c_longlong)
    lib.spec_bandit_create.argtypes = [i32, i32]
    lib.spec_bandit_create.restype = vp
    lib.spec_bandit_destroy.argtypes = [vp]
    lib.spec_bandit_destroy.restype = None
    lib.spec_bandit_select.argtypes = [vp, f64, f64]
    lib.spec_bandit_select.restype = i32
    lib.spec_bandit_update.argtypes = [vp, i32, f64]
    lib.spec_bandit_update.restype = i32
    lib.spec_bandit_stats.argtypes = [vp, vp, vp, vp]
    lib.spec_bandit_stats.restype = i32
    lib.spec_accept_stats.argtypes = [vp, i32, i32, vp, vp]
    lib.spec_accept_stats.restype = i32
    lib.spec_read_probe.argtypes = [vp, sz, vp, i32, vp]
    lib.spec_read_probe.restype = i32
    lib.spec_status_string.argtypes = [i32]
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_version.argtypes = []
    lib.spec_version.restype = i32
    _LIB = lib
    return lib


def exported_symbols():
    lib = load()
    return {name: hasattr(lib, name) for name in EXPORTS}


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise SpecVerifyError(fn, status)


def _need(t, name, dtype=None, shape=None):
    """Type, dtype, shape and layout of one tensor argument (no device check:
    _on_gpu does that after every argument's shape is known to be right)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None:
        _shape(t, name, shape)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _dims(t, name, nd):
    if t.dim() != nd:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, nd, tuple(t.shape)))


def _on_gpu(**tensors):
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s must be on the GPU" % name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other arguments on %s" % (name, t.device, dev))


def _kv_caches(k_cache, v_cache, dtype):
    """(NB, Hkv, D) of a paged K cache [NB, Hkv, D/X, 16, X] (X = 16 bytes /
    element) and V cache [NB, Hkv, D, 16], after checking both."""
    _need(k_cache, "k_cache", dtype)
    _need(v_cache, "v_cache", dtype)
    _dims(k_cache, "k_cache", 5)
    _dims(v_cache, "v_cache", 4)
    x = 16 // k_cache.element_size()
    NB, Hkv, DX, BS, X = k_cache.shape
    if X != x or BS != 16:
        raise ValueError("k_cache must be [NB, Hkv, D/%d, 16, %d], got %s" % (x, x, tuple(k_cache.shape)))
    D = DX * X
    _shape(v_cache, "v_cache", (NB, Hkv, D, 16))
    return NB, Hkv, D


def verify_attn_workspace_bytes(B, K, Hq, Hkv, D, max_kv_len):
    return int(load().spec_verify_attn_workspace_bytes(B, K, Hq, Hkv, D, max_kv_len))


def reject_sample_workspace_bytes(B, K, V):
    return int(load().spec_reject_sample_workspace_bytes(B, K, V))


def reject_sample_tree_workspace_bytes(B, N, V):
    return int(load().spec_reject_sample_tree_workspace_bytes(B, N, V))


def reject_sample_filtered_workspace_bytes(B, K, V):
    """Workspace of the filtered chain call with room for the sweep's window."""
    return int(load().spec_reject_sample_filtered_workspace_bytes(B, K, V))


def reject_sample_tree_filtered_workspace_bytes(B, N, V):
    """Workspace of the filtered tree calls with room for the sweep's window."""
    return int(load().spec_reject_sample_tree_filtered_workspace_bytes(B, N, V))


def _workspace(workspace, ws_bytes, device):
    import torch
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    if workspace is not None:
        _need(workspace, "workspace")
        _on_gpu(workspace=workspace)
    return workspace, (0 if workspace is None else workspace.numel() * workspace.element_size())


def verify_attn(q, k_cache, v_cache, block_table, kv_len, out=None, max_kv_len=None,
                scale=0.0, workspace=None, stream=None):
    """Window-causal GQA of the K+1 verify positions (see ``spec_verify_attn``).

    q [B, K+1, Hq, D]; k_cache [NB, Hkv, D/X, 16, X]; v_cache [NB, Hkv, D, 16]
    (bf16 or fp32, X = 8 or 4); block_table [B, max_blocks] int32; kv_len [B]
    int32 (committed lengths, read only).  ``max_kv_len`` bounds kv_len; it
    defaults to the block table's capacity.  Returns ``out``.
    """
    return _verify_attn(q, k_cache, v_cache, block_table, kv_len, None, out, max_kv_len, scale,
                        workspace, stream)


def verify_attn_tree(q, k_cache, v_cache, block_table, kv_len, anc, out=None, max_kv_len=None,
                     scale=0.0, workspace=None, stream=None):
    """Attention over a flattened draft tree (see ``spec_verify_attn_tree``).

    As ``verify_attn`` with N = q.shape[1] tree nodes, plus anc [B, N] int32
    (the uint32 ancestor-or-self bit set of each node, bit j = node j).
    """
    import torch
    _need(anc, "anc", torch.int32)
    _dims(q, "q", 4)
    _shape(anc, "anc", (q.shape[0], q.shape[1]))
    return _verify_attn(q, k_cache, v_cache, block_table, kv_len, anc, out, max_kv_len, scale,
                        workspace, stream)


def _attn_common(q, k_cache, v_cache, block_table, kv_len, out):
    """Checks shared by the attention calls; returns (B, N, Hq, D, NB, Hkv, dtype code)."""
    import torch
    _need(q, "q")
    dt = _dtype_code(q)
    _dims(q, "q", 4)
    B, N, Hq, D = q.shape
    NB, Hkv, Dk = _kv_caches(k_cache, v_cache, q.dtype)
    if Dk != D:
        raise ValueError("q has head dim %d, the caches %d" % (D, Dk))
    _need(block_table, "block_table", torch.int32)
    _dims(block_table, "block_table", 2)
    if block_table.shape[0] != B:
        raise ValueError("block_table must have B = %d rows, got %d" % (B, block_table.shape[0]))
    _need(kv_len, "kv_len", torch.int32, (B,))
    if out is not None:
        _need(out, "out", q.dtype, tuple(q.shape))
    return B, N, Hq, D, NB, Hkv, dt


def _verify_attn(q, k_cache, v_cache, block_table, kv_len, anc, out, max_kv_len, scale,
                 workspace, stream):
    import torch
    lib = load()
    B, K1, Hq, D, NB, Hkv, dt = _attn_common(q, k_cache, v_cache, block_table, kv_len, out)
    _on_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, kv_len=kv_len,
            anc=anc, out=out)
    mbps = block_table.shape[1]
    if max_kv_len is None:
        max_kv_len = max(0, mbps * 16 - K1)
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = verify_attn_workspace_bytes(B, K1 - 1, Hq, Hkv, D, max_kv_len)
    workspace, ws_have = _workspace(workspace, ws_bytes, q.device)
    if anc is None:
        st = lib.spec_verify_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                  _ptr(kv_len), _ptr(out), B, K1 - 1, Hq, Hkv, D, 16, NB,
                                  mbps, int(max_kv_len), float(scale), dt, _ptr(workspace),
                                  ws_have, _stream(stream))
        _check("spec_verify_attn", st)
    else:
        st = lib.spec_verify_attn_tree(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                       _ptr(kv_len), _ptr(anc), _ptr(out), B, K1, Hq, Hkv, D,
                                       16, NB, mbps, int(max_kv_len), float(scale), dt,
                                       _ptr(workspace), ws_have, _stream(stream))
        _check("spec_verify_attn_tree", st)
    return out


def _reject_outputs(B, N, device, out_tokens, num_accepted, counters, out_nodes=False):
    import torch
    if out_tokens is None:
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=device)
    else:
        _need(out_tokens, "out_tokens", torch.int32, (B, N))
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=device)
    else:
        _need(num_accepted, "num_accepted", torch.int32, (B,))
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    return out_tokens, num_accepted


def reject_sample(target, draft, draft_tokens, uniforms, temperature, kv_len,
                  out_tokens=None, num_accepted=None, counters=None, workspace=None,
                  stream=None, top_k=None, top_p=None):
    """Lossless verifier + KV commit (see ``spec_reject_sample``); with
    top_k [B] int32 and / or top_p [B] float32, on the filtered laws (see
    ``spec_reject_sample_filtered``).

    target [B, K+1, V], draft [B, K, V] or None (greedy for every sequence);
    draft_tokens [B, K] int32; uniforms [B, K+1] float32; temperature [B]
    float32; kv_len [B] int32, updated in place to kv_len + n + 1.
    Returns (out_tokens [B, K+1] int32, num_accepted [B] int32).
    """
    import torch
    lib = load()
    _need(target, "target")
    dt = _dtype_code(target)
    _dims(target, "target", 3)
    B, K1, V = target.shape
    K = K1 - 1
    if draft is not None:
        _need(draft, "draft", target.dtype, (B, K, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, K))
    _need(uniforms, "uniforms", torch.float32, (B, K1))
    _need(temperature, "temperature", torch.float32, (B,))
    _need(kv_len, "kv_len", torch.int32, (B,))
    if top_k is not None:
        _need(top_k, "top_k", torch.int32, (B,))
    if top_p is not None:
        _need(top_p, "top_p", torch.float32, (B,))
    if out_tokens is not None:
        _need(out_tokens, "out_tokens", torch.int32, (B, K1))
    if num_accepted is not None:
        _need(num_accepted, "num_accepted", torch.int32, (B,))
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    _on_gpu(target=target, draft=draft, draft_tokens=draft_tokens, uniforms=uniforms,
            temperature=temperature, kv_len=kv_len, top_k=top_k, top_p=top_p,
            out_tokens=out_tokens, num_accepted=num_accepted, counters=counters)
    out_tokens, num_accepted = _reject_outputs(B, K1, target.device, out_tokens, num_accepted,
                                               counters)
    filtered = top_k is not None or top_p is not None
    ws_bytes = (reject_sample_filtered_workspace_bytes(B, K, V) if filtered else
                reject_sample_workspace_bytes(B, K, V))
    workspace, ws_have = _workspace(workspace, ws_bytes, target.device)
    if filtered:
        st = lib.spec_reject_sample_filtered(_ptr(target), _ptr(draft), _ptr(draft_tokens),
                                             _ptr(uniforms), _ptr(temperature), _ptr(top_k),
                                             _ptr(top_p), _ptr(out_tokens), _ptr(num_accepted),
                                             _ptr(kv_len), _ptr(counters), B, K, V, dt,
                                             _ptr(workspace), ws_have, _stream(stream))
        _check("spec_reject_sample_filtered", st)
        return out_tokens, num_accepted
    st = lib.spec_reject_sample(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                                _ptr(temperature), _ptr(out_tokens), _ptr(num_accepted),
                                _ptr(kv_len), _ptr(counters), B, K, V, dt, _ptr(workspace),
                                ws_have, _stream(stream))
    _check("spec_reject_sample", st)
    return out_tokens, num_accepted


def reject_sample_noalloc(target, draft, draft_tokens, uniforms, temperature, kv_len,
                          out_tokens, num_accepted, counters=None, stream=None):
    """``spec_reject_sample_noalloc``: the verifier with the library's own
    per-device scratch array as its workspace.  Every output is the
    caller's (nothing is allocated here either); the shapes and results are
    those of :func:`reject_sample`.  Returns (out_tokens, num_accepted)."""
    import torch
    lib = load()
    _need(target, "target")
    dt = _dtype_code(target)
    _dims(target, "target", 3)
    B, K1, V = target.shape
    K = K1 - 1
    if draft is not None:
        _need(draft, "draft", target.dtype, (B, K, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, K))
    _need(uniforms, "uniforms", torch.float32, (B, K1))
    _need(temperature, "temperature", torch.float32, (B,))
    _need(kv_len, "kv_len", torch.int32, (B,))
    _need(out_tokens, "out_tokens", torch.int32, (B, K1))
    _need(num_accepted, "num_accepted", torch.int32, (B,))
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    _on_gpu(target=target, draft=draft, draft_tokens=draft_tokens, uniforms=uniforms,
            temperature=temperature, kv_len=kv_len, out_tokens=out_tokens,
            num_accepted=num_accepted, counters=counters)
    st = lib.spec_reject_sample_noalloc(_ptr(target), _ptr(draft), _ptr(draft_tokens),
                                        _ptr(uniforms), _ptr(temperature), _ptr(out_tokens),
                                        _ptr(num_accepted), _ptr(kv_len), _ptr(counters), B, K, V,
                                        dt, _stream(stream))
    _check("spec_reject_sample_noalloc", st)
    return out_tokens, num_accepted


def _tree_inputs(target, draft, tokens, uniforms, temperature, kv_len, out_tokens, out_nodes,
                 num_accepted, counters, top_k, top_p, parents=None):
    """Shape and dtype checks shared by the tree calls; (B, N, V, dtype code)."""
    import torch
    _need(target, "target")
    dt = _dtype_code(target)
    _dims(target, "target", 3)
    B, N, V = target.shape
    if draft is not None:
        _need(draft, "draft", target.dtype, (B, N, V))
    _need(tokens, "tokens", torch.int32, (B, N))
    _need(uniforms, "uniforms", torch.float32, (B, N))
    _need(temperature, "temperature", torch.float32, (B,))
    _need(kv_len, "kv_len", torch.int32, (B,))
    if parents is not None:
        _need(parents, "parents", torch.int32, (B, N))
    if out_nodes is not None:
        _need(out_nodes, "out_nodes", torch.int32, (B, N))
    if out_tokens is not None:
        _need(out_tokens, "out_tokens", torch.int32, (B, N))
    if num_accepted is not None:
        _need(num_accepted, "num_accepted", torch.int32, (B,))
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    if top_k is not None:
        _need(top_k, "top_k", torch.int32, (B,))
    if top_p is not None:
        _need(top_p, "top_p", torch.float32, (B,))
    return B, N, V, dt


def _tree_outputs(B, N, device, out_tokens, out_nodes, num_accepted, counters):
    import torch
    out_tokens, num_accepted = _reject_outputs(B, N, device, out_tokens, num_accepted, counters)
    if out_nodes is None:
        out_nodes = torch.empty((B, N), dtype=torch.int32, device=device)
    return out_tokens, out_nodes, num_accepted


def reject_sample_tree(target, draft, parent, tokens, uniforms, temperature, kv_len,
                       out_tokens=None, out_nodes=None, num_accepted=None, counters=None,
                       workspace=None, stream=None, top_k=None, top_p=None):
    """Lossless verifier over a draft tree + KV commit (see ``spec_reject_sample_tree``);
    with top_k [B] int32 and / or top_p [B] float32, on the filtered laws
    (see ``spec_reject_sample_tree_filtered``).

    target [B, N, V], draft [B, N, V] or None (greedy for every sequence);
    parent: N host integers (parent[0] = -1, parent[i] < i), shared by the
    batch; tokens [B, N] int32; uniforms [B, N] float32 (u[i] tests node i,
    u[0] the final draw); temperature [B] float32; kv_len [B] int32, updated
    in place to kv_len + n + 1.
    Returns (out_tokens [B, N], out_nodes [B, N], num_accepted [B]), int32.
    """
    lib = load()
    B, N, V, dt = _tree_inputs(target, draft, tokens, uniforms, temperature, kv_len, out_tokens,
                               out_nodes, num_accepted, counters, top_k, top_p)
    par = [int(x) for x in parent]
    if len(par) != N:
        raise ValueError("parent must have N = %d entries" % N)
    _on_gpu(target=target, draft=draft, tokens=tokens, uniforms=uniforms,
            temperature=temperature, kv_len=kv_len, out_tokens=out_tokens, out_nodes=out_nodes,
            num_accepted=num_accepted, counters=counters, top_k=top_k, top_p=top_p)
    c_par = (ctypes.c_int32 * N)(*par)
    out_tokens, out_nodes, num_accepted = _tree_outputs(B, N, target.device, out_tokens, out_nodes,
                                                        num_accepted, counters)
    filtered = top_k is not None or top_p is not None
    ws_bytes = (reject_sample_tree_filtered_workspace_bytes(B, N, V) if filtered else
                reject_sample_tree_workspace_bytes(B, N, V))
    workspace, ws_have = _workspace(workspace, ws_bytes, target.device)
    if filtered:
        st = lib.spec_reject_sample_tree_filtered(
            _ptr(target), _ptr(draft), ctypes.cast(c_par, ctypes.c_void_p), _ptr(tokens),
            _ptr(uniforms), _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(out_tokens),
            _ptr(out_nodes), _ptr(num_accepted), _ptr(kv_len), _ptr(counters), B, N, V, dt,
            _ptr(workspace), ws_have, _stream(stream))
        _check("spec_reject_sample_tree_filtered", st)
        return out_tokens, out_nodes, num_accepted
    st = lib.spec_reject_sample_tree(_ptr(target), _ptr(draft), ctypes.cast(c_par, ctypes.c_void_p),
                                     _ptr(tokens), _ptr(uniforms), _ptr(temperature),
                                     _ptr(out_tokens), _ptr(out_nodes), _ptr(num_accepted),
                                     _ptr(kv_len), _ptr(counters), B, N, V, dt, _ptr(workspace),
                                     ws_have, _stream(stream))
    _check("spec_reject_sample_tree", st)
    return out_tokens, out_nodes, num_accepted


def reject_sample_trees(target, draft, parents, tokens, uniforms, temperature, kv_len,
                        out_tokens=None, out_nodes=None, num_accepted=None, counters=None,
                        workspace=None, stream=None, top_k=None, top_p=None):
    """The tree verifier with one tree per sequence (see ``spec_reject_sample_trees``):
    parents [B, N] int32 on the device, parents[b][0] = -1 and
    parents[b][i] < i.  Everything else as ``reject_sample_tree``.
    Returns (out_tokens [B, N], out_nodes [B, N], num_accepted [B]), int32.
    """
    lib = load()
    B, N, V, dt = _tree_inputs(target, draft, tokens, uniforms, temperature, kv_len, out_tokens,
                               out_nodes, num_accepted, counters, top_k, top_p, parents=parents)
    _on_gpu(target=target, draft=draft, parents=parents, tokens=tokens, uniforms=uniforms,
            temperature=temperature, kv_len=kv_len, out_tokens=out_tokens, out_nodes=out_nodes,
            num_accepted=num_accepted, counters=counters, top_k=top_k, top_p=top_p)
    out_tokens, out_nodes, num_accepted = _tree_outputs(B, N, target.device, out_tokens, out_nodes,
                                                        num_accepted, counters)
    ws_bytes = (reject_sample_tree_filtered_workspace_bytes(B, N, V)
                if top_k is not None or top_p is not None else
                reject_sample_tree_workspace_bytes(B, N, V))
    workspace, ws_have = _workspace(workspace, ws_bytes, target.device)
    st = lib.spec_reject_sample_trees(
        _ptr(target), _ptr(draft), _ptr(parents), _ptr(tokens), _ptr(uniforms), _ptr(temperature),
        _ptr(top_k), _ptr(top_p), _ptr(out_tokens), _ptr(out_nodes), _ptr(num_accepted),
        _ptr(kv_len), _ptr(counters), B, N, V, dt, _ptr(workspace), ws_have, _stream(stream))
    _check("spec_reject_sample_trees", st)
    return out_tokens, out_nodes, num_accepted


def verify_attn_window(q, k_new, v_new, k_cache, v_cache, block_table, kv_len, anc=None,
                       mode=SV_WINDOW_APPEND, out=None, max_kv_len=None, scale=0.0,
                       workspace=None, stream=None):
    """Verify attention with the window's K/V from k_new / v_new [B, N, Hkv, D]
    (see ``spec_verify_attn_window``); mode SV_WINDOW_APPEND also stores them
    into the cache, SV_WINDOW_READ leaves the cache as it is.  anc: None
    (chain) or [B, N] int32 ancestor sets of a tree.  Returns out."""
    import torch
    lib = load()
    B, N, Hq, D, NB, Hkv, dt = _attn_common(q, k_cache, v_cache, block_table, kv_len, out)
    _need(k_new, "k_new", q.dtype, (B, N, Hkv, D))
    _need(v_new, "v_new", q.dtype, (B, N, Hkv, D))
    if anc is not None:
        _need(anc, "anc", torch.int32, (B, N))
    _on_gpu(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
            block_table=block_table, kv_len=kv_len, anc=anc, out=out)
    mbps = block_table.shape[1]
    if max_kv_len is None:
        max_kv_len = int(kv_len.max().item()) if B > 0 else 0
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = verify_attn_workspace_bytes(B, N - 1, Hq, Hkv, D, max_kv_len)
    workspace, ws_have = _workspace(workspace, ws_bytes, q.device)
    st = lib.spec_verify_attn_window(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(block_table), _ptr(kv_len), _ptr(anc),
                                     _ptr(out), B, N, Hq, Hkv, D, 16, NB, mbps, int(max_kv_len),
                                     float(scale), dt, int(mode), _ptr(workspace), ws_have,
                                     _stream(stream))
    _check("spec_verify_attn_window", st)
    return out


def kv_commit(k_cache, v_cache, block_table, kv_len, num_accepted, nodes=None, k_src=None,
              v_src=None, N=None, stream=None):
    """The surviving window rows into positions L0 .. L0 + n (see
    ``spec_kv_commit``).  nodes: None (chain) or [B, N] int32 (a tree's
    out_nodes); k_src / v_src: [B, N, Hkv, D] scratch rows, or None to move
    them in place.  N defaults to nodes.shape[1] or k_src.shape[1]."""
    import torch
    lib = load()
    _need(k_cache, "k_cache")
    dt = _dtype_code(k_cache)
    NB, Hkv, D = _kv_caches(k_cache, v_cache, k_cache.dtype)
    _need(num_accepted, "num_accepted", torch.int32)
    _dims(num_accepted, "num_accepted", 1)
    B = num_accepted.shape[0]
    _need(block_table, "block_table", torch.int32)
    _dims(block_table, "block_table", 2)
    if block_table.shape[0] != B:
        raise ValueError("block_table must have B = %d rows, got %d" % (B, block_table.shape[0]))
    _need(kv_len, "kv_len", torch.int32, (B,))
    if N is None:
        N = nodes.shape[1] if nodes is not None else (k_src.shape[1] if k_src is not None else 1)
    if nodes is not None:
        _need(nodes, "nodes", torch.int32, (B, N))
    if (k_src is None) != (v_src is None):
        raise ValueError("k_src and v_src go together")
    if k_src is not None:
        _need(k_src, "k_src", k_cache.dtype, (B, N, Hkv, D))
        _need(v_src, "v_src", k_cache.dtype, (B, N, Hkv, D))
    _on_gpu(k_cache=k_cache, v_cache=v_cache, block_table=block_table, kv_len=kv_len,
            num_accepted=num_accepted, nodes=nodes, k_src=k_src, v_src=v_src)
    st = lib.spec_kv_commit(_ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(kv_len),
                            _ptr(num_accepted), _ptr(nodes), _ptr(k_src), _ptr(v_src), B, int(N),
                            Hkv, D, 16, NB, block_table.shape[1], dt, _stream(stream))
    _check("spec_kv_commit", st)


class PagePool:
    """Host page list with provisional window pages (see ``spec_pages_*``)."""

    def __init__(self, num_blocks, max_seqs, max_blocks_per_seq):
        self._lib = load()
        self._h = self._lib.spec_pages_create(num_blocks, max_seqs, max_blocks_per_seq)
        if not self._h:
            raise SpecVerifyError("spec_pages_create", -1)
        self.num_blocks, self.max_seqs, self.mbps = num_blocks, max_seqs, max_blocks_per_seq

    def close(self):
        if self._h:
            self._lib.spec_pages_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reserve(self, seq, total_len):
        _check("spec_pages_reserve", self._lib.spec_pages_reserve(self._h, seq, total_len))

    def commit(self, seq, length):
        _check("spec_pages_commit", self._lib.spec_pages_commit(self._h, seq, length))

    def release(self, seq):
        _check("spec_pages_release", self._lib.spec_pages_release(self._h, seq))

    def free_count(self):
        return int(self._lib.spec_pages_free_count(self._h))

    def seq_blocks(self, seq):
        return int(self._lib.spec_pages_seq_blocks(self._h, seq))

    def check(self):
        return int(self._lib.spec_pages_check(self._h))

    def block_table(self):
        """A numpy copy of the [max_seqs, max_blocks_per_seq] int32 table."""
        import numpy as np
        ptr = self._lib.spec_pages_block_table(self._h)
        n = self.max_seqs * self.mbps
        return np.ctypeslib.as_array(ptr, shape=(n,)).copy().reshape(self.max_seqs, self.mbps)


class DraftLengthBandit:
    """Epsilon-greedy choice of the draft length (see ``spec_bandit_*``).

    arms: the draft lengths (the page's {0, 2, 4, 6, 8} by default).
    select(u_explore, u_arm) -> arm index; arms[index] is the length.
    update(index, reward) with the measured output tokens per second.
    """

    def __init__(self, arms=(0, 2, 4, 6, 8), warmup_rounds=2):
        self._lib = load()
        self.arms = tuple(int(a) for a in arms)
        self._h = self._lib.spec_bandit_create(len(self.arms), warmup_rounds)
        if not self._h:
            raise SpecVerifyError("spec_bandit_create", -1)

    def close(self):
        if self._h:
            self._lib.spec_bandit_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def select(self, u_explore, u_arm):
        r = self._lib.spec_bandit_select(self._h, float(u_explore), float(u_arm))
        if r < 0:
            raise SpecVerifyError("spec_bandit_select", r)
        return r

    def update(self, arm, reward):
        _check("spec_bandit_update", self._lib.spec_bandit_update(self._h, int(arm), float(reward)))

    def stats(self):
        """(pulls [n_arms], means [n_arms], t)."""
        k = len(self.arms)
        pulls = (ctypes.c_longlong * k)()
        means = (ctypes.c_double * k)()
        t = ctypes.c_longlong()
        _check("spec_bandit_stats", self._lib.spec_bandit_stats(
            self._h, ctypes.cast(pulls, ctypes.c_void_p), ctypes.cast(means, ctypes.c_void_p),
            ctypes.byref(t)))
        return list(pulls), list(means), t.value


def read_probe(buf, sink, grid, stream=None):
    """``spec_read_probe``: one streaming read of the bytes of ``buf`` (a
    device tensor, size a multiple of 8192 bytes) by ``grid`` workgroups;
    ``sink`` is a device int32 tensor of at least ``grid`` entries."""
    import torch
    _need(buf, "buf")
    _need(sink, "sink", torch.int32)
    if sink.numel() < grid:
        raise ValueError("sink needs %d entries" % grid)
    _on_gpu(buf=buf, sink=sink)
    _check("spec_read_probe", load().spec_read_probe(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(grid), _stream(stream)))


def accept_stats(num_accepted, K):
    """(a [K], mean_len) from a host array of num_accepted (see ``spec_accept_stats``)."""
    import numpy as np
    n = np.ascontiguousarray(num_accepted, dtype=np.int32)
    a = np.zeros(max(K, 1), dtype=np.float64)
    L = ctypes.c_double()
    _check("spec_accept_stats", load().spec_accept_stats(
        n.ctypes.data_as(ctypes.c_void_p), int(n.size), int(K), a.ctypes.data_as(ctypes.c_void_p),
        ctypes.byref(L)))
    return a[:K], L.value
