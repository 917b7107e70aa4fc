"""The C-ABI library: it loads, exports every symbol the header declares, and
its host-side checks return the documented status codes (no GPU needed: every
case here returns before anything is launched)."""

import ctypes
import os
import re

import pytest

import speculative_decoding_verification_verify_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")

FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.lib_path()):
        from speculative_decoding_verification_verify_amd import build
        build.build()
    return sv.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w ]*[\s*]+(spec_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == len(sv.EXPORTS) >= 7
    assert set(names) == set(sv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.spec_status_string(0) == b"ok"
    assert lib.spec_status_string(-3) == b"workspace too small"
    assert lib.spec_status_string(-6) == b"input breaks a precondition (validation mode)"
    assert lib.spec_status_string(99) == b"unknown status"
    assert lib.spec_version() >= 100


def test_workspace_sizes(lib):
    assert sv.reject_sample_workspace_bytes(0, 7, 128256) == 0
    assert sv.reject_sample_workspace_bytes(64, 0, 128256) == 0
    a = sv.reject_sample_workspace_bytes(64, 7, 128256)
    assert a > 0 and a % 256 == 0
    # 15 rows x 32 chunks x 8 B per sequence for the row statistics at least.
    assert a >= 64 * 15 * 32 * 8
    assert sv.reject_sample_workspace_bytes(128, 7, 128256) > a
    # The filtered sizes add the sweep's window: per swept row, two float64
    # sums per chunk and a 16-bit count per window value (512) per sweep block
    # of 4 chunks; invalid sizes give 0 as for the plain queries.
    f = sv.reject_sample_filtered_workspace_bytes(64, 7, 128256)
    nc = (128256 + 4095) // 4096
    assert f % 256 == 0 and f >= a + 64 * 15 * ((nc + 3) // 4) * 512 * 2 + 64 * 15 * nc * 16
    assert sv.reject_sample_filtered_workspace_bytes(0, 7, 128256) == 0
    assert sv.reject_sample_filtered_workspace_bytes(64, 17, 128256) == 0
    t = sv.reject_sample_tree_workspace_bytes(64, 15, 128256)
    tf = sv.reject_sample_tree_filtered_workspace_bytes(64, 15, 128256)
    assert tf % 256 == 0 and tf >= t + 64 * 29 * ((nc + 3) // 4) * 512 * 2
    assert sv.reject_sample_tree_filtered_workspace_bytes(4, 18, 100) == 0
    w = sv.verify_attn_workspace_bytes(64, 7, 32, 8, 128, 8192)
    assert w % 256 == 0 and w > 0
    assert sv.verify_attn_workspace_bytes(1, 1, 1, 1, 64, 0) == 0   # one split: no partials


def _reject(lib, B=4, K=3, V=100, dtype=1, ws_bytes=1 << 20, ptrs=True, draft=True):
    p = FAKE if ptrs else None
    return lib.spec_reject_sample(p, p if draft else None, p, p, p, p, p, p, None, B, K, V, dtype,
                                  p, ws_bytes, None)


def test_reject_validation(lib):
    assert _reject(lib, B=-1) == -1
    assert _reject(lib, K=0) == -1
    assert _reject(lib, V=0) == -1
    assert _reject(lib, dtype=7) == -1
    assert _reject(lib, K=17) == -2
    assert _reject(lib, B=1 << 27, K=16) == -2           # grid rows over 2^31
    assert _reject(lib, ptrs=False) == -1
    assert _reject(lib, ws_bytes=16) == -3
    assert _reject(lib, B=0, ptrs=False) == 0            # empty batch: no-op


def test_reject_noalloc_validation(lib):
    # Every case returns before the scratch array is looked up (no GPU call).
    f = lib.spec_reject_sample_noalloc
    p = FAKE
    assert f(p, p, p, p, p, p, p, p, None, -1, 3, 100, 1, None) == -1
    assert f(p, p, p, p, p, p, p, p, None, 4, 0, 100, 1, None) == -1
    assert f(p, p, p, p, p, p, p, p, None, 4, 3, 100, 9, None) == -1
    assert f(p, p, p, p, p, p, p, p, None, 4, 17, 100, 1, None) == -2
    assert f(None, None, None, None, None, None, None, None, None, 0, 3, 100, 1, None) == 0
    # Beyond the fixed array: refused.
    assert sv.reject_sample_workspace_bytes(4096, 16, 128256) > sv.NOALLOC_SCRATCH_BYTES
    assert f(p, p, p, p, p, p, p, p, None, 4096, 16, 128256, 1, None) == -3
    # The serving batches fit.
    assert sv.reject_sample_workspace_bytes(256, 7, 128256) <= sv.NOALLOC_SCRATCH_BYTES


def _attn(lib, B=2, K=7, Hq=32, Hkv=8, D=128, bs=16, nb=10, mbps=600, mkl=8192, dtype=1,
          ptrs=True, ws=1 << 30):
    p = FAKE if ptrs else None
    return lib.spec_verify_attn(p, p, p, p, p, p, B, K, Hq, Hkv, D, bs, nb, mbps, mkl,
                                ctypes.c_float(0.0), dtype, p, ws, None)


def test_attn_validation(lib):
    assert _attn(lib, B=-1) == -1
    assert _attn(lib, K=0) == -1
    assert _attn(lib, dtype=3) == -1
    assert _attn(lib, K=17) == -2
    assert _attn(lib, D=96) == -2
    assert _attn(lib, bs=32) == -2
    assert _attn(lib, Hq=30, Hkv=8) == -2                # Hq % Hkv != 0
    assert _attn(lib, Hq=72, Hkv=8) == -2                # 9 * 8 rows > 64
    assert _attn(lib, mbps=10, mkl=8192) == -1           # table too short for max_kv_len
    assert _attn(lib, ptrs=False) == -1
    assert _attn(lib, ws=100) == -3
    assert _attn(lib, B=0, ptrs=False) == 0


def test_python_wrapper_rejects_cpu_tensors(lib):
    import torch
    q = torch.zeros((1, 2, 1, 64))
    with pytest.raises(ValueError):
        sv.verify_attn(q, q, q, q.int(), q.int())


def test_tree_attn_validation(lib):
    p = FAKE
    f = lib.spec_verify_attn_tree
    # anc missing, N < 2, then the shared checks (D unsupported).
    assert f(p, p, p, p, p, None, p, 2, 8, 32, 8, 128, 16, 10, 600, 8192, 0.0, 1, p, 1 << 30, None) == -1
    assert f(p, p, p, p, p, p, p, 2, 1, 32, 8, 128, 16, 10, 600, 8192, 0.0, 1, p, 1 << 30, None) == -1
    assert f(p, p, p, p, p, p, p, 2, 8, 32, 8, 96, 16, 10, 600, 8192, 0.0, 1, p, 1 << 30, None) == -2
    assert f(p, p, p, p, p, p, p, 2, 18, 32, 8, 128, 16, 10, 600, 8192, 0.0, 1, p, 1 << 30, None) == -2
    assert f(None, None, None, None, None, None, None, 0, 8, 32, 8, 128, 16, 10, 600, 8192, 0.0, 1,
             None, 0, None) == 0                               # empty batch: no-op


def _tree_reject(lib, parent=(-1, 0, 0, 1), B=4, V=100, dtype=1, ws_bytes=1 << 24, ptrs=True,
                 N=None):
    p = FAKE if ptrs else None
    n = (4 if parent is None else len(parent)) if N is None else N
    par = None if parent is None else (ctypes.c_int32 * len(parent))(*parent)
    return lib.spec_reject_sample_tree(p, p, None if par is None else ctypes.cast(par, ctypes.c_void_p),
                                       p, p, p, p, p, p, p, None, B, n, V, dtype, p, ws_bytes, None)


def test_tree_reject_validation(lib):
    need = sv.reject_sample_tree_workspace_bytes(4, 4, 100)
    assert need > 0 and need % 256 == 0
    assert _tree_reject(lib, ws_bytes=need - 1) == -3
    assert _tree_reject(lib, parent=None) == -1                  # no topology
    assert _tree_reject(lib, parent=(0, 0, 1)) == -1             # root must have parent -1
    assert _tree_reject(lib, parent=(-1, 0, 2)) == -1            # parent[i] >= i
    assert _tree_reject(lib, parent=(-1, -1, 0)) == -1           # a second root
    assert _tree_reject(lib, parent=(-1, 0, 0, 5)) == -1         # parent out of range
    assert _tree_reject(lib, B=-1) == -1
    assert _tree_reject(lib, V=0) == -1
    assert _tree_reject(lib, dtype=5) == -1
    assert _tree_reject(lib, parent=tuple([-1] + list(range(17)))) == -2   # N = 18 > SV_MAX_K + 1
    assert _tree_reject(lib, ptrs=False) == -1
    assert _tree_reject(lib, B=0, ptrs=False) == 0               # empty batch: no-op
    assert _tree_reject(lib, parent=(-1,), B=0, ptrs=False) == 0 # a root alone is a valid tree


def test_filtered_tree_reject_validation(lib):
    """The filtered tree call checks its arguments as the plain one does
    (nothing is launched: every return below comes before any device work)."""
    def call(parent=(-1, 0, 0, 1), B=4, V=100, dtype=1, ws_bytes=1 << 24, ptrs=True):
        p = FAKE if ptrs else None
        par = None if parent is None else (ctypes.c_int32 * len(parent))(*parent)
        n = 4 if parent is None else len(parent)
        return lib.spec_reject_sample_tree_filtered(
            p, p, None if par is None else ctypes.cast(par, ctypes.c_void_p), p, p, p, p, p, p, p,
            p, p, None, B, n, V, dtype, p, ws_bytes, None)
    need = sv.reject_sample_tree_workspace_bytes(4, 4, 100)
    assert call(ws_bytes=need - 1) == -3
    assert call(parent=None) == -1
    assert call(parent=(-1, 0, 2)) == -1
    assert call(B=-1) == -1 and call(V=0) == -1 and call(dtype=5) == -1
    assert call(parent=tuple([-1] + list(range(17)))) == -2
    assert call(ptrs=False) == -1
    assert call(B=0, ptrs=False) == 0                            # an empty batch is a no-op


def test_per_sequence_tree_reject_validation(lib):
    """spec_reject_sample_trees: parents live on the device, so only their
    presence is checked here (nothing is launched below)."""
    def call(B=4, N=4, V=100, dtype=1, ws_bytes=1 << 24, parents=True, ptrs=True):
        p = FAKE if ptrs else None
        return lib.spec_reject_sample_trees(p, p, FAKE if parents else None, p, p, p, None, None, p,
                                            p, p, p, None, B, N, V, dtype, p, ws_bytes, None)
    need = sv.reject_sample_tree_workspace_bytes(4, 4, 100)
    assert call(ws_bytes=need - 1) == -3
    assert call(parents=False) == -1                          # B > 0 needs the parents
    assert call(B=0, parents=False, ptrs=False) == 0          # empty batch: no-op
    assert call(N=0) == -1 and call(V=0) == -1 and call(dtype=5) == -1 and call(B=-1) == -1
    assert call(N=18) == -2
    assert call(ptrs=False) == -1


def test_tree_reject_workspace_matches_chain(lib):
    # A chain of K + 1 nodes sweeps the same 2K + 1 rows as the chain call;
    # the tree adds its walk state and merged row statistics, the chain its
    # per-row top-k / top-p results.
    for B, K, V in [(64, 7, 128256), (1, 1, 1000), (3, 16, 152064)]:
        t = sv.reject_sample_tree_workspace_bytes(B, K + 1, V)
        c = sv.reject_sample_workspace_bytes(B, K, V)
        filters = (B * (2 * K + 1) * 16 + 255) // 256 * 256   # the chain's per-row filter results
        assert t >= c - filters > 0
    assert sv.reject_sample_tree_workspace_bytes(0, 4, 100) == 0
    assert sv.reject_sample_tree_workspace_bytes(4, 0, 100) == 0
    assert sv.reject_sample_tree_workspace_bytes(4, 18, 100) == 0


def _win(lib, B=2, N=8, mode=1, kn=True, D=128, dtype=1, ws=1 << 30):
    p = FAKE
    k = p if kn else None
    return lib.spec_verify_attn_window(p, k, k, p, p, p, p, None, p, B, N, 32, 8, D, 16, 10, 600,
                                       8192, ctypes.c_float(0.0), dtype, mode, p, ws, None)


def test_window_attn_validation(lib):
    assert _win(lib, N=1) == -1                          # a window needs the root and a draft
    assert _win(lib, mode=2) == -1
    assert _win(lib, kn=False) == -1
    assert _win(lib, D=96) == -2                         # then the shared checks
    assert _win(lib, N=18) == -2
    assert _win(lib, ws=10) == -3
    assert _win(lib, B=0, kn=False) == 0                 # empty batch: no-op


def _commit(lib, B=2, N=8, nodes=True, src=0, D=128, dtype=1):
    p = FAKE
    s = p if src else None
    return lib.spec_kv_commit(p, p, p, p, p, p if nodes else None, s, p if src == 2 else s, B, N, 8,
                              D, 16, 10, 600, dtype, None)


def test_kv_commit_validation(lib):
    assert _commit(lib, B=-1) == -1
    assert _commit(lib, N=0) == -1
    assert _commit(lib, dtype=4) == -1
    assert lib.spec_kv_commit(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 2, 8, 8, 128, 16, 10,
                              600, 1, None) == -1          # only one of k_src / v_src
    assert _commit(lib, N=18) == -2
    assert _commit(lib, D=80) == -2
    assert _commit(lib, B=0) == 0
    assert _commit(lib, nodes=False, src=0) == 0          # chain in place: nothing to move


MISALIGNED = ctypes.c_void_p(0x10008)   # 8-byte but not 16-byte aligned; never dereferenced


def test_vector_copies_need_16_byte_alignment(lib):
    # spec_kv_commit moves keys, value runs and scratch rows as 16-byte
    # vectors in either dtype.
    assert lib.spec_kv_commit(FAKE, FAKE, FAKE, FAKE, FAKE, None, MISALIGNED, FAKE, 2, 8, 8, 128, 16,
                              10, 600, 0, None) == -1
    assert lib.spec_kv_commit(MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 2, 8, 8, 128, 16,
                              10, 600, 0, None) == -1
    # Append mode's copy as well, fp32 included; read mode in fp32 has no
    # such requirement, so only the append case is checked here.
    p = FAKE
    for dtype in (0, 1):
        assert lib.spec_verify_attn_window(p, MISALIGNED, MISALIGNED, p, p, p, p, None, p, 2, 8, 32,
                                           8, 128, 16, 10, 600, 8192, ctypes.c_float(0.0), dtype, 1,
                                           p, 1 << 30, None) == -1


# ---- the Python binding's argument checks (CPU tensors: every shape error is
# raised before the device check, and nothing reaches the library) -----------

def _rej_args(B=3, K=4, V=50, dtype=None):
    import torch
    dt = torch.bfloat16 if dtype is None else dtype
    return dict(target=torch.zeros((B, K + 1, V), dtype=dt), draft=torch.zeros((B, K, V), dtype=dt),
                draft_tokens=torch.zeros((B, K), dtype=torch.int32),
                uniforms=torch.zeros((B, K + 1), dtype=torch.float32),
                temperature=torch.ones((B,), dtype=torch.float32),
                kv_len=torch.zeros((B,), dtype=torch.int32))


def _raises_about(name, fn, **kw):
    with pytest.raises((ValueError, TypeError)) as ei:
        fn(**kw)
    assert name in str(ei.value), (name, str(ei.value))


def test_binding_reject_shapes(lib):
    import torch
    f = sv.reject_sample
    a = _rej_args()
    _raises_about("target", f, **a)                                   # right shapes: on the GPU check
    bad = {
        "draft": torch.zeros((3, 5, 50), dtype=torch.bfloat16),         # [B, K+1, V] instead of [B, K, V]
        "draft_tokens": torch.zeros((3, 5), dtype=torch.int32),
        "uniforms": torch.zeros((3, 4), dtype=torch.float32),
        "temperature": torch.ones((4,), dtype=torch.float32),
        "kv_len": torch.zeros((2,), dtype=torch.int32),
        "out_tokens": torch.zeros((3, 4), dtype=torch.int32),
        "num_accepted": torch.zeros((3, 1), dtype=torch.int32),
        "counters": torch.zeros((3,), dtype=torch.int64),
        "top_k": torch.zeros((2,), dtype=torch.int32),
        "top_p": torch.zeros((3, 1), dtype=torch.float32),
    }
    for name, t in bad.items():
        kw = dict(_rej_args())
        kw[name] = t
        _raises_about(name, f, **kw)
    kw = dict(_rej_args())
    kw["draft_tokens"] = torch.zeros((3, 4), dtype=torch.int64)       # wrong dtype
    _raises_about("draft_tokens", f, **kw)
    kw = dict(_rej_args())
    kw["draft"] = torch.zeros((3, 4, 50), dtype=torch.float32)        # dtype differs from target
    _raises_about("draft", f, **kw)
    kw = dict(_rej_args())
    kw["target"] = torch.zeros((3, 5), dtype=torch.bfloat16)
    _raises_about("target", f, **kw)
    # The no-allocation call takes the same shapes.
    kw = dict(_rej_args())
    kw.update(out_tokens=torch.zeros((3, 5), dtype=torch.int32),
              num_accepted=torch.zeros((4,), dtype=torch.int32))
    _raises_about("num_accepted", sv.reject_sample_noalloc, **kw)


def test_binding_tree_reject_shapes(lib):
    import torch
    B, N, V = 2, 4, 30
    base = dict(target=torch.zeros((B, N, V), dtype=torch.bfloat16),
                draft=torch.zeros((B, N, V), dtype=torch.bfloat16), parent=[-1, 0, 0, 1],
                tokens=torch.zeros((B, N), dtype=torch.int32),
                uniforms=torch.zeros((B, N), dtype=torch.float32),
                temperature=torch.ones((B,), dtype=torch.float32),
                kv_len=torch.zeros((B,), dtype=torch.int32))
    f = sv.reject_sample_tree
    _raises_about("target", f, **base)
    for name, t in {"draft": torch.zeros((B, N - 1, V), dtype=torch.bfloat16),
                    "tokens": torch.zeros((B, N - 1), dtype=torch.int32),
                    "uniforms": torch.zeros((B + 1, N), dtype=torch.float32),
                    "out_nodes": torch.zeros((B, N + 1), dtype=torch.int32),
                    "kv_len": torch.zeros((B, 1), dtype=torch.int32)}.items():
        kw = dict(base)
        kw[name] = t
        _raises_about(name, f, **kw)
    kw = dict(base)
    kw["parent"] = [-1, 0, 0]
    _raises_about("parent", f, **kw)


def _attn_args(B=2, K1=8, Hq=32, Hkv=8, D=128, NB=40, mbps=20, dt=None):
    import torch
    dt = torch.bfloat16 if dt is None else dt
    x = 16 // torch.zeros((), dtype=dt).element_size()
    return dict(q=torch.zeros((B, K1, Hq, D), dtype=dt),
                k_cache=torch.zeros((NB, Hkv, D // x, 16, x), dtype=dt),
                v_cache=torch.zeros((NB, Hkv, D, 16), dtype=dt),
                block_table=torch.zeros((B, mbps), dtype=torch.int32),
                kv_len=torch.zeros((B,), dtype=torch.int32))


def test_binding_attention_shapes(lib):
    import torch
    f = sv.verify_attn
    _raises_about("q", f, **_attn_args())                             # right shapes: device check
    a = _attn_args()
    for name, t in {"k_cache": torch.zeros((40, 8, 16, 16, 4), dtype=torch.bfloat16),   # X = 4 for bf16
                    "v_cache": torch.zeros((40, 8, 16, 128), dtype=torch.bfloat16),     # [NB,Hkv,16,D]
                    "block_table": torch.zeros((3, 20), dtype=torch.int32),
                    "kv_len": torch.zeros((3,), dtype=torch.int32),
                    "out": torch.zeros((2, 8, 32, 64), dtype=torch.bfloat16)}.items():
        kw = dict(a)
        kw[name] = t
        _raises_about(name, f, **kw)
    kw = _attn_args(D=64)
    kw["q"] = torch.zeros((2, 8, 32, 128), dtype=torch.bfloat16)      # q's D disagrees with the caches
    _raises_about("head dim", f, **kw)
    kw = _attn_args(dt=torch.float32)                                 # fp32 caches use X = 4
    _raises_about("q", f, **kw)
    kw = _attn_args()
    _raises_about("anc", sv.verify_attn_tree, anc=torch.zeros((2, 7), dtype=torch.int32), **kw)
    # Window call: k_new / v_new are [B, N, Hkv, D].
    kw = _attn_args()
    kn = torch.zeros((2, 8, 8, 128), dtype=torch.bfloat16)
    _raises_about("v_new", sv.verify_attn_window, k_new=kn,
                  v_new=torch.zeros((2, 8, 8, 64), dtype=torch.bfloat16), **kw)
    _raises_about("anc", sv.verify_attn_window, k_new=kn, v_new=kn,
                  anc=torch.zeros((2, 9), dtype=torch.int32), **kw)


def test_binding_kv_commit_shapes(lib):
    import torch
    a = _attn_args()
    base = dict(k_cache=a["k_cache"], v_cache=a["v_cache"], block_table=a["block_table"],
                kv_len=a["kv_len"], num_accepted=torch.zeros((2,), dtype=torch.int32))
    f = sv.kv_commit
    _raises_about("k_cache", f, **base)                               # right shapes: device check
    kw = dict(base)
    kw["nodes"] = torch.zeros((2, 8), dtype=torch.int32)
    kw["kv_len"] = torch.zeros((3,), dtype=torch.int32)
    _raises_about("kv_len", f, **kw)
    kw = dict(base)
    kw.update(k_src=torch.zeros((2, 8, 8, 128), dtype=torch.bfloat16),
              v_src=torch.zeros((2, 8, 4, 128), dtype=torch.bfloat16))
    _raises_about("v_src", f, **kw)
    kw = dict(base)
    kw.update(k_src=torch.zeros((2, 8, 8, 128), dtype=torch.bfloat16))
    _raises_about("v_src", f, **kw)
