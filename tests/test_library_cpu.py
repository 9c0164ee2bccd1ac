"""Host-side checks of libloopspec that need no GPU: the shared library loads, exports every
function include/loopspec.h declares, the Python binding names the same set, and the
host-only Philox generator agrees with the oracle's (and with the published known answers,
through the oracle's own pinned test)."""

import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loopspec.h")
LIB = os.path.join(ROOT, "looped_transformer_self_amd", "libloopspec.so")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    pat = re.compile(r"(?:ls_status|void|size_t|const\s+char\s*\*)\s*\*?\s*(ls_[a-z0-9_]+)\s*\(")
    return sorted(set(pat.findall(text)))


def _lib():
    if not os.path.exists(LIB):
        pytest.skip("libloopspec.so is not built (run __graft_entry__.build())")
    return C.CDLL(LIB)


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("ls_prelude", "ls_loop_step", "ls_readout", "ls_verify", "ls_model_create", "ls_model_destroy",
              "ls_workspace_bytes", "ls_bind_workspace", "ls_sync_status", "ls_last_error"):
        assert n in names, n


def test_library_exports_every_declared_function():
    lib = _lib()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared in loopspec.h but not exported: {missing}"


def test_binding_names_match_header():
    from looped_transformer_self_amd import _lib as binding
    assert sorted(binding.EXPORTS) == _declared_functions()


def test_last_error_is_callable_without_gpu():
    lib = _lib()
    lib.ls_last_error.restype = C.c_char_p
    assert isinstance(lib.ls_last_error(), bytes)


@pytest.mark.parametrize("seed,pos", [(2, 0), (2, 511), (0xDEADBEEFCAFEF00D, 123456789), (7, 2 ** 33 + 5)])
def test_host_philox_matches_oracle(seed, pos):
    from oracle import philox
    lib = _lib()
    purposes = np.array([0, 1, 2, 3, 4, 5, 8, 9, 23], dtype=np.int32)
    out = np.zeros(len(purposes), dtype=np.uint32)
    lib.ls_philox_uniforms(C.c_uint64(seed), C.c_int64(pos), purposes.ctypes.data_as(C.c_void_p),
                           C.c_int(len(purposes)), out.ctypes.data_as(C.c_void_p))
    want = [philox.uniform(seed, pos, int(p)) for p in purposes]
    assert out.tolist() == want


def _desc(**kw):
    from looped_transformer_self_amd import _lib as binding
    d = binding.ls_model_desc()
    d.V, d.d, d.n_heads, d.head_dim, d.F = 49152, 2048, 16, 128, 5632
    d.L, d.L_pre, d.L_coda, d.R = 24, 0, 0, 4
    d.n_readout = 3
    for i, r in enumerate((2, 3, 4)):
        d.readout_depths[i] = r
    d.dtype, d.rope_theta, d.norm_eps = binding.LS_BF16, 10000.0, 1e-6
    d.slot_capacity = 1024
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("fields,status", [
    ({"V": 65537}, 2), ({"head_dim": 136, "d": 16 * 136}, 2), ({"head_dim": 120, "d": 16 * 120}, 2),
    ({"F": 5640}, 2), ({"n_heads": 15}, 1), ({"R": 0}, 1), ({"slot_capacity": 0}, 1)])
def test_model_create_rejects_unsupported_shapes(fields, status):
    """Shape checks happen on the host before any device work: out-of-contract descriptors
    come back as LS_ERR_INVALID (1) or LS_ERR_UNSUPPORTED (2) with a message."""
    from looped_transformer_self_amd import _lib as binding
    lib = _lib()
    lib.ls_model_create.restype = C.c_int
    lib.ls_last_error.restype = C.c_char_p
    d = _desc(**fields)
    w = binding.ls_weight_ptrs()
    out = C.c_void_p()
    st = lib.ls_model_create(C.byref(d), C.byref(w), C.byref(out))
    assert st == status, (st, lib.ls_last_error())
    assert lib.ls_last_error()


def test_prefill_host_contract():
    """ls_prefill's host-side checks and scratch size need no GPU: the scratch holds the
    chunk's residual stream and its coda copy (fp32), the normalised rows, attention outputs
    and SwiGLU outputs (model dtype) and q|k|v (fp32), each 256-byte aligned; a call without
    a bound workspace, with negative sizes or without a model is rejected before any device
    work, and n = 0 is a no-op."""
    from looped_transformer_self_amd import _lib as binding
    lib = _lib()
    lib.ls_model_create.restype = C.c_int
    lib.ls_prefill_workspace_bytes.restype = C.c_size_t
    lib.ls_prefill_workspace_bytes.argtypes = [C.c_void_p, C.c_int]
    lib.ls_prefill.restype = C.c_int
    lib.ls_prefill.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_uint,
                               C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    assert lib.ls_prefill_workspace_bytes(None, 16) == 0
    assert lib.ls_prefill(None, None, None, 4, None, 0, 1, None, None, None, 0, None) == binding.LS_ERR_INVALID
    d = _desc()
    fake = 0x1000                                  # pointers are only stored at creation
    lay = (binding.ls_layer_ptrs * d.L)(*[binding.ls_layer_ptrs(*([fake] * 9)) for _ in range(d.L)])
    w = binding.ls_weight_ptrs(fake, fake, None, lay, None)
    m = C.c_void_p()
    assert lib.ls_model_create(C.byref(d), C.byref(w), C.byref(m)) == binding.LS_OK
    try:
        al = lambda x: (x + 255) // 256 * 256
        for n in (1, 130, 2048):
            want = 2 * al(n * d.d * 4) + al(n * d.d * 2) + al(n * 3 * d.d * 4) + al(n * d.d * 2) + al(n * d.F * 2)
            assert lib.ls_prefill_workspace_bytes(m, n) == want, n
        kv = binding.ls_kv(fake, None, None)
        args = (fake, fake, 4, None, 0, 1, fake, C.addressof(kv), fake, 1 << 30, None)
        assert lib.ls_prefill(m, *args) == binding.LS_ERR_INVALID          # no workspace bound
        assert lib.ls_prefill(m, fake, fake, -1, None, 0, 1, fake, C.addressof(kv), fake, 1 << 30,
                              None) == binding.LS_ERR_INVALID
    finally:
        lib.ls_model_destroy(m)
