"""ctypes binding of libloopspec (include/loopspec.h): same names, argument marshalling only.

The shared library is built in-tree (looped_transformer_self_amd/libloopspec.so) by
`build_lib.build()`; importing this module without it raises, so no path can silently run
without the HIP kernels.
"""

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libloopspec.so")

LS_OK, LS_ERR_INVALID, LS_ERR_UNSUPPORTED, LS_ERR_CAPACITY, LS_ERR_HIP = range(5)
LS_F32, LS_BF16 = 0, 1
LS_MAX_READOUT_DEPTHS = 8
LS_MAX_ROWS = 128
LS_STATIC_SCRATCH_BYTES = 64 << 20
LS_UNIFORMS_PER_JOB = 24
LS_JOB_SAMPLE, LS_JOB_DRAW1, LS_JOB_DRAW2, LS_JOB_VERIFY, LS_JOB_VERIFY_COPY, LS_JOB_SCREEN = range(6)
LS_JOB_NON_RESIDUAL = 1
LS_OUT_ACC1, LS_OUT_ACC2, LS_OUT_RESAMPLED, LS_OUT_DRAWN, LS_OUT_ACC_COPY, LS_OUT_SCREENED = 1, 2, 3, 4, 5, 6

EXPORTS = ("ls_last_error", "ls_model_create", "ls_model_destroy", "ls_workspace_bytes", "ls_bind_workspace",
           "ls_prelude", "ls_loop_step", "ls_readout", "ls_verify", "ls_sync_status", "ls_philox_uniforms",
           "ls_debug_trace", "ls_set_wait_limit", "ls_loop_step_static", "ls_measure_stream_read",
           "ls_prefill_workspace_bytes", "ls_prefill")


class ls_model_desc(C.Structure):
    _fields_ = [("V", C.c_int), ("d", C.c_int), ("n_heads", C.c_int), ("head_dim", C.c_int), ("F", C.c_int),
                ("L", C.c_int), ("L_pre", C.c_int), ("L_coda", C.c_int), ("R", C.c_int),
                ("n_readout", C.c_int), ("readout_depths", C.c_int * LS_MAX_READOUT_DEPTHS),
                ("dtype", C.c_int), ("rope_theta", C.c_float), ("norm_eps", C.c_float),
                ("slot_capacity", C.c_int)]


class ls_layer_ptrs(C.Structure):
    _fields_ = [(k, C.c_void_p) for k in ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd", "g1", "g2")]


class ls_weight_ptrs(C.Structure):
    _fields_ = [("emb", C.c_void_p), ("g_final", C.c_void_p), ("pre", C.POINTER(ls_layer_ptrs)),
                ("core", C.POINTER(ls_layer_ptrs)), ("coda", C.POINTER(ls_layer_ptrs))]


class ls_kv(C.Structure):
    _fields_ = [("core", C.c_void_p), ("pre", C.c_void_p), ("coda", C.c_void_p)]


class ls_rows(C.Structure):
    _fields_ = [("n", C.c_int), ("n_fin", C.c_int), ("max_anc", C.c_int),
                ("slot", C.c_void_p), ("pos", C.c_void_p), ("depth", C.c_void_p), ("fin_slots", C.c_void_p),
                ("anc_off", C.c_void_p), ("anc_slots", C.c_void_p)]


class ls_sampling(C.Structure):
    _fields_ = [("greedy", C.c_int), ("temperature", C.c_float), ("top_p", C.c_float)]


class ls_verify_job(C.Structure):
    _fields_ = [(k, C.c_int32) for k in ("op", "p_row", "q1_row", "q2_row", "x1", "x2", "gate", "cand_off",
                                          "n_cand", "flags")]


class ls_verify_out(C.Structure):
    _fields_ = [(k, C.c_int32) for k in ("token", "outcome", "gate", "aux")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with looped_transformer_self_amd.build_lib.build() "
                          "(there is no CPU fallback)")
    # PyTorch owns the device memory and streams the library works on, and it brings its own
    # HIP runtime (same soname as the system one).  Loading torch first makes the library bind
    # to that runtime; loaded the other way round, the process would hold two HIP runtimes and
    # the library would see none of torch's allocations.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    sig = {
        "ls_last_error": (C.c_char_p, []),
        "ls_model_create": (C.c_int, [C.POINTER(ls_model_desc), C.POINTER(ls_weight_ptrs), C.POINTER(P)]),
        "ls_model_destroy": (None, [P]),
        "ls_workspace_bytes": (C.c_size_t, [P, C.c_int, C.c_int, C.c_int]),
        "ls_bind_workspace": (C.c_int, [P, P, C.c_int, C.c_int, C.c_int, P]),
        "ls_prelude": (C.c_int, [P, C.POINTER(ls_rows), P, P, C.POINTER(ls_kv), P]),
        "ls_loop_step": (C.c_int, [P, C.POINTER(ls_rows), P, C.POINTER(ls_kv), P]),
        "ls_readout": (C.c_int, [P, C.POINTER(ls_rows), P, C.POINTER(ls_sampling), P, P, C.c_int, P, P,
                                 C.POINTER(ls_kv), P]),
        "ls_verify": (C.c_int, [P, P, C.c_int, P, C.c_int, P, C.c_int, P, P, P]),
        "ls_sync_status": (C.c_int, [P, P]),
        "ls_debug_trace": (C.c_int, [P, P, C.POINTER(C.c_int)]),
        "ls_set_wait_limit": (C.c_int, [P, C.c_double]),
        "ls_loop_step_static": (C.c_int, [P, C.POINTER(ls_rows), P, C.POINTER(ls_kv), P, P]),
        "ls_measure_stream_read": (C.c_int, [P, C.c_size_t, C.c_int, P]),
        "ls_prefill_workspace_bytes": (C.c_size_t, [P, C.c_int]),
        "ls_prefill": (C.c_int, [P, P, P, C.c_int, P, C.c_int, C.c_uint, P, C.POINTER(ls_kv), P, C.c_size_t, P]),
        "ls_philox_uniforms": (None, [C.c_uint64, C.c_int64, C.POINTER(C.c_int32), C.c_int,
                                      C.POINTER(C.c_uint32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


class LoopSpecError(RuntimeError):
    def __init__(self, status, where):
        msg = lib.ls_last_error().decode(errors="replace")
        super().__init__(f"{where} failed with status {status}: {msg}")
        self.status = status


def check(status, where):
    if status != LS_OK:
        raise LoopSpecError(status, where)


def philox_uniforms(seed, pos, purposes):
    n = len(purposes)
    arr_p = (C.c_int32 * n)(*purposes)
    out = (C.c_uint32 * n)()
    lib.ls_philox_uniforms(C.c_uint64(seed), C.c_int64(pos), arr_p, n, out)
    return list(out)
