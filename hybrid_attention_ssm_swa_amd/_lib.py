"""ctypes binding of libhymba_mixer.so: the C-ABI functions under the same names.

Argument marshalling only.  Pointers are plain integers (device addresses,
e.g. ``tensor.data_ptr()``) and streams are raw hipStream_t handles
(``torch.cuda.current_stream().cuda_stream``).  A non-zero status raises
HymbaError carrying hymba_last_error().  Loading fails loudly if the library
has not been built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhymba_mixer.so")

HYMBA_OK = 0
HYMBA_ERR_INVALID_ARG = -1
HYMBA_ERR_UNSUPPORTED = -2
HYMBA_ERR_WORKSPACE = -3
HYMBA_ERR_BIND = -4
HYMBA_ERR_HIP = -5
HYMBA_ERR_RANGE = -6
HYMBA_F32 = 0
HYMBA_BF16 = 1
HYMBA_F16 = 2
HYMBA_GEMM_LIBRARY = 0
HYMBA_GEMM_TILED = 1

EXPORTED = [
    "hymba_layer_persistent_bytes", "hymba_layer_create", "hymba_layer_destroy",
    "hymba_kv_share_bind", "hymba_mixer_workspace_bytes", "hymba_layer_prepare",
    "hymba_mixer_prefill", "hymba_mixer_decode", "hymba_layer_meta_outputs",
    "hymba_last_error", "hymba_status_string", "hymba_kernel_attention",
    "hymba_kernel_selective_scan", "hymba_kernel_epilogue", "hymba_kernel_gemm_rows",
    "hymba_kernel_gemm_rows_workspace", "hymba_kernel_selective_scan_workspace",
    "hymba_layer_profile", "hymba_layer_profile_read", "hymba_stage_name",
    "hymba_layer_check", "hymba_layer_set_overlap", "hymba_mixer_decode_static",
    "hymba_kernel_gemm_tiles", "hymba_layer_set_gemm",
    "griffin_block_persistent_bytes", "griffin_block_prepare", "griffin_workspace_bytes",
    "griffin_block_prefill", "griffin_block_decode",
]
HYMBA_N_STAGES = 9
GRIFFIN_N_STAGES = 5
GRIFFIN_STAGES = ["in_proj", "conv", "gate_proj", "rglru", "out_proj"]


class HymbaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)} ({status}): {message}")
        self.status = status


class hymba_layer_cfg(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("d_inner", c_int32), ("d_state", c_int32),
                ("n_meta", c_int32), ("window", c_int32), ("own_kv", c_int32),
                ("dtype", c_int32), ("rms_eps", c_float),
                ("rope_base", c_float)]


class hymba_layer_weights(ctypes.Structure):
    _fields_ = [("w_in", c_void_p), ("w_o", c_void_p), ("w_out", c_void_p), ("meta", c_void_p),
                ("A", c_void_p), ("D", c_void_p), ("dt_bias", c_void_p), ("beta1", c_void_p),
                ("beta2", c_void_p)]


class griffin_block_cfg(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("d_rnn", c_int32), ("dtype", c_int32), ("c", c_float)]


class griffin_block_weights(ctypes.Structure):
    _fields_ = [("w_in", c_void_p), ("conv_w", c_void_p), ("w_gate", c_void_p), ("lam", c_void_p),
                ("w_out", c_void_p)]


class hymba_kv(ctypes.Structure):
    _fields_ = [("k_meta", c_void_p), ("v_meta", c_void_p), ("k", c_void_p), ("v", c_void_p),
                ("k_cache", c_void_p), ("v_cache", c_void_p), ("cache_len", c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run hybrid_attention_ssm_swa_amd/build.py "
                           "(or __graft_entry__.build()) first")
    # PyTorch ships its own HIP runtime: load it first so that the library binds to the same
    # runtime as the tensors and streams it is handed (a second runtime sees no device).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = c_void_p
    sig = {
        "hymba_layer_persistent_bytes": (c_size_t, [POINTER(hymba_layer_cfg)]),
        "hymba_layer_create": (c_int32, [POINTER(hymba_layer_cfg), POINTER(hymba_layer_weights), P, c_size_t,
                                         POINTER(c_void_p)]),
        "hymba_layer_destroy": (None, [P]),
        "hymba_kv_share_bind": (c_int32, [P, P]),
        "hymba_mixer_workspace_bytes": (c_size_t, [P, c_int32, c_int32]),
        "hymba_layer_prepare": (c_int32, [P, POINTER(hymba_kv), P, c_size_t, P]),
        "hymba_mixer_prefill": (c_int32, [P, P, c_int32, c_int32, P, POINTER(hymba_kv), P, P, c_size_t, P]),
        "hymba_mixer_decode": (c_int32, [P, P, P, c_int32, P, POINTER(hymba_kv), P, P, c_size_t, P]),
        "hymba_layer_meta_outputs": (c_int32, [P, POINTER(c_void_p), POINTER(c_void_p), POINTER(c_void_p),
                                               POINTER(c_void_p)]),
        "hymba_last_error": (c_char_p, []),
        "hymba_status_string": (c_char_p, [c_int32]),
        "hymba_kernel_attention": (c_int32, [c_int32, P, c_int64, P, P, c_int64, c_int64, P, P, c_int32, P,
                                             c_int64, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, P]),
        "hymba_kernel_selective_scan": (c_int32, [c_int32, P, P, c_int64, P, c_int64, P, P, P, P, P, c_int64, P,
                                                  c_int32, c_int32, c_int32, c_int32, P, c_size_t, P]),
        "hymba_kernel_epilogue": (c_int32, [c_int32, P, c_int64, P, c_int64, P, c_int64, P, P, P, c_int64,
                                            c_int64, c_int32, c_float, P]),
        "hymba_kernel_gemm_rows": (c_int32, [c_int32, c_int32, c_int32, P, c_int64, P, c_int64, P, c_int64, P,
                                             c_int64, c_int32, c_int32, c_int32, c_int32, c_int32, P, c_size_t, P]),
        "hymba_kernel_gemm_rows_workspace": (c_size_t, [c_int32, c_int32, c_int32]),
        "hymba_kernel_gemm_tiles": (c_int32, [c_int32, c_int32, P, c_int64, P, c_int64, P, c_int64, P, c_int64,
                                              c_int32, c_int32, c_int64, c_int32, c_int32, P]),
        "hymba_layer_set_gemm": (c_int32, [P, c_int32]),
        "hymba_kernel_selective_scan_workspace": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
        "hymba_layer_profile": (c_int32, [P, c_int32]),
        "hymba_layer_profile_read": (c_int32, [P, POINTER(c_float), c_int32]),
        "hymba_stage_name": (c_char_p, [c_int32]),
        "hymba_layer_check": (c_int32, [P, P]),
        "hymba_layer_set_overlap": (c_int32, [P, c_int32]),
        "hymba_mixer_decode_static": (c_int32, [P, P, P, c_int32, P, POINTER(hymba_kv), P, P]),
        "griffin_block_persistent_bytes": (c_size_t, [POINTER(griffin_block_cfg)]),
        "griffin_block_prepare": (c_int32, [POINTER(griffin_block_cfg), POINTER(griffin_block_weights), P,
                                            c_size_t, P]),
        "griffin_workspace_bytes": (c_size_t, [POINTER(griffin_block_cfg), c_int32, c_int32]),
        "griffin_block_prefill": (c_int32, [POINTER(griffin_block_cfg), POINTER(griffin_block_weights), P, P,
                                            c_int32, c_int32, P, P, P, P, P, P, c_size_t, P, POINTER(c_float)]),
        "griffin_block_decode": (c_int32, [POINTER(griffin_block_cfg), POINTER(griffin_block_weights), P, P,
                                           c_int32, P, P, P, P, c_size_t, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_name(status: int) -> str:
    names = {0: "HYMBA_OK", -1: "HYMBA_ERR_INVALID_ARG", -2: "HYMBA_ERR_UNSUPPORTED",
             -3: "HYMBA_ERR_WORKSPACE", -4: "HYMBA_ERR_BIND", -5: "HYMBA_ERR_HIP", -6: "HYMBA_ERR_RANGE"}
    return names.get(status, "HYMBA_UNKNOWN_STATUS")


def _check(status: int) -> int:
    if status != HYMBA_OK:
        raise HymbaError(status, hymba_last_error())
    return status


def _kv_ptr(kv):
    return None if kv is None else ctypes.byref(kv)


# --- the C-ABI, same names -------------------------------------------------------

def hymba_last_error() -> str:
    msg = load_library().hymba_last_error()
    return msg.decode() if msg else ""


def hymba_status_string(status: int) -> str:
    return load_library().hymba_status_string(status).decode()


def hymba_layer_persistent_bytes(cfg: hymba_layer_cfg) -> int:
    return load_library().hymba_layer_persistent_bytes(ctypes.byref(cfg))


def hymba_layer_create(cfg: hymba_layer_cfg, weights: hymba_layer_weights, persistent: int,
                       persistent_bytes: int) -> int:
    out = c_void_p()
    _check(load_library().hymba_layer_create(ctypes.byref(cfg), ctypes.byref(weights), persistent,
                                             persistent_bytes, ctypes.byref(out)))
    return out.value


def hymba_layer_destroy(layer: int) -> None:
    load_library().hymba_layer_destroy(layer)


def hymba_kv_share_bind(consumer: int, producer) -> None:
    _check(load_library().hymba_kv_share_bind(consumer, producer))


def hymba_mixer_workspace_bytes(layer: int, batch: int, seq: int) -> int:
    return load_library().hymba_mixer_workspace_bytes(layer, batch, seq)


def hymba_layer_prepare(layer: int, kv, workspace: int, workspace_bytes: int, stream: int) -> None:
    _check(load_library().hymba_layer_prepare(layer, _kv_ptr(kv), workspace, workspace_bytes, stream))


def hymba_mixer_prefill(layer: int, x: int, B: int, T: int, y: int, kv, ssm_state_out, workspace: int,
                        workspace_bytes: int, stream: int) -> None:
    _check(load_library().hymba_mixer_prefill(layer, x, B, T, y, _kv_ptr(kv), ssm_state_out, workspace,
                                               workspace_bytes, stream))


def hymba_mixer_decode(layer: int, x_t: int, pos: int, B: int, y_t: int, kv, ssm_state: int, workspace: int,
                       workspace_bytes: int, stream: int) -> None:
    _check(load_library().hymba_mixer_decode(layer, x_t, pos, B, y_t, _kv_ptr(kv), ssm_state, workspace,
                                              workspace_bytes, stream))


def hymba_mixer_decode_static(layer: int, x_t: int, pos: int, B: int, y_t: int, kv, ssm_state: int,
                              stream: int) -> None:
    _check(load_library().hymba_mixer_decode_static(layer, x_t, pos, B, y_t, _kv_ptr(kv), ssm_state, stream))


def hymba_layer_meta_outputs(layer: int):
    k, v, h, y = c_void_p(), c_void_p(), c_void_p(), c_void_p()
    _check(load_library().hymba_layer_meta_outputs(layer, ctypes.byref(k), ctypes.byref(v), ctypes.byref(h),
                                                    ctypes.byref(y)))
    return k.value, v.value, h.value, y.value


def hymba_kernel_attention(dtype, q, ld_q, k, v, ld_kv, kv_seq_stride, k_meta, v_meta, n_meta, o, ld_o, B, T,
                           n_heads, n_kv_heads, head_dim, window, stream) -> None:
    _check(load_library().hymba_kernel_attention(dtype, q, ld_q, k, v, ld_kv, kv_seq_stride, k_meta, v_meta,
                                                 n_meta, o, ld_o, B, T, n_heads, n_kv_heads, head_dim, window,
                                                 stream))


def hymba_kernel_selective_scan(dtype, u, dt, ld, bc, ld_bc, A, D, dt_bias, h0, y, ldy, h_out, B, T, E, N,
                                workspace, workspace_bytes, stream) -> None:
    _check(load_library().hymba_kernel_selective_scan(dtype, u, dt, ld, bc, ld_bc, A, D, dt_bias, h0, y, ldy,
                                                      h_out, B, T, E, N, workspace, workspace_bytes, stream))


def hymba_kernel_epilogue(dtype, ao, ld_ao, y, ld_y, z, ld_z, beta1, beta2, f, ld_f, rows, E, eps,
                          stream) -> None:
    _check(load_library().hymba_kernel_epilogue(dtype, ao, ld_ao, y, ld_y, z, ld_z, beta1, beta2, f, ld_f,
                                                rows, E, eps, stream))


def hymba_kernel_gemm_rows(w_dtype, x_dtype, y_dtype, w, ldw, x, ldx, y, ldy, y32, ldy32, c0, c1, M, N, K,
                           workspace, workspace_bytes, stream) -> None:
    _check(load_library().hymba_kernel_gemm_rows(w_dtype, x_dtype, y_dtype, w, ldw, x, ldx, y, ldy, y32, ldy32,
                                                 c0, c1, M, N, K, workspace, workspace_bytes, stream))


def hymba_kernel_gemm_tiles(in_dtype, y_dtype, w, ldw, x, ldx, y, ldy, y32, ldy32, c0, c1, M, N, K,
                            stream) -> None:
    _check(load_library().hymba_kernel_gemm_tiles(in_dtype, y_dtype, w, ldw, x, ldx, y, ldy, y32, ldy32, c0, c1,
                                                  M, N, K, stream))


def hymba_layer_set_gemm(layer: int, backend: int) -> None:
    _check(load_library().hymba_layer_set_gemm(layer, backend))


def hymba_kernel_gemm_rows_workspace(M: int, N: int, K: int) -> int:
    return load_library().hymba_kernel_gemm_rows_workspace(M, N, K)


def hymba_kernel_selective_scan_workspace(B: int, T: int, E: int, N: int) -> int:
    return load_library().hymba_kernel_selective_scan_workspace(B, T, E, N)


def hymba_layer_check(layer: int, stream: int) -> None:
    _check(load_library().hymba_layer_check(layer, stream))


def hymba_layer_set_overlap(layer: int, enable: bool) -> None:
    _check(load_library().hymba_layer_set_overlap(layer, 1 if enable else 0))


def hymba_layer_profile(layer: int, enable: bool) -> None:
    _check(load_library().hymba_layer_profile(layer, 1 if enable else 0))


def hymba_layer_profile_read(layer: int):
    """Mean per-call milliseconds of each stage over the calls recorded since profiling was enabled
    (list of HYMBA_N_STAGES floats)."""
    buf = (c_float * HYMBA_N_STAGES)()
    _check(load_library().hymba_layer_profile_read(layer, buf, HYMBA_N_STAGES))
    return [float(x) for x in buf]


def hymba_stage_name(stage: int) -> str:
    return load_library().hymba_stage_name(stage).decode()


def griffin_block_persistent_bytes(cfg: griffin_block_cfg) -> int:
    return load_library().griffin_block_persistent_bytes(ctypes.byref(cfg))


def griffin_block_prepare(cfg: griffin_block_cfg, weights: griffin_block_weights, persistent, persistent_bytes: int,
                          stream) -> None:
    _check(load_library().griffin_block_prepare(ctypes.byref(cfg), ctypes.byref(weights), persistent,
                                                persistent_bytes, stream))


def griffin_workspace_bytes(cfg: griffin_block_cfg, batch: int, seq: int) -> int:
    return load_library().griffin_workspace_bytes(ctypes.byref(cfg), batch, seq)


def griffin_block_prefill(cfg: griffin_block_cfg, weights: griffin_block_weights, persistent, x: int, B: int, T: int,
                          y: int, conv_state, h, conv_state_out, h_out, workspace: int, workspace_bytes: int,
                          stream, timed: bool = False):
    """With timed=True the call returns the milliseconds of each of GRIFFIN_STAGES (and waits for the work)."""
    ms = (c_float * GRIFFIN_N_STAGES)() if timed else None
    _check(load_library().griffin_block_prefill(ctypes.byref(cfg), ctypes.byref(weights), persistent, x, B, T, y,
                                                conv_state, h, conv_state_out, h_out, workspace, workspace_bytes,
                                                stream, ms))
    return [float(v) for v in ms] if timed else None


def griffin_block_decode(cfg: griffin_block_cfg, weights: griffin_block_weights, persistent, x_t: int, B: int,
                         y_t: int, conv_state: int, h: int, workspace: int, workspace_bytes: int, stream) -> None:
    _check(load_library().griffin_block_decode(ctypes.byref(cfg), ctypes.byref(weights), persistent, x_t, B, y_t,
                                               conv_state, h, workspace, workspace_bytes, stream))
