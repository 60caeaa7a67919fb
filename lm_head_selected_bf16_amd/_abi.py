"""ctypes binding of libflp.so: the C ABI of include/flp.h, name for name.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind these calls; there is no other implementation to fall back on.
If the library is missing, loading fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflp.so")

# flp_dtype
FLP_BF16, FLP_F32, FLP_I64, FLP_I32, FLP_F16 = 0, 1, 2, 3, 4
# flp_status
STATUS_NAMES = {
    0: "FLP_OK",
    1: "FLP_INVALID_ARGUMENT",
    2: "FLP_UNSUPPORTED_DTYPE",
    3: "FLP_UNSUPPORTED_SHAPE",
    4: "FLP_MISALIGNED",
    5: "FLP_WORKSPACE_TOO_SMALL",
    6: "FLP_UNSUPPORTED_DEVICE",
    7: "FLP_HIP_ERROR",
}
FLP_OK = 0

# Every symbol include/flp.h declares, with (restype, argtypes).
_i64, _sz, _vp, _fp, _int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "flp_forward_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "flp_forward": (_int, [_i64, _i64, _i64, _int, _vp, _vp, _fp, _vp, _int, _fp, _fp, _fp, _vp,
                           _sz, _vp]),
    "flp_forward_noalloc": (_int, [_i64, _i64, _i64, _int, _vp, _vp, _fp, _vp, _int, _fp, _fp, _fp,
                                   _vp]),
    "flp_forward_partial_bytes": (_sz, [_i64, _i64]),
    "flp_forward_partial": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _fp, _vp, _int, _fp,
                                   _vp, _fp, _vp]),
    "flp_merge": (_int, [_i64, _i64, _vp, _fp, _vp, _int, _fp, _fp, _vp]),
    "flp_logits_forward": (_int, [_i64, _i64, _int, _vp, _vp, _int, _fp, _fp, _vp]),
    "flp_logits_backward": (_int, [_i64, _i64, _int, _fp, _fp, _vp, _vp, _int, _vp, _vp]),
    "flp_backward_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int, _i64]),
    "flp_backward_chunk_rows": (_i64, [_i64, _i64, _i64, _int, _int, _sz, _int, _int, _int]),
    "flp_backward": (_int, [_i64, _i64, _i64, _int, _fp, _fp, _vp, _vp, _fp, _vp, _int, _fp, _vp,
                            _vp, _int, _fp, _vp, _sz, _vp]),
    "flp_forward_indexed_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _i64]),
    "flp_forward_indexed": (_int, [_i64, _i64, _i64, _int, _vp, _vp, _fp, _vp, _int, _fp, _vp, _int,
                                   _i64, _fp, _fp, _vp, _sz, _vp]),
    "flp_backward_indexed_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int, _i64, _i64]),
    "flp_backward_indexed": (_int, [_i64, _i64, _i64, _int, _fp, _fp, _vp, _vp, _fp, _vp, _int, _fp,
                                    _vp, _int, _i64, _vp, _vp, _int, _fp, _vp, _sz, _vp]),
    "flp_logits_indexed_workspace_bytes": (_sz, [_i64]),
    "flp_logits_forward_indexed": (_int, [_i64, _i64, _int, _vp, _vp, _int, _vp, _int, _i64, _fp,
                                          _fp, _vp, _sz, _vp]),
    "flp_logits_backward_indexed": (_int, [_i64, _i64, _int, _fp, _fp, _vp, _vp, _int, _vp, _int,
                                           _i64, _vp, _vp, _sz, _vp]),
    "flp_embedding_forward": (_int, [_i64, _i64, _i64, _int, _vp, _vp, _int, _vp, _vp]),
    "flp_embedding_backward_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "flp_embedding_backward": (_int, [_i64, _i64, _i64, _int, _vp, _vp, _int, _vp, _int, _vp, _sz,
                                      _vp]),
    "flp_probe_scratch_bytes": (_sz, []),
    "flp_probe_mfma": (_int, [_int, _i64, _vp, _sz, ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(ctypes.c_double), _vp]),
    "flp_probe_read": (_int, [_vp, _sz, _vp, _sz, ctypes.POINTER(ctypes.c_double), _vp]),
    "flp_profile_enable": (None, [_int]),
    "flp_profile_read": (_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), _int]),
    "flp_status_string": (ctypes.c_char_p, [_int]),
    "flp_build_info": (ctypes.c_char_p, []),
}

_lock = threading.Lock()
_lib = None


class FlpError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load libflp.so from the package directory (raises if it was not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m lm_head_selected_bf16_amd.build` "
                    "(hipcc, gfx950).  There is no other implementation of this operator.")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    try:
        return load().flp_status_string(int(status)).decode()
    except ImportError:
        return STATUS_NAMES.get(int(status), f"status {status}")


def flp_forward_workspace_bytes(N: int, D: int, V: int) -> int:
    return int(load().flp_forward_workspace_bytes(N, D, V))


# Size of the allocation-free forward's fixed per-device scratch array (FLP_FORWARD_NOALLOC_MAX_BYTES).
FLP_FORWARD_NOALLOC_MAX_BYTES = 33 << 20


def flp_forward_noalloc(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype, temperature,
                        out_logp, out_lse, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_forward_noalloc(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype,
                                          temperature, out_logp, out_lse, stream))


def flp_forward_partial_bytes(N: int, V_local: int) -> int:
    return int(load().flp_forward_partial_bytes(N, V_local))


def flp_forward_partial(N, D, V_local, vocab_start, V_total, x_dtype, hidden, weight, bias, targets,
                        t_dtype, temperature, partial, zt, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_forward_partial(N, D, V_local, vocab_start, V_total, x_dtype, hidden,
                                          weight, bias, targets, t_dtype, temperature, partial,
                                          zt, stream))


def flp_merge(N, V_total, partials, zt, targets, t_dtype, out_logp, out_lse, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_merge(N, V_total, partials, zt, targets, t_dtype, out_logp, out_lse,
                                stream))


def flp_logits_forward(N, V, x_dtype, logits, targets, t_dtype, out_logp, out_lse, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_logits_forward(N, V, x_dtype, logits, targets, t_dtype, out_logp,
                                         out_lse, stream))


def flp_logits_backward(N, V, x_dtype, grad_out, lse, logits, targets, t_dtype, d_logits,
                        stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_logits_backward(N, V, x_dtype, grad_out, lse, logits, targets, t_dtype,
                                          d_logits, stream))


def flp_backward_workspace_bytes(N: int, D: int, V: int, x_dtype: int, dw_dtype: int,
                                 chunk_rows: int = 0) -> int:
    return int(load().flp_backward_workspace_bytes(N, D, V, x_dtype, dw_dtype, chunk_rows))


def flp_backward_chunk_rows(N: int, D: int, V: int, x_dtype: int, dw_dtype: int,
                            workspace_bytes: int, need_d_hidden: bool = True,
                            need_d_weight: bool = True, need_d_bias: bool = True) -> int:
    return int(load().flp_backward_chunk_rows(N, D, V, x_dtype, dw_dtype, workspace_bytes,
                                              int(need_d_hidden), int(need_d_weight),
                                              int(need_d_bias)))


def flp_forward(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype, temperature,
                out_logp, out_lse, workspace, workspace_bytes, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_forward(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype,
                                  temperature, out_logp, out_lse, workspace, workspace_bytes, stream))


def flp_backward(N, D, V, x_dtype, grad_out, lse, hidden, weight, bias, targets, t_dtype,
                 temperature, d_hidden, d_weight, dw_dtype, d_bias, workspace, workspace_bytes,
                 stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_backward(N, D, V, x_dtype, grad_out, lse, hidden, weight, bias, targets,
                                   t_dtype, temperature, d_hidden, d_weight, dw_dtype, d_bias,
                                   workspace, workspace_bytes, stream))


def flp_forward_indexed_workspace_bytes(N: int, D: int, V: int, x_dtype: int, n_rows: int) -> int:
    return int(load().flp_forward_indexed_workspace_bytes(N, D, V, x_dtype, n_rows))


def flp_forward_indexed(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype, temperature,
                        rows, r_dtype, n_rows, out_logp, out_lse, workspace, workspace_bytes,
                        stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_forward_indexed(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype,
                                          temperature, rows, r_dtype, n_rows, out_logp, out_lse,
                                          workspace, workspace_bytes, stream))


def flp_backward_indexed_workspace_bytes(N: int, D: int, V: int, x_dtype: int, dw_dtype: int,
                                         n_rows: int, chunk_rows: int = 0) -> int:
    return int(load().flp_backward_indexed_workspace_bytes(N, D, V, x_dtype, dw_dtype, n_rows,
                                                           chunk_rows))


def flp_backward_indexed(N, D, V, x_dtype, grad_out, lse, hidden, weight, bias, targets, t_dtype,
                         temperature, rows, r_dtype, n_rows, d_hidden, d_weight, dw_dtype, d_bias,
                         workspace, workspace_bytes, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_backward_indexed(N, D, V, x_dtype, grad_out, lse, hidden, weight, bias,
                                           targets, t_dtype, temperature, rows, r_dtype, n_rows,
                                           d_hidden, d_weight, dw_dtype, d_bias, workspace,
                                           workspace_bytes, stream))


def flp_logits_indexed_workspace_bytes(N: int) -> int:
    return int(load().flp_logits_indexed_workspace_bytes(N))


def flp_logits_forward_indexed(N, V, x_dtype, logits, targets, t_dtype, rows, r_dtype, n_rows,
                               out_logp, out_lse, workspace, workspace_bytes, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_logits_forward_indexed(N, V, x_dtype, logits, targets, t_dtype, rows,
                                                 r_dtype, n_rows, out_logp, out_lse, workspace,
                                                 workspace_bytes, stream))


def flp_logits_backward_indexed(N, V, x_dtype, grad_out, lse, logits, targets, t_dtype, rows,
                                r_dtype, n_rows, d_logits, workspace, workspace_bytes,
                                stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_logits_backward_indexed(N, V, x_dtype, grad_out, lse, logits, targets,
                                                  t_dtype, rows, r_dtype, n_rows, d_logits,
                                                  workspace, workspace_bytes, stream))


def flp_embedding_forward(N, D, V, x_dtype, weight, ids, id_dtype, out, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_embedding_forward(N, D, V, x_dtype, weight, ids, id_dtype, out, stream))


def flp_embedding_backward_workspace_bytes(N: int, D: int, V: int) -> int:
    return int(load().flp_embedding_backward_workspace_bytes(N, D, V))


def flp_embedding_backward(N, D, V, x_dtype, grad, ids, id_dtype, d_weight, dw_dtype, workspace,
                           workspace_bytes, stream) -> int:
    """Raw call: every pointer argument is an int address (0 for NULL)."""
    return int(load().flp_embedding_backward(N, D, V, x_dtype, grad, ids, id_dtype, d_weight,
                                             dw_dtype, workspace, workspace_bytes, stream))


def flp_probe_scratch_bytes() -> int:
    return int(load().flp_probe_scratch_bytes())


def flp_probe_mfma(zero_operands: bool, iters: int, scratch: int, scratch_bytes: int, stream: int):
    """(status, TFLOP/s, shader clock GHz) of the dense MFMA probe (synchronises the stream)."""
    tf, ghz = ctypes.c_double(0.0), ctypes.c_double(0.0)
    st = int(load().flp_probe_mfma(int(bool(zero_operands)), iters, scratch, scratch_bytes,
                                   ctypes.byref(tf), ctypes.byref(ghz), stream))
    return st, tf.value, ghz.value


def flp_probe_read(buffer: int, nbytes: int, scratch: int, scratch_bytes: int, stream: int):
    """(status, GB/s) of the streaming-read probe (synchronises the stream)."""
    gbs = ctypes.c_double(0.0)
    st = int(load().flp_probe_read(buffer, nbytes, scratch, scratch_bytes, ctypes.byref(gbs), stream))
    return st, gbs.value


KERNEL_KINDS = ("forward", "merge", "dlogits", "transpose", "d_hidden", "d_weight", "d_bias",
                "logits_forward", "logits_backward", "rows", "embedding")


def flp_profile_enable(on: bool) -> None:
    load().flp_profile_enable(1 if on else 0)


def flp_profile_read() -> dict:
    """{kind: (total_ms, launches)} since the previous read."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    st = int(load().flp_profile_read(ms, cnt, n))
    if st != FLP_OK:
        raise FlpError("flp_profile_read", st)
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_KINDS)}


def flp_status_string(status: int) -> str:
    return load().flp_status_string(int(status)).decode()


def flp_build_info() -> str:
    return load().flp_build_info().decode()
