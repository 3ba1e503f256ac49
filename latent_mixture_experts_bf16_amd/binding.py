"""ctypes binding of libmoe_latent.so (the C ABI in include/moe_latent.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of the
library. The functions carry the C names. Device buffers are passed as integer device
addresses (e.g. a torch tensor's data_ptr()); streams as integer hipStream_t handles.
If the library has not been built this module raises at import -- there is no fallback.

torch (when installed) is imported before the library is loaded, so that the library binds
to the HIP runtime torch brings: a process must drive the GPU through one HIP runtime.
"""
from __future__ import annotations

import ctypes
import os

try:  # load torch's HIP runtime first (see above)
    import torch  # noqa: F401
except ImportError:  # pragma: no cover
    pass

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LATENT_LIB names another build of the same sources to load instead (the CPU sanitizer
# tests point it at a host-only build instrumented with AddressSanitizer and UBSan).
LIB_PATH = os.environ.get("MOE_LATENT_LIB") or os.path.join(_PKG, "libmoe_latent.so")

# enum values of include/moe_latent.h
MOE_DT_BF16, MOE_DT_F16, MOE_DT_F32, MOE_DT_U32, MOE_DT_I32 = 1, 2, 3, 4, 5
MOE_ACT_RELU2 = 1
STATUS = {
    0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_TOPK_GT_EXPERTS", 3: "MOE_ERR_GROUPS",
    4: "MOE_ERR_SHAPE", 5: "MOE_ERR_MISSING_TENSOR", 6: "MOE_ERR_DTYPE", 7: "MOE_ERR_LAYOUT",
    8: "MOE_ERR_EXPERTS_OVER_HIDDEN", 9: "MOE_ERR_DEVICE", 10: "MOE_ERR_ROWS", 11: "MOE_ERR_ALIAS",
    12: "MOE_ERR_HIP", 13: "MOE_ERR_OOM", 14: "MOE_ERR_DEVICE_CHECK",
}
STAGE = {"logits": 1, "latent": 2, "expert_act": 3, "expert_out": 4, "combine": 5,
         "shared_act": 6, "shared_out": 7}


class moe_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class moe_latent_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "latent", "n_experts", "n_group", "topk_group", "top_k", "expert_inter",
        "shared_inter", "group_size", "act_dtype", "router_dtype", "activation", "has_bias",
        "norm_topk", "max_rows")] + [("routed_scaling", ctypes.c_float), ("quant_bits", ctypes.c_int32)]


WEIGHT_FIELDS = ("gate_w", "corr_bias", "fc1_w", "fc2_w", "up_q", "up_scales", "up_biases",
                 "down_q", "down_scales", "down_biases", "shared_up", "shared_down")


class moe_latent_weights(ctypes.Structure):
    _fields_ = [(n, moe_tensor) for n in WEIGHT_FIELDS]


class MoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code
        self.name = STATUS.get(code, str(code))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sig = {
        "moe_latent_create": (ctypes.c_int, [ctypes.POINTER(moe_latent_config),
                                             ctypes.POINTER(moe_latent_weights), P,
                                             ctypes.POINTER(P)]),
        "moe_latent_forward": (ctypes.c_int, [P, ctypes.c_int32, P, P]),
        "moe_latent_prefill": (ctypes.c_int, [P, ctypes.c_int32, P, P]),
        "moe_latent_destroy": (None, [P]),
        "moe_latent_set_stream": (ctypes.c_int, [P, P]),
        "moe_latent_set_variant": (ctypes.c_int, [P, ctypes.c_int32]),
        "moe_latent_get_routing": (ctypes.c_int, [P, P, P]),
        "moe_latent_read_stage": (ctypes.c_int, [P, ctypes.c_int32, P, ctypes.c_size_t]),
        "moe_latent_status": (ctypes.c_int, [P]),
        "moe_latent_last_error": (ctypes.c_char_p, []),
        "moe_latent_live_allocations": (ctypes.c_int32, []),
        "moe_latent_launch_group": (ctypes.c_int, [P, ctypes.c_int32, P, P, ctypes.c_int32]),
        "moe_latent_group_items": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32]),
        "moe_latent_group_stages": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32, P, P, P]),
        "moe_latent_group_kernel": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_char_p,
                                                   ctypes.c_int32]),
        "moe_latent_forward_timed": (ctypes.c_int, [P, ctypes.c_int32, P, P, ctypes.POINTER(P), ctypes.c_int32]),
        "moe_latent_stream_read": (ctypes.c_int, [P, ctypes.c_size_t, P, P]),
        "moe_lm_head_gemv": (ctypes.c_int, [ctypes.POINTER(moe_tensor), ctypes.c_int32, P, P, ctypes.c_int32, P]),
        "moe_latent_forward_static": (ctypes.c_int, [ctypes.POINTER(moe_latent_config),
                                                     ctypes.POINTER(moe_latent_weights), ctypes.c_int32,
                                                     P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("moe_latent_create", "moe_latent_forward", "moe_latent_destroy", "moe_latent_set_stream",
            "moe_latent_set_variant", "moe_latent_get_routing", "moe_latent_read_stage",
            "moe_latent_status", "moe_latent_last_error", "moe_latent_live_allocations",
            "moe_latent_launch_group", "moe_latent_group_items", "moe_latent_forward_timed",
            "moe_latent_stream_read", "moe_latent_forward_static", "moe_latent_group_stages",
            "moe_lm_head_gemv", "moe_latent_prefill", "moe_latent_group_kernel")


def lib():
    return _lib


def moe_latent_last_error() -> str:
    return _lib.moe_latent_last_error().decode()


def _check(rc: int):
    if rc:
        raise MoeError(rc, moe_latent_last_error())


def make_tensor(ptr: int, dtype: int, shape, strides=None) -> moe_tensor:
    t = moe_tensor()
    t.data = ptr or None
    t.dtype = dtype
    t.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for d in reversed(shape):
            strides.insert(0, acc)
            acc *= d
    for i, (d, s) in enumerate(zip(shape, strides)):
        t.shape[i] = d
        t.stride[i] = s
    return t


def moe_latent_create(cfg: moe_latent_config, weights: moe_latent_weights, stream: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(_lib.moe_latent_create(ctypes.byref(cfg), ctypes.byref(weights), stream or None,
                                  ctypes.byref(h)))
    return h.value


def moe_latent_create_rc(cfg: moe_latent_config, weights: moe_latent_weights, stream: int = 0):
    """Like moe_latent_create but returns (status, handle or None) without raising."""
    h = ctypes.c_void_p()
    rc = _lib.moe_latent_create(ctypes.byref(cfg), ctypes.byref(weights), stream or None,
                                ctypes.byref(h))
    return rc, h.value


def moe_latent_forward(h: int, rows: int, hidden_in: int, out: int) -> None:
    _check(_lib.moe_latent_forward(h, rows, hidden_in, out))


def moe_latent_forward_rc(h: int, rows: int, hidden_in: int, out: int) -> int:
    return _lib.moe_latent_forward(h, rows, hidden_in, out)


def moe_latent_prefill(h: int, rows: int, hidden_in: int, out: int) -> None:
    _check(_lib.moe_latent_prefill(h, rows, hidden_in, out))


def moe_latent_prefill_rc(h: int, rows: int, hidden_in: int, out: int) -> int:
    return _lib.moe_latent_prefill(h, rows, hidden_in, out)


def moe_latent_destroy(h: int) -> None:
    _lib.moe_latent_destroy(h)


def moe_latent_set_stream(h: int, stream: int) -> None:
    _check(_lib.moe_latent_set_stream(h, stream or None))


def moe_latent_set_variant(h: int, variant: int) -> None:
    _check(_lib.moe_latent_set_variant(h, variant))


def moe_latent_get_routing(h: int, idx_dev: int, w_dev: int) -> None:
    _check(_lib.moe_latent_get_routing(h, idx_dev, w_dev))


def moe_latent_read_stage(h: int, stage: int, dst_dev: int, nbytes: int) -> None:
    _check(_lib.moe_latent_read_stage(h, stage, dst_dev, nbytes))


def moe_latent_status(h: int) -> None:
    _check(_lib.moe_latent_status(h))


def moe_latent_live_allocations() -> int:
    return _lib.moe_latent_live_allocations()


def moe_latent_launch_group(h: int, rows: int, hidden_in: int, out: int, group: int) -> None:
    _check(_lib.moe_latent_launch_group(h, rows, hidden_in, out, group))


def moe_latent_group_items(h: int, rows: int, group: int) -> int:
    return _lib.moe_latent_group_items(h, rows, group)


def moe_latent_group_stages(h: int, rows: int, group: int):
    """(workgroups, first stage, last stage, side) of launch group `group`; workgroups <= 0
    when there is no such group."""
    f, l, sd = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    n = _lib.moe_latent_group_stages(h, rows, group, ctypes.byref(f), ctypes.byref(l), ctypes.byref(sd))
    return n, f.value, l.value, sd.value


def moe_latent_group_kernel(h: int, rows: int, group: int) -> str:
    """The kernel launch group `group` runs (its name as a profiler lists it); "" when there
    is no such group."""
    buf = ctypes.create_string_buffer(128)
    n = _lib.moe_latent_group_kernel(h, rows, group, buf, len(buf))
    if n < 0:
        raise MoeError(-1, "moe_latent_group_kernel: invalid handle or rows")
    return buf.value.decode()


def moe_latent_forward_timed(h: int, rows: int, hidden_in: int, out: int, events) -> None:
    """events: hipEvent_t handles (integers), two per launch group (start, end)."""
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(_lib.moe_latent_forward_timed(h, rows, hidden_in, out, arr, len(events)))


def moe_latent_stream_read(src: int, nbytes: int, sink_dev: int, stream: int = 0) -> None:
    _check(_lib.moe_latent_stream_read(src, nbytes, sink_dev, stream))


def moe_latent_forward_static(cfg: moe_latent_config, weights: moe_latent_weights, rows: int, hidden_in: int,
                              out: int, stream: int = 0) -> None:
    _check(_lib.moe_latent_forward_static(ctypes.byref(cfg), ctypes.byref(weights), rows, hidden_in, out,
                                          stream or None))


def moe_latent_forward_static_rc(cfg: moe_latent_config, weights: moe_latent_weights, rows: int, hidden_in: int,
                                 out: int, stream: int = 0) -> int:
    return _lib.moe_latent_forward_static(ctypes.byref(cfg), ctypes.byref(weights), rows, hidden_in, out,
                                          stream or None)


def moe_lm_head_gemv(w: moe_tensor, rows: int, x: int, out: int, out_dtype: int = MOE_DT_F32, stream: int = 0) -> None:
    _check(_lib.moe_lm_head_gemv(ctypes.byref(w), rows, x, out, out_dtype, stream or None))


def moe_lm_head_gemv_rc(w: moe_tensor, rows: int, x: int, out: int, out_dtype: int = MOE_DT_F32,
                        stream: int = 0) -> int:
    return _lib.moe_lm_head_gemv(ctypes.byref(w), rows, x, out, out_dtype, stream or None)
