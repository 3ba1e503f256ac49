"""ctypes wrapper of the CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path. It shares no code with the HIP library;
the seeded input generator is the only module both consume.
"""
from __future__ import annotations

import concurrent.futures
import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

BF16, F16, F32 = 1, 2, 3


def build() -> str:
    """Compile the oracle with plain IEEE semantics (no contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
           "-Wall", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "latent", "n_experts", "n_group", "topk_group", "top_k",
        "expert_inter", "shared_inter", "group_size", "act_dtype", "router_dtype",
        "has_bias", "norm_topk")] + [("routed_scaling", ctypes.c_float), ("quant_bits", ctypes.c_int32)]


_P = ctypes.c_void_p


class _Weights(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "gate_w16", "gate_w32", "corr_bias", "fc1_w", "fc2_w", "up_q", "up_s", "up_b",
        "dn_q", "dn_s", "dn_b", "sh_up", "sh_dn")]


class _Stages(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("z", "s", "u", "a", "y", "c", "m", "sh")]


_lib = None

# MOE_ORACLE_LIB names another build of moe_oracle.c to load instead of the default one
# (the planted-control tests point it at deliberately altered copies).
_OVERRIDE_ENV = "MOE_ORACLE_LIB"


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get(_OVERRIDE_ENV)
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        _lib = ctypes.CDLL(path)
        f = _lib
        f.oracle_bf16_to_f32.restype = ctypes.c_float
        f.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        f.oracle_f32_to_bf16.restype = ctypes.c_uint16
        f.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        f.oracle_f16_to_f32.restype = ctypes.c_float
        f.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        f.oracle_f32_to_f16.restype = ctypes.c_uint16
        f.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        f.oracle_sigmoid.restype = ctypes.c_float
        f.oracle_sigmoid.argtypes = [ctypes.c_float]
        f.oracle_gate_c64.restype = ctypes.c_float
        f.oracle_gate_c64.argtypes = [_P, _P, ctypes.c_int]
        f.oracle_dequant.restype = ctypes.c_float
        f.oracle_dequant.argtypes = [ctypes.c_uint32, ctypes.c_uint16, ctypes.c_uint16]
        f.oracle_route.restype = ctypes.c_int
        f.oracle_route.argtypes = [ctypes.POINTER(_Cfg), _P, _P, _P, _P, _P]
        f.oracle_dense.restype = None
        f.oracle_dense.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, _P]
        f.oracle_q4_matvec.restype = None
        f.oracle_q4_matvec.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]
        f.oracle_qb_matvec.restype = None
        f.oracle_qb_matvec.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]
        f.oracle_code.restype = ctypes.c_uint32
        f.oracle_code.argtypes = [_P, ctypes.c_int, ctypes.c_int]
        f.oracle_combine.restype = None
        f.oracle_combine.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, _P]
        f.oracle_forward_row.restype = ctypes.c_int
        f.oracle_forward_row.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Weights), _P, _P, _P,
                                         _P, _P, ctypes.POINTER(_Stages)]
        for n in ("oracle_sigmoid_n", "oracle_f32_to_bf16_n", "oracle_f32_to_f16_n",
                  "oracle_f16_to_f32_n"):
            getattr(f, n).restype = None
            getattr(f, n).argtypes = [_P, _P, ctypes.c_long]
        f.oracle_stage.restype = ctypes.c_int
        f.oracle_stage.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Weights), ctypes.c_int,
                                   ctypes.c_int, _P, _P, _P, _P, _P]
        f.oracle_gate_c64_rows.restype = None
        f.oracle_gate_c64_rows.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def make_cfg(dims) -> _Cfg:
    return _Cfg(dims.hidden, dims.latent, dims.n_experts, dims.n_group, dims.topk_group,
                dims.top_k, dims.expert_inter, dims.shared_inter, dims.group_size,
                dims.act_dtype, dims.router_dtype, int(dims.has_bias), int(dims.norm_topk),
                float(dims.routed_scaling), int(getattr(dims, "quant_bits", 4)))


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


class _Bound:
    """Keeps the contiguous arrays alive while the C structs point at them."""

    def __init__(self, dims, arrays: Dict[str, np.ndarray]):
        self.cfg = make_cfg(dims)
        g = arrays["gate_w"]
        self.keep = {
            "gate_w16": _c(g, np.uint16) if dims.router_dtype != F32 else None,
            "gate_w32": _c(g, np.float32) if dims.router_dtype == F32 else None,
            "corr_bias": _c(arrays.get("corr_bias"), np.float32),
            "fc1_w": _c(arrays.get("fc1_w"), np.uint16),
            "fc2_w": _c(arrays.get("fc2_w"), np.uint16),
            "up_q": _c(arrays["up_q"], np.uint32),
            "up_s": _c(arrays["up_scales"], np.uint16),
            "up_b": _c(arrays["up_biases"], np.uint16),
            "dn_q": _c(arrays["down_q"], np.uint32),
            "dn_s": _c(arrays["down_scales"], np.uint16),
            "dn_b": _c(arrays["down_biases"], np.uint16),
            "sh_up": _c(arrays.get("shared_up"), np.uint16),
            "sh_dn": _c(arrays.get("shared_down"), np.uint16),
        }
        self.w = _Weights(**{k: _ptr(v) for k, v in self.keep.items()})


def forward(dims, arrays: Dict[str, np.ndarray], x: Optional[np.ndarray] = None,
            rows: Optional[list] = None, stages: bool = False, threads: int = 1) -> Dict[str, np.ndarray]:
    """Run the layer on the rows of x (default arrays['x']); `rows` picks a subset of row
    indices (rows are independent). Returns out (bits), out_f32, idx, w and, when
    `stages`, the per-row intermediates z, s, u, a, y, c, m, sh as float32 arrays.
    threads > 1 runs the rows on that many threads (each row is one call into the C
    oracle, which holds no shared state; ctypes releases the interpreter lock)."""
    L = lib()
    b = _Bound(dims, arrays)
    x = arrays["x"] if x is None else x
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sel = list(range(x.shape[0])) if rows is None else list(rows)
    H, E, K, I = dims.hidden, dims.n_experts, dims.top_k, dims.expert_inter
    D = dims.latent or dims.hidden
    n = len(sel)
    res = {"out": np.zeros((n, H), np.uint16), "out_f32": np.zeros((n, H), np.float32),
           "idx": np.zeros((n, K), np.int32), "w": np.zeros((n, K), np.float32)}
    shapes = {"z": E, "s": E, "u": D, "a": K * I, "y": K * D, "c": D, "m": H, "sh": H}
    if stages:
        for k, sz in shapes.items():
            res[k] = np.zeros((n, sz), np.float32)
    def one(i, r):
        st = None
        if stages:
            st = _Stages(**{k: _ptr(res[k][i]) for k in shapes})
        rc = L.oracle_forward_row(ctypes.byref(b.cfg), ctypes.byref(b.w), _ptr(x[r]),
                                  _ptr(res["out"][i]), _ptr(res["out_f32"][i]),
                                  _ptr(res["idx"][i]), _ptr(res["w"][i]),
                                  ctypes.byref(st) if st is not None else None)
        if rc:
            raise ValueError(f"oracle_forward_row failed: {rc}")

    if threads > 1 and n > 1:
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(threads, n)) as ex:
            for f in [ex.submit(one, i, r) for i, r in enumerate(sel)]:
                f.result()
    else:
        for i, r in enumerate(sel):
            one(i, r)
    if stages:
        res["a"] = res["a"].reshape(n, K, I)
        res["y"] = res["y"].reshape(n, K, D)
    return res


STAGES = {"latent": 2, "expert_act": 3, "expert_out": 4, "shared_act": 6, "shared_out": 7,
          "fc2": 8, "final": 9}


def stage(dims, arrays: Dict[str, np.ndarray], name: str, inp: np.ndarray, expert: int = 0,
          in2: Optional[np.ndarray] = None, in3: Optional[np.ndarray] = None):
    """One stage of one row from its own input (fp32 values). Returns (rounded values as
    fp32, fp32 value before the last rounding)."""
    L = lib()
    b = _Bound(dims, arrays)
    D = dims.latent or dims.hidden
    n = {"latent": dims.latent, "expert_act": dims.expert_inter, "expert_out": D,
         "shared_act": dims.shared_inter, "shared_out": dims.hidden, "fc2": dims.hidden,
         "final": dims.hidden}[name]
    inp = np.ascontiguousarray(inp, np.float32)
    in2 = _c(in2, np.float32)
    in3 = _c(in3, np.float32)
    out = np.zeros(n, np.float32)
    pre = np.zeros(n, np.float32)
    rc = L.oracle_stage(ctypes.byref(b.cfg), ctypes.byref(b.w), STAGES[name], int(expert), _ptr(inp),
                        _ptr(in2), _ptr(in3), _ptr(out), _ptr(pre))
    if rc:
        raise ValueError(f"oracle_stage {name} failed: {rc}")
    return out, pre


def route(dims, z: np.ndarray, bias: Optional[np.ndarray]):
    """Route one row of fp32 logits z [E]. Returns (idx [k], w [k], s [E])."""
    L = lib()
    cfg = make_cfg(dims)
    z = np.ascontiguousarray(z, np.float32)
    bias = _c(bias, np.float32)
    idx = np.zeros(dims.top_k, np.int32)
    w = np.zeros(dims.top_k, np.float32)
    s = np.zeros(dims.n_experts, np.float32)
    rc = L.oracle_route(ctypes.byref(cfg), _ptr(z), _ptr(bias), _ptr(idx), _ptr(w), _ptr(s))
    if rc:
        raise ValueError(f"oracle_route failed: {rc}")
    return idx, w, s


def gate_c64(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """C64 gate sums: x [rows][H] fp32 values, w [E][H] fp32 values -> [rows][E] fp32."""
    x = np.ascontiguousarray(np.atleast_2d(x), np.float32)
    w = np.ascontiguousarray(np.atleast_2d(w), np.float32)
    z = np.zeros((x.shape[0], w.shape[0]), np.float32)
    lib().oracle_gate_c64_rows(_ptr(x), _ptr(w), x.shape[0], w.shape[0], x.shape[1], _ptr(z))
    return z


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, np.float32)
    s = np.empty_like(z)
    lib().oracle_sigmoid_n(_ptr(z), _ptr(s), z.size)
    return s


def dense(W_bits: np.ndarray, x: np.ndarray) -> np.ndarray:
    """fp32 W . x for a bf16 matrix [N][K] and fp32 values x [K]."""
    W_bits = np.ascontiguousarray(W_bits, np.uint16)
    x = np.ascontiguousarray(x, np.float32)
    out = np.zeros(W_bits.shape[0], np.float32)
    lib().oracle_dense(_ptr(W_bits), _ptr(x), W_bits.shape[0], W_bits.shape[1], _ptr(out))
    return out


def q4_matvec(Q, S, B, x, group_size=64) -> np.ndarray:
    """fp32 U . x for one 4-bit affine matrix: Q [N][K/8] u32, S, B [N][K/gs] bf16."""
    Q = np.ascontiguousarray(Q, np.uint32)
    S = np.ascontiguousarray(S, np.uint16)
    B = np.ascontiguousarray(B, np.uint16)
    x = np.ascontiguousarray(x, np.float32)
    N, K = Q.shape[0], Q.shape[1] * 8
    out = np.zeros(N, np.float32)
    lib().oracle_q4_matvec(_ptr(Q), _ptr(S), _ptr(B), _ptr(x), N, K, group_size, _ptr(out))
    return out


def qb_matvec(Q, S, B, x, bits, group_size=64) -> np.ndarray:
    """fp32 U . x for one b-bit affine matrix: Q [N][K b / 32] u32, S, B [N][K/gs] bf16."""
    Q = np.ascontiguousarray(Q, np.uint32)
    S = np.ascontiguousarray(S, np.uint16)
    B = np.ascontiguousarray(B, np.uint16)
    x = np.ascontiguousarray(x, np.float32)
    N, K = Q.shape[0], x.shape[0]
    assert Q.shape[1] * 32 == K * bits
    out = np.zeros(N, np.float32)
    lib().oracle_qb_matvec(_ptr(Q), _ptr(S), _ptr(B), _ptr(x), N, K, group_size, bits, _ptr(out))
    return out


def code(qrow, k: int, bits: int) -> int:
    qrow = np.ascontiguousarray(qrow, np.uint32)
    return int(lib().oracle_code(_ptr(qrow), k, bits))


def combine(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """fp32 combine (before rounding): y [k][D] fp32 values, w [k] fp32 -> [D]."""
    y = np.ascontiguousarray(y, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    out = np.zeros(y.shape[1], np.float32)
    lib().oracle_combine(_ptr(y), _ptr(w), y.shape[0], y.shape[1], _ptr(out))
    return out


def dequant(q: int, scale_bits: int, bias_bits: int) -> float:
    return lib().oracle_dequant(q, scale_bits, bias_bits)


def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    h = np.empty(v.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(_ptr(v), _ptr(h), v.size)
    return h


def f32_to_f16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    h = np.empty(v.shape, np.uint16)
    lib().oracle_f32_to_f16_n(_ptr(v), _ptr(h), v.size)
    return h


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16)
    v = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_n(_ptr(h), _ptr(v), h.size)
    return v


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def act_to_f32(dims, h: np.ndarray) -> np.ndarray:
    return f16_to_f32(h) if dims.act_dtype == F16 else bf16_to_f32(h)
