"""C ABI tests that need no GPU: the library loads, exports what the header declares, and
refuses bad configurations and tensor descriptors by name before touching a device
(TensorFold pull request 1038, «What's in it»: refusals before load; review thread: each
refusal has a test, and nothing stays allocated after one)."""
import os
import re

import pytest

from latent_mixture_experts_bf16_amd import binding as B
from latent_mixture_experts_bf16_amd import layer as LY
from latent_mixture_experts_bf16_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000   # a non-NULL address; refused descriptors are never dereferenced


def _header_functions():
    with open(os.path.join(ROOT, "include", "moe_latent.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(moe_(?:latent|lm)_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = _header_functions()
    assert declared, "no declarations found"
    lib = B.lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTED) == declared


class _Cpu:
    """Tensor descriptors with fake addresses for the shapes of a LayerDims."""

    def __init__(self, dims, **over):
        self.dims = dims
        self.shapes = self._shapes(dims)
        self.over = over

    @staticmethod
    def _shapes(d):
        H, L, E, I, SI = d.hidden, d.latent, d.n_experts, d.expert_inter, d.shared_inter
        D = L or H
        b, gs = d.quant_bits, d.group_size
        s = {"gate_w": [E, H], "up_q": [E, I, D * b // 32], "up_scales": [E, I, D // gs],
             "up_biases": [E, I, D // gs], "down_q": [E, D, I * b // 32], "down_scales": [E, D, I // gs],
             "down_biases": [E, D, I // gs]}
        if d.has_bias:
            s["corr_bias"] = [E]
        if L:
            s["fc1_w"] = [L, H]
            s["fc2_w"] = [H, L]
        if SI:
            s["shared_up"] = [SI, H]
            s["shared_down"] = [H, SI]
        return s

    def weights(self):
        w = B.moe_latent_weights()
        for name, shape in self.shapes.items():
            dt = LY._DT[name] or (B.MOE_DT_F32 if self.dims.router_dtype == 3 else B.MOE_DT_BF16)
            spec = dict(ptr=FAKE, dtype=dt, shape=shape, strides=None)
            spec.update(self.over.get(name, {}))
            setattr(w, name, B.make_tensor(spec["ptr"], spec["dtype"], spec["shape"], spec["strides"]))
        return w


def _create(dims, max_rows=1, cfg_over=None, **tensor_over):
    cfg = LY.config_of(dims, max_rows)
    for k, v in (cfg_over or {}).items():
        setattr(cfg, k, v)
    before = B.moe_latent_live_allocations()
    rc, h = B.moe_latent_create_rc(cfg, _Cpu(dims, **tensor_over).weights())
    assert B.moe_latent_live_allocations() == before
    return B.STATUS[rc], h, B.moe_latent_last_error()


BOLT = synth.WORKLOADS[1].layers[0]
NONLAT = synth.WORKLOADS[3].layers[0]


@pytest.mark.parametrize("over,code,word", [
    ({"top_k": 300}, "MOE_ERR_TOPK_GT_EXPERTS", "top_k"),
    ({"n_group": 7}, "MOE_ERR_GROUPS", "n_group"),
    ({"topk_group": 9}, "MOE_ERR_GROUPS", "topk_group"),
    ({"n_group": 120, "topk_group": 1}, "MOE_ERR_GROUPS", "kept groups"),
    ({"hidden": 4000}, "MOE_ERR_SHAPE", "hidden"),
    ({"latent": 1000}, "MOE_ERR_SHAPE", "latent"),
    ({"group_size": 16}, "MOE_ERR_SHAPE", "group_size"),
    ({"group_size": 256}, "MOE_ERR_SHAPE", "group_size"),
    ({"quant_bits": 7}, "MOE_ERR_SHAPE", "quant_bits"),
    ({"quant_bits": 1}, "MOE_ERR_SHAPE", "quant_bits"),
    ({"quant_bits": 3, "expert_inter": 192}, "MOE_ERR_SHAPE", "multiples of 128"),
    ({"max_rows": 0}, "MOE_ERR_ROWS", "max_rows"),
    ({"max_rows": 4097}, "MOE_ERR_ROWS", "max_rows"),
    ({"act_dtype": B.MOE_DT_F16}, "MOE_ERR_DTYPE", "f16"),
    ({"router_dtype": B.MOE_DT_U32}, "MOE_ERR_DTYPE", "router_dtype"),
    ({"n_experts": 2048, "n_group": 8}, "MOE_ERR_SHAPE", "n_experts"),
])
def test_config_refusals(over, code, word):
    rc, h, msg = _create(BOLT, cfg_over=over)
    assert rc == code and h is None
    assert word in msg


def test_other_widths_refuse_f16_activations():
    rc, h, msg = _create(NONLAT, cfg_over={"quant_bits": 3})
    assert rc == "MOE_ERR_DTYPE" and h is None
    assert "bf16 activations" in msg


@pytest.mark.parametrize("bits,gs", [(2, 32), (3, 64), (5, 128), (8, 64), (4, 128)])
def test_other_widths_check_code_and_group_shapes(bits, gs):
    """A descriptor laid out for 4-bit codes in groups of 64 is refused by name for another
    width or group size; the shapes of the width itself pass every check before the device."""
    import dataclasses
    dims = dataclasses.replace(BOLT, quant_bits=bits, group_size=gs)
    if bits != 4:
        rc, h, msg = _create(dims, up_q={"shape": [BOLT.n_experts, BOLT.expert_inter, BOLT.latent // 8]})
        assert rc == "MOE_ERR_LAYOUT" and "up_q" in msg, msg
    if gs != 64:
        rc, h, msg = _create(dims, down_scales={"shape": [BOLT.n_experts, BOLT.latent, BOLT.expert_inter // 64]})
        assert rc == "MOE_ERR_LAYOUT" and "down_scales" in msg, msg
    rc, h, msg = _create(dims)
    assert rc in ("MOE_ERR_DEVICE", "MOE_OK"), (rc, msg)
    if h is not None:
        B.moe_latent_destroy(h)


def test_non_latent_shared_expert_refused():
    # a non-latent layer has no fc2 epilogue, where the shared output is added
    rc, h, msg = _create(NONLAT, cfg_over={"shared_inter": 512, "act_dtype": B.MOE_DT_BF16})
    assert rc == "MOE_ERR_SHAPE" and h is None
    assert "latent layer" in msg


@pytest.mark.parametrize("name,over,code,word", [
    ("fc1_w", {"ptr": 0}, "MOE_ERR_MISSING_TENSOR", "fc1_latent_proj"),
    ("fc2_w", {"ptr": 0}, "MOE_ERR_MISSING_TENSOR", "fc2_latent_proj"),
    ("fc1_w", {"dtype": B.MOE_DT_U32}, "MOE_ERR_DTYPE", "quantized"),
    ("fc2_w", {"dtype": B.MOE_DT_F16}, "MOE_ERR_DTYPE", "fc2_latent_proj"),
    ("fc1_w", {"shape": [4096, 1024]}, "MOE_ERR_LAYOUT", "transposed"),
    ("fc2_w", {"shape": [4096, 1024], "strides": [1, 4096]}, "MOE_ERR_LAYOUT", "transposed"),
    ("up_q", {"shape": [240, 2048, 512]}, "MOE_ERR_EXPERTS_OVER_HIDDEN", "over hidden"),
    ("down_q", {"shape": [240, 4096, 256]}, "MOE_ERR_EXPERTS_OVER_HIDDEN", "over hidden"),
    ("gate_w", {"dtype": B.MOE_DT_F32}, "MOE_ERR_DTYPE", "gate_w"),
    ("corr_bias", {"ptr": 0}, "MOE_ERR_MISSING_TENSOR", "corr_bias"),
    ("up_scales", {"shape": [240, 2048, 8]}, "MOE_ERR_LAYOUT", "up_scales"),
    ("shared_down", {"strides": [8192, 1]}, "MOE_ERR_LAYOUT", "shared_down"),
    ("up_q", {"ptr": FAKE + 4}, "MOE_ERR_LAYOUT", "16-byte aligned"),
    ("fc2_w", {"ptr": FAKE + 2}, "MOE_ERR_LAYOUT", "16-byte aligned"),
])
def test_tensor_refusals(name, over, code, word):
    rc, h, msg = _create(BOLT, **{name: over})
    assert rc == code and h is None, msg
    assert word in msg


def test_valid_descriptors_reach_the_device_check():
    """A valid non-latent layer (no latent or shared tensors) passes every descriptor check;
    without a GPU the last check, the device, refuses it."""
    import torch
    if torch.cuda.device_count() > 0:   # fake addresses must never reach a real create
        pytest.skip("a device is present; covered by the GPU tests")
    rc, h, msg = _create(NONLAT, max_rows=4)
    assert rc == "MOE_ERR_DEVICE" and h is None, msg


def test_null_arguments():
    assert B.lib().moe_latent_create(None, None, None, None) == 1
    assert B.lib().moe_latent_forward(None, 1, None, None) == 1
    assert B.lib().moe_latent_forward_timed(None, 1, None, None, None, 0) == 1
    # the stream reference refuses NULL, misaligned and odd sizes before touching a device
    assert B.lib().moe_latent_stream_read(None, 16, None, None) == 1
    assert B.lib().moe_latent_stream_read(8, 16, 64, None) == 1
    assert B.lib().moe_latent_stream_read(16, 24, 64, None) == 1
    B.moe_latent_destroy(None)   # NULL-safe
    assert B.lib().moe_latent_status(None) == 1


def test_lm_head_refusals_before_the_device():
    """moe_lm_head_gemv refuses bad descriptors, sizes, rows and dtypes by name before it
    looks for a device (no GPU here)."""
    def rc(shape=(64, 256), dtype=B.MOE_DT_BF16, rows=1, out_dtype=B.MOE_DT_F32, strides=None, x=FAKE, out=FAKE * 4):
        t = B.make_tensor(FAKE, dtype, list(shape), strides)
        return B.STATUS[B.moe_lm_head_gemv_rc(t, rows, x, out, out_dtype)], B.moe_latent_last_error()
    assert rc(dtype=B.MOE_DT_F32)[0] == "MOE_ERR_DTYPE"
    assert rc(dtype=B.MOE_DT_U32)[0] == "MOE_ERR_DTYPE"
    assert rc(shape=(64, 256), strides=[1, 64])[0] == "MOE_ERR_LAYOUT"
    assert rc(shape=(40, 256))[0] == "MOE_ERR_SHAPE"
    assert rc(shape=(64, 200))[0] == "MOE_ERR_SHAPE"
    assert rc(rows=0)[0] == "MOE_ERR_ROWS"
    assert rc(rows=257)[0] == "MOE_ERR_ROWS"
    assert rc(out_dtype=B.MOE_DT_F16)[0] == "MOE_ERR_DTYPE"
    assert rc(x=0)[0] == "MOE_ERR_INVALID_ARG"
    assert rc(x=FAKE + 2)[0] == "MOE_ERR_LAYOUT"
    code, msg = rc(x=FAKE * 4 + 16)
    assert code == "MOE_ERR_ALIAS", msg
    code, msg = rc()
    assert code == "MOE_ERR_DEVICE", msg      # a valid call reaches the device check
