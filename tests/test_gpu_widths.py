"""Routed experts of the other affine widths (2, 3, 5, 6 and 8 bits; 4 bits in groups of 32
or 128) through the width-generic expert kernels, against the oracle.

The mlx-bun decode-speed program (§7.4, experiment axes) sweeps the affine family over code
widths and group sizes; the layer's own format is 4 bits in groups of 64. Bars as in the
parity tests of that format: routing bit for bit, each expert activation and expert output
fed its own GPU input within one unit in the last place (five after relu^2) of the
oracle's stage, outputs within the relative 2-norm and magnitude-scaled max bars, and each
row of a multi-row pass equal to its own one-row pass bit for bit (the one-row pass combines
inside fc2, the multi-row pass in the last expert item of each block).
"""
import dataclasses

import numpy as np
import pytest
import torch

from latent_mixture_experts_bf16_amd import synth
from oracle import oracle as O

from test_gpu_parity import _act, assert_out_close, run_gpu, stage_close

pytestmark = pytest.mark.gpu

TINY = synth.LayerDims(hidden=512, latent=128, n_experts=16, n_group=4, topk_group=2, top_k=2,
                       expert_inter=256, shared_inter=512)

FORMATS = [(2, 32), (2, 128), (3, 64), (3, 32), (4, 32), (4, 128), (5, 64), (6, 32), (6, 128),
           (8, 64), (8, 128)]


def _check_stages(dims, arrays, lay, rows, idx):
    x = _act(dims, arrays["x"])
    I, D = dims.expert_inter, dims.latent or dims.hidden
    u = _act(dims, lay.stage("latent", rows)) if dims.latent else x
    a = _act(dims, lay.stage("expert_act", rows)).reshape(rows, dims.top_k, I)
    y = _act(dims, lay.stage("expert_out", rows)).reshape(rows, dims.top_k, D)
    for r in range(rows):
        for j in range(dims.top_k):
            e = int(idx[r, j])
            stage_close(dims, a[r, j], O.stage(dims, arrays, "expert_act", u[r], e), f"expert_act {r} {j}", ulps=5)
            stage_close(dims, y[r, j], O.stage(dims, arrays, "expert_out", a[r, j], e), f"expert_out {r} {j}")


def _run_and_check(dims, arrays, what, stages=True):
    rows = arrays["x"].shape[0]
    ref = O.forward(dims, arrays)
    lay, xd, out = run_gpu(dims, arrays)
    idx, w = lay.routing(rows)
    assert np.array_equal(idx, ref["idx"]), what
    assert np.array_equal(w.view(np.uint32), ref["w"].view(np.uint32)), what
    if stages:
        _check_stages(dims, arrays, lay, rows, idx)
    got = out.cpu().numpy().view(np.uint16)
    assert_out_close(dims, got, ref["out_f32"], what)
    if rows > 1:
        for r in sorted({0, rows - 1}):
            o1 = torch.empty_like(xd[r:r + 1])
            lay.forward(xd[r:r + 1], o1, 1)
            torch.cuda.synchronize()
            lay.status()
            assert np.array_equal(o1.cpu().numpy().view(np.uint16)[0], got[r]), (what, r)
    lay.close()


@pytest.mark.parametrize("bits,gs", FORMATS)
def test_tiny_latent_layer_every_format(bits, gs):
    dims = dataclasses.replace(TINY, quant_bits=bits, group_size=gs)
    arrays = synth.make_layer(dims, 5, weight_seed=7000 + 10 * bits + gs, input_seed=7001)
    _run_and_check(dims, arrays, f"tiny {bits}-bit g{gs}")


@pytest.mark.parametrize("bits,gs", [(2, 64), (3, 128), (8, 32)])
def test_bolt_like_layer_other_widths(bits, gs):
    """Hidden 4096, latent 1024, 64 experts in 8 groups, top-9, expert width 2048, shared
    width 4096: the routed shapes of the Bolt-like layer at a smaller expert count."""
    dims = dataclasses.replace(synth.WORKLOADS[1].layers[0], n_experts=64, quant_bits=bits, group_size=gs)
    arrays = synth.make_layer(dims, 3, weight_seed=7100 + bits, input_seed=7101)
    _run_and_check(dims, arrays, f"bolt-like E64 {bits}-bit g{gs}", stages=False)


@pytest.mark.parametrize("bits,gs", [(3, 32), (6, 64)])
def test_non_latent_bf16_layer_other_widths(bits, gs):
    """A non-latent bf16 layer (experts over the hidden vector; the combine adds the input)."""
    dims = synth.LayerDims(hidden=1024, latent=0, n_experts=32, n_group=1, topk_group=1, top_k=4,
                           expert_inter=512, shared_inter=0, quant_bits=bits, group_size=gs)
    arrays = synth.make_layer(dims, 4, weight_seed=7200 + bits, input_seed=7201)
    _run_and_check(dims, arrays, f"non-latent {bits}-bit g{gs}")


@pytest.mark.parametrize("bits,gs", [(5, 128), (2, 32)])
def test_wide_expert_rows_other_widths(bits, gs):
    """Expert inputs wider than 2048 (the wide kernel variant: one input row in LDS)."""
    dims = synth.LayerDims(hidden=3072, latent=0, n_experts=16, n_group=4, topk_group=2, top_k=3,
                           expert_inter=384, shared_inter=0, quant_bits=bits, group_size=gs)
    arrays = synth.make_layer(dims, 2, weight_seed=7300 + bits, input_seed=7301)
    _run_and_check(dims, arrays, f"wide {bits}-bit g{gs}")

