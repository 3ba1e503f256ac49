"""The fused prefill (moe_latent_prefill) against the oracle.

TensorFold pull request 1038, «Not yet / next», names a fused prefill for the latent MoE
(prompts otherwise run through the decode kernels 16 rows at a time). The prefill computes
the layer the decode path computes, row by row, so the oracle is the same per-row forward.
Bars, as for the decode path: gate logits and routing bit for bit (the prefill gate keeps
the decode gate's order); each expert activation and output, fed its own GPU input, within
one unit in the last place of the oracle's stage (five after relu^2), at least 95 % of them
equal (the decode path, whose sums run closer to the oracle's order, keeps 99 %: the MFMA
group sums here take another order, so a rounding lands one unit off somewhat more often);
outputs within the
relative 2-norm bar 5e-3 and the magnitude-scaled max bar 2e-2; each row of a prefill equal
to that row's one-row prefill bit for bit; two runs equal bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

from latent_mixture_experts_bf16_amd import synth
from oracle import oracle as O

from test_gpu_parity import _act, _oracle_threads, assert_out_close, stage_close

pytestmark = pytest.mark.gpu

TINY = synth.LayerDims(hidden=512, latent=128, n_experts=16, n_group=4, topk_group=2, top_k=2,
                       expert_inter=256, shared_inter=512)
BOLT = synth.WORKLOADS[1].layers[0]
EQ = 0.95   # share of stage values equal to the oracle's


def _LY():
    from latent_mixture_experts_bf16_amd import layer as LY
    return LY


def _B():
    from latent_mixture_experts_bf16_amd import binding as B
    return B


def _prefill(dims, arrays, rows=None, max_rows=None, x=None):
    LY = _LY()
    x = arrays["x"] if x is None else x
    rows = x.shape[0] if rows is None else rows
    lay = LY.DeviceLayer(dims, arrays, max_rows or rows)
    xd = LY.to_device(x)
    out = torch.empty_like(xd)
    print(f"prefill: rows {rows} E {dims.n_experts} H {dims.hidden} L {dims.latent}", flush=True)
    lay.prefill(xd, out, rows)
    torch.cuda.synchronize()
    lay.status()
    return lay, xd, out


def _check_rows_alone(lay, xd, got, rows_to_check):
    for r in rows_to_check:
        o1 = torch.empty_like(xd[r:r + 1])
        lay.prefill(xd[r:r + 1], o1, 1)
        torch.cuda.synchronize()
        lay.status()
        assert np.array_equal(o1.cpu().numpy().view(np.uint16)[0], got[r]), r


def _check_layer(dims, arrays, what, sample=None, stage_rows=(), alone=()):
    rows = arrays["x"].shape[0]
    sel = list(range(rows)) if sample is None else list(sample)
    ref = O.forward(dims, arrays, rows=sel, threads=_oracle_threads())
    lay, xd, out = _prefill(dims, arrays)
    idx, w = lay.routing(rows)
    assert np.array_equal(idx[sel], ref["idx"]), what
    assert np.array_equal(w[sel].view(np.uint32), ref["w"].view(np.uint32)), what
    got = out.cpu().numpy().view(np.uint16)
    assert_out_close(dims, got[sel], ref["out_f32"], what)
    if stage_rows:
        x = _act(dims, arrays["x"])
        D, I = dims.latent or dims.hidden, dims.expert_inter
        u = _act(dims, lay.stage("latent", rows)) if dims.latent else x
        a = _act(dims, lay.stage("expert_act", rows)).reshape(rows, dims.top_k, I)
        y = _act(dims, lay.stage("expert_out", rows)).reshape(rows, dims.top_k, D)
        for r in stage_rows:
            if dims.latent:
                stage_close(dims, u[r], O.stage(dims, arrays, "latent", x[r]), f"latent {r}", eq_min=EQ)
            for j in range(dims.top_k):
                e = int(idx[r, j])
                stage_close(dims, a[r, j], O.stage(dims, arrays, "expert_act", u[r], e), f"act {r} {j}", ulps=5,
                            eq_min=EQ)
                stage_close(dims, y[r, j], O.stage(dims, arrays, "expert_out", a[r, j], e), f"out {r} {j}",
                            eq_min=EQ)
            if dims.shared_inter:
                sa = _act(dims, lay.stage("shared_act", rows))
                so = _act(dims, lay.stage("shared_out", rows))
                stage_close(dims, sa[r], O.stage(dims, arrays, "shared_act", x[r]), "shared_act", ulps=5, eq_min=EQ)
                stage_close(dims, so[r], O.stage(dims, arrays, "shared_out", sa[r]), "shared_out", eq_min=EQ)
    # a second run: the same bits
    out2 = torch.empty_like(xd)
    lay.prefill(xd, out2, rows)
    torch.cuda.synchronize()
    lay.status()
    assert np.array_equal(out2.cpu().numpy().view(np.uint16), got), what
    _check_rows_alone(lay, xd, got, alone)
    lay.close()
    return got


@pytest.mark.parametrize("rows", [1, 5, 130, 700])
def test_prefill_tiny_layer_all_rows(rows):
    """A small latent layer: every row against the oracle (rows across several 128-row
    tiles with a ragged tail, and experts with several 64-pick tiles)."""
    arrays = synth.make_layer(TINY, rows, weight_seed=9100, input_seed=9101 + rows)
    _check_layer(TINY, arrays, f"tiny rows {rows}", stage_rows=sorted({0, rows // 2, rows - 1}),
                 alone=sorted({0, rows - 1}))


def test_prefill_bolt_layer_512_rows():
    """The Bolt-like layer (240 experts, top-9, latent 1024, shared 4096) at 512 rows: routing
    of every row bit for bit (gate logits too), outputs of 64 sampled rows against the oracle,
    stages of 3 rows, and 3 rows against their one-row prefill."""
    rows = 512
    d, arrays = next(synth.workload_layers(1, rows=rows))
    sample = sorted(set(np.random.default_rng(3).choice(rows, 64, replace=False).tolist()) | {0, rows - 1})
    lay_got = _check_layer(d, arrays, "bolt 512", sample=sample, stage_rows=(0, 255, 511), alone=(0, 300, 511))
    assert lay_got.shape == (rows, d.hidden)


def test_prefill_logits_and_routing_every_row_bolt():
    """Gate logits of all 512 rows bit for bit against the oracle's (C64 order), and every
    row's routing."""
    rows = 512
    d, arrays = next(synth.workload_layers(1, rows=rows))
    lay, xd, out = _prefill(d, arrays)
    z = O.bf16_to_f32(lay.stage("logits", rows)).reshape(rows, -1)
    x = O.bf16_to_f32(arrays["x"])
    wg = O.bf16_to_f32(arrays["gate_w"])
    zr = O.gate_c64(x, wg)
    zr_b = O.bf16_to_f32(O.f32_to_bf16(zr))
    assert np.array_equal(z.view(np.uint32), zr_b.view(np.uint32))
    lay.close()


def test_prefill_matches_decode_within_bar():
    """The 16-row Bolt-like pass (496 experts): prefill and decode give the same routing and
    outputs within the bar of each other."""
    LY = _LY()
    d, arrays = next(synth.workload_layers(2))
    rows = arrays["x"].shape[0]
    lay = LY.DeviceLayer(d, arrays, rows)
    xd = LY.to_device(arrays["x"])
    o_dec, o_pf = torch.empty_like(xd), torch.empty_like(xd)
    lay.forward(xd, o_dec, rows)
    torch.cuda.synchronize()
    idx_d, w_d = lay.routing(rows)
    lay.prefill(xd, o_pf, rows)
    torch.cuda.synchronize()
    lay.status()
    idx_p, w_p = lay.routing(rows)
    assert np.array_equal(idx_d, idx_p) and np.array_equal(w_d.view(np.uint32), w_p.view(np.uint32))
    ref = _act(d, o_dec.cpu().numpy().view(np.uint16))
    assert_out_close(d, o_pf.cpu().numpy().view(np.uint16), ref, "prefill vs decode")
    lay.close()


def test_prefill_496_experts():
    """More than 256 experts (the route's large table): the Bolt-like layer with 496 experts
    at 40 rows, routing bit for bit and outputs within the bar on every row."""
    d, arrays = next(synth.workload_layers(2, rows=40))
    _check_layer(d, arrays, "bolt E496", stage_rows=(0, 39), alone=(17,))


def test_prefill_non_latent_bf16_layer():
    dims = synth.LayerDims(hidden=1024, latent=0, n_experts=32, n_group=1, topk_group=1, top_k=4,
                           expert_inter=512, shared_inter=0)
    arrays = synth.make_layer(dims, 300, weight_seed=9300, input_seed=9301)
    _check_layer(dims, arrays, "non-latent", stage_rows=(0, 299), alone=(7,))


def test_prefill_fp32_router():
    dims = dataclasses.replace(TINY, router_dtype=synth.F32, has_bias=False, n_group=1, topk_group=1)
    arrays = synth.make_layer(dims, 200, weight_seed=9400, input_seed=9401)
    _check_layer(dims, arrays, "fp32 router", stage_rows=(3,), alone=(199,))


def test_prefill_in_place():
    arrays = synth.make_layer(TINY, 150, weight_seed=9500, input_seed=9501)
    LY = _LY()
    lay = LY.DeviceLayer(TINY, arrays, 150)
    xd = LY.to_device(arrays["x"])
    out = torch.empty_like(xd)
    lay.prefill(xd, out, 150)
    lay.prefill(xd, xd, 150)
    torch.cuda.synchronize()
    lay.status()
    assert np.array_equal(xd.cpu().numpy(), out.cpu().numpy())
    lay.close()


def test_prefill_refusals():
    B, LY = _B(), _LY()
    arrays = synth.make_layer(TINY, 4, weight_seed=9600, input_seed=9601)
    lay = LY.DeviceLayer(TINY, arrays, 300)
    xd = LY.to_device(np.zeros((300, TINY.hidden), np.uint16))
    out = torch.empty_like(xd)
    assert B.STATUS[B.moe_latent_prefill_rc(lay.handle, 301, xd.data_ptr(), out.data_ptr())] == "MOE_ERR_ROWS"
    assert B.STATUS[B.moe_latent_prefill_rc(lay.handle, 0, xd.data_ptr(), out.data_ptr())] == "MOE_ERR_ROWS"
    # a decode pass takes at most 256 rows
    assert B.STATUS[B.moe_latent_forward_rc(lay.handle, 257, xd.data_ptr(), out.data_ptr())] == "MOE_ERR_ROWS"
    assert "moe_latent_prefill" in B.moe_latent_last_error()
    lay.prefill(xd, out, 300)
    torch.cuda.synchronize()
    lay.close()
    # other expert formats and f16 activations are refused by name
    d3 = dataclasses.replace(TINY, quant_bits=3)
    lay = LY.DeviceLayer(d3, synth.make_layer(d3, 2, weight_seed=9602), 8)
    x8 = LY.to_device(np.zeros((8, TINY.hidden), np.uint16))
    o8 = torch.empty_like(x8)
    assert B.STATUS[B.moe_latent_prefill_rc(lay.handle, 8, x8.data_ptr(), o8.data_ptr())] == "MOE_ERR_SHAPE"
    assert "4-bit" in B.moe_latent_last_error()
    lay.close()
    d16 = synth.WORKLOADS[3].layers[0]
    d16 = dataclasses.replace(d16, n_experts=16, top_k=4, n_group=1, topk_group=1)
    lay = LY.DeviceLayer(d16, synth.make_layer(d16, 2, weight_seed=9603), 8)
    x8 = LY.to_device(np.zeros((8, d16.hidden), np.uint16))
    o8 = torch.empty_like(x8)
    assert B.STATUS[B.moe_latent_prefill_rc(lay.handle, 8, x8.data_ptr(), o8.data_ptr())] == "MOE_ERR_DTYPE"
    lay.close()


def test_prefill_4096_rows_bolt():
    """4096 rows (the largest prefill) of the Bolt-like layer: routing of every row bit for
    bit against a 64-row oracle sample, outputs of those rows within the bar, and 2 rows
    against their one-row prefill."""
    rows = 4096
    d, arrays = next(synth.workload_layers(1, rows=rows))
    sample = sorted(set(np.random.default_rng(11).choice(rows, 62, replace=False).tolist()) | {0, rows - 1})
    _check_layer(d, arrays, "bolt 4096", sample=sample, alone=(0, 4095))


@pytest.mark.parametrize("rows,chunk", [(4096, 512), (3500, 512), (1500, 500)])
def test_prefill_big_tiles_match_small_tiles(rows, chunk):
    """At 4096 rows (and at 3500, whose last tile of 256 rows holds 172) the dense projections
    run in tiles of 256 rows x 320 or 256 outputs; passes of at most 512 rows run them in
    128 x 128 tiles of 128 inputs a step. At 1500 rows (a last tile of 92 rows) they run in
    128 x 128 tiles of 64 inputs a step. Every shape sums each output in the same order, so
    every row's latent, shared expert stages and output are the same bits either way."""
    d, arrays = next(synth.workload_layers(1, rows=rows))
    lay, xd, out = _prefill(d, arrays)
    got = out.cpu().numpy().view(np.uint16)
    stages = {n: lay.stage(n, rows).copy() for n in ("latent", "shared_act", "shared_out")}
    for c in range(0, rows, chunk):
        n_rows = min(chunk, rows - c)
        o = torch.empty_like(xd[c:c + n_rows])
        lay.prefill(xd[c:c + n_rows], o, n_rows)
        torch.cuda.synchronize()
        lay.status()
        assert np.array_equal(o.cpu().numpy().view(np.uint16), got[c:c + n_rows]), c
        for n, full in stages.items():
            assert np.array_equal(lay.stage(n, n_rows), full[c:c + n_rows]), (n, c)
    lay.close()


@pytest.mark.parametrize("rows", [70, 300])
def test_prefill_graph_replays_match_eager(rows):
    """A prefill captured in a HIP graph gives the eager bits on every replay, with eager work
    (a prefill of other rows and a decode pass) between the replays; the per-expert counts
    are cleared by a kernel, not a memset node."""
    B, LY = _B(), _LY()
    arrays = synth.make_layer(TINY, rows, weight_seed=9700, input_seed=9701 + rows)
    lay = LY.DeviceLayer(TINY, arrays, rows)
    xd = LY.to_device(arrays["x"])
    eager = torch.empty_like(xd)
    lay.prefill(xd, eager, rows)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy()
    s = torch.cuda.Stream()
    B.moe_latent_set_stream(lay.handle, s.cuda_stream)
    out = torch.empty_like(xd)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        lay.prefill(xd, out, rows)      # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            lay.prefill(xd, out, rows)
    x_other = xd[5:40].contiguous()
    other = torch.empty_like(x_other)
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), i
        with torch.cuda.stream(s):
            lay.prefill(x_other, other, 35)
            lay.forward(x_other[:3], other[:3], 3)
        torch.cuda.synchronize()
    lay.status()
    lay.close()
