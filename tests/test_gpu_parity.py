"""Parity of the HIP layer (through the C ABI) with the CPU oracle, on the seeded workloads.

Bars (the oracle's readings):
* routing indices and weights: bit for bit;
* gate logits: bit for bit (both sides use the same fixed summation order);
* combine: bit for bit when the oracle combines the GPU's own expert outputs and weights;
* layer outputs, against the oracle's fp32 value before its final rounding: relative error
  in the 2-norm <= 5e-3, and max-abs error <= 2e-2 with each element's error scaled by
  1 / max(RMS(oracle), |oracle value|). Scaling by 1 / RMS alone is below one bf16 unit in
  the last place for outputs beyond about 2.6 x RMS, which these layers reach (up to about
  6 x RMS): the fp32 sums before each intermediate bf16 rounding (fc2, shared expert) run in
  different orders on the two sides, so such a rounding can land one unit apart and move the
  output by about a unit there. The max-abs error scaled by 1 / RMS alone, the raw max-abs
  error and the largest error in units of the last place are printed beside the bar;
* each row of a multi-row pass equals its own one-row pass bit for bit.
"""
import gc
import os

import numpy as np
import pytest
import torch

from latent_mixture_experts_bf16_amd import synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu

REL_RMS = 5e-3
REL_MAX = 2e-2


def _LY():
    from latent_mixture_experts_bf16_amd import layer as LY
    return LY


def _x_dev(dims, x_bits):
    return _LY().to_device(x_bits)


def _act(dims, bits):
    return O.act_to_f32(dims, bits)


def out_errors(dims, got_bits, ref_f32):
    """Errors of the GPU's outputs against the oracle's fp32 values before their final
    rounding: (relative 2-norm error; the bar's max error, each element's error divided by
    max(RMS(oracle), |oracle value|); the max-abs error divided by RMS(oracle) alone, reported;
    the raw max-abs error; the largest error in units of the last place of the activation
    dtype, over outputs at least as large as RMS(oracle))."""
    got = _act(dims, got_bits).astype(np.float64)
    ref = ref_f32.astype(np.float64)
    d = np.abs(got - ref)
    rms = np.sqrt((ref ** 2).mean())
    rel_rms = np.sqrt((d ** 2).mean()) / rms
    rel_max = float((d / np.maximum(rms, np.abs(ref))).max())
    max_abs = float(d.max())
    big = np.abs(ref) >= rms
    ulps = float((d[big] / act_ulp(dims, ref_f32[big])).max()) if big.any() else 0.0
    return rel_rms, rel_max, max_abs / rms, max_abs, ulps


def assert_out_close(dims, got_bits, ref_f32, what=""):
    assert np.isfinite(_act(dims, got_bits)).all(), what
    rel_rms, rel_max, lit, max_abs, ulps = out_errors(dims, got_bits, ref_f32)
    print(f"{what}: rel_rms {rel_rms:.2e} max_rel {rel_max:.2e} (max_abs/rms {lit:.2e}, raw max_abs "
          f"{max_abs:.3g}, max {ulps:.2f} ulp where |ref| >= rms)", flush=True)
    assert rel_rms <= REL_RMS and rel_max <= REL_MAX, (what, rel_rms, rel_max, lit, max_abs, ulps)


def act_ulp(dims, v):
    """Unit in the last place of each value in the activation dtype."""
    v = np.abs(np.asarray(v, np.float32))
    if dims.act_dtype == 2:
        return np.spacing(v.astype(np.float16)).astype(np.float64)
    return np.spacing(v).astype(np.float64) * 65536.0


def stage_close(dims, got, ref, what, ulps=1, eq_min=0.99):
    ref_vals, ref_pre = ref
    got = np.asarray(got, np.float64)
    rv = ref_vals.astype(np.float64)
    rms = np.sqrt((rv ** 2).mean()) + 1e-30
    err = np.abs(got - rv)
    tol = ulps * act_ulp(dims, ref_vals) + 1e-4 * rms
    eq = float((got == rv).mean())
    assert eq >= eq_min and (err <= tol).all(), (what, eq, float((err / tol).max()))


_data = {}


def workload(cid, rows=None, layer=0, instance=0):
    key = (cid, rows, layer, instance)
    if key not in _data:
        if len(_data) > 3:
            _data.clear()
        dims, arrays = next(synth.workload_layers(cid, instance=instance, rows=rows, layers=[layer]))
        _data[key] = (dims, arrays)
    return _data[key]


def run_gpu(dims, arrays, rows=None, variant=None, max_rows=None, x=None):
    x = arrays["x"] if x is None else x
    rows = x.shape[0] if rows is None else rows
    lay = _LY().DeviceLayer(dims, arrays, max_rows or rows, variant=variant)
    xd = _x_dev(dims, x)
    out = torch.empty_like(xd)
    lay.forward(xd, out, rows)
    torch.cuda.synchronize()
    lay.status()
    return lay, xd, out


# ---------------------------------------------------------------------------------- per config

@pytest.mark.parametrize("cid", [0, 1, 3])
def test_layer_matches_oracle(cid):
    dims, arrays = workload(cid)
    rows = arrays["x"].shape[0]
    ref = O.forward(dims, arrays, stages=True)
    lay, xd, out = run_gpu(dims, arrays)
    idx, w = lay.routing(rows)
    assert np.array_equal(idx, ref["idx"]), (idx, ref["idx"])
    assert np.array_equal(w.view(np.uint32), ref["w"].view(np.uint32))
    # gate logits: bit for bit
    z = lay.stage("logits", rows)
    zf = z if dims.router_dtype == 3 else O.bf16_to_f32(z)
    assert np.array_equal(zf.reshape(rows, -1).view(np.uint32), ref["z"].view(np.uint32))
    # combine of the GPU's own expert outputs: bit for bit
    D = dims.latent or dims.hidden
    y = _act(dims, lay.stage("expert_out", rows)).reshape(rows, dims.top_k, D)
    c = lay.stage("combine", rows)
    for r in range(rows):
        cc = O.combine(y[r], w[r])
        want = O.f32_to_f16(cc) if dims.act_dtype == 2 else O.f32_to_bf16(cc)
        assert np.array_equal(c[r], want)
    # every other stage, fed its own GPU input: equal to the oracle's stage up to fp32
    # summation order -- one unit in the last place (plus 1e-4 of the stage's RMS for sums
    # that cancel); after relu^2 five: a one-unit flip of the rounded pre-activation h moves
    # h^2 by 2*h*ulp(h), up to 4 units of h^2 when h^2 falls in the lower half of its binade
    x = _act(dims, arrays["x"])
    I = dims.expert_inter
    u = _act(dims, lay.stage("latent", rows)) if dims.latent else x
    a = _act(dims, lay.stage("expert_act", rows)).reshape(rows, dims.top_k, I)
    for r in range(rows):
        if dims.latent:
            stage_close(dims, u[r], O.stage(dims, arrays, "latent", x[r]), "latent")
        for j in range(dims.top_k):
            e = int(idx[r, j])
            stage_close(dims, a[r, j], O.stage(dims, arrays, "expert_act", u[r], e), "expert_act", ulps=5)
            stage_close(dims, y[r, j], O.stage(dims, arrays, "expert_out", a[r, j], e), "expert_out")
        if dims.shared_inter:
            sa = _act(dims, lay.stage("shared_act", rows))
            so = _act(dims, lay.stage("shared_out", rows))
            stage_close(dims, sa[r], O.stage(dims, arrays, "shared_act", x[r]), "shared_act", ulps=5)
            stage_close(dims, so[r], O.stage(dims, arrays, "shared_out", sa[r]), "shared_out")
    assert_out_close(dims, out.cpu().numpy().view(np.uint16), ref["out_f32"], f"cfg{cid}")
    lay.close()


def test_wide_projections_split_over_items():
    """Projections wider than 4096 inputs (fc1, shared up and shared down at hidden = shared
    width = 8192) are cut into parts whose partial sums the last part adds: outputs within
    the bar, and each row of a 3-row pass equal to its own one-row pass."""
    dims = synth.LayerDims(hidden=8192, latent=1024, n_experts=16, n_group=4, topk_group=2, top_k=2,
                           expert_inter=256, shared_inter=8192, group_size=64, act_dtype=1,
                           router_dtype=1, has_bias=True, norm_topk=True, routed_scaling=2.5)
    arrays = synth.make_layer(dims, 3, weight_seed=4242, input_seed=4243)
    ref = O.forward(dims, arrays)
    lay, xd, out = run_gpu(dims, arrays)
    idx, w = lay.routing(3)
    assert np.array_equal(idx, ref["idx"])
    assert np.array_equal(w.view(np.uint32), ref["w"].view(np.uint32))
    got = out.cpu().numpy().view(np.uint16)
    assert_out_close(dims, got, ref["out_f32"], "hidden 8192")
    for r in range(3):
        o1 = torch.empty_like(xd[r:r + 1])
        lay.forward(xd[r:r + 1], o1, 1)
        torch.cuda.synchronize()
        lay.status()
        assert np.array_equal(o1.cpu().numpy().view(np.uint16)[0], got[r]), r
    lay.close()


def _routing_layer(case):
    """Small layers whose routing takes the less common paths: more than 64 groups, more
    than 64 candidates (both ranked by the multi-step LDS path), planted ties of scores and
    of group scores, NaN logits, and more than 64 experts without group selection in a number
    that is not a multiple of 64 (ranked inside blocks of 64, the last block holding fewer
    experts than top_k), with ties across the blocks."""
    if case == "ungrouped_ragged":
        dims = synth.LayerDims(hidden=512, latent=128, n_experts=70, n_group=1, topk_group=1, top_k=8,
                               expert_inter=256, shared_inter=512, group_size=64, act_dtype=1,
                               router_dtype=1, has_bias=True, norm_topk=True, routed_scaling=2.5)
    elif case == "groups_over_64":
        dims = synth.LayerDims(hidden=512, latent=128, n_experts=256, n_group=128, topk_group=6, top_k=9,
                               expert_inter=256, shared_inter=0, group_size=64, act_dtype=1,
                               router_dtype=1, has_bias=True, norm_topk=True, routed_scaling=2.5)
    elif case == "candidates_over_64":
        dims = synth.LayerDims(hidden=512, latent=128, n_experts=256, n_group=32, topk_group=12, top_k=9,
                               expert_inter=256, shared_inter=0, group_size=64, act_dtype=1,
                               router_dtype=1, has_bias=True, norm_topk=True, routed_scaling=2.5)
    else:
        dims = synth.LayerDims(hidden=512, latent=128, n_experts=64, n_group=8, topk_group=4, top_k=6,
                               expert_inter=256, shared_inter=0, group_size=64, act_dtype=1,
                               router_dtype=1, has_bias=True, norm_topk=True, routed_scaling=2.5)
    arrays = synth.make_layer(dims, 3, weight_seed=5150 + len(case), input_seed=5151)
    wg, cb = arrays["gate_w"], arrays["corr_bias"]
    if case == "ties":
        # equal scores inside a group (experts 3, 5 of group 0) and across groups (11, 12),
        # and group 5 a copy of group 2 (equal group scores)
        for e in (5, 11, 12):
            wg[e] = wg[3]
            cb[e] = cb[3]
        wg[40:48] = wg[16:24]
        cb[40:48] = cb[16:24]
        # raise the planted experts so that they are picked
        cb[[3, 5, 11, 12]] += np.float32(0.5)
    elif case == "nan":
        wg[7, 100] = 0x7FC0          # a NaN weight: expert 7's logit is NaN
        wg[56:64, 0] = 0x7FC0        # all of group 7
        cb[7] = np.float32(1.0)      # would rank first otherwise
    elif case == "ungrouped_ragged":
        # experts 66 and 68 (the last block, of 6) tie with 2 and 40 (the first), all raised
        # so that they are picked: the tie goes to the lower id across the blocks
        for a, b in ((66, 2), (68, 40)):
            wg[a] = wg[b]
            cb[a] = cb[b]
        cb[[2, 40, 66, 68]] += np.float32(0.5)
    return dims, arrays


@pytest.mark.parametrize("case", ["groups_over_64", "candidates_over_64", "ties", "nan", "ungrouped_ragged"])
def test_routing_edge_cases(case):
    """Routing bit for bit in a 3-row pass (the stage kernel's route items) and in each row's
    one-row pass (the front kernel's route workgroup), and each row's output equal in both."""
    dims, arrays = _routing_layer(case)
    ref = O.forward(dims, arrays)
    lay, xd, out = run_gpu(dims, arrays)
    idx, w = lay.routing(3)
    assert np.array_equal(idx, ref["idx"]), (case, idx, ref["idx"])
    assert np.array_equal(w.view(np.uint32), ref["w"].view(np.uint32)), case
    got = out.cpu().numpy().view(np.uint16)
    assert_out_close(dims, got, ref["out_f32"], case)
    if case == "ties":
        assert {3, 5}.issubset(set(ref["idx"][0].tolist()))
    if case == "nan":
        assert 7 not in ref["idx"][0].tolist()
    if case == "ungrouped_ragged":
        assert {2, 40, 66, 68}.issubset(set(ref["idx"][0].tolist()))
    for r in range(3):
        o1 = torch.empty_like(xd[r:r + 1])
        lay.forward(xd[r:r + 1], o1, 1)
        torch.cuda.synchronize()
        lay.status()
        i1, w1 = lay.routing(1)
        assert np.array_equal(i1[0], ref["idx"][r]), (case, r)
        assert np.array_equal(w1[0].view(np.uint32), ref["w"][r].view(np.uint32)), (case, r)
        assert np.array_equal(o1.cpu().numpy().view(np.uint16)[0], got[r]), (case, r)
    lay.close()


def test_sigmoid_of_every_finite_bf16_logit():
    """The route's sigmoid (binary64, rounded once to fp32) on the GPU equals the oracle's on
    every finite bf16 logit. A 256-row pass of a 16-expert layer with every expert picked,
    no normalisation and a scale of 1 returns w = s exactly; row r's input is the unit
    vector e_r, so expert e's logit is exactly its gate weight at column r. Sixteen passes
    cover the 65,280 finite bf16 values."""
    dims = synth.LayerDims(hidden=512, latent=128, n_experts=16, n_group=1, topk_group=1, top_k=16,
                           expert_inter=256, shared_inter=0, group_size=64, act_dtype=1,
                           router_dtype=1, has_bias=False, norm_topk=False, routed_scaling=1.0)
    rows, E = 256, 16
    arrays = synth.make_layer(dims, rows, weight_seed=6060, input_seed=6061)
    x = np.zeros((rows, dims.hidden), np.uint16)
    x[np.arange(rows), np.arange(rows)] = 0x3F80            # bf16 1.0
    arrays["x"] = x
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7F80) != 0x7F80]
    lay = None
    for f in range(16):
        chunk = finite[f * rows * E:(f + 1) * rows * E]
        if chunk.size == 0:
            break
        vals = np.zeros(rows * E, np.uint16)
        vals[:chunk.size] = chunk
        wg = np.zeros((E, dims.hidden), np.uint16)
        wg[:, :rows] = vals.reshape(rows, E).T                   # expert e, column r
        arrays["gate_w"] = wg
        if lay is not None:
            lay.close()
        lay, xd, out = run_gpu(dims, arrays, max_rows=rows)
        idx, w = lay.routing(rows)
        got = np.empty((rows, E), np.float32)
        got[np.arange(rows)[:, None], idx] = w
        want = O.sigmoid(O.bf16_to_f32(vals.reshape(rows, E)))
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f
    lay.close()


@pytest.mark.skip(reason="the one-launch fused variant is disabled: its first GPU run did not "
                         "complete, and the library refuses it (variant 0) until a cause is shown")
def test_fused_and_staged_launches_agree_bitwise():
    for cid in (0, 1):
        dims, arrays = workload(cid)
        outs = []
        for variant in (0, 1, 0):
            lay, xd, out = run_gpu(dims, arrays, variant=variant)
            outs.append((out.cpu().numpy(), *lay.routing(xd.shape[0])))
            lay.close()
        for o in outs[1:]:
            for a, b in zip(outs[0], o):
                assert np.array_equal(a, b)


@pytest.mark.parametrize("rows", [1, 9])
def test_graph_replays_match_eager(rows):
    """A forward captured in a HIP graph gives the eager bits on every replay, with eager
    work (another forward on different rows) between the replays."""
    from latent_mixture_experts_bf16_amd import binding as B
    dims, arrays = workload(0, rows=9)
    lay = _LY().DeviceLayer(dims, arrays, 9)
    xd = _x_dev(dims, arrays["x"][:rows])
    eager = torch.empty_like(xd)
    lay.forward(xd, eager)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy()
    s = torch.cuda.Stream()
    B.moe_latent_set_stream(lay.handle, s.cuda_stream)
    out = torch.empty_like(xd)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        lay.forward(xd, out)            # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            lay.forward(xd, out)
    x_other = _x_dev(dims, arrays["x"][3:6])
    other = torch.empty_like(x_other)
    for i in range(5):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), i
        with torch.cuda.stream(s):
            lay.forward(x_other, other, 3)
        torch.cuda.synchronize()
    lay.status()
    lay.close()


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_repeated_forwards_are_deterministic(cid):
    """Five forwards of the same input give the same bits and routing (workload 4: its
    first layer)."""
    dims, arrays = workload(cid)
    rows = arrays["x"].shape[0]
    lay = _LY().DeviceLayer(dims, arrays, rows)
    xd = _x_dev(dims, arrays["x"])
    first = None
    for _ in range(5):
        out = torch.empty_like(xd)
        lay.forward(xd, out)
        torch.cuda.synchronize()
        o = (out.cpu().numpy(), *lay.routing(rows))
        if first is None:
            first = o
        for a, b in zip(o, first):
            assert np.array_equal(a, b)
    lay.status()
    lay.close()


def test_timed_forward_equals_forward_and_records_each_launch():
    """The per-launch timed forward writes the same output as a plain forward, its events
    hold a positive duration for every launch group, and too few events are refused."""
    from latent_mixture_experts_bf16_amd import binding as B
    dims, arrays = workload(1)
    lay = _LY().DeviceLayer(dims, arrays, 1)
    xd = _x_dev(dims, arrays["x"])
    ref = torch.empty_like(xd)
    lay.forward(xd, ref)
    torch.cuda.synchronize()
    ng = sum(1 for g in range(10) if B.moe_latent_group_items(lay.handle, 1, g) > 0)
    assert ng == 4      # one row, one stream: gate + fc1 + shared up, up, down, fc2
    # the first launch: the front kernel (256 slice workgroups and the route workgroup), or
    # stage-kernel items under variant 4
    assert B.moe_latent_group_kernel(lay.handle, 1, 0) == "moe_front_kernel"
    assert B.moe_latent_group_items(lay.handle, 1, 0) == 257
    assert B.moe_latent_group_kernel(lay.handle, 1, 3) == "moe_stage_kernel<8, 8, false, 0>"
    assert B.moe_latent_group_kernel(lay.handle, 1, 4) == ""
    B.moe_latent_set_variant(lay.handle, 4)
    assert B.moe_latent_group_kernel(lay.handle, 1, 0) == "moe_stage_kernel<0, 2, false, 0>"
    B.moe_latent_set_variant(lay.handle, 2)
    ng2 = sum(1 for g in range(10) if B.moe_latent_group_items(lay.handle, 1, g) > 0)
    assert ng2 == 7     # two streams: gate + fc1, expert up, shared up, shared down x 2, down, fc2
    sides = [B.moe_latent_group_stages(lay.handle, 1, g)[3] for g in range(ng2)]
    assert sides == [0, 0, 1, 1, 1, 0, 0]
    evs2 = [torch.cuda.Event(enable_timing=True) for _ in range(2 * ng2)]
    for e in evs2:
        e.record()
    torch.cuda.synchronize()
    out2 = torch.empty_like(xd)
    B.moe_latent_forward_timed(lay.handle, 1, xd.data_ptr(), out2.data_ptr(), [e.cuda_event for e in evs2])
    torch.cuda.synchronize()
    lay.status()
    assert np.array_equal(out2.cpu().numpy(), ref.cpu().numpy())
    for g in range(ng2):
        assert evs2[2 * g].elapsed_time(evs2[2 * g + 1]) > 0.0, g
    B.moe_latent_set_variant(lay.handle, 3)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * ng)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    handles = [e.cuda_event for e in evs]
    out = torch.empty_like(xd)
    B.moe_latent_forward_timed(lay.handle, 1, xd.data_ptr(), out.data_ptr(), handles)
    torch.cuda.synchronize()
    lay.status()
    assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy())
    for g in range(ng):
        assert evs[2 * g].elapsed_time(evs[2 * g + 1]) > 0.0, g
    with pytest.raises(B.MoeError):
        B.moe_latent_forward_timed(lay.handle, 1, xd.data_ptr(), out.data_ptr(), handles[:-1])
    lay.close()


def test_stream_read_reads_every_word_once():
    """The read-only stream reference folds every 32-bit word of the buffer exactly once."""
    from latent_mixture_experts_bf16_amd import binding as B
    for nbytes in (16, 4096 + 48, (64 << 20) + 16 * 77):
        rng = np.random.default_rng(nbytes)
        host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
        src = torch.from_numpy(host.view(np.int32)).cuda()
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.moe_latent_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), 0)
        torch.cuda.synchronize()
        assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(host)), nbytes


def test_sixteen_rows_equal_sixteen_single_row_passes():
    """The 16-row E=496 workload (prompt rows pushed through the decode kernels 16 at a time,
    TensorFold pull request 1038, «Not yet / next»): each row equals its own 1-row pass bit
    for bit, and all rows match the oracle."""
    dims, arrays = workload(2)
    lay, xd, out = run_gpu(dims, arrays)
    multi = out.cpu().numpy()
    idx16, w16 = lay.routing(16)
    for r in range(16):
        o1 = torch.empty_like(xd[r:r + 1])
        lay.forward(xd[r:r + 1].contiguous(), o1, 1)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy()[0], multi[r]), r
        i1, w1 = lay.routing(1)
        assert np.array_equal(i1[0], idx16[r]) and np.array_equal(w1[0], w16[r])
    lay.status()
    ref = O.forward(dims, arrays)
    assert np.array_equal(idx16, ref["idx"])
    assert np.array_equal(w16.view(np.uint32), ref["w"].view(np.uint32))
    assert_out_close(dims, multi.view(np.uint16), ref["out_f32"], "cfg2 16 rows")
    lay.close()


@pytest.mark.parametrize("rows", [2, 7])
def test_identical_rows_share_every_expert(rows):
    """Degenerate routing: every row is the same token, so each of the k picked experts is
    picked by every row and its items take all `rows` pairs (passes of two pairs, and one
    pair alone for an odd count). Every output row equals the one-row pass of that token bit
    for bit and matches the oracle on it (Bolt-like layer, TensorFold pull request 1038,
    «What's in it»)."""
    dims, arrays = workload(1)
    x1 = np.ascontiguousarray(arrays["x"][:1])
    xr = np.ascontiguousarray(np.repeat(x1, rows, axis=0))
    lay, xd, out = run_gpu(dims, arrays, x=xr)
    multi = out.cpu().numpy()
    idx, w = lay.routing(rows)
    o1 = torch.empty_like(xd[:1])
    lay.forward(xd[:1].contiguous(), o1, 1)
    torch.cuda.synchronize()
    lay.status()
    single = o1.cpu().numpy()[0]
    ref = O.forward(dims, arrays)   # the workload's one row is this token
    for r in range(rows):
        assert np.array_equal(idx[r], ref["idx"][0]) and np.array_equal(w[r].view(np.uint32), ref["w"][0].view(np.uint32))
        assert np.array_equal(multi[r], single), r
    assert_out_close(dims, single.view(np.uint16)[None], ref["out_f32"][:1], f"identical rows {rows}")
    lay.close()


@pytest.mark.parametrize("rows", [1, 2, 9, 16, 17, 64, 256])
def test_tiny_layer_ragged_and_max_rows(rows):
    """Row counts that span several 16-row tiles with a ragged tail, up to max_rows = 256."""
    dims, arrays = workload(0, rows=rows)
    ref = O.forward(dims, arrays)
    lay, xd, out = run_gpu(dims, arrays, max_rows=256)
    idx, w = lay.routing(rows)
    assert np.array_equal(idx, ref["idx"])
    assert np.array_equal(w.view(np.uint32), ref["w"].view(np.uint32))
    assert_out_close(dims, out.cpu().numpy().view(np.uint16), ref["out_f32"], f"cfg0 rows {rows}")
    lay.close()


def test_in_place_output():
    dims, arrays = workload(0, rows=9)
    ref = O.forward(dims, arrays)
    lay = _LY().DeviceLayer(dims, arrays, 9)
    xd = _x_dev(dims, arrays["x"])
    lay.forward(xd, xd)          # out == hidden_in
    torch.cuda.synchronize()
    lay.status()
    assert_out_close(dims, xd.cpu().numpy().view(np.uint16), ref["out_f32"], "in place")
    lay.close()


def _oracle_threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("layer", list(range(8)))
def test_eight_layer_stack_64_rows(layer):
    """One layer of the 8-layer, 64-row stack (expert counts cycling 240..496, each layer with
    its own seeded input): routing of all 64 rows bit for bit, and all 64 output rows against
    the oracle (its rows run on the host's cores)."""
    dims, arrays = workload(4, layer=layer)
    lay, xd, out = run_gpu(dims, arrays)
    idx, w = lay.routing(64)
    got = out.cpu().numpy().view(np.uint16)
    lay.close()
    ref = O.forward(dims, arrays, threads=_oracle_threads())
    assert np.array_equal(idx, ref["idx"])
    assert np.array_equal(w.view(np.uint32), ref["w"].view(np.uint32))
    assert_out_close(dims, got, ref["out_f32"], f"cfg4 layer {layer}")
    del lay, xd, out
    _data.clear()
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", [0, 4])
def test_sixty_four_rows_equal_sixty_four_single_row_passes(layer):
    """Per-row invariance above 16 rows on a layer with the Bolt-like shared expert (width
    4096): each row of a 64-row pass of a workload-4 layer equals its own one-row pass bit for
    bit, routing included (TensorFold pull request 1038, «Per operator and row invariance»)."""
    dims, arrays = workload(4, layer=layer)
    lay, xd, out = run_gpu(dims, arrays)
    multi = out.cpu().numpy()
    idx64, w64 = lay.routing(64)
    o1 = torch.empty_like(xd[:1])
    for r in range(64):
        lay.forward(xd[r:r + 1].contiguous(), o1, 1)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy()[0], multi[r]), r
        i1, w1 = lay.routing(1)
        assert np.array_equal(i1[0], idx64[r]) and np.array_equal(w1[0].view(np.uint32), w64[r].view(np.uint32)), r
    lay.status()
    lay.close()
    del lay, xd, out
    _data.clear()
    gc.collect()
    torch.cuda.empty_cache()


def test_fp32_router_sigmoid_on_ten_million_logits():
    """The route's sigmoid of fp32 logits (the fp32 router of the non-latent fp16 layer, TensorFold
    pull request 1295, «What this changes») equals the oracle's on 10^7 random fp32 values
    and on every logit of the fp16 workload. A non-latent fp16 layer of 16 experts with every
    expert picked, no normalisation and a scale of 1 returns w = s exactly; row r's input is
    the unit vector e_r, so expert e's logit is exactly its fp32 gate weight at column r (one
    fused multiply-add by 1, the other terms add +-0). 2,442 passes of 256 rows x 16 experts
    cover the sample."""
    dims = synth.LayerDims(hidden=512, latent=0, n_experts=16, n_group=1, topk_group=1, top_k=16,
                           expert_inter=64, shared_inter=0, group_size=64, act_dtype=2,
                           router_dtype=3, has_bias=False, norm_topk=False, routed_scaling=1.0)
    rows, E = 256, 16
    per = rows * E
    arrays = synth.make_layer(dims, rows, weight_seed=7070, input_seed=7071)
    x = np.zeros((rows, dims.hidden), np.uint16)
    x[np.arange(rows), np.arange(rows)] = 0x3C00            # fp16 1.0
    arrays["x"] = x
    rng = np.random.default_rng(7072)
    n_rand = 10_000_000
    sample = np.concatenate([
        (rng.standard_normal(n_rand // 2) * 6).astype(np.float32),
        rng.uniform(-40, 40, n_rand - n_rand // 2).astype(np.float32)])
    # every fp32 logit of the fp16 workload's own pass
    dw, aw = workload(3)
    xw = O.f16_to_f32(aw["x"])
    zw = O.gate_c64(xw, aw["gate_w"]).ravel()
    sample = np.concatenate([sample, zw])
    sample = np.concatenate([sample, np.zeros((-len(sample)) % per, np.float32)])
    want = O.sigmoid(sample)
    lay = _LY().DeviceLayer(dims, arrays, rows)
    xd = _x_dev(dims, x)
    out = torch.empty_like(xd)
    wg = lay.dev["gate_w"]
    idx_d = torch.empty((rows, E), dtype=torch.int32, device="cuda")
    w_d = torch.empty((rows, E), dtype=torch.float32, device="cuda")
    from latent_mixture_experts_bf16_amd import binding as B
    passes = len(sample) // per
    for f in range(passes):
        chunk = sample[f * per:(f + 1) * per].reshape(rows, E)
        g = np.zeros((E, dims.hidden), np.float32)
        g[:, :rows] = chunk.T                                    # expert e, column r
        wg.copy_(torch.from_numpy(g))
        lay.forward(xd, out, rows)
        B.moe_latent_get_routing(lay.handle, idx_d.data_ptr(), w_d.data_ptr())
        idx = idx_d.cpu().numpy()
        wv = w_d.cpu().numpy()
        got = np.empty((rows, E), np.float32)
        got[np.arange(rows)[:, None], idx] = wv
        ref = want[f * per:(f + 1) * per].reshape(rows, E)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f
    lay.status()
    lay.close()
    assert passes * per >= 10_000_000


# ---------------------------------------------------------------------------------- the boundary

def test_rows_and_alias_refused():
    from latent_mixture_experts_bf16_amd import binding as B
    dims, arrays = workload(0, rows=4)
    lay = _LY().DeviceLayer(dims, arrays, 4)
    xd = _x_dev(dims, arrays["x"])
    out = torch.empty_like(xd)
    assert B.STATUS[B.moe_latent_forward_rc(lay.handle, 5, xd.data_ptr(), out.data_ptr())] == "MOE_ERR_ROWS"
    assert B.STATUS[B.moe_latent_forward_rc(lay.handle, 0, xd.data_ptr(), out.data_ptr())] == "MOE_ERR_ROWS"
    assert B.STATUS[B.moe_latent_forward_rc(lay.handle, 4, xd.data_ptr(), xd.data_ptr() + 16)] == "MOE_ERR_ALIAS"
    assert B.STATUS[B.moe_latent_forward_rc(lay.handle, 1, xd.data_ptr() + 2, out.data_ptr())] == "MOE_ERR_LAYOUT"
    assert B.STATUS[B.moe_latent_forward_rc(lay.handle, 1, xd.data_ptr(), out.data_ptr() + 8)] == "MOE_ERR_LAYOUT"
    lay.close()


def test_injected_allocation_failure_releases_everything():
    """A create whose n-th device allocation or runtime object fails (MOE_LATENT_FAIL_ALLOC_AT=n
    counts from the moment the variable is set: 1 the workspace, 2 the side stream, 3 and 4
    its events) returns MOE_ERR_OOM with *out NULL and leaves the live count unchanged; with
    the variable cleared a create succeeds again (TensorFold pull request 1038, review thread:
    a failed load releases what it built)."""
    from latent_mixture_experts_bf16_amd import binding as B
    dims, arrays = workload(0)
    lay = _LY().DeviceLayer(dims, arrays, 1)      # device copies of the weights
    before = B.moe_latent_live_allocations()
    for n in (1, 2, 3, 4, 5):      # the workspace, the side stream, the two events, none
        os.environ["MOE_LATENT_FAIL_ALLOC_AT"] = str(n)
        try:
            rc, h = B.moe_latent_create_rc(lay.cfg, lay.w)
        finally:
            del os.environ["MOE_LATENT_FAIL_ALLOC_AT"]
        if n <= 4:
            assert B.STATUS[rc] == "MOE_ERR_OOM", (n, rc, B.moe_latent_last_error())
        if rc:
            assert h is None, n
            assert B.moe_latent_live_allocations() == before, n
        else:
            B.moe_latent_destroy(h)
            assert B.moe_latent_live_allocations() == before, n
    rc, h = B.moe_latent_create_rc(lay.cfg, lay.w)
    assert rc == 0 and h
    B.moe_latent_destroy(h)
    assert B.moe_latent_live_allocations() == before
    lay.close()


def test_create_destroy_leaves_nothing_allocated():
    from latent_mixture_experts_bf16_amd import binding as B
    dims, arrays = workload(0)
    before = B.moe_latent_live_allocations()
    lay = _LY().DeviceLayer(dims, arrays, 8)
    assert B.moe_latent_live_allocations() > before
    lay.close()
    assert B.moe_latent_live_allocations() == before


def test_variant_zero_is_refused():
    from latent_mixture_experts_bf16_amd import binding as B
    dims, arrays = workload(0)
    lay = _LY().DeviceLayer(dims, arrays, 1)
    with pytest.raises(B.MoeError):
        B.moe_latent_set_variant(lay.handle, 0)
    with pytest.raises(B.MoeError):
        B.moe_latent_set_variant(lay.handle, 5)
    for v in (1, 2, 3, 4):
        B.moe_latent_set_variant(lay.handle, v)
    lay.close()


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_one_stream_and_two_stream_variants_agree_bitwise(cid):
    """The shared expert on the side stream (variant 2) and inside the chain's launches
    (variant 1), and a one-row pass's first launch as the front kernel (variant 1) or as
    stage-kernel items (variant 4), give the same bits: outputs, routing, and every stage."""
    dims, arrays = workload(cid)
    rows = arrays["x"].shape[0]
    res = []
    for variant in (1, 2, 3, 4):
        lay, xd, out = run_gpu(dims, arrays, variant=variant)
        st = [lay.stage(n, rows) for n in ("logits", "expert_act", "expert_out", "combine")]
        if dims.latent:
            st.append(lay.stage("latent", rows))
        if dims.shared_inter:
            st += [lay.stage("shared_act", rows), lay.stage("shared_out", rows)]
        res.append((out.cpu().numpy(), *lay.routing(rows), *st))
        lay.close()
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert np.array_equal(a, b)


def test_wrong_architecture_and_device_checks_pass_on_gfx950():
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
