"""The HIP path's 4-bit experts held to the two facts that pin the oracle's: the dequantised
weight is q * scale + bias (every code, nearly every positive bf16 scale), and an expert
projection's fp32 sum lies within the fp64 error bound gamma_K * sum |w x| of the exact sum
(TensorFold pull request 1038, «What's in it»: 4-bit routed experts, up, relu^2, down).

The kernels do not form q * scale + bias: they sum (128 + q) x per group of 64 inputs and
add scale * that + (bias - 128 scale) * sum x. These tests compare what they produce with
closed forms computed here in numpy, not with the oracle.
"""
import numpy as np
import pytest
import torch

from latent_mixture_experts_bf16_amd import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24   # fp32 unit roundoff


def _LY():
    from latent_mixture_experts_bf16_amd import layer as LY
    return LY


def _bf16_round(v):
    """float32 values -> the nearest bf16 (ties to even), as float32; inf stays inf."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.view(np.float32)


def _bf16(bits):
    return synth.bf16_bits_to_f32(bits)


def _codes(words, K):
    """4-bit codes of packed rows [..., K / 8] -> [..., K] (code k in bits 4 (k % 8) of word k / 8)."""
    sh = (4 * np.arange(8, dtype=np.uint32))
    return ((words[..., None] >> sh) & np.uint32(0xF)).reshape(words.shape[:-1] + (K,)).astype(np.float32)


def _dequant(q_words, scales, biases, K):
    """fp32 weights q * scale + bias (one rounding, as fp32 arithmetic does) of [N][K]."""
    q = _codes(q_words, K)
    G = K // 64
    s = _bf16(scales).astype(np.float32)[..., None]
    b = _bf16(biases).astype(np.float32)[..., None]
    w = q.reshape(q.shape[:-1] + (G, 64)) * s + b
    return w.astype(np.float32).reshape(q.shape)


def _act_f(v):
    """rnd(relu^2(rnd(v))) of fp32 pre-activations (squares past the fp32 range are inf)."""
    h = _bf16_round(v)
    r = np.maximum(h, 0.0).astype(np.float32)
    with np.errstate(over="ignore"):
        return _bf16_round(r * r)


# ------------------------------------------------------------------ every code x every scale

# One expert (expert 0 of 16, picked by every row: zero gate weights give equal scores, and
# ties go to the lower id) whose up projection has, in row n and group g, the codes 0 .. 15 at
# the group's first 16 inputs, scale s[n][g] and bias s[n][g] (so w = (q + 1) s, positive
# before relu^2). fc1 is the identity, and row 16 g + j of the input is one-hot at input
# 64 g + j: its up sum in row n is exactly (j + 1) s[n][g], and the stage holds
# rnd(relu^2(rnd((j + 1) s))). The 2048 x 16 scales run through every positive bf16 pattern
# below 2^119 (0x0001 .. 0x7AFF, 31487 of them, then from the start again); larger scales
# would overflow 128 s in the kernels' offset form, where q s + b itself is finite.
P1_DIMS = synth.LayerDims(hidden=1024, latent=1024, n_experts=16, n_group=1, topk_group=1, top_k=1,
                          expert_inter=2048, shared_inter=0, has_bias=False, routed_scaling=1.0)
SCALE_CAP = 0x7B00


def _p1_layer():
    d = P1_DIMS
    rows, H, I, D = 256, d.hidden, d.expert_inter, d.latent
    a = synth.make_layer(d, rows, weight_seed=7100, input_seed=7101)
    a["gate_w"] = np.zeros_like(a["gate_w"])
    one = np.uint16(0x3F80)
    fc1 = np.zeros((D, H), dtype=np.uint16)
    fc1[np.arange(D), np.arange(D)] = one
    a["fc1_w"] = fc1
    x = np.zeros((rows, H), dtype=np.uint16)
    r = np.arange(rows)
    x[r, 64 * (r // 16) + (r % 16)] = one
    a["x"] = x
    G = D // 64
    codes = np.zeros((I, D), dtype=np.uint32)
    for g in range(G):
        codes[:, 64 * g:64 * g + 16] = np.arange(16, dtype=np.uint32)
    words = np.zeros((I, D // 8), dtype=np.uint32)
    for i in range(8):
        words |= codes[:, i::8] << np.uint32(4 * i)
    a["up_q"][0] = words
    pat = (np.arange(I * G, dtype=np.int64) % (SCALE_CAP - 1) + 1).astype(np.uint16).reshape(I, G)
    a["up_scales"][0] = pat
    a["up_biases"][0] = pat
    # expected stage: row 16 g + j, output n -> f((j + 1) s[n][g])
    s = _bf16(pat).astype(np.float32)                                   # [I][G]
    j = (r % 16).astype(np.float32)[:, None]                            # [rows][1]
    v = (j * s[:, r // 16].T + s[:, r // 16].T).astype(np.float32)      # (j + 1) s, exact
    return d, a, _act_f(v)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_dequant_every_code_and_scale(path):
    LY = _LY()
    d, a, want = _p1_layer()
    rows = a["x"].shape[0]
    print(f"dequant P1: {path}, rows {rows}", flush=True)
    lay = LY.DeviceLayer(d, a, max_rows=rows)
    xd = LY.to_device(a["x"])
    out = torch.empty_like(xd)
    if path == "decode":
        lay.forward(xd, out)
    else:
        lay.prefill(xd, out, rows)
    torch.cuda.synchronize()
    lay.status()
    idx, _ = lay.routing(rows)
    assert (idx == 0).all()
    got = _bf16(lay.stage("expert_act", rows).reshape(rows, d.expert_inter))
    lay.close()
    bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, (len(bad), bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])


# ------------------------------------------------------------------ the fp64 bound

def _gamma(K):
    return K * U / (1.0 - K * U)


def _check_within_bound(got, w, x, f, what):
    """got[n] (bf16 stage values) against f(exact -/+ bound) for the sums w[n] . x."""
    w64, x64 = w.astype(np.float64), x.astype(np.float64)
    exact = w64 @ x64
    bound = _gamma(w.shape[1]) * (np.abs(w64) @ np.abs(x64))
    lo = f((exact - bound).astype(np.float32))
    hi = f((exact + bound).astype(np.float32))
    # float32 conversion of exact -/+ bound may round inwards: widen by one fp32 step each way
    lo = np.minimum(lo, f(np.nextafter((exact - bound).astype(np.float32), np.float32(-np.inf))))
    hi = np.maximum(hi, f(np.nextafter((exact + bound).astype(np.float32), np.float32(np.inf))))
    ok = (got >= lo) & (got <= hi)
    assert ok.all(), (what, int((~ok).sum()), np.argwhere(~ok)[:3].tolist())




@pytest.mark.parametrize("path,rows,check", [("decode", 4, (0, 1, 2, 3)), ("prefill", 64, (0, 21, 42, 63))])
def test_expert_stages_within_fp64_bound(path, rows, check):
    """The Bolt-like layer: every routed pick's up (pre-relu^2 sum over 1024 latent inputs)
    and down (sum over 2048 activations) of the checked rows lies, before its bf16 rounding,
    within gamma_K * sum |w x| of the exact sum of the fp32 dequantised weights times the
    stage's own input from the GPU."""
    LY = _LY()
    d, a = next(synth.workload_layers(1, rows=rows))
    print(f"dequant P2: {path}, rows {rows}", flush=True)
    lay = LY.DeviceLayer(d, a, max_rows=rows)
    xd = LY.to_device(a["x"])
    out = torch.empty_like(xd)
    if path == "decode":
        lay.forward(xd, out)
    else:
        lay.prefill(xd, out, rows)
    torch.cuda.synchronize()
    lay.status()
    I, D, K = d.expert_inter, d.latent, d.top_k
    idx, _ = lay.routing(rows)
    u = _bf16(lay.stage("latent", rows))
    act = _bf16(lay.stage("expert_act", rows).reshape(rows, K, I))
    eo = _bf16(lay.stage("expert_out", rows).reshape(rows, K, D))
    lay.close()
    cache = {}
    for r in check:
        for j in range(K):
            e = int(idx[r, j])
            if e not in cache:
                cache[e] = (_dequant(a["up_q"][e], a["up_scales"][e], a["up_biases"][e], D),
                            _dequant(a["down_q"][e], a["down_scales"][e], a["down_biases"][e], I))
            wu, wd = cache[e]
            _check_within_bound(act[r, j], wu, u[r], _act_f, f"{path} up row {r} pick {j}")
            _check_within_bound(eo[r, j], wd, act[r, j], _bf16_round, f"{path} down row {r} pick {j}")
