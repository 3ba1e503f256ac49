"""The forward without allocation (moe_latent_forward_static), for callers that cannot
allocate device memory: its output equals moe_latent_forward's bit for bit, on two calls in
a row whose second has fewer rows (the static workspace keeps the first call's contents), it
allocates nothing, and a pass whose workspace does not fit its array is refused."""
import numpy as np
import pytest
import torch

from latent_mixture_experts_bf16_amd import synth

pytestmark = pytest.mark.gpu


def _mods():
    from latent_mixture_experts_bf16_amd import binding as B
    from latent_mixture_experts_bf16_amd import layer as LY
    return B, LY


@pytest.mark.parametrize("cid,rows_seq", [(2, (16, 5)), (1, (1, 1)), (0, (9, 2)), (3, (4, 3))])
def test_static_forward_equals_handle_forward(cid, rows_seq):
    B, LY = _mods()
    rmax = max(rows_seq)
    dims, arrays = next(synth.workload_layers(cid, rows=rmax))
    lay = LY.DeviceLayer(dims, arrays, max_rows=rmax)
    xd = LY.to_device(arrays["x"])
    before = B.moe_latent_live_allocations()
    for rows in rows_seq:
        x = xd[:rows].contiguous()
        ref = torch.empty_like(x)
        lay.forward(x, ref, rows)
        got = torch.full_like(x, -1)
        B.moe_latent_forward_static(lay.cfg, lay.w, rows, x.data_ptr(), got.data_ptr(), 0)
        torch.cuda.synchronize()
        lay.status()
        assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy()), (cid, rows)
    assert B.moe_latent_live_allocations() == before
    lay.close()


def test_static_forward_refuses_a_workspace_beyond_its_array():
    B, LY = _mods()
    dims, arrays = next(synth.workload_layers(1, rows=1))
    lay = LY.DeviceLayer(dims, arrays, max_rows=1)
    cfg = LY.config_of(dims, 256)
    x = torch.zeros((256, dims.hidden), dtype=torch.int16, device="cuda")
    out = torch.empty_like(x)
    before = B.moe_latent_live_allocations()
    rc = B.moe_latent_forward_static_rc(cfg, lay.w, 256, x.data_ptr(), out.data_ptr(), 0)
    assert B.STATUS[rc] == "MOE_ERR_SHAPE", (rc, B.moe_latent_last_error())
    assert "static scratch" in B.moe_latent_last_error()
    rc = B.moe_latent_forward_static_rc(cfg, lay.w, 0, x.data_ptr(), out.data_ptr(), 0)
    assert B.STATUS[rc] == "MOE_ERR_ROWS"
    torch.cuda.synchronize()
    assert B.moe_latent_live_allocations() == before
    lay.close()
