"""The no-allocation entry point ssm_decode_fused_noalloc (include/ssm_layer.h) against the
entry point it varies, ssm_decode_fused, through the C ABI (needs an MI355X): the same kernels on
the same inputs, with the library's fixed scratch instead of a workspace, must give the same bits
-- on two calls in a row, the second with a smaller input, so that the second call runs on
scratch the first one left full."""
import pytest
import torch

import selective_state_space_causal_amd as ssm
from selective_state_space_causal_amd import _lib as L
from selective_state_space_causal_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def case(B, D, R, seed):
    N = 16
    prm = {k: v.to(DEV) for k, v in I.make_params_distinct(D, N, seed=seed).items()}
    g = torch.Generator(device=DEV).manual_seed(seed)
    bf = torch.bfloat16
    w_x = (torch.randn(R + 2 * N, D, generator=g, device=DEV) / D ** 0.5).to(bf)
    w_dt = (0.5 * torch.randn(D, R, generator=g, device=DEV) / R ** 0.5).to(bf)
    x = torch.randn(B, D, generator=g, device=DEV).to(bf)
    z = torch.randn(B, D, generator=g, device=DEV).to(bf)
    h = torch.randn(B, D, N, generator=g, device=DEV)
    c = torch.randn(B, D, 3, generator=g, device=DEV).to(bf).float()
    return prm, w_x, w_dt, x, z, h, c


@pytest.mark.parametrize("sizes", [[(64, 5120, 256), (1, 2048, 256)], [(3, 1000, 24), (2, 70, 8)]])
def test_noalloc_matches_the_workspace_entry_point(sizes):
    for i, (B, D, R) in enumerate(sizes):
        prm, w_x, w_dt, x, z, h, c = case(B, D, R, seed=100 + i)
        h1, c1, h2, c2 = h.clone(), c.clone(), h.clone(), c.clone()
        y1 = ssm.decode_fused(x, z, prm, w_x, w_dt, R, h1, c1)
        y2 = torch.empty_like(x)
        L.decode_fused_noalloc(x, z, prm, w_x, w_dt, R, h2, c2, y_t=y2)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), (B, D, R)
        assert torch.equal(h1, h2) and torch.equal(c1, c2), (B, D, R)
        assert not torch.equal(h1, h), "the step must have run"


def test_noalloc_refuses_sizes_beyond_its_scratch():
    prm, w_x, w_dt, x, z, h, c = case(200, 5120, 256, seed=7)   # 200 x 80 x 288 x 4 bytes > 16 MiB
    with pytest.raises(ssm.SsmError) as e:
        L.decode_fused_noalloc(x, z, prm, w_x, w_dt, 256, h, c, y_t=torch.empty_like(x))
    assert e.value.status == 8
