"""Seeded synthetic inputs: determinism, distributions, parameter recipe (no GPU)."""
import numpy as np
import torch
import torch.nn.functional as F

from selective_state_space_causal_amd import inputs as I


def test_deterministic_and_independent_streams():
    a = I.make_sequence(2, 40, 8, 4, "bf16", seed=0)
    b = I.make_sequence(2, 40, 8, 4, "bf16", seed=0)
    c = I.make_sequence(2, 40, 8, 4, "bf16", seed=1)
    for k in a:
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))
        assert not torch.equal(a[k].float(), c[k].float())
    assert not torch.equal(a["x"].float(), a["z"].float())
    t0 = I.make_decode_token(2, 8, 4, 0)
    t1 = I.make_decode_token(2, 8, 4, 1)
    assert t0["x"].shape == (2, 8) and t0["Bm"].shape == (2, 4)
    assert not torch.equal(t0["x"].float(), t1["x"].float())


def test_moments():
    s = I.make_sequence(1, 4096, 64, 16, "f32", seed=3)
    for k, std in (("x", 1.0), ("z", 1.0), ("Bm", 1.0), ("Cm", 1.0), ("dt", 0.5)):
        v = s[k].double()
        assert abs(v.mean().item()) < 0.02 * std * 4, k
        assert abs(v.std().item() / std - 1.0) < 0.02, k


def test_bf16_is_round_to_nearest_even():
    s32 = I.make_sequence(1, 64, 16, 4, "f32", seed=5)
    s16 = I.make_sequence(1, 64, 16, 4, "bf16", seed=5)
    x = s32["x"].numpy().view(np.uint32).astype(np.uint64)
    lsb = (x >> 16) & 1
    rne = ((x + 0x7FFF + lsb) >> 16).astype(np.uint16)
    assert np.array_equal(rne, s16["x"].view(torch.int16).numpy().view(np.uint16))


def test_params_recipe():
    for lo, hi in ((1e-3, 1e-1), (1e-4, 1e-1)):
        p = I.make_params(512, 16, seed=0, dt_range=(lo, hi))
        dt0 = F.softplus(p["dt_bias"].double(), threshold=1e9)
        assert dt0.min() >= lo * 0.999 and dt0.max() <= hi * 1.001
        # log-uniform: the mean of log(dt0) sits mid-range
        assert abs(torch.log(dt0).mean().item() - 0.5 * (np.log(lo) + np.log(hi))) < 0.3
        assert torch.equal(p["A"], -torch.arange(1, 17, dtype=torch.float32).expand(512, 16))
        assert torch.all(p["Dskip"] == 1) and torch.all(p["conv_b"] == 0)
        assert p["conv_w"].abs().max() <= 0.5 and p["conv_w"].shape == (512, 4)
        for v in p.values():
            assert v.dtype == torch.float32 and v.is_contiguous()


def test_workloads_table():
    w = I.WORKLOADS
    assert (w["tiny"].batch, w["tiny"].seqlen, w["tiny"].d_inner, w["tiny"].d_state, w["tiny"].io) == (1, 64, 16, 4, "f32")
    assert (w["slice7b"].seqlen, w["slice7b"].d_inner, w["slice7b"].decode_steps) == (32768, 2048, 128)
    assert w["long64k"].dt_range == (1e-4, 1e-1)
