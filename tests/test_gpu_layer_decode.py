"""One rank's mixer layer, decode side, on the GPU against the oracle (needs an MI355X): a
prefill of the prompt leaves the cache, then each decoded token runs in_proj, the conv front from
the cache, x_proj, dt_proj, the decode step and out_proj -- as separate calls or with the
middle four fused (ssm_decode_fused) -- and every step's out partial, state and conv window are
compared with the oracle's composition of the same stages (oracle/proj.py layer_decode_step)."""
import numpy as np
import pytest
import torch

import selective_state_space_causal_amd as ssm
from oracle import proj as P
from selective_state_space_causal_amd import inputs as I
from selective_state_space_causal_amd import layer
from tests.gpu_common import DEV, assert_close, f64, note, threads

pytestmark = pytest.mark.gpu
TAU = 2e-2      # bf16 io, as for the layer's prefill
T_STEPS = 8


@pytest.fixture(scope="module")
def pj():
    p = ssm.Projector(DEV)
    yield p
    p.close()


def weights_on_device(wts):
    wd = {k: v.to(DEV) for k, v in wts.items() if k not in ("in_x", "in_z", "x_dt", "x_B", "x_C")}
    D = wts["in_x"].shape[0]
    R, N = wts["x_dt"].shape[0], wts["x_B"].shape[0]
    wd["in_x"], wd["in_z"] = wd["in_xz"][:D], wd["in_xz"][D:]
    wd["x_dt"], wd["x_B"], wd["x_C"] = wd["x_all"][:R], wd["x_all"][R:R + N], wd["x_all"][R + N:]
    return wd


def check_steps(name, wts, wd, prm, pd, hidden_all, L, h, c, h_ref, c_ref, pj, fused):
    """T_STEPS decode steps on tokens L, L+1, ... of hidden_all, GPU against oracle."""
    for t in range(T_STEPS):
        ht = hidden_all[:, L + t].contiguous()
        out = layer.mixer_decode_step(ht.to(DEV), wd, pd, pj, h, c, fused=fused)
        torch.cuda.synchronize()
        out_ref, _, h_ref, c_ref = P.layer_decode_step(ht, wts, prm, h_ref, c_ref, "bf16")
        assert_close(out, out_ref, TAU, f"{name} out step {t}", step=t, exact_inputs=False)
        assert_close(h, h_ref, TAU, f"{name} h step {t}", step=t, exact_inputs=False)
        # the conv window holds in_proj outputs, which the GPU's fp32 GEMM may round to another
        # bf16 value than the oracle's fp64 sum: held to the same bar
        assert_close(c, c_ref, TAU, f"{name} conv step {t}", step=t, exact_inputs=False)
    return h_ref, c_ref


@pytest.mark.parametrize("rows", [1, 2])
@pytest.mark.parametrize("fused", [False, True])
def test_layer_small_decode_matches_oracle(pj, rows, fused):
    """layer_small: a GPU prefill of 200 tokens (against the oracle's), then 8 decode steps."""
    w = I.LAYERS["layer_small"]
    note(f"layer_small decode rows={rows} fused={fused}")
    prm = I.make_params_distinct(w.d_inner, w.d_state)
    wts = I.make_proj_weights(w.d_model, w.d_inner, w.dt_rank, w.d_state, w.io)
    hidden_all = I.make_hidden(w.batch, w.seqlen + T_STEPS, w.d_model, w.io)[:rows].contiguous()
    L = w.seqlen
    wd = weights_on_device(wts)
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    _, h, c = layer.mixer_prefill(hidden_all[:, :L].contiguous().to(DEV), wd, pd, pj)
    _, h_ref, c_ref = P.layer_prefill(hidden_all[:, :L], wts, prm, "bf16", nthreads=threads())
    torch.cuda.synchronize()
    assert_close(h, h_ref, TAU, "layer_small prefill h", exact_inputs=False)
    check_steps("layer_small", wts, wd, prm, pd, hidden_all, L, h, c, h_ref, c_ref, pj, fused)


@pytest.mark.parametrize("fused", [False, True])
def test_layer7b_decode_from_a_cache(pj, fused):
    """The 7B-class layer (d_model 4096, d_inner 2048 of 8192, dt_rank 256) at full size: 8
    decode steps from a random cache, every output against the oracle."""
    w = I.LAYERS["layer7b"]
    note(f"layer7b decode fused={fused}")
    prm = I.make_params_distinct(w.d_inner, w.d_state)
    wts = I.make_proj_weights(w.d_model, w.d_inner, w.dt_rank, w.d_state, w.io)
    hidden_all = I.make_hidden(1, T_STEPS, w.d_model, w.io)
    wd = weights_on_device(wts)
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    g = torch.Generator().manual_seed(7)
    h0 = torch.randn(1, w.d_inner, w.d_state, generator=g)
    c0 = torch.randn(1, w.d_inner, 3, generator=g).to(torch.bfloat16).float()
    h, c = h0.to(DEV), c0.to(DEV)
    check_steps("layer7b", wts, wd, prm, pd, hidden_all, 0, h, c, f64(h0), f64(c0), pj, fused)


@pytest.mark.parametrize("B,DM,D,R", [(3, 64, 200, 64), (2, 48, 196, 24)])
@pytest.mark.parametrize("fused", [False, True])
def test_ragged_layer_decode_matches_oracle(pj, B, DM, D, R, fused):
    """Channel counts that leave a ragged last block in both fused kernels (200 and 196 channels:
    blocks of 64 in xproj_partial, of 32 in dt_decode), 196 also not a whole number of 16-byte
    pieces and rank 24 not a multiple of 32 (the element-wise forms of both kernels), several batch
    rows: 8 decode steps from a random cache, every output against the oracle."""
    N = 16
    note(f"ragged layer decode B={B} d_model={DM} d_inner={D} rank={R} fused={fused}")
    prm = I.make_params_distinct(D, N, seed=D + R)
    wts = I.make_proj_weights(DM, D, R, N, "bf16", seed=D)
    hidden_all = I.make_hidden(B, T_STEPS, DM, "bf16", seed=R)
    wd = weights_on_device(wts)
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    g = torch.Generator().manual_seed(D * R)
    h0 = torch.randn(B, D, N, generator=g)
    c0 = torch.randn(B, D, 3, generator=g).to(torch.bfloat16).float()
    h, c = h0.to(DEV), c0.to(DEV)
    check_steps(f"ragged D={D}", wts, wd, prm, pd, hidden_all, 0, h, c, f64(h0), f64(c0), pj, fused)


def test_fused_and_unfused_decode_agree(pj):
    """The fused stages round at the same points as the separate calls, so from the same cache
    the two paths agree to within the fp32 summation order (which can move a rounded
    intermediate by one bf16 ulp): y within 2^-6 relative, h within 1e-3."""
    w = I.LAYERS["layer7b"]
    prm = I.make_params_distinct(w.d_inner, w.d_state)
    wts = I.make_proj_weights(w.d_model, w.d_inner, w.dt_rank, w.d_state, w.io, device=DEV)
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    g = torch.Generator(device=DEV).manual_seed(9)
    h = torch.randn(1, w.d_inner, w.d_state, generator=g, device=DEV)
    c = torch.randn(1, w.d_inner, 3, generator=g, device=DEV).to(torch.bfloat16).float()
    h2, c2 = h.clone(), c.clone()
    hidden = I.make_hidden(1, 4, w.d_model, w.io, device=DEV)
    for t in range(4):
        bu = layer.alloc_decode_buffers(hidden[:, t], wts, w.d_state, False)
        bf = layer.alloc_decode_buffers(hidden[:, t], wts, w.d_state, True)
        layer.mixer_decode_step(hidden[:, t].contiguous(), wts, pd, pj, h, c, fused=False, bufs=bu)
        layer.mixer_decode_step(hidden[:, t].contiguous(), wts, pd, pj, h2, c2, fused=True, bufs=bf)
        torch.cuda.synchronize()
        yu, yf = f64(bu["y"]), f64(bf["y"])
        assert np.all(np.abs(yu - yf) <= 2.0 ** -6 * (1 + np.abs(yu))), t
        assert np.all(np.abs(f64(h) - f64(h2)) <= 1e-3 * (1 + np.abs(f64(h)))), t
        assert torch.equal(c, c2), t   # both paths run the same in_proj GEMM on the same input


@pytest.mark.parametrize("fused", [False, True])
def test_decode_graph_replays_match_eager(pj, fused):
    """Four decode steps of the 7B-class layer captured in one HIP graph (the GEMM library calls
    included) and replayed from the same cache, with eager work in between: every replay equals
    the eager steps bit for bit."""
    w = I.LAYERS["layer7b"]
    prm = I.make_params_distinct(w.d_inner, w.d_state)
    wts = I.make_proj_weights(w.d_model, w.d_inner, w.dt_rank, w.d_state, w.io, device=DEV)
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    g = torch.Generator(device=DEV).manual_seed(11)
    h0 = torch.randn(1, w.d_inner, w.d_state, generator=g, device=DEV)
    c0 = torch.randn(1, w.d_inner, 3, generator=g, device=DEV).to(torch.bfloat16).float()
    hidden = I.make_hidden(1, 4, w.d_model, w.io, device=DEV)
    toks = [hidden[:, t].contiguous() for t in range(4)]
    h, c = h0.clone(), c0.clone()
    bufs = layer.alloc_decode_buffers(toks[0], wts, w.d_state, fused)
    outs = torch.empty(4, 1, w.d_model, dtype=hidden.dtype, device=DEV)

    def steps():
        for t, ht in enumerate(toks):
            for _, call in layer.decode_stages(ht, wts, pd, pj, h, c, bufs, fused):
                call()
            outs[t].copy_(bufs["out"].view(1, -1))

    steps()
    torch.cuda.synchronize()
    ref = (outs.clone(), h.clone(), c.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.copy_(h0)
        c.copy_(c0)
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    for rep in range(4):
        h.copy_(h0)                      # eager work between replays restores the cache
        c.copy_(c0)
        outs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs.view(torch.int16), ref[0].view(torch.int16)), f"replay {rep}: out differs"
        assert torch.equal(h, ref[1]) and torch.equal(c, ref[2]), f"replay {rep}: cache differs"
