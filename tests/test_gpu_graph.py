"""Decode steps captured in a HIP graph: every replay matches the eager result (needs a GPU).

Replays are interleaved with the program's own eager work (a fresh prefill that rewrites the
cache, host synchronisations), and each one is checked."""
import pytest
import torch

import selective_state_space_causal_amd as ssm
from selective_state_space_causal_amd import inputs as I
from tests.gpu_common import DEV, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,D", [(1, 2048), (3, 70)])
def test_graph_replays_match_eager(B, D):
    N, L, T = 16, 200, 8
    prm = dev(I.make_params(D, N, seed=31))
    s = dev(I.make_sequence(B, L, D, N, "bf16", seed=31))
    toks = [dev(I.make_decode_token(B, D, N, t, "bf16", seed=31)) for t in range(T)]
    h = torch.empty(B, D, N, device=DEV)
    c = torch.empty(B, D, 3, device=DEV)
    ys = torch.empty(T, B, D, dtype=torch.bfloat16, device=DEV)

    def prefill():
        ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm, h_out=h, conv_out=c)

    def loop():
        for t, tk in enumerate(toks):
            ssm.decode_step(tk["x"], tk["dt"], tk["z"], tk["Bm"], tk["Cm"], prm, h, c, y_t=ys[t])

    prefill()
    loop()
    torch.cuda.synchronize()
    ref = (ys.clone(), h.clone(), c.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prefill()
        loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    for rep in range(4):
        prefill()                     # eager work between replays resets the cache
        ys.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys.view(torch.int16), ref[0].view(torch.int16)), f"replay {rep}: y differs"
        assert torch.equal(h, ref[1]) and torch.equal(c, ref[2]), f"replay {rep}: cache differs"
