"""Captured HIP graphs (decode steps, prefill) replay to the eager result, and concurrent host
threads on their own streams get the results of the same work run alone (needs a GPU).

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
    prm = dev(I.make_params_distinct(D, N, seed=31))
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


@pytest.mark.parametrize("N,hint", [(16, 0), (16, 1), (8, 0)])
def test_prefill_graph_replays_match_eager(N, hint):
    """A captured prefill (windowed and one-lane forms) replayed on new inputs copied into its
    static buffers: each replay equals an eager prefill of those inputs, bit for bit."""
    B, L, D = 2, 777, 96
    prm = dev(I.make_params_distinct(D, N, seed=33))
    sets = [dev(I.make_sequence(B, L, D, N, "bf16", seed=33 + k)) for k in range(3)]
    refs = []
    for s in sets:
        y, h, c = ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm, chunk_hint=hint)
        refs.append((y.clone(), h.clone(), c.clone()))
    torch.cuda.synchronize()
    st = {k: v.clone() for k, v in sets[0].items()}
    y = torch.empty_like(st["x"])
    h = torch.empty(B, D, N, device=DEV)
    c = torch.empty(B, D, 3, device=DEV)

    def run():
        ssm.prefill(st["x"], st["dt"], st["z"], st["Bm"], st["Cm"], prm, y=y, h_out=h, conv_out=c, chunk_hint=hint)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(6):
        k = (rep * 2 + 1) % 3
        for name, v in sets[k].items():
            st[name].copy_(v)
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), refs[k][0].view(torch.int16)), f"replay {rep}: y differs"
        assert torch.equal(h, refs[k][1]) and torch.equal(c, refs[k][2]), f"replay {rep}: cache differs"


def test_concurrent_host_threads_and_streams():
    """Four host threads, each on its own stream with its own tensors, call prefill and decode
    at the same time (the library keeps no mutable global state; ctypes releases the GIL
    during each call): every result equals the same work run alone."""
    import threading

    N, L, D, T = 16, 300, 64, 4
    prm = dev(I.make_params_distinct(D, N, seed=35))
    work = []
    for k in range(4):
        B = 1 + k
        s = dev(I.make_sequence(B, L, D, N, "bf16", seed=35 + k))
        toks = [dev(I.make_decode_token(B, D, N, t, "bf16", seed=35 + k)) for t in range(T)]
        work.append((s, toks))

    def job(s, toks, out, stream=None):
        with torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream()):
            for _ in range(5):
                y, h, c = ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm)
                ys = [ssm.decode_step(tk["x"], tk["dt"], tk["z"], tk["Bm"], tk["Cm"], prm, h, c) for tk in toks]
            (stream or torch.cuda.current_stream()).synchronize()
        out.append((y, torch.stack(ys), h, c))

    alone = []
    for s, toks in work:
        r = []
        job(s, toks, r)
        alone.append(r[0])
    results = [[] for _ in work]
    streams = [torch.cuda.Stream() for _ in work]
    threads = [threading.Thread(target=job, args=(s, toks, results[k], streams[k])) for k, (s, toks) in enumerate(work)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    torch.cuda.synchronize()
    for k in range(len(work)):
        assert results[k], f"thread {k} produced nothing"
        for a, b in zip(results[k][0], alone[k]):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                               b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), k
