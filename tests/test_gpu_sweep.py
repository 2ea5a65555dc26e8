"""A seeded random sweep of small prefill / decode configurations against the oracle (needs an
MI355X): batch, length (aligned and ragged), channels, d_state, io dtype, gate, resumed state,
decomposition.  Each case is a full comparison: y and h within tolerance, the conv cache bitwise."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as ssm
from selective_state_space_causal_amd import inputs as I
from tests.gpu_common import DEV, TAU, assert_bitwise, assert_close, dev, f64, note, threads

pytestmark = pytest.mark.gpu


def cases(n=40, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(B=int(g.integers(1, 4)), L=int(g.choice([1, 2, 5, 8, 63, 64, 100, 511, 512, 513, 777, 1200])),
                        D=int(g.choice([1, 3, 8, 17, 40, 64, 96])), N=int(g.choice([1, 4, 8, 15, 16, 16, 16])),
                        io=str(g.choice(["f32", "bf16"])), gate=bool(g.integers(0, 2)), resume=bool(g.integers(0, 2)),
                        hint=int(g.choice([0, 0, 1, 8])), seed=1000 + i))
    return out


@pytest.mark.parametrize("c", cases(), ids=lambda c: "B{B}L{L}D{D}N{N}{io}g{gate:d}r{resume:d}h{hint}".format(**c))
def test_prefill_then_decode_random(c):
    B, L, D, N, io = c["B"], c["L"], c["D"], c["N"], c["io"]
    note(f"sweep {c}")
    prm = I.make_params(D, N, seed=c["seed"])
    prm["conv_b"] = prm["conv_b"] + 0.03
    seq = I.make_sequence(B, L, D, N, io, seed=c["seed"])
    g = torch.Generator().manual_seed(c["seed"])
    h0 = torch.randn(B, D, N, generator=g) if c["resume"] else None
    c0 = torch.randn(B, D, 3, generator=g).to(seq["x"].dtype).float() if c["resume"] else None
    s, pd = dev(seq), dev(prm)
    y, h, cv = ssm.prefill(s["x"], s["dt"], s["z"] if c["gate"] else None, s["Bm"], s["Cm"], pd,
                           h0=None if h0 is None else h0.to(DEV), conv0=None if c0 is None else c0.to(DEV),
                           chunk_hint=c["hint"])
    torch.cuda.synchronize()
    yr, hr, cr = oracle.scan(seq["x"], seq["dt"], seq["z"] if c["gate"] else None, seq["Bm"], seq["Cm"], prm["A"],
                             prm["Dskip"], prm["dt_bias"], prm["conv_w"], prm["conv_b"],
                             h0=None if h0 is None else h0.double().numpy(),
                             conv0=None if c0 is None else c0.double().numpy(), nthreads=threads())
    assert_close(y, yr, TAU[io], "y")
    assert_close(h, hr, TAU[io], "h")
    assert_bitwise(cv, cr, "conv")
    for t in range(3):                                 # three decode steps from the cache
        tok = I.make_decode_token(B, D, N, t, io, seed=c["seed"])
        td = dev(tok)
        yt = ssm.decode_step(td["x"], td["dt"], td["z"] if c["gate"] else None, td["Bm"], td["Cm"], pd, h, cv)
        yr, hr, cr = oracle.decode_step(tok, prm, hr, cr, gate=c["gate"])
        assert_close(yt, yr, TAU[io], f"decode y {t}")
        assert_close(h, hr, TAU[io], f"decode h {t}")
        assert_bitwise(cv, cr, f"decode conv {t}")
