"""A seeded random sweep of small prefill / decode configurations against the oracle (needs an
MI355X): batch, length (aligned and ragged), channels, d_state, io dtype, gate, resumed state,
decomposition, with per-channel parameters (tests/parity_cases.py).  Each case is a full
comparison: y and h within tolerance, the conv cache bitwise."""
import pytest
import torch

import oracle
import selective_state_space_causal_amd as ssm
from tests import parity_cases as PC
from tests.gpu_common import DEV, TAU, assert_bitwise, assert_close, dev, note, threads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("c", PC.sweep_cases(), ids=PC.sweep_id)
def test_prefill_then_decode_random(c):
    io = c["io"]
    note(f"sweep {c}")
    prm, seq, h0, c0, toks = PC.sweep_inputs(c)
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
    for t, tok in enumerate(toks):                     # three decode steps from the cache
        td = dev(tok)
        yt = ssm.decode_step(td["x"], td["dt"], td["z"] if c["gate"] else None, td["Bm"], td["Cm"], pd, h, cv)
        yr, hr, cr = oracle.decode_step(tok, prm, hr, cr, gate=c["gate"])
        assert_close(yt, yr, TAU[io], f"decode y {t}")
        assert_close(h, hr, TAU[io], f"decode h {t}")
        assert_bitwise(cv, cr, f"decode conv {t}")
