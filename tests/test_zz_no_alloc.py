"""The no-allocation Markov draft (dspark_draft_markov_noalloc) through the C
ABI against dspark_draft_markov on the same inputs: two calls in a row on one
GPU, the second with a smaller batch, every output bitwise equal."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_head_amd as D
from draft_verify_sampling_head_amd import _lib as L
from draft_verify_sampling_head_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(cfg, rnd):
    inp = synth.make_inputs(cfg, device=DEV)
    R, g = cfg.R, cfg.gamma
    outs = []
    for noalloc in (False, True):
        x = torch.full((R, g + 1), -7, dtype=torch.int32, device=DEV)
        lp = torch.full((R, g), 7.0, dtype=torch.float32, device=DEV)
        lse = torch.full((R, g), 7.0, dtype=torch.float32, device=DEV)
        if noalloc:
            flags = torch.full((1,), 0xFFFF, dtype=torch.int32, device=DEV)
            L.draft_markov_noalloc(inp["U"], inp["W1"], inp["W2t"], inp["x0"], cfg.T,
                                   cfg.philox_seed, rnd, x, lp, lse, flags=flags)
            torch.cuda.synchronize()
            assert int(flags.item()) == 0
        else:
            ws = D.workspace(R, g, cfg.V, device=DEV)
            D.draft_markov(inp["U"], inp["W1"], inp["W2t"], inp["x0"], cfg.T, cfg.philox_seed,
                           rnd, x, lp, lse, ws)
            torch.cuda.synchronize()
            assert D.get_status(ws) == 0
        outs.append((x, lp, lse))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    return outs[1][0]


@pytest.mark.parametrize("base,big,small", [
    (2, dict(R=256, gamma=16, V=129280, d=64), dict(R=40, gamma=5, V=3000, d=64)),
    (1, dict(R=64, gamma=7, V=151936, d=64), dict(R=5, gamma=3, V=1001, d=16, rank=32)),
    (2, dict(R=48, gamma=6, V=2600, d=64, rank=0), dict(R=9, gamma=4, V=700, d=16, rank=0)),
])
def test_noalloc_matches_workspace_draft(base, big, small):
    print(f"[case] noalloc base {base} {big} then {small}", flush=True)
    x1 = _pair(synth.scaled(synth.config(base), **big), 11)
    x2 = _pair(synth.scaled(synth.config(base), **small), 12)
    assert x1.shape != x2.shape


def test_noalloc_rejects_oversized_shape():
    # 12 R ceil(V/128) + 32 R ceil(V/512) beyond the 32 MiB array
    FAKE = __import__("ctypes").c_void_p(0x100000)
    code = L.load().dspark_draft_markov_noalloc(8192, 4, 151936, 0, 1.0, 0, 0, FAKE, 1, None, None,
                                                1, FAKE, FAKE, FAKE, FAKE, None, None, None)
    assert code == 3                                   # DSPARK_E_WORKSPACE
