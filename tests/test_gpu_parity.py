"""GPU parity: every stage of the round through the C ABI against the oracle.

Small cases span several chunks, several 32-row MFMA tiles and ragged tails
(vocabularies that are not multiples of the 128-entry chunk, of 8, or below
one chunk; row counts that are not multiples of 32).  Full-size cases run the
benchmark's configurations and check a sample of requests one by one plus the
whole schedule and both packs.
"""
import os

import numpy as np
import pytest
import torch

import draft_verify_sampling_head_amd as D
from draft_verify_sampling_head_amd import round as RD
from draft_verify_sampling_head_amd import synth
from oracle import parity as PC

pytestmark = pytest.mark.gpu
DEV = "cuda"


def n(t):
    return t.detach().cpu().numpy()


def f(t):
    return None if t is None else t.detach().float().cpu().numpy()


def to_dev(inp):
    return {k: (v.to(DEV) if torch.is_tensor(v) and k != "hard" else v) for k, v in inp.items()}


THREADS = max(1, min(16, os.cpu_count() or 1))   # host threads for the oracle's request rows


def run_and_check(cfg, inp_cpu=None, layout=1, rnd=0, reqs=None, inp_dev=None, sts=None):
    """Run a full round on the GPU; check all stages (on `reqs` if given)."""
    print(f"[case] {cfg.name} R={cfg.R} g={cfg.gamma} V={cfg.V} r={cfg.rank} T={cfg.T} "
          f"layout={layout} reqs={None if reqs is None else list(reqs)}", flush=True)
    if inp_dev is None:
        inp_dev = to_dev(inp_cpu)
    g = dict(inp_dev)
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    if layout == 0:
        # the target model would produce rows in verify order: run the first
        # four stages, gather the packed target rows, then verify
        RD.run_round(g, buf, cfg.T, cfg.philox_seed, rnd, scheduler=cfg.scheduler, layout=1,
                     sts_T=sts)
        torch.cuda.synchronize()
        N = int(n(buf.N)[0])
        packed = g["target"][buf.marker_req[:N].long(), buf.marker_pos[:N].long()].contiguous()
        g["target"] = packed
        RD.run_round(g, buf, cfg.T, cfg.philox_seed, rnd, scheduler=cfg.scheduler, layout=0,
                     sts_T=sts)
    else:
        RD.run_round(g, buf, cfg.T, cfg.philox_seed, rnd, scheduler=cfg.scheduler, layout=1,
                     sts_T=sts)
    torch.cuda.synchronize()
    status = D.get_status(buf.ws)
    rep = PC.Report()
    sel = slice(None) if reqs is None else np.asarray(reqs)
    src = inp_cpu if inp_cpu is not None else None

    def host(key, rows=True):
        t = (src[key] if src is not None else inp_dev[key])
        if t is None:
            return None
        if rows and reqs is not None:
            t = t[torch.as_tensor(np.asarray(reqs), device=t.device)]
        return f(t) if t.is_floating_point() else n(t)

    U, tgt, h = host("U"), host("target"), host("h")
    W1, W2t, w = host("W1", False), host("W2t", False), host("w", False)
    x0 = host("x0")
    x = n(buf.x)[sel]
    rq = None if reqs is None else np.asarray(reqs, np.int32)
    lp_o, lse_o = PC.check_draft(rep, U, W1, W2t, x0, cfg.T, cfg.philox_seed, rnd, x,
                                 n(buf.logp_d)[sel], n(buf.lse_d)[sel], rq, threads=THREADS)
    stsn = None if sts is None else n(sts)
    PC.check_confidence(rep, h, W1, w, x, n(buf.c)[sel], stsn)
    PC.check_schedule(rep, n(buf.c), n(inp_dev["sps"]), cfg.scheduler, n(buf.ell), n(buf.a),
                      n(buf.N)[0], n(buf.theta)[0])
    PC.check_pack(rep, n(buf.x), n(buf.ell) + 1, n(buf.cu), n(buf.flat), n(buf.marker_req),
                  n(buf.marker_pos), n(buf.N)[0], "verify batch")
    PC.check_verify(rep, n(buf.ell)[sel], None, tgt, 1, x, lp_o, lse_o, U, W1, W2t, cfg.T,
                    cfg.philox_seed, rnd, n(buf.m)[sel], n(buf.tau)[sel], n(buf.emitted)[sel],
                    n(buf.next_anchor)[sel], n(buf.logp_t)[sel], rq, threads=THREADS)
    PC.check_pack(rep, n(buf.emitted), n(buf.tau), n(buf.cu_out), n(buf.flat_out), None, None,
                  n(buf.N_out)[0], "emitted")
    print(f"  {rep.summary()} status={status} sum_ell={int(n(buf.ell).sum())} "
          f"sum_m={int(n(buf.m).sum())}", flush=True)
    assert status == 0, f"device flags {status}"
    assert rep.ok(), rep.summary()
    return buf, rep


# ------------------------------------------------------------- small cases
SMALL = [
    # (base config, overrides)
    (0, {}),                                                            # config 0 itself
    (2, dict(R=40, gamma=5, V=3000, d=256)),                             # bf16, rank 256
    (2, dict(R=33, gamma=4, V=2000, d=64, rank=64)),
    (2, dict(R=9, gamma=3, V=1500, d=64, rank=16)),
    (2, dict(R=37, gamma=6, V=2600, d=64, rank=0)),                      # DFlash case
    (2, dict(R=35, gamma=4, V=2000, d=64, rank=512)),
    (1, dict(R=33, gamma=7, V=5000, d=128)),                             # greedy, no scheduler
    (1, dict(R=20, gamma=5, V=3001, d=96, rank=0)),
    (3, dict(R=70, gamma=6, V=2500, d=64)),                              # T = 0.7, hard/easy mix
    (2, dict(R=5, gamma=3, V=100, d=32)),                                # one chunk
    (2, dict(R=6, gamma=4, V=1001, d=40, rank=32)),                      # rows not 16-byte aligned
    (2, dict(R=1, gamma=1, V=700, d=16)),
    (2, dict(R=12, gamma=32, V=900, d=32, rank=32)),                     # longest block
    (2, dict(R=24, gamma=4, V=1800, d=64, T=0.3)),
    (2, dict(R=24, gamma=4, V=1800, d=64, T=2.0, scheduler=False)),
    (2, dict(R=300, gamma=3, V=2048, d=32, rank=128)),                   # two 256-row groups
    (1, dict(R=260, gamma=3, V=4096, d=32, rank=64)),                    # greedy, two row groups
    # rows of more than 4096 chunks: verify statistics outside LDS (three launches)
    (2, dict(R=3, gamma=2, V=600_001, d=32, rank=16)),
    (1, dict(R=2, gamma=2, V=530_000, d=32, rank=0)),
]


@pytest.mark.parametrize("base,over", SMALL, ids=[f"cfg{b}-{i}" for i, (b, _) in enumerate(SMALL)])
def test_small_round_parity(base, over):
    cfg = synth.scaled(synth.config(base), **over) if over else synth.config(base)
    inp = synth.make_inputs(cfg, device="cpu")
    run_and_check(cfg, inp)


def test_packed_target_layout():
    cfg = synth.scaled(synth.config(2), R=30, gamma=5, V=2100, d=64)
    inp = synth.make_inputs(cfg, device="cpu")
    run_and_check(cfg, inp, layout=0)


ROUND_ONE_CALL = [
    (0, {}, True),
    (2, dict(R=40, gamma=5, V=3000, d=256), True),
    (1, dict(R=33, gamma=7, V=5000, d=128), False),                  # greedy, static block
    (2, dict(R=37, gamma=6, V=2600, d=64, rank=0), "async"),
    (2, dict(R=300, gamma=3, V=2048, d=32, rank=128), True),
]


@pytest.mark.parametrize("base,over,sched", ROUND_ONE_CALL,
                         ids=[f"cfg{b}-{i}" for i, (b, _, _) in enumerate(ROUND_ONE_CALL)])
def test_round_markov_one_call_matches_calls(base, over, sched):
    """dspark_round_markov enqueues the same kernels in the same order as the
    five calls made one by one: every output is bit-identical, over two rounds
    (with the asynchronous scheduler each run keeps its own capacity ring),
    and the first round also matches the oracle."""
    cfg = synth.scaled(synth.config(base), **over)
    print(f"[case] one-call round {cfg.name} R={cfg.R} g={cfg.gamma} V={cfg.V} r={cfg.rank} "
          f"sched={sched}", flush=True)
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    outs = []
    for single in (False, True):
        buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
        ring = RD.CapacityRing(cfg.R, cfg.gamma, inp["sps"].numel() - 1, device=DEV)
        per_round = []
        for rnd in range(2):
            D.clear_status(buf.ws)
            RD.run_round(inp, buf, cfg.T, cfg.philox_seed, rnd, scheduler=sched, ring=ring,
                         single_call=single)
            torch.cuda.synchronize()
            assert D.get_status(buf.ws) == 0
            per_round.append({k: n(getattr(buf, k)).copy() for k in (
                "x", "logp_d", "lse_d", "c", "ell", "a", "N", "theta", "cu", "flat",
                "marker_req", "marker_pos", "m", "tau", "emitted", "next_anchor", "logp_t",
                "cu_out", "flat_out", "N_out")})
        outs.append(per_round)
    for rnd in range(2):
        for k, v in outs[0][rnd].items():
            w = outs[1][rnd][k]
            if k in ("flat", "marker_req", "marker_pos"):
                N = int(outs[0][rnd]["N"][0])
                v, w = v[:N], w[:N]
            if k == "flat_out":
                N = int(outs[0][rnd]["N_out"][0])
                v, w = v[:N], w[:N]
            assert np.array_equal(v.view(np.uint8), w.view(np.uint8)), (rnd, k)
    if sched is not True:
        return
    rep = PC.Report()
    inc = synth.make_inputs(cfg, device="cpu")
    x, r0 = outs[1][0]["x"], outs[1][0]
    lp, lse = PC.check_draft(rep, f(inc["U"]), f(inc["W1"]), f(inc["W2t"]), n(inc["x0"]), cfg.T,
                             cfg.philox_seed, 0, x, r0["logp_d"], r0["lse_d"], None,
                             threads=THREADS)
    PC.check_verify(rep, r0["ell"], None, f(inc["target"]), 1, x, lp, lse, f(inc["U"]),
                    f(inc["W1"]), f(inc["W2t"]), cfg.T, cfg.philox_seed, 0, r0["m"], r0["tau"],
                    r0["emitted"], r0["next_anchor"], r0["logp_t"], None, threads=THREADS)
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("single", [False, True], ids=["calls", "one_call"])
def test_round_replays_in_a_hip_graph(single):
    """A whole round captured in a HIP graph (torch.cuda.graph) and replayed
    several times, with eager rounds on other buffers in between: every
    replay rewrites every output bit-identically to the eager round.  The
    verify's cross-workgroup epoch lives on the device, so each replay gets a
    new one (an epoch frozen into the captured arguments would let replays
    after the first count rows before their counters were cleared)."""
    cfg = synth.scaled(synth.config(2), R=40, gamma=5, V=3000, d=64)
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    keys = ("x", "logp_d", "lse_d", "c", "ell", "N", "m", "tau", "emitted", "next_anchor",
            "cu_out", "N_out")
    ref_buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    RD.run_round(inp, ref_buf, cfg.T, cfg.philox_seed, 3, scheduler=True)
    torch.cuda.synchronize()
    assert D.get_status(ref_buf.ws) == 0
    ref = {k: n(getattr(ref_buf, k)).copy() for k in keys}
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up outside the capture
        RD.run_round(inp, buf, cfg.T, cfg.philox_seed, 3, scheduler=True, single_call=single)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        RD.run_round(inp, buf, cfg.T, cfg.philox_seed, 3, scheduler=True, single_call=single)
    torch.cuda.synchronize()
    for rep in range(4):
        for k in ("x", "m", "tau", "emitted", "next_anchor", "cu_out", "ell"):
            getattr(buf, k).fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert D.get_status(buf.ws) == 0, rep
        for k in keys:
            assert np.array_equal(n(getattr(buf, k)).view(np.uint8), ref[k].view(np.uint8)), (rep, k)
        N_out = int(ref["N_out"][0])
        assert np.array_equal(n(buf.flat_out)[:N_out], n(ref_buf.flat_out)[:N_out]), rep
        # eager work on other buffers between replays
        RD.run_round(inp, ref_buf, cfg.T, cfg.philox_seed, 3, scheduler=True)
        torch.cuda.synchronize()


def test_fp32_logits_bf16_weights():
    cfg = synth.scaled(synth.config(2), R=34, gamma=4, V=1900, d=64)
    inp = synth.make_inputs(cfg, device="cpu")
    inp["U"] = inp["U"].float()
    inp["target"] = inp["target"].float()
    inp["h"] = inp["h"].float()
    run_and_check(cfg, inp)


def test_sts_temperatures_and_rounds():
    cfg = synth.scaled(synth.config(2), R=16, gamma=4, V=1300, d=64)
    inp = synth.make_inputs(cfg, device="cpu")
    sts = torch.tensor([1.0, 1.5, 0.7, 2.0], dtype=torch.float32, device=DEV)
    b1, _ = run_and_check(cfg, inp, rnd=5, sts=sts)
    b2, _ = run_and_check(cfg, inp, rnd=6, sts=sts)
    assert not torch.equal(b1.x, b2.x)   # the round counter changes the stream


def test_determinism_bitwise():
    cfg = synth.scaled(synth.config(2), R=64, gamma=6, V=4000, d=64)
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    outs = []
    for _ in range(2):
        buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
        RD.run_round(inp, buf, cfg.T, 0, 0, scheduler=True)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (buf.x, buf.logp_d, buf.lse_d, buf.c, buf.ell, buf.m,
                                           buf.emitted, buf.flat_out)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_nonfinite_logits_are_flagged():
    cfg = synth.scaled(synth.config(2), R=4, gamma=2, V=600, d=16)
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    inp["U"][1, 0, 77] = float("nan")
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    D.clear_status(buf.ws)
    RD.run_round(inp, buf, cfg.T, 0, 0)
    torch.cuda.synchronize()
    assert D.get_status(buf.ws) & D._lib.FLAG_NONFINITE


@pytest.fixture
def switch():
    """Set library test switches (dspark_set_switch) for one test; restored after."""
    saved = {}

    def set_to(key, value):
        prev = D._lib.set_switch(key, value)
        saved.setdefault(key, prev)
    yield set_to
    for key, value in saved.items():
        D._lib.set_switch(key, value)


@pytest.fixture
def draft_schedule(switch):
    """None: the default persistent kernel (one grid barrier per step, plain
    launch); "coop": the same kernel in a cooperative launch; "pipe": the
    pipelined persistent kernel; "steps": one launch per step."""
    def set_to(name):
        switch(D._lib.SWITCH_FORCE_PER_STEP, 1 if name == "steps" else 0)
        switch(D._lib.SWITCH_DRAFT_KERNEL, 1 if name == "pipe" else 0)
        switch(D._lib.SWITCH_PERSIST_LAUNCH, 1 if name == "coop" else 0)
    return set_to


@pytest.mark.parametrize("base,rank,R", [(2, 256, 45), (1, 128, 45), (3, 64, 45), (2, 256, 200),
                                         (3, 128, 300), (2, 64, 1)])
def test_draft_schedules_all_match_oracle(draft_schedule, base, rank, R):
    # the persistent kernels (grid barrier, pipelined) and the per-step
    # schedule of the draft on the same inputs: each must match the oracle.
    # R = 45, 200, 300: one, two and three request groups of 128 with ragged
    # last groups (odd tile counts padded to even)
    cfg = synth.scaled(synth.config(base), R=R, gamma=4, V=3072, d=32, rank=rank)
    inp = synth.make_inputs(cfg, device="cpu")
    xs = []
    for name in (None, "coop", "pipe", "steps"):
        draft_schedule(name)
        buf, _ = run_and_check(cfg, inp)
        xs.append(n(buf.x))
    # decisions agree except where the oracle flags a near-tie
    for other in xs[1:]:
        assert (xs[0] != other).mean() <= 0.01


@pytest.mark.parametrize("kernel", [0, 1], ids=["barrier", "pipe"])
def test_barrier_wait_is_bounded(switch, kernel):
    # a one-poll limit on the persistent draft's cross-workgroup waits: the
    # launch must still finish; a wait that gave up is reported through the
    # status word
    switch(D._lib.SWITCH_DRAFT_KERNEL, kernel)
    switch(D._lib.SWITCH_BARRIER_SPINS, 1)
    cfg = synth.scaled(synth.config(2), R=64, gamma=4, V=4096, d=32)
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    D.clear_status(buf.ws)
    D._lib.draft_markov(inp["U"], inp["W1"], inp["W2t"], inp["x0"], cfg.T, 0, 0, buf.x,
                        buf.logp_d, buf.lse_d, buf.ws)
    torch.cuda.synchronize()
    st = D.get_status(buf.ws)
    x = n(buf.x)
    assert ((x >= 0) & (x < cfg.V)).all()
    if not st & D._lib.FLAG_BARRIER:
        # every barrier happened to complete within one poll: results are valid
        rep = PC.Report()
        f32 = lambda t: t.float().cpu().numpy()
        PC.check_draft(rep, f32(inp["U"]), f32(inp["W1"]), f32(inp["W2t"]), n(inp["x0"]), cfg.T, 0,
                       0, x, n(buf.logp_d), n(buf.lse_d), None)
        assert rep.ok(), rep.summary()
    switch(D._lib.SWITCH_BARRIER_SPINS, 0)
    D.clear_status(buf.ws)
    D._lib.draft_markov(inp["U"], inp["W1"], inp["W2t"], inp["x0"], cfg.T, 0, 0, buf.x,
                        buf.logp_d, buf.lse_d, buf.ws)
    torch.cuda.synchronize()
    assert D.get_status(buf.ws) == 0


def test_rounds_with_more_slices_than_compute_units():
    """V = 151936: 297 vocabulary slices of 512, more than the compute units
    (the draft then takes the per-step schedule): several rounds in a row
    finish with a clean status and match the oracle."""
    cfg = synth.scaled(synth.config(3), R=24, gamma=4, d=64)
    inp = synth.make_inputs(cfg, device="cpu")
    for rnd in range(3):
        run_and_check(cfg, inp, rnd=rnd)


@pytest.mark.parametrize("T", [1.0, 0.0], ids=["sampled", "greedy"])
def test_verify_epoch_wait_is_bounded(switch, T):
    # a one-poll limit on the fused verify's wait for its cleared counters:
    # the launch must still finish; a wait that gave up is reported through
    # the status word, and otherwise the outputs equal those of a run with
    # the default limit
    cfg = synth.scaled(synth.config(2), R=64, gamma=4, V=4096, d=32, T=T)
    inp = to_dev(synth.make_inputs(cfg, device="cpu"))
    outs = []
    for spins in (0, 1, 0):
        switch(D._lib.SWITCH_BARRIER_SPINS, spins)
        buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
        D.clear_status(buf.ws)
        RD.run_round(inp, buf, cfg.T, cfg.philox_seed, 0, scheduler=cfg.scheduler)
        torch.cuda.synchronize()
        st = D.get_status(buf.ws)
        outs.append((st, n(buf.m), n(buf.tau), n(buf.emitted), n(buf.next_anchor)))
    assert outs[0][0] == 0 and outs[2][0] == 0
    for a, b in zip(outs[0][1:], outs[2][1:]):
        np.testing.assert_array_equal(a, b)
    if not outs[1][0] & D._lib.FLAG_BARRIER:
        for a, b in zip(outs[0][1:], outs[1][1:]):
            np.testing.assert_array_equal(a, b)


# -------------------------------------------------------- stage: scheduler
def _sched_case(c, sps, enabled=True, N_max=None):
    R, g = c.shape
    cd = torch.as_tensor(c, device=DEV)
    spsd = torch.as_tensor(sps, device=DEV)
    ell = torch.empty(R, dtype=torch.int32, device=DEV)
    a = torch.empty(R, g, dtype=torch.float32, device=DEV)
    N = torch.empty(1, dtype=torch.int32, device=DEV)
    th = torch.empty(1, dtype=torch.float64, device=DEV)
    D.prefix_schedule(cd, spsd, ell, enabled=enabled, N_max=N_max, a=a, N_out=N, theta_best=th)
    torch.cuda.synchronize()
    import oracle as O
    e, ao, No, tho, _ = O.prefix_schedule(c, sps, N_max=N_max, enabled=enabled)
    np.testing.assert_array_equal(n(ell), e)
    np.testing.assert_array_equal(n(a).view(np.uint32), ao.view(np.uint32))
    assert int(n(N)[0]) == No
    assert float(n(th)[0]) == tho


def test_scheduler_bitexact_random_and_ties():
    rng = np.random.default_rng(0)
    for it in range(40):
        R, g = int(rng.integers(1, 300)), int(rng.integers(1, 33))
        if R * g > 16384:
            continue
        c = rng.uniform(0, 1, (R, g)).astype(np.float32)
        if it % 3 == 0:
            c = rng.choice(np.array([0, 0.25, 0.5, 0.75, 1.0], np.float32), (R, g))
        if it % 5 == 0:
            c[:, :] = 1.0
        B = np.arange(R * (g + 1) + 1, dtype=np.float64)
        sps = [1.0 / (0.020 + 5e-5 * B), 1.0 / (0.02 + 0.002 * B),
               1.0 / (0.015 + 4e-5 * B + 0.003 * (B // 7))][it % 3]
        _sched_case(c, sps, N_max=None if it % 4 else int(rng.integers(R, R * (g + 1) + 1)))
        _sched_case(c, sps, enabled=False)


def test_scheduler_stress_size():
    # 1024 requests x 15 positions with the tabulated, stepped SPS curve
    cfg = synth.config(3)
    rng = np.random.default_rng(3)
    z = rng.normal(0, 3.2, (cfg.R, cfg.gamma))
    c = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    sps = synth.sps_table(cfg, cfg.R * (cfg.gamma + 1)).numpy()
    _sched_case(c, sps)
    c2 = rng.uniform(0.97, 1.0, (1024, 16)).astype(np.float32)
    B = np.arange(1024 * 17 + 1, dtype=np.float64)
    _sched_case(c2, 1.0 / (0.020 + 5e-6 * B))
    # runs padded to 32 positions would exceed the key buffer: packed keys and
    # the bitonic network instead of the run merge
    for R, g in [(600, 17), (900, 17)]:
        c3 = rng.uniform(0.6, 1.0, (R, g)).astype(np.float32)
        B = np.arange(R * (g + 1) + 1, dtype=np.float64)
        _sched_case(c3, 1.0 / (0.020 + 5e-5 * B))


def test_scheduler_prefix_selection_paths():
    """Algorithm 1 first sorts only the ~512 largest a (selected by histograms of
    the keys' high bits) and falls back to the whole sort when that cannot decide.
    Every path against the oracle, bit for bit: the prefix decides (early stop),
    the second histogram level (a packed into one bucket), ties too many for the
    prefix (one value of a shared by 1100 requests), no stop inside the prefix
    (SPS flat, so everything is admitted), and fewer candidates than the prefix."""
    rng = np.random.default_rng(11)

    def flat(R, g):
        return np.ones(R * (g + 1) + 1)

    def falling(R, g, k=5e-5):
        return 1.0 / (0.020 + k * np.arange(R * (g + 1) + 1, dtype=np.float64))

    # the prefix decides: configs 2 and 3 (run merge and radix shapes) with their
    # synthetic SPS tables
    for idx in (2, 3):
        cfg = synth.config(idx)
        z = rng.normal(0, 3.2, (cfg.R, cfg.gamma))
        c = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
        _sched_case(c, synth.sps_table(cfg, cfg.R * (cfg.gamma + 1)).numpy())
    # second level: every a within 1e-3 of 1, so one first-level bucket holds
    # them all; the steep curve stops inside the prefix (about 340 of ~670 keys)
    c = (1.0 - rng.uniform(0, 6e-5, (1000, 16))).astype(np.float32)
    _sched_case(c, falling(1000, 16, 1.0))
    # ties: a = 1/2 for 1024 requests (the crossing bucket, ranked; the capacity
    # stops it inside, so the (r, j) order of equal a decides) and for 1100
    # (more than the prefix takes: the whole sort)
    for R, g in [(1024, 15), (1100, 14)]:
        c = np.full((R, g), 0.5, np.float32)
        _sched_case(c, flat(R, g), N_max=R + 300)
    # no stop inside the prefix: the flat curve admits every candidate
    for R, g in [(256, 16), (700, 20)]:
        c = rng.uniform(0.3, 1.0, (R, g)).astype(np.float32)
        c[rng.uniform(size=(R, g)) < 0.05] = 0.0
        _sched_case(c, flat(R, g))
        _sched_case(c, flat(R, g), N_max=R + 600)        # the capacity stops it past 512
    # fewer candidates than the prefix holds
    c = rng.uniform(0, 1, (9, 5)).astype(np.float32)
    _sched_case(c, flat(9, 5))
    _sched_case(c, falling(9, 5, 0.01))


def _async_case(c, sps, K_in, N_max=None, alias=False):
    import oracle as O
    R, g = c.shape
    cd = torch.as_tensor(c, device=DEV)
    spsd = torch.as_tensor(sps, device=DEV)
    ell = torch.empty(R, dtype=torch.int32, device=DEV)
    a = torch.empty(R, g, dtype=torch.float32, device=DEV)
    N = torch.empty(1, dtype=torch.int32, device=DEV)
    th = torch.empty(1, dtype=torch.float64, device=DEV)
    thp = torch.empty(1, dtype=torch.float64, device=DEV)
    Kin = torch.full((1,), K_in, dtype=torch.int32, device=DEV)
    Kp = Kin if alias else torch.empty(1, dtype=torch.int32, device=DEV)
    D.async_schedule(cd, spsd, Kin, Kp, ell, N_max=N_max, a=a, N_out=N, theta=th, theta_plan=thp)
    torch.cuda.synchronize()
    e, ao, No, tho, Ko, thpo = O.async_schedule(c, sps, K_in, N_max=N_max)
    np.testing.assert_array_equal(n(ell), e)
    np.testing.assert_array_equal(n(a).view(np.uint32), ao.view(np.uint32))
    assert int(n(N)[0]) == No
    assert float(n(th)[0]) == tho
    assert int(n(Kp)[0]) == Ko
    assert float(n(thp)[0]) == thpo


def test_async_scheduler_bitexact_random_and_ties():
    rng = np.random.default_rng(5)
    for it in range(40):
        R, g = int(rng.integers(1, 300)), int(rng.integers(1, 33))
        if R * g > 16384:
            continue
        c = rng.uniform(0, 1, (R, g)).astype(np.float32)
        if it % 3 == 0:
            c = rng.choice(np.array([0, 0.25, 0.5, 0.75, 1.0], np.float32), (R, g))
        if it % 5 == 0:
            c[:, :] = 1.0
        B = np.arange(R * (g + 1) + 1, dtype=np.float64)
        sps = [1.0 / (0.020 + 5e-5 * B), 1.0 / (0.02 + 0.002 * B),
               1.0 / (0.015 + 4e-5 * B + 0.003 * (B // 7)), 1.0 / np.maximum(B, 1.0)][it % 4]
        N_max = None if it % 4 else int(rng.integers(R, R * (g + 1) + 1))
        for K_in in [int(rng.integers(R, R * (g + 1) + 1)), 0, R, R * (g + 1) + 5]:
            _async_case(c, sps, K_in, N_max=N_max, alias=(it % 2 == 0))


def test_async_scheduler_stress_size():
    cfg = synth.config(3)
    rng = np.random.default_rng(4)
    z = rng.normal(0, 3.2, (cfg.R, cfg.gamma))
    c = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    sps = synth.sps_table(cfg, cfg.R * (cfg.gamma + 1)).numpy()
    for K_in in [cfg.R, cfg.R + 3000, cfg.R * (cfg.gamma + 1)]:
        _async_case(c, sps, K_in)
    for R, g in [(600, 17), (900, 17)]:
        c3 = rng.uniform(0.6, 1.0, (R, g)).astype(np.float32)
        B = np.arange(R * (g + 1) + 1, dtype=np.float64)
        _async_case(c3, 1.0 / (0.015 + 4e-5 * B + 0.003 * (B // 64)), R + 4000)


def test_async_scheduler_two_round_pipeline():
    """Rounds t = 0..7 through the round driver's two-slot capacity ring: the
    capacity round t admits with is the one planned at round t - 2 (the seed
    for t < 2), in the same stream order as a live decode loop."""
    import oracle as O
    rng = np.random.default_rng(6)
    R, g = 48, 7
    B = np.arange(R * (g + 1) + 1, dtype=np.float64)
    sps = 1.0 / (0.015 + 4e-5 * B + 0.003 * (B // 16))
    spsd = torch.as_tensor(sps, device=DEV)
    ring = RD.CapacityRing(R, g, len(sps) - 1, device=DEV)
    ell = torch.empty(R, dtype=torch.int32, device=DEV)
    cs = [(1.0 / (1.0 + np.exp(-rng.normal(1.5, 2.5, (R, g))))).astype(np.float32) for _ in range(8)]
    outs = []
    for t, c in enumerate(cs):
        kin, kplan = ring.slots(t)
        D.async_schedule(torch.as_tensor(c, device=DEV), spsd, kin, kplan, ell)
        outs.append(n(ell).copy())
    torch.cuda.synchronize()
    hist = [min(R * (g + 1), len(sps) - 1)] * 2
    for t, c in enumerate(cs):
        e, _, _, _, Kp, _ = O.async_schedule(c, sps, hist[t])
        np.testing.assert_array_equal(outs[t], e)
        hist.append(Kp)


# ------------------------------------------------------- verify: cap-accept
CAP = [
    (2, dict(R=40, gamma=5, V=3000, d=64), "sched", 1),        # bf16, rank 256, sampled
    (2, dict(R=33, gamma=6, V=2600, d=64, rank=0), "random", 1),
    (1, dict(R=33, gamma=7, V=5000, d=128), "random", 1),      # greedy
    (0, {}, "random", 1),                                       # fp32
    (2, dict(R=24, gamma=4, V=1800, d=64, T=0.3), "sched", 0),  # packed target rows
    (3, dict(R=70, gamma=6, V=2500, d=64), "sched", 1),
]


@pytest.mark.parametrize("base,over,capk,layout", CAP, ids=[f"cap{i}" for i in range(len(CAP))])
def test_cap_accept_parity(base, over, capk, layout):
    """Whole-block verification committed within a window: the scheduler's
    ell (Algorithm 1) or random windows, against the oracle's cap-accept."""
    cfg = synth.scaled(synth.config(base), **over) if over else synth.config(base)
    print(f"[case] cap-accept {cfg.name} R={cfg.R} g={cfg.gamma} V={cfg.V} r={cfg.rank} T={cfg.T} "
          f"cap={capk} layout={layout}", flush=True)
    inp = synth.make_inputs(cfg, device="cpu")
    g = to_dev(inp)
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    D.draft_markov(g["U"], g["W1"], g["W2t"], g["x0"], cfg.T, cfg.philox_seed, 2, buf.x,
                   buf.logp_d, buf.lse_d, buf.ws)
    D.confidence(g["h"], g["W1"], g["w"], buf.x, buf.c, V=cfg.V)
    D.prefix_schedule(buf.c, g["sps"], buf.ell, N_out=buf.N)
    full = torch.full((cfg.R,), cfg.gamma, dtype=torch.int32, device=DEV)
    D.pack(buf.x, full, 1, buf.cu, buf.flat, buf.marker_req, buf.marker_pos, buf.N, ws=buf.ws)
    if capk == "sched":
        cap = buf.ell.clone()
    else:
        rng = np.random.default_rng(cfg.R)
        cap = torch.as_tensor(rng.integers(0, cfg.gamma + 3, cfg.R).astype(np.int32), device=DEV)
    tgt = g["target"]
    if layout == 0:
        torch.cuda.synchronize()
        Np = int(n(buf.N)[0])
        tgt = g["target"][buf.marker_req[:Np].long(), buf.marker_pos[:Np].long()].contiguous()
    mfull = torch.empty(cfg.R, dtype=torch.int32, device=DEV)
    D.verify_cap_accept(full, cap, buf.cu, tgt, layout, buf.x, buf.logp_d, buf.lse_d, g["U"],
                        g["W1"], g["W2t"], cfg.T, cfg.philox_seed, 2, buf.m, buf.tau, buf.emitted,
                        buf.next_anchor, buf.ws, m_full=mfull, logp_t=buf.logp_t)
    torch.cuda.synchronize()
    status = D.get_status(buf.ws)
    rep = PC.Report()
    W1, W2t = f(inp["W1"]), f(inp["W2t"])
    tg = f(tgt) if layout == 0 else f(inp["target"])
    m, mf = PC.check_verify_cap_accept(rep, n(full), n(cap), n(buf.cu), tg, layout, n(buf.x),
                                       n(buf.logp_d), n(buf.lse_d), f(inp["U"]), W1, W2t, cfg.T,
                                       cfg.philox_seed, 2, n(buf.m), n(buf.tau), n(buf.emitted),
                                       n(buf.next_anchor), n(mfull), None)
    print(f"  {rep.summary()} status={status} sum_m={int(m.sum())} sum_m_full={int(mf.sum())} "
          f"closed_by_draft={int((mf > np.minimum(n(cap), cfg.gamma)).sum())}", flush=True)
    assert status == 0, f"device flags {status}"
    assert rep.ok(), rep.summary()
    assert (mf >= m).all()


def test_round_driver_async_cap_accept_tiers():
    """The round driver with the production options together: asynchronous
    scheduler (two-slot ring), whole-block verify committed within the window,
    verify batch padded to a tier; every stage against the oracle."""
    import oracle as O
    cfg = synth.scaled(synth.config(2), R=48, gamma=5, V=2600, d=64)
    inp = synth.make_inputs(cfg, device="cpu")
    g = to_dev(inp)
    tiers = [64, 128, 192, 256, 320]
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV, slots=320)
    nmax = g["sps"].numel() - 1
    ring = RD.CapacityRing(cfg.R, cfg.gamma, nmax, device=DEV)
    hist = [min(cfg.R * (cfg.gamma + 1), nmax)] * 2
    for rnd in range(4):
        print(f"[case] driver round {rnd}", flush=True)
        D.clear_status(buf.ws)
        RD.run_round(g, buf, cfg.T, cfg.philox_seed, rnd, scheduler="async", ring=ring,
                     verify_mode="cap-accept", tiers=tiers, pad_token=7)
        torch.cuda.synchronize()
        assert D.get_status(buf.ws) == 0
        c = n(buf.c)
        e, _, Ne, _, Kp, _ = O.async_schedule(c, n(g["sps"]), hist[rnd])
        hist.append(Kp)
        np.testing.assert_array_equal(n(buf.ell), e)
        pk = O.pack_tiered(n(buf.x), np.full(cfg.R, cfg.gamma + 1), tiers, 7, slots=320)
        np.testing.assert_array_equal(n(buf.flat), pk[1])
        assert int(n(buf.N)[0]) == pk[4] and int(n(buf.N_pad)[0]) == pk[5]
        rep = PC.Report()
        PC.check_verify_cap_accept(rep, n(buf.full), e, None, f(inp["target"]), 1, n(buf.x),
                                   n(buf.logp_d), n(buf.lse_d), f(inp["U"]), f(inp["W1"]),
                                   f(inp["W2t"]), cfg.T, cfg.philox_seed, rnd, n(buf.m),
                                   n(buf.tau), n(buf.emitted), n(buf.next_anchor), n(buf.m_full),
                                   None)
        assert rep.ok(), rep.summary()
        PC.check_pack(rep, n(buf.emitted), n(buf.tau), n(buf.cu_out), n(buf.flat_out), None, None,
                      n(buf.N_out)[0], "emitted")
        assert rep.ok(), rep.summary()


def test_cap_accept_negative_window_is_flagged():
    cfg = synth.scaled(synth.config(2), R=8, gamma=3, V=700, d=16)
    inp = synth.make_inputs(cfg, device="cpu")
    g = to_dev(inp)
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    D.clear_status(buf.ws)
    D.draft_markov(g["U"], g["W1"], g["W2t"], g["x0"], cfg.T, 1, 0, buf.x, buf.logp_d, buf.lse_d,
                   buf.ws)
    full = torch.full((cfg.R,), cfg.gamma, dtype=torch.int32, device=DEV)
    D.pack(buf.x, full, 1, buf.cu, buf.flat, ws=buf.ws)
    cap = torch.full((cfg.R,), -3, dtype=torch.int32, device=DEV)
    D.verify_cap_accept(full, cap, buf.cu, g["target"], 1, buf.x, buf.logp_d, buf.lse_d, g["U"],
                        g["W1"], g["W2t"], cfg.T, 1, 0, buf.m, buf.tau, buf.emitted,
                        buf.next_anchor, buf.ws)
    torch.cuda.synchronize()
    assert D.get_status(buf.ws) & D._lib.FLAG_BAD_LEN
    assert (n(buf.m) == 0).all() and (n(buf.tau) == 1).all()


# ------------------------------------------- diagnostics: c*, STS fit
CSTAR = [
    (2, dict(R=40, gamma=5, V=3000, d=64)),               # bf16 rank 256: W2-slice kernel
    (2, dict(R=33, gamma=4, V=2000, d=64, rank=64)),
    (2, dict(R=37, gamma=6, V=2600, d=64, rank=0)),       # no bias: per-tile kernel
    (0, {}),                                               # fp32
    (1, dict(R=33, gamma=7, V=5000, d=128)),               # T = 0
    (2, dict(R=5, gamma=3, V=300, d=32, rank=16)),         # 3 chunks: batched work list
    (3, dict(R=70, gamma=6, V=2500, d=64)),
]


@pytest.mark.parametrize("base,over", CSTAR, ids=[f"cstar{i}" for i in range(len(CSTAR))])
def test_acceptance_rate_parity(base, over):
    import oracle as O
    cfg = synth.scaled(synth.config(base), **over) if over else synth.config(base)
    print(f"[case] c* {cfg.name} R={cfg.R} g={cfg.gamma} V={cfg.V} r={cfg.rank} T={cfg.T}",
          flush=True)
    inp = synth.make_inputs(cfg, device="cpu")
    g = to_dev(inp)
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    D.draft_markov(g["U"], g["W1"], g["W2t"], g["x0"], cfg.T, cfg.philox_seed, 1, buf.x,
                   buf.logp_d, buf.lse_d, buf.ws)
    cs = torch.empty(cfg.R, cfg.gamma, dtype=torch.float32, device=DEV)
    D.acceptance_rate(g["target"], buf.x, buf.lse_d, g["U"], g["W1"], g["W2t"], cfg.T, cs, buf.ws)
    torch.cuda.synchronize()
    assert D.get_status(buf.ws) == 0
    ref, mg = O.acceptance_rate(f(inp["target"]), n(buf.x), f(inp["U"]), f(inp["W1"]),
                                f(inp["W2t"]), cfg.T)
    got = n(cs).astype(np.float64)
    if cfg.T > 0:
        rel = np.abs(got - ref) / np.maximum(ref, 1e-30)
        print(f"  c* max rel err {rel.max():.3g}, range [{ref.min():.3g}, {ref.max():.3g}]",
              flush=True)
        assert rel.max() <= 1e-5
    else:
        bad = (got != ref) & (mg >= 1e-5)
        assert not bad.any() and (got != ref).sum() <= 0.001 * got.size + 1


def test_confidence_logits_parity():
    import oracle as O
    for base, over in [(2, dict(R=40, gamma=5, V=3000, d=256)), (0, {}),
                       (2, dict(R=9, gamma=3, V=1500, d=64, rank=0))]:
        cfg = synth.scaled(synth.config(base), **over) if over else synth.config(base)
        inp = synth.make_inputs(cfg, device="cpu")
        g = to_dev(inp)
        rng = np.random.default_rng(cfg.R)
        x = np.concatenate([n(inp["x0"])[:, None], rng.integers(0, cfg.V, (cfg.R, cfg.gamma))], 1)
        xd = torch.as_tensor(x.astype(np.int32), device=DEV)
        z = torch.empty(cfg.R, cfg.gamma, dtype=torch.float32, device=DEV)
        D.confidence_logits(g["h"], g["W1"], g["w"], xd, z, V=cfg.V)
        torch.cuda.synchronize()
        _, zo = O.confidence(f(inp["h"]), f(inp["W1"]), f(inp["w"]), x)
        err = np.abs(n(z).astype(np.float64) - zo) / (1.0 + np.abs(zo))
        assert err.max() <= 1e-5, err.max()


def _sts_case(n_, g_, grid, nbins, seed, t_true=None):
    import oracle as O
    rng = np.random.default_rng(seed)
    t_true = t_true or list(rng.choice(grid, g_))
    zc = rng.normal(1.5, 2.0, (n_, g_)).astype(np.float32)
    p = 1.0 / (1.0 + np.exp(-zc.astype(np.float64) / np.asarray(t_true)))
    acc = rng.uniform(size=(n_, g_)) < p
    m = np.where(acc.all(1), g_, np.argmin(acc, axis=1)).astype(np.int32)
    zd, md = torch.as_tensor(zc, device=DEV), torch.as_tensor(m, device=DEV)
    t = torch.empty(g_, dtype=torch.float32, device=DEV)
    e = torch.empty(g_, dtype=torch.float64, device=DEV)
    ws = D.sts_workspace(n_, device=DEV)
    D.sts_fit(zd, md, grid, t, ws, nbins=nbins, ece_out=e)
    torch.cuda.synchronize()
    tg, eg = n(t), n(e)
    # lock-step: a differing choice is allowed only where the oracle's margin
    # (ECE gap to the runner-up, or a value on a bin edge) is below 1e-9
    to, eo, mo = O.sts_fit(zc, m, grid, nbins=nbins, force_t=tg)
    t_own, _, _ = O.sts_fit(zc, m, grid, nbins=nbins)
    for k in range(g_):
        if tg[k] != t_own[k]:
            assert mo[k] < 1e-9, (k, tg[k], t_own[k], mo[k])
    np.testing.assert_allclose(eg, eo, rtol=1e-12, atol=1e-15)
    return tg, eg


def test_sts_fit_parity():
    grid = np.round(np.linspace(0.3, 3.0, 28), 6).astype(np.float32)
    _sts_case(20000, 6, grid, 15, 1)
    _sts_case(777, 3, grid, 7, 2)
    _sts_case(1, 2, grid, 1, 3)                           # one block, one bin
    _sts_case(5000, 4, grid[:1], 64, 4)                   # one candidate, 64 bins
    tg, _ = _sts_case(200_000, 5, grid, 15, 5, t_true=[grid[3], grid[9], grid[17], grid[5], grid[12]])
    np.testing.assert_array_equal(tg, grid[[3, 9, 17, 5, 12]])


def _schedule_pack_case(c, sps, x, mode, N_max=None, K_in=None):
    """dspark_schedule_pack against the oracle's scheduler followed by its pack
    of x with lengths ell + 1."""
    import oracle as O
    R, g = c.shape
    dev = lambda v: torch.as_tensor(v, device=DEV)
    ell = torch.full((R,), -7, dtype=torch.int32, device=DEV)
    a = torch.empty(R, g, dtype=torch.float32, device=DEV)
    N = torch.empty(1, dtype=torch.int32, device=DEV)
    th = torch.empty(1, dtype=torch.float64, device=DEV)
    thp = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    cu = torch.full((R + 1,), -7, dtype=torch.int32, device=DEV)
    flat = torch.full((R * (g + 1),), -7, dtype=torch.int32, device=DEV)
    mr, mp = torch.full_like(flat, -7), torch.full_like(flat, -7)
    Kin = Kp = None
    if mode == 2:
        Kin = torch.full((1,), K_in, dtype=torch.int32, device=DEV)
        Kp = torch.empty(1, dtype=torch.int32, device=DEV)
    D.schedule_pack(dev(c), dev(sps), dev(x), ell, cu, flat, mode=mode, marker_req=mr,
                    marker_pos=mp, K_in=Kin, K_plan=Kp, N_max=N_max, a=a, N_out=N, theta=th,
                    theta_plan=thp)
    torch.cuda.synchronize()
    if mode == 2:
        e, ao, No, tho, Ko, thpo = O.async_schedule(c, sps, K_in, N_max=N_max)
        assert int(n(Kp)[0]) == Ko
        assert float(n(thp)[0]) == thpo
    else:
        e, ao, No, tho, _ = O.prefix_schedule(c, sps, N_max=N_max, enabled=mode == 1)
        assert float(n(thp)[0]) == -1.0                  # not written outside mode 2
    np.testing.assert_array_equal(n(ell), e)
    np.testing.assert_array_equal(n(a).view(np.uint32), ao.view(np.uint32))
    assert int(n(N)[0]) == No
    assert float(n(th)[0]) == tho
    pe = O.pack(x, np.asarray(e) + 1)
    np.testing.assert_array_equal(n(cu), pe[0])
    np.testing.assert_array_equal(n(flat), pe[1])
    np.testing.assert_array_equal(n(mr), pe[2])
    np.testing.assert_array_equal(n(mp), pe[3])
    assert pe[4] == No


def test_schedule_pack_matches_oracle():
    """The fused schedule + verify-batch pack: static, greedy and asynchronous
    modes over random shapes (merge-sorted runs, and the bitonic network for
    packed keys), ties, zeros inside a block and all-ones confidences."""
    rng = np.random.default_rng(11)
    cases = [(int(rng.integers(1, 300)), int(rng.integers(1, 33))) for _ in range(12)]
    cases += [(256, 16), (1, 1), (1024, 16), (600, 17)]
    for it, (R, g) in enumerate(cases):
        if R * g > 16384:
            continue
        c = rng.uniform(0, 1, (R, g)).astype(np.float32)
        if it % 3 == 0:
            c = rng.choice(np.array([0, 0.25, 0.5, 0.75, 1.0], np.float32), (R, g))
        if it % 5 == 4:
            c[:, :] = 1.0
        if it % 7 == 6:
            c[rng.uniform(0, 1, (R, g)) < 0.2] = 0.0             # runs cut short by c = 0
        x = rng.integers(0, 129280, (R, g + 1)).astype(np.int32)
        B = np.arange(R * (g + 1) + 1, dtype=np.float64)
        sps = [1.0 / (0.020 + 5e-5 * B), 1.0 / (0.015 + 4e-5 * B + 0.003 * (B // 7))][it % 2]
        N_max = None if it % 4 else int(rng.integers(R, R * (g + 1) + 1))
        _schedule_pack_case(c, sps, x, 1, N_max=N_max)
        _schedule_pack_case(c, sps, x, 0)
        for K_in in [int(rng.integers(R, R * (g + 1) + 1)), 0, R * (g + 1) + 5]:
            _schedule_pack_case(c, sps, x, 2, N_max=N_max, K_in=K_in)


# ------------------------------------------------------------- stage: pack
def test_pack_tiered_bitexact():
    import oracle as O
    rng = np.random.default_rng(2)
    for R, width, off, tiers, extra in [(300, 17, 1, [512, 1024, 2048, 4096, 8192], 100),
                                        (5, 4, 0, [1, 2, 4, 8, 16], 0),
                                        (2000, 9, 0, [64, 128], 7),       # no tier holds N
                                        (1, 1, 0, [1], 0),
                                        (700, 6, 1, list(range(128, 4200, 128)), 0)]:
        slots = R * width + extra
        tiers = [t for t in tiers if t <= slots][:32]       # every tier fits the slots
        rows = rng.integers(0, 100000, (R, width)).astype(np.int32)
        lens = rng.integers(0, width + 1 - off, R).astype(np.int32)
        rd, ld = torch.as_tensor(rows, device=DEV), torch.as_tensor(lens, device=DEV)
        cu = torch.empty(R + 1, dtype=torch.int32, device=DEV)
        flat = torch.empty(slots, dtype=torch.int32, device=DEV)
        mr, mp = torch.empty_like(flat), torch.empty_like(flat)
        N = torch.empty(1, dtype=torch.int32, device=DEV)
        Np = torch.empty(1, dtype=torch.int32, device=DEV)
        ws = D.workspace(1, 1, 1, device=DEV)
        D.clear_status(ws)
        D.pack_tiered(rd, ld, off, tiers, 99, cu, flat, mr, mp, N, Np, ws=ws)
        torch.cuda.synchronize()
        e = O.pack_tiered(rows, lens + off, tiers, 99, slots=slots)
        np.testing.assert_array_equal(n(cu), e[0])
        np.testing.assert_array_equal(n(flat), e[1])
        np.testing.assert_array_equal(n(mr), e[2])
        np.testing.assert_array_equal(n(mp), e[3])
        assert int(n(N)[0]) == e[4] and int(n(Np)[0]) == e[5]
        assert bool(D.get_status(ws) & D._lib.FLAG_TIER) == e[6]


def test_pack_bitexact():
    import oracle as O
    rng = np.random.default_rng(1)
    for R, width, off in [(1, 1, 0), (3000, 17, 1), (1025, 9, 0), (64, 33, 1)]:
        rows = rng.integers(0, 100000, (R, width)).astype(np.int32)
        lens = rng.integers(0, width + 1 - off, R).astype(np.int32)
        rd, ld = torch.as_tensor(rows, device=DEV), torch.as_tensor(lens, device=DEV)
        cu = torch.empty(R + 1, dtype=torch.int32, device=DEV)
        flat = torch.empty(R * width, dtype=torch.int32, device=DEV)
        mr, mp = torch.empty_like(flat), torch.empty_like(flat)
        N = torch.empty(1, dtype=torch.int32, device=DEV)
        D.pack(rd, ld, off, cu, flat, mr, mp, N)
        torch.cuda.synchronize()
        e = O.pack(rows, lens + off)
        np.testing.assert_array_equal(n(cu), e[0])
        np.testing.assert_array_equal(n(flat), e[1])
        np.testing.assert_array_equal(n(mr), e[2])
        np.testing.assert_array_equal(n(mp), e[3])
        assert int(n(N)[0]) == e[4]


# --------------------------------------------------------- full-size cases
def _full(idx, reqs, **cell):
    cfg = synth.config(idx, **cell)
    inp = synth.make_inputs(cfg, device=DEV)
    buf, rep = run_and_check(cfg, None, inp_dev=inp, reqs=reqs)
    return cfg, inp, buf, rep


def test_full_config2_all_requests():
    """The headline workload (R=256, gamma=16, V=129280, r=256, bf16, T=1,
    Algorithm 1): every request's draft decisions, log p_d, lse_d, confidences
    and verification against the oracle, the schedule and both packs."""
    _full(2, None)


def test_full_config1_all_requests():
    _full(1, None)


@pytest.mark.parametrize("idx,cell", [(2, {}), (1, {}), (4, dict(R=512, gamma=16, rank=64)),
                                      (4, dict(R=32, gamma=8, rank=256))],
                         ids=["config2", "config1", "R512-g16-r64", "R32-g8-r256"])
def test_full_pipelined_kernel(draft_schedule, idx, cell):
    """The pipelined persistent draft kernel at full sizes: the headline
    workload and the greedy one on every request, two rank-sweep cells on the
    requests _cell_reqs spreads over the batch."""
    draft_schedule("pipe")
    reqs = _cell_reqs(cell["R"]) if cell else None
    _full(idx, reqs, **cell)


def test_full_config3_sampled():
    """R=1024, gamma=15, V=151936, T=0.7: 64 requests spread over the batch
    (hard and easy), the schedule over all 1024 and both packs."""
    _full(3, sorted(set(np.linspace(0, 1023, 60).round().astype(int).tolist()
                        + [255, 256, 511, 512, 767, 768, 1023])))


def _cell_reqs(R):
    if R <= 32:
        return None                                   # every request
    # spread over the batch, including both sides of the 256-row boundaries
    return sorted(set(np.linspace(0, R - 1, 20).round().astype(int).tolist()
                      + [255, 256, 257, R - 1]))


CELLS = [(R, g, r) for R in (1, 32, 512) for g in (4, 8, 16) for r in (0, 64, 256)]


@pytest.mark.parametrize("R,gamma,rank", CELLS, ids=[f"R{R}-g{g}-r{r}" for R, g, r in CELLS])
def test_full_config4_cell(R, gamma, rank):
    """Every cell of the rank and length sweep (V=129280, d=4096, bf16, T=1,
    Algorithm 1) at full vocabulary.  Rank 0 (independent per-position
    sampling, the DFlash case) must reproduce the oracle's tokens bit for bit."""
    cfg, inp, buf, rep = _full(4, _cell_reqs(R), R=R, gamma=gamma, rank=rank)
    if rank == 0:
        assert rep.flagged.get("draft", 0) == 0 and rep.flagged.get("verify", 0) == 0, \
            rep.summary()


def test_full_config2_bitwise_repeat():
    """The headline round twice on the same inputs and buffers: every output
    of every stage is bitwise identical."""
    cfg = synth.config(2)
    inp = synth.make_inputs(cfg, device=DEV)
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
    outs = []
    for _ in range(2):
        D.clear_status(buf.ws)
        RD.run_round(inp, buf, cfg.T, cfg.philox_seed, 3, scheduler=True)
        torch.cuda.synchronize()
        assert D.get_status(buf.ws) == 0
        outs.append([t.clone() for t in (buf.x, buf.logp_d, buf.lse_d, buf.c, buf.ell, buf.a,
                                           buf.N, buf.theta, buf.cu, buf.flat, buf.m, buf.tau,
                                           buf.emitted, buf.next_anchor, buf.logp_t, buf.flat_out)])
    for i, (a, b) in enumerate(zip(*outs)):
        assert torch.equal(a, b), i


def test_full_config2_zero_w2_equals_rank0():
    """W2 = 0 at rank 256 adds an exactly zero bias, so the draft must sample
    the tokens of the rank-0 draft (independent per-position sampling) on the
    same U: identical everywhere except where the oracle's decision margin is
    below 1e-5 (the two schedules sum the softmax in different orders)."""
    import oracle as O
    cfg = synth.config(2)
    inp = synth.make_inputs(cfg, device=DEV)
    xs, lps = [], []
    for W1, W2t in ((inp["W1"], torch.zeros_like(inp["W2t"])), (None, None)):
        buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV)
        D.clear_status(buf.ws)
        D.draft_markov(inp["U"], W1, W2t, inp["x0"], cfg.T, cfg.philox_seed, 9, buf.x,
                       buf.logp_d, buf.lse_d, buf.ws)
        torch.cuda.synchronize()
        assert D.get_status(buf.ws) == 0
        xs.append(n(buf.x))
        lps.append((n(buf.logp_d), n(buf.lse_d)))
    diff = xs[0] != xs[1]
    print(f"  tokens differing: {int(diff.sum())} of {diff[:, 1:].size}", flush=True)
    if diff.any():
        # only near-ties may differ: the oracle's margins on the rank-0 chain
        bad = np.argwhere(diff)
        rows = sorted(set(int(r) for r, _ in bad))
        Uh = f(inp["U"][torch.as_tensor(rows, device=DEV)])
        _, _, _, mg = O.draft_markov(Uh, None, None, n(inp["x0"])[rows], cfg.T, cfg.philox_seed, 9,
                                     req_ids=np.asarray(rows, np.int32), force_x=xs[1][rows])
        for r, k in bad:
            assert mg[rows.index(int(r)), k - 1] < PC.MARGIN, (r, k)
        assert diff.sum() <= 0.001 * diff[:, 1:].size
    else:
        np.testing.assert_allclose(lps[0][0], lps[1][0], atol=1e-5, rtol=0)
        np.testing.assert_allclose(lps[0][1], lps[1][1], atol=1e-5, rtol=0)


# ---------------------------------------------------------------- RNN head
def run_and_check_rnn(cfg, inp_cpu=None, inp_dev=None, gain=3.0, reqs=None, rnd=0, buf=None):
    """A full round drafted by the RNN head (its features verified by
    dspark_verify_features); every stage checked against the oracle."""
    print(f"[case rnn] {cfg.name} R={cfg.R} g={cfg.gamma} V={cfg.V} r={cfg.rank} d={cfg.d} "
          f"T={cfg.T} gain={gain} reqs={None if reqs is None else list(reqs)}", flush=True)
    if inp_dev is None:
        inp_dev = to_dev(inp_cpu)
    g = dict(inp_dev)
    g["Wr"] = synth.rnn_weights(cfg, device=DEV, gain=gain)
    if buf is None:
        buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV, rnn=(cfg.rank, cfg.d, cfg.dtype))
    RD.run_round(g, buf, cfg.T, cfg.philox_seed, rnd, scheduler=cfg.scheduler, layout=1,
                 head="rnn")
    torch.cuda.synchronize()
    status = D.get_status(buf.ws)
    rep = PC.Report()
    sel = slice(None) if reqs is None else np.asarray(reqs)

    def host(key, rows=True):
        t = inp_cpu[key] if inp_cpu is not None else g[key]
        if rows and reqs is not None:
            t = t[torch.as_tensor(np.asarray(reqs), device=t.device)]
        return f(t) if t.is_floating_point() else n(t)

    U, tgt, h = host("U"), host("target"), host("h")
    W1, W2t, w = host("W1", False), host("W2t", False), host("w", False)
    Wr = f(g["Wr"])
    x0 = host("x0")
    x = n(buf.x)[sel]
    rq = None if reqs is None else np.asarray(reqs, np.int32)
    feat = f(buf.feat)[sel]
    bf16_e = cfg.dtype == torch.bfloat16
    lp_o, lse_o = PC.check_draft_rnn(rep, U, W1, W2t, Wr, h, x0, cfg.T, cfg.philox_seed, rnd, x,
                                     n(buf.logp_d)[sel], n(buf.lse_d)[sel], feat,
                                     n(buf.state)[sel], rq, bf16_e)
    PC.check_confidence(rep, h, W1, w, x, n(buf.c)[sel])
    PC.check_schedule(rep, n(buf.c), n(g["sps"]), cfg.scheduler, n(buf.ell), n(buf.a),
                      n(buf.N)[0], n(buf.theta)[0])
    PC.check_pack(rep, n(buf.x), n(buf.ell) + 1, n(buf.cu), n(buf.flat), n(buf.marker_req),
                  n(buf.marker_pos), n(buf.N)[0], "verify batch")
    m, *_ = PC.check_verify(rep, n(buf.ell)[sel], None, tgt, 1, x, lp_o, lse_o, U, W1, W2t,
                            cfg.T, cfg.philox_seed, rnd,
                            n(buf.m)[sel], n(buf.tau)[sel], n(buf.emitted)[sel],
                            n(buf.next_anchor)[sel], n(buf.logp_t)[sel], rq, feat=feat)
    PC.check_pack(rep, n(buf.emitted), n(buf.tau), n(buf.cu_out), n(buf.flat_out), None, None,
                  n(buf.N_out)[0], "emitted")
    n_rej = int((n(buf.m) < n(buf.ell)).sum())
    print(f"  {rep.summary()} status={status} sum_ell={int(n(buf.ell).sum())} "
          f"sum_m={int(n(buf.m).sum())} rejected={n_rej}", flush=True)
    assert status == 0, f"device flags {status}"
    assert rep.ok(), rep.summary()
    return buf, rep, n_rej


RNN_SMALL = [
    (0, {}),                                                            # float32 throughout
    (2, dict(R=40, gamma=5, V=3000, d=256)),                             # bf16, rank 256, MFMA h part
    (2, dict(R=33, gamma=4, V=2000, d=64, rank=64)),
    (2, dict(R=9, gamma=3, V=1500, d=40, rank=16)),
    (2, dict(R=6, gamma=4, V=1001, d=36, rank=32)),                      # d not a multiple of 8
    (2, dict(R=35, gamma=4, V=2000, d=72, rank=512)),
    (1, dict(R=20, gamma=5, V=3001, d=96, rank=32)),                     # greedy
    (3, dict(R=70, gamma=6, V=2500, d=64)),                              # T = 0.7
    (2, dict(R=24, gamma=4, V=1800, d=64, scheduler=False)),             # every position verified
    (2, dict(R=1, gamma=1, V=700, d=16)),
    # shapes the fused persistent launch takes (bf16, rank 64/128/256, V % 8 == 0)
    (1, dict(R=33, gamma=7, V=4096, d=128, rank=128)),                   # greedy
    (3, dict(R=70, gamma=6, V=2504, d=64)),                              # T = 0.7
    (2, dict(R=300, gamma=3, V=2048, d=32)),                             # more cell tiles than CUs
    (2, dict(R=17, gamma=16, V=1536, d=64, rank=64)),
    (2, dict(R=8, gamma=32, V=1024, d=64, rank=64)),                     # longest block, fused
    (2, dict(R=12, gamma=32, V=900, d=32, rank=32)),                     # longest block, per step
    (2, dict(R=24, gamma=4, V=1800, d=64, T=0.3)),                       # low temperature, fused
]
RNN_FUSED = [RNN_SMALL[i] for i in (1, 2, 8, 10, 11, 12, 13, 14, 16)]


@pytest.mark.parametrize("base,over", RNN_SMALL, ids=[f"rnn{i}" for i in range(len(RNN_SMALL))])
def test_rnn_round_parity(base, over):
    cfg = synth.scaled(synth.config(base), **over) if over else synth.config(base)
    inp = synth.make_inputs(cfg, device="cpu")
    run_and_check_rnn(cfg, inp)


@pytest.mark.parametrize("base,over", RNN_FUSED, ids=[f"steps{i}" for i in range(len(RNN_FUSED))])
def test_rnn_per_step_schedule(switch, base, over):
    """The shapes of the fused launch, forced onto the per-step schedule."""
    switch(D._lib.SWITCH_FORCE_PER_STEP, 1)
    cfg = synth.scaled(synth.config(base), **over)
    run_and_check_rnn(cfg, synth.make_inputs(cfg, device="cpu"))


def test_rnn_rounds_reuse_buffers():
    """Several rounds on the same buffers (features and states rewritten in
    place), each checked against the oracle."""
    cfg = synth.scaled(synth.config(2), R=40, gamma=5, V=3000, d=256)
    inp = synth.make_inputs(cfg, device="cpu")
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV, rnn=(cfg.rank, cfg.d, cfg.dtype))
    for rnd in range(3):
        run_and_check_rnn(cfg, inp, rnd=rnd, buf=buf)


def test_rnn_feature_residuals_exercised():
    """Static block, T = 1: many rejections, so the residual rows rebuilt from
    the features are checked; the same drafts verified without the features
    (as a Markov head) give other emitted tokens."""
    cfg = synth.scaled(synth.config(2), R=48, gamma=6, V=2500, d=64, scheduler=False)
    inp = synth.make_inputs(cfg, device="cpu")
    buf, rep, n_rej = run_and_check_rnn(cfg, inp)
    assert n_rej >= 10, n_rej
    g = to_dev(inp)
    alt = torch.empty_like(buf.emitted)
    m2, t2, na2 = (torch.empty_like(buf.m) for _ in range(3))
    D.verify(buf.ell, buf.cu, g["target"], 1, buf.x, buf.logp_d, buf.lse_d, g["U"], g["W1"],
             g["W2t"], cfg.T, cfg.philox_seed, 0, m2, t2, alt, na2, buf.ws)
    torch.cuda.synchronize()
    assert not torch.equal(alt, buf.emitted)


def test_rnn_full_config2_sampled():
    cfg = synth.config(2)
    inp = synth.make_inputs(cfg, device=DEV)
    run_and_check_rnn(cfg, None, inp_dev=inp, gain=1.0, reqs=[0, 77, 160, 255])


@pytest.mark.parametrize("over", [dict(R=40, gamma=5, V=3000, d=256),
                                  dict(R=35, gamma=4, V=2000, d=72, rank=512)],
                         ids=["r256", "r512"])
def test_rnn_vector_alu_cell(switch, over):
    """The fp32 vector-ALU cell (the path of float32 weights and unaligned
    rows) on bf16 weights, forced by the library switch."""
    switch(D._lib.SWITCH_RNN_CELL_VALU, 1)
    cfg = synth.scaled(synth.config(2), **over)
    run_and_check_rnn(cfg, synth.make_inputs(cfg, device="cpu"))


def test_rnn_full_config3_sampled():
    """R=1024 requests (four 256-row groups, four cell tiles per workgroup),
    gamma=15, V=151936, T=0.7, tabulated SPS: sampled requests one by one."""
    cfg = synth.config(3)
    inp = synth.make_inputs(cfg, device=DEV)
    run_and_check_rnn(cfg, None, inp_dev=inp, gain=1.0, reqs=[3, 700, 1023])


@pytest.mark.parametrize("base,over", [(2, dict(R=40, gamma=5, V=3000, d=256)),
                                       (2, dict(R=33, gamma=4, V=2000, d=64, rank=64)),
                                       (0, {}),
                                       (1, dict(R=20, gamma=5, V=3001, d=96, rank=32))],
                         ids=["r256", "r64", "fp32", "greedy"])
def test_rnn_acceptance_rate_parity(base, over):
    """c* of RNN-head drafts (features in place of W1[x_{k-1}]) against the oracle."""
    import oracle as O
    cfg = synth.scaled(synth.config(base), **over) if over else synth.config(base)
    inp = synth.make_inputs(cfg, device="cpu")
    g = to_dev(inp)
    Wr = synth.rnn_weights(cfg, device=DEV, gain=3.0)
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV, rnn=(cfg.rank, cfg.d, cfg.dtype))
    D.draft_rnn(g["U"], g["W1"], g["W2t"], Wr, g["h"], g["x0"], cfg.T, cfg.philox_seed, 2, buf.x,
                buf.logp_d, buf.lse_d, buf.feat, buf.ws, state=buf.state)
    cs = torch.empty(cfg.R, cfg.gamma, dtype=torch.float32, device=DEV)
    D.acceptance_rate_features(g["target"], buf.x, buf.lse_d, g["U"], buf.feat, g["W2t"], cfg.T,
                               cs, buf.ws)
    torch.cuda.synchronize()
    assert D.get_status(buf.ws) == 0
    ref, mg = O.acceptance_rate(f(inp["target"]), n(buf.x), f(inp["U"]), None, f(inp["W2t"]),
                                cfg.T, feat=f(buf.feat))
    got = n(cs).astype(np.float64)
    if cfg.T > 0:
        rel = np.abs(got - ref) / np.maximum(ref, 1e-30)
        print(f"  c* max rel err {rel.max():.3g}", flush=True)
        assert rel.max() <= 1e-5
    else:
        bad = (got != ref) & (mg >= 1e-5)
        assert not bad.any() and (got != ref).sum() <= 0.001 * got.size + 1


def test_rnn_round_driver_async_tiers():
    """The RNN head through the round driver with the asynchronous scheduler
    (two-slot capacity ring) and a tier-padded verify batch, over several
    rounds on the same buffers; draft, schedule, packs and verify against the
    oracle."""
    import oracle as O
    cfg = synth.scaled(synth.config(2), R=48, gamma=5, V=2600, d=64)
    inp = synth.make_inputs(cfg, device="cpu")
    g = to_dev(inp)
    g["Wr"] = synth.rnn_weights(cfg, device=DEV, gain=3.0)
    tiers = [64, 128, 192, 256, 320]
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV, slots=320,
                          rnn=(cfg.rank, cfg.d, cfg.dtype))
    nmax = g["sps"].numel() - 1
    ring = RD.CapacityRing(cfg.R, cfg.gamma, nmax, device=DEV)
    hist = [min(cfg.R * (cfg.gamma + 1), nmax)] * 2
    U, W1, W2t, h = f(inp["U"]), f(inp["W1"]), f(inp["W2t"]), f(inp["h"])
    for rnd in range(3):
        print(f"[case] rnn driver round {rnd}", flush=True)
        D.clear_status(buf.ws)
        RD.run_round(g, buf, cfg.T, cfg.philox_seed, rnd, scheduler="async", ring=ring,
                     tiers=tiers, pad_token=7, head="rnn")
        torch.cuda.synchronize()
        assert D.get_status(buf.ws) == 0
        rep = PC.Report()
        feat = f(buf.feat)
        lp_o, lse_o = PC.check_draft_rnn(rep, U, W1, W2t, f(g["Wr"]), h, n(inp["x0"]), cfg.T,
                                         cfg.philox_seed, rnd, n(buf.x), n(buf.logp_d),
                                         n(buf.lse_d), feat, n(buf.state), None, True)
        e, _, Ne, _, Kp, _ = O.async_schedule(n(buf.c), n(g["sps"]), hist[rnd])
        hist.append(Kp)
        np.testing.assert_array_equal(n(buf.ell), e)
        pk = O.pack_tiered(n(buf.x), e + 1, tiers, 7, slots=320)
        np.testing.assert_array_equal(n(buf.flat), pk[1])
        assert int(n(buf.N)[0]) == pk[4] and int(n(buf.N_pad)[0]) == pk[5]
        PC.check_verify(rep, e, None, f(inp["target"]), 1, n(buf.x), lp_o, lse_o, U, W1, W2t,
                        cfg.T, cfg.philox_seed, rnd, n(buf.m),
                        n(buf.tau), n(buf.emitted), n(buf.next_anchor), n(buf.logp_t), None,
                        feat=feat)
        PC.check_pack(rep, n(buf.emitted), n(buf.tau), n(buf.cu_out), n(buf.flat_out), None, None,
                      n(buf.N_out)[0], "emitted")
        print(f"  {rep.summary()}", flush=True)
        assert rep.ok(), rep.summary()


@pytest.mark.parametrize("over", [dict(R=40, gamma=5, V=3000, d=256),
                                  dict(R=33, gamma=4, V=2001, d=64, rank=32)],
                         ids=["fused", "per-step"])
def test_rnn_cap_accept_parity(over):
    """Cap-accept verification of RNN drafts (the whole block verified with
    the draft's features, committed within the scheduled window) through the
    round driver, against the oracle."""
    cfg = synth.scaled(synth.config(2), **over)
    inp = synth.make_inputs(cfg, device="cpu")
    g = to_dev(inp)
    g["Wr"] = synth.rnn_weights(cfg, device=DEV, gain=3.0)
    buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=DEV, rnn=(cfg.rank, cfg.d, cfg.dtype))
    RD.run_round(g, buf, cfg.T, cfg.philox_seed, 4, scheduler=True, verify_mode="cap-accept",
                 head="rnn")
    torch.cuda.synchronize()
    assert D.get_status(buf.ws) == 0
    rep = PC.Report()
    feat = f(buf.feat)
    m, mfull = PC.check_verify_cap_accept(rep, n(buf.full), n(buf.ell), None, f(inp["target"]), 1,
                                          n(buf.x), n(buf.logp_d), n(buf.lse_d), f(inp["U"]),
                                          f(inp["W1"]), f(inp["W2t"]), cfg.T, cfg.philox_seed, 4,
                                          n(buf.m), n(buf.tau), n(buf.emitted),
                                          n(buf.next_anchor), n(buf.m_full), None, feat=feat)
    PC.check_pack(rep, n(buf.emitted), n(buf.tau), n(buf.cu_out), n(buf.flat_out), None, None,
                  n(buf.N_out)[0], "emitted")
    print(f"  {rep.summary()} cut={int((mfull > n(buf.ell)).sum())}", flush=True)
    assert rep.ok(), rep.summary()
    assert (mfull > n(buf.ell)).any()           # the window cut some requests


@pytest.mark.parametrize("r,V,dtype", [(64, 1000, torch.bfloat16), (256, 129280, torch.bfloat16),
                                       (48, 77, torch.float32), (256, 151936, torch.bfloat16)])
def test_w2_transpose_is_exact(r, V, dtype):
    """dspark_w2_transpose moves bits: W2t equals W2.T element for element."""
    g = torch.Generator(device="cpu").manual_seed(r * 7 + V)
    W2 = torch.randn(r, V, generator=g).to(dtype).to(DEV)
    W2t = torch.empty(V, r, dtype=dtype, device=DEV)
    D.w2_transpose(W2, W2t)
    torch.cuda.synchronize()
    ref = W2.t().contiguous()
    assert torch.equal(W2t.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       ref.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


def test_draft_from_w2_in_method_layout():
    """The draft fed W2 [r][V] through dspark_w2_transpose matches the oracle."""
    cfg = synth.scaled(synth.config(2), R=45, gamma=4, V=3072, d=32, rank=128)
    inp = synth.make_inputs(cfg, device="cpu")
    W2 = inp["W2t"].t().contiguous()                 # the method's layout, r x V
    W2t = torch.empty(cfg.V, cfg.rank, dtype=W2.dtype, device=DEV)
    D.w2_transpose(W2.to(DEV), W2t)
    torch.cuda.synchronize()
    inp2 = dict(inp)
    inp2["W2t"] = W2t.cpu()
    run_and_check(cfg, inp2)
