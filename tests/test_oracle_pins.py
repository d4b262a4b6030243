"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something it does not share code with:
an independent Philox implementation (rocRAND's header-only engine), the
Gumbel distribution, closed-form softmax / sigmoid evaluated by scipy, the
pages' worked example (Appendix A of the DSpark summary page), a brute-force
exact-rational transcription of the scheduler on tiny inputs, and invariants
of the method (causality of the early stop, greedy reduction, tau = m + 1,
acceptance rate = 1 - TV).  Losslessness is pinned in test_oracle_lossless.py.
"""
import json
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# the library takes the temperature as a float32; the pins use that value
T07 = float(np.float32(0.7))


# ---------------------------------------------------------------- Philox --
@pytest.fixture(scope="module")
def rocrand_pin(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("pin") / "rocrand_philox_pin")
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", "-I/opt/rocm/include",
                    os.path.join(HERE, "pins", "rocrand_philox_pin.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def test_philox_matches_rocrand(rocrand_pin):
    rng = np.random.default_rng(7)
    n = 3000
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64)
    ctr[:, 1] %= 2**30          # rocRAND's 64-bit offset spans counter words 0..1 only below 2^62
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64)
    ctr[:4] = [[0, 0, 0, 0], [1, 0, 0, 0], [0, 1, 0, 0], [5, 65539, 255, 7]]
    key[:4] = [[0, 0], [0, 0], [1, 2], [2**32 - 1, 123]]
    inp = "\n".join(" ".join(str(int(v)) for v in list(c) + list(k)) for c, k in zip(ctr, key))
    out = subprocess.run([rocrand_pin], input=inp, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()],
                   dtype=np.uint64)
    got = np.array([O.philox4x32_10(c, k) for c, k in zip(ctr, key)], dtype=np.uint64)
    assert ref.shape == got.shape
    np.testing.assert_array_equal(got, ref)


def test_stream_counter_assembly():
    # counter = (idx >> 2, k | tag << 16, request, lo32(round)), key = (lo32, hi32 of seed)
    seed, rnd = 0x123456789ABCDEF0, 0x1_0000_0005
    for tag, req, k, idx in [(1, 0, 1, 0), (2, 17, 16, 129279), (3, 1023, 15, 0), (7, 5, 3, 6)]:
        w = O.stream_word(seed, rnd, tag, req, k, idx)
        ref = O.philox4x32_10([idx >> 2, k | (tag << 16), req, rnd & 0xFFFFFFFF],
                              [seed & 0xFFFFFFFF, seed >> 32])[idx & 3]
        assert w == int(ref)


def test_gumbel_distribution():
    g = np.array([O.gumbel(3, 1, 2, r, 4, v) for r in range(40) for v in range(500)])
    assert np.isfinite(g).all()
    ks = stats.kstest(g, "gumbel_r")
    assert ks.pvalue > 1e-3, ks
    assert abs(g.mean() - np.euler_gamma) < 0.03


# -------------------------------------------------------------------- CGM --
@pytest.mark.parametrize("V", [8, 64, 129, 300, 1000])
def test_cgm_matches_softmax(V):
    rng = np.random.default_rng(V)
    score = rng.normal(0.0, 1.5, V)
    n = 200_000
    xs = O.cgm_batch(score, 11, 2, O.TAG_DRAFT_CHUNK, O.TAG_DRAFT_ELEM, 0, n, 3)
    assert xs.min() >= 0 and xs.max() < V
    p = special.softmax(score)
    counts = np.bincount(xs, minlength=V)
    exp = p * n
    # merge the low-expectation cells so that the chi-square approximation holds
    order = np.argsort(exp)
    cexp, ccnt, bins_e, bins_c = 0.0, 0, [], []
    for i in order:
        cexp += exp[i]
        ccnt += counts[i]
        if cexp >= 20:
            bins_e.append(cexp)
            bins_c.append(ccnt)
            cexp, ccnt = 0.0, 0
    if cexp > 0:
        bins_e[-1] += cexp
        bins_c[-1] += ccnt
    chi = stats.chisquare(bins_c, bins_e)
    assert chi.pvalue > 1e-4, chi


def test_cgm_single_chunk_is_plain_gumbel_max():
    rng = np.random.default_rng(1)
    for V in [1, 2, 7, 128]:
        score = rng.normal(size=V)
        for req in range(20):
            j, _ = O.cgm(score, 5, 0, O.TAG_BONUS_CHUNK, O.TAG_BONUS_ELEM, req, 2)
            keys = [score[v] + O.gumbel(5, 0, O.TAG_BONUS_ELEM, req, 2, v) for v in range(V)]
            assert j == int(np.argmax(keys))


def test_cgm_never_picks_zero_mass():
    score = np.full(700, -np.inf)
    allowed = np.array([3, 200, 201, 650])
    score[allowed] = [0.0, 1.0, -2.0, 0.5]
    xs = O.cgm_batch(score, 1, 0, O.TAG_RESID_CHUNK, O.TAG_RESID_ELEM, 0, 20000, 1)
    assert set(np.unique(xs)) <= set(allowed.tolist())
    p = special.softmax(score[allowed])
    freq = np.array([(xs == a).mean() for a in allowed])
    assert np.abs(freq - p).max() < 0.015


def test_cgm_temperature_to_zero_is_argmax():
    rng = np.random.default_rng(2)
    U = rng.normal(0, 2, (3, 4, 500)).astype(np.float32)
    x_small, _, _, _ = O.draft_markov(U, None, None, [0, 1, 2], T=1e-4)
    x_greedy, _, _, _ = O.draft_markov(U, None, None, [0, 1, 2], T=0.0)
    np.testing.assert_array_equal(x_small, x_greedy)
    np.testing.assert_array_equal(x_greedy[:, 1:], U.argmax(-1))


# ------------------------------------------------------------------ draft --
def test_draft_row_uniform_logits():
    V = 1000
    p = O.draft_row(np.full(V, 0.37, np.float32), None, None, 0, 1.0)
    np.testing.assert_allclose(p, 1.0 / V, rtol=0, atol=1e-15)


def test_draft_row_rank0_is_softmax():
    rng = np.random.default_rng(3)
    U = rng.normal(0, 3, 777).astype(np.float32)
    for T in [1.0, T07, 2.5]:
        p = O.draft_row(U, None, None, 0, T)
        np.testing.assert_allclose(p, special.softmax(U.astype(np.float64) / T), rtol=1e-12,
                                   atol=1e-300)


def test_draft_row_onehot_embedding_selects_W2_row():
    # W1[prev] = e_j  =>  bias = W2[j, :] = W2t[:, j]  (pins the W2 orientation)
    rng = np.random.default_rng(4)
    V, rank = 300, 16
    U = rng.normal(0, 1, V).astype(np.float32)
    W1 = np.zeros((V, rank), np.float32)
    W2t = rng.normal(0, 1, (V, rank)).astype(np.float32)
    prev, j = 42, 5
    W1[prev, j] = 1.0
    T = float(np.float32(0.9))
    p = O.draft_row(U, W1, W2t, prev, T)
    ref = special.softmax((U.astype(np.float64) + W2t[:, j]) / T)
    np.testing.assert_allclose(p, ref, rtol=1e-12)


def test_draft_row_low_rank_bias():
    rng = np.random.default_rng(5)
    V, rank = 500, 32
    U = rng.normal(0, 2, V).astype(np.float32)
    W1 = rng.normal(0, 0.3, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 0.3, (V, rank)).astype(np.float32)
    p = O.draft_row(U, W1, W2t, 17, 1.0)
    bias = W2t.astype(np.float64) @ W1[17].astype(np.float64)
    np.testing.assert_allclose(p, special.softmax(U + bias), rtol=1e-11)


def test_draft_zero_W2_equals_rank0():
    # a Markov head whose logit projection is zero reduces to the DFlash case
    rng = np.random.default_rng(6)
    R, g, V, rank = 3, 5, 700, 256
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    W1 = rng.normal(0, 0.02, (V, rank)).astype(np.float32)
    W2t = np.zeros((V, rank), np.float32)
    x0 = rng.integers(0, V, R)
    for T in [1.0, 0.0]:
        a = O.draft_markov(U, W1, W2t, x0, T, seed=9)
        b = O.draft_markov(U, None, None, x0, T, seed=9)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_draft_rank0_positions_independent():
    # markov_rank = 0: position k's token depends only on U_k and the stream,
    # not on the tokens drawn before it (DFlash: independent per-position sampling)
    rng = np.random.default_rng(7)
    R, g, V = 4, 6, 400
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    x_a = O.draft_markov(U, None, None, [1, 2, 3, 4], 1.0, seed=3)[0]
    x_b = O.draft_markov(U, None, None, [9, 8, 7, 6], 1.0, seed=3)[0]
    np.testing.assert_array_equal(x_a[:, 1:], x_b[:, 1:])
    for k in range(1, g + 1):
        for r in range(R):
            j, _ = O.cgm(U[r, k - 1].astype(np.float64), 3, 0, 1, 2, r, k)
            assert x_a[r, k] == j


def test_draft_logp_matches_distribution_and_chain():
    rng = np.random.default_rng(8)
    R, g, V, rank = 2, 4, 300, 16
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    W1 = rng.normal(0, 0.5, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 0.5, (V, rank)).astype(np.float32)
    x, lp, lse, _ = O.draft_markov(U, W1, W2t, [5, 6], 0.8, seed=1)
    for r in range(R):
        for k in range(1, g + 1):
            p = O.draft_row(U[r, k - 1], W1, W2t, x[r, k - 1], 0.8)
            assert abs(np.log(p[x[r, k]]) - lp[r, k - 1]) < 1e-10


def test_draft_greedy_chain():
    rng = np.random.default_rng(9)
    R, g, V, rank = 3, 4, 600, 32
    U = rng.normal(0, 1, (R, g, V)).astype(np.float32)
    W1 = rng.normal(0, 1, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 1, (V, rank)).astype(np.float32)
    x0 = np.array([1, 2, 3])
    x, lp, lse, _ = O.draft_markov(U, W1, W2t, x0, 0.0)
    for r in range(R):
        prev = x0[r]
        for k in range(1, g + 1):
            s = U[r, k - 1].astype(np.float64) + W2t.astype(np.float64) @ W1[prev].astype(np.float64)
            assert x[r, k] == int(np.argmax(s))
            assert lp[r, k - 1] == 0.0 and abs(lse[r, k - 1] - s.max()) < 1e-12
            prev = x[r, k]


def test_draft_empirical_first_position():
    # sampled tokens at position 1 follow the closed-form p_1(. | x_0)
    rng = np.random.default_rng(10)
    V, rank, n = 40, 8, 60000
    Uk = rng.normal(0, 1, V).astype(np.float32)
    W1 = rng.normal(0, 0.6, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 0.6, (V, rank)).astype(np.float32)
    U = np.broadcast_to(Uk, (n, 1, V))
    x, _, _, _ = O.draft_markov(U, W1, W2t, np.full(n, 3), 1.0, seed=4)
    p = O.draft_row(Uk, W1, W2t, 3, 1.0)
    chi = stats.chisquare(np.bincount(x[:, 1], minlength=V), p * n)
    assert chi.pvalue > 1e-4


# ------------------------------------------------------------- confidence --
def test_confidence_closed_form():
    rng = np.random.default_rng(11)
    R, g, d, V, rank = 3, 5, 64, 50, 16
    h = rng.normal(0, 1, (R, g, d)).astype(np.float32)
    W1 = rng.normal(0, 0.1, (V, rank)).astype(np.float32)
    w = rng.normal(0, 0.2, d + rank).astype(np.float32)
    x = rng.integers(0, V, (R, g + 1))
    c, z = O.confidence(h, W1, w, x)
    for r in range(R):
        for k in range(1, g + 1):
            feat = np.concatenate([h[r, k - 1], W1[x[r, k - 1]]]).astype(np.float64)
            zz = float(w.astype(np.float64) @ feat)
            assert abs(z[r, k - 1] - zz) < 1e-12
            assert c[r, k - 1] == np.float32(special.expit(zz))


def test_confidence_special_cases():
    R, g, d, V, rank = 2, 3, 8, 10, 4
    rng = np.random.default_rng(12)
    h = rng.normal(0, 1, (R, g, d)).astype(np.float32)
    W1 = rng.normal(0, 1, (V, rank)).astype(np.float32)
    x = rng.integers(0, V, (R, g + 1))
    c, _ = O.confidence(h, W1, np.zeros(d + rank, np.float32), x)
    assert (c == np.float32(0.5)).all()
    w = np.zeros(d + rank, np.float32)
    w[2] = 1.0
    sts = np.array([1.0, 2.0, 0.5], np.float32)
    c, _ = O.confidence(h, W1, w, x, sts)
    np.testing.assert_array_equal(c, special.expit(h[:, :, 2].astype(np.float64) / sts).astype(np.float32))
    # rank 0: the confidence vector has d entries only
    c0, _ = O.confidence(h, None, w[:d], x)
    np.testing.assert_array_equal(c0, special.expit(h[:, :, 2].astype(np.float64)).astype(np.float32))


# -------------------------------------------------------------- scheduler --
def test_appendix_a_worked_example():
    gold = json.load(open(os.path.join(HERE, "golden", "appendix_a.json")))
    sps = np.array(gold["sps"])
    for case in gold["cases"]:
        c = np.array([[gold["c1"], case["c2"]]], np.float32)
        ell, a, N, th, _ = O.prefix_schedule(c, sps, mode=0)
        assert ell[0] == case["ell_early_stop"]
        assert N == 1 + case["ell_early_stop"]
        assert abs(th - case["theta0"]) < 1e-12
        assert abs(a[0, 1] - case["a2"]) < 1e-6
        ell_g, _, _, th_g, _ = O.prefix_schedule(c, sps, mode=1)
        assert ell_g[0] == case["ell_global"]
        assert abs(th_g - max(case["theta0"], case["theta1"], case["theta2"])) < 1e-6
    # Theta_1 = (1 + a_1) * SPS(2) = 0.9 < Theta_0: the early stop fires at the first candidate
    c = np.array([[gold["c1"], 1.0]], np.float32)
    ell, _, _, th, _ = O.prefix_schedule(c, sps[:3], mode=0)
    assert ell[0] == 0 and th == 1.0


def _sched_bruteforce(c, sps, n_max, global_search=False):
    """Exact-rational transcription of the greedy scheduler (tiny inputs only).

    Survival a is the same float32 running product; the candidate order is
    Python's sort on (-a, r, j); tau and Theta are exact rationals built from
    the 2^-32 fixed-point amounts."""
    R, g = c.shape
    a = np.ones((R, g), np.float32)
    for r in range(R):
        acc = np.float32(1.0)
        for j in range(g):
            acc = np.float32(acc * np.float32(c[r, j]))
            a[r, j] = acc
    cands = sorted([(-float(a[r, j]), r, j + 1) for r in range(R) for j in range(g) if a[r, j] > 0])

    def theta(prefix_len):
        B = R + prefix_len
        if B > n_max:
            return Fraction(0)
        tau = Fraction(R)
        for q in range(prefix_len):
            tau += Fraction(int(np.rint(np.float64(-cands[q][0]) * 2.0**32)), 2**32)
        return tau * Fraction(sps[B])

    ell = [0] * R
    if not global_search:
        best = theta(0)
        for q in range(len(cands)):
            th = theta(q + 1)
            if th > best:
                best = th
                ell[cands[q][1]] = cands[q][2]
            else:
                break
    else:
        ths = [theta(q) for q in range(len(cands) + 1)]
        qbest = int(np.argmax([float(t) for t in ths]))
        best = ths[qbest]
        for q in range(qbest):
            ell[cands[q][1]] = cands[q][2]
    return np.array(ell), best


def _sps_curves(n_max):
    B = np.arange(n_max + 1, dtype=np.float64)
    yield 1.0 / (0.020 + 5e-5 * B)                        # the round's SPS form
    yield 1.0 / (0.02 + 0.004 * B)                        # steep: the early stop binds
    yield 1.0 / (0.015 + 4e-5 * B + 0.003 * (B // 3))     # discrete capacity steps
    yield np.concatenate([[0.0], np.sort(np.random.default_rng(n_max).uniform(0.2, 1.0, n_max))[::-1]])


@pytest.mark.parametrize("R,g", [(1, 1), (1, 4), (2, 2), (2, 3), (3, 2), (1, 6), (6, 1)])
def test_scheduler_exhaustive_grid(R, g):
    levels = np.array([0.0, 0.25, 0.5, 0.75, 1.0], np.float32)
    n_max = R * (g + 1)
    grid = np.array(np.meshgrid(*([levels] * (R * g)), indexing="ij")).reshape(R * g, -1).T
    rng = np.random.default_rng(R * 10 + g)
    sel = grid if len(grid) <= 4000 else grid[rng.choice(len(grid), 4000, replace=False)]
    for sps in _sps_curves(n_max):
        for flat in sel[:: max(1, len(sel) // 1500)]:
            c = flat.reshape(R, g).astype(np.float32)
            ell, _, N, th, mg = O.prefix_schedule(c, sps, n_max)
            ref, best = _sched_bruteforce(c, sps, n_max)
            if mg > 1e-12:
                np.testing.assert_array_equal(ell, ref)
                assert N == int((1 + ref).sum())
                assert th == float(best)


def test_scheduler_random_vs_bruteforce():
    rng = np.random.default_rng(13)
    for it in range(3000):
        R, g = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        c = rng.uniform(0, 1, (R, g)).astype(np.float32)
        c[rng.uniform(size=(R, g)) < 0.1] = 1.0
        n_max = int(rng.integers(R, R * (g + 1) + 1))
        sps = list(_sps_curves(R * (g + 1)))[it % 4]
        ell, _, N, th, mg = O.prefix_schedule(c, sps, n_max)
        ref, best = _sched_bruteforce(c, sps, n_max)
        if mg > 1e-12:
            np.testing.assert_array_equal(ell, ref)
        ellg, _, _, thg, _ = O.prefix_schedule(c, sps, n_max, mode=1)
        refg, bestg = _sched_bruteforce(c, sps, n_max, global_search=True)
        np.testing.assert_array_equal(ellg, refg)
        assert N <= n_max


def test_scheduler_causality_and_negative_control():
    # {ell_r >= j} must not change when c_{r,j+1..} are resampled: the early
    # stop never looks at a candidate beyond the one that stops it.
    rng = np.random.default_rng(14)
    B = np.arange(64, dtype=np.float64)
    sps_list = [1.0 / (0.02 + 0.01 * B), 1.0 / (0.015 + 0.004 * B + 0.01 * (B // 4))]
    violations_global = 0
    for it in range(1500):
        R, g = int(rng.integers(1, 5)), int(rng.integers(2, 6))
        sps = sps_list[it % 2]
        c = rng.uniform(0.3, 1.0, (R, g)).astype(np.float32)
        ell = O.prefix_schedule(c, sps)[0]
        ellg = O.prefix_schedule(c, sps, mode=1)[0]
        r = int(rng.integers(0, R))
        j = int(rng.integers(1, g))
        c2 = c.copy()
        c2[r, j:] = rng.uniform(0.0, 1.0, g - j).astype(np.float32)
        ell2 = O.prefix_schedule(c2, sps)[0]
        assert (ell[r] >= j) == (ell2[r] >= j)
        ellg2 = O.prefix_schedule(c2, sps, mode=1)[0]
        violations_global += int((ellg[r] >= j) != (ellg2[r] >= j))
    assert violations_global > 0   # the Appendix-A global search is not causal


def test_scheduler_invariants_and_disabled():
    rng = np.random.default_rng(15)
    R, g = 64, 16
    c = special.expit(rng.normal(0, 3.2, (R, g))).astype(np.float32)
    B = np.arange(R * (g + 1) + 1, dtype=np.float64)
    sps = 1.0 / (0.020 + 5e-5 * B)
    ell, a, N, th, _ = O.prefix_schedule(c, sps)
    assert (np.diff(a, axis=1) <= 0).all()
    assert N == int((1 + ell).sum())
    # Theta strictly increased along every admitted candidate
    adm = sorted([(-float(a[r, j - 1]), r, j) for r in range(R) for j in range(1, ell[r] + 1)])
    tau, best = R * 2**32, R * sps[R]
    for q, (na, r, j) in enumerate(adm):
        tau += int(np.rint(-na * 2.0**32))
        t = (tau * 2.0**-32) * sps[R + q + 1]
        assert t > best
        best = t
    assert best == th
    ell_d, _, N_d, _, _ = O.prefix_schedule(c, sps, enabled=False)
    assert (ell_d == g).all() and N_d == R * (g + 1)
    # capacity: N never exceeds N_max
    ell_c, _, N_c, _, _ = O.prefix_schedule(np.ones((R, g), np.float32), sps, N_max=R + 10)
    assert N_c <= R + 10


# ------------------------------------------------- asynchronous scheduler --
def _survival_f32(c):
    R, g = c.shape
    a = np.ones((R, g), np.float32)
    for r in range(R):
        acc = np.float32(1.0)
        for j in range(g):
            acc = np.float32(acc * np.float32(c[r, j]))
            a[r, j] = acc
    return a


def _theta_exact(a, ell, sps, n_max):
    """Theta of an arbitrary prefix schedule ell, as an exact rational (the
    2^-32 fixed-point amounts of a, no ordering involved)."""
    R = a.shape[0]
    B = R + int(sum(ell))
    if B > n_max:
        return Fraction(0)
    tau = Fraction(R)
    for r in range(R):
        for j in range(int(ell[r])):
            tau += Fraction(int(np.rint(np.float64(a[r, j]) * 2.0**32)), 2**32)
    return tau * Fraction(sps[B])


def test_async_appendix_a_plan():
    # Appendix A: the capacity plan is the global search of that example.
    gold = json.load(open(os.path.join(HERE, "golden", "appendix_a.json")))
    sps = np.array(gold["sps"])
    for case in gold["cases"]:
        c = np.array([[gold["c1"], case["c2"]]], np.float32)
        for K_in in range(0, 5):
            ell, _, N, th, K, thp = O.async_schedule(c, sps, K_in)
            assert K == 1 + case["ell_global"]
            assert abs(thp - max(case["theta0"], case["theta1"], case["theta2"])) < 1e-6
            npos = 2 if case["a2"] > 0 else 1
            assert int(ell.sum()) == max(0, min(min(K_in, 3) - 1, npos))
            assert N == 1 + int(ell.sum())
    # c2 = 0.9 with the capacity planned on the same round admits ell = 2, which
    # the early stop of Algorithm 1 never reaches (it stops at Theta_1 < Theta_0)
    c = np.array([[gold["c1"], 0.9]], np.float32)
    K = O.async_schedule(c, sps, 0)[4]
    assert O.async_schedule(c, sps, K)[0][0] == 2
    assert O.prefix_schedule(c, sps, mode=0)[0][0] == 0


@pytest.mark.parametrize("R,g", [(1, 3), (2, 2), (2, 3), (3, 2), (3, 3)])
def test_async_plan_is_optimum_over_all_prefix_schedules(R, g):
    """The planned capacity is the best verify batch over EVERY per-request
    prefix schedule (not only sorted prefixes): for a fixed batch size the
    largest tau takes the largest survivals, and monotone a keeps them a
    prefix.  Brute force over all (g+1)^R schedules, no sort involved."""
    import itertools
    rng = np.random.default_rng(100 * R + g)
    n_max = R * (g + 1)
    for it in range(150):
        c = rng.uniform(0, 1, (R, g)).astype(np.float32)
        c[rng.uniform(size=(R, g)) < 0.15] = 0.0
        c[rng.uniform(size=(R, g)) < 0.15] = 1.0
        sps = list(_sps_curves(n_max))[it % 4]
        nm = int(rng.integers(R, n_max + 1))
        a = _survival_f32(c)
        best, bestB = None, None
        for ell in itertools.product(range(g + 1), repeat=R):
            th = _theta_exact(a, ell, sps, nm)
            B = R + sum(ell)
            if best is None or th > best or (th == best and B < bestB):
                best, bestB = th, B
        _, _, _, _, K, thp = O.async_schedule(c, sps, 0, N_max=nm)
        assert thp == float(best)
        assert K == bestB
    # ties: with SPS(B) = 1/B and every c = 1, every schedule has Theta = 1;
    # the first maximum is the smallest batch
    Bv = np.arange(n_max + 1, dtype=np.float64)
    sps = 1.0 / np.maximum(Bv, 1.0)
    _, _, _, _, K, thp = O.async_schedule(np.ones((R, g), np.float32), sps, 0)
    assert K == R and thp == 1.0


def test_async_admission_is_topk():
    """The admitted set holds exactly min(K, N_max) - R candidates (clamped to
    [0, |E|]), every admitted survival precedes every rejected positive one in
    the (a desc, r, j) order, it is prefix-closed per request, and Theta is the
    admitted schedule's."""
    rng = np.random.default_rng(21)
    for it in range(1500):
        R, g = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        c = rng.uniform(0, 1, (R, g)).astype(np.float32)
        c[rng.uniform(size=(R, g)) < 0.1] = 0.0
        c[rng.uniform(size=(R, g)) < 0.1] = 1.0
        nm = int(rng.integers(R, R * (g + 1) + 3))
        sps = list(_sps_curves(nm))[it % 4]
        K_in = int(rng.integers(-2, R * (g + 1) + 4))
        ell, a, N, th, _, _ = O.async_schedule(c, sps, K_in, N_max=nm)
        np.testing.assert_array_equal(a, _survival_f32(c))
        pos = [(-float(a[r, j]), r, j + 1) for r in range(R) for j in range(g) if a[r, j] > 0]
        adm = [p for p in pos if p[2] <= ell[p[1]]]
        rej = [p for p in pos if p[2] > ell[p[1]]]
        assert len(adm) == int(ell.sum())            # every admitted position has a > 0
        assert len(adm) == max(0, min(min(K_in, nm) - R, len(pos)))
        if adm and rej:
            assert max(adm) < min(rej)
        assert N == R + len(adm) <= max(nm, R)
        assert th == float(_theta_exact(a, ell, sps, nm))


def test_async_reduces_to_algorithm1_and_global_search():
    """Given the batch size Algorithm 1 chose, the top-K admission returns
    Algorithm 1's schedule (it admits a prefix of the same order); given the
    capacity planned on the same round, it returns the global search's."""
    rng = np.random.default_rng(22)
    for it in range(800):
        R, g = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        c = special.expit(rng.normal(1.0, 2.0, (R, g))).astype(np.float32)
        sps = list(_sps_curves(R * (g + 1)))[it % 4]
        ell1, _, N1, th1, _ = O.prefix_schedule(c, sps, mode=0)
        ell, _, N, th, K, thp = O.async_schedule(c, sps, N1)
        np.testing.assert_array_equal(ell, ell1)
        assert N == N1 and th == th1
        ellg, _, Ng, thg, _ = O.prefix_schedule(c, sps, mode=1)
        ell2, _, N2, th2, _, _ = O.async_schedule(c, sps, K)
        np.testing.assert_array_equal(ell2, ellg)
        assert N2 == Ng == K and th2 == thg == thp
        assert thp >= th1                           # the global search never does worse


def test_async_causal_barrier_and_static_limits():
    """The number of admitted tokens depends only on the capacity handed in
    (and on how many candidates exist), never on this round's values; a
    capacity of the whole block verifies everything, one of R verifies the
    anchors only."""
    rng = np.random.default_rng(23)
    R, g = 12, 6
    B = np.arange(R * (g + 1) + 1, dtype=np.float64)
    sps = 1.0 / (0.015 + 4e-5 * B + 0.003 * (B // 5))
    for it in range(200):
        K_in = int(rng.integers(R, R * (g + 1) + 1))
        c1 = rng.uniform(0.05, 1.0, (R, g)).astype(np.float32)
        c2 = rng.uniform(0.05, 1.0, (R, g)).astype(np.float32)
        n1 = int(O.async_schedule(c1, sps, K_in)[0].sum())
        n2 = int(O.async_schedule(c2, sps, K_in)[0].sum())
        assert n1 == n2 == K_in - R
    c = rng.uniform(0.05, 1.0, (R, g)).astype(np.float32)
    assert (O.async_schedule(c, sps, R * (g + 1))[0] == g).all()
    assert (O.async_schedule(c, sps, R)[0] == 0).all()
    assert (O.async_schedule(c, sps, 0)[0] == 0).all()


# ------------------------------------------------------------------- pack --
def test_pack_identities():
    rng = np.random.default_rng(16)
    R, width = 37, 9
    rows = rng.integers(0, 1000, (R, width))
    lens = rng.integers(0, width + 1, R)
    cu, flat, mr, mp, N = O.pack(rows, lens)
    assert cu[0] == 0 and N == lens.sum() and cu[-1] == N
    assert (np.diff(cu) == lens).all()
    exp = np.concatenate([rows[r, :lens[r]] for r in range(R)])
    np.testing.assert_array_equal(flat[:N], exp)
    np.testing.assert_array_equal(mr[:N], np.repeat(np.arange(R), lens))
    np.testing.assert_array_equal(mp[:N], np.concatenate([np.arange(l) for l in lens]))
    assert (flat[N:] == -1).all() and (mr[N:] == -1).all() and (mp[N:] == -1).all()


# ----------------------------------------------------------------- verify --
def _markov_case(seed, R, g, V, rank, sig_t=0.5):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    W1 = rng.normal(0, 0.3, (V, rank)).astype(np.float32) if rank else None
    W2t = rng.normal(0, 0.3, (V, rank)).astype(np.float32) if rank else None
    tgt = np.concatenate([U, rng.normal(0, 2, (R, 1, V)).astype(np.float32)], axis=1)
    tgt = (tgt + rng.normal(0, sig_t, tgt.shape)).astype(np.float32)
    x0 = rng.integers(0, V, R)
    return U, W1, W2t, tgt, x0


def test_verify_greedy_reduction():
    R, g, V = 40, 5, 300
    U, W1, W2t, tgt, x0 = _markov_case(17, R, g, V, 8, sig_t=0.4)
    x, lp, lse, _ = O.draft_markov(U, W1, W2t, x0, 0.0)
    ell = np.random.default_rng(0).integers(0, g + 1, R)
    m, tau, em, na, lpt, _ = O.verify(ell, None, tgt, 1, x, lp, lse, U, W1, W2t, 0.0)
    for r in range(R):
        am = tgt[r].argmax(-1)
        mm = 0
        while mm < ell[r] and x[r, mm + 1] == am[mm]:
            mm += 1
        assert m[r] == mm and tau[r] == mm + 1
        np.testing.assert_array_equal(em[r, :mm], x[r, 1:mm + 1])
        assert em[r, mm] == am[mm] == na[r]
        assert (em[r, mm + 1:] == -1).all()


def test_verify_bookkeeping_and_layouts():
    R, g, V, rank = 12, 6, 500, 16
    U, W1, W2t, tgt, x0 = _markov_case(18, R, g, V, rank)
    x, lp, lse, _ = O.draft_markov(U, W1, W2t, x0, 1.0, seed=5)
    ell = np.random.default_rng(1).integers(0, g + 1, R)
    cu, flat, mr, mp, N = O.pack(x, ell + 1)
    packed = np.stack([tgt[mr[q], mp[q]] for q in range(N)])
    a = O.verify(ell, cu, packed, 0, x, lp, lse, U, W1, W2t, 1.0, seed=5)
    b = O.verify(ell, None, tgt, 1, x, lp, lse, U, W1, W2t, 1.0, seed=5)
    for p, q in zip(a, b):
        np.testing.assert_array_equal(p, q)
    m, tau, em, na, lpt, _ = a
    assert (tau == m + 1).all() and (m <= ell).all() and (m >= 0).all()
    for r in range(R):
        np.testing.assert_array_equal(em[r, :m[r]], x[r, 1:m[r] + 1])
        assert em[r, m[r]] == na[r] and 0 <= na[r] < V
        for k in range(1, ell[r] + 1):
            lt = tgt[r, k - 1].astype(np.float64)
            ref = lt[x[r, k]] - special.logsumexp(lt)
            assert abs(lpt[r, k - 1] - ref) < 1e-10


def test_verify_cap_accept_invariants():
    """Cap-accept commits a prefix of the full-window verification: m =
    min(m_full, cap), the committed tokens are the first m + 1 of the full
    window's, a cap at or above the window is plain verification, and at T = 0
    the committed tokens follow the target's argmax chain."""
    R, g, V, rank = 30, 6, 400, 16
    U, W1, W2t, tgt, x0 = _markov_case(19, R, g, V, rank, sig_t=0.3)
    rng = np.random.default_rng(2)
    for T in [1.0, 0.0]:
        x, lp, lse, _ = O.draft_markov(U, W1, W2t, x0, T, seed=6)
        ell = np.full(R, g, np.int32)
        cap = rng.integers(-1, g + 2, R).astype(np.int32)
        full = O.verify(ell, None, tgt, 1, x, lp, lse, U, W1, W2t, T, seed=6)
        m, tau, em, na, lpt, _, m_full = O.verify_cap_accept(ell, cap, None, tgt, 1, x, lp, lse, U,
                                                             W1, W2t, T, seed=6)
        np.testing.assert_array_equal(m_full, full[0])
        c = np.clip(cap, 0, g)
        np.testing.assert_array_equal(m, np.minimum(full[0], c))
        assert (tau == m + 1).all()
        np.testing.assert_array_equal(lpt, full[4])
        for r in range(R):
            np.testing.assert_array_equal(em[r, :tau[r]], full[2][r, :tau[r]])
            assert (em[r, tau[r]:] == -1).all() and na[r] == em[r, tau[r] - 1]
            if full[0][r] > c[r]:
                assert na[r] == x[r, c[r] + 1]          # the accepted draft closes the window
            if T == 0.0:
                am = tgt[r].argmax(-1)
                np.testing.assert_array_equal(em[r, :tau[r]], am[:tau[r]])
        same = O.verify_cap_accept(ell, np.full(R, g + 3), None, tgt, 1, x, lp, lse, U, W1, W2t,
                                   T, seed=6)
        for p_, q_ in zip(same[:5], full[:5]):
            np.testing.assert_array_equal(p_, q_)


def test_pack_tiered():
    rng = np.random.default_rng(3)
    for it in range(300):
        R, width = int(rng.integers(1, 20)), int(rng.integers(1, 9))
        rows = rng.integers(0, 1000, (R, width)).astype(np.int32)
        lens = rng.integers(0, width + 1, R).astype(np.int32)
        slots = R * width + int(rng.integers(0, 100))
        tiers = [t for t in [8, 16, 32, 64, 128] if t <= slots]
        cu, flat, mr, mp, N, N_pad, over = O.pack_tiered(rows, lens, tiers, 7, slots=slots)
        cu0, flat0, mr0, mp0, N0 = O.pack(rows, lens)
        assert N == N0 == int(lens.sum())
        np.testing.assert_array_equal(cu, cu0)
        np.testing.assert_array_equal(flat[:N], flat0[:N])
        np.testing.assert_array_equal(mr[:N], mr0[:N])
        np.testing.assert_array_equal(mp[:N], mp0[:N])
        bigger = [t for t in tiers if t >= N]
        assert over == (not bigger)
        assert N_pad == (bigger[0] if bigger else N)
        assert (flat[N:N_pad] == 7).all() and (flat[N_pad:] == -1).all() and flat.size == slots
        assert (mr[N:] == -1).all() and (mp[N:] == -1).all()


def test_verify_first_position_acceptance_rate():
    # P(accept x_1) = sum_v min(p_d, p_t) = 1 - TV(p_d, p_t)  (the confidence
    # head's training label c* on the DSpark summary page)
    rng = np.random.default_rng(19)
    V, rank, n = 300, 16, 40000
    Uk = rng.normal(0, 2, V).astype(np.float32)
    W1 = rng.normal(0, 0.3, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 0.3, (V, rank)).astype(np.float32)
    t1 = (Uk + rng.normal(0, 0.8, V)).astype(np.float32)
    U = np.broadcast_to(Uk, (n, 1, V))
    x, lp, lse, _ = O.draft_markov(U, W1, W2t, np.full(n, 7), 1.0, seed=2)
    tgt = np.broadcast_to(np.stack([t1, t1]), (n, 2, V))
    m, *_ = O.verify(np.ones(n, np.int32), None, tgt, 1, x, lp, lse, U, W1, W2t, 1.0, seed=2)
    p_d = O.draft_row(Uk, W1, W2t, 7, 1.0)
    p_t = special.softmax(t1.astype(np.float64))
    alpha = 1.0 - 0.5 * np.abs(p_d - p_t).sum()
    emp = (m == 1).mean()
    assert abs(emp - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / n), (emp, alpha)


def test_residual_row_closed_form():
    rng = np.random.default_rng(20)
    V = 257
    t = rng.normal(0, 1, V).astype(np.float32)
    s = rng.normal(0, 1, V)
    lse_d = special.logsumexp(s)
    for T in [1.0, float(np.float32(0.6))]:
        q, tot = O.residual_row(t, s, lse_d, T)
        pt = special.softmax(t.astype(np.float64) / T)
        pd = special.softmax(s)
        ref = np.maximum(pt - pd, 0)
        assert abs(tot - ref.sum()) < 1e-12
        np.testing.assert_allclose(q, ref / ref.sum(), atol=1e-14)
    # p_d == p_t: zero residual mass, falls back to p_t
    q, tot = O.residual_row(t, t.astype(np.float64), special.logsumexp(t.astype(np.float64)), 1.0)
    assert tot < 1e-15
    np.testing.assert_allclose(q, special.softmax(t.astype(np.float64)), atol=1e-15)


# ------------------------------------------------ acceptance rate c* --
def test_acceptance_rate_closed_forms():
    rng = np.random.default_rng(30)
    R, g, V = 3, 4, 500
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    x = np.concatenate([rng.integers(0, V, (R, 1)), rng.integers(0, V, (R, g))], 1)
    # rank 0, target row k-1 = U_k: identical distributions, c* = 1
    tgt = np.concatenate([U, U[:, :1]], axis=1)
    cs, _ = O.acceptance_rate(tgt, x, U, None, None, 1.0)
    np.testing.assert_allclose(cs, 1.0, rtol=0, atol=1e-12)
    # disjoint supports: c* = 0
    U2 = U.copy()
    U2[:, :, : V // 2] = -1e4
    tgt2 = np.full((R, g + 1, V), -1e4, np.float32)
    tgt2[:, :, : V // 2] = U[:, :1, : V // 2]            # target mass where the draft has none
    cs, _ = O.acceptance_rate(tgt2, x, U2, None, None, 0.8)
    assert np.abs(cs).max() == 0.0
    # rank 16: 1 - TV by scipy softmax of an independently computed bias
    rank = 16
    W1 = rng.normal(0, 0.4, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 0.4, (V, rank)).astype(np.float32)
    tgt3 = (np.concatenate([U, U[:, :1]], 1) + rng.normal(0, 1, (R, g + 1, V))).astype(np.float32)
    for T in [1.0, float(np.float32(0.6))]:
        cs, _ = O.acceptance_rate(tgt3, x, U, W1, W2t, T)
        for i in range(R):
            for k in range(1, g + 1):
                bias = W2t.astype(np.float64) @ W1[x[i, k - 1]].astype(np.float64)
                pd = special.softmax((U[i, k - 1].astype(np.float64) + bias) / T)
                pt = special.softmax(tgt3[i, k - 1].astype(np.float64) / T)
                assert abs(cs[i, k - 1] - (1 - 0.5 * np.abs(pd - pt).sum())) < 1e-12
    # T = 0: x_k against the target row's argmax
    cs, mg = O.acceptance_rate(tgt3, x, U, W1, W2t, 0.0)
    ref = (x[:, 1:] == tgt3[:, :g].argmax(-1)).astype(np.float64)
    np.testing.assert_array_equal(cs, ref)
    x2 = x.copy()
    x2[:, 1:] = tgt3[:, :g].argmax(-1)
    assert (O.acceptance_rate(tgt3, x2, U, W1, W2t, 0.0)[0] == 1.0).all()


def test_acceptance_rate_with_rnn_features():
    """With per-position bias features e_k (RNN head), c*_k = 1 - TV between
    softmax((U_k + W2^T e_k) / T) and the target row, both by scipy on an
    independently computed bias; the features replace W1[x_{k-1}] (W1 is not
    read: passing nonsense for it changes nothing)."""
    rng = np.random.default_rng(31)
    R, g, V, rank = 3, 4, 400, 16
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    x = np.concatenate([rng.integers(0, V, (R, 1)), rng.integers(0, V, (R, g))], 1)
    W2t = rng.normal(0, 0.4, (V, rank)).astype(np.float32)
    feat = np.tanh(rng.normal(0, 1, (R, g, rank))).astype(np.float32)
    tgt = (np.concatenate([U, U[:, :1]], 1) + rng.normal(0, 1, (R, g + 1, V))).astype(np.float32)
    junk = rng.normal(0, 5, (V, rank)).astype(np.float32)
    for T in [1.0, T07]:
        cs, _ = O.acceptance_rate(tgt, x, U, junk, W2t, T, feat=feat)
        for i in range(R):
            for k in range(1, g + 1):
                bias = W2t.astype(np.float64) @ feat[i, k - 1].astype(np.float64)
                pd = special.softmax((U[i, k - 1].astype(np.float64) + bias) / T)
                pt = special.softmax(tgt[i, k - 1].astype(np.float64) / T)
                assert abs(cs[i, k - 1] - (1 - 0.5 * np.abs(pd - pt).sum())) < 1e-12
        cs2, _ = O.acceptance_rate(tgt, x, U, None, W2t, T, feat=feat)
        np.testing.assert_array_equal(cs, cs2)


def test_acceptance_rate_is_the_verify_acceptance_probability():
    """c*_1 is the probability that the oracle's rejection test accepts x_1."""
    rng = np.random.default_rng(31)
    V, rank, n = 300, 16, 40000
    Uk = rng.normal(0, 2, V).astype(np.float32)
    W1 = rng.normal(0, 0.3, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 0.3, (V, rank)).astype(np.float32)
    t1 = (Uk + rng.normal(0, 0.8, V)).astype(np.float32)
    U = np.broadcast_to(Uk, (n, 1, V))
    x, lp, lse, _ = O.draft_markov(U, W1, W2t, np.full(n, 7), 1.0, seed=3)
    tgt = np.broadcast_to(np.stack([t1, t1]), (n, 2, V))
    m, *_ = O.verify(np.ones(n, np.int32), None, tgt, 1, x, lp, lse, U, W1, W2t, 1.0, seed=3)
    cs, _ = O.acceptance_rate(tgt[:1], x[:1], U[:1], W1, W2t, 1.0)
    alpha = cs[0, 0]
    emp = (m == 1).mean()
    assert abs(emp - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / n), (emp, alpha)


# ----------------------------------------------------------- STS fit --
def test_sts_fit_hand_example():
    # four blocks, one position, logit 0 (c = 0.5, bin 7 of 15), three accepted:
    # ECE = |4 * 0.5 - 3| / 4 = 0.25 at every temperature; the first grid value wins
    z = np.zeros((4, 1), np.float32)
    m = np.array([1, 1, 1, 0])
    t, ece, _ = O.sts_fit(z, m, [2.0, 1.0, 0.5])
    assert t[0] == 2.0 and ece[0] == 0.25
    # two positions by hand: z = (ln 3, 0): c_1 = 0.75, A_2 = 0.375 (bins 11 and 5)
    z = np.array([[np.log(3.0), 0.0]] * 4, np.float32)
    m = np.array([2, 1, 1, 0])
    t, ece, _ = O.sts_fit(z, m, [1.0])
    c1 = 1 / (1 + np.exp(-np.float64(np.float32(np.log(3.0)))))
    assert abs(ece[0] - abs(4 * c1 - 3) / 4) < 1e-15
    assert abs(ece[1] - abs(4 * c1 * 0.5 - 1) / 4) < 1e-15
    # two bins whose errors cancel in total: c = 0.75, 0.75 (bin 11) never
    # accepted, c = 0.25, 0.25 (bin 3) always accepted -> ECE = (1.5 + 1.5) / 4
    z = np.array([[np.log(3.0)], [np.log(3.0)], [-np.log(3.0)], [-np.log(3.0)]], np.float32)
    t, ece, _ = O.sts_fit(z, np.array([0, 0, 1, 1]), [1.0])
    assert abs(ece[0] - 0.75) < 1e-7
    # the top two bins kept apart: c = 0.9 (bin 13) always accepted, c = 0.98
    # (bin 14) never: ECE = (|1.8 - 2| + |1.96 - 0|) / 4
    z = np.array([[np.log(9.0)]] * 2 + [[np.log(49.0)]] * 2, np.float32)
    t, ece, _ = O.sts_fit(z, np.array([1, 1, 0, 0]), [1.0])
    assert abs(ece[0] - 0.54) < 1e-6


def _sts_data(rng, n, t_true, mu=1.5, sd=2.0):
    """Blocks whose true prefix-acceptance law is prod_j sigmoid(z_j / t*_j):
    position k is accepted (given the prefix) with probability sigmoid(z_k / t*_k)."""
    g = len(t_true)
    z = rng.normal(mu, sd, (n, g)).astype(np.float32)
    p = 1.0 / (1.0 + np.exp(-z.astype(np.float64) / np.asarray(t_true)))
    acc = rng.uniform(size=(n, g)) < p
    m = np.where(acc.all(1), g, np.argmin(acc, axis=1))
    return z, m


def test_sts_fit_recovers_true_temperatures():
    rng = np.random.default_rng(32)
    grid = np.round(np.arange(0.4, 3.01, 0.2), 6).astype(np.float32)
    t_true = [grid[3], grid[6], grid[10], grid[1], grid[8]]
    z, m = _sts_data(rng, 300_000, t_true)
    t, ece, _ = O.sts_fit(z, m, grid)
    np.testing.assert_array_equal(t, np.asarray(t_true, np.float32))
    assert (ece < 0.01).all()
    # an uncalibrated head (t = 1 everywhere) has a larger ECE at every
    # position whose true temperature is not 1
    t1, ece1, _ = O.sts_fit(z, m, [1.0])
    assert (ece1[1:] > 3 * ece[1:]).all() and ece1[0] == ece[0]   # t*_1 = 1.0


def test_sts_fit_left_to_right_freezing():
    """t_1..t_k depend only on labels of positions 1..k: accepted counts above
    k may change without moving them."""
    rng = np.random.default_rng(33)
    grid = np.linspace(0.5, 2.0, 16).astype(np.float32)
    z, m = _sts_data(rng, 20_000, [1.3, 0.7, 1.0, 1.6])
    t, _, _ = O.sts_fit(z, m, grid)
    for k in range(1, 4):
        m2 = np.where(m > k, k + rng.integers(0, 4 - k + 1, m.size), m)
        m2 = np.minimum(m2, 4)
        t2, _, _ = O.sts_fit(z, m2, grid)
        np.testing.assert_array_equal(t2[:k], t[:k])
    # order preservation: calibrated confidences rank as the raw logits do
    for k in range(4):
        c = 1 / (1 + np.exp(-z[:, k].astype(np.float64) / t[k]))
        assert (np.argsort(c, kind="stable") == np.argsort(z[:, k], kind="stable")).all()


# --------------------------------------------------------------- RNN head --
def _rnn_case(seed, R, g, V, rank, d):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    W1 = rng.normal(0, 0.5, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 0.3, (V, rank)).astype(np.float32)
    Wr = rng.normal(0, 0.3, (3 * rank, 2 * rank + d)).astype(np.float32)
    h = rng.normal(0, 1, (R, g, d)).astype(np.float32)
    x0 = rng.integers(0, V, R)
    return U, W1, W2t, Wr, h, x0


def test_rnn_zero_projection_is_the_rank0_draft():
    # Wr = 0: every feature is tanh(0) = 0, the bias vanishes (DFlash case)
    U, W1, W2t, Wr, h, x0 = _rnn_case(40, 4, 5, 600, 16, 8)
    for T in [1.0, 0.0]:
        a = O.draft_rnn(U, W1, W2t, np.zeros_like(Wr), h, x0, T, seed=3)
        b = O.draft_markov(U, None, None, x0, T, seed=3)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)
        assert np.abs(a[5]).max() == 0.0 and np.abs(a[6]).max() == 0.0


def test_rnn_closed_gate_is_a_markov_head_on_tanh_embeddings():
    """Gate saturated open-state (g = 1 exactly: s stays 0) and an output part
    that reads only the embedding: e_k = tanh(W1[x_{k-1}]), so the head is the
    Markov head with the table tanh(W1) (computed here by numpy)."""
    R, g, V, rank, d = 6, 5, 700, 16, 4
    U, W1, W2t, Wr, h, x0 = _rnn_case(41, R, g, V, rank, d)
    h[:, :, 0] = 1.0                                   # a constant feature
    Wr = np.zeros_like(Wr)
    Wr[:rank, 2 * rank] = 60.0                         # gate: sigmoid(60) == 1 in double
    Wr[rank:2 * rank] = np.random.default_rng(1).normal(0, 1, (rank, 2 * rank + d))
    Wr[2 * rank:, rank:2 * rank] = np.eye(rank)        # output: the embedding part
    W1t = np.tanh(W1.astype(np.float64)).astype(np.float32)
    for T in [1.0, T07, 0.0]:
        a = O.draft_rnn(U, W1, W2t, Wr, h, x0, T, seed=4, bf16_e=False)
        b = O.draft_markov(U, W1t, W2t, x0, T, seed=4, own=True)
        assert np.abs(a[6]).max() == 0.0               # the state never moves
        close = (b[3] > 1e-6)                          # decisions away from a tie
        assert (a[0][:, 1:][close] == b[0][:, 1:][close]).all()
        if T > 0:
            np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-6)


def test_rnn_state_and_features_layout():
    """Rows [0, r) of Wr are the gate, [r, 2r) the candidate, [2r, 3r) the
    output; z = [s ; W1[x] ; h].  Checked at k = 1 and k = 2 against numpy."""
    from scipy import special as sp
    R, g, V, rank, d = 3, 2, 200, 8, 5
    U, W1, W2t, Wr, h, x0 = _rnn_case(42, R, g, V, rank, d)
    x, _, _, _, _, e, s, _ = O.draft_rnn(U, W1, W2t, Wr, h, x0, 1.0, seed=5, bf16_e=False)
    W = Wr.astype(np.float64)
    for i in range(R):
        st = np.zeros(rank)
        for k in range(1, g + 1):
            z = np.concatenate([st, W1[x[i, k - 1]].astype(np.float64), h[i, k - 1]])
            gt = sp.expit(W[:rank] @ z)
            st = gt * st + (1 - gt) * np.tanh(W[rank:2 * rank] @ z)
            np.testing.assert_allclose(s[i, k - 1], st, rtol=0, atol=1e-12)
            np.testing.assert_allclose(e[i, k - 1], np.tanh(W[2 * rank:] @ z), rtol=0, atol=1e-12)


def test_rnn_bf16_features_and_memory():
    R, g, V, rank, d = 5, 4, 300, 16, 6
    U, W1, W2t, Wr, h, x0 = _rnn_case(43, R, g, V, rank, d)
    x, lp, lse, mg, xo, e, s, em = O.draft_rnn(U, W1, W2t, Wr, h, x0, 1.0, seed=6)
    xr, _, _, _, _, er, _, _ = O.draft_rnn(U, W1, W2t, Wr, h, x0, 1.0, seed=6, bf16_e=False)
    np.testing.assert_array_equal(x[:, :2], xr[:, :2])
    # e is the bf16 rounding (nearest even) of the unrounded feature: torch's
    # float32 -> bfloat16 conversion agrees wherever no float32 rounding sits
    # between the two
    import torch
    # the reported margin is the absolute distance of the unrounded feature to
    # the midpoint between its two neighbouring bf16 values (8 significant bits)
    a = np.abs(er[:, :1])
    ulp = np.exp2(np.floor(np.log2(a)) - 7)
    mid = np.floor(a / ulp) * ulp + ulp / 2
    np.testing.assert_allclose(em[:, :1], np.abs(a - mid), rtol=1e-9, atol=0)
    ref = torch.tensor(er[:, :1], dtype=torch.float32).to(torch.bfloat16).double().numpy()
    ok = em[:, :1] > 1e-6
    assert ok.mean() > 0.99
    np.testing.assert_array_equal(e[:, :1][ok], ref[ok])
    # memory: e_3 depends on x_1 with x_2 held fixed (a Markov head cannot)
    f1 = x.copy()
    f1[:, 1] = (x[:, 1] + 1) % V
    f1[:, 3:] = -1
    _, _, _, _, _, e2, _, _ = O.draft_rnn(U, W1, W2t, Wr, h, x0, 1.0, seed=6, force_x=f1)
    assert (np.abs(e2[:, 2] - e[:, 2]).max(axis=1) > 0).all()


def test_cap_accept_with_rnn_features_is_a_prefix_of_the_feature_verify():
    """Cap-accept of RNN drafts: the committed tokens are the first
    min(m, C) + 1 of the feature verify's sequence, and differ from a
    feature-less verify's where a residual was drawn."""
    R, g, V, rank, d = 40, 4, 300, 16, 6
    rng = np.random.default_rng(44)
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    W1 = rng.normal(0, 0.5, (V, rank)).astype(np.float32)
    W2t = rng.normal(0, 0.5, (V, rank)).astype(np.float32)
    Wr = rng.normal(0, 0.4, (3 * rank, 2 * rank + d)).astype(np.float32)
    h = rng.normal(0, 1, (R, g, d)).astype(np.float32)
    x0 = rng.integers(0, V, R)
    x, lp, lse, _, _, e, _, _ = O.draft_rnn(U, W1, W2t, Wr, h, x0, 1.0, seed=8)
    tgt = (np.concatenate([U, U[:, :1]], 1) + rng.normal(0, 1, (R, g + 1, V))).astype(np.float32)
    ell = np.full(R, g, np.int32)
    cap = rng.integers(0, g + 1, R).astype(np.int32)
    m, tau, em, na, _, _ = O.verify(ell, None, tgt, 1, x, lp, lse, U, W1, W2t, 1.0, seed=8, feat=e)
    mc, tc, ec, nc, _, _, mf = O.verify_cap_accept(ell, cap, None, tgt, 1, x, lp, lse, U, W1, W2t,
                                                   1.0, seed=8, feat=e)
    np.testing.assert_array_equal(mf, m)
    np.testing.assert_array_equal(mc, np.minimum(m, cap))
    for i in range(R):
        np.testing.assert_array_equal(ec[i, :tc[i]], em[i, :tc[i]] if tc[i] <= tau[i]
                                      else x[i, 1:tc[i] + 1])
        if mc[i] < cap[i]:                    # not cut by the window: plain verification
            assert tc[i] == tau[i] and nc[i] == na[i]
        else:                                  # cut: the last committed token is the draft x_{C+1}
            assert nc[i] == x[i, mc[i] + 1] if mc[i] < m[i] else nc[i] == na[i]
    _, _, e2, *_ = O.verify_cap_accept(ell, cap, None, tgt, 1, x, lp, lse, U, W1, W2t, 1.0, seed=8)
    assert (e2 != ec).any()
