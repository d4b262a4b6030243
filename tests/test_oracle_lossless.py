"""Losslessness pins of the oracle (CPU only).

A speculative round with rejection-sampling verification must emit tokens
distributed exactly as the target model's own autoregressive sampling (the
acceptance rule on the DSpark summary page, Background; residual and bonus
rules in section 2.2 of the MTP survey page), and the early-stopping prefix
scheduler must keep that property (DSpark summary page, Method details: greedy
solution and causality; Appendix A).

Setting: vocabulary of 8, block size 3, one request per round, a Markov draft
head and an x-dependent confidence head, and a target whose next-token
distribution depends on the whole in-block prefix.  Each round is completed to
gamma + 1 tokens by sampling the target, so that every round yields a sequence
of gamma + 1 tokens whose law must equal the product of target conditionals.

* exact enumeration: builds the law of the emitted sequence from the oracle's
  draft distribution, residual distribution, confidence head and scheduler,
  with acceptance probability min(1, p_t / p_d); must equal the target law to
  1e-12.  The Appendix-A global search (no early stop) must fail.
* Monte Carlo: runs the oracle's sampled draft + verify path and compares the
  empirical law of the completed sequences with the target law (chi-square).
"""
import itertools

import numpy as np
import pytest
from scipy import special, stats

import oracle as O

V, G, RANK, D = 8, 3, 4, 6

# the library takes the temperature as a float32; the pins use that value
T07 = float(np.float32(0.7))


def _setup(seed):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 1.2, (G, V)).astype(np.float32)
    W1 = rng.normal(0, 0.8, (V, RANK)).astype(np.float32)
    W2t = rng.normal(0, 0.8, (V, RANK)).astype(np.float32)
    h = rng.normal(0, 1, (G, D)).astype(np.float32)
    w = rng.normal(0, 0.8, D + RANK).astype(np.float32)
    # target logits for every in-block prefix: tl[prefix tuple] -> [V]
    tl = {}
    for j in range(G + 2):
        for pre in itertools.product(range(V), repeat=j):
            base = U[min(j, G - 1)]
            tl[pre] = (base + rng.normal(0, 0.9, V)).astype(np.float32)
    return U, W1, W2t, h, w, tl


_PT_CACHE = {}


def _pt(tl, pre, T):
    key = (id(tl), tuple(pre), T)
    if key not in _PT_CACHE:
        _PT_CACHE[key] = special.softmax(tl[tuple(pre)].astype(np.float64) / T)
    return _PT_CACHE[key]


def _complete(tl, emitted_law, T):
    """Extend a law over emitted prefixes to gamma + 1 tokens with target sampling."""
    law = {}
    for e, pe in emitted_law.items():
        for tail in itertools.product(range(V), repeat=G + 1 - len(e)):
            seq = e + tail
            pc = pe
            for j in range(len(e), G + 1):
                pc *= _pt(tl, seq[:j], T)[seq[j]]
            law[seq] = law.get(seq, 0.0) + pc
    return law


def _target_law(tl, T):
    return _complete(tl, {(): 1.0}, T)


def _enumerate_round(U, W1, W2t, h, w, tl, T, sps, anchor, scheduler_mode):
    emitted_law = {}
    for xs in itertools.product(range(V), repeat=G):
        x = (anchor,) + xs
        pd = [O.draft_row(U[k - 1], W1, W2t, x[k - 1], T) for k in range(1, G + 1)]
        p_draft = np.prod([pd[k - 1][x[k]] for k in range(1, G + 1)])
        if scheduler_mode is None:
            ell = G
        else:
            c, _ = O.confidence(h[None], W1, w, np.array([x]))
            ell = int(O.prefix_schedule(c, sps, mode=scheduler_mode)[0][0])
        # P(m = j, y) for the verification of positions 1..ell
        outcomes = []
        p_reach = 1.0
        for k in range(1, ell + 1):
            pt = _pt(tl, x[1:k], T)
            alpha = min(1.0, pt[x[k]] / pd[k - 1][x[k]])
            s = np.log(pd[k - 1])          # tempered draft scores up to a constant
            q, _ = O.residual_row(tl[tuple(x[1:k])], s, 0.0, T)
            outcomes.append((k - 1, p_reach * (1.0 - alpha), q))
            p_reach *= alpha
        outcomes.append((ell, p_reach, _pt(tl, x[1:ell + 1], T)))
        for m, pm, ydist in outcomes:
            if pm == 0.0:
                continue
            for y in range(V):
                e = tuple(int(t) for t in x[1:m + 1]) + (y,)
                emitted_law[e] = emitted_law.get(e, 0.0) + p_draft * pm * ydist[y]
    return _complete(tl, emitted_law, T)


def _sps_dynamic():
    # with anchor 5 the cut is 2 or 3 depending on the drafted tokens
    return np.array([0.0, 1.0, 0.9, 0.82, 0.77])


def _sps_appendix_a_like():
    # dip then rise: the global search's choice depends on c_2, i.e. on x_1
    return np.array([0.0, 1.0, 0.5, 0.45, 0.44])


@pytest.mark.parametrize("T,mode", [(1.0, None), (1.0, 0), (T07, 0)])
def test_exact_enumeration_lossless(T, mode):
    U, W1, W2t, h, w, tl = _setup(31)
    sps = _sps_dynamic()
    law = _enumerate_round(U, W1, W2t, h, w, tl, T, sps, anchor=5, scheduler_mode=mode)
    ref = _target_law(tl, T)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    tv = 0.5 * sum(abs(law.get(s, 0.0) - p) for s, p in ref.items())
    assert tv < 1e-12, tv
    if mode == 0:
        # the schedule must actually vary with the drafted tokens
        ells = set()
        for xs in itertools.product(range(V), repeat=G):
            c, _ = O.confidence(h[None], W1, w, np.array([(5,) + xs]))
            ells.add(int(O.prefix_schedule(c, sps)[0][0]))
        assert len(ells) >= 2, ells


def test_exact_enumeration_global_search_is_biased():
    U, W1, W2t, h, w, tl = _setup(31)
    w = w.copy()
    w[D:] *= 4.0            # make c_2 depend strongly on x_1
    sps = _sps_appendix_a_like()
    law = _enumerate_round(U, W1, W2t, h, w, tl, 1.0, sps, anchor=0, scheduler_mode=1)
    ref = _target_law(tl, 1.0)
    tv = 0.5 * sum(abs(law.get(s, 0.0) - p) for s, p in ref.items())
    assert tv > 1e-4, tv
    law0 = _enumerate_round(U, W1, W2t, h, w, tl, 1.0, sps, anchor=0, scheduler_mode=0)
    tv0 = 0.5 * sum(abs(law0.get(s, 0.0) - p) for s, p in ref.items())
    assert tv0 < 1e-12


@pytest.mark.parametrize("T", [1.0, T07])
def test_monte_carlo_sampled_path_lossless(T):
    U, W1, W2t, h, w, tl = _setup(31)
    n = 120_000
    anchor = 5
    Ub = np.broadcast_to(U, (n, G, V))
    x, lp, lse, _ = O.draft_markov(Ub, W1, W2t, np.full(n, anchor), T, seed=77, rnd=3)
    c, _ = O.confidence(np.broadcast_to(h, (n, G, D)), W1, w, x)
    sps = _sps_dynamic()
    ell = np.array([O.prefix_schedule(c[i:i + 1], sps)[0][0] for i in range(n)], np.int32)
    # target rows for every verify position, conditioned on the drafted prefix
    keys = list(tl.keys())
    index = {k: i for i, k in enumerate(keys)}
    table = np.stack([tl[k] for k in keys])
    rows = np.zeros((n, G + 1), np.int64)
    for j in range(G + 1):
        rows[:, j] = [index[tuple(x[i, 1:j + 1])] for i in range(n)]
    tgt = table[rows]
    m, tau, em, na, _, _ = O.verify(ell, None, tgt, 1, x, lp, lse, Ub, W1, W2t, T, seed=77, rnd=3)
    assert np.unique(ell).size >= 2
    rng = np.random.default_rng(99)
    seqs = np.full((n, G + 1), -1, np.int64)
    for i in range(n):
        s = list(em[i, :tau[i]])
        while len(s) < G + 1:
            p = _pt(tl, s, T)
            s.append(int(rng.choice(V, p=p)))
        seqs[i] = s
    codes = (seqs * (V ** np.arange(G, -1, -1))).sum(1)
    counts = np.bincount(codes, minlength=V ** (G + 1))
    ref = _target_law(tl, T)
    probs = np.zeros(V ** (G + 1))
    for s, p in ref.items():
        probs[int(sum(v * V ** (G - j) for j, v in enumerate(s)))] = p
    order = np.argsort(probs)
    be, bc, ce, cc = [], [], 0.0, 0
    for i in order:
        ce += probs[i] * n
        cc += counts[i]
        if ce >= 10:
            be.append(ce)
            bc.append(cc)
            ce, cc = 0.0, 0
    be[-1] += ce
    bc[-1] += cc
    chi = stats.chisquare(bc, be)
    assert chi.pvalue > 1e-4, chi


def _enumerate_cap_accept(U, W1, W2t, h, w, tl, T, sps, anchor):
    """Law of the committed tokens of a cap-accept round: every position of
    the block is verified, the commit window is Algorithm 1's ell; when more
    than ell drafts were accepted the committed tokens are x_1..x_{ell+1}."""
    emitted_law = {}
    for xs in itertools.product(range(V), repeat=G):
        x = (anchor,) + xs
        pd = [O.draft_row(U[k - 1], W1, W2t, x[k - 1], T) for k in range(1, G + 1)]
        p_draft = np.prod([pd[k - 1][x[k]] for k in range(1, G + 1)])
        c, _ = O.confidence(h[None], W1, w, np.array([x]))
        cap = int(O.prefix_schedule(c, sps, mode=0)[0][0])
        p_reach = 1.0
        outcomes = []
        for k in range(1, G + 1):
            pt = _pt(tl, x[1:k], T)
            alpha = min(1.0, pt[x[k]] / pd[k - 1][x[k]])
            q, _ = O.residual_row(tl[tuple(x[1:k])], np.log(pd[k - 1]), 0.0, T)
            outcomes.append((k - 1, p_reach * (1.0 - alpha), q))
            p_reach *= alpha
        outcomes.append((G, p_reach, _pt(tl, x[1:G + 1], T)))
        for m, pm, ydist in outcomes:
            if pm == 0.0:
                continue
            if m > cap:
                e = tuple(int(t) for t in x[1:cap + 2])
                emitted_law[e] = emitted_law.get(e, 0.0) + p_draft * pm
                continue
            for y in range(V):
                e = tuple(int(t) for t in x[1:m + 1]) + (y,)
                emitted_law[e] = emitted_law.get(e, 0.0) + p_draft * pm * ydist[y]
    return _complete(tl, emitted_law, T)


@pytest.mark.parametrize("T", [1.0, T07])
def test_exact_enumeration_cap_accept_lossless(T):
    U, W1, W2t, h, w, tl = _setup(31)
    law = _enumerate_cap_accept(U, W1, W2t, h, w, tl, T, _sps_dynamic(), anchor=5)
    ref = _target_law(tl, T)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    tv = 0.5 * sum(abs(law.get(s, 0.0) - p) for s, p in ref.items())
    assert tv < 1e-12, tv


def test_monte_carlo_cap_accept_lossless():
    """The oracle's sampled cap-accept path (full-block verify, commit within
    Algorithm 1's window) against the target law."""
    T = 1.0
    U, W1, W2t, h, w, tl = _setup(31)
    n = 120_000
    anchor = 5
    Ub = np.broadcast_to(U, (n, G, V))
    x, lp, lse, _ = O.draft_markov(Ub, W1, W2t, np.full(n, anchor), T, seed=78, rnd=4)
    c, _ = O.confidence(np.broadcast_to(h, (n, G, D)), W1, w, x)
    sps = _sps_dynamic()
    cap = np.array([O.prefix_schedule(c[i:i + 1], sps)[0][0] for i in range(n)], np.int32)
    keys = list(tl.keys())
    index = {k: i for i, k in enumerate(keys)}
    table = np.stack([tl[k] for k in keys])
    rows = np.zeros((n, G + 1), np.int64)
    for j in range(G + 1):
        rows[:, j] = [index[tuple(x[i, 1:j + 1])] for i in range(n)]
    tgt = table[rows]
    full = np.full(n, G, np.int32)
    m, tau, em, na, _, _, m_full = O.verify_cap_accept(full, cap, None, tgt, 1, x, lp, lse, Ub,
                                                       W1, W2t, T, seed=78, rnd=4)
    assert (m_full > cap).any() and (m == np.minimum(m_full, cap)).all()
    rng = np.random.default_rng(98)
    seqs = np.full((n, G + 1), -1, np.int64)
    for i in range(n):
        s = list(em[i, :tau[i]])
        while len(s) < G + 1:
            s.append(int(rng.choice(V, p=_pt(tl, s, T))))
        seqs[i] = s
    codes = (seqs * (V ** np.arange(G, -1, -1))).sum(1)
    counts = np.bincount(codes, minlength=V ** (G + 1))
    probs = np.zeros(V ** (G + 1))
    for s, p in _target_law(tl, T).items():
        probs[int(sum(v * V ** (G - j) for j, v in enumerate(s)))] = p
    order = np.argsort(probs)
    be, bc, ce, cc = [], [], 0.0, 0
    for i in order:
        ce += probs[i] * n
        cc += counts[i]
        if ce >= 10:
            be.append(ce)
            bc.append(cc)
            ce, cc = 0.0, 0
    be[-1] += ce
    bc[-1] += cc
    chi = stats.chisquare(bc, be)
    assert chi.pvalue > 1e-4, chi


def test_monte_carlo_rnn_draft_lossless():
    """Sampled RNN-head drafts verified with the residual rebuilt from the
    draft's features: the emitted law is the target's."""
    T = 1.0
    U, W1, W2t, h, w, tl = _setup(31)
    rng = np.random.default_rng(5)
    Wr = rng.normal(0, 0.6, (3 * RANK, 2 * RANK + D)).astype(np.float32)
    n = 120_000
    anchor = 5
    Ub = np.broadcast_to(U, (n, G, V))
    hb = np.broadcast_to(h, (n, G, D))
    x, lp, lse, _, _, e, _, _ = O.draft_rnn(Ub, W1, W2t, Wr, hb, np.full(n, anchor), T, seed=79,
                                            rnd=5)
    keys = list(tl.keys())
    index = {k: i for i, k in enumerate(keys)}
    table = np.stack([tl[k] for k in keys])
    rows = np.zeros((n, G + 1), np.int64)
    for j in range(G + 1):
        rows[:, j] = [index[tuple(x[i, 1:j + 1])] for i in range(n)]
    tgt = table[rows]
    ell = np.full(n, G, np.int32)
    m, tau, em, na, _, _ = O.verify(ell, None, tgt, 1, x, lp, lse, Ub, W1, W2t, T, seed=79, rnd=5,
                                    feat=e)
    rng2 = np.random.default_rng(97)
    seqs = np.full((n, G + 1), -1, np.int64)
    for i in range(n):
        s = list(em[i, :tau[i]])
        while len(s) < G + 1:
            s.append(int(rng2.choice(V, p=_pt(tl, s, T))))
        seqs[i] = s
    codes = (seqs * (V ** np.arange(G, -1, -1))).sum(1)
    counts = np.bincount(codes, minlength=V ** (G + 1))
    probs = np.zeros(V ** (G + 1))
    for s_, p in _target_law(tl, T).items():
        probs[int(sum(v * V ** (G - j) for j, v in enumerate(s_)))] = p
    order = np.argsort(probs)
    be, bc, ce, cc = [], [], 0.0, 0
    for i in order:
        ce += probs[i] * n
        cc += counts[i]
        if ce >= 10:
            be.append(ce)
            bc.append(cc)
            ce, cc = 0.0, 0
    be[-1] += ce
    bc[-1] += cc
    chi = stats.chisquare(bc, be)
    assert chi.pvalue > 1e-4, chi
    # the same drafts verified as if they came from a Markov head (features
    # ignored) emit a different law
    m2, tau2, em2, *_ = O.verify(ell, None, tgt, 1, x, lp, lse, Ub, W1, W2t, T, seed=79, rnd=5)
    assert (em2 != em).any()


def _rnn_setup(seed):
    U, W1, W2t, h, w, tl = _setup(seed)
    rng = np.random.default_rng(seed + 100)
    Wr = rng.normal(0, 0.6, (3 * RANK, 2 * RANK + D)).astype(np.float32)
    return U, W1, W2t, Wr, h, w, tl


def _rnn_draft_conditionals(U, W1, W2t, Wr, h, anchor, T):
    """p_d(. | x_1..x_{k-1}) of the oracle's RNN head for every in-block prefix,
    from log p_d of every candidate token forced after every prefix (the
    features, and so the distribution, depend on the whole prefix)."""
    seqs = list(itertools.product(range(V), repeat=G))
    X = np.array([(anchor,) + s for s in seqs], np.int32)
    n = len(seqs)
    out = O.draft_rnn(np.broadcast_to(U, (n, G, V)), W1, W2t, Wr, np.broadcast_to(h, (n, G, D)),
                      X[:, 0], T, force_x=X)
    lp = out[1]
    cond = {}
    for i, s in enumerate(seqs):
        for k in range(1, G + 1):
            cond.setdefault(s[:k - 1], np.zeros(V))[s[k - 1]] = np.exp(lp[i, k - 1])
    for pre, p in cond.items():
        assert abs(p.sum() - 1.0) < 1e-12, (pre, p.sum())
    return cond


def _enumerate_round_rnn(U, W1, W2t, Wr, h, w, tl, T, sps, anchor, scheduler_mode,
                         residual_from_markov=False):
    cond = _rnn_draft_conditionals(U, W1, W2t, Wr, h, anchor, T)
    emitted_law = {}
    for xs in itertools.product(range(V), repeat=G):
        x = (anchor,) + xs
        pd = [cond[xs[:k - 1]] for k in range(1, G + 1)]
        p_draft = np.prod([pd[k - 1][x[k]] for k in range(1, G + 1)])
        if scheduler_mode is None:
            ell = G
        else:
            c, _ = O.confidence(h[None], W1, w, np.array([x]))
            ell = int(O.prefix_schedule(c, sps, mode=scheduler_mode)[0][0])
        outcomes = []
        p_reach = 1.0
        for k in range(1, ell + 1):
            pt = _pt(tl, x[1:k], T)
            alpha = min(1.0, pt[x[k]] / pd[k - 1][x[k]])
            # the residual uses the distribution the draft sampled from; the
            # negative control rebuilds it as a Markov head would (W1[x_{k-1}] only)
            pr = O.draft_row(U[k - 1], np.tanh(W1), W2t, x[k - 1], T) if residual_from_markov \
                else pd[k - 1]
            q, _ = O.residual_row(tl[tuple(x[1:k])], np.log(pr), 0.0, T)
            outcomes.append((k - 1, p_reach * (1.0 - alpha), q))
            p_reach *= alpha
        outcomes.append((ell, p_reach, _pt(tl, x[1:ell + 1], T)))
        for m, pm, ydist in outcomes:
            if pm == 0.0:
                continue
            for y in range(V):
                e = tuple(int(t) for t in x[1:m + 1]) + (y,)
                emitted_law[e] = emitted_law.get(e, 0.0) + p_draft * pm * ydist[y]
    return _complete(tl, emitted_law, T)


@pytest.mark.parametrize("T,mode", [(1.0, None), (1.0, 0), (T07, 0)])
def test_exact_enumeration_lossless_rnn_head(T, mode):
    """RNN-head drafts (a distribution at each position that depends on the
    whole prefix), verified with the residual of the sampled distribution and
    scheduled by Algorithm 1 on x-dependent confidences: the emitted law is the
    target's to 1e-12; rebuilding the residual without the features is not."""
    U, W1, W2t, Wr, h, w, tl = _rnn_setup(31)
    sps = _sps_dynamic()
    law = _enumerate_round_rnn(U, W1, W2t, Wr, h, w, tl, T, sps, 5, mode)
    ref = _target_law(tl, T)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    tv = 0.5 * sum(abs(law.get(s, 0.0) - p) for s, p in ref.items())
    assert tv < 1e-12, tv
    bad = _enumerate_round_rnn(U, W1, W2t, Wr, h, w, tl, T, sps, 5, mode,
                               residual_from_markov=True)
    tv_bad = 0.5 * sum(abs(bad.get(s, 0.0) - p) for s, p in ref.items())
    assert tv_bad > 1e-4, tv_bad
