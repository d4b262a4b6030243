"""Lock-step parity of a GPU round against the CPU oracle (test infrastructure).

Used by tests/, __graft_entry__.smoke() and nothing in the product path.
Every stage is checked on the inputs the GPU stage itself consumed (the GPU's
own upstream outputs), so each stage is compared in isolation:

  draft       oracle re-runs the chain forced onto the GPU's tokens and reports
              its own choice at every position; a different choice is allowed
              only where the oracle's decision margin is below MARGIN (flagged)
  rnn draft   as draft, after the states and the bf16 features of the RNN
              head are checked (check_draft_rnn)
  confidence  float32 relative error <= TOL_REL
  schedule    ell, a, N, Theta bit-exact on the GPU's float32 confidences
  pack        bit-exact
  verify      m, tau, emitted, next anchor bit-exact, except requests whose
              oracle margin is below MARGIN (flagged); log p_t within TOL_LOG
  commit pack bit-exact
Probabilities are compared in log space: |d log p| <= 1e-5 is a relative error
of 1e-5 on p.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle as O

MARGIN = 1e-5
TOL_REL = 1e-5
TOL_LOG = 1e-5


@dataclass
class Report:
    """Decisions are counted per kind ("draft" token picks, "verify" requests,
    "rnn_e" bf16 feature roundings): `compared[kind]` decisions were checked and
    `flagged[kind]` of them differed from the oracle at a position whose oracle
    margin is below MARGIN.  Each kind must keep flagged <= 0.001 * compared
    (no allowance beyond that); any other difference is an error."""
    compared: dict = field(default_factory=dict)
    flagged: dict = field(default_factory=dict)
    errors: list = field(default_factory=list)
    max_err: dict = field(default_factory=dict)

    def err(self, msg):
        self.errors.append(msg)

    def note(self, key, val):
        self.max_err[key] = max(self.max_err.get(key, 0.0), float(val))

    def count(self, kind, compared, flagged=0):
        self.compared[kind] = self.compared.get(kind, 0) + int(compared)
        self.flagged[kind] = self.flagged.get(kind, 0) + int(flagged)

    def flag_ok(self):
        return all(self.flagged.get(k, 0) <= 0.001 * self.compared.get(k, 0) for k in self.flagged)

    def ok(self):
        return not self.errors and self.flag_ok()

    def total_flagged(self):
        return sum(self.flagged.values())

    def summary(self):
        kinds = " ".join(f"{k}={self.flagged.get(k, 0)}/{self.compared.get(k, 0)}"
                         for k in sorted(self.compared))
        return (f"flagged/compared: {kinds} errors={len(self.errors)} "
                f"max_err={ {k: float(f'{v:.3g}') for k, v in self.max_err.items()} }"
                + ("" if self.flag_ok() else " FLAGGED ABOVE 0.1%")
                + ("" if not self.errors else "\n  " + "\n  ".join(self.errors[:20])))


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _parts(n, threads):
    """Contiguous row ranges for `threads` workers (the oracle is single
    threaded C; ctypes releases the GIL, so threads run the parts at once)."""
    threads = max(1, min(int(threads), n))
    b = np.linspace(0, n, threads + 1).round().astype(int)
    return [(int(b[i]), int(b[i + 1])) for i in range(threads) if b[i + 1] > b[i]]


def _by_rows(fn, n, threads):
    """fn(lo, hi) -> tuple of arrays with rows lo..hi; the parts concatenated
    in row order (requests are independent in the draft and the verify)."""
    parts = _parts(n, threads)
    if len(parts) == 1:
        return fn(0, n)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(parts)) as ex:
        outs = list(ex.map(lambda p: fn(*p), parts))
    return tuple(np.concatenate([o[j] for o in outs]) for j in range(len(outs[0])))


def _rows(a, lo, hi):
    return None if a is None else a[lo:hi]


def check_draft(rep, U, W1, W2t, x0, T, seed, rnd, dev_x, dev_lp, dev_lse, reqs, threads=1):
    """Returns the oracle's (logp_d, lse_d) on the GPU's token chain."""
    rq = np.arange(len(x0), dtype=np.int32) if reqs is None else np.asarray(reqs, np.int32)

    def run(lo, hi):
        _, lp, lse, mg, own = O.draft_markov(U[lo:hi], W1, W2t, x0[lo:hi], T, seed, rnd,
                                             req_ids=rq[lo:hi], force_x=dev_x[lo:hi], own=True)
        return lp, lse, mg, own
    lp, lse, mg, own = _by_rows(run, len(x0), threads)
    return _compare_draft(rep, x0, T, dev_x, dev_lp, dev_lse, reqs, lp, lse, mg, own)


def check_draft_rnn(rep, U, W1, W2t, Wr, h, x0, T, seed, rnd, dev_x, dev_lp, dev_lse, dev_feat,
                    dev_state, reqs, bf16_e):
    """RNN head.  Pass 1 forces the oracle onto the GPU's tokens: its states
    must agree within TOL_REL (absolute; states lie in (-1, 1)) and its
    features bit for bit after rounding to bf16, except elements whose
    rounding margin is below MARGIN (flagged; at most 0.1% of the elements),
    or within TOL_REL for float32 features.  The features do not feed back
    into the state, so pass 2 forces the GPU's features as well and compares
    every token decision, log p_d and lse_d as for the Markov head."""
    _, _, _, _, _, e, st, em = O.draft_rnn(U, W1, W2t, Wr, h, x0, T, seed, rnd, req_ids=reqs,
                                           force_x=dev_x, bf16_e=bf16_e)
    fe = dev_feat.astype(np.float64)
    es = np.abs(dev_state.astype(np.float64) - st)
    rep.note("rnn_state", es.max())
    if es.max() > TOL_REL:
        rep.err(f"rnn state max err {es.max():.3g}")
    if bf16_e:
        diff = fe != e
        nflag = int((diff & (em < MARGIN)).sum())
        nbad = int((diff & (em >= MARGIN)).sum())
        rep.note("rnn_e_flagged", nflag)
        rep.count("rnn_e", e.size, nflag)
        if nbad:
            i = np.argwhere(diff & (em >= MARGIN))[0]
            rep.err(f"rnn features: {nbad} bf16 values differ away from a rounding tie "
                    f"(first {tuple(i)}: gpu {fe[tuple(i)]!r} oracle {e[tuple(i)]!r})")
    else:
        ee = np.abs(fe - e)
        rep.note("rnn_e", ee.max())
        if ee.max() > TOL_REL:
            rep.err(f"rnn features max err {ee.max():.3g}")
    _, lp, lse, mg, own, _, _, _ = O.draft_rnn(U, W1, W2t, Wr, h, x0, T, seed, rnd, req_ids=reqs,
                                               force_x=dev_x, force_e=fe, bf16_e=bf16_e)
    return _compare_draft(rep, x0, T, dev_x, dev_lp, dev_lse, reqs, lp, lse, mg, own)


def _compare_draft(rep, x0, T, dev_x, dev_lp, dev_lse, reqs, lp, lse, mg, own):
    diff = own[:, 1:] != dev_x[:, 1:]
    bad = diff & (mg >= MARGIN)
    rep.count("draft", diff.size, int((diff & (mg < MARGIN)).sum()))
    for r, k in zip(*np.nonzero(bad)):
        rep.err(f"draft req {reqs[r] if reqs is not None else r} pos {k + 1}: gpu {dev_x[r, k + 1]} "
                f"oracle {own[r, k + 1]} margin {mg[r, k]:.3g}")
    if (dev_x[:, 0] != np.asarray(x0)).any():
        rep.err("draft: x[:, 0] is not the anchor")
    e_lp = np.abs(dev_lp.astype(np.float64) - lp)
    e_lse = np.abs(dev_lse.astype(np.float64) - lse)
    rep.note("logp_d", e_lp.max())
    rep.note("lse_d", e_lse.max())
    if T > 0:
        # both are log-probabilities (lse_d is the log-normaliser): an absolute
        # error of 1e-5 is a relative error of 1e-5 on the probability
        if e_lp.max() > TOL_LOG:
            rep.err(f"draft logp_d max err {e_lp.max():.3g}")
        if e_lse.max() > TOL_LOG:
            rep.err(f"draft lse_d max err {e_lse.max():.3g}")
    else:
        if e_lse.max() > 1e-5 * max(1.0, np.abs(lse).max()):
            rep.err(f"greedy lse_d (max score) err {e_lse.max():.3g}")
    return lp, lse


def check_confidence(rep, h, W1, w, dev_x, dev_c, sts=None):
    c, _ = O.confidence(h, W1, w, dev_x, sts)
    rel = np.abs(dev_c.astype(np.float64) - c) / np.maximum(np.abs(c.astype(np.float64)), 1e-30)
    rep.note("c_rel", rel.max())
    if rel.max() > TOL_REL:
        rep.err(f"confidence max rel err {rel.max():.3g}")


def check_schedule(rep, dev_c, sps, enabled, dev_ell, dev_a, dev_N, dev_theta):
    ell, a, N, th, _ = O.prefix_schedule(dev_c, sps, enabled=enabled)
    if not np.array_equal(ell, dev_ell):
        bad = np.nonzero(ell != dev_ell)[0]
        rep.err(f"schedule ell differs at {bad[:10]} (gpu {dev_ell[bad[:10]]} oracle {ell[bad[:10]]})")
    if dev_a is not None and not np.array_equal(a.view(np.uint32), f32(dev_a).view(np.uint32)):
        rep.err("schedule survival products a differ")
    if dev_N is not None and int(dev_N) != N:
        rep.err(f"schedule N gpu {int(dev_N)} oracle {N}")
    if dev_theta is not None and float(dev_theta) != th:
        rep.err(f"schedule Theta gpu {float(dev_theta)!r} oracle {th!r}")
    return ell


def check_pack(rep, rows, lens, dev_cu, dev_flat, dev_mr, dev_mp, dev_N, what):
    cu, flat, mr, mp, N = O.pack(rows, lens)
    ok = np.array_equal(cu, dev_cu) and np.array_equal(flat, dev_flat) and int(dev_N) == N
    if dev_mr is not None:
        ok = ok and np.array_equal(mr, dev_mr) and np.array_equal(mp, dev_mp)
    if not ok:
        rep.err(f"pack ({what}) differs")
    return cu


def check_verify(rep, ell, cu, target, layout, x, lp_d, lse_d, U, W1, W2t, T, seed, rnd,
                 dev_m, dev_tau, dev_em, dev_na, dev_lpt, reqs, full_R=None, feat=None,
                 threads=1):
    """reqs: request ids of the rows given (None: all); cu / target in the
    layout the GPU consumed (for a subset, pass dense rows of the subset).
    lp_d, lse_d: the draft's log p_d and log-normaliser the oracle verifies
    with (the oracle's own values on the GPU's token chain, from check_draft,
    so that every accept margin is measured on oracle values).
    feat: the draft's per-position bias features (RNN head)."""
    lp_d = np.asarray(lp_d, np.float64)
    lse_d = np.asarray(lse_d, np.float64)
    if layout == 0 or threads <= 1:
        m, tau, em, na, lpt, mg = O.verify(ell, cu, target, layout, x, lp_d, lse_d, U, W1, W2t, T,
                                           seed, rnd, req_ids=reqs, feat=feat)
    else:
        rq = np.arange(ell.size, dtype=np.int32) if reqs is None else np.asarray(reqs, np.int32)
        m, tau, em, na, lpt, mg = _by_rows(
            lambda lo, hi: O.verify(ell[lo:hi], None, target[lo:hi], 1, x[lo:hi], lp_d[lo:hi],
                                    lse_d[lo:hi], U[lo:hi], W1, W2t, T, seed, rnd,
                                    req_ids=rq[lo:hi], feat=_rows(feat, lo, hi)),
            ell.size, threads)
    R = ell.size
    nflag = 0
    for r in range(R):
        same = (m[r] == dev_m[r] and tau[r] == dev_tau[r] and na[r] == dev_na[r]
                and np.array_equal(em[r], dev_em[r]))
        if not same:
            if mg[r] < MARGIN:
                nflag += 1
            else:
                rid = reqs[r] if reqs is not None else r
                rep.err(f"verify req {rid}: gpu m={dev_m[r]} y={dev_na[r]} oracle m={m[r]} "
                        f"y={na[r]} margin {mg[r]:.3g}")
    rep.count("verify", R, nflag)
    if T > 0 and dev_lpt is not None:
        mask = np.arange(x.shape[1] - 1)[None, :] < ell[:, None]
        e = np.abs(dev_lpt.astype(np.float64) - lpt)[mask]
        if e.size:
            rep.note("logp_t", e.max())
            if e.max() > TOL_LOG:
                rep.err(f"verify logp_t max err {e.max():.3g}")
    return m, tau, em, na


def check_verify_cap_accept(rep, ell, cap, cu, target, layout, x, dev_lp, dev_lse, U, W1, W2t, T,
                            seed, rnd, dev_m, dev_tau, dev_em, dev_na, dev_mfull, reqs, feat=None):
    """Cap-accept verify: the committed result and the whole-window accepted
    count, bit-exact except requests whose oracle margin is below MARGIN."""
    m, tau, em, na, lpt, mg, mfull = O.verify_cap_accept(ell, cap, cu, target, layout, x,
                                                         dev_lp.astype(np.float64),
                                                         dev_lse.astype(np.float64), U, W1, W2t,
                                                         T, seed, rnd, req_ids=reqs, feat=feat)
    R = ell.size
    nflag = 0
    for r in range(R):
        same = (m[r] == dev_m[r] and tau[r] == dev_tau[r] and na[r] == dev_na[r]
                and np.array_equal(em[r], dev_em[r])
                and (dev_mfull is None or mfull[r] == dev_mfull[r]))
        if not same:
            if mg[r] < MARGIN:
                nflag += 1
            else:
                rid = reqs[r] if reqs is not None else r
                rep.err(f"cap-accept req {rid}: gpu m={dev_m[r]} y={dev_na[r]} oracle m={m[r]} "
                        f"y={na[r]} m_full gpu {None if dev_mfull is None else dev_mfull[r]} "
                        f"oracle {mfull[r]} margin {mg[r]:.3g}")
    rep.count("verify", R, nflag)
    return m, mfull
