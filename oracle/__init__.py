"""ctypes binding of the CPU oracle (``oracle/dspark_oracle.cpp``).

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product package never imports
it.  Arrays are numpy; floating inputs are passed as float32 (bf16 values widen
to float32 exactly) and widened to double inside the oracle.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
# DSPARK_ORACLE_LIB: a prebuilt variant of the same source (the CPU sanitizer
# test runs the oracle tests against an AddressSanitizer/UBSan build)
_LIB_OVERRIDE = os.environ.get("DSPARK_ORACLE_LIB")

TAG_DRAFT_CHUNK, TAG_DRAFT_ELEM, TAG_ACCEPT = 1, 2, 3
TAG_RESID_CHUNK, TAG_RESID_ELEM, TAG_BONUS_CHUNK, TAG_BONUS_ELEM = 4, 5, 6, 7


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (plain IEEE double, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = C.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = C.CDLL(_LIB)
        P = C.c_void_p
        i32, i64, u32, u64, f64 = C.c_int, C.c_int64, C.c_uint32, C.c_uint64, C.c_double
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_stream_word.argtypes = [u64, u64, u32, u32, u32, u32]
        L.orc_stream_word.restype = u32
        L.orc_gumbel.argtypes = [u64, u64, u32, u32, u32, u32]
        L.orc_gumbel.restype = f64
        L.orc_chunk_width.restype = i64
        L.orc_cgm.argtypes = [P, i64, u64, u64, u32, u32, u32, u32, P]
        L.orc_cgm.restype = i64
        L.orc_cgm_batch.argtypes = [P, i64, u64, u64, u32, u32, u32, i64, u32, P]
        L.orc_draft_row.argtypes = [i64, i32, f64, P, P, P, C.c_int32, P]
        L.orc_residual_row.argtypes = [i64, f64, P, P, f64, P]
        L.orc_residual_row.restype = f64
        L.orc_draft_markov.argtypes = [i32, i32, i64, i32, f64, u64, u64, P, P, P, P, P, P,
                                       P, P, P, P, P]
        L.orc_draft_markov.restype = i32
        L.orc_confidence.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.orc_prefix_schedule.argtypes = [i32, i32, P, P, i32, i32, i32, P, P, P, P, P]
        L.orc_prefix_schedule.restype = i32
        L.orc_async_schedule.argtypes = [i32, i32, P, P, i32, i32, P, P, P, P, P, P]
        L.orc_async_schedule.restype = i32
        L.orc_acceptance_rate.argtypes = [i32, i32, i64, i32, f64, P, P, P, P, P, P, P, P]
        L.orc_acceptance_rate.restype = i32
        L.orc_sts_fit.argtypes = [i32, i32, P, P, P, i32, i32, P, P, P, P]
        L.orc_sts_fit.restype = i32
        L.orc_pack.argtypes = [i32, i32, P, P, P, P, P, P, P]
        L.orc_verify.argtypes = [i32, i32, i64, i32, f64, u64, u64, P, P, P, i32, P, P, P,
                                 P, P, P, P, P, P, P, P, P, P, P, P]
        L.orc_draft_rnn.argtypes = [i32, i32, i64, i32, i32, f64, u64, u64, P, P, P, P, P, P, P,
                                    P, P, i32, P, P, P, P, P, P, P, P]
        L.orc_draft_rnn.restype = i32
        L.orc_verify.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _T(T):
    """The sampling temperature as the GPU library receives it: the C ABI takes
    a float32, so the oracle computes with that value widened to double."""
    return float(np.float32(T))


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


# ------------------------------------------------------------ random stream
def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def stream_word(seed, rnd, tag, req, k, idx):
    return int(lib().orc_stream_word(seed, rnd, tag, req, k, idx))


def gumbel(seed, rnd, tag, req, k, idx):
    return float(lib().orc_gumbel(seed, rnd, tag, req, k, idx))


def chunk_width():
    return int(lib().orc_chunk_width())


def cgm(score, seed, rnd, tag_chunk, tag_elem, req, k):
    s = _f64(score)
    mg = np.zeros(1)
    j = lib().orc_cgm(_p(s), s.size, seed, rnd, tag_chunk, tag_elem, req, k, _p(mg))
    return int(j), float(mg[0])


def cgm_batch(score, seed, rnd, tag_chunk, tag_elem, req0, count, k):
    s = _f64(score)
    out = np.zeros(count, np.int64)
    lib().orc_cgm_batch(_p(s), s.size, seed, rnd, tag_chunk, tag_elem, req0, count, k, _p(out))
    return out


# ------------------------------------------------------------ distributions
def draft_row(Uk, W1, W2t, prev, T):
    Uk = _f32(Uk)
    rank = 0 if W1 is None else W1.shape[1]
    p = np.zeros(Uk.size)
    lib().orc_draft_row(Uk.size, rank, _T(T), _p(Uk), _p(_f32(W1)), _p(_f32(W2t)),
                        int(prev), _p(p))
    return p


def residual_row(t, s, lse_d, T):
    t = _f32(t)
    s = _f64(s)
    q = np.zeros(t.size)
    tot = lib().orc_residual_row(t.size, _T(T), _p(t), _p(s), float(lse_d), _p(q))
    return q, float(tot)


# -------------------------------------------------------------- the stages
def draft_rnn(U, W1, W2t, Wr, h, x0, T, seed=0, rnd=0, req_ids=None, force_x=None,
              force_e=None, bf16_e=True):
    """RNN draft head.  U [R][gamma][V]; W1, W2t [V][r]; Wr [3r][2r+d]; h
    [R][gamma][d]; x0 [R].  Returns (x, logp_d, lse_d, margin, x_own, e, s,
    e_margin)."""
    U = _f32(U)
    R, gamma, V = U.shape
    rank = int(W1.shape[1])
    h = _f32(h)
    d = h.shape[-1]
    x = np.zeros((R, gamma + 1), np.int32)
    lp, lse, mg = np.zeros((R, gamma)), np.zeros((R, gamma)), np.zeros((R, gamma))
    xo = np.zeros((R, gamma + 1), np.int32)
    e = np.zeros((R, gamma, rank))
    s = np.zeros((R, gamma, rank))
    em = np.zeros((R, gamma, rank))
    rc = lib().orc_draft_rnn(R, gamma, V, rank, d, _T(T), seed, rnd, _p(U), _p(_f32(W1)),
                             _p(_f32(W2t)), _p(_f32(Wr)), _p(h), _p(_i32(x0)), _p(_i32(req_ids)),
                             _p(_i32(force_x)), _p(_f32(force_e)), int(bool(bf16_e)), _p(x),
                             _p(lp), _p(lse), _p(mg), _p(xo), _p(e), _p(s), _p(em))
    assert rc == 0, rc
    return x, lp, lse, mg, xo, e, s, em


def draft_markov(U, W1, W2t, x0, T, seed=0, rnd=0, req_ids=None, force_x=None, own=False):
    """U [R][gamma][V]; W1, W2t [V][rank] or None; x0 [R].  With own=True also
    returns the oracle's own choice at every position given the forced prefix."""
    U = _f32(U)
    R, gamma, V = U.shape
    rank = 0 if W1 is None else int(W1.shape[1])
    W1c, W2c = _f32(W1), _f32(W2t)
    x0 = _i32(x0)
    x = np.zeros((R, gamma + 1), np.int32)
    lp = np.zeros((R, gamma))
    lse = np.zeros((R, gamma))
    mg = np.zeros((R, gamma))
    xo = np.zeros((R, gamma + 1), np.int32) if own else None
    rc = lib().orc_draft_markov(R, gamma, V, rank, _T(T), seed, rnd, _p(U), _p(W1c),
                                _p(W2c), _p(x0), _p(_i32(req_ids)), _p(_i32(force_x)),
                                _p(x), _p(lp), _p(lse), _p(mg), _p(xo))
    assert rc == 0, rc
    if own:
        return x, lp, lse, mg, xo
    return x, lp, lse, mg


def confidence(h, W1, w, x, sts_T=None):
    h = _f32(h)
    R, gamma, d = h.shape
    rank = 0 if W1 is None else int(W1.shape[1])
    c = np.zeros((R, gamma), np.float32)
    z = np.zeros((R, gamma))
    lib().orc_confidence(R, gamma, d, rank, _p(h), _p(_f32(W1)), _p(_f32(w)),
                         _p(_f32(sts_T)), _p(_i32(x)), _p(c), _p(z))
    return c, z


def prefix_schedule(c, sps, N_max=None, enabled=True, mode=0):
    c = _f32(c)
    R, gamma = c.shape
    sps = _f64(sps)
    if N_max is None:
        N_max = sps.size - 1
    ell = np.zeros(R, np.int32)
    a = np.zeros((R, gamma), np.float32)
    N = np.zeros(1, np.int32)
    th = np.zeros(1)
    mg = np.zeros(1)
    rc = lib().orc_prefix_schedule(R, gamma, _p(c), _p(sps), int(N_max), int(bool(enabled)),
                                   int(mode), _p(ell), _p(a), _p(N), _p(th), _p(mg))
    assert rc == 0, rc
    return ell, a, int(N[0]), float(th[0]), float(mg[0])


def async_schedule(c, sps, K_in, N_max=None):
    """Production asynchronous scheduler: admit the K_in - R best candidates of
    this round, plan the capacity of the round two rounds later.
    Returns (ell, a, N, theta_admitted, K_plan, theta_plan)."""
    c = _f32(c)
    R, gamma = c.shape
    sps = _f64(sps)
    if N_max is None:
        N_max = sps.size - 1
    ell = np.zeros(R, np.int32)
    a = np.zeros((R, gamma), np.float32)
    N = np.zeros(1, np.int32)
    th = np.zeros(1)
    K = np.zeros(1, np.int32)
    thp = np.zeros(1)
    rc = lib().orc_async_schedule(R, gamma, _p(c), _p(sps), int(N_max), int(K_in), _p(ell), _p(a),
                                  _p(N), _p(th), _p(K), _p(thp))
    assert rc == 0, rc
    return ell, a, int(N[0]), float(th[0]), int(K[0]), float(thp[0])


def pack(rows, lens):
    rows = _i32(rows)
    R, width = rows.shape
    lens = _i32(lens)
    cu = np.zeros(R + 1, np.int32)
    flat = np.zeros(R * width, np.int32)
    mr = np.zeros(R * width, np.int32)
    mp = np.zeros(R * width, np.int32)
    N = np.zeros(1, np.int32)
    lib().orc_pack(R, width, _p(rows), _p(lens), _p(cu), _p(flat), _p(mr), _p(mp), _p(N))
    return cu, flat, mr, mp, int(N[0])


def acceptance_rate(target, x, U, W1, W2t, T, feat=None):
    """c*_k = sum_v min(p_d^k, p_t^k) for every request and position (dense
    target [R][gamma+1][V]); feat [R][gamma][rank]: the RNN head's bias
    features in place of W1[x_{k-1}].  Returns (c_star [R][gamma], margin)."""
    target = _f32(target)
    R, g1, V = target.shape
    gamma = g1 - 1
    rank = 0 if W1 is None else int(W1.shape[1])
    if feat is not None:
        rank = int(np.shape(feat)[-1])
    cs = np.zeros((R, gamma))
    mg = np.zeros((R, gamma))
    rc = lib().orc_acceptance_rate(R, gamma, V, rank, _T(T), _p(target), _p(_i32(x)),
                                   _p(_f32(U)), _p(_f32(W1)), _p(_f32(W2t)), _p(cs), _p(mg),
                                   _p(_f32(feat)))
    assert rc == 0, rc
    return cs, mg


def sts_fit(z, m, grid, nbins=15, force_t=None):
    """Sequential temperature scaling on held-out logits z [n][gamma] and
    accepted counts m [n].  Returns (t [gamma] float32, ece [gamma], margin)."""
    z = _f32(z)
    n, gamma = z.shape
    grid = _f32(grid)
    t = np.zeros(gamma, np.float32)
    ece = np.zeros(gamma)
    mg = np.zeros(gamma)
    rc = lib().orc_sts_fit(n, gamma, _p(z), _p(_i32(m)), _p(grid), grid.size, int(nbins),
                           _p(None if force_t is None else _f32(force_t)), _p(t), _p(ece), _p(mg))
    assert rc == 0, rc
    return t, ece, mg


def pack_tiered(rows, lens, tiers, pad_token, slots=None):
    """Ragged pack padded to a captured graph tier (bevisy.github.io DeepSpec
    analysis, section 5.4, DSpark in SGLang: ragged verify packs the requests
    into one compact buffer whose total is rounded up to a captured CUDA-graph
    tier).  The pack itself is `pack`; N_pad = the smallest tier >= N (N itself,
    flagged, when no tier holds N); slots [N, N_pad) hold pad_token with
    markers -1, slots from N_pad to `slots` hold -1.
    Returns (cu, flat, marker_req, marker_pos, N, N_pad, overflow)."""
    rows = _i32(rows)
    R, width = rows.shape
    slots = R * width if slots is None else int(slots)
    assert all(0 < int(t) <= slots for t in tiers) and slots >= R * width
    cu, flat, mr, mp, N = pack(rows, lens)
    fits = [int(t) for t in tiers if int(t) >= N]
    N_pad = min(fits) if fits else N
    out = np.full(slots, -1, np.int32)
    omr, omp = np.full(slots, -1, np.int32), np.full(slots, -1, np.int32)
    out[:N], omr[:N], omp[:N] = flat[:N], mr[:N], mp[:N]
    out[N:N_pad] = pad_token
    return cu, out, omr, omp, N, N_pad, not fits


def verify_cap_accept(ell, cap, cu, target, layout, x, logp_d, lse_d, U, W1, W2t, T, seed=0,
                      rnd=0, req_ids=None, feat=None):
    """Cap-accept verification (bevisy.github.io DeepSpec analysis, section
    5.4, DSpark in SGLang, the verify modes: verify the whole window, commit
    only the scheduler's truncated window).  Request i is verified over its window ell[i] exactly
    as in `verify`; of the token sequence that produces (m accepted drafts,
    then the correction or bonus), the first min(m, c) + 1 tokens are
    committed, c = cap[i] clamped to [0, ell[i]].  When m > c the committed
    token at position c + 1 is the accepted draft x_{c+1} itself.  feat: the
    RNN head's per-position bias features, as for `verify`.
    Returns (m, tau, emitted, next_anchor, logp_t, margin, m_full)."""
    m_full, _, em_full, _, lpt, mg = verify(ell, cu, target, layout, x, logp_d, lse_d, U, W1, W2t,
                                            T, seed, rnd, req_ids=req_ids, feat=feat)
    ell = _i32(ell)
    c = np.clip(_i32(cap), 0, ell)
    m = np.minimum(m_full, c).astype(np.int32)
    tau = m + 1
    em = np.full_like(em_full, -1)
    for i in range(ell.size):
        em[i, :tau[i]] = em_full[i, :tau[i]]
    na = em[np.arange(ell.size), tau - 1].astype(np.int32)
    return m, tau.astype(np.int32), em, na, lpt, mg, m_full


def verify(ell, cu, target, layout, x, logp_d, lse_d, U, W1, W2t, T, seed=0, rnd=0,
           req_ids=None, force_m=None, feat=None):
    ell = _i32(ell)
    R = ell.size
    x = _i32(x)
    gamma = x.shape[1] - 1
    target = _f32(target)
    V = target.shape[-1]
    rank = 0 if W1 is None else int(W1.shape[1])
    m = np.zeros(R, np.int32)
    tau = np.zeros(R, np.int32)
    em = np.zeros((R, gamma + 1), np.int32)
    na = np.zeros(R, np.int32)
    lpt = np.zeros((R, gamma))
    mg = np.zeros(R)
    rc = lib().orc_verify(R, gamma, V, rank, _T(T), seed, rnd, _p(ell), _p(_i32(cu)),
                          _p(target), int(layout), _p(x), _p(_f64(logp_d)), _p(_f64(lse_d)),
                          _p(_f32(U)), _p(_f32(W1)), _p(_f32(W2t)), _p(_i32(req_ids)),
                          _p(_i32(force_m)), _p(m), _p(tau), _p(em), _p(na), _p(lpt), _p(mg),
                          _p(_f32(feat)))
    assert rc == 0, rc
    return m, tau, em, na, lpt, mg
