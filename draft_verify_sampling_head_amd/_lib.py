"""ctypes binding of libdspark.so: argument marshalling only.

Each function takes torch tensors that already live on the GPU, passes their
device pointers, sizes and dtype codes to the C entry point of the same name
and raises on a non-OK status.  Every step of the round runs in the library's
HIP kernels; nothing here computes.  There is no fallback: if the library is
missing or fails to load, the import raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# DSPARK_LIB_PATH: another build of this library (the CPU sanitizer tests load
# a build with host-side AddressSanitizer/UBSan instrumentation)
LIB_PATH = os.environ.get("DSPARK_LIB_PATH") or os.path.join(_PKG, "libdspark.so")

F32, BF16 = 0, 1
STATUS = {0: "DSPARK_OK", 1: "DSPARK_E_INVALID", 2: "DSPARK_E_UNSUPPORTED",
          3: "DSPARK_E_WORKSPACE", 4: "DSPARK_E_HIP"}
FLAG_NONFINITE, FLAG_BAD_LEN, FLAG_BAD_TOKEN, FLAG_BARRIER, FLAG_TIER = 1, 2, 4, 8, 16
CHUNK = 128
EXPORTS = ("dspark_workspace_bytes", "dspark_status_string", "dspark_version",
           "dspark_clear_status", "dspark_get_status", "dspark_draft_markov",
           "dspark_confidence", "dspark_prefix_schedule", "dspark_pack", "dspark_verify",
           "dspark_draft_markov_profiled", "dspark_async_schedule", "dspark_pack_tiered",
           "dspark_verify_cap_accept", "dspark_acceptance_rate", "dspark_sts_fit",
           "dspark_sts_workspace_bytes", "dspark_confidence_logits", "dspark_rnn_workspace_bytes",
           "dspark_draft_rnn", "dspark_verify_features", "dspark_draft_rnn_profiled",
           "dspark_acceptance_rate_features", "dspark_verify_cap_accept_features",
           "dspark_set_switch", "dspark_get_switch", "dspark_draft_markov_noalloc",
           "dspark_w2_transpose", "dspark_schedule_pack", "dspark_round_markov")
SWITCH_FORCE_PER_STEP, SWITCH_RNN_CELL_VALU, SWITCH_BARRIER_SPINS, SWITCH_DRAFT_KERNEL = 1, 2, 3, 4
SWITCH_PERSIST_LAUNCH = 5


class RoundMarkovArgs(C.Structure):
    """dspark_round_markov_args, field for field."""
    _fields_ = ([(n, C.c_int) for n in ("R", "gamma", "V", "r", "d")] + [("T", C.c_float)]
                + [("seed", C.c_uint64), ("round", C.c_uint64)]
                + [(n, C.c_int) for n in ("sched_mode", "N_max", "target_layout", "U_dt", "W_dt",
                                          "h_dt", "w_dt", "t_dt")]
                + [(n, C.c_void_p) for n in (
                    "U", "W1", "W2t", "x0", "h", "w", "sts_T", "sps", "target", "K_in", "K_plan",
                    "x", "logp_d", "lse_d", "c", "ell", "a", "N", "theta", "theta_plan", "cu",
                    "flat", "marker_req", "marker_pos", "m", "tau", "emitted", "next_anchor",
                    "logp_t", "cu_out", "flat_out", "N_out")])


class DsparkError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}")
        self.code = code


_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or `python draft_verify_sampling_head_amd/build.py`")
    L = C.CDLL(LIB_PATH)
    P, i32, u64, f32, sz = C.c_void_p, C.c_int, C.c_uint64, C.c_float, C.c_size_t
    L.dspark_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.dspark_workspace_bytes.restype = sz
    L.dspark_status_string.argtypes = [i32]
    L.dspark_status_string.restype = C.c_char_p
    L.dspark_version.restype = C.c_char_p
    L.dspark_clear_status.argtypes = [P, sz, P]
    L.dspark_get_status.argtypes = [P, sz, P]
    L.dspark_draft_markov.argtypes = [i32, i32, i32, i32, f32, u64, u64, P, i32, P, P, i32, P, P,
                                      P, P, P, P, sz, P]
    L.dspark_draft_markov_profiled.argtypes = L.dspark_draft_markov.argtypes + [P, P, P]
    L.dspark_confidence.argtypes = [i32, i32, i32, i32, i32, P, i32, P, i32, P, i32, P, P, P, P]
    L.dspark_prefix_schedule.argtypes = [i32, i32, P, P, i32, i32, P, P, P, P, P]
    L.dspark_async_schedule.argtypes = [i32, i32, P, P, i32, P, P, P, P, P, P, P, P]
    L.dspark_pack.argtypes = [i32, i32, P, P, i32, P, P, P, P, P, P, sz, P]
    L.dspark_schedule_pack.argtypes = [i32, i32, i32, P, P, i32, P, P, P, P, P, P, P, P, P, P, P,
                                       P, P]
    L.dspark_sts_workspace_bytes.argtypes = [i32]
    L.dspark_sts_workspace_bytes.restype = sz
    L.dspark_sts_fit.argtypes = [i32, i32, P, P, P, i32, i32, P, P, P, sz, P]
    L.dspark_confidence_logits.argtypes = [i32, i32, i32, i32, i32, P, i32, P, i32, P, i32, P, P, P]
    L.dspark_acceptance_rate.argtypes = [i32, i32, i32, i32, f32, P, i32, P, P, P, i32, P, P, i32,
                                         P, P, sz, P]
    L.dspark_pack_tiered.argtypes = [i32, i32, P, P, i32, P, i32, i32, C.c_int64, P, P, P, P, P,
                                     P, P, sz, P]
    L.dspark_verify_cap_accept.argtypes = [i32, i32, i32, i32, f32, u64, u64, P, P, P, P, i32, i32,
                                           P, P, P, P, i32, P, P, i32, P, P, P, P, P, P, P, sz, P]
    L.dspark_verify.argtypes = [i32, i32, i32, i32, f32, u64, u64, P, P, P, i32, i32, P, P, P, P,
                                i32, P, P, i32, P, P, P, P, P, P, sz, P]
    L.dspark_rnn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.dspark_rnn_workspace_bytes.restype = sz
    L.dspark_draft_rnn.argtypes = [i32, i32, i32, i32, i32, f32, u64, u64, P, i32, P, P, i32, P, P,
                                   i32, P, P, P, P, P, P, P, P, sz, P]
    L.dspark_draft_rnn_profiled.argtypes = L.dspark_draft_rnn.argtypes + [P, P, P]
    L.dspark_verify_features.argtypes = L.dspark_verify.argtypes
    L.dspark_acceptance_rate_features.argtypes = L.dspark_acceptance_rate.argtypes
    L.dspark_verify_cap_accept_features.argtypes = L.dspark_verify_cap_accept.argtypes
    L.dspark_w2_transpose.argtypes = [i32, i32, P, P, i32, P]
    L.dspark_draft_markov_noalloc.argtypes = [i32, i32, i32, i32, f32, u64, u64, P, i32, P, P, i32,
                                              P, P, P, P, P, P, P]
    L.dspark_round_markov.argtypes = [C.POINTER(RoundMarkovArgs), P, sz, P]
    L.dspark_set_switch.argtypes = [i32, C.c_int64]
    L.dspark_get_switch.argtypes = [i32]
    L.dspark_get_switch.restype = C.c_int64
    for fn in EXPORTS:
        getattr(L, fn).restype = getattr(L, fn).restype or i32
    L.dspark_workspace_bytes.restype = sz
    L.dspark_sts_workspace_bytes.restype = sz
    L.dspark_rnn_workspace_bytes.restype = sz
    L.dspark_status_string.restype = C.c_char_p
    L.dspark_version.restype = C.c_char_p
    _lib = L
    return L


def set_switch(key, value):
    """Set a test / measurement switch (SWITCH_*); returns the previous value."""
    prev = int(load().dspark_get_switch(key))
    _check("dspark_set_switch", load().dspark_set_switch(key, int(value)))
    return prev


def get_switch(key):
    return int(load().dspark_get_switch(key))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dt(t):
    if t is None:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(fn, code):
    if code != 0:
        raise DsparkError(fn, code)


def workspace_bytes(R, gamma, V, r=0, d=0):
    return int(load().dspark_workspace_bytes(R, gamma, V, r, d))


def workspace(R, gamma, V, device="cuda"):
    """Allocate a zeroed workspace tensor (uint8) of the size the library asks
    for (the status word in its header must start at zero)."""
    return torch.zeros(max(256, workspace_bytes(R, gamma, V)), dtype=torch.uint8, device=device)


def version():
    return load().dspark_version().decode()


def clear_status(ws, stream=None):
    _check("dspark_clear_status", load().dspark_clear_status(_ptr(ws), ws.numel(), _stream(stream)))


def get_status(ws):
    out = C.c_uint32(0)
    _check("dspark_get_status", load().dspark_get_status(_ptr(ws), ws.numel(), C.byref(out)))
    return int(out.value)


def draft_markov(U, W1, W2t, x0, T, seed, rnd, x, logp_d, lse_d, ws, margin=None, stream=None):
    R, gamma, V = U.shape
    r = 0 if W1 is None else int(W1.shape[1])
    code = load().dspark_draft_markov(R, gamma, V, r, float(T), seed, rnd, _ptr(U), _dt(U),
                                      _ptr(W1), _ptr(W2t), _dt(W1), _ptr(x0), _ptr(x),
                                      _ptr(logp_d), _ptr(lse_d), _ptr(margin), _ptr(ws),
                                      ws.numel(), _stream(stream))
    _check("dspark_draft_markov", code)


def draft_markov_noalloc(U, W1, W2t, x0, T, seed, rnd, x, logp_d, lse_d, flags=None, margin=None,
                         stream=None):
    """dspark_draft_markov without a workspace: the library's static device
    scratch holds the draft's intermediate state (calls on one GPU must not
    overlap).  flags: nullable device uint32 tensor receiving the status word."""
    R, gamma, V = U.shape
    r = 0 if W1 is None else int(W1.shape[1])
    code = load().dspark_draft_markov_noalloc(R, gamma, V, r, float(T), seed, rnd, _ptr(U), _dt(U),
                                              _ptr(W1), _ptr(W2t), _dt(W1), _ptr(x0), _ptr(x),
                                              _ptr(logp_d), _ptr(lse_d), _ptr(margin), _ptr(flags),
                                              _stream(stream))
    _check("dspark_draft_markov_noalloc", code)


def w2_transpose(W2, W2t, stream=None):
    """dspark_w2_transpose: W2 [r][V] (the method's layout) into W2t [V][r]."""
    r, V = W2.shape
    code = load().dspark_w2_transpose(r, V, _ptr(W2), _ptr(W2t), _dt(W2), _stream(stream))
    _check("dspark_w2_transpose", code)


def draft_markov_profiled(U, W1, W2t, x0, T, seed, rnd, x, logp_d, lse_d, ws, ev_begin, ev_end,
                          margin=None, stream=None):
    """As draft_markov, recording the caller's HIP events (ctypes arrays of
    gamma hipEvent_t each) around the draft's dominant kernel; returns the
    number of event pairs recorded (1: one persistent launch for all steps,
    gamma: one statistics launch per step)."""
    R, gamma, V = U.shape
    r = 0 if W1 is None else int(W1.shape[1])
    n_timed = C.c_int(0)
    code = load().dspark_draft_markov_profiled(R, gamma, V, r, float(T), seed, rnd, _ptr(U), _dt(U),
                                               _ptr(W1), _ptr(W2t), _dt(W1), _ptr(x0), _ptr(x),
                                               _ptr(logp_d), _ptr(lse_d), _ptr(margin), _ptr(ws),
                                               ws.numel(), _stream(stream), ev_begin, ev_end,
                                               C.byref(n_timed))
    _check("dspark_draft_markov_profiled", code)
    return int(n_timed.value)


def confidence(h, W1, w, x, c, sts_T=None, V=None, stream=None):
    R, gamma, d = h.shape
    r = 0 if W1 is None else int(W1.shape[1])
    V = int(W1.shape[0]) if (V is None and W1 is not None) else (V or 0)
    code = load().dspark_confidence(R, gamma, d, r, V, _ptr(h), _dt(h), _ptr(W1), _dt(W1), _ptr(w),
                                    _dt(w), _ptr(sts_T), _ptr(x), _ptr(c), _stream(stream))
    _check("dspark_confidence", code)


def prefix_schedule(c, sps, ell, enabled=True, N_max=None, a=None, N_out=None, theta_best=None,
                    stream=None):
    R, gamma = c.shape
    N_max = sps.numel() - 1 if N_max is None else N_max
    code = load().dspark_prefix_schedule(R, gamma, _ptr(c), _ptr(sps), int(N_max), int(bool(enabled)),
                                         _ptr(ell), _ptr(a), _ptr(N_out), _ptr(theta_best),
                                         _stream(stream))
    _check("dspark_prefix_schedule", code)


def async_schedule(c, sps, K_in, K_plan, ell, N_max=None, a=None, N_out=None, theta=None,
                   theta_plan=None, stream=None):
    R, gamma = c.shape
    N_max = sps.numel() - 1 if N_max is None else N_max
    code = load().dspark_async_schedule(R, gamma, _ptr(c), _ptr(sps), int(N_max), _ptr(K_in),
                                        _ptr(K_plan), _ptr(ell), _ptr(a), _ptr(N_out), _ptr(theta),
                                        _ptr(theta_plan), _stream(stream))
    _check("dspark_async_schedule", code)


def schedule_pack(c, sps, x, ell, cu, flat, mode=1, marker_req=None, marker_pos=None, K_in=None,
                  K_plan=None, N_max=None, a=None, N_out=None, theta=None, theta_plan=None,
                  stream=None):
    """mode 0 static, 1 greedy, 2 asynchronous; outputs as prefix_schedule /
    async_schedule followed by pack(x, ell, 1, ...)."""
    R, gamma = c.shape
    N_max = sps.numel() - 1 if N_max is None else N_max
    code = load().dspark_schedule_pack(R, gamma, int(mode), _ptr(c), _ptr(sps), int(N_max),
                                       _ptr(K_in), _ptr(K_plan), _ptr(x), _ptr(ell), _ptr(a),
                                       _ptr(N_out), _ptr(theta), _ptr(theta_plan), _ptr(cu),
                                       _ptr(flat), _ptr(marker_req), _ptr(marker_pos),
                                       _stream(stream))
    _check("dspark_schedule_pack", code)


def pack(rows, lens, len_offset, cu, flat, marker_req=None, marker_pos=None, N_out=None, ws=None,
         stream=None):
    R, width = rows.shape
    code = load().dspark_pack(R, width, _ptr(rows), _ptr(lens), int(len_offset), _ptr(cu), _ptr(flat),
                              _ptr(marker_req), _ptr(marker_pos), _ptr(N_out), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream))
    _check("dspark_pack", code)


def pack_tiered(rows, lens, len_offset, tiers, pad_token, cu, flat, marker_req=None,
                marker_pos=None, N_out=None, N_pad=None, ws=None, stream=None):
    """`tiers` is a host sequence of ints; `flat` (and the markers) may be longer
    than rows.numel(): their length is the slot count."""
    R, width = rows.shape
    t = (C.c_int32 * max(1, len(tiers)))(*[int(v) for v in tiers])
    code = load().dspark_pack_tiered(R, width, _ptr(rows), _ptr(lens), int(len_offset),
                                     C.cast(t, C.c_void_p), len(tiers), int(pad_token),
                                     int(flat.numel()), _ptr(cu), _ptr(flat), _ptr(marker_req),
                                     _ptr(marker_pos), _ptr(N_out), _ptr(N_pad), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(stream))
    _check("dspark_pack_tiered", code)


def verify_cap_accept(ell, cap, cu, target, layout, x, logp_d, lse_d, U, W1, W2t, T, seed, rnd, m,
                      tau, emitted, next_anchor, ws, m_full=None, logp_t=None, stream=None):
    R = ell.shape[0]
    gamma = x.shape[1] - 1
    V = target.shape[-1]
    r = 0 if W1 is None else int(W1.shape[1])
    code = load().dspark_verify_cap_accept(R, gamma, V, r, float(T), seed, rnd, _ptr(ell),
                                           _ptr(cap), _ptr(cu), _ptr(target), _dt(target),
                                           int(layout), _ptr(x), _ptr(logp_d), _ptr(lse_d), _ptr(U),
                                           _dt(U), _ptr(W1), _ptr(W2t), _dt(W1), _ptr(m), _ptr(tau),
                                           _ptr(emitted), _ptr(next_anchor), _ptr(m_full),
                                           _ptr(logp_t), _ptr(ws), ws.numel(), _stream(stream))
    _check("dspark_verify_cap_accept", code)


def confidence_logits(h, W1, w, x, z, V=None, stream=None):
    R, gamma, d = h.shape
    r = 0 if W1 is None else int(W1.shape[1])
    V = int(W1.shape[0]) if (V is None and W1 is not None) else (V or 0)
    code = load().dspark_confidence_logits(R, gamma, d, r, V, _ptr(h), _dt(h), _ptr(W1), _dt(W1),
                                           _ptr(w), _dt(w), _ptr(x), _ptr(z), _stream(stream))
    _check("dspark_confidence_logits", code)


def sts_workspace(n, device="cuda"):
    return torch.zeros(int(load().dspark_sts_workspace_bytes(int(n))), dtype=torch.uint8,
                       device=device)


def sts_fit(z, m, grid, t_out, ws, nbins=15, ece_out=None, stream=None):
    """z [n][gamma] float32 logits, m [n] int32 accepted counts (device);
    grid: host sequence of candidate temperatures."""
    n, gamma = z.shape
    g = (C.c_float * max(1, len(grid)))(*[float(v) for v in grid])
    code = load().dspark_sts_fit(n, gamma, _ptr(z), _ptr(m), C.cast(g, C.c_void_p), len(grid),
                                 int(nbins), _ptr(t_out), _ptr(ece_out), _ptr(ws), ws.numel(),
                                 _stream(stream))
    _check("dspark_sts_fit", code)


def acceptance_rate(target, x, lse_d, U, W1, W2t, T, c_star, ws, stream=None):
    """target dense [R][gamma+1][V]; c_star out [R][gamma]."""
    R, g1, V = target.shape
    r = 0 if W1 is None else int(W1.shape[1])
    code = load().dspark_acceptance_rate(R, g1 - 1, V, r, float(T), _ptr(target), _dt(target),
                                         _ptr(x), _ptr(lse_d), _ptr(U), _dt(U), _ptr(W1),
                                         _ptr(W2t), _dt(W1), _ptr(c_star), _ptr(ws), ws.numel(),
                                         _stream(stream))
    _check("dspark_acceptance_rate", code)


def verify(ell, cu, target, layout, x, logp_d, lse_d, U, W1, W2t, T, seed, rnd, m, tau, emitted,
           next_anchor, ws, logp_t=None, stream=None):
    R = ell.shape[0]
    gamma = x.shape[1] - 1
    V = target.shape[-1]
    r = 0 if W1 is None else int(W1.shape[1])
    code = load().dspark_verify(R, gamma, V, r, float(T), seed, rnd, _ptr(ell), _ptr(cu),
                                _ptr(target), _dt(target), int(layout), _ptr(x), _ptr(logp_d),
                                _ptr(lse_d), _ptr(U), _dt(U), _ptr(W1), _ptr(W2t), _dt(W1),
                                _ptr(m), _ptr(tau), _ptr(emitted), _ptr(next_anchor),
                                _ptr(logp_t), _ptr(ws), ws.numel(), _stream(stream))
    _check("dspark_verify", code)


def round_markov(U, W1, W2t, x0, h, w, sps, target, layout, T, seed, rnd, x, logp_d, lse_d, c,
                 ell, cu, flat, m, tau, emitted, next_anchor, cu_out, flat_out, ws, mode=1,
                 sts_T=None, K_in=None, K_plan=None, N_max=None, a=None, N=None, theta=None,
                 theta_plan=None, marker_req=None, marker_pos=None, logp_t=None, N_out=None,
                 stream=None):
    """dspark_round_markov: draft, confidence, schedule + verify-batch pack
    (mode 0 static, 1 Algorithm 1, 2 asynchronous), verify and the output pack
    in one call."""
    R, gamma, V = U.shape
    r = 0 if W1 is None else int(W1.shape[1])
    d = int(h.shape[2])
    A = RoundMarkovArgs()
    A.R, A.gamma, A.V, A.r, A.d, A.T = R, gamma, V, r, d, float(T)
    A.seed, A.round = int(seed), int(rnd)
    A.sched_mode = int(mode)
    A.N_max = sps.numel() - 1 if N_max is None else int(N_max)
    A.target_layout = int(layout)
    A.U_dt, A.W_dt, A.h_dt, A.w_dt, A.t_dt = _dt(U), _dt(W1), _dt(h), _dt(w), _dt(target)
    for name, t in (("U", U), ("W1", W1), ("W2t", W2t), ("x0", x0), ("h", h), ("w", w),
                    ("sts_T", sts_T), ("sps", sps), ("target", target), ("K_in", K_in),
                    ("K_plan", K_plan), ("x", x), ("logp_d", logp_d), ("lse_d", lse_d), ("c", c),
                    ("ell", ell), ("a", a), ("N", N), ("theta", theta), ("theta_plan", theta_plan),
                    ("cu", cu), ("flat", flat), ("marker_req", marker_req),
                    ("marker_pos", marker_pos), ("m", m), ("tau", tau), ("emitted", emitted),
                    ("next_anchor", next_anchor), ("logp_t", logp_t), ("cu_out", cu_out),
                    ("flat_out", flat_out), ("N_out", N_out)):
        setattr(A, name, None if t is None else t.data_ptr())
    code = load().dspark_round_markov(C.byref(A), _ptr(ws), ws.numel(), _stream(stream))
    _check("dspark_round_markov", code)


def rnn_workspace_bytes(R, gamma, V, r, d):
    return int(load().dspark_rnn_workspace_bytes(R, gamma, V, r, d))


def rnn_workspace(R, gamma, V, r, d, device="cuda"):
    """Zeroed workspace for dspark_draft_rnn (its head is the shared layout,
    so the same buffer serves the rest of the round)."""
    return torch.zeros(max(256, rnn_workspace_bytes(R, gamma, V, r, d)), dtype=torch.uint8,
                       device=device)


def draft_rnn(U, W1, W2t, Wr, h, x0, T, seed, rnd, x, logp_d, lse_d, feat, ws, state=None,
              margin=None, stream=None):
    """U [R][gamma][V]; W1, W2t [V][r]; Wr [3r][2r+d]; h [R][gamma][d]; feat out
    [R][gamma][r] in the weights' dtype; state out (nullable) [R][gamma][r] fp32."""
    R, gamma, V = U.shape
    r = int(W1.shape[1])
    d = int(h.shape[-1])
    code = load().dspark_draft_rnn(R, gamma, V, r, d, float(T), seed, rnd, _ptr(U), _dt(U),
                                   _ptr(W1), _ptr(W2t), _dt(W1), _ptr(Wr), _ptr(h), _dt(h),
                                   _ptr(x0), _ptr(x), _ptr(logp_d), _ptr(lse_d), _ptr(margin),
                                   _ptr(feat), _ptr(state), _ptr(ws), ws.numel(), _stream(stream))
    _check("dspark_draft_rnn", code)


def draft_rnn_profiled(U, W1, W2t, Wr, h, x0, T, seed, rnd, x, logp_d, lse_d, feat, ws, ev_begin,
                       ev_end, state=None, margin=None, stream=None):
    """As draft_rnn, recording the caller's HIP events (ctypes arrays of gamma
    hipEvent_t each) around each step's statistics kernel; returns gamma."""
    R, gamma, V = U.shape
    r = int(W1.shape[1])
    d = int(h.shape[-1])
    n_timed = C.c_int(0)
    code = load().dspark_draft_rnn_profiled(R, gamma, V, r, d, float(T), seed, rnd, _ptr(U),
                                            _dt(U), _ptr(W1), _ptr(W2t), _dt(W1), _ptr(Wr),
                                            _ptr(h), _dt(h), _ptr(x0), _ptr(x), _ptr(logp_d),
                                            _ptr(lse_d), _ptr(margin), _ptr(feat), _ptr(state),
                                            _ptr(ws), ws.numel(), _stream(stream), ev_begin,
                                            ev_end, C.byref(n_timed))
    _check("dspark_draft_rnn_profiled", code)
    return int(n_timed.value)


def acceptance_rate_features(target, x, lse_d, U, feat, W2t, T, c_star, ws, stream=None):
    """c* of RNN-head drafts: target dense [R][gamma+1][V]; feat [R][gamma][r]."""
    R, g1, V = target.shape
    r = int(feat.shape[-1])
    code = load().dspark_acceptance_rate_features(R, g1 - 1, V, r, float(T), _ptr(target),
                                                  _dt(target), _ptr(x), _ptr(lse_d), _ptr(U),
                                                  _dt(U), _ptr(feat), _ptr(W2t), _dt(feat),
                                                  _ptr(c_star), _ptr(ws), ws.numel(),
                                                  _stream(stream))
    _check("dspark_acceptance_rate_features", code)


def verify_cap_accept_features(ell, cap, cu, target, layout, x, logp_d, lse_d, U, feat, W2t, T,
                               seed, rnd, m, tau, emitted, next_anchor, ws, m_full=None,
                               logp_t=None, stream=None):
    """dspark_verify_cap_accept with the draft's per-position features."""
    R = ell.shape[0]
    gamma = x.shape[1] - 1
    V = target.shape[-1]
    r = int(feat.shape[-1])
    code = load().dspark_verify_cap_accept_features(
        R, gamma, V, r, float(T), seed, rnd, _ptr(ell), _ptr(cap), _ptr(cu), _ptr(target),
        _dt(target), int(layout), _ptr(x), _ptr(logp_d), _ptr(lse_d), _ptr(U), _dt(U), _ptr(feat),
        _ptr(W2t), _dt(feat), _ptr(m), _ptr(tau), _ptr(emitted), _ptr(next_anchor), _ptr(m_full),
        _ptr(logp_t), _ptr(ws), ws.numel(), _stream(stream))
    _check("dspark_verify_cap_accept_features", code)


def verify_features(ell, cu, target, layout, x, logp_d, lse_d, U, feat, W2t, T, seed, rnd, m, tau,
                    emitted, next_anchor, ws, logp_t=None, stream=None):
    """dspark_verify with the draft's per-position features feat [R][gamma][r]."""
    R = ell.shape[0]
    gamma = x.shape[1] - 1
    V = target.shape[-1]
    r = int(feat.shape[-1])
    code = load().dspark_verify_features(R, gamma, V, r, float(T), seed, rnd, _ptr(ell), _ptr(cu),
                                         _ptr(target), _dt(target), int(layout), _ptr(x),
                                         _ptr(logp_d), _ptr(lse_d), _ptr(U), _dt(U), _ptr(feat),
                                         _ptr(W2t), _dt(feat), _ptr(m), _ptr(tau), _ptr(emitted),
                                         _ptr(next_anchor), _ptr(logp_t), _ptr(ws), ws.numel(),
                                         _stream(stream))
    _check("dspark_verify_features", code)
