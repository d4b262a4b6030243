"""One DSpark round on the GPU: the C-ABI calls enqueued back to back (or, for
the Markov head with compact verify, the one call that enqueues them all).

draft (Markov head, or the RNN head) -> confidence -> prefix schedule (Algorithm 1, static, or
the asynchronous form with a two-slot capacity ring) -> pack the verify batch
(optionally padded to a graph tier) -> verify (compact: the scheduled window;
cap-accept: the whole block, committed within the scheduled window) -> pack
the emitted tokens.  This module only allocates the output
tensors (torch is the memory allocator) and calls the library in order; the
scheduled lengths, N, m and tau never leave the device.
"""
from __future__ import annotations

import torch

from . import _lib as L


class RoundBuffers:
    """Outputs and workspace of one round, allocated once and reused."""

    def __init__(self, R, gamma, V, device="cuda", slots=None, rnn=None):
        """rnn: (rank, d, weight dtype) to hold the RNN head's features and
        states (and its larger workspace)."""
        i32, f32 = torch.int32, torch.float32
        dev = torch.device(device)
        self.R, self.gamma, self.V = R, gamma, V
        self.x = torch.empty(R, gamma + 1, dtype=i32, device=dev)
        self.logp_d = torch.empty(R, gamma, dtype=f32, device=dev)
        self.lse_d = torch.empty(R, gamma, dtype=f32, device=dev)
        self.c = torch.empty(R, gamma, dtype=f32, device=dev)
        self.ell = torch.empty(R, dtype=i32, device=dev)
        self.a = torch.empty(R, gamma, dtype=f32, device=dev)
        self.N = torch.empty(1, dtype=i32, device=dev)
        self.theta = torch.empty(1, dtype=torch.float64, device=dev)
        cap = R * (gamma + 1)
        vs = max(cap, slots or 0)            # verify-batch slots (a graph tier may exceed cap)
        self.cu = torch.empty(R + 1, dtype=i32, device=dev)
        self.flat = torch.empty(vs, dtype=i32, device=dev)
        self.marker_req = torch.empty(vs, dtype=i32, device=dev)
        self.marker_pos = torch.empty(vs, dtype=i32, device=dev)
        self.N_pad = torch.empty(1, dtype=i32, device=dev)
        self.full = torch.full((R,), gamma, dtype=i32, device=dev)
        self.m_full = torch.empty(R, dtype=i32, device=dev)
        self.m = torch.empty(R, dtype=i32, device=dev)
        self.tau = torch.empty(R, dtype=i32, device=dev)
        self.emitted = torch.empty(R, gamma + 1, dtype=i32, device=dev)
        self.next_anchor = torch.empty(R, dtype=i32, device=dev)
        self.logp_t = torch.empty(R, gamma, dtype=f32, device=dev)
        self.cu_out = torch.empty(R + 1, dtype=i32, device=dev)
        self.flat_out = torch.empty(cap, dtype=i32, device=dev)
        self.N_out = torch.empty(1, dtype=i32, device=dev)
        self.feat = self.state = None
        if rnn is not None:
            rank, d, wdt = rnn
            self.feat = torch.empty(R, gamma, rank, dtype=wdt, device=dev)
            self.state = torch.empty(R, gamma, rank, dtype=f32, device=dev)
            self.ws = L.rnn_workspace(R, gamma, V, rank, d, device=dev)
        else:
            self.ws = L.workspace(R, gamma, V, device=dev)


class CapacityRing:
    """Verify capacities of the asynchronous scheduler, two device slots.

    The capacity that round t admits with was planned at round t - 2 from that
    round's confidences, so slot t % 2 is read and rewritten by round t (the
    scheduler reads its capacity before it writes the new plan).  Both slots
    start at the static block, min(R (gamma + 1), N_max)."""

    def __init__(self, R, gamma, N_max, device="cuda"):
        self.K = torch.full((2,), min(R * (gamma + 1), N_max), dtype=torch.int32,
                            device=torch.device(device))

    def slots(self, rnd):
        """(K_in, K_plan) of round `rnd`: the same device int."""
        s = self.K[rnd % 2: rnd % 2 + 1]
        return s, s


def run_round(inp, buf: RoundBuffers, T, seed, rnd, scheduler=True, layout=1, sts_T=None,
              stream=None, ring: CapacityRing = None, verify_mode="compact", tiers=None,
              pad_token=0, head="markov", single_call=False):
    """Enqueue one full round on `stream` (default: torch's current stream).

    `inp` holds U, W1, W2t, x0, h, w, sps and target (dense [R][gamma+1][V] for
    layout 1; packed rows in verify order for layout 0).  `scheduler`: True =
    Algorithm 1, False = static block, "async" = the asynchronous scheduler
    with capacities from `ring`.  `verify_mode` "cap-accept" packs and verifies
    the whole block and commits within the scheduled window.  `tiers` (host
    ints, ascending) pads the verify batch to the smallest tier that holds it
    (`buf.N_pad`; the buffers need slots >= the largest tier).  `head` "rnn"
    drafts with the RNN head (`inp["Wr"]`; buffers made with `rnn=`) and
    verifies with its features.  `single_call` enqueues the Markov-head round
    with compact verify (no tiers) as one call, dspark_round_markov, with the
    same results."""
    rnn = head == "rnn"
    if single_call:
        if rnn or verify_mode != "compact" or tiers:
            raise ValueError("single_call covers the Markov head with compact verify, no tiers")
        kin = kplan = None
        if scheduler == "async":
            kin, kplan = ring.slots(rnd)
        mode = 2 if scheduler == "async" else (1 if scheduler else 0)
        L.round_markov(inp["U"], inp["W1"], inp["W2t"], inp["x0"], inp["h"], inp["w"], inp["sps"],
                       inp["target"], layout, T, seed, rnd, buf.x, buf.logp_d, buf.lse_d, buf.c,
                       buf.ell, buf.cu, buf.flat, buf.m, buf.tau, buf.emitted, buf.next_anchor,
                       buf.cu_out, buf.flat_out, buf.ws, mode=mode, sts_T=sts_T, K_in=kin,
                       K_plan=kplan, a=buf.a, N=buf.N, theta=buf.theta,
                       marker_req=buf.marker_req, marker_pos=buf.marker_pos, logp_t=buf.logp_t,
                       N_out=buf.N_out, stream=stream)
        return
    if rnn:
        L.draft_rnn(inp["U"], inp["W1"], inp["W2t"], inp["Wr"], inp["h"], inp["x0"], T, seed, rnd,
                    buf.x, buf.logp_d, buf.lse_d, buf.feat, buf.ws, state=buf.state,
                    stream=stream)
    else:
        L.draft_markov(inp["U"], inp["W1"], inp["W2t"], inp["x0"], T, seed, rnd, buf.x,
                       buf.logp_d, buf.lse_d, buf.ws, stream=stream)
    L.confidence(inp["h"], inp["W1"], inp["w"], buf.x, buf.c, sts_T=sts_T, V=buf.V, stream=stream)
    kin = kplan = None
    if scheduler == "async":
        kin, kplan = ring.slots(rnd)
    if verify_mode != "cap-accept" and not tiers:
        # the schedule and the verify batch it implies in one launch
        mode = 2 if scheduler == "async" else (1 if scheduler else 0)
        L.schedule_pack(buf.c, inp["sps"], buf.x, buf.ell, buf.cu, buf.flat, mode=mode,
                        marker_req=buf.marker_req, marker_pos=buf.marker_pos, K_in=kin,
                        K_plan=kplan, a=buf.a, N_out=buf.N, theta=buf.theta, stream=stream)
    else:
        if scheduler == "async":
            L.async_schedule(buf.c, inp["sps"], kin, kplan, buf.ell, a=buf.a, N_out=buf.N,
                             theta=buf.theta, stream=stream)
        else:
            L.prefix_schedule(buf.c, inp["sps"], buf.ell, enabled=bool(scheduler), a=buf.a,
                              N_out=buf.N, theta_best=buf.theta, stream=stream)
        win = buf.full if verify_mode == "cap-accept" else buf.ell
        if tiers:
            L.pack_tiered(buf.x, win, 1, tiers, pad_token, buf.cu, buf.flat, buf.marker_req,
                          buf.marker_pos, buf.N, buf.N_pad, ws=buf.ws, stream=stream)
        else:
            L.pack(buf.x, win, 1, buf.cu, buf.flat, buf.marker_req, buf.marker_pos, buf.N,
                   ws=buf.ws, stream=stream)
    if verify_mode == "cap-accept" and rnn:
        L.verify_cap_accept_features(buf.full, buf.ell, buf.cu, inp["target"], layout, buf.x,
                                     buf.logp_d, buf.lse_d, inp["U"], buf.feat, inp["W2t"], T, seed,
                                     rnd, buf.m, buf.tau, buf.emitted, buf.next_anchor, buf.ws,
                                     m_full=buf.m_full, logp_t=buf.logp_t, stream=stream)
    elif verify_mode == "cap-accept":
        L.verify_cap_accept(buf.full, buf.ell, buf.cu, inp["target"], layout, buf.x, buf.logp_d,
                            buf.lse_d, inp["U"], inp["W1"], inp["W2t"], T, seed, rnd, buf.m,
                            buf.tau, buf.emitted, buf.next_anchor, buf.ws, m_full=buf.m_full,
                            logp_t=buf.logp_t, stream=stream)
    elif rnn:
        L.verify_features(buf.ell, buf.cu, inp["target"], layout, buf.x, buf.logp_d, buf.lse_d,
                          inp["U"], buf.feat, inp["W2t"], T, seed, rnd, buf.m, buf.tau,
                          buf.emitted, buf.next_anchor, buf.ws, logp_t=buf.logp_t, stream=stream)
    else:
        L.verify(buf.ell, buf.cu, inp["target"], layout, buf.x, buf.logp_d, buf.lse_d, inp["U"],
                 inp["W1"], inp["W2t"], T, seed, rnd, buf.m, buf.tau, buf.emitted, buf.next_anchor,
                 buf.ws, logp_t=buf.logp_t, stream=stream)
    L.pack(buf.emitted, buf.tau, 0, buf.cu_out, buf.flat_out, N_out=buf.N_out, ws=buf.ws,
           stream=stream)
