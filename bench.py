"""Benchmark: one DSpark round (draft -> confidence -> schedule -> pack ->
verify -> pack) on one MI355X at the headline workload, R = 256 requests,
block size 16, vocabulary 129280, Markov rank 256, hidden 4096, bf16, T = 1,
scheduler on (Algorithm 1; --scheduler async selects the asynchronous form).

Prints ONE JSON line.  `value` = verified draft tokens per second
(sum of scheduled lengths ell over the timed rounds / their device time, each
round timed with events around its six stages on the launch stream), inputs
resident in HBM before the timed region; between rounds a 512 MiB scratch
buffer is written and a second one read, so that no round starts with W2 or U
in the memory-side cache (nor with the write's dirty lines in it).  The `roofline` object covers the
dominant kernel (the persistent draft kernel: all gamma steps in one
co-resident launch; the per-step statistics kernel when the shape takes the
per-step schedule), timed live with HIP events recorded on the launch stream
around each of its launches.  `cpu_baseline` is the single-threaded CPU oracle on a bounded
sample of requests of the same workload, scaled to a full round.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=2)
    p.add_argument("--R", type=int, default=None, help="config 4 (rank and length sweep): requests")
    p.add_argument("--gamma", type=int, default=None, help="config 4: block size")
    p.add_argument("--rank", type=int, default=None, help="config 4: Markov rank")
    p.add_argument("--scheduler", choices=["greedy", "async", "static"], default=None,
                   help="Algorithm 1, the asynchronous production form (capacity planned two "
                        "rounds earlier, top-K admission), or the static block; default: the "
                        "configuration's (Algorithm 1, or static where it turns scheduling off)")
    p.add_argument("--verify-mode", choices=["compact", "cap-accept"], default="compact",
                   help="verify the scheduled window (default) or the whole block, committed "
                        "within the scheduled window")
    p.add_argument("--head", choices=["markov", "rnn"], default="markov",
                   help="draft head: the Markov head (default) or the RNN head (recurrent cell "
                        "with per-position bias features; per-step schedule)")
    p.add_argument("--diagnostics", action="store_true",
                   help="also time the acceptance-rate (c*) pass on the last round and an STS "
                        "fit on synthetic held-out blocks")
    p.add_argument("--cpu-sample", type=int, default=48, help="requests in the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--flush-mib", type=int, default=512,
                   help="between timed rounds a scratch buffer of this many MiB is written, "
                        "then a second one read, so that no round starts with W2 or U warm in "
                        "the memory-side cache nor with dirty lines in it; 0 disables")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="before the rounds, copy a buffer of this many MiB three times "
                        "(device to device), the known-size reference for HBM byte counters")
    return p.parse_args()


class HipEvents:
    """Raw HIP events from the runtime torch already loaded."""

    def __init__(self, n):
        self.rt = C.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventDestroy.argtypes = [C.c_void_p]
        self.ev = (C.c_void_p * n)()
        for i in range(n):
            e = C.c_void_p()
            assert self.rt.hipEventCreate(C.byref(e)) == 0
            self.ev[i] = e
        self.n = n

    def array(self, start, count):
        return C.cast(C.byref(self.ev, start * C.sizeof(C.c_void_p)), C.POINTER(C.c_void_p))

    def elapsed_ms(self, a, b):
        out = C.c_float()
        rc = self.rt.hipEventElapsedTime(C.byref(out), self.ev[a], self.ev[b])
        assert rc == 0, rc
        return out.value

    def close(self):
        for i in range(self.n):
            self.rt.hipEventDestroy(self.ev[i])


def algorithmic_bytes(cfg, sum_tau, n_rej, N, head="markov"):
    """Bytes the round must move (per round): U once, the target rows up to
    the first rejection (or the bonus row), U rows of rejected positions, h,
    W2 once and the gathered W1 rows, w, and the outputs.  The RNN head adds
    its projection Wr once and its features (written once, read back by the
    statistics kernel)."""
    sU = sT = sh = sW = sw = 2 if cfg.dtype.itemsize == 2 else 4
    R, G, V, r, d = cfg.R, cfg.gamma, cfg.V, cfg.rank, cfg.d
    extra = sW * (3 * r * (2 * r + d) + 2 * R * G * r) if head == "rnn" else 0
    return (sU * R * G * V + sT * V * sum_tau + sU * V * n_rej + sh * R * G * d
            + sW * (r * V + R * G * r) + sw * (d + r) + R * G * 16 + N * 12 + extra)


def stats_kernel_bytes(cfg):
    """Algorithmic bytes of one launch of the draft statistics kernel: one U_k
    slab, the gathered W1 rows, the chunk statistics written, and W2 once per
    round amortised over the gamma launches."""
    s = cfg.dtype.itemsize
    nch = (cfg.V + 127) // 128
    return (s * cfg.R * cfg.V + s * cfg.R * cfg.rank + 8 * cfg.R * nch
            + (s * cfg.rank * cfg.V) / cfg.gamma)


# (kernel, head) -> (sources it is built from, committed counter summary of
# the headline workload R=256, gamma=16, V=129280, r=256)
_PERSIST_SRC = ("draft.hip", "persist_common.hpp", "launch.hpp", "device_common.hpp", "sampling.hpp",
                "workspace.hpp")
KERNELS = {
    ("k_draft_persistent", "markov"): (_PERSIST_SRC,
                                       "k_draft_persistent_R256_g16_V129280_r256_counters.txt"),
    ("k_draft_persistent", "rnn"): (_PERSIST_SRC,
                                    "k_draft_persistent_rnn_R256_g16_V129280_r256_counters.txt"),
}


def source_sha(key):
    """sha256 over the sources a kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNELS[key][0]:
        with open(os.path.join(ROOT, "draft_verify_sampling_head_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(key, cfg, config_idx):
    """HBM bytes per launch of the kernel `key` = (name, head) from its
    committed FETCH_SIZE / WRITE_SIZE summary, calibrated against a device copy
    of known size; None for other workloads, when the file is missing, or when
    the kernel sources have changed since the counters were taken."""
    if key not in KERNELS or config_idx != 2:
        return None
    try:
        kv = {}
        with open(os.path.join(ROOT, "profiles", KERNELS[key][1])) as fh:
            for line in fh:
                if ":" in line and not line.startswith((" ", "#", "|")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != source_sha(key):
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def draft_kernel_bytes(cfg):
    """Algorithmic bytes of the persistent draft launch (all gamma steps): U
    once, W2 once, the gathered W1 rows, the anchors and the outputs (x,
    logp_d, lse_d)."""
    s = cfg.dtype.itemsize
    R, G, V, r = cfg.R, cfg.gamma, cfg.V, cfg.rank
    return s * R * G * V + s * r * V + s * R * G * r + 4 * R + 12 * R * G


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the round shards by requests; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import draft_verify_sampling_head_amd as D
    from draft_verify_sampling_head_amd import _lib as L
    from draft_verify_sampling_head_amd import round as RD
    from draft_verify_sampling_head_amd import synth

    dev = torch.device("cuda:0")
    if args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: 3 x {nb} bytes")
        del src, dst
    if args.config == 4:
        cfg = synth.config(4, R=args.R, gamma=args.gamma, rank=args.rank)
    else:
        cfg = synth.config(args.config)
    t0 = time.time()
    inp = synth.make_inputs(cfg, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] config {args.config} ({cfg.name}) inputs ready in {time.time() - t0:.1f}s")
    K, W = args.steps, args.warmup
    rnn = args.head == "rnn"
    if rnn:
        inp["Wr"] = synth.rnn_weights(cfg, device=dev)
        buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=dev, rnn=(cfg.rank, cfg.d, cfg.dtype))
    else:
        buf = RD.RoundBuffers(cfg.R, cfg.gamma, cfg.V, device=dev)
    vmode = args.verify_mode
    ells = torch.empty(K + W, cfg.R, dtype=torch.int32, device=dev)
    ms = torch.empty(K + W, cfg.R, dtype=torch.int32, device=dev)
    Ns = torch.empty(K + W, dtype=torch.int32, device=dev)
    Nouts = torch.empty(K + W, dtype=torch.int32, device=dev)
    ev = HipEvents(2 * cfg.gamma * K)
    stream = torch.cuda.current_stream()

    n_timed = [0]
    sched = args.scheduler or ("greedy" if cfg.scheduler else "static")
    ring = RD.CapacityRing(cfg.R, cfg.gamma, inp["sps"].numel() - 1, device=dev)

    def one_round(i, timed):
        buf.ell, buf.m = ells[i], ms[i]
        buf.N, buf.N_out = Ns[i:i + 1], Nouts[i:i + 1]
        if rnn:
            j = (i - W) * 2 * cfg.gamma
            args_ = (inp["U"], inp["W1"], inp["W2t"], inp["Wr"], inp["h"], inp["x0"], cfg.T,
                     cfg.philox_seed, i, buf.x, buf.logp_d, buf.lse_d, buf.feat, buf.ws)
            if timed:
                n_timed[0] = L.draft_rnn_profiled(*args_, ev.array(j, cfg.gamma),
                                                  ev.array(j + cfg.gamma, cfg.gamma),
                                                  state=buf.state)
            else:
                L.draft_rnn(*args_, state=buf.state)
        elif timed:
            j = (i - W) * 2 * cfg.gamma
            n_timed[0] = L.draft_markov_profiled(inp["U"], inp["W1"], inp["W2t"], inp["x0"], cfg.T,
                                                 cfg.philox_seed, i, buf.x, buf.logp_d, buf.lse_d,
                                                 buf.ws, ev.array(j, cfg.gamma),
                                                 ev.array(j + cfg.gamma, cfg.gamma))
        else:
            L.draft_markov(inp["U"], inp["W1"], inp["W2t"], inp["x0"], cfg.T, cfg.philox_seed, i,
                           buf.x, buf.logp_d, buf.lse_d, buf.ws)
        L.confidence(inp["h"], inp["W1"], inp["w"], buf.x, buf.c, V=cfg.V)
        kin = kplan = None
        if sched == "async":
            kin, kplan = ring.slots(i)
        if vmode == "compact":
            # schedule and verify-batch pack in one launch
            L.schedule_pack(buf.c, inp["sps"], buf.x, buf.ell, buf.cu, buf.flat,
                            mode={"static": 0, "greedy": 1, "async": 2}[sched],
                            marker_req=buf.marker_req, marker_pos=buf.marker_pos, K_in=kin,
                            K_plan=kplan, a=buf.a, N_out=buf.N, theta=buf.theta)
        else:
            if sched == "async":
                L.async_schedule(buf.c, inp["sps"], kin, kplan, buf.ell, a=buf.a, N_out=buf.N,
                                 theta=buf.theta)
            else:
                L.prefix_schedule(buf.c, inp["sps"], buf.ell, enabled=(sched == "greedy"),
                                  a=buf.a, N_out=buf.N, theta_best=buf.theta)
            L.pack(buf.x, buf.full, 1, buf.cu, buf.flat, buf.marker_req, buf.marker_pos, buf.N,
                   ws=buf.ws)
        if vmode == "cap-accept" and rnn:
            L.verify_cap_accept_features(buf.full, buf.ell, buf.cu, inp["target"], 1, buf.x,
                                         buf.logp_d, buf.lse_d, inp["U"], buf.feat, inp["W2t"],
                                         cfg.T, cfg.philox_seed, i, buf.m, buf.tau, buf.emitted,
                                         buf.next_anchor, buf.ws, m_full=buf.m_full,
                                         logp_t=buf.logp_t)
        elif vmode == "cap-accept":
            L.verify_cap_accept(buf.full, buf.ell, buf.cu, inp["target"], 1, buf.x, buf.logp_d,
                                buf.lse_d, inp["U"], inp["W1"], inp["W2t"], cfg.T, cfg.philox_seed,
                                i, buf.m, buf.tau, buf.emitted, buf.next_anchor, buf.ws,
                                m_full=buf.m_full, logp_t=buf.logp_t)
        elif rnn:
            L.verify_features(buf.ell, buf.cu, inp["target"], 1, buf.x, buf.logp_d, buf.lse_d,
                              inp["U"], buf.feat, inp["W2t"], cfg.T, cfg.philox_seed, i, buf.m,
                              buf.tau, buf.emitted, buf.next_anchor, buf.ws, logp_t=buf.logp_t)
        else:
            L.verify(buf.ell, buf.cu, inp["target"], 1, buf.x, buf.logp_d, buf.lse_d, inp["U"],
                     inp["W1"], inp["W2t"], cfg.T, cfg.philox_seed, i, buf.m, buf.tau,
                     buf.emitted, buf.next_anchor, buf.ws, logp_t=buf.logp_t)
        L.pack(buf.emitted, buf.tau, 0, buf.cu_out, buf.flat_out, N_out=buf.N_out, ws=buf.ws)

    # between rounds a scratch buffer is written, so every round reads W2 and
    # U from HBM (the 256 MB memory-side cache holds nothing of them), and then
    # a second buffer is read: the write leaves the cache full of dirty lines,
    # and the read makes them drain before the round instead of inside it.
    # Each round is timed with events on the launch stream around its stages.
    flush = flush_rd = None
    if args.flush_mib > 0:
        flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
        flush_rd = torch.ones((args.flush_mib << 20) // 8, dtype=torch.int64, device=dev)

    def flush_caches(i):
        if flush is not None:
            flush.fill_(i & 0xFF)
            flush_rd.amax()
    r_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(K)]
    for i in range(W):
        flush_caches(i)
        one_round(i, False)
    torch.cuda.synchronize()
    log(f"[bench] {W} warmup rounds done")
    t_start = time.perf_counter()
    for i in range(W, W + K):
        flush_caches(i)
        r_ev[i - W][0].record(stream)
        one_round(i, True)
        r_ev[i - W][1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    round_ms = np.array([a.elapsed_time(b) for a, b in r_ev])
    t_total = float(round_ms.sum()) * 1e-3
    status = D.get_status(buf.ws)
    ms_per_step = float(round_ms.mean())

    ell_t = ells[W:].cpu().numpy().astype(np.int64)
    m_t = ms[W:].cpu().numpy().astype(np.int64)
    sum_ell = int(ell_t.sum())
    sum_tau = int((m_t + 1).sum())
    n_rej = int((m_t < ell_t).sum()) if cfg.T > 0 else 0
    N_avg = float(Ns[W:].cpu().numpy().mean())
    value = sum_ell / t_total
    bytes_round = sum(algorithmic_bytes(cfg, int((m_t[i] + 1).sum()), int((m_t[i] < ell_t[i]).sum()),
                                        int(Ns[W + i].item()), args.head) for i in range(K)) / K
    hbm_frac_round = bytes_round / (t_total / K) / (HBM_PEAK_GBS * 1e9)

    # dominant kernel, timed with events on its launch stream: the persistent
    # draft (one launch per round) or the per-step draft statistics kernel
    nt = n_timed[0]
    durs = []
    for i in range(K):
        j = i * 2 * cfg.gamma
        for k in range(nt):
            durs.append(ev.elapsed_ms(j + k, j + cfg.gamma + k))
    ev.close()
    avg_ms = float(np.mean(durs))
    if cfg.rank == 0 and not rnn:
        kernel = "k_row_stats"
        kdesc = "k_row_stats (rank 0: statistics of all R*gamma rows of U, one launch)"
        s = cfg.dtype.itemsize
        kb = s * cfg.R * cfg.gamma * cfg.V + 8 * cfg.R * cfg.gamma * ((cfg.V + 127) // 128)
        kflops = 0.0
    elif nt == 1:
        kernel = "k_draft_persistent"
        kdesc = ("k_draft_persistent (RNN head: cell, statistics and pick of all gamma steps, one "
                 "co-resident launch)" if rnn else
                 "k_draft_persistent (whole draft: gamma steps, one co-resident launch)")
        kb = draft_kernel_bytes(cfg)
        kflops = 2.0 * cfg.R * cfg.rank * cfg.V * cfg.gamma
    else:
        kernel = "k_markov_mfma" if cfg.dtype == torch.bfloat16 else "k_markov_valu"
        kdesc = (f"{kernel} (draft statistics of U_k + W2^T e_k, per step; RNN head)" if rnn
                 else f"{kernel} (draft statistics, per step)")
        kb = stats_kernel_bytes(cfg)
        kflops = 2.0 * cfg.R * cfg.rank * cfg.V
    achieved = kb / (avg_ms * 1e-3) / 1e9
    mfma_tf = kflops / (avg_ms * 1e-3) / 1e12
    log(f"[bench] round time (events, W2/U cold): median {np.median(round_ms):.3f} ms, p10 "
        f"{np.percentile(round_ms, 10):.3f}, p90 {np.percentile(round_ms, 90):.3f}; wall clock "
        f"{1e3 * t_wall / K:.3f} ms per round with the {args.flush_mib} MiB scratch write and read")
    log(f"[bench] {K} rounds: {ms_per_step:.3f} ms/round, sum_ell={sum_ell}, sum_tau={sum_tau}, "
        f"N_avg={N_avg:.1f}, n_rej={n_rej}, {kernel} {avg_ms * 1e3:.1f} us/launch "
        f"({achieved:.0f} GB/s, {mfma_tf:.0f} TFLOP/s), round HBM frac {hbm_frac_round:.3f}, "
        f"status={status}")

    copy_gbs = copy_bandwidth(torch, dev)
    log(f"[bench] device copy bandwidth {copy_gbs:.0f} GB/s (read + write, 1 GiB, median of 5)")
    diag = diagnostics(cfg, inp, buf, torch, np, D) if args.diagnostics else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, buf, args.cpu_sample, sum_ell / K, torch, np, sched,
                           int(Ns[W + K - 1].item()), args.head)
    out = {
        "metric": "verified draft tokens/s per round (B=256,γ=16,V=129280) + % peak HBM",
        "value": value,
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"dspark-round config {args.config} ({cfg.name})", "R": cfg.R,
                   "gamma": cfg.gamma, "V": cfg.V, "rank": cfg.rank, "d": cfg.d, "T": cfg.T,
                   "scheduler": sched, "verify_mode": vmode, "head": args.head,
                   "parallelism": "single-gpu"},
        "round_ms_median": float(np.median(round_ms)),
        "round_ms_p10": float(np.percentile(round_ms, 10)),
        "round_ms_p90": float(np.percentile(round_ms, 90)),
        "wall_ms_per_step_incl_flush": 1e3 * t_wall / K,
        "flush_mib_between_rounds": args.flush_mib,
        "hbm_frac_round": hbm_frac_round,
        "round_bytes_alg": bytes_round,
        "emitted_tokens_per_s": sum_tau / t_total,
        "mean_ell": sum_ell / (K * cfg.R),
        "mean_tau": sum_tau / (K * cfg.R),
        "device_status": status,
        "roofline": {"bound": "hbm", "kernel": kdesc,  # MFMA is the co-bound at rank > 0
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic((kernel, args.head), cfg, args.config),
                     "avg_launch_us": avg_ms * 1e3, "bytes_per_launch": kb,
                     "mfma_tflops": mfma_tf, "mfma_frac": mfma_tf / MFMA_BF16_PEAK_TFLOPS,
                     "copy_gbps_measured": copy_gbs, "frac_of_copy": achieved / copy_gbs},
        "hbm_frac_round_of_copy": bytes_round / (t_total / K) / (copy_gbs * 1e9),
        "cpu_baseline": cpu,
    }
    if diag is not None:
        out["diagnostics"] = diag
    print(json.dumps(out), flush=True)
    # orderly teardown while the runtime is fully alive: all work finished,
    # every device buffer released before the interpreter exits
    torch.cuda.synchronize()
    del buf, inp, flush, flush_rd, ells, ms, Ns, Nouts
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=5):
    """HBM bandwidth a plain device-to-device copy reaches on this GPU (bytes
    read + written per second, median of `reps` copies), measured after the
    timed rounds."""
    import statistics
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    times = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src)
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e) * 1e-3)
    del src, dst
    return 2 * nbytes / statistics.median(times) / 1e9


def diagnostics(cfg, inp, buf, torch, np, D):
    """Times (torch events on the launch stream) of the acceptance-rate pass
    over the whole block of the last round and of an STS fit on synthetic
    held-out blocks (n = 1024 rounds of R requests, 64 temperatures, 15 bins)."""
    dev = inp["U"].device
    cs = torch.empty(cfg.R, cfg.gamma, dtype=torch.float32, device=dev)
    if buf.feat is not None:          # RNN head: p_d from the draft's features
        run_c = lambda: D.acceptance_rate_features(inp["target"], buf.x, buf.lse_d, inp["U"],
                                                   buf.feat, inp["W2t"], cfg.T, cs, buf.ws)
    else:
        run_c = lambda: D.acceptance_rate(inp["target"], buf.x, buf.lse_d, inp["U"], inp["W1"],
                                          inp["W2t"], cfg.T, cs, buf.ws)
    n = 1024 * cfg.R
    g = torch.Generator(device="cpu").manual_seed(7)
    z = (torch.randn(n, cfg.gamma, generator=g) * 2.0 + 1.5).to(dev)
    m = torch.randint(0, cfg.gamma + 1, (n,), generator=g, dtype=torch.int32).to(dev)
    grid = [0.25 + 0.05 * i for i in range(64)]
    t = torch.empty(cfg.gamma, dtype=torch.float32, device=dev)
    ws = D.sts_workspace(n, device=dev)
    run_s = lambda: D.sts_fit(z, m, grid, t, ws, nbins=15)
    res = {}
    for name, fn, reps in [("acceptance_rate", run_c, 5), ("sts_fit", run_s, 3)]:
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name + "_ms"] = e0.elapsed_time(e1) / reps
    s = cfg.dtype.itemsize
    alg = 2.0 * s * cfg.R * cfg.gamma * cfg.V + s * cfg.rank * cfg.V
    res["acceptance_rate_alg_bytes"] = alg
    res["acceptance_rate_hbm_frac"] = alg / (res["acceptance_rate_ms"] * 1e-3) / (HBM_PEAK_GBS * 1e9)
    res["sts_fit_shape"] = {"n": n, "gamma": cfg.gamma, "grid": len(grid), "nbins": 15}
    res["sts_sigmoids_per_s"] = cfg.gamma * len(grid) * n / (res["sts_fit_ms"] * 1e-3)
    log(f"[bench] diagnostics: c* pass {res['acceptance_rate_ms']:.3f} ms "
        f"({res['acceptance_rate_hbm_frac']:.3f} of HBM peak on U + target + W2), STS fit "
        f"{res['sts_fit_ms']:.3f} ms for n={n}")
    return res


def cpu_baseline(cfg, inp, buf, n_req, ell_per_round, torch, np, sched="greedy", K_in=0,
                 head="markov"):
    """The oracle as it stands, on a bounded sample: draft + confidence +
    verify for n_req requests, the scheduler and both packs on the full batch;
    the per-request part is scaled to all R requests."""
    import oracle as O
    n_req = max(1, min(n_req, cfg.R))
    reqs = np.linspace(0, cfg.R - 1, n_req).round().astype(np.int32)
    sel = torch.as_tensor(reqs, device=inp["U"].device).long()
    f = lambda t: t.float().cpu().numpy()
    U, tgt, h = f(inp["U"][sel]), f(inp["target"][sel]), f(inp["h"][sel])
    W1, W2t, w = f(inp["W1"]), f(inp["W2t"]), f(inp["w"])
    x0 = inp["x0"][sel].cpu().numpy()
    sps = inp["sps"].cpu().numpy()
    c_all = buf.c.cpu().numpy()
    x_all = buf.x.cpu().numpy()
    t0 = time.perf_counter()
    feat = None
    if head == "rnn":
        x, lp, lse, _, _, feat, _, _ = O.draft_rnn(U, W1, W2t, f(inp["Wr"]), h, x0, cfg.T,
                                                   cfg.philox_seed, 0, req_ids=reqs,
                                                   bf16_e=cfg.dtype == torch.bfloat16)
    else:
        x, lp, lse, _ = O.draft_markov(U, W1, W2t, x0, cfg.T, cfg.philox_seed, 0, req_ids=reqs)
    c, _ = O.confidence(h, W1, w, x)
    t1 = time.perf_counter()
    c_all = c_all.copy()
    c_all[reqs] = c
    if sched == "async":
        ell = O.async_schedule(c_all, sps, K_in)[0]
    else:
        ell = O.prefix_schedule(c_all, sps, enabled=(sched == "greedy"))[0]
    O.pack(x_all, ell + 1)
    t2 = time.perf_counter()
    O.verify(ell[reqs], None, tgt, 1, x, lp, lse, U, W1, W2t, cfg.T, cfg.philox_seed, 0,
             req_ids=reqs, feat=feat)
    t3 = time.perf_counter()
    O.pack(x_all, ell + 1)
    t4 = time.perf_counter()
    per_req = ((t1 - t0) + (t3 - t2)) / n_req
    t_round = per_req * cfg.R + (t2 - t1) + (t4 - t3)
    log(f"[bench] oracle: {per_req:.2f} s/request (draft+conf+verify), schedule+pack "
        f"{(t2 - t1) + (t4 - t3):.3f} s, est. round {t_round:.1f} s")
    # the same sample with the requests split over the host's cores (the
    # oracle is single-threaded C called through ctypes, which releases the
    # interpreter lock, so the parts run at once); the scheduler and packs
    # stay single-threaded as above
    import concurrent.futures as cf
    cores = max(1, min(os.cpu_count() or 1, 16, n_req))
    parts = [p for p in np.array_split(np.arange(n_req), cores) if len(p)]

    def part(ix):
        rq = reqs[ix]
        if head == "rnn":
            xp, lpp, lsep, _, _, fp, _, _ = O.draft_rnn(U[ix], W1, W2t, f(inp["Wr"]), h[ix], x0[ix],
                                                       cfg.T, cfg.philox_seed, 0, req_ids=rq,
                                                       bf16_e=cfg.dtype == torch.bfloat16)
        else:
            xp, lpp, lsep, _ = O.draft_markov(U[ix], W1, W2t, x0[ix], cfg.T, cfg.philox_seed, 0,
                                              req_ids=rq)
            fp = None
        O.confidence(h[ix], W1, w, xp)
        O.verify(ell[rq], None, tgt[ix], 1, xp, lpp, lsep, U[ix], W1, W2t, cfg.T,
                 cfg.philox_seed, 0, req_ids=rq, feat=fp)

    t5 = time.perf_counter()
    with cf.ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(part, parts))
    t6 = time.perf_counter()
    t_round_all = (t6 - t5) / n_req * cfg.R + (t2 - t1) + (t4 - t3)
    log(f"[bench] oracle on {len(parts)} cores: {(t6 - t5):.2f} s for the sample, est. round "
        f"{t_round_all:.2f} s")
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": ell_per_round / t_round, "unit": "verified draft tokens/s", "cores": 1,
            "kind": "oracle", "host_cpu": model, "host_nproc": os.cpu_count(),
            "sample": f"{n_req} of {cfg.R} requests (draft+confidence+verify, {t3 - t0:.1f} s of "
                      f"CPU) scaled to {cfg.R}; scheduler and packs on the full batch; tokens per "
                      f"round = the GPU rounds' mean sum of ell ({ell_per_round:.1f})",
            "est_round_s": t_round,
            "all_cores": {"value": ell_per_round / t_round_all, "cores": len(parts),
                          "sample": "the same requests split over the cores, one oracle call per "
                                    "part; scheduler and packs single-threaded",
                          "est_round_s": t_round_all}}


if __name__ == "__main__":
    main()
