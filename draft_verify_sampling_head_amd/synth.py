"""Seeded synthetic inputs shaped like the DSpark round's workloads.

This module only draws inputs; it holds none of the round's arithmetic.  Both
the GPU path and the CPU oracle consume the tensors it returns (the oracle via
host copies), so the two sides always see identical inputs.

The backbone (base logits U_k, hidden states h_k) and the target model
(target logits of the verify rows) are outside the round, so they are drawn:
  U_k     ~ N(0, sigma_U^2) per logit plus one planted peak per (request, k)
  target  row j (input x_j, distribution p_t^{j+1}) = U_{j+1} + N(0, sigma_{j+1}^2);
          row gamma (the bonus row) is a fresh base row plus noise of
          position gamma's width
  W1, W2  ~ N(0, 0.02^2)  (W2 stored transposed, [V][r])
  w       ~ N(0, 0.05^2), h ~ N(0, 1), anchors uniform in [0, V)
  SPS(B)  the engine cost table, dense for B = 0..N_max
  Wr      (RNN head) ~ N(0, (gain / sqrt(2r + d))^2), so the cell's
          pre-activations have a spread of about `gain`; drawn from a stream of
          its own, so the other inputs do not change
Sizes follow the pages' settings: block sizes 7-16, Qwen3 / DeepSeek
vocabularies (151936 / 129280), up to 1024 concurrent requests.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

VOCAB_QWEN3 = 151936
VOCAB_DEEPSEEK = 129280


@dataclass
class Config:
    name: str
    R: int
    gamma: int
    V: int
    rank: int
    d: int
    dtype: torch.dtype
    T: float
    scheduler: bool
    sigma_u: float
    peak: float                  # planted peak height (0: use margin mode)
    margin_mode: bool            # plant a top-1 margin ~ N(2, 1) instead of a fixed peak
    noise: tuple                 # per-position target noise std, length gamma
    hard_frac: float = 0.0       # fraction of requests with hard_noise
    hard_noise: float = 0.0
    sps: str = "linear"          # "linear" or "tabulated"
    data_seed: int = 1000
    philox_seed: int = 0
    extra: dict = field(default_factory=dict)


def _ramp(gamma, lo=0.4, hi=1.2):
    if gamma == 1:
        return (lo,)
    return tuple(lo + (hi - lo) * (k - 1) / (gamma - 1) for k in range(1, gamma + 1))


def config(idx: int, R=None, gamma=None, rank=None) -> Config:
    """Configurations 0-4; config 4 is a family, select a cell with R/gamma/rank."""
    if idx == 0:
        return Config("tiny-fp32", 4, 7, 32000, 256, 512, torch.float32, 1.0, True, 2.0, 6.0, False,
                      (0.5,) * 7, data_seed=1000)
    if idx == 1:
        return Config("greedy-qwen3-4b-shape", 64, 7, VOCAB_QWEN3, 256, 2560, torch.bfloat16, 0.0,
                      False, 3.0, 0.0, True, (1.0,) * 7, data_seed=1001)
    if idx == 2:
        return Config("stochastic-deepseek-vocab", 256, 16, VOCAB_DEEPSEEK, 256, 4096,
                      torch.bfloat16, 1.0, True, 2.0, 6.0, False, _ramp(16), data_seed=1002)
    if idx == 3:
        return Config("scheduler-stress", 1024, 15, VOCAB_QWEN3, 256, 4096, torch.bfloat16, 0.7,
                      True, 2.0, 6.0, False, (0.4,) * 15, hard_frac=0.3, hard_noise=2.0,
                      sps="tabulated", data_seed=1003)
    if idx == 4:
        R = 32 if R is None else R
        gamma = 8 if gamma is None else gamma
        rank = 256 if rank is None else rank
        return Config(f"sweep-R{R}-g{gamma}-r{rank}", R, gamma, VOCAB_DEEPSEEK, rank, 4096,
                      torch.bfloat16, 1.0, True, 2.0, 6.0, False, _ramp(gamma),
                      data_seed=1004 + 7 * R + 131 * gamma + rank)
    raise ValueError(idx)


def scaled(cfg: Config, **kw) -> Config:
    """The same recipe at other sizes (parity tests at oracle-friendly sizes)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    if "gamma" in kw and "noise" not in kw:
        g = kw["gamma"]
        d["noise"] = _ramp(g) if cfg.noise[0] != cfg.noise[-1] else (cfg.noise[0],) * g
    return Config(**d)


def sps_table(cfg: Config, N_max: int) -> torch.Tensor:
    """SPS(B) for B = 0..N_max, float64 (engine steps per second at batch B)."""
    B = torch.arange(N_max + 1, dtype=torch.float64)
    if cfg.sps == "linear":
        return 1.0 / (0.020 + 5e-5 * B)
    # 64 profiled points n_i = 32 (i + 1) with a step penalty every 256 tokens,
    # linear interpolation between points, SPS_0 below the first point and 0
    # (capacity exceeded) past the last one.
    n = torch.tensor([32.0 * (i + 1) for i in range(64)], dtype=torch.float64)
    t = 0.015 + 4e-5 * n + 0.003 * torch.floor(n / 256.0)
    s = 1.0 / t
    out = torch.zeros(N_max + 1, dtype=torch.float64)
    for b in range(N_max + 1):
        if b < 32:
            out[b] = s[0]
        elif b > 2048:
            out[b] = 0.0
        else:
            i = min(int((b - 32) // 32), 62)
            f = (b - n[i]) / 32.0
            out[b] = s[i] * (1 - f) + s[i + 1] * f
    return out


def _base_rows(g: torch.Generator, n_rows: int, V: int, cfg: Config, device) -> torch.Tensor:
    u = torch.randn(n_rows, V, generator=g, device=device, dtype=torch.float32) * cfg.sigma_u
    idx = torch.randint(0, V, (n_rows,), generator=g, device=device)
    ar = torch.arange(n_rows, device=device)
    if cfg.margin_mode:
        delta = torch.randn(n_rows, generator=g, device=device) + 2.0
        u[ar, idx] = -math.inf
        u[ar, idx] = u.max(dim=1).values + delta
    else:
        u[ar, idx] += cfg.peak
    return u


def make_inputs(cfg: Config, device="cpu", batch_rows: int = 2048) -> dict:
    """Draw every input of one round for `cfg` on `device` (deterministic per
    config and device type)."""
    g = torch.Generator(device=device)
    g.manual_seed(cfg.data_seed)
    R, G, V, r, d = cfg.R, cfg.gamma, cfg.V, cfg.rank, cfg.d
    dt = cfg.dtype
    hard = torch.zeros(R, dtype=torch.bool)
    if cfg.hard_frac > 0:
        perm = torch.randperm(R, generator=torch.Generator().manual_seed(cfg.data_seed))
        hard[perm[: int(round(cfg.hard_frac * R))]] = True
    noise = torch.tensor(cfg.noise, dtype=torch.float32)
    U = torch.empty(R, G, V, dtype=dt, device=device)
    target = torch.empty(R, G + 1, V, dtype=dt, device=device)
    per = max(1, batch_rows // (G + 1))
    for r0 in range(0, R, per):
        r1 = min(R, r0 + per)
        n = r1 - r0
        base = _base_rows(g, n * (G + 1), V, cfg, device).view(n, G + 1, V)
        U[r0:r1] = base[:, :G].to(dt)
        sig = noise.to(device).repeat(n, 1)                           # [n][G]
        if cfg.hard_frac > 0:
            hsel = hard[r0:r1].to(device)
            sig[hsel] = cfg.hard_noise
        sig = torch.cat([sig, sig[:, -1:]], dim=1)                    # bonus row: position G's width
        tb = torch.cat([base[:, :G].to(dt).float(), base[:, G:]], dim=1)
        eps = torch.randn(n, G + 1, V, generator=g, device=device)
        target[r0:r1] = (tb + eps * sig[:, :, None]).to(dt)
        del base, eps, tb
    out = dict(U=U, target=target)
    if r > 0:
        out["W1"] = (torch.randn(V, r, generator=g, device=device) * 0.02).to(dt)
        out["W2t"] = (torch.randn(V, r, generator=g, device=device) * 0.02).to(dt)
    else:
        out["W1"] = None
        out["W2t"] = None
    out["w"] = (torch.randn(d + r, generator=g, device=device) * 0.05).to(dt)
    out["h"] = torch.randn(R, G, d, generator=g, device=device).to(dt)
    out["x0"] = torch.randint(0, V, (R,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    N_max = R * (G + 1)
    out["sps"] = sps_table(cfg, N_max).to(device)
    out["hard"] = hard
    return out


def rnn_weights(cfg: Config, device="cpu", gain: float = 1.0) -> torch.Tensor:
    """Projection of the RNN head, Wr [3r][2r + d] in the config's dtype."""
    r, d = cfg.rank, cfg.d
    g = torch.Generator(device=device)
    g.manual_seed(cfg.data_seed + 7919)
    std = gain / math.sqrt(2 * r + d)
    return (torch.randn(3 * r, 2 * r + d, generator=g, device=device) * std).to(cfg.dtype)
