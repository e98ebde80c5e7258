"""Seeded synthetic inputs for one DSpark draft/verify round.

This module is shared by the tests, the smoke check and the benchmark.  It holds none of
the method's arithmetic: it draws the backbone outputs (base logits U, hidden states h),
the Markov-head and confidence-head weights, anchors and the engine step-time table, and
it stands in for the target model by synthesising target logits from the drafted tokens.
All randomness comes from numpy's PCG64 seeded per (configuration, seed, stream), so a
configuration is reproduced bit for bit.

Configurations (sizes and distributions of the five synthetic workloads):
  tiny     B=4,   gamma=4,  V=1024,   r=16,  d=64,   fp32 everything
  qwen1    B=1,   gamma=16, V=151936, r=256, d=2560, bf16 weights, full-block verify
  serve128 B=128, gamma=16, V=151936, r=256, d=2560, bf16 weights, scheduled verify
  v4dspark5 B=256, gamma=5, V=129280, r=256, d=4096, temperature 0.7, table x1.5
  bigvocab B=64,  gamma=16, V=262144, r=256, d=3840, peaked/flat logits, TV on all rows

Target logits (the stand-in for the target model's forward, computed after drafting):
  T_k = U_k + W1[x_{k-1}] W2 + sigma_k * N(0, 1),   k = 1..gamma+1,
where U_{gamma+1} is an extra base-logit row drawn only for this purpose.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# ------------------------------------------------------------------------------------
# configurations
# ------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int
    B: int
    gamma: int
    V: int
    r: int
    d: int
    bf16: bool              # weights / hidden states stored as bf16 (else fp32)
    temperature: float
    sched_mode: int         # 0 = greedy scheduler, 1 = full block
    logits: str             # "gauss2" | "zipf" | "peaked_flat"
    sigma0: float           # target noise sigma_k = sigma0 + sigma1 * k
    sigma1: float
    sigma_mix: bool         # per-request sigma scale from {0.2, 0.5, 1.0}
    table: str              # "tiny" | "serve" | "serve15"
    tv: bool                # analytic accept rate on every position
    wsigma: float = 0.0     # weight s.d. (0: 0.02 for bf16 weights, 0.1 for fp32)


CONFIGS = {
    "tiny": Config("tiny", 0, 4, 4, 1024, 16, 64, False, 1.0, 0, "gauss2", 0.5, 0.1, False,
                   "tiny", True),
    "qwen1": Config("qwen1", 1, 1, 16, 151936, 256, 2560, True, 1.0, 1, "zipf", 0.3, 0.05,
                    False, "serve", False),
    "serve128": Config("serve128", 2, 128, 16, 151936, 256, 2560, True, 1.0, 0, "zipf", 0.3,
                       0.05, True, "serve", False),
    "v4dspark5": Config("v4dspark5", 3, 256, 5, 129280, 256, 4096, True, 0.7, 0, "zipf", 0.3,
                        0.05, True, "serve15", False),
    "bigvocab": Config("bigvocab", 4, 64, 16, 262144, 256, 3840, True, 1.0, 0, "peaked_flat",
                       0.2, 0.08, False, "serve", True),
}
CONFIG_ORDER = ["tiny", "qwen1", "serve128", "v4dspark5", "bigvocab"]


def custom(name="custom", B=4, gamma=4, V=1024, r=16, d=64, bf16=False, temperature=1.0,
           sched_mode=0, logits="gauss2", sigma0=0.5, sigma1=0.1, sigma_mix=False,
           table="tiny", tv=True, wsigma=0.0) -> Config:
    """A configuration of arbitrary shape with the distributions of a named family."""
    return Config(name, 99, B, gamma, V, r, d, bf16, temperature, sched_mode, logits, sigma0,
                  sigma1, sigma_mix, table, tv, wsigma)


def step_time_ms(table: str, N: np.ndarray) -> np.ndarray:
    """Synthetic engine step time t(N) in ms at N verify tokens."""
    N = np.asarray(N, dtype=np.float64)
    if table == "tiny":
        return 10.0 + 0.05 * N
    if table == "serve":
        return 12.0 + 0.02 * N + 1e-5 * N * N
    if table == "serve15":
        return 1.5 * (12.0 + 0.02 * N + 1e-5 * N * N)
    if table == "flat":
        return np.full_like(N, 10.0)
    raise ValueError(table)


def sps_table(cfg: Config) -> np.ndarray:
    """Steps per second SPS(N) = 1000 / t(N) for N = 0..B(gamma+1), fp64."""
    N = np.arange(cfg.B * (cfg.gamma + 1) + 1, dtype=np.float64)
    return 1000.0 / step_time_ms(cfg.table, N)


# ------------------------------------------------------------------------------------
# helpers
# ------------------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the raw uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, cfg: Config, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed) & 0xFFFFFFFF, int(seed) >> 32, cfg.index, stream])


def _normal(rng, shape, sigma, chunk_rows=256):
    """fp32 N(0, sigma^2) of the given shape, drawn in row chunks to bound memory."""
    out = np.empty(shape, dtype=np.float32)
    if out.size == 0:           # e.g. no hidden state (d = 0)
        return out
    flat = out.reshape(-1, shape[-1])
    for i in range(0, flat.shape[0], chunk_rows):
        blk = rng.standard_normal(size=(min(chunk_rows, flat.shape[0] - i), shape[-1]),
                                  dtype=np.float32)
        if sigma != 1.0:
            blk *= np.float32(sigma)
        flat[i:i + blk.shape[0]] = blk
    return out


def _base_logits(rng, cfg: Config, rows: int, row_ids: np.ndarray) -> np.ndarray:
    """Base logits for `rows` rows of V entries; row_ids give (b*(gamma+1)+k) parities."""
    V = cfg.V
    if cfg.logits == "gauss2":
        return _normal(rng, (rows, V), 2.0)
    if cfg.logits == "zipf":
        # N(0, 3^2), then the 32 largest entries of each row get a Zipf(1.1)-ranked
        # boost of +8 * rank^-1.1 (rank 1 = largest).
        U = _normal(rng, (rows, V), 3.0)
        top = min(32, V)
        boost = (8.0 * np.arange(1, top + 1, dtype=np.float64) ** -1.1).astype(np.float32)
        for i in range(0, rows, 64):
            blk = U[i:i + 64]
            idx = np.argpartition(blk, V - top, axis=1)[:, V - top:]
            vals = np.take_along_axis(blk, idx, axis=1)
            order = np.take_along_axis(idx, np.argsort(-vals, axis=1, kind="stable"), axis=1)
            np.put_along_axis(blk, order, np.take_along_axis(blk, order, axis=1) + boost, axis=1)
        return U
    if cfg.logits == "peaked_flat":
        # Peaked rows (even b*gamma+k): N(0, 4^2) with +12 on the row's argmax.
        # Flat rows (odd): all-zero base logits, i.e. a uniform backbone distribution.
        U = np.zeros((rows, V), dtype=np.float32)
        for i in range(rows):
            if row_ids[i] % 2 == 0:
                row = rng.standard_normal(size=V, dtype=np.float32) * np.float32(4.0)
                row[int(np.argmax(row))] += np.float32(12.0)
                U[i] = row
        return U
    raise ValueError(cfg.logits)


# ------------------------------------------------------------------------------------
# inputs of one round
# ------------------------------------------------------------------------------------
@dataclasses.dataclass
class RoundInputs:
    cfg: Config
    seed: int               # RNG key handed to the method (draft/verify draws)
    U: np.ndarray           # [B][gamma][V] fp32 base logits
    U_extra: np.ndarray     # [B][V] fp32 base-logit row gamma+1 (target synthesis only)
    W1: np.ndarray          # [V][r] bf16 bits (uint16) or fp32
    W2t: np.ndarray         # [V][r] bf16 bits or fp32; W2 = W2t^T is [r][V]
    h: np.ndarray           # [B][gamma][d] bf16 bits or fp32
    w: np.ndarray           # [d + r] bf16 bits or fp32, order [h ; W1-row]
    anchor: np.ndarray      # [B] int32
    sigma: np.ndarray       # [B][gamma+1] fp32 target noise scale per row
    sps: np.ndarray         # [B(gamma+1)+1] fp64 steps/s

    @property
    def wdt(self) -> str:
        return "bf16" if self.cfg.bf16 else "f32"


def generate(cfg: Config, seed: int = 0) -> RoundInputs:
    """Draw every input of one round of `cfg` from `seed`."""
    B, G, V, r, d = cfg.B, cfg.gamma, cfg.V, cfg.r, cfg.d
    wsig = cfg.wsigma if cfg.wsigma > 0 else (0.02 if cfg.bf16 else 0.1)
    rng_w = _rng(seed, cfg, 1)
    W1 = _normal(rng_w, (V, r), wsig)
    W2t = _normal(rng_w, (V, r), wsig)
    rng_h = _rng(seed, cfg, 2)
    h = _normal(rng_h, (B, G, d), 1.0)
    w = _normal(rng_h, (1, d + r), 0.1)[0]
    anchor = rng_h.integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    rng_u = _rng(seed, cfg, 3)
    row_ids = (np.arange(B)[:, None] * G + np.arange(1, G + 2)[None, :])
    Uall = _base_logits(rng_u, cfg, B * (G + 1), row_ids.reshape(-1)).reshape(B, G + 1, V)
    U = np.ascontiguousarray(Uall[:, :G])
    U_extra = np.ascontiguousarray(Uall[:, G])
    del Uall
    k = np.arange(1, G + 2, dtype=np.float64)
    sig = cfg.sigma0 + cfg.sigma1 * k
    if cfg.sigma_mix:
        scale = _rng(seed, cfg, 4).choice(np.array([0.2, 0.5, 1.0]), size=B)
    else:
        scale = np.ones(B)
    sigma = (scale[:, None] * sig[None, :]).astype(np.float32)
    if cfg.bf16:
        W1, W2t, h, w = (to_bf16_bits(a) for a in (W1, W2t, h, w))
    method_seed = (0x5EED0000 + cfg.index * 0x1000 + int(seed)) | (0xD5A4 << 40)
    return RoundInputs(cfg, method_seed, U, U_extra, W1, W2t, h, w, anchor, sigma,
                       sps_table(cfg))


def weights_f32(x: np.ndarray) -> np.ndarray:
    """fp32 view of a weight array (bf16 bits widened, fp32 passed through)."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float32)


def synthesize_target(inp: RoundInputs, tokens: np.ndarray, rows: Optional[np.ndarray] = None,
                      noise_seed: int = 0) -> np.ndarray:
    """Target logits [len(rows)][gamma+1][V] fp32 for the drafted tokens [B][gamma].

    Stands in for the target model: T_k = U_k + W1[x_{k-1}] W2 + sigma_k N(0, 1), with
    x_0 = anchor and U_{gamma+1} the extra row.  `rows` selects requests (default all).
    The noise of request b depends only on (seed, b), so a subset reproduces the full
    batch's rows.
    """
    cfg = inp.cfg
    B, G, V = cfg.B, cfg.gamma, cfg.V
    rows = np.arange(B) if rows is None else np.asarray(rows)
    W1 = weights_f32(inp.W1)
    W2t = weights_f32(inp.W2t)
    T = np.empty((len(rows), G + 1, V), dtype=np.float32)
    for i, b in enumerate(rows):
        prev = np.concatenate([[inp.anchor[b]], np.asarray(tokens[b], dtype=np.int64)])
        bias = W1[prev] @ W2t.T                      # [gamma+1][V]
        base = np.concatenate([inp.U[b], inp.U_extra[b][None, :]], axis=0)
        rng = np.random.default_rng([int(inp.seed) & 0xFFFFFFFF, int(b), 77, noise_seed])
        noise = rng.standard_normal(size=(G + 1, V), dtype=np.float32)
        T[i] = base + bias + inp.sigma[b][:, None] * noise
    return T


# ------------------------------------------------------------------------------------
# a training batch of the draft and confidence heads
# ------------------------------------------------------------------------------------
@dataclasses.dataclass
class TrainingInputs:
    zd: np.ndarray         # [B][gamma][V] float32 draft logits
    zt: np.ndarray         # [B][gamma][V] float32 target logits
    labels: np.ndarray     # [B][gamma] int32 true next tokens
    conf_logit: np.ndarray  # [B][gamma] float32 confidence-head logits


def training_inputs(cfg: Config, seed: int = 0, B: Optional[int] = None) -> TrainingInputs:
    """One training batch of B (default cfg.B) blocks of gamma positions.
    Target logits: the configuration's base-logit family.  Draft logits: the target's plus
    N(0, s_k^2) with s_k = 2 (sigma0 + sigma1 k), so the draft drifts from the target with
    depth.  Labels: the target's argmax with probability 0.7, else a uniform token.
    Confidence logits: N(1, 1.5^2)."""
    B = cfg.B if B is None else int(B)
    G, V = cfg.gamma, cfg.V
    rng = _rng(seed, cfg, 7)
    R = B * G
    zt = _base_logits(rng, cfg, R, np.arange(R))
    zd = np.empty_like(zt)
    s_k = 2.0 * (cfg.sigma0 + cfg.sigma1 * np.arange(1, G + 1))
    for i in range(0, R, 256):
        n = min(256, R - i)
        noise = rng.standard_normal(size=(n, V), dtype=np.float32)
        noise *= s_k[(np.arange(i, i + n) % G)].astype(np.float32)[:, None]
        zd[i:i + n] = zt[i:i + n] + noise
    top = np.argmax(zt, axis=1)
    uni = rng.integers(0, V, size=R)
    labels = np.where(rng.random(R) < 0.7, top, uni).astype(np.int32)
    conf = (rng.normal(size=R) * 1.5 + 1.0).astype(np.float32)
    return TrainingInputs(zd.reshape(B, G, V), zt.reshape(B, G, V), labels.reshape(B, G),
                          conf.reshape(B, G))


# ------------------------------------------------------------------------------------
# held-out data for calibrating the confidence head
# ------------------------------------------------------------------------------------
@dataclasses.dataclass
class CalibrationInputs:
    logit: np.ndarray      # [n][gamma] float32 confidence logits of an over-confident head
    n_accept: np.ndarray   # [n] int32 accepted prefix lengths
    t_true: np.ndarray     # [gamma] float64 temperature that makes the head calibrated


def calibration_inputs(n: int, gamma: int, seed: int = 0,
                       t_true: Optional[np.ndarray] = None) -> CalibrationInputs:
    """n held-out drafted blocks.  The logit of position k is N(2 - 0.1 k, 2^2); the
    position is accepted, given the earlier ones were, with probability
    sigmoid(logit / t_true[k-1]) (by default t_true[k-1] = 1.3 + 0.05 k: a head that is
    over-confident by that temperature); n_accept is the length of the accepted prefix."""
    rng = np.random.Generator(np.random.PCG64([0xCA11B8, seed, n, gamma]))
    k = np.arange(1, gamma + 1)
    if t_true is None:
        t_true = 1.3 + 0.05 * k
    t_true = np.asarray(t_true, np.float64)
    logit = (rng.normal(size=(n, gamma)) * 2.0 + (2.0 - 0.1 * k)).astype(np.float32)
    p_acc = 1.0 / (1.0 + np.exp(-logit.astype(np.float64) / t_true))
    ok = rng.random((n, gamma)) < p_acc
    alive = np.cumprod(ok, axis=1)
    return CalibrationInputs(logit, alive.sum(axis=1).astype(np.int32), t_true)
