"""Seeded synthetic inputs for the recurrent-state step (shared by tests and bench).

This module only draws random numbers and rounds them to the stored dtypes; it
contains none of the state-update arithmetic, so the float64 oracle and the HIP
library can both consume its output without sharing any code.

Recipes (all drawn with numpy's PCG64, seeded per (config seed, stream, step) so
that any step can be regenerated on its own):

* q, k ~ N(0, 1) per element, then l2-normalised within each head in float64
  (the pages normalise queries and keys per head before the state update:
  DAMP paper, section 3.1), then rounded to the stored dtype;
* v ~ N(0, 1);
* GDN decay alpha ~ U(lo, hi) per (request, head);
* KDA decay alpha = exp(-softplus(x)), x ~ N(-4, 2) per key channel, so the
  channels span fast and slow retention;
* beta = sigmoid(N(0, 1));
* the initial state is zero (toy) or N(0, 0.05) in FP32 (serving shapes).

N(mu, sigma) means standard deviation sigma.  bf16 values are produced by
rounding the float64 draw to float32 and then to bf16, both round-to-nearest-
even; both sides read the same bits, so the double rounding is immaterial.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------- dtypes


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_stored(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 draw to its stored representation ('f32', 'bf16' bits or 'f16'
    binary16), through float32, round to nearest even at each step."""
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f16":
        return x32.astype(np.float16)
    raise ValueError(dtype)


def stored_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array."""
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, np.float16).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------- configs


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    dk: int
    dv: int
    steps: int
    in_dtype: str  # 'f32', 'bf16' or 'f16'
    decay: str  # 'scalar' (GDN) or 'vector' (KDA)
    alpha_lo: float = 0.90
    alpha_hi: float = 0.9999
    state_sigma: float = 0.0  # 0 -> zero initial state
    seed: int = 0
    K_hi: int = 0  # DAMP: rows kept in FP16
    plan_seed: int = 0
    group: int = 0  # DAMP: INT8 values per FP32 scale (0: one scale per row)
    sr: bool = False  # DAMP: value scaling and reordering plan
    # dasc static-horizon selection: gate kind (0 softplus, 1 bounded), a_s, cutoff
    gate: int = 0
    a_s: float = 0.0
    W_max: int = 0
    # dasc + replay
    L: int = 0
    slots: int = 0
    retention: float = 0.0
    K: int = 0
    extra: dict = field(default_factory=dict, compare=False, hash=False)


CONFIGS = {
    "gdn_toy": Config("gdn_toy", B=1, H=4, dk=64, dv=64, steps=32, in_dtype="f32",
                      decay="scalar", alpha_lo=0.80, alpha_hi=0.999, state_sigma=0.0,
                      seed=1001),
    "gdn_serving": Config("gdn_serving", B=256, H=32, dk=128, dv=128, steps=100,
                          in_dtype="bf16", decay="scalar", alpha_lo=0.90, alpha_hi=0.9999,
                          state_sigma=0.05, seed=1002),
    "kda_serving": Config("kda_serving", B=256, H=32, dk=128, dv=128, steps=100,
                          in_dtype="bf16", decay="vector", state_sigma=0.05, seed=1003),
    "damp_kda": Config("damp_kda", B=256, H=32, dk=128, dv=128, steps=100, in_dtype="bf16",
                       decay="vector", state_sigma=0.05, seed=1004, K_hi=16,
                       plan_seed=2004),
    # the DAMP paper's deployed layout: group-32 scales and value scaling/reordering
    "damp_kda_g32sr": Config("damp_kda_g32sr", B=256, H=32, dk=128, dv=128, steps=100,
                             in_dtype="bf16", decay="vector", state_sigma=0.05, seed=1006,
                             K_hi=16, plan_seed=2006, group=32, sr=True),
    # KDA checkpoints: one unit per (head, key channel) row, selected by static horizons
    "dasc_kda": Config("dasc_kda", B=512, H=32, dk=128, dv=128, steps=1, in_dtype="f32",
                       decay="vector", state_sigma=0.05, seed=1007, plan_seed=2007, L=4,
                       slots=512, K=8, gate=0, a_s=-0.3, W_max=16),
    "dasc_gdn": Config("dasc_gdn", B=512, H=32, dk=128, dv=128, steps=1, in_dtype="f32",
                       decay="scalar", alpha_lo=0.90, alpha_hi=0.9999, state_sigma=0.05,
                       seed=1005, plan_seed=2005, L=4, slots=512, retention=0.5, K=8),
}


def shrink(cfg: Config, **kw) -> Config:
    """Same recipe at other sizes (parity cases at sizes the oracle finishes fast)."""
    d = {f: getattr(cfg, f) for f in cfg.__dataclass_fields__}
    d.update(kw)
    return Config(**d)


def rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


_STREAM_STEP, _STREAM_STATE, _STREAM_PLAN, _STREAM_MASK, _STREAM_REPLAY = 1, 2, 3, 4, 5
_STREAM_VPLAN = 6
_STREAM_GATE = 7


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def draw_qkv_ab(g: np.random.Generator, lead: tuple, H: int, dk: int, dv: int, decay: str,
                alpha_lo: float, alpha_hi: float, in_dtype: str) -> dict:
    """Draw one set of per-token projections in the fixed order q, k, v, alpha, beta."""
    q = _l2n(g.standard_normal(lead + (H, dk)))
    k = _l2n(g.standard_normal(lead + (H, dk)))
    v = g.standard_normal(lead + (H, dv))
    if decay == "scalar":
        alpha = g.uniform(alpha_lo, alpha_hi, size=lead + (H,))
    else:
        alpha = np.exp(-_softplus(g.normal(-4.0, 2.0, size=lead + (H, dk))))
    beta = _sigmoid(g.standard_normal(lead + (H,)))
    return {
        "q": to_stored(q, in_dtype),
        "k": to_stored(k, in_dtype),
        "v": to_stored(v, in_dtype),
        "alpha": alpha.astype(np.float32),
        "beta": beta.astype(np.float32),
    }


def step_inputs(cfg: Config, step: int, B: int | None = None) -> dict:
    """Inputs of decode step `step`: q, k [B,H,dk]; v [B,H,dv] (stored dtype),
    alpha fp32 [B,H] or [B,H,dk], beta fp32 [B,H]."""
    B = cfg.B if B is None else B
    g = rng(cfg.seed, _STREAM_STEP, step)
    return draw_qkv_ab(g, (B,), cfg.H, cfg.dk, cfg.dv, cfg.decay, cfg.alpha_lo, cfg.alpha_hi,
                       cfg.in_dtype)


def initial_state(cfg: Config, S: int | None = None, layer: int = 0) -> np.ndarray:
    """FP32 state [S, H, dk, dv]: zero, or N(0, state_sigma)."""
    S = cfg.B if S is None else S
    shape = (S, cfg.H, cfg.dk, cfg.dv)
    if cfg.state_sigma == 0.0:
        return np.zeros(shape, np.float32)
    g = rng(cfg.seed, _STREAM_STATE, layer)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(cfg.state_sigma))


# ----------------------------------------------------------------- DAMP plan


def damp_key_perm(cfg: Config, n_cal: int = 256) -> np.ndarray:
    """Static per-head key-channel order for the mixed-precision state: the
    K_hi FP16 rows first, then the INT8 rows, each region in ascending channel
    order.  The FP16 set is a seeded draw biased toward slow decay: per head, a
    calibration sample of n_cal decay vectors is drawn from the same
    distribution as the inputs, channels are ranked by the geometric mean of
    their decay (largest first), and K_hi channels are chosen uniformly from the
    2*K_hi slowest.  Returns int32 [H, dk]."""
    g = rng(cfg.plan_seed, _STREAM_PLAN)
    H, dk, K_hi = cfg.H, cfg.dk, cfg.K_hi
    perm = np.zeros((H, dk), np.int32)
    for h in range(H):
        x = g.normal(-4.0, 2.0, size=(n_cal, dk))
        log_a = -_softplus(x)  # log of exp(-softplus(x))
        a_eff = np.exp(log_a.mean(axis=0))
        pool = np.argsort(-a_eff, kind="stable")[: min(dk, 2 * K_hi)]
        hi = np.sort(g.choice(pool, size=K_hi, replace=False))
        lo = np.setdiff1d(np.arange(dk), hi)
        perm[h] = np.concatenate([hi, lo]).astype(np.int32)
    return perm


def damp_value_plan(cfg: Config, sigma: float = 0.5) -> tuple[np.ndarray, np.ndarray]:
    """Static per-head value scaling and order for the mixed-precision state.

    Per head, value dimension v gets a scale c_v = exp(N(0, sigma)) (seeded); the
    stored order sorts the dimensions by the RMS they have after scaling, largest
    first.  The synthetic state has the same RMS in every dimension, so that order is
    ascending c_v (ties by index).  Returns (val_perm int32 [H, dv]: stored column ->
    original dimension, val_scale float32 [H, dv]: c of the dimension stored in each
    column)."""
    g = rng(cfg.plan_seed, _STREAM_VPLAN)
    H, dv = cfg.H, cfg.dv
    perm = np.zeros((H, dv), np.int32)
    scale = np.zeros((H, dv), np.float32)
    for h in range(H):
        c = np.exp(g.normal(0.0, sigma, size=dv)).astype(np.float32)
        order = np.argsort(c, kind="stable")  # RMS after scaling is proportional to 1 / c
        perm[h] = order.astype(np.int32)
        scale[h] = c[order]
    return perm, scale


def damp_group(cfg: Config) -> int:
    return cfg.dv if cfg.group == 0 else cfg.group


# ----------------------------------------------------------------- dasc


def gate_params(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic learned gate parameters (A_log, d), float32 [L, H, dk] (one per KDA
    (head, key) channel).  Layers differ in their typical decay and heads within a layer
    around it, so the static-horizon selection is ragged across layers and mixed within
    heads: per layer mu_l ~ U(-0.5, 1.5), per head an offset ~ N(0, 0.5), per channel
    d = mu_l + offset + N(0, 1) and A_log ~ N(0, 0.5)."""
    g = rng(cfg.plan_seed, _STREAM_GATE)
    L, H, dk = cfg.L, cfg.H, cfg.dk
    mu = g.uniform(-0.5, 1.5, L)
    head = g.normal(0.0, 0.5, (L, H))
    A_log = g.normal(0.0, 0.5, (L, H, dk))
    d = mu[:, None, None] + head[:, :, None] + g.normal(0.0, 1.0, (L, H, dk))
    return A_log.astype(np.float32), d.astype(np.float32)



def dasc_masks(cfg: Config, lo: int | None = None, hi: int | None = None) -> np.ndarray:
    """Seeded per-layer head masks uint8 [L, H] with ragged retained counts.

    The total retained count is retention * L * H; per-layer counts are drawn
    uniformly from [lo, hi] (default H/4 .. 3H/4) until they sum to the total,
    then each layer's heads are a uniform random subset."""
    g = rng(cfg.plan_seed, _STREAM_MASK)
    L, H = cfg.L, cfg.H
    total = int(round(cfg.retention * L * H))
    lo = H // 4 if lo is None else lo
    hi = (3 * H) // 4 if hi is None else hi
    while True:
        r = g.integers(lo, hi + 1, size=L - 1)
        last = total - int(r.sum())
        if lo <= last <= hi:
            r = np.append(r, last)
            break
    mask = np.zeros((L, H), np.uint8)
    for l in range(L):
        mask[l, g.choice(H, size=int(r[l]), replace=False)] = 1
    return mask


def replay_inputs(cfg: Config, layer: int, B: int | None = None) -> dict:
    """Cached draft projections for K draft tokens and the accepted counts.

    q, k [B,K,H,dk]; v [B,K,H,dv]; alpha [B,K,H] (scalar decay) or [B,K,H,dk];
    beta [B,K,H]; n_accept int32 [B] ~ U{0..K}."""
    B = cfg.B if B is None else B
    g = rng(cfg.seed, _STREAM_REPLAY, layer)
    d = draw_qkv_ab(g, (B, cfg.K), cfg.H, cfg.dk, cfg.dv, cfg.decay, cfg.alpha_lo,
                    cfg.alpha_hi, cfg.in_dtype)
    d["n_accept"] = g.integers(0, cfg.K + 1, size=B).astype(np.int32)
    return d
