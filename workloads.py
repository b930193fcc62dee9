"""Seeded synthetic Q/K/V and the workload presets.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark, so that both sides see bit-identical inputs. It holds input
generation only: none of the attention method's arithmetic lives here.

Inputs stand in for video-DiT self-attention activations. The pages evaluate
on Wan2.1 and HunyuanVideo; neither model nor any dataset is used here.
The field follows the shape of the AR(1) feature-drift proxy of
"DynamicRad: Content-Adaptive Sparse Attention for Long Video Diffusion"
(arXiv 2604.20470), Appendix C.2, Eq. 20: per token, features at frame f are
rho * (features at frame f-1) + sqrt(1 - rho^2) * fresh N(0, I) noise, so every
frame has unit variance. Here rho plays the role of sqrt(1 - delta^2).
Space is iid; a per-frame roll along the width axis models camera/object
shift. Q and K share the field, as in the proxy A_ij ~ exp(h_i^T h_j / sqrt(D)).

Generation recipe (per batch index b and head h):

* rng = numpy.random.default_rng([seed, b, h]); any head subset reproduces.
* X[0] ~ N(0, I) over (H_s, W_s, D); X[f] = rho * roll(X[f-1], shift, W)
  + sqrt(1 - rho^2) * N(0, I).
* periodic heads only: P ~ N(0, I) over (period, H_s, W_s, D), then
  X[f] <- sqrt(1 - a^2) * X[f] + a * P[f mod period].
* Q = X + 0.1 * N(0, I), K = X + 0.1 * N(0, I) (drawn in that order).
* V = X + 0.1 * N(0, I) when ``v_from_field`` else iid N(0, I).
* tokens are flattened frame-major, raster order within a frame, giving a
  [S, D] matrix with S = N_f * H_s * W_s.
* values are drawn in float32 and rounded to bfloat16 (round to nearest
  even); the oracle receives the same rounded values.

Head-level draws (per-head rho) use default_rng([seed, 9999]).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "bf16_round",
    "bf16_bits",
    "head_qkv",
    "head_rhos",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    num_frames: int
    frame_h: int
    frame_w: int
    block_size: int
    gamma: float
    lam: float
    seed: int
    # motion: one rho for all heads, or a per-head range drawn uniformly
    rho: Optional[float] = None
    rho_range: Optional[tuple] = None
    shift: int = 0
    periodic_frac: float = 0.0
    periodic_period: int = 8
    periodic_amp: float = 0.5
    v_from_field: bool = False
    theta_c: float = 0.0
    theta_m: float = 0.0
    # selection settings: the headline mode(s) and parity-only extras
    static_ratio: Optional[float] = None
    dynamic_tau: Optional[float] = None
    headline_modes: tuple = ()

    @property
    def tokens_per_frame(self) -> int:
        return self.frame_h * self.frame_w

    @property
    def seq_len(self) -> int:
        return self.num_frames * self.tokens_per_frame

    @property
    def num_blocks(self) -> int:
        return -(-self.seq_len // self.block_size)

    def periodic_heads(self) -> list:
        n = math.ceil(self.periodic_frac * self.heads - 1e-12) if self.periodic_frac > 0 else 0
        return list(range(self.heads - n, self.heads))

    def radial_kwargs(self) -> dict:
        return dict(num_frames=self.num_frames, tokens_per_frame=self.tokens_per_frame,
                    block_size=self.block_size, gamma=self.gamma, lam=self.lam,
                    theta_c=self.theta_c, theta_m=self.theta_m)


WORKLOADS = {
    # Tiny, CPU-checkable: 4 frames of 8x8 tokens, 2 heads, head_dim 64.
    "tiny": Workload(
        name="tiny", batch=1, heads=2, head_dim=64, num_frames=4, frame_h=8, frame_w=8,
        block_size=32, gamma=1.0, lam=2.0, seed=0, rho=0.9, shift=0, v_from_field=True,
        static_ratio=0.5, dynamic_tau=0.8, headline_modes=("static", "dynamic")),
    # Wan2.1-1.3B-shaped 480p: 21 latent frames of 30x52 tokens, low motion.
    "wan13b_480p": Workload(
        name="wan13b_480p", batch=1, heads=12, head_dim=128, num_frames=21, frame_h=30,
        frame_w=52, block_size=32, gamma=1.0, lam=4.0, seed=2, rho=0.95, shift=1,
        static_ratio=0.20, dynamic_tau=0.8, headline_modes=("static",)),
    # Wan2.1-14B-shaped 480p, high motion, 5% periodic heads (8-frame period).
    "wan14b_480p": Workload(
        name="wan14b_480p", batch=1, heads=40, head_dim=128, num_frames=21, frame_h=30,
        frame_w=52, block_size=32, gamma=0.7, lam=2.0, seed=3, rho=0.6, shift=4,
        periodic_frac=0.05, static_ratio=0.20, dynamic_tau=0.8, headline_modes=("dynamic",)),
    # Wan2.1-14B-shaped 720p: 21 latent frames of 45x80 tokens, mid motion.
    "wan14b_720p": Workload(
        name="wan14b_720p", batch=1, heads=40, head_dim=128, num_frames=21, frame_h=45,
        frame_w=80, block_size=32, gamma=1.0, lam=4.0, seed=4, rho=0.8, shift=2,
        static_ratio=0.15, dynamic_tau=0.8, headline_modes=("static", "dynamic")),
    # HunyuanVideo-shaped long 720p: 33 latent frames of 45x80, block size 64,
    # mixed motion across heads.
    "hunyuan_720p": Workload(
        name="hunyuan_720p", batch=1, heads=24, head_dim=128, num_frames=33, frame_h=45,
        frame_w=80, block_size=64, gamma=1.0, lam=4.0, seed=5, rho_range=(0.5, 0.95),
        shift=0, static_ratio=0.10, dynamic_tau=0.85, headline_modes=("dynamic", "static")),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32)


def head_rhos(w: Workload) -> np.ndarray:
    if w.rho_range is not None:
        rng = np.random.default_rng([w.seed, 9999])
        return rng.uniform(w.rho_range[0], w.rho_range[1], size=w.heads)
    return np.full(w.heads, float(w.rho))


def head_qkv(w: Workload, b: int, h: int, as_bits: bool = False):
    """Q, K, V of one (batch, head) as [S, D] arrays.

    Returns bfloat16-rounded float32 arrays, or their uint16 bit patterns when
    ``as_bits`` is set (for upload as torch.bfloat16).
    """
    rho = float(head_rhos(w)[h])
    rng = np.random.default_rng([w.seed, b, h])
    shape = (w.frame_h, w.frame_w, w.head_dim)
    X = np.empty((w.num_frames,) + shape, dtype=np.float32)
    X[0] = rng.standard_normal(shape, dtype=np.float32)
    keep = np.float32(rho)
    fresh = np.float32(math.sqrt(max(0.0, 1.0 - rho * rho)))
    for f in range(1, w.num_frames):
        prev = np.roll(X[f - 1], w.shift, axis=1) if w.shift else X[f - 1]
        X[f] = keep * prev + fresh * rng.standard_normal(shape, dtype=np.float32)
    if h in w.periodic_heads():
        P = rng.standard_normal((w.periodic_period,) + shape, dtype=np.float32)
        a = w.periodic_amp
        ca, sa = np.float32(math.sqrt(1.0 - a * a)), np.float32(a)
        for f in range(w.num_frames):
            X[f] = ca * X[f] + sa * P[f % w.periodic_period]
    S, D = w.seq_len, w.head_dim
    noise = np.float32(0.1)
    q = X.reshape(S, D) + noise * rng.standard_normal((S, D), dtype=np.float32)
    k = X.reshape(S, D) + noise * rng.standard_normal((S, D), dtype=np.float32)
    if w.v_from_field:
        v = X.reshape(S, D) + noise * rng.standard_normal((S, D), dtype=np.float32)
    else:
        v = rng.standard_normal((S, D), dtype=np.float32)
    if as_bits:
        return bf16_bits(q), bf16_bits(k), bf16_bits(v)
    return bf16_round(q), bf16_round(k), bf16_round(v)


def qkv(w: Workload, heads: Optional[Sequence[int]] = None, batches: Optional[Sequence[int]] = None,
        as_bits: bool = False):
    """Stacked [B', H', S, D] arrays for the requested batch/head subsets."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    dt = np.uint16 if as_bits else np.float32
    out = [np.empty((len(batches), len(heads), w.seq_len, w.head_dim), dtype=dt) for _ in range(3)]
    for i, b in enumerate(batches):
        for j, h in enumerate(heads):
            t = head_qkv(w, b, h, as_bits=as_bits)
            for o, x in zip(out, t):
                o[i, j] = x
    return tuple(out)


def _head_bits(args):
    w, b, h = args
    return head_qkv(w, b, h, as_bits=True)


def qkv_bits_parallel(w: Workload, heads: Optional[Sequence[int]] = None, workers: int = 8):
    """[B, H', S, D] uint16 bf16 patterns of Q, K, V, heads generated in worker
    processes (same values as head_qkv)."""
    from concurrent.futures import ProcessPoolExecutor
    heads = list(range(w.heads)) if heads is None else list(heads)
    jobs = [(w, b, h) for b in range(w.batch) for h in heads]
    out = [np.empty((w.batch, len(heads), w.seq_len, w.head_dim), dtype=np.uint16) for _ in range(3)]
    if workers <= 1 or len(jobs) == 1:
        results = map(_head_bits, jobs)
    else:
        ex = ProcessPoolExecutor(max_workers=min(workers, len(jobs)))
        results = ex.map(_head_bits, jobs)
    for (_, b, h), t in zip(jobs, results):
        j = heads.index(h)
        for o, x in zip(out, t):
            o[b, j] = x
    if workers > 1 and len(jobs) > 1:
        ex.shutdown()
    return tuple(out)


def proxy_qkz(num_frames: int, frame_h: int, frame_w: int, head_dim: int, heads: int, delta: float, seed: int,
              batch: int = 1, as_bits: bool = False):
    """Inputs of the proxy task of "DynamicRad" (arXiv 2604.20470) App. C.2:
    per token (spatial position) a feature that drifts over frames as the AR(1)
    process of Eq. 20, h_f = sqrt(1 - delta^2) h_{f-1} + delta eps_f with
    h_0, eps_f ~ N(0, I) (unit variance at every frame); queries and keys are
    that feature (the proxy attention A_ij ~ exp(h_i . h_j / sqrt(D))), and the
    values are an independent N(0, I) probe Z. Per (b, h):
    rng = default_rng([seed, 7, b, h]); draws in the order h_0, eps_1 ..
    eps_{N_f-1}, Z; float32, rounded to bfloat16. Returns [B, H, S, D] arrays
    (Q, K, Z), Q and K identical."""
    S, D = num_frames * frame_h * frame_w, head_dim
    dt = np.uint16 if as_bits else np.float32
    q = np.empty((batch, heads, S, D), dtype=dt)
    z = np.empty((batch, heads, S, D), dtype=dt)
    keep = np.float32(math.sqrt(1.0 - delta * delta))
    fresh = np.float32(delta)
    for b in range(batch):
        for h in range(heads):
            rng = np.random.default_rng([seed, 7, b, h])
            shape = (frame_h * frame_w, D)
            X = np.empty((num_frames,) + shape, dtype=np.float32)
            X[0] = rng.standard_normal(shape, dtype=np.float32)
            for f in range(1, num_frames):
                X[f] = keep * X[f - 1] + fresh * rng.standard_normal(shape, dtype=np.float32)
            Z = rng.standard_normal((S, D), dtype=np.float32)
            if as_bits:
                q[b, h], z[b, h] = bf16_bits(X.reshape(S, D)), bf16_bits(Z)
            else:
                q[b, h], z[b, h] = bf16_round(X.reshape(S, D)), bf16_round(Z)
    return q, q.copy(), z


# drift rates of the proxy task's motion regimes (App. C.2)
PROXY_DRIFT = {"low": 0.02, "mid": 0.15, "high": 0.40}


# [DR] Table 2, dynamic-threshold rows (BO-optimised presets of the paper's
# token-level selector): decay gamma, long-range lambda, mask threshold
# theta_m, column threshold theta_c, near / far thresholds tau_1 / tau_2.
TOKEN_PRESETS = {
    "low": dict(gamma=1.3, lam=0.4, theta_m=0.70, theta_c=0.45, tau_near=-1.2, tau_far=2.4),
    "mid": dict(gamma=1.4, lam=0.7, theta_m=0.70, theta_c=0.45, tau_near=-1.5, tau_far=2.0),
    "high": dict(gamma=1.6, lam=0.9, theta_m=0.55, theta_c=0.40, tau_near=-2.0, tau_far=2.4),
}


# [DR] Table 2, static rows: decay gamma, long-range lambda, theta_m, theta_c,
# near / far retention ratios rho_1 / rho_2 (Eq. 8).
STATIC_PRESETS = {
    "low": dict(gamma=2.0, lam=0.3, theta_m=0.75, theta_c=0.20, rho_near=0.25, rho_far=0.55),
    "mid": dict(gamma=1.3, lam=0.7, theta_m=0.60, theta_c=0.15, rho_near=0.75, rho_far=0.55),
    "high": dict(gamma=1.6, lam=0.8, theta_m=0.65, theta_c=0.15, rho_near=0.55, rho_far=0.50),
}


def static_workload(base: str, preset: str):
    """A workload's shape under a Table 2 static preset; returns
    (workload, (rho_near, rho_far))."""
    pr = STATIC_PRESETS[preset]
    w = dataclasses.replace(get_workload(base), name=f"{base}+static-{preset}", gamma=pr["gamma"], lam=pr["lam"],
                            theta_c=pr["theta_c"], theta_m=pr["theta_m"])
    return w, (pr["rho_near"], pr["rho_far"])


def token_workload(base: str, preset: str):
    """A workload's tensors (same seed and field) under a Table 2 preset of
    the token-level selector; returns (workload, (tau_near, tau_far))."""
    pr = TOKEN_PRESETS[preset]
    w = dataclasses.replace(get_workload(base), name=f"{base}+{preset}", gamma=pr["gamma"], lam=pr["lam"],
                            theta_c=pr["theta_c"], theta_m=pr["theta_m"])
    return w, (pr["tau_near"], pr["tau_far"])
