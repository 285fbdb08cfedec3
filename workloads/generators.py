"""Seeded synthetic Q/K/V for the five benchmark shapes of the SparsePR attention call.

The pages ("Partition the Support, Reconstruct the Residual", Sec. 5 and
App. C) measure on activations of four video models that are not available
here; these generators stand in for them with the same shapes and structure:

* ``tiny``  - one head, 1024 tokens on an 8x8x16 (t,h,w) grid, d=64, fp32.
  Q and K are 8-component Gaussian mixtures that share one set of N(0,1)
  centres; every token draws its component independently; noise sigma 0.3;
  both scaled by d**-0.25.  V ~ N(0,1).
* ``small`` / ``mid`` / ``long`` / ``joint`` - random Fourier features of the
  integer (t,h,w) position: 64 frequency vectors Omega ~ N(0, 0.5^2) in 3-D
  (shared by Q and K and by all heads of a config), features
  [cos(p Omega), sin(p Omega)] (d=128, unnormalised), plus independent
  N(0, 0.5^2) token noise for Q and for K; V ~ N(0,1); four sink tokens per
  head whose key rows are scaled to 5x their norm; cast to bf16 (round to
  nearest even).
* ``joint`` appends 256 text tokens per head with Q, K ~ N(0, 0.75) per
  coordinate and V ~ N(0,1).

Token order is row-major over (t, h, w): n = (t*Hg + h)*Wg + w.

Seeds: per-head draws use ``numpy.random.default_rng([cfg_seed, b, h])``,
sink positions ``[cfg_seed, b, h, 7]``, text tokens ``[cfg_seed, b, h, 11]``
and draws shared by a whole config ``[cfg_seed, 999]``.

Grouped-query attention (``Hkv`` > 0, dividing ``H``): q holds the H query heads
drawn as above and k, v hold Hkv heads, K/V head j of batch entry b being the
k, v drawn for head (b, j * H / Hkv).

``step`` > 0 gives the inputs of a later call of the same heads (consecutive
denoising steps): same frequencies, positions, sinks and mixture centres, fresh
token noise and values from ``[cfg_seed, b, h, 1000 + step]`` (text tokens from
``[cfg_seed, b, h, 11, step]``).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    seed: int
    B: int
    H: int
    grid: Tuple[int, int, int]
    d: int
    dtype: str            # "f32" or "bf16"
    n_text: int
    Ck: int
    Cq: int
    M: int
    Ms: int
    rho: float
    lam: float
    rK: int = 48
    rQ: int = 64
    max_iters: int = 25
    tol: float = 1e-4
    generator: str = "rff"
    Hkv: int = 0          # K/V heads under grouped-query attention (0: one per query head)

    @property
    def Nv(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def N(self) -> int:
        return self.Nv + self.n_text

    @property
    def heads(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, WorkloadConfig] = {
    "tiny": WorkloadConfig("tiny", 1, 1, 1, (8, 8, 16), 64, "f32", 0, 16, 16, 32, 1024,
                           0.22, 1e-3, generator="mixture"),
    "small": WorkloadConfig("small", 2, 1, 12, (8, 32, 32), 128, "bf16", 0, 128, 128, 128, 256,
                            0.25, 1.0),
    "mid": WorkloadConfig("mid", 3, 1, 40, (21, 39, 40), 128, "bf16", 0, 512, 512, 256, 2048,
                          0.22, 1.0),
    "long": WorkloadConfig("long", 4, 1, 24, (33, 60, 60), 128, "bf16", 0, 1024, 1024, 512, 2048,
                           0.22, 1.0),
    "joint": WorkloadConfig("joint", 5, 2, 24, (21, 39, 40), 128, "bf16", 256, 512, 512, 256, 2048,
                            0.22, 1.0),
}
# parity-test shape with text tokens: the small video latent plus 128 text tokens, two heads
CONFIGS["small_text"] = CONFIGS["small"].with_(name="small_text", H=2, n_text=128)
# grouped-query attention parity shapes: two query heads on one K/V head (fp32, d = 64), and
# six query heads on two K/V heads with 64 text tokens (bf16, d = 128)
CONFIGS["tiny_gqa"] = CONFIGS["tiny"].with_(name="tiny_gqa", H=2, Hkv=1)
CONFIGS["small_gqa"] = CONFIGS["small"].with_(name="small_gqa", H=6, Hkv=2, n_text=64)


def config(name: str) -> WorkloadConfig:
    return CONFIGS[name]


def _positions(grid: Tuple[int, int, int]) -> np.ndarray:
    t, h, w = grid
    tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    return np.stack([tt.ravel(), hh.ravel(), ww.ravel()], axis=1).astype(np.float64)


_FEAT_CACHE: Dict[Tuple[int, Tuple[int, int, int], int], np.ndarray] = {}


def _fourier_features(cfg: WorkloadConfig) -> np.ndarray:
    key = (cfg.seed, cfg.grid, cfg.d)
    if key not in _FEAT_CACHE:
        rng = np.random.default_rng([cfg.seed, 999])
        omega = rng.normal(0.0, 0.5, size=(3, cfg.d // 2))
        ang = _positions(cfg.grid) @ omega
        _FEAT_CACHE[key] = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return _FEAT_CACHE[key]


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def head_inputs(cfg: WorkloadConfig, b: int, h: int, step: int = 0):
    """Q, K, V of one head as float32 arrays [N, d] (bf16-exact values for bf16 configs)."""
    N, Nv, d = cfg.N, cfg.Nv, cfg.d
    key = [cfg.seed, b, h] if step == 0 else [cfg.seed, b, h, 1000 + step]
    if cfg.generator == "mixture":
        centres = np.random.default_rng([cfg.seed, 999]).standard_normal((8, d))
        rng = np.random.default_rng(key)
        q_id = rng.integers(0, 8, size=Nv)
        q_noise = rng.standard_normal((Nv, d))
        k_id = rng.integers(0, 8, size=Nv)
        k_noise = rng.standard_normal((Nv, d))
        v = rng.standard_normal((Nv, d))
        scale = d ** -0.25
        q = scale * (centres[q_id] + 0.3 * q_noise)
        k = scale * (centres[k_id] + 0.3 * k_noise)
        q, k, v = (x.astype(np.float32) for x in (q, k, v))
    else:
        feat = _fourier_features(cfg)
        rng = np.random.default_rng(key)
        q = feat + np.float32(0.5) * rng.standard_normal((Nv, d), dtype=np.float32)
        k = feat + np.float32(0.5) * rng.standard_normal((Nv, d), dtype=np.float32)
        v = rng.standard_normal((Nv, d), dtype=np.float32)
        sinks = np.random.default_rng([cfg.seed, b, h, 7]).choice(Nv, size=4, replace=False)
        k[sinks] *= np.float32(5.0)
    if cfg.n_text:
        rng_t = np.random.default_rng([cfg.seed, b, h, 11] if step == 0 else [cfg.seed, b, h, 11, step])
        s = np.float32(np.sqrt(0.75))
        qt = s * rng_t.standard_normal((cfg.n_text, d), dtype=np.float32)
        kt = s * rng_t.standard_normal((cfg.n_text, d), dtype=np.float32)
        vt = rng_t.standard_normal((cfg.n_text, d), dtype=np.float32)
        q = np.concatenate([q, qt])
        k = np.concatenate([k, kt])
        v = np.concatenate([v, vt])
    assert q.shape == (N, d)
    if cfg.dtype == "bf16":
        q, k, v = _round_bf16(q), _round_bf16(k), _round_bf16(v)
    return q, k, v


def batch_inputs(cfg: WorkloadConfig, heads=None, step: int = 0):
    """Q, K, V as float32 arrays [B, H, N, d]; ``heads`` optionally restricts to a list of (b, h).
    Under grouped-query attention K and V are [B, Hkv, N, d] (no ``heads`` restriction)."""
    B, H = cfg.B, cfg.H
    out = np.empty((3, B, H, cfg.N, cfg.d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                out[:, b, h] = 0.0
                continue
            out[0, b, h], out[1, b, h], out[2, b, h] = head_inputs(cfg, b, h, step)
    if 0 < cfg.Hkv < H:
        assert heads is None and H % cfg.Hkv == 0
        G = H // cfg.Hkv
        return out[0], np.ascontiguousarray(out[1][:, ::G]), np.ascontiguousarray(out[2][:, ::G])
    return out[0], out[1], out[2]
