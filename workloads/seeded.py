"""Seeded Gaussian inputs for latent-cache chunk attention.

Every array is drawn from ``numpy.random.Generator(PCG64(SeedSequence(key)))``
with ``key = [cfg_id, layer, role, t, step, b]``:

* weights use ``t = step = b = 0``; ``role`` tells them apart;
* the token activations ``x`` are drawn per latent frame ``t``, batch element
  ``b`` and denoising step ``step``, so the content of any ring slot can be
  regenerated on its own.

Distributions: x ~ N(0, 1); W_Q, W_down, W_KR ~ N(0, 1/d_model);
W_K_up, W_V_up ~ N(0, 1/d_c) (std = 1/sqrt(fan_in), fan_in = input width).
For bf16 workloads every value is drawn in fp32 and rounded to bf16
(round-to-nearest-even); the returned fp32 arrays then hold exactly the bf16
values that the device receives, so a CPU reference can consume them as fp64.

Weight layouts (y = x @ W, row-major):
  w_q    [d_model, n_heads * (d_nope + d_rope)]  head-major columns, each head
                                                  [nope(d_nope) | rope(d_rope)]
  w_down [d_model, d_c]
  w_kr   [d_model, d_rope]
  w_k_up [n_heads, d_c, d_nope]
  w_v_up [n_heads, d_c, d_v]

``mixer_weights`` adds the query-latent and output-mixer weights of the full
attention layer:

  w_dq   [d_model, d_q]                    query down-projection
  w_uq   [d_q, n_heads * (d_nope + d_rope)] query up-projection, head-major
  w_o    [n_heads * d_v, d_model]           output mixer
"""
from __future__ import annotations

import numpy as np

ROLE_WQ, ROLE_WDOWN, ROLE_WKR, ROLE_WKUP, ROLE_WVUP, ROLE_X, ROLE_WDQ, ROLE_WUQ, ROLE_WO = range(9)


def _rng(key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def round_bf16(a) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32. Finite inputs only."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(a) -> np.ndarray:
    """bf16 bit patterns (uint16) of values already representable in bf16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("bf16_bits: values are not bf16-representable; round_bf16 first")
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(key, shape, std, dtype):
    a = _rng(key).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_bf16(a) if dtype == "bf16" else a


def weights(w, layer: int = 0) -> dict:
    """Seeded weights of one layer of workload ``w`` (fp32 arrays)."""
    D, H, dc = w.d_model, w.n_heads, w.d_c
    sd = 1.0 / np.sqrt(D)
    su = 1.0 / np.sqrt(dc)
    return {
        "w_q": _normal([w.cfg_id, layer, ROLE_WQ, 0, 0, 0], (D, H * w.d_head), sd, w.dtype),
        "w_down": _normal([w.cfg_id, layer, ROLE_WDOWN, 0, 0, 0], (D, dc), sd, w.dtype),
        "w_kr": _normal([w.cfg_id, layer, ROLE_WKR, 0, 0, 0], (D, w.d_rope), sd, w.dtype),
        "w_k_up": _normal([w.cfg_id, layer, ROLE_WKUP, 0, 0, 0], (H, dc, w.d_nope), su, w.dtype),
        "w_v_up": _normal([w.cfg_id, layer, ROLE_WVUP, 0, 0, 0], (H, dc, w.d_v), su, w.dtype),
    }


def mixer_weights(w, layer: int = 0) -> dict:
    """Seeded query-latent and output-mixer weights of one layer (fp32 arrays).
    Scaled so that the query latent, the queries and the layer output keep unit
    variance per entry for unit-variance inputs."""
    D, H = w.d_model, w.n_heads
    return {
        "w_dq": _normal([w.cfg_id, layer, ROLE_WDQ, 0, 0, 0], (D, w.d_q), 1.0 / np.sqrt(D), w.dtype),
        "w_uq": _normal([w.cfg_id, layer, ROLE_WUQ, 0, 0, 0], (w.d_q, H * w.d_head),
                        1.0 / np.sqrt(w.d_q), w.dtype),
        "w_o": _normal([w.cfg_id, layer, ROLE_WO, 0, 0, 0], (H * w.d_v, D),
                       1.0 / np.sqrt(H * w.d_v), w.dtype),
    }


def x_frame(w, t: int, b: int = 0, step: int = 0, layer: int = 0) -> np.ndarray:
    """Token activations of latent frame ``t`` for batch element ``b``: [T, d_model]."""
    return _normal([w.cfg_id, layer, ROLE_X, t, step, b], (w.tokens_per_frame, w.d_model),
                   1.0, w.dtype)


def x_frames(w, frames, b: int = 0, step: int = 0, layer: int = 0) -> np.ndarray:
    """Concatenation of ``x_frame`` over ``frames``: [len(frames) * T, d_model]."""
    frames = list(frames)
    if not frames:
        return np.zeros((0, w.d_model), np.float32)
    return np.concatenate([x_frame(w, t, b, step, layer) for t in frames], axis=0)
