"""Closed-form memory and batch capacity of the latent cache.

Per request, every layer keeps d_c + d_rope scalars per cached token instead of
the 2 * n_heads * d_head of dense multi-head attention ([PL] §3 "Shared
low-rank KV cache", App. D.2: 224 against 3072 at the defaults). Over a
21-frame window of 1560-token latent frames and 30 layers that is the
per-request slope of the cache's memory; the pages measure the whole
per-request slope on a B200 ([PL] §4 "Batch Scaling Under Fixed Memory": 6.26
GB per request for dense attention, 0.57-1.43 GB across d_c in {64, ..., 512}),
which also holds per-request activations that the pages do not itemise.

Host-side planning arithmetic only: no GPU work, nothing of the kernels.
"""
from __future__ import annotations

GB = 1e9


def latent_scalars_per_token(d_c: int = 192, d_rope: int = 32) -> int:
    """Cached scalars per token per layer of the latent cache: [c | k_R]."""
    return d_c + d_rope


def dense_scalars_per_token(n_heads: int = 12, d_head: int = 128) -> int:
    """Cached scalars per token per layer of dense attention: K and V of every head."""
    return 2 * n_heads * d_head


def cache_bytes_per_request(scalars_per_token: int, layers: int = 30, frames: int = 21,
                            tokens_per_frame: int = 1560, bytes_per_scalar: int = 2,
                            sink_frames: int = 0) -> int:
    """Bytes one request keeps cached: every layer, every slot of the window."""
    return layers * (frames + sink_frames) * tokens_per_frame * scalars_per_token * bytes_per_scalar


def max_batch(budget_bytes: float, per_request_bytes: float, fixed_bytes: float = 0.0) -> int:
    """Largest batch whose per-request memory fits next to the fixed part."""
    if per_request_bytes <= 0:
        raise ValueError("per_request_bytes must be positive")
    return max(0, int((budget_bytes - fixed_bytes) // per_request_bytes))


# Per-request memory slopes measured on the pages ([PL] §4 "Batch Scaling
# Under Fixed Memory"), in GB per request: dense attention and the two ends of
# the d_c sweep.
PAGE_SLOPES_GB = {"mha": 6.26, 64: 0.57, 512: 1.43}


def _model_cache_bytes(key, **window) -> int:
    if key == "mha":
        return cache_bytes_per_request(dense_scalars_per_token(), **window)
    return cache_bytes_per_request(latent_scalars_per_token(key), **window)


def overhead_from_slopes(slopes=PAGE_SLOPES_GB, **window) -> float:
    """Per-request memory next to the cache, in bytes: the mean, over the
    measured slopes, of slope minus the closed-form cache bytes. It does not
    depend on the cache layout (activations of one request), so one value
    serves every width."""
    res = [slopes[k] * GB - _model_cache_bytes(k, **window) for k in slopes]
    return sum(res) / len(res)


def budget_window(limit_batch: int, per_request_bytes: float) -> tuple:
    """Budgets (bytes, next to the fixed part) under which ``limit_batch`` is
    the largest batch that fits: [B s, (B + 1) s)."""
    return limit_batch * per_request_bytes, (limit_batch + 1) * per_request_bytes


def sweep(d_cs=(64, 128, 192, 256, 512), budget_bytes: float = 288 * GB, fixed_bytes: float = 0.0,
          overhead_per_request: float = 0.0, **window) -> dict:
    """Cache bytes per request and the batch that fits, for dense attention and
    every latent width in ``d_cs``; ``overhead_per_request`` adds the
    non-cache per-request memory (activations) when it is known."""
    rows = {"mha": cache_bytes_per_request(dense_scalars_per_token(), **window)}
    for d_c in d_cs:
        rows[f"d_c={d_c}"] = cache_bytes_per_request(latent_scalars_per_token(d_c), **window)
    return {k: {"cache_bytes": v,
                "max_batch": max_batch(budget_bytes, v + overhead_per_request, fixed_bytes)}
            for k, v in rows.items()}
