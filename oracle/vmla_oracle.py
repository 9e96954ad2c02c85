"""CPU fp64 oracle for VideoMLA latent-cache chunk attention.

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference that the
HIP path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the product library
never does, and it shares no code with the HIP kernels (the only common import
is the seeded input generator in ``workloads/``, which holds no arithmetic of
the method).

Sources (web pages about arXiv:2605.30351v1, "VideoMLA: Low-Rank Latent KV
Cache for Minute-Scale Autoregressive Video Diffusion"):
  [PL] paperlayer.ai section-by-section summary (the most detailed page);
  [GI] gist.science Italian technical summary ("Riepilogo Tecnico: VideoMLA"),
       section "Metodologia", items 1-4.

What is computed, per batch element (all in float64, no intermediate
rounding):
  cache entry of token t   c_t = x_t W_down  (d_c)            [GI] item 1, [PL] §3
                           k^R_t = RoPE3D(x_t W_KR, p_t)     [GI] item 3, [PL] App. D.3
  per-head reconstruction  k^nope_{t,h} = c_t W_K_up[h]      [GI] item 2, [PL] §3
                           v_{t,h}      = c_t W_V_up[h]
  queries                  q = x W_Q; head h takes columns [h*d_h, (h+1)*d_h),
                           the first d_nope are q^nope, the last d_rope are
                           rotated: q^R = RoPE3D(., p_q)       [PL] App. D.3
  scores                   s = (q^nope . k^nope + q^R . k^R) * scale, over every
                           valid key of the window (no mask inside the window:
                           the query chunk sees earlier chunks and itself)
                                                               [PL] App. D.4
  softmax                  p = exp(s - max s) / sum exp(s - max s)
  output                   o_h = sum_k p_k v_{k,h}

Readings of points the pages leave open:
  * RoPE3D: 16 complex pairs, the first 6 on the t axis, then 5 on h, then 5 on
    w ([PL] App. D.3); pair j is the adjacent channels (2j, 2j+1); within an
    axis group of width D_a (12, 10, 10) pair i turns at
    omega_i = theta^(-2 i / D_a), theta = 10000, so i = 0 is the group's
    highest-frequency band. The pages print no frequencies; the law is
    pinned per axis group against the standard RoPE inverse frequencies of
    the transformers library (widths 12 / 10 / 10 and the split variants'
    groups), next to the (6,5,5) split and "highest bands first".
  * k^R is rotated with absolute (t, h, w) when it is cached. The pages rotate
    at window-assembly time with window-local t ([PL] App. D.5, App. E); with
    no sink frame both give the same scores by RoPE's relative invariance,
    which tests/test_oracle_pins.py checks.
  * y = x @ W with W stored [in, out]; W_Q columns are head-major, each head
    [nope | rope]; scale = 1/sqrt(d_nope + d_rope).
  * Token n of a frame is at (h, w) = (n // grid_w, n % grid_w); t is the
    absolute latent-frame index from 0.
  * Ring slot of token n of frame t: (t mod W) * T + n.
  * Long-horizon context ([PL] App. D.4-D.5): the sink frames are the first
    ones (frame 0 for one sink frame); the active context is the sink frames
    followed by the most recent window frames, numbered 0, 1, 2, ... oldest
    first, and those local numbers are the temporal RoPE coordinate of keys
    and queries (``chunk_attention_reindexed_reference``).
  * Whole clip under the chunk-causal block mask
    (``clip_chunk_causal_reference``): a query of chunk c sees the frames
    [e - window, e), e the end of chunk c -- its own chunk and earlier frames
    of the rolling window, never a later chunk ([PL] App. D.4); positions are
    absolute, as in the default cache mode.
  * Whole layer (``chunk_layer_reference``): queries through a query latent
    c_q = x W_DQ (d_q = 768, [PL] §4) and q = c_q W_UQ, no normalisation of
    c_q (the pages name none); the head outputs are concatenated head-major
    and mixed by W_O [H d_v, d_model]; A_h and B_h W_O[h] are the folded
    weights of [PL] App. E.
The pages print no worked example, so no output value comes from them; the
outputs are pinned through the identities, library routines (torch SDPA in
fp64, transformers' RoPE rates), closed forms and brute force of
tests/test_oracle_pins.py, at the benchmark geometry (30x52 grid, t up to 20,
the real widths) among others.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# Storage figures ([GI] item 4; [PL] §3 "Cache efficiency", App. D.2)
# ---------------------------------------------------------------------------

def cached_scalars_per_token(d_c: int, d_rope: int) -> int:
    """Per-token, per-layer cached state of the latent layout: d_c + d_rope."""
    return d_c + d_rope


def dense_scalars_per_token(n_heads: int, d_head: int) -> int:
    """Per-token, per-layer cached state of dense per-head KV: 2 * n_h * d_h."""
    return 2 * n_heads * d_head


# ---------------------------------------------------------------------------
# 3D-RoPE ([PL] App. C.1 and App. D.3)
# ---------------------------------------------------------------------------

def rope_pair_axes(pairs=(6, 5, 5)) -> np.ndarray:
    """Axis (0 = t, 1 = h, 2 = w) that each complex pair rotates with."""
    return np.concatenate([np.full(n, a, dtype=np.int64) for a, n in enumerate(pairs)])


def rope_frequencies(pairs=(6, 5, 5), axis_dims=(12, 10, 10), theta=10000.0) -> np.ndarray:
    """Angular rate of every pair: omega_i = theta^(-2 i / D_a) within its axis group."""
    om = []
    for n_pairs, dim in zip(pairs, axis_dims):
        for i in range(n_pairs):
            om.append(float(theta) ** (-2.0 * i / dim))
    return np.array(om, dtype=F64)


def frame_positions(t: int, grid_h: int, grid_w: int) -> np.ndarray:
    """(t, h, w) of every token of latent frame t, token order n = h * grid_w + w."""
    n = np.arange(grid_h * grid_w)
    return np.stack([np.full_like(n, t), n // grid_w, n % grid_w], axis=-1).astype(np.int64)


def rope3d(v, pos, omega, pairs=(6, 5, 5)) -> np.ndarray:
    """Rotate each adjacent pair (v[2j], v[2j+1]) by angle pos[axis(j)] * omega[j].

    v: [..., 2 * len(omega)]; pos: [..., 3] integer positions broadcastable to
    v's leading dims.
    """
    v = np.asarray(v, dtype=F64)
    pos = np.asarray(pos, dtype=F64)
    axes = rope_pair_axes(pairs)
    phi = pos[..., axes] * np.asarray(omega, dtype=F64)          # [..., n_pairs]
    cos, sin = np.cos(phi), np.sin(phi)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape, phi.shape[:-1] + (v.shape[-1],)), dtype=F64)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


# ---------------------------------------------------------------------------
# Latent cache entry ([GI] items 1 and 3; [PL] §3, App. D.2)
# ---------------------------------------------------------------------------

def latent_entry(x, w_down, w_kr, pos, omega, pairs=(6, 5, 5)):
    """Cache pair of each token: c = x W_down, k^R = RoPE3D(x W_KR, pos)."""
    x = np.asarray(x, dtype=F64)
    c = x @ np.asarray(w_down, dtype=F64)
    k_r = rope3d(x @ np.asarray(w_kr, dtype=F64), pos, omega, pairs)
    return c, k_r


# ---------------------------------------------------------------------------
# Explicit per-head reconstruction ([GI] item 2; [PL] §3 "On-demand reconstruction")
# ---------------------------------------------------------------------------

def reconstruct_heads(c, w_k_up, w_v_up):
    """k^nope_{t,h} = c_t W_K_up[h]  -> [N, H, d_nope];  v_{t,h} = c_t W_V_up[h] -> [N, H, d_v]."""
    c = np.asarray(c, dtype=F64)
    w_k_up = np.asarray(w_k_up, dtype=F64)
    w_v_up = np.asarray(w_v_up, dtype=F64)
    k_nope = np.stack([c @ w_k_up[h] for h in range(w_k_up.shape[0])], axis=1)
    v = np.stack([c @ w_v_up[h] for h in range(w_v_up.shape[0])], axis=1)
    return k_nope, v


def queries(x, w_q, pos, omega, n_heads, d_nope, d_rope, pairs=(6, 5, 5)):
    """q = x W_Q split per head into q^nope [N, H, d_nope] and rotated q^R [N, H, d_rope]."""
    q = (np.asarray(x, dtype=F64) @ np.asarray(w_q, dtype=F64)).reshape(-1, n_heads, d_nope + d_rope)
    q_nope = q[..., :d_nope]
    q_rope = rope3d(q[..., d_nope:], np.asarray(pos)[:, None, :], omega, pairs)
    return q_nope, q_rope


# ---------------------------------------------------------------------------
# Attention over reconstructed heads
# ---------------------------------------------------------------------------

def softmax_rows(s) -> np.ndarray:
    """Two-pass softmax over the last axis: exp(s - max) / sum exp(s - max)."""
    s = np.asarray(s, dtype=F64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_explicit(q_nope, q_rope, k_nope, k_r, v, scale, row_block=256):
    """o[q, h] = sum_k softmax_k(s[q, k, h]) v[k, h] with
    s = (q^nope_h . k^nope_{k,h} + q^R_h . k^R_k) * scale.

    Shapes: q_nope [Nq, H, dn], q_rope [Nq, H, dr], k_nope [Nk, H, dn],
    k_r [Nk, dr] (shared by all heads), v [Nk, H, dv]  ->  [Nq, H, dv].
    Query rows are independent; they are processed ``row_block`` at a time
    only to bound memory.
    """
    nq, nh, _ = q_nope.shape
    out = np.empty((nq, nh, v.shape[-1]), dtype=F64)
    k_r = np.asarray(k_r, dtype=F64)
    for h in range(nh):
        kh = np.concatenate([k_nope[:, h, :], k_r], axis=1)          # [Nk, dn + dr]
        vh = np.ascontiguousarray(v[:, h, :])
        for r0 in range(0, nq, row_block):
            qh = np.concatenate([q_nope[r0:r0 + row_block, h, :],
                                 q_rope[r0:r0 + row_block, h, :]], axis=1)
            p = softmax_rows((qh @ kh.T) * scale)
            out[r0:r0 + row_block, h, :] = p @ vh
    return out


def attention_absorbed(q_nope, q_rope, c, k_r, w_k_up, w_v_up, scale):
    """Latent-form inference ([PL] App. E), used only to cross-check the
    explicit form: q~_h = q^nope_h W_K_up[h]^T scores against c directly,
    the positional branch stays separate, the softmax-weighted latents are
    accumulated and then projected by W_V_up[h]."""
    c = np.asarray(c, dtype=F64)
    k_r = np.asarray(k_r, dtype=F64)
    nq, nh, _ = q_nope.shape
    out = np.empty((nq, nh, w_v_up.shape[-1]), dtype=F64)
    for h in range(nh):
        q_lat = q_nope[:, h, :] @ np.asarray(w_k_up[h], dtype=F64).T   # [Nq, d_c]
        s = (q_lat @ c.T + q_rope[:, h, :] @ k_r.T) * scale
        p = softmax_rows(s)
        out[:, h, :] = (p @ c) @ np.asarray(w_v_up[h], dtype=F64)
    return out


# ---------------------------------------------------------------------------
# Sliding-window ring of latent frames ([PL] App. C.1, App. D.4)
# ---------------------------------------------------------------------------

def ring_slot(t: int, n, tokens_per_frame: int, window_frames: int):
    """Slot of token n of absolute latent frame t: (t mod W) * T + n."""
    return (t % window_frames) * tokens_per_frame + np.asarray(n)


class LatentRing:
    """Per-batch-element ring of cached pairs (c, k^R), one row per slot.

    Appending frame t overwrites the slots of frame t - W (FIFO eviction);
    appending the same frame again (a later denoising step) overwrites it in
    place. Slots [0, n_valid_frames * T) are the valid window before the ring
    first wraps and all slots afterwards.
    """

    def __init__(self, batch, window_frames, grid_h, grid_w, d_c, d_rope):
        self.W, self.gh, self.gw = window_frames, grid_h, grid_w
        self.T = grid_h * grid_w
        self.c = np.full((batch, window_frames * self.T, d_c), np.nan, dtype=F64)
        self.k_r = np.full((batch, window_frames * self.T, d_rope), np.nan, dtype=F64)

    def append_frame(self, b, t, x_frame, w_down, w_kr, omega, pairs=(6, 5, 5)):
        pos = frame_positions(t, self.gh, self.gw)
        c, k_r = latent_entry(x_frame, w_down, w_kr, pos, omega, pairs)
        slots = ring_slot(t, np.arange(self.T), self.T, self.W)
        self.c[b, slots] = c
        self.k_r[b, slots] = k_r

    def valid(self, b, n_valid_frames):
        n = n_valid_frames * self.T
        return self.c[b, :n], self.k_r[b, :n]


# ---------------------------------------------------------------------------
# One chunk step: append the chunk, attend over the window
# ---------------------------------------------------------------------------

def window_frames(t_first: int, chunk_frames: int, window: int):
    """Latent frames held by the window once the chunk is appended (oldest first)."""
    t_end = t_first + chunk_frames
    return list(range(max(0, t_end - window), t_end))


def chunk_attention_reference(w, wts, x_of_frame, query_tokens=None):
    """Reference output of one chunk step of workload ``w`` for one batch element.

    ``wts``: dict of weights (``workloads.weights`` layout). ``x_of_frame(t)``
    returns the [T, d_model] activations last written for frame t (the query
    chunk's own frames included). ``query_tokens``: optional indices into the
    chunk's N_q tokens; default all. Returns [len(query_tokens), H, d_v].
    Keys are taken in frame order; by permutation invariance of the softmax
    this equals the ring's slot order (checked in the pins).
    """
    omega = rope_frequencies(w.rope_pairs, w.rope_axis_dims, w.rope_theta)
    frames = window_frames(w.t_first, w.chunk_frames, w.window_frames)
    cs, krs = [], []
    for t in frames:
        c, k_r = latent_entry(x_of_frame(t), wts["w_down"], wts["w_kr"],
                              frame_positions(t, w.grid_h, w.grid_w), omega, w.rope_pairs)
        cs.append(c)
        krs.append(k_r)
    c = np.concatenate(cs, axis=0)
    k_r = np.concatenate(krs, axis=0)
    k_nope, v = reconstruct_heads(c, wts["w_k_up"], wts["w_v_up"])

    chunk = list(range(w.t_first, w.t_first + w.chunk_frames))
    xq = np.concatenate([np.asarray(x_of_frame(t), dtype=F64) for t in chunk], axis=0)
    pos_q = np.concatenate([frame_positions(t, w.grid_h, w.grid_w) for t in chunk], axis=0)
    if query_tokens is not None:
        query_tokens = np.asarray(query_tokens)
        xq, pos_q = xq[query_tokens], pos_q[query_tokens]
    q_nope, q_rope = queries(xq, wts["w_q"], pos_q, omega, w.n_heads, w.d_nope, w.d_rope,
                             w.rope_pairs)
    scale = 1.0 / np.sqrt(w.d_nope + w.d_rope)
    return attention_explicit(q_nope, q_rope, k_nope, k_r, v, scale)


# ---------------------------------------------------------------------------
# Long-horizon context: sink frame + sliding window, RoPE at read time
# ([PL] App. D.4 "Chunk-Causal Sliding-Window Attention", App. D.5 "Long-Horizon
# RoPE Re-indexing", App. E "RoPE branch")
# ---------------------------------------------------------------------------

def active_context(t_first: int, chunk_frames: int, window: int, sink: int):
    """(absolute t, local t) of every frame of the active context once the chunk
    is appended, oldest first. The first ``sink`` frames stay for good; of the
    others the ``window`` most recent stay (FIFO eviction, [PL] App. D.4). The
    context is numbered 0, 1, 2, ... in that order: the frames get local
    temporal coordinates inside the sink-plus-window context ([PL] App. D.5)."""
    t_end = t_first + chunk_frames
    frames = list(range(min(sink, t_end))) + list(range(max(sink, t_end - window), t_end))
    return [(t, i) for i, t in enumerate(frames)]


def chunk_attention_reindexed_reference(w, wts, x_of_frame, query_tokens=None):
    """Reference output of one chunk step with read-time RoPE re-indexing.

    The cached positional keys are kept before RoPE (x W_KR); at attention time
    every frame of the active context (``active_context``) gets its local
    temporal coordinate, and the cached keys and the query chunk are rotated
    with it ([PL] App. D.5; App. E "RoPE branch"). Everything else is the
    definition of ``chunk_attention_reference``: explicit per-head K/V, softmax
    over every key of the context, no mask. Same arguments and result layout.
    """
    omega = rope_frequencies(w.rope_pairs, w.rope_axis_dims, w.rope_theta)
    ctx = active_context(w.t_first, w.chunk_frames, w.window_frames, w.sink_frames)
    local = dict(ctx)
    cs, krs = [], []
    for t, tl in ctx:
        x = np.asarray(x_of_frame(t), dtype=F64)
        cs.append(x @ np.asarray(wts["w_down"], dtype=F64))
        k_raw = x @ np.asarray(wts["w_kr"], dtype=F64)            # stored before RoPE
        krs.append(rope3d(k_raw, frame_positions(tl, w.grid_h, w.grid_w), omega, w.rope_pairs))
    c = np.concatenate(cs, axis=0)
    k_r = np.concatenate(krs, axis=0)
    k_nope, v = reconstruct_heads(c, wts["w_k_up"], wts["w_v_up"])

    chunk = list(range(w.t_first, w.t_first + w.chunk_frames))
    xq = np.concatenate([np.asarray(x_of_frame(t), dtype=F64) for t in chunk], axis=0)
    pos_q = np.concatenate([frame_positions(local[t], w.grid_h, w.grid_w) for t in chunk], axis=0)
    if query_tokens is not None:
        query_tokens = np.asarray(query_tokens)
        xq, pos_q = xq[query_tokens], pos_q[query_tokens]
    q_nope, q_rope = queries(xq, wts["w_q"], pos_q, omega, w.n_heads, w.d_nope, w.d_rope,
                             w.rope_pairs)
    scale = 1.0 / np.sqrt(w.d_nope + w.d_rope)
    return attention_explicit(q_nope, q_rope, k_nope, k_r, v, scale)


# ---------------------------------------------------------------------------
# A whole clip at once under the chunk-causal block mask ([PL] App. D.4
# "Chunk-Causal Sliding-Window Attention"; [PL] §3 "Integration with causal
# attention": causal block masks keep working on the reconstructed heads)
# ---------------------------------------------------------------------------

def chunk_causal_frame_mask(n_frames: int, chunk_frames: int, window: int) -> np.ndarray:
    """allowed[fq, fk] over the latent frames of a clip cut into chunks of
    ``chunk_frames`` frames (the last chunk may be shorter).

    A query in chunk c = fq // chunk_frames attends inside its own chunk and to
    earlier frames, never to a later chunk ([PL] App. D.4), and only to the
    ``window`` frames that end with its chunk: e - window <= fk < e with
    e = min((c + 1) chunk_frames, n_frames), i.e. exactly the frames a rolling
    cache of ``window`` frames holds right after chunk c is appended."""
    f = np.arange(n_frames)
    end = np.minimum((f // chunk_frames + 1) * chunk_frames, n_frames)
    return (f[None, :] < end[:, None]) & (f[None, :] >= end[:, None] - window)


def masked_attention(q_nope, q_rope, k_nope, k_r, v, scale, allowed, row_block=256):
    """``attention_explicit`` with a mask: scores of keys that are not allowed
    are -inf before the softmax, so their weight is exactly 0.
    allowed: bool [Nq, Nk], at least one key allowed per query row."""
    nq, nh, _ = q_nope.shape
    out = np.empty((nq, nh, v.shape[-1]), dtype=F64)
    k_r = np.asarray(k_r, dtype=F64)
    allowed = np.asarray(allowed, dtype=bool)
    for h in range(nh):
        kh = np.concatenate([k_nope[:, h, :], k_r], axis=1)
        vh = np.ascontiguousarray(v[:, h, :])
        for r0 in range(0, nq, row_block):
            qh = np.concatenate([q_nope[r0:r0 + row_block, h, :],
                                 q_rope[r0:r0 + row_block, h, :]], axis=1)
            s = np.where(allowed[r0:r0 + row_block], (qh @ kh.T) * scale, -np.inf)
            out[r0:r0 + row_block, h, :] = softmax_rows(s) @ vh
    return out


def clip_chunk_causal_reference(w, wts, x_of_frame, n_frames, window, query_tokens=None):
    """Reference output of the whole-clip form for one batch element: frames
    0 .. n_frames - 1 are cached at their absolute (t, h, w), every token of
    the clip is a query (absolute positions as well), keys and values are
    reconstructed per head, and the softmax runs over the keys that
    ``chunk_causal_frame_mask`` (chunks of ``w.chunk_frames``, ``window``
    frames) allows. ``query_tokens``: indices into the clip's n_frames * T
    tokens (frame-major); default all. Returns [len(query_tokens), H, d_v]."""
    omega = rope_frequencies(w.rope_pairs, w.rope_axis_dims, w.rope_theta)
    T = w.tokens_per_frame
    xs = [np.asarray(x_of_frame(t), dtype=F64) for t in range(n_frames)]
    pos = np.concatenate([frame_positions(t, w.grid_h, w.grid_w) for t in range(n_frames)], axis=0)
    xk = np.concatenate(xs, axis=0)
    c, k_r = latent_entry(xk, wts["w_down"], wts["w_kr"], pos, omega, w.rope_pairs)
    k_nope, v = reconstruct_heads(c, wts["w_k_up"], wts["w_v_up"])

    qt = np.arange(n_frames * T) if query_tokens is None else np.asarray(query_tokens)
    q_nope, q_rope = queries(xk[qt], wts["w_q"], pos[qt], omega, w.n_heads, w.d_nope, w.d_rope,
                             w.rope_pairs)
    frame_ok = chunk_causal_frame_mask(n_frames, w.chunk_frames, window)
    allowed = frame_ok[qt // T][:, np.arange(n_frames * T) // T]
    scale = 1.0 / np.sqrt(w.d_nope + w.d_rope)
    return masked_attention(q_nope, q_rope, k_nope, k_r, v, scale, allowed)


# ---------------------------------------------------------------------------
# The whole attention layer: query latent and output mixer
# ([PL] §4 "Implementation Details": d_q = 768; App. E "Content-path
# absorption", "Value-path absorption")
# ---------------------------------------------------------------------------

def query_latent_queries(x, w_dq, w_uq, pos, omega, n_heads, d_nope, d_rope, pairs=(6, 5, 5)):
    """Queries through the query latent: c_q = x W_DQ (d_q wide), then
    q = c_q W_UQ, split per head and rotated exactly as ``queries`` does."""
    c_q = np.asarray(x, dtype=F64) @ np.asarray(w_dq, dtype=F64)
    return queries(c_q, w_uq, pos, omega, n_heads, d_nope, d_rope, pairs)


def output_mixer(o, w_o):
    """Layer output y = [o_0 | o_1 | ... | o_{H-1}] W_O of the head outputs
    o [Nq, H, d_v] -> [Nq, d_model]."""
    o = np.asarray(o, dtype=F64)
    return o.reshape(o.shape[0], -1) @ np.asarray(w_o, dtype=F64)


def context_keys(w, wts, x_of_frame):
    """Keys of the attended context once the chunk is appended, and the
    temporal RoPE coordinate of every frame in it.

    Plain window (``w.rope_at_read`` false): the window's frames at their
    absolute t. Long-horizon mode: the sink-plus-window context of
    ``active_context`` at local coordinates. Returns (c [Nk, d_c],
    k_R [Nk, d_rope] rotated at those coordinates, {t: coordinate})."""
    omega = rope_frequencies(w.rope_pairs, w.rope_axis_dims, w.rope_theta)
    if w.rope_at_read:
        ctx = active_context(w.t_first, w.chunk_frames, w.window_frames, w.sink_frames)
    else:
        ctx = [(t, t) for t in window_frames(w.t_first, w.chunk_frames, w.window_frames)]
    cs, krs = [], []
    for t, tc in ctx:
        x = np.asarray(x_of_frame(t), dtype=F64)
        cs.append(x @ np.asarray(wts["w_down"], dtype=F64))
        krs.append(rope3d(x @ np.asarray(wts["w_kr"], dtype=F64),
                          frame_positions(tc, w.grid_h, w.grid_w), omega, w.rope_pairs))
    return np.concatenate(cs, axis=0), np.concatenate(krs, axis=0), dict(ctx)


def chunk_layer_reference(w, wts, mix, x_of_frame, query_tokens=None):
    """Reference output of one chunk step through the whole attention layer.

    Queries come from the query latent (``query_latent_queries`` with
    ``mix["w_dq"]``, ``mix["w_uq"]``); keys and values are reconstructed per
    head from the context of ``context_keys``; softmax over every key of it
    (no mask); the head outputs are mixed by ``mix["w_o"]``. ``wts`` holds the
    cache weights (``w_down``, ``w_kr``, ``w_k_up``, ``w_v_up``). Returns
    [len(query_tokens), d_model]."""
    omega = rope_frequencies(w.rope_pairs, w.rope_axis_dims, w.rope_theta)
    c, k_r, coord = context_keys(w, wts, x_of_frame)
    k_nope, v = reconstruct_heads(c, wts["w_k_up"], wts["w_v_up"])
    chunk = list(range(w.t_first, w.t_first + w.chunk_frames))
    xq = np.concatenate([np.asarray(x_of_frame(t), dtype=F64) for t in chunk], axis=0)
    pos_q = np.concatenate([frame_positions(coord[t], w.grid_h, w.grid_w) for t in chunk], axis=0)
    if query_tokens is not None:
        query_tokens = np.asarray(query_tokens)
        xq, pos_q = xq[query_tokens], pos_q[query_tokens]
    q_nope, q_rope = query_latent_queries(xq, mix["w_dq"], mix["w_uq"], pos_q, omega, w.n_heads,
                                          w.d_nope, w.d_rope, w.rope_pairs)
    scale = 1.0 / np.sqrt(w.d_nope + w.d_rope)
    return output_mixer(attention_explicit(q_nope, q_rope, k_nope, k_r, v, scale), mix["w_o"])


def fold_query_weights(w_uq, w_k_up, n_heads, d_nope, d_rope):
    """Per head [A_h | W_UQ^R[h]], head-major -> [d_q, H (d_c + d_rope)].

    A_h = W_UQ^nope[h] W_K_up[h]^T takes the query latent straight to the
    content score against c; it depends on no token, time step or position,
    so it is formed once ([PL] App. E "Content-path absorption"). The rope
    columns W_UQ^R[h] stay as they are: RoPE cannot be folded ("RoPE branch")."""
    w_uq = np.asarray(w_uq, dtype=F64).reshape(-1, n_heads, d_nope + d_rope)
    w_k_up = np.asarray(w_k_up, dtype=F64)
    blocks = [np.concatenate([w_uq[:, h, :d_nope] @ w_k_up[h].T, w_uq[:, h, d_nope:]], axis=1)
              for h in range(n_heads)]
    return np.concatenate(blocks, axis=1)


def fold_output_weights(w_v_up, w_o):
    """Per head B_h W_O[h], stacked head-major -> [H d_c, d_model]: the value
    up-projection folded into the output mixer, W_O[h] being the d_v rows of
    W_O that mix head h ([PL] App. E "Value-path absorption")."""
    w_v_up = np.asarray(w_v_up, dtype=F64)
    w_o = np.asarray(w_o, dtype=F64)
    d_v = w_v_up.shape[2]
    return np.concatenate([w_v_up[h] @ w_o[h * d_v:(h + 1) * d_v] for h in range(w_v_up.shape[0])],
                          axis=0)


def layer_latent_folded(c_q, pos_q, c, k_r, w_qa, w_vo, omega, n_heads, d_c, d_rope, scale,
                        pairs=(6, 5, 5)):
    """The layer in latent form, used to cross-check ``chunk_layer_reference``
    ([PL] App. E): per head, content score (c_q A_h) . c, positional score
    RoPE(c_q W_UQ^R[h]) . k_R, softmax, weighted latents p c, then
    y += (p c) (B_h W_O[h]). No per-head key or value is formed."""
    c_q = np.asarray(c_q, dtype=F64)
    c = np.asarray(c, dtype=F64)
    k_r = np.asarray(k_r, dtype=F64)
    row = d_c + d_rope
    y = np.zeros((c_q.shape[0], w_vo.shape[1]), dtype=F64)
    for h in range(n_heads):
        qa = c_q @ w_qa[:, h * row:h * row + d_c]
        qr = rope3d(c_q @ w_qa[:, h * row + d_c:(h + 1) * row], pos_q, omega, pairs)
        p = softmax_rows((qa @ c.T + qr @ k_r.T) * scale)
        y += (p @ c) @ w_vo[h * d_c:(h + 1) * d_c]
    return y


def append_reference_raw(w, wts, x_chunk):
    """Cache rows [n_frames * T, d_c + d_rope] = [c | x W_KR] when the
    positional keys are cached before RoPE ([PL] App. D.5)."""
    x = np.asarray(x_chunk, dtype=F64)
    return np.concatenate([x @ np.asarray(wts["w_down"], dtype=F64),
                           x @ np.asarray(wts["w_kr"], dtype=F64)], axis=1)


def append_reference(w, wts, x_chunk, t_first, n_frames):
    """Cache rows [n_frames * T, d_c + d_rope] = [c | k^R] of the appended frames."""
    omega = rope_frequencies(w.rope_pairs, w.rope_axis_dims, w.rope_theta)
    pos = np.concatenate([frame_positions(t, w.grid_h, w.grid_w)
                          for t in range(t_first, t_first + n_frames)], axis=0)
    c, k_r = latent_entry(x_chunk, wts["w_down"], wts["w_kr"], pos, omega, w.rope_pairs)
    return np.concatenate([c, k_r], axis=1)
