"""Workload shapes for latent-cache chunk attention.

Shapes follow the Wan2.1-T2V-1.3B backbone as the VideoMLA pages describe it
(paperlayer.ai summary of arXiv:2605.30351v1, "VideoMLA: Low-Rank Latent KV
Cache for Minute-Scale Autoregressive Video Diffusion" -- cited below as [PL]):
hidden size 1536, 12 heads of 128 ([PL] §4 and App. C.1), latent width
d_c = 192 with a 32-wide positional key ([PL] App. D.2), a 96/32 NoPE/RoPE
split ([PL] App. D.3, App. F), 1560 tokens per latent frame, 21 latent frames
per 5-second clip, chunks of 3 latent frames ([PL] App. D.1).

Token n of a frame sits at grid row n // grid_w and column n % grid_w.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    batch: int
    grid_h: int
    grid_w: int
    window_frames: int      # ring-buffer capacity in latent frames
    chunk_frames: int       # frames appended and queried per call
    t_first: int            # absolute latent-frame index of the query chunk
    dtype: str = "bf16"     # "bf16" or "f32": dtype of x, weights, cache and output
    n_layers: int = 1
    n_steps: int = 1        # denoising steps per chunk (rollout only)
    n_chunks: int = 1       # chunks in a rollout (rollout only)
    d_model: int = 1536
    n_heads: int = 12
    d_nope: int = 96
    d_rope: int = 32
    d_c: int = 192
    d_v: int = 128
    d_q: int = 768                    # query latent width ([PL] §4 Implementation Details)
    rope_pairs: tuple = (6, 5, 5)     # complex pairs on the t, h, w axes
    rope_axis_dims: tuple = (12, 10, 10)
    rope_theta: float = 10000.0
    sink_frames: int = 0              # latent frames kept for good at the front of the context
    rope_at_read: bool = False        # k_R cached before RoPE, rotated in the active context

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def n_q(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def n_valid_frames(self) -> int:
        """Frames in the active context once the chunk is appended: the sink
        frames plus the window, or the whole history while it is shorter."""
        return min(self.t_first + self.chunk_frames, self.sink_frames + self.window_frames)

    @property
    def n_k(self) -> int:
        return self.n_valid_frames * self.tokens_per_frame

    @property
    def d_head(self) -> int:
        return self.d_nope + self.d_rope

    @property
    def cache_row(self) -> int:
        return self.d_c + self.d_rope

    @property
    def prior_frames(self) -> tuple:
        """Frames that sit in the cache before the query chunk is appended: the
        sink frames, then the window's earlier frames."""
        lo = max(self.sink_frames, self.t_first + self.chunk_frames - self.window_frames)
        return tuple(range(min(self.sink_frames, self.t_first))) + tuple(range(lo, self.t_first))

    @property
    def chunk_frame_ids(self) -> tuple:
        return tuple(range(self.t_first, self.t_first + self.chunk_frames))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS = {
    1: Workload(1, "single layer B=1 fp32, 4x6 grid, 3-frame window, 1-frame chunk",
                batch=1, grid_h=4, grid_w=6, window_frames=3, chunk_frames=1,
                t_first=2, dtype="f32"),
    2: Workload(2, "Wan-1.3B shape, B=1, 30x52 grid, 21-frame window, 3-frame chunk",
                batch=1, grid_h=30, grid_w=52, window_frames=21, chunk_frames=3,
                t_first=18),
    3: Workload(3, "Wan-1.3B shape, B=8, 30 layers, 21-frame window, 3-frame chunk",
                batch=8, grid_h=30, grid_w=52, window_frames=21, chunk_frames=3,
                t_first=18, n_layers=30),
    4: Workload(4, "single-frame chunk, B=16, 21-frame window",
                batch=16, grid_h=30, grid_w=52, window_frames=21, chunk_frames=1,
                t_first=20),
    5: Workload(5, "minute-scale rollout, B=8, 240 frames in 80 chunks x 4 steps x 30 layers",
                batch=8, grid_h=30, grid_w=52, window_frames=21, chunk_frames=3,
                t_first=0, n_layers=30, n_steps=4, n_chunks=80),
}


def config(cfg_id: int) -> Workload:
    return CONFIGS[cfg_id]


def custom(grid_h: int, grid_w: int, window_frames: int, chunk_frames: int,
           t_first: int, batch: int = 1, dtype: str = "bf16", cfg_id: int = 100,
           name: str = "custom") -> Workload:
    """A workload with the model dims above and a free grid/window/chunk."""
    return Workload(cfg_id, name, batch=batch, grid_h=grid_h, grid_w=grid_w,
                    window_frames=window_frames, chunk_frames=chunk_frames,
                    t_first=t_first, dtype=dtype)


# NoPE/RoPE split variants of the 128-wide head ([PL] App. F "NoPE/RoPE
# split"): d_rope = 16, 64 or 96 next to the default 32. The pages give the
# t/h/w allocation of the default 16 complex pairs only, (6, 5, 5) over axis
# groups 12/10/10 wide; the variants keep its proportions (t takes 3/8 of the
# pairs, h the larger half of the rest) with groups twice as wide as their pair
# counts, so every axis keeps its highest-frequency band.
SPLIT_ROPE = {16: ((3, 3, 2), (6, 6, 4)), 32: ((6, 5, 5), (12, 10, 10)),
              64: ((12, 10, 10), (24, 20, 20)), 96: ((18, 15, 15), (36, 30, 30))}


def split_variant(w: Workload, d_rope: int) -> Workload:
    """Workload ``w`` with the NoPE/RoPE split (128 - d_rope) / d_rope."""
    pairs, dims = SPLIT_ROPE[d_rope]
    return w.with_(d_nope=128 - d_rope, d_rope=d_rope, rope_pairs=pairs, rope_axis_dims=dims)
