"""CPU fp64 oracle (test infrastructure only; see vmla_oracle.py's header)."""
from .vmla_oracle import *  # noqa: F401,F403
from .vmla_oracle import (cached_scalars_per_token, dense_scalars_per_token, rope_pair_axes,
                          rope_frequencies, frame_positions, rope3d, latent_entry,
                          reconstruct_heads, queries, softmax_rows, attention_explicit,
                          attention_absorbed, ring_slot, LatentRing, window_frames,
                          chunk_attention_reference, append_reference)
