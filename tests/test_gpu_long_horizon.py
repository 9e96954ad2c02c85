"""GPU parity of the long-horizon cache modes against the CPU fp64 oracle.

One sink latent frame plus a sliding window, with the positional keys cached
before RoPE and rotated in the active context at attention time ([PL] App.
D.4 "Chunk-Causal Sliding-Window Attention", App. D.5 "Long-Horizon RoPE
Re-indexing", App. E "RoPE branch"); the reference is
``oracle.chunk_attention_reindexed_reference``. Same acceptance bar as the
other parity tests (relative Frobenius <= 1e-2, max abs <= 3e-2).
"""
import numpy as np
import pytest
import torch

import latent_kv_attention_cache_amd as vm
from gpu_cases import Run, compare
from workloads import custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    vm.load_library()


def _np(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy()


def test_sink_window_rollout_across_evictions():
    # 4x6 grid, one sink frame + a 6-frame window, 3-frame chunks: the context
    # fills up over chunks 0-1, frames leave it from chunk 2 on, and the ring
    # wraps repeatedly; the sink frame stays in slots [0, T) throughout.
    w = custom(4, 6, window_frames=6, chunk_frames=3, t_first=0).with_(sink_frames=1,
                                                                       rope_at_read=True)
    r = Run(w, fill=float("nan"))
    for c in range(10):
        t = 3 * c
        r.append(t, 3)
        out = r.attention(t, 3)
        if c in (0, 1, 2, 3, 5, 9):
            compare(_np(out)[0], r.reference(t_first=t, n_frames=3), f"sink rollout chunk {c}",
                    per_head_axis=1)
    compare(r.cache_rows(0, 1), r.append_reference(0, 1), "sink frame rows after 10 chunks")
    compare(r.cache_rows(27, 3), r.append_reference(27, 3), "raw k_R rows of the last chunk")


def test_sink_window_wan_shape_sampled_rows():
    # Wan2.1-1.3B latent grid, chunk at t = 18..20 (12 frames evicted), batch 2.
    w = custom(30, 52, window_frames=6, chunk_frames=3, t_first=18, batch=2).with_(
        sink_frames=1, rope_at_read=True)
    r = Run(w)
    out = _np(r.chunk_step())
    rng = np.random.default_rng(7)
    for b in range(2):
        idx = np.unique(np.concatenate([[0, 1559, 1560, w.n_q - 1], rng.choice(w.n_q, 60, replace=False)]))
        compare(out[b, idx], r.reference(b=b, query_tokens=idx), f"sink Wan b={b}", per_head_axis=1)


def test_rope_at_read_without_sink():
    w = custom(5, 13, window_frames=4, chunk_frames=2, t_first=7).with_(rope_at_read=True)
    r = Run(w)
    out = _np(r.chunk_step())
    compare(out[0], r.reference(), "rope at read, no sink", per_head_axis=1)
    compare(r.cache_rows(7, 2), r.append_reference(7, 2), "raw k_R rows")


def test_sink_window_fp32():
    w = custom(4, 6, window_frames=3, chunk_frames=1, t_first=5, dtype="f32").with_(
        sink_frames=1, rope_at_read=True)
    r = Run(w)
    out = _np(r.chunk_step())
    compare(out[0], r.reference(), "sink fp32", per_head_axis=1)
