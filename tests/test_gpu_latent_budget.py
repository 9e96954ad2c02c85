"""GPU parity of the append and the attention core at other content widths:
d_c = 64, 128, 256 and 512 next to the default 192 (256 and 512 run the
wide-latent attention kernel, one wave per SIMD) (the latent-budget sweep, [PL] §4
"Batch Scaling Under Fixed Memory" over d_c in {64, 128, 192, 256, 512} and
App. F "Latent dimension"). The oracle is the same, dims-generic CPU fp64
reference; same acceptance bar (relative Frobenius <= 1e-2, max abs <= 3e-2).
"""
import numpy as np
import pytest
import torch

import latent_kv_attention_cache_amd as vm
from gpu_cases import Run, compare
from workloads import config, custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    vm.load_library()


def _np(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy()


@pytest.mark.parametrize("d_c", [64, 128])
def test_small_full_with_nan_ring(d_c):
    w = custom(4, 6, window_frames=3, chunk_frames=2, t_first=3).with_(d_c=d_c)
    r = Run(w, fill=float("nan"))
    out = _np(r.chunk_step())
    compare(out[0], r.reference(), f"d_c={d_c} 4x6", per_head_axis=1)
    compare(r.cache_rows(3, 2), r.append_reference(3, 2), f"d_c={d_c} cache rows")


@pytest.mark.parametrize("d_c", [64, 128])
def test_ragged_batch2_odd_heads(d_c):
    # 208 queries, 520 keys, batch 2, 5 heads (units of two heads share workgroups)
    w = custom(8, 13, window_frames=5, chunk_frames=2, t_first=3, batch=2).with_(d_c=d_c, n_heads=5)
    r = Run(w)
    out = _np(r.chunk_step())
    for b in range(2):
        compare(out[b], r.reference(b=b), f"d_c={d_c} ragged b={b}", per_head_axis=1)
        compare(r.cache_rows(0, 5, b=b), r.append_reference(0, 5, b=b), f"d_c={d_c} cache b={b}")


@pytest.mark.parametrize("d_c,n_rows", [(64, 32), (64, 320), (128, 160), (128, 4680)])
def test_append_tile_heights(d_c, n_rows):
    # row counts that select 1, 5, 3 and several rounds of row blocks per wave
    w = custom(1, n_rows, window_frames=2, chunk_frames=1, t_first=0).with_(d_c=d_c)
    r = Run(w)
    r.append(0, 1)
    compare(r.cache_rows(0, 1), r.append_reference(0, 1), f"d_c={d_c} append {n_rows} rows")


@pytest.mark.parametrize("d_c", [64, 128])
def test_sink_window_read_time_rope(d_c):
    w = custom(4, 6, window_frames=3, chunk_frames=1, t_first=6).with_(
        d_c=d_c, sink_frames=1, rope_at_read=True)
    r = Run(w, fill=float("nan"))
    out = _np(r.chunk_step())
    compare(out[0], r.reference(), f"d_c={d_c} sink + window", per_head_axis=1)


def test_fp32_d_c_64():
    w = custom(4, 6, window_frames=3, chunk_frames=1, t_first=5, dtype="f32").with_(d_c=64)
    r = Run(w)
    out = _np(r.chunk_step())
    compare(out[0], r.reference(), "d_c=64 fp32", per_head_axis=1)


@pytest.mark.parametrize("d_c", [64, 128])
def test_wan_shape_sampled_rows(d_c):
    w = config(2).with_(d_c=d_c)
    r = Run(w)
    out = _np(r.chunk_step())
    rng = np.random.default_rng(d_c)
    idx = np.unique(np.concatenate([[0, 31, 32, 1559, 1560, w.n_q - 1],
                                    rng.choice(w.n_q, 40, replace=False)]))
    compare(out[0, idx], r.reference(query_tokens=idx), f"d_c={d_c} config 2 sampled", per_head_axis=1)
    compare(r.cache_rows(18, 3), r.append_reference(18, 3), f"d_c={d_c} config 2 cache rows")


@pytest.mark.parametrize("d_c", [256, 512])
def test_wide_small_full_with_nan_ring(d_c):
    # 4x6 grid, 2-frame chunk at t = 3 after a wrap, B = 2, NaN-filled ring
    print(f"[case] wide d_c={d_c} small", flush=True)
    w = custom(4, 6, window_frames=3, chunk_frames=2, t_first=3, batch=2).with_(d_c=d_c)
    r = Run(w, fill=float("nan"))
    out = _np(r.chunk_step())
    for b in range(2):
        compare(out[b], r.reference(b=b), f"d_c={d_c} 4x6 b={b}", per_head_axis=1)
        compare(r.cache_rows(3, 2, b=b), r.append_reference(3, 2, b=b), f"d_c={d_c} cache rows b={b}")


@pytest.mark.parametrize("d_c", [256, 512])
def test_wide_ragged_odd_heads(d_c):
    # 7x9 grid: 126 queries (a partial unit, 4 units padded per head), 252
    # keys (a ragged last tile), 5 heads
    print(f"[case] wide d_c={d_c} ragged", flush=True)
    w = custom(7, 9, window_frames=4, chunk_frames=2, t_first=5).with_(d_c=d_c, n_heads=5)
    r = Run(w)
    out = _np(r.chunk_step())
    compare(out[0], r.reference(), f"d_c={d_c} ragged 5 heads", per_head_axis=1)


@pytest.mark.parametrize("d_c,n_rows", [(256, 160), (256, 4680), (512, 64), (512, 4680)])
def test_wide_append_tile_heights(d_c, n_rows):
    # 160-row ranges (5 blocks per wave) at 256; 64-row ranges (2 blocks) at 512
    print(f"[case] wide d_c={d_c} append {n_rows}", flush=True)
    w = custom(1, n_rows, window_frames=2, chunk_frames=1, t_first=0).with_(d_c=d_c)
    r = Run(w)
    r.append(0, 1)
    compare(r.cache_rows(0, 1), r.append_reference(0, 1), f"d_c={d_c} append {n_rows} rows")


@pytest.mark.parametrize("d_c", [256, 512])
def test_wide_wan_shape_sampled_rows(d_c):
    print(f"[case] wide d_c={d_c} Wan shape", flush=True)
    w = config(2).with_(d_c=d_c)
    r = Run(w)
    out = _np(r.chunk_step())
    rng = np.random.default_rng(d_c)
    idx = np.unique(np.concatenate([[0, 127, 128, w.n_q - 1], rng.choice(w.n_q, 28, replace=False)]))
    compare(out[0, idx], r.reference(query_tokens=idx), f"d_c={d_c} Wan sampled", per_head_axis=1)
    compare(r.cache_rows(18, 3), r.append_reference(18, 3), f"d_c={d_c} Wan chunk rows")


@pytest.mark.parametrize("d_c", [64, 128, 256, 512])
def test_query_prologue_tall_tiles(d_c):
    # 12 x 930 query rows: more than two rounds of 128-row prologue
    # workgroups, so the query prologue runs its 256-row tiles at this width;
    # sampled rows of the first and the last batch element (whose last rows
    # sit in the final, 152-row tile)
    print(f"[case] d_c {d_c} tall prologue tiles", flush=True)
    w = custom(30, 31, window_frames=2, chunk_frames=1, t_first=1, batch=12).with_(d_c=d_c)
    r = Run(w)
    out = _np(r.chunk_step())
    rng = np.random.default_rng(70 + d_c)
    for b in (0, 11):
        idx = np.unique(np.concatenate([[0, 31, 32, 255, 256, w.n_q - 1], rng.choice(w.n_q, 40, replace=False)]))
        compare(out[b, idx], r.reference(b=b, query_tokens=idx), f"d_c={d_c} tall tiles b={b}", per_head_axis=1)
