"""GPU parity of the explicit-reconstruction route (per-head K/V rebuilt from
the latent cache, then ordinary 128-dimensional attention; [PL] §3 "On-demand
reconstruction") against the CPU fp64 oracle ``chunk_attention_reference``,
which is itself the explicit definition. Same acceptance bar as the latent
path: relative Frobenius <= 1e-2, max abs <= 3e-2.
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


def _explicit(r, t_first=None, n_frames=None):
    w = r.w
    t_first = w.t_first if t_first is None else t_first
    n_frames = w.chunk_frames if n_frames is None else n_frames
    w_kv = vm.vmla_pack_kv_weights(r.dw["w_k_up"], r.dw["w_v_up"], dims=r.dims)
    x = r.x_dev(range(t_first, t_first + n_frames))
    n_valid = r.cache.n_valid_frames(t_first, n_frames)
    return vm.vmla_chunk_attention_explicit(r.cache, x, r.dw["w_q"], w_kv, t_first, n_frames, n_valid,
                                            dims=r.dims)


def test_packed_kv_weights_are_a_copy():
    w = custom(2, 3, window_frames=1, chunk_frames=1, t_first=0)
    r = Run(w)
    w_kv = _np(vm.vmla_pack_kv_weights(r.dw["w_k_up"], r.dw["w_v_up"], dims=r.dims))
    H, dn, dv = w.n_heads, w.d_nope, w.d_v
    blocks = w_kv.reshape(w.d_c, H, dn + dv)
    np.testing.assert_array_equal(blocks[:, :, :dn], r.wts["w_k_up"].transpose(1, 0, 2))
    np.testing.assert_array_equal(blocks[:, :, dn:], r.wts["w_v_up"].transpose(1, 0, 2))


def test_explicit_small_full():
    w = custom(4, 6, window_frames=3, chunk_frames=2, t_first=3)
    r = Run(w, fill=float("nan"))
    r.fill_window()
    r.append(w.t_first, w.chunk_frames)
    out = _np(_explicit(r))
    compare(out[0], r.reference(), "explicit 4x6", per_head_axis=1)


def test_explicit_ragged_batch2_and_key_counts():
    # 208 queries (6.5 units of 32), 520 keys (8.1 tiles of 64), batch 2
    w = custom(8, 13, window_frames=5, chunk_frames=2, t_first=3, batch=2)
    r = Run(w)
    r.fill_window()
    r.append(w.t_first, w.chunk_frames)
    out = _np(_explicit(r))
    for b in range(2):
        compare(out[b], r.reference(b=b), f"explicit ragged b={b}", per_head_axis=1)


@pytest.mark.parametrize("grid_h,grid_w", [(1, 1), (5, 13), (7, 223)])
def test_explicit_key_count_sweep(grid_h, grid_w):
    # N_k = 1, 65, 1561 with one frame: every key matters
    w = custom(grid_h, grid_w, window_frames=1, chunk_frames=1, t_first=0)
    r = Run(w)
    r.append(0, 1)
    out = _np(_explicit(r))
    compare(out[0], r.reference(), f"explicit N_k={grid_h * grid_w}", per_head_axis=1)


def test_explicit_equals_latent_route():
    # both routes against the same oracle, and against each other
    w = custom(6, 10, window_frames=4, chunk_frames=2, t_first=6)
    r = Run(w)
    latent = _np(r.chunk_step())
    explicit = _np(_explicit(r))
    ref = r.reference()
    compare(explicit[0], ref, "explicit", per_head_axis=1)
    compare(latent[0], ref, "latent", per_head_axis=1)
    compare(explicit[0], latent[0], "explicit vs latent", rel_frob=1e-2)


def test_explicit_wan_shape_sampled_rows():
    w = config(2)
    r = Run(w)
    r.fill_window()
    r.append(w.t_first, w.chunk_frames)
    out = _np(_explicit(r))
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([[0, 31, 32, 1559, 1560, w.n_q - 1],
                                    rng.choice(w.n_q, 40, replace=False)]))
    compare(out[0, idx], r.reference(query_tokens=idx), "explicit config 2 sampled", per_head_axis=1)


def test_explicit_fp32():
    w = custom(4, 6, window_frames=3, chunk_frames=1, t_first=5, dtype="f32")
    r = Run(w)
    r.fill_window()
    r.append(w.t_first, w.chunk_frames)
    out = _np(_explicit(r))
    compare(out[0], r.reference(), "explicit fp32", per_head_axis=1)
