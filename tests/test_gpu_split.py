"""GPU parity of the NoPE/RoPE split variants ([PL] App. F "NoPE/RoPE
split"): 112/16, 64/64 and 32/96 next to the default 96/32, at d_c = 192. The
cache rows are d_c + d_rope wide, the absorbed queries [q_lat | q_rope] too;
the append, the query prologue, the attention kernel and the explicit route
take the split as a template width. Compared with the oracle on the same
seeded inputs (t/h/w pair allocation of ``workloads.SPLIT_ROPE``)."""
import numpy as np
import pytest
import torch

import latent_kv_attention_cache_amd as vm
from gpu_cases import Run, compare
from workloads import config, custom, split_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    vm.load_library()


def _np(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy()


def _explicit(r, w):
    w_kv = vm.vmla_pack_kv_weights(r.dw["w_k_up"], r.dw["w_v_up"], dims=r.dims)
    x = r.x_dev(range(w.t_first, w.t_first + w.chunk_frames))
    n_valid = r.cache.n_valid_frames(w.t_first, w.chunk_frames)
    return vm.vmla_chunk_attention_explicit(r.cache, x, r.dw["w_q"], w_kv, w.t_first, w.chunk_frames,
                                            n_valid, dims=r.dims)


@pytest.mark.parametrize("d_rope", [16, 64, 96])
def test_split_small_full_outputs(d_rope):
    # 4x6 grid, 3-frame window, 2-frame chunk at t = 3 (the ring has wrapped),
    # B = 2, NaN-filled ring: the appended rows and every output, both routes
    print(f"[case] split {128 - d_rope}/{d_rope} small", flush=True)
    w = split_variant(custom(4, 6, window_frames=3, chunk_frames=2, t_first=3, batch=2), d_rope)
    r = Run(w, fill=float("nan"))
    got = _np(r.chunk_step())
    gx = _np(_explicit(r, w))
    for b in range(2):
        ref = r.reference(b)
        compare(r.cache_rows(3, 2, b), r.append_reference(3, 2, b), f"split {d_rope} rows b={b}")
        compare(got[b], ref, f"split {d_rope} latent b={b}", per_head_axis=1)
        compare(gx[b], ref, f"split {d_rope} explicit b={b}", per_head_axis=1)


@pytest.mark.parametrize("d_rope", [16, 96])
def test_split_ragged_units_and_tiles(d_rope):
    # 7x9 grid: 63 tokens per frame, 2-frame chunk = 126 queries (a partial
    # 32-query unit), 4 frames = 252 keys (a ragged last key tile)
    print(f"[case] split {128 - d_rope}/{d_rope} ragged", flush=True)
    w = split_variant(custom(7, 9, window_frames=4, chunk_frames=2, t_first=5, batch=1), d_rope)
    r = Run(w)
    got = _np(r.chunk_step())
    compare(got[0], r.reference(0), f"split {d_rope} ragged latent", per_head_axis=1)


@pytest.mark.parametrize("d_rope", [16, 64, 96])
def test_split_wan_shape_sampled_rows(d_rope):
    # the Wan-1.3B chunk-layer geometry (30x52 grid, 21-frame window, 3-frame
    # chunk at t = 18) with the split variant; sampled rows against the oracle
    print(f"[case] split {128 - d_rope}/{d_rope} Wan shape", flush=True)
    w = split_variant(config(2), d_rope)
    r = Run(w)
    got = _np(r.chunk_step())
    rng = np.random.default_rng(11 + d_rope)
    idx = np.unique(np.concatenate([[0, 255, 256, w.n_q - 1], rng.choice(w.n_q, 28, replace=False)]))
    ref = r.reference(query_tokens=idx)
    compare(got[0, idx], ref, f"split {d_rope} Wan latent, {len(idx)} rows", per_head_axis=1)
    compare(_np(_explicit(r, w))[0, idx], ref, f"split {d_rope} Wan explicit", per_head_axis=1)
    compare(r.cache_rows(18, 3), r.append_reference(18, 3), f"split {d_rope} Wan chunk rows")


@pytest.mark.parametrize("d_rope", [16, 64, 96])
def test_split_query_prologue_tall_tiles(d_rope):
    # 12 x 930 query rows: the query prologue runs its 256-row tiles with the
    # split variant's NoPE/RoPE widths; sampled rows of the first and the last
    # batch element
    print(f"[case] split {128 - d_rope}/{d_rope} tall prologue tiles", flush=True)
    w = split_variant(custom(30, 31, window_frames=2, chunk_frames=1, t_first=1, batch=12), d_rope)
    r = Run(w)
    got = _np(r.chunk_step())
    rng = np.random.default_rng(90 + d_rope)
    for b in (0, 11):
        idx = np.unique(np.concatenate([[0, 255, 256, w.n_q - 1], rng.choice(w.n_q, 28, replace=False)]))
        compare(got[b, idx], r.reference(b=b, query_tokens=idx), f"split {d_rope} tall tiles b={b}",
                per_head_axis=1)
