"""GPU parity of the whole-clip form under the chunk-causal block mask
([PL] App. D.4 "Chunk-Causal Sliding-Window Attention"; [PL] §3 "Integration
with causal attention"): every token of a clip attends to its own chunk and to
the earlier frames of a window, never to a later chunk. The latent route and
the explicit-reconstruction route are both compared with the oracle's
clip_chunk_causal_reference on the same seeded inputs."""
import numpy as np
import pytest
import torch

import latent_kv_attention_cache_amd as vm
import oracle.vmla_oracle as orc
from gpu_cases import Run, compare
from workloads import custom

pytestmark = pytest.mark.gpu


def _np(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy()


def _clip_run(w, n_frames):
    """A run whose cache holds exactly the clip's frames 0 .. n_frames - 1 at
    slots t T + n (appended in pieces of at most one chunk)."""
    r = Run(w.with_(window_frames=n_frames))
    for t0 in range(0, n_frames, w.chunk_frames):
        r.append(t0, min(w.chunk_frames, n_frames - t0))
    return r, r.x_dev(range(n_frames))


def _reference(r, n_frames, window, b=0, query_tokens=None):
    return orc.clip_chunk_causal_reference(r.w, r.wts, lambda t: r.x_host(t, b), n_frames, window,
                                           query_tokens)


# (grid_h, grid_w, frames, chunk frames, mask window, batch, dtype)
CASES = [
    (4, 6, 7, 3, 5, 2, "bf16"),    # T = 24: 72-query chunks (ragged units), a 1-frame last chunk
    (4, 6, 7, 3, 7, 1, "f32"),     # window = clip: the plain block-causal mask
    (3, 5, 6, 1, 6, 1, "bf16"),    # one-frame chunks: frame-causal
    (4, 6, 5, 5, 5, 1, "bf16"),    # one chunk: plain attention over the clip
    (8, 12, 8, 2, 3, 1, "bf16"),   # T = 96: key ranges start inside a 64-key tile
]


@pytest.mark.parametrize("gh,gw,F,C,W,B,dt", CASES)
def test_chunk_causal_latent_small(gh, gw, F, C, W, B, dt):
    print(f"[case] latent chunk-causal grid {gh}x{gw} F={F} C={C} W={W} B={B} {dt}", flush=True)
    w = custom(gh, gw, window_frames=F, chunk_frames=C, t_first=0, batch=B, dtype=dt)
    r, x = _clip_run(w, F)
    out = vm.vmla_chunk_causal_attention(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"],
                                         F, C, W, dims=r.dims)
    got = _np(out)
    for b in range(B):
        compare(got[b], _reference(r, F, W, b), f"latent clip F={F} C={C} W={W} b={b}", per_head_axis=1)


@pytest.mark.parametrize("d_c", [64, 128])
@pytest.mark.parametrize("gh,gw,F,C,W,B,dt", [CASES[0], CASES[4]])
def test_chunk_causal_latent_narrow_latents(d_c, gh, gw, F, C, W, B, dt):
    # the latent route at d_c 64 (two 64-key sub-tiles per step) and 128
    print(f"[case] latent chunk-causal d_c={d_c} grid {gh}x{gw} F={F} C={C} W={W} B={B} {dt}", flush=True)
    w = custom(gh, gw, window_frames=F, chunk_frames=C, t_first=0, batch=B, dtype=dt).with_(d_c=d_c)
    r, x = _clip_run(w, F)
    out = vm.vmla_chunk_causal_attention(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"],
                                         F, C, W, dims=r.dims)
    got = _np(out)
    for b in range(B):
        compare(got[b], _reference(r, F, W, b), f"latent clip d_c={d_c} F={F} C={C} W={W} b={b}",
                per_head_axis=1)


@pytest.mark.parametrize("gh,gw,F,C,W,B,dt", CASES)
def test_chunk_causal_explicit_small(gh, gw, F, C, W, B, dt):
    print(f"[case] explicit chunk-causal grid {gh}x{gw} F={F} C={C} W={W} B={B} {dt}", flush=True)
    w = custom(gh, gw, window_frames=F, chunk_frames=C, t_first=0, batch=B, dtype=dt)
    r, x = _clip_run(w, F)
    w_kv = vm.vmla_pack_kv_weights(r.dw["w_k_up"], r.dw["w_v_up"], dims=r.dims)
    out = vm.vmla_chunk_causal_attention_explicit(r.cache, x, r.dw["w_q"], w_kv, F, C, W, dims=r.dims)
    got = _np(out)
    for b in range(B):
        compare(got[b], _reference(r, F, W, b), f"explicit clip F={F} C={C} W={W} b={b}",
                per_head_axis=1)


def test_chunk_causal_stages_equal_the_whole_call():
    # vmla_query_prologue (t_first = 0, the whole clip) + the attention stage is
    # the same launch sequence as vmla_chunk_causal_attention: equal bit for bit.
    print("[case] chunk-causal two stages vs one call", flush=True)
    F, C, W = 7, 3, 5
    w = custom(4, 6, window_frames=F, chunk_frames=C, t_first=0, batch=2)
    r, x = _clip_run(w, F)
    whole = vm.vmla_chunk_causal_attention(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"],
                                           F, C, W, dims=r.dims)
    n_q = F * w.tokens_per_frame
    ws = torch.empty(vm.vmla_attention_workspace_bytes(2, n_q, r.dims), dtype=torch.uint8, device="cuda")
    vm.vmla_query_prologue(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], 0, F, F, ws, dims=r.dims)
    out = torch.empty_like(whole)
    vm.vmla_chunk_causal_latent_attention(r.cache, r.dw["w_v_up"], F, C, W, out, ws, dims=r.dims)
    torch.cuda.synchronize()
    assert torch.equal(out, whole)


def _sample_rows(n_frames, C, T, per_chunk, seed):
    # query tokens spread over the first, a middle and the last chunk, each
    # chunk's first and last token included
    rng = np.random.default_rng(seed)
    n_chunks = -(-n_frames // C)
    rows = []
    for c in sorted({0, n_chunks // 2, n_chunks - 1}):
        lo, hi = c * C * T, min((c + 1) * C, n_frames) * T
        rows += [lo, hi - 1] + list(rng.integers(lo, hi, per_chunk - 2))
    return np.array(sorted(set(rows)))


@pytest.mark.parametrize("route", ["latent", "explicit"])
def test_chunk_causal_full_clip_sampled(route):
    # The Wan-1.3B clip at full size: 21 latent frames of 30 x 52 tokens in
    # 3-frame chunks under a 21-frame window (the block-causal mask), B = 1;
    # sampled query rows against the oracle.
    print(f"[case] full clip chunk-causal {route}", flush=True)
    F, C, W = 21, 3, 21
    w = custom(30, 52, window_frames=F, chunk_frames=C, t_first=0, batch=1)
    r, x = _clip_run(w, F)
    if route == "latent":
        out = vm.vmla_chunk_causal_attention(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"],
                                             F, C, W, dims=r.dims)
    else:
        w_kv = vm.vmla_pack_kv_weights(r.dw["w_k_up"], r.dw["w_v_up"], dims=r.dims)
        out = vm.vmla_chunk_causal_attention_explicit(r.cache, x, r.dw["w_q"], w_kv, F, C, W,
                                                      dims=r.dims)
    rows = _sample_rows(F, C, w.tokens_per_frame, 24, seed=7)
    got = _np(out)[0, rows]
    compare(got, _reference(r, F, W, 0, rows), f"full clip {route}, {len(rows)} sampled rows",
            per_head_axis=1)
