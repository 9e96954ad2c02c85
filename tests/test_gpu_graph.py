"""The hot path under HIP-graph capture: the entry points launch kernels only
(no allocation, no memset, no host synchronisation), so a chunk step captured
once replays like the eager calls. Each replay is checked bit for bit against
the eager result, with eager work and synchronisations between the replays."""
import pytest
import torch

import latent_kv_attention_cache_amd as vm
from gpu_cases import Run
from workloads import custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    vm.load_library()


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def test_chunk_step_replays_bitwise():
    w = custom(8, 13, window_frames=3, chunk_frames=2, t_first=4, batch=2)
    r = Run(w)
    r.fill_window()
    x = r.x_dev(range(4, 6))
    n_q = 2 * w.tokens_per_frame
    ws = torch.empty(vm.vmla_attention_workspace_bytes(2, n_q, r.dims), dtype=torch.uint8, device="cuda")
    out = torch.empty((2, n_q, w.n_heads, w.d_v), dtype=torch.bfloat16, device="cuda")

    def step():
        vm.vmla_cache_append(r.cache, x, r.dw["w_down"], r.dw["w_kr"], 4, 2, dims=r.dims)
        vm.vmla_chunk_attention(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"], 4, 2, 3,
                                out=out, workspace=ws, dims=r.dims)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    cache_eager = r.cache.data.clone()
    g = _capture(step)
    other = Run(custom(4, 6, window_frames=3, chunk_frames=1, t_first=2))
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        assert torch.equal(r.cache.data, cache_eager), f"replay {i} cache"
        other.chunk_step()                    # unrelated eager work between replays
        torch.cuda.synchronize()


def test_whole_layer_replays_bitwise():
    w = custom(4, 6, window_frames=3, chunk_frames=2, t_first=3).with_(sink_frames=1, rope_at_read=True)
    r = Run(w)
    r.fill_window()
    r.append(3, 2)
    r._mixer()
    x = r.x_dev(range(3, 5))
    n_q = 2 * w.tokens_per_frame
    ws = torch.empty(vm.vmla_layer_workspace_bytes(1, n_q, w.d_q, r.dims), dtype=torch.uint8, device="cuda")
    out = torch.empty((1, n_q, w.d_model), dtype=torch.bfloat16, device="cuda")
    n_valid = r.cache.n_valid_frames(3, 2)

    def step():
        vm.vmla_chunk_attention_layer(r.cache, x, r.dmix["w_dq"], r.w_qa, r.w_vo, 3, 2, n_valid,
                                      out=out, workspace=ws, dims=r.dims)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = _capture(step)
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        step()                                # the eager call again between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def _replay_check(step, out):
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = _capture(step)
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        step()                                # the eager call again between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


@pytest.mark.parametrize("route", ["latent", "explicit"])
def test_chunk_causal_clip_replays_bitwise(route):
    # the whole-clip form under the chunk-causal mask (7 frames, chunks of 3, window 5)
    w = custom(4, 6, window_frames=7, chunk_frames=3, t_first=0, batch=2)
    r = Run(w)
    r.append(0, 3)
    r.append(3, 3)
    r.append(6, 1)
    x = r.x_dev(range(7))
    n_q = 7 * w.tokens_per_frame
    out = torch.empty((2, n_q, w.n_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    if route == "latent":
        ws = torch.empty(vm.vmla_attention_workspace_bytes(2, n_q, r.dims), dtype=torch.uint8, device="cuda")

        def step():
            vm.vmla_chunk_causal_attention(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"], 7, 3, 5,
                                           out=out, workspace=ws, dims=r.dims)
    else:
        w_kv = vm.vmla_pack_kv_weights(r.dw["w_k_up"], r.dw["w_v_up"], dims=r.dims)
        ws = torch.empty(vm.vmla_explicit_workspace_bytes(2, n_q, n_q, r.dims), dtype=torch.uint8,
                         device="cuda")

        def step():
            vm.vmla_chunk_causal_attention_explicit(r.cache, x, r.dw["w_q"], w_kv, 7, 3, 5, out=out,
                                                    workspace=ws, dims=r.dims)
    _replay_check(step, out)


@pytest.mark.parametrize("kind", ["split 32/96", "d_c 512"])
def test_variant_chunk_step_replays_bitwise(kind):
    from workloads import split_variant
    base = custom(4, 6, window_frames=3, chunk_frames=2, t_first=4, batch=2)
    w = split_variant(base, 96) if kind.startswith("split") else base.with_(d_c=512)
    r = Run(w)
    r.fill_window()
    x = r.x_dev(range(4, 6))
    n_q = 2 * w.tokens_per_frame
    ws = torch.empty(vm.vmla_attention_workspace_bytes(2, n_q, r.dims), dtype=torch.uint8, device="cuda")
    out = torch.empty((2, n_q, w.n_heads, w.d_v), dtype=torch.bfloat16, device="cuda")

    def step():
        vm.vmla_cache_append(r.cache, x, r.dw["w_down"], r.dw["w_kr"], 4, 2, dims=r.dims)
        vm.vmla_chunk_attention(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"], 4, 2, 3,
                                out=out, workspace=ws, dims=r.dims)
    _replay_check(step, out)
