"""GPU check of vmla_chunk_attention_noalloc, the attention entry point that
allocates nothing: its query rows live in the library's own scratch array
instead of a caller's workspace. It runs the same kernels as
vmla_chunk_attention, so on the same inputs the two outputs must agree bit
for bit; two calls in a row, the second with a smaller input (the array still
holds the first call's rows), and the small one also against the oracle."""
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


def _both(r):
    """The chunk's attention through both entry points on the same inputs."""
    w = r.w
    x = r.x_dev(range(w.t_first, w.t_first + w.chunk_frames))
    n_valid = r.cache.n_valid_frames(w.t_first, w.chunk_frames)
    ref = vm.vmla_chunk_attention(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"], w.t_first,
                                  w.chunk_frames, n_valid, dims=r.dims)
    out = torch.full_like(ref, float("nan"))
    vm.vmla_chunk_attention_noalloc(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"], w.t_first,
                                    w.chunk_frames, n_valid, out, dims=r.dims)
    return _np(out), _np(ref)


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    # 1) the Wan-1.3B chunk: B = 1, 4680 queries over 32,760 keys, 25.2 MB of
    #    the 32 MiB array; seeded weights, device-noise activations
    print("[case] noalloc: Wan-1.3B chunk, B=1", flush=True)
    w = config(2)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)

    def noise(t, b):
        return torch.randn((w.tokens_per_frame, w.d_model), generator=gen, device="cuda").to(torch.bfloat16)

    r = Run(w, batch_x=noise)
    r.fill_window()
    r.append(w.t_first, w.chunk_frames)
    got, ref = _both(r)
    assert np.array_equal(got, ref), "noalloc differs from vmla_chunk_attention (Wan chunk)"
    compare(got[0], ref[0], "noalloc vs workspace, Wan chunk", per_head_axis=1)
    del r
    # 2) a smaller call right after: 4x6 grid, B = 2, 2-frame chunk after a ring wrap
    print("[case] noalloc: 4x6 grid, B=2, second call", flush=True)
    w2 = custom(4, 6, window_frames=3, chunk_frames=2, t_first=3, batch=2)
    r2 = Run(w2, fill=float("nan"))
    r2.fill_window()
    r2.append(w2.t_first, w2.chunk_frames)
    got2, ref2 = _both(r2)
    assert np.array_equal(got2, ref2), "noalloc differs from vmla_chunk_attention (second call)"
    for b in range(2):
        compare(got2[b], r2.reference(b=b), f"noalloc second call vs oracle, b={b}", per_head_axis=1)


def test_noalloc_rejects_a_chunk_beyond_the_array():
    # B = 2 at 4680 queries needs 50.3 MB of query rows: refused before any launch
    w = config(2).with_(batch=2, window_frames=3, t_first=0)
    r = Run(w)
    x = torch.zeros((2, w.n_q, w.d_model), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((2, w.n_q, w.n_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vm.VmlaError) as e:
        vm.vmla_chunk_attention_noalloc(r.cache, x, r.dw["w_q"], r.dw["w_k_up"], r.dw["w_v_up"], 0, 3, 3, out,
                                        dims=r.dims)
    assert e.value.status == vm.VMLA_ERR_WORKSPACE
