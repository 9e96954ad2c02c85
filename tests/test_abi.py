"""C-ABI checks that need no GPU: the library loads, exports every function that
include/vmla.h declares, and rejects bad arguments on the host, before any HIP
call, with the documented status codes."""
import ctypes
import os
import re

import pytest

import latent_kv_attention_cache_amd as vm
from latent_kv_attention_cache_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vmla.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vmla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return vm.load_library()


def test_library_exports_every_declared_function(lib):
    names = _declared_functions()
    assert set(names) == set(vm.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.vmla_abi_version() == 9
    for code in range(-8, 1):
        s = vm.vmla_status_string(code)
        assert s and s != "unknown status"
    assert vm.vmla_status_string(-99) == "unknown status"


def test_default_dims_are_wan_videomla(lib):
    d = vm.default_dims()
    assert (d.d_model, d.n_heads, d.d_nope, d.d_rope, d.d_c, d.d_v) == (1536, 12, 96, 32, 192, 128)
    assert list(d.rope_pairs) == [6, 5, 5] and list(d.rope_axis_dims) == [12, 10, 10]
    assert d.rope_theta == 10000.0
    assert abs(d.scale - 128 ** -0.5) < 1e-7


def test_workspace_bytes(lib):
    d = vm.default_dims()
    assert vm.vmla_attention_workspace_bytes(1, 4680, d) == 12 * 4680 * 224 * 2
    assert vm.vmla_attention_workspace_bytes(0, 4680, d) == 0
    bad = vm.default_dims(d_c=96)
    assert vm.vmla_attention_workspace_bytes(1, 10, bad) == 0
    # the latent-budget sweep widths: rows of d_c + 32
    assert vm.vmla_attention_workspace_bytes(1, 10, vm.default_dims(d_c=64)) == 12 * 10 * 96 * 2
    assert vm.vmla_attention_workspace_bytes(1, 10, vm.default_dims(d_c=128)) == 12 * 10 * 160 * 2


# Fake, never-dereferenced device addresses: validation must fail before any use.
A = 0x10000
B = 0x20000
C = 0x30000
MIS = 0x30008   # 8-byte aligned only


def _cache(**kw):
    c = dict(data=A, dtype=vm.VMLA_BF16, batch=1, window_frames=3, grid_h=4, grid_w=6)
    c.update(kw)
    return bd.vmla_cache(**c)


def _append(lib, dims=None, cache=None, dtype=vm.VMLA_BF16, x=B, wd=C, wk=A, t_first=0, n_frames=1):
    d = dims if dims is not None else vm.default_dims()
    cs = cache if cache is not None else _cache()
    return lib.vmla_cache_append(ctypes.byref(d), ctypes.byref(cs), dtype, x, wd, wk, t_first,
                                 n_frames, None)


def _attn(lib, dims=None, cache=None, dtype=vm.VMLA_BF16, t_first=2, n_frames=1, n_valid=3,
          ws_bytes=None, ws=B, out=C, x=A):
    d = dims if dims is not None else vm.default_dims()
    cs = cache if cache is not None else _cache()
    if ws_bytes is None:
        ws_bytes = vm.vmla_attention_workspace_bytes(cs.batch, n_frames * cs.grid_h * cs.grid_w, d)
    return lib.vmla_chunk_attention(ctypes.byref(d), ctypes.byref(cs), dtype, x, B, C, A, t_first,
                                    n_frames, n_valid, out, ws, ws_bytes, None)


def test_append_validation(lib):
    assert _append(lib, x=None) == vm.VMLA_ERR_NULL
    assert _append(lib, wd=None) == vm.VMLA_ERR_NULL
    assert _append(lib, cache=_cache(data=None)) == vm.VMLA_ERR_NULL
    assert lib.vmla_cache_append(None, None, 1, A, B, C, 0, 1, None) == vm.VMLA_ERR_NULL
    assert _append(lib, x=MIS) == vm.VMLA_ERR_ALIGN
    assert _append(lib, cache=_cache(data=MIS)) == vm.VMLA_ERR_ALIGN
    assert _append(lib, dtype=7) == vm.VMLA_ERR_DTYPE
    assert _append(lib, dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE          # cache is bf16
    assert _append(lib, dims=vm.default_dims(d_c=96)) == vm.VMLA_ERR_SHAPE   # not 64 / 128 / 192 / 256 / 512
    assert _append(lib, dims=vm.default_dims(d_c=384)) == vm.VMLA_ERR_SHAPE
    assert _append(lib, dims=vm.default_dims(d_model=100)) == vm.VMLA_ERR_SHAPE
    assert _append(lib, dims=vm.default_dims(rope_pairs=(6, 5, 4))) == vm.VMLA_ERR_SHAPE
    assert _append(lib, dims=vm.default_dims(n_heads=0)) == vm.VMLA_ERR_SHAPE
    assert _append(lib, cache=_cache(grid_w=0)) == vm.VMLA_ERR_SHAPE
    assert _append(lib, cache=_cache(batch=0)) == vm.VMLA_ERR_SHAPE
    assert _append(lib, t_first=-1) == vm.VMLA_ERR_RANGE
    assert _append(lib, n_frames=0) == vm.VMLA_ERR_RANGE
    assert _append(lib, n_frames=4) == vm.VMLA_ERR_RANGE                 # > window_frames
    assert _append(lib, t_first=(1 << 20) - 1, n_frames=2) == vm.VMLA_ERR_RANGE   # t_end > 2^20


def test_attention_validation(lib):
    assert _attn(lib, x=None) == vm.VMLA_ERR_NULL
    assert _attn(lib, out=None) == vm.VMLA_ERR_NULL
    assert _attn(lib, out=MIS) == vm.VMLA_ERR_ALIGN
    assert _attn(lib, dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
    assert _attn(lib, dims=vm.default_dims(d_v=64)) == vm.VMLA_ERR_SHAPE
    assert _attn(lib, t_first=-1) == vm.VMLA_ERR_RANGE
    assert _attn(lib, n_frames=4, n_valid=3) == vm.VMLA_ERR_RANGE
    assert _attn(lib, n_valid=2) == vm.VMLA_ERR_RANGE                     # must be min(t_end, W) = 3
    assert _attn(lib, t_first=0, n_frames=1, n_valid=3) == vm.VMLA_ERR_RANGE   # only 1 frame written
    assert _attn(lib, t_first=10, n_frames=1, n_valid=4) == vm.VMLA_ERR_RANGE  # > window
    assert _attn(lib, ws=None) == vm.VMLA_ERR_WORKSPACE
    assert _attn(lib, ws_bytes=10) == vm.VMLA_ERR_WORKSPACE
    assert _attn(lib, ws=MIS) == vm.VMLA_ERR_ALIGN


def test_cache_mode_validation(lib):
    # sink_frames in {0, 1}, rope_at_read in {0, 1}, and a sink only with read-time RoPE
    assert _append(lib, cache=_cache(sink_frames=2, rope_at_read=1)) == vm.VMLA_ERR_SHAPE
    assert _append(lib, cache=_cache(rope_at_read=2)) == vm.VMLA_ERR_SHAPE
    assert _append(lib, cache=_cache(sink_frames=1, rope_at_read=0)) == vm.VMLA_ERR_SHAPE
    assert _attn(lib, cache=_cache(sink_frames=1, rope_at_read=0)) == vm.VMLA_ERR_SHAPE
    sink = _cache(sink_frames=1, rope_at_read=1)
    # valid frames = min(t_first + n_frames, sink + W): 4 once the ring is full
    assert _attn(lib, cache=sink, t_first=10, n_frames=1, n_valid=3) == vm.VMLA_ERR_RANGE
    assert _attn(lib, cache=sink, t_first=10, n_frames=1, n_valid=5) == vm.VMLA_ERR_RANGE
    assert _attn(lib, cache=sink, t_first=0, n_frames=2, n_valid=3) == vm.VMLA_ERR_RANGE
    assert _append(lib, cache=sink, n_frames=4) == vm.VMLA_ERR_RANGE   # > window_frames


def _layer(lib, dims=None, cache=None, dtype=vm.VMLA_BF16, d_q=768, t_first=2, n_frames=1, n_valid=3,
           ws_bytes=None, ws=B, out=C, x=A, w_dq=B, w_qa=C, w_vo=A):
    d = dims if dims is not None else vm.default_dims()
    cs = cache if cache is not None else _cache()
    if ws_bytes is None:
        ws_bytes = lib.vmla_layer_workspace_bytes(ctypes.byref(d), 768, cs.batch,
                                                  n_frames * cs.grid_h * cs.grid_w)
    return lib.vmla_chunk_attention_layer(ctypes.byref(d), ctypes.byref(cs), dtype, x, w_dq, d_q, w_qa,
                                          w_vo, t_first, n_frames, n_valid, out, ws, ws_bytes, None)


def test_layer_workspace_bytes(lib):
    d = vm.default_dims()
    qhat = 12 * 4680 * 224 * 2
    inner = 4680 * max(768, 12 * 192) * 2
    assert vm.vmla_layer_workspace_bytes(1, 4680, 768, d) == qhat + (inner + 255) // 256 * 256
    assert vm.vmla_layer_workspace_bytes(2, 24, 4096, d) == 2 * 12 * 24 * 224 * 2 + 2 * 24 * 4096 * 2
    assert vm.vmla_layer_workspace_bytes(1, 4680, 700, d) == 0        # d_q not a multiple of 64
    assert vm.vmla_layer_workspace_bytes(1, 4680, 0, d) == 0
    assert vm.vmla_layer_workspace_bytes(0, 4680, 768, d) == 0


def test_layer_validation(lib):
    d = vm.default_dims()
    assert _layer(lib, x=None) == vm.VMLA_ERR_NULL
    assert _layer(lib, w_qa=None) == vm.VMLA_ERR_NULL
    assert _layer(lib, w_vo=None) == vm.VMLA_ERR_NULL
    assert _layer(lib, w_vo=MIS) == vm.VMLA_ERR_ALIGN
    assert _layer(lib, d_q=100) == vm.VMLA_ERR_SHAPE
    assert _layer(lib, d_q=16384) == vm.VMLA_ERR_SHAPE
    assert _layer(lib, dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
    assert _layer(lib, n_valid=2) == vm.VMLA_ERR_RANGE
    assert _layer(lib, ws=None) == vm.VMLA_ERR_WORKSPACE
    # the attention-only workspace is too small for the layer
    small = vm.vmla_attention_workspace_bytes(1, 24, d)
    assert _layer(lib, ws_bytes=small) == vm.VMLA_ERR_WORKSPACE
    cs = _cache()
    assert lib.vmla_layer_attention(ctypes.byref(d), ctypes.byref(cs), vm.VMLA_BF16, 768, None, 2, 1, 3,
                                    C, B, 1 << 20, None) == vm.VMLA_ERR_NULL
    assert lib.vmla_layer_query_prologue(ctypes.byref(d), ctypes.byref(cs), vm.VMLA_BF16, A, B, 768, C,
                                         2, 1, 3, B, 16, None) == vm.VMLA_ERR_WORKSPACE
    assert lib.vmla_fold_query_weights(ctypes.byref(d), vm.VMLA_BF16, 100, A, B, C, None) == vm.VMLA_ERR_SHAPE
    assert lib.vmla_fold_query_weights(ctypes.byref(d), 5, 768, A, B, C, None) == vm.VMLA_ERR_DTYPE
    assert lib.vmla_fold_query_weights(ctypes.byref(d), vm.VMLA_BF16, 768, None, B, C, None) == vm.VMLA_ERR_NULL
    assert lib.vmla_fold_output_weights(ctypes.byref(d), vm.VMLA_BF16, A, MIS, C, None) == vm.VMLA_ERR_ALIGN
    assert lib.vmla_fold_output_weights(ctypes.byref(vm.default_dims(d_v=64)), vm.VMLA_BF16, A, B, C,
                                        None) == vm.VMLA_ERR_SHAPE
    assert lib.vmla_output_projection(ctypes.byref(d), vm.VMLA_BF16, 0, A, B, C, None) == vm.VMLA_ERR_SHAPE
    assert lib.vmla_output_projection(ctypes.byref(d), vm.VMLA_BF16, 1 << 25, A, B, C, None) == vm.VMLA_ERR_SHAPE
    assert lib.vmla_output_projection(ctypes.byref(d), vm.VMLA_BF16, 8, None, B, C, None) == vm.VMLA_ERR_NULL
    assert lib.vmla_output_projection(ctypes.byref(d), 3, 8, A, B, C, None) == vm.VMLA_ERR_DTYPE


def test_latent_budget_widths_only_on_the_core_path(lib):
    # d_c 64 / 128 are accepted by the append and the attention core; the whole
    # layer, the explicit route and the weight folds run at d_c = 192 only
    d64 = vm.default_dims(d_c=64)
    assert lib.vmla_layer_workspace_bytes(ctypes.byref(d64), 768, 1, 24) == 0
    assert lib.vmla_explicit_workspace_bytes(ctypes.byref(d64), 1, 24, 72) == 0
    assert lib.vmla_fold_query_weights(ctypes.byref(d64), vm.VMLA_BF16, 768, A, B, C, None) == vm.VMLA_ERR_SHAPE
    assert lib.vmla_pack_kv_weights(ctypes.byref(d64), vm.VMLA_BF16, A, B, C, None) == vm.VMLA_ERR_SHAPE
    assert _attn(lib, dims=d64, ws=None) == vm.VMLA_ERR_WORKSPACE        # validation passed up to the workspace


def test_explicit_validation(lib):
    d = vm.default_dims()
    assert vm.vmla_explicit_workspace_bytes(1, 4680, 32760, d) == 12 * 2 * (4680 * 128 + 32760 * 256)
    assert vm.vmla_explicit_workspace_bytes(1, 4680, 0, d) == 0
    cs = _cache()
    big = 1 << 30

    def call(cache=cs, dtype=vm.VMLA_BF16, x=A, wq=B, wkv=C, n_valid=3, ws=B, ws_bytes=big, out=C):
        return lib.vmla_chunk_attention_explicit(ctypes.byref(d), ctypes.byref(cache), dtype, x, wq, wkv,
                                                 2, 1, n_valid, out, ws, ws_bytes, None)
    assert call(wkv=None) == vm.VMLA_ERR_NULL
    assert call(dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
    assert call(n_valid=2) == vm.VMLA_ERR_RANGE
    assert call(cache=_cache(rope_at_read=1)) == vm.VMLA_ERR_SHAPE       # read-time RoPE not supported
    assert call(ws_bytes=1024) == vm.VMLA_ERR_WORKSPACE
    assert call(ws=None) == vm.VMLA_ERR_WORKSPACE
    assert call(wkv=MIS) == vm.VMLA_ERR_ALIGN
    assert lib.vmla_pack_kv_weights(ctypes.byref(d), vm.VMLA_BF16, A, None, C, None) == vm.VMLA_ERR_NULL
    assert lib.vmla_pack_kv_weights(ctypes.byref(d), 9, A, B, C, None) == vm.VMLA_ERR_DTYPE
    assert lib.vmla_pack_kv_weights(ctypes.byref(d), vm.VMLA_BF16, A, B, MIS, None) == vm.VMLA_ERR_ALIGN


def test_chunk_causal_validation(lib):
    d = vm.default_dims()
    clip = _cache(window_frames=7)
    need = vm.vmla_attention_workspace_bytes(1, 7 * 24, d)

    def call(dims=d, cache=clip, dtype=vm.VMLA_BF16, x=A, out=C, n_frames=7, chunk=3, win=5,
             ws=B, ws_bytes=need):
        return lib.vmla_chunk_causal_attention(ctypes.byref(dims), ctypes.byref(cache), dtype, x, B, C,
                                               A, n_frames, chunk, win, out, ws, ws_bytes, None)
    assert call(x=None) == vm.VMLA_ERR_NULL
    assert call(out=None) == vm.VMLA_ERR_NULL
    assert call(dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
    assert call(cache=_cache(window_frames=7, rope_at_read=1)) == vm.VMLA_ERR_SHAPE
    assert call(cache=_cache(window_frames=7, sink_frames=1, rope_at_read=1)) == vm.VMLA_ERR_SHAPE
    assert call(cache=_cache(window_frames=7, batch=40000)) == vm.VMLA_ERR_SHAPE   # 120,000 grid z
    assert call(n_frames=0) == vm.VMLA_ERR_RANGE
    assert call(n_frames=8) == vm.VMLA_ERR_RANGE                          # > the cache's frames
    assert call(chunk=0) == vm.VMLA_ERR_RANGE
    assert call(n_frames=2, chunk=3) == vm.VMLA_ERR_RANGE                 # chunk longer than the clip
    assert call(win=2) == vm.VMLA_ERR_RANGE                               # window shorter than a chunk
    assert call(ws=None) == vm.VMLA_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == vm.VMLA_ERR_WORKSPACE
    assert call(ws=MIS) == vm.VMLA_ERR_ALIGN
    assert call(out=MIS) == vm.VMLA_ERR_ALIGN
    d64 = vm.default_dims(d_c=64)
    assert call(dims=d64, ws=None) == vm.VMLA_ERR_WORKSPACE               # passed up to the workspace
    # the attention stage alone
    st = lib.vmla_chunk_causal_latent_attention(ctypes.byref(d), ctypes.byref(clip), vm.VMLA_BF16, A,
                                                7, 3, 5, None, B, need, None)
    assert st == vm.VMLA_ERR_NULL
    st = lib.vmla_chunk_causal_latent_attention(ctypes.byref(d), ctypes.byref(clip), vm.VMLA_BF16, A,
                                                7, 3, 5, C, B, 100, None)
    assert st == vm.VMLA_ERR_WORKSPACE
    # explicit form: d_c = 192 only, its own workspace size
    big = vm.vmla_explicit_workspace_bytes(1, 7 * 24, 7 * 24, d)
    assert big == 12 * 2 * (168 * 128 + 168 * 256)

    def xcall(dims=d, ws_bytes=big, wkv=C):
        return lib.vmla_chunk_causal_attention_explicit(ctypes.byref(dims), ctypes.byref(clip),
                                                        vm.VMLA_BF16, A, B, wkv, 7, 3, 5, C, B,
                                                        ws_bytes, None)
    assert xcall(wkv=None) == vm.VMLA_ERR_NULL
    assert xcall(dims=d64) == vm.VMLA_ERR_SHAPE
    assert xcall(ws_bytes=need) == vm.VMLA_ERR_WORKSPACE
    assert xcall(wkv=MIS) == vm.VMLA_ERR_ALIGN


def test_split_variant_validation(lib):
    # NoPE/RoPE split variants: d_rope 16 / 64 / 96 at d_c = 192, bf16, k_R
    # rotated at append, the attention core and the explicit route only
    def split(d_rope, **kw):
        pairs = {16: (3, 3, 2), 64: (12, 10, 10), 96: (18, 15, 15)}[d_rope]
        f = dict(d_nope=128 - d_rope, d_rope=d_rope, rope_pairs=pairs,
                 rope_axis_dims=tuple(2 * p for p in pairs))
        f.update(kw)
        return vm.default_dims(**f)
    for dr in (16, 64, 96):
        d = split(dr)
        cache = _cache(window_frames=3)
        assert vm.vmla_attention_workspace_bytes(1, 24, d) == 12 * 24 * (192 + dr) * 2
        assert _attn(lib, dims=d, cache=cache, ws=None) == vm.VMLA_ERR_WORKSPACE   # valid up to there
        assert _append(lib, dims=d, x=MIS) == vm.VMLA_ERR_ALIGN                      # valid up to there
        assert _attn(lib, dims=d, cache=_cache(dtype=vm.VMLA_F32), dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
        assert _append(lib, dims=d, cache=_cache(dtype=vm.VMLA_F32), dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
        assert _attn(lib, dims=d, cache=_cache(rope_at_read=1)) == vm.VMLA_ERR_SHAPE
        assert _append(lib, dims=split(dr, d_c=128)) == vm.VMLA_ERR_SHAPE      # splits run at d_c = 192
        assert vm.vmla_layer_workspace_bytes(1, 24, 768, d) == 0              # default split only
        assert lib.vmla_fold_query_weights(ctypes.byref(d), vm.VMLA_BF16, 768, A, B, C, None) == vm.VMLA_ERR_SHAPE
        assert vm.vmla_explicit_workspace_bytes(1, 24, 72, d) > 0              # the explicit route takes splits
        st = lib.vmla_chunk_causal_attention(ctypes.byref(d), ctypes.byref(_cache(window_frames=7)),
                                             vm.VMLA_BF16, A, B, C, A, 7, 3, 5, C, B, 1 << 30, None)
        assert st == vm.VMLA_ERR_SHAPE                                        # default split only
    # pair counts must sum to d_rope / 2; d_nope + d_rope must be 128; only the listed splits
    assert _append(lib, dims=split(64, rope_pairs=(6, 5, 5))) == vm.VMLA_ERR_SHAPE
    assert _append(lib, dims=vm.default_dims(d_nope=80, d_rope=48, rope_pairs=(9, 8, 7))) == vm.VMLA_ERR_SHAPE
    assert _append(lib, dims=vm.default_dims(d_nope=64, d_rope=32)) == vm.VMLA_ERR_SHAPE


def test_wide_latent_validation(lib):
    # d_c = 256 / 512 (the wide-latent kernel): bf16, k_R rotated at append,
    # the append and the attention core only
    for dc in (256, 512):
        d = vm.default_dims(d_c=dc)
        assert vm.vmla_attention_workspace_bytes(1, 24, d) == 12 * 24 * (dc + 32) * 2
        assert _attn(lib, dims=d, ws=None) == vm.VMLA_ERR_WORKSPACE              # valid up to there
        assert _append(lib, dims=d, x=MIS) == vm.VMLA_ERR_ALIGN                   # valid up to there
        assert _attn(lib, dims=d, cache=_cache(dtype=vm.VMLA_F32), dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
        assert _append(lib, dims=d, cache=_cache(dtype=vm.VMLA_F32), dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
        assert _attn(lib, dims=d, cache=_cache(rope_at_read=1)) == vm.VMLA_ERR_SHAPE
        assert vm.vmla_explicit_workspace_bytes(1, 24, 72, d) == 0
        assert vm.vmla_layer_workspace_bytes(1, 24, 768, d) == 0
        st = lib.vmla_chunk_causal_attention(ctypes.byref(d), ctypes.byref(_cache(window_frames=7)),
                                             vm.VMLA_BF16, A, B, C, A, 7, 3, 5, C, B, 1 << 30, None)
        assert st == vm.VMLA_ERR_SHAPE


# Widely spaced fake device addresses (16 GiB apart) for the aliasing checks:
# every call below is valid except for the one overlap it tests, which the
# host validation must reject before any launch.
def R(i):
    return (1 << 40) + i * (1 << 34)


def test_overlapping_buffers_are_rejected(lib):
    d = vm.default_dims()
    OV = vm.VMLA_ERR_OVERLAP
    cache = _cache(data=R(0))            # 1 x 72 slots x 224 bf16 = 32,256 bytes
    row = 224 * 2
    ws_need = vm.vmla_attention_workspace_bytes(1, 24, d)      # 12 x 24 x 224 x 2
    dr = ctypes.byref(d)
    cr = ctypes.byref(cache)

    # append: x, W_down or W_KR inside the cache it writes
    assert _append(lib, cache=cache, x=R(0) + 10 * row, wd=R(2), wk=R(3)) == OV
    assert _append(lib, cache=cache, x=R(1), wd=R(0) + 71 * row, wk=R(3)) == OV
    assert _append(lib, cache=cache, x=R(1), wd=R(2), wk=R(0) - 16) == OV    # W_KR ends inside slot 0

    def attn(x=R(1), wq=R(2), wku=R(3), wvu=R(4), out=R(5), ws=R(6)):
        return lib.vmla_chunk_attention(dr, cr, vm.VMLA_BF16, x, wq, wku, wvu, 2, 1, 3, out, ws,
                                        ws_need, None)
    assert attn(ws=R(0) + 32256 - 16) == OV            # workspace starts in the cache's last row
    assert attn(ws=R(0) - ws_need + 16) == OV          # workspace ends in the cache's first row
    assert attn(out=R(6) + ws_need - 16) == OV         # out starts in the workspace's tail
    assert attn(out=R(1)) == OV                        # out is x
    assert attn(ws=R(2) + 1536 * 1536 * 2 - 16) == OV  # workspace starts in W_Q's tail
    assert attn(wvu=R(5) + 16) == OV                   # out overlaps W_V_up
    # the two stages
    assert lib.vmla_query_prologue(dr, cr, vm.VMLA_BF16, R(1), R(2), R(3), 2, 1, 3, R(0), ws_need,
                                   None) == OV
    assert lib.vmla_latent_attention(dr, cr, vm.VMLA_BF16, R(4), 2, 1, 3, R(0) + 64, R(6), ws_need,
                                     None) == OV
    assert lib.vmla_latent_attention(dr, cr, vm.VMLA_BF16, R(4), 2, 1, 3, R(6) + 32, R(6), ws_need,
                                     None) == OV

    # the whole layer
    lw = lib.vmla_layer_workspace_bytes(dr, 768, 1, 24)
    assert lib.vmla_chunk_attention_layer(dr, cr, vm.VMLA_BF16, R(1), R(2), 768, R(3), R(4), 2, 1, 3,
                                          R(6) + lw - 16, R(6), lw, None) == OV
    assert lib.vmla_layer_query_prologue(dr, cr, vm.VMLA_BF16, R(1), R(2), 768, R(3), 2, 1, 3, R(0),
                                         lw, None) == OV
    assert lib.vmla_layer_attention(dr, cr, vm.VMLA_BF16, 768, R(4), 2, 1, 3, R(5), R(4), lw,
                                     None) == OV
    # explicit route
    xw = vm.vmla_explicit_workspace_bytes(1, 24, 72, d)
    assert lib.vmla_chunk_attention_explicit(dr, cr, vm.VMLA_BF16, R(1), R(2), R(3), 2, 1, 3, R(5),
                                             R(0), xw, None) == OV
    # whole clip
    clip = _cache(data=R(0), window_frames=7)
    need = vm.vmla_attention_workspace_bytes(1, 7 * 24, d)
    assert lib.vmla_chunk_causal_attention(dr, ctypes.byref(clip), vm.VMLA_BF16, R(1), R(2), R(3),
                                           R(4), 7, 3, 5, R(6), R(6), need, None) == OV
    assert lib.vmla_chunk_causal_latent_attention(dr, ctypes.byref(clip), vm.VMLA_BF16, R(4), 7, 3, 5,
                                                  R(0), R(6), need, None) == OV
    big = vm.vmla_explicit_workspace_bytes(1, 7 * 24, 7 * 24, d)
    assert lib.vmla_chunk_causal_attention_explicit(dr, ctypes.byref(clip), vm.VMLA_BF16, R(1), R(2),
                                                    R(3), 7, 3, 5, R(5), R(1), big, None) == OV
    # weight folds and packing, the unfolded mixer
    assert lib.vmla_fold_query_weights(dr, vm.VMLA_BF16, 768, R(1), R(2), R(1) + 32, None) == OV
    assert lib.vmla_fold_output_weights(dr, vm.VMLA_BF16, R(1), R(2), R(2), None) == OV
    assert lib.vmla_pack_kv_weights(dr, vm.VMLA_BF16, R(1), R(2), R(1), None) == OV
    assert lib.vmla_output_projection(dr, vm.VMLA_BF16, 8, R(1), R(2), R(1) + 16, None) == OV


def test_valid_calls_reach_the_launchers(lib):
    # Only in the host-only sanitizer build, whose launchers are counting stubs
    # that return hipErrorNoDevice: every entry point, called with valid
    # arguments at disjoint fake addresses, passes validation, fills its launch
    # arguments and reaches a launcher (VMLA_ERR_HIP). No device is touched.
    if not hasattr(lib, "vmla_stub_launch_count"):
        pytest.skip("needs the host-only stub build (tests/test_abi_sanitizers.py)")
    count = lib.vmla_stub_launch_count
    count.restype = ctypes.c_int
    HIP = vm.VMLA_ERR_HIP

    def reaches(st):
        before = reaches.n
        reaches.n = count()
        return st == HIP and reaches.n == before + 1
    reaches.n = count()

    for dims, cache_kw in [(vm.default_dims(), {}), (vm.default_dims(d_c=64), {}),
                           (vm.default_dims(d_c=512), {}),
                           (vm.default_dims(), dict(sink_frames=1, rope_at_read=1))]:
        d = dims
        cache = _cache(data=R(0), window_frames=21, grid_h=30, grid_w=52, batch=8, **cache_kw)
        dr, cr = ctypes.byref(d), ctypes.byref(cache)
        n_q = 3 * 1560
        t_first = 18 + 4 * cache.sink_frames
        n_valid = min(t_first + 3, 21 + cache.sink_frames)
        ws = vm.vmla_attention_workspace_bytes(8, n_q, d)
        assert reaches(lib.vmla_cache_append(dr, cr, vm.VMLA_BF16, R(1), R(2), R(3), t_first, 3, None))
        assert reaches(lib.vmla_query_prologue(dr, cr, vm.VMLA_BF16, R(1), R(2), R(3), t_first, 3,
                                               n_valid, R(6), ws, None))
        assert reaches(lib.vmla_latent_attention(dr, cr, vm.VMLA_BF16, R(4), t_first, 3, n_valid, R(5),
                                                 R(6), ws, None))
        # the fused call stops at its first launcher
        assert reaches(lib.vmla_chunk_attention(dr, cr, vm.VMLA_BF16, R(1), R(2), R(3), R(4), t_first, 3,
                                                n_valid, R(5), R(6), ws, None))
    d = vm.default_dims()
    dr = ctypes.byref(d)
    cache = _cache(data=R(0), window_frames=21, grid_h=30, grid_w=52, batch=2)
    cr = ctypes.byref(cache)
    lw = lib.vmla_layer_workspace_bytes(dr, 768, 2, 4680)
    assert reaches(lib.vmla_chunk_attention_layer(dr, cr, vm.VMLA_BF16, R(1), R(2), 768, R(3), R(4), 18, 3,
                                                  21, R(5), R(6), lw, None))
    assert reaches(lib.vmla_layer_attention(dr, cr, vm.VMLA_BF16, 768, R(4), 18, 3, 21, R(5), R(6), lw,
                                            None))
    xw = vm.vmla_explicit_workspace_bytes(2, 4680, 32760, d)
    assert reaches(lib.vmla_chunk_attention_explicit(dr, cr, vm.VMLA_BF16, R(1), R(2), R(3), 18, 3, 21,
                                                     R(5), R(6), xw, None))
    need = vm.vmla_attention_workspace_bytes(2, 21 * 1560, d)
    assert reaches(lib.vmla_chunk_causal_latent_attention(dr, cr, vm.VMLA_BF16, R(4), 21, 3, 21, R(5),
                                                          R(6), need, None))
    assert reaches(lib.vmla_fold_query_weights(dr, vm.VMLA_BF16, 768, R(1), R(2), R(3), None))
    assert reaches(lib.vmla_fold_output_weights(dr, vm.VMLA_BF16, R(1), R(2), R(3), None))
    assert reaches(lib.vmla_pack_kv_weights(dr, vm.VMLA_BF16, R(1), R(2), R(3), None))
    assert reaches(lib.vmla_output_projection(dr, vm.VMLA_BF16, 4680, R(1), R(2), R(3), None))
    # the no-allocation entry point passes every check and stops at the scratch
    # lookup (a stub without a device here), before any launch
    wan1 = _cache(data=R(0), window_frames=21, grid_h=30, grid_w=52)
    before = count()
    assert lib.vmla_chunk_attention_noalloc(dr, ctypes.byref(wan1), vm.VMLA_BF16, R(1), R(2), R(3), R(4), 18,
                                            3, 21, R(5), None) == HIP
    assert count() == before


def test_noalloc_validation(lib):
    # every host-side check runs before the scratch array is looked up (the
    # only HIP call before the launches); none of these calls reaches it
    d = vm.default_dims()
    dr = ctypes.byref(d)

    def call(cache, x=R(1), wq=R(2), wku=R(3), wvu=R(4), out=R(5), t_first=18, n_frames=3, n_valid=21,
             dtype=vm.VMLA_BF16, dims=dr):
        return lib.vmla_chunk_attention_noalloc(dims, ctypes.byref(cache), dtype, x, wq, wku, wvu, t_first,
                                                n_frames, n_valid, out, None)
    wan = _cache(data=R(0), window_frames=21, grid_h=30, grid_w=52)
    assert vm.VMLA_NOALLOC_SCRATCH_BYTES == 32 << 20
    # 4680 queries at B = 1 need 25.2 MB: fits; at B = 2, 50.3 MB: too large
    assert vm.vmla_attention_workspace_bytes(1, 4680, d) <= vm.VMLA_NOALLOC_SCRATCH_BYTES
    assert call(_cache(data=R(0), window_frames=21, grid_h=30, grid_w=52, batch=2)) == vm.VMLA_ERR_WORKSPACE
    assert call(_cache(data=R(0), window_frames=21, grid_h=30, grid_w=52, batch=16), t_first=20,
                n_frames=1) == vm.VMLA_ERR_WORKSPACE
    assert call(wan, x=None) == vm.VMLA_ERR_NULL
    assert call(wan, out=None) == vm.VMLA_ERR_NULL
    assert lib.vmla_chunk_attention_noalloc(None, ctypes.byref(wan), 1, R(1), R(2), R(3), R(4), 18, 3, 21,
                                            R(5), None) == vm.VMLA_ERR_NULL
    assert call(wan, out=MIS) == vm.VMLA_ERR_ALIGN
    assert call(wan, dtype=vm.VMLA_F32) == vm.VMLA_ERR_DTYPE
    assert call(wan, n_valid=20) == vm.VMLA_ERR_RANGE
    assert call(wan, dims=ctypes.byref(vm.default_dims(d_v=64))) == vm.VMLA_ERR_SHAPE
    assert call(wan, out=R(1)) == vm.VMLA_ERR_OVERLAP                    # out is x
    assert call(wan, out=R(0) + 64) == vm.VMLA_ERR_OVERLAP               # out inside the cache


def test_binding_cache_geometry():
    import torch
    c = vm.LatentCache(torch.zeros(1, 7 * 24, 224), 6, 4, 6, sink_frames=1, rope_at_read=True)
    assert [c.slot_frame(t) for t in (0, 1, 6, 7, 12, 13)] == [0, 1, 6, 1, 6, 1]
    assert c.n_valid_frames(0, 3) == 3 and c.n_valid_frames(18, 3) == 7
    plain = vm.LatentCache(torch.zeros(1, 3 * 24, 224), 3, 4, 6)
    assert [plain.slot_frame(t) for t in (0, 2, 3, 7)] == [0, 2, 0, 1]
    assert plain.n_valid_frames(7, 1) == 3
    cs = c.c_struct()
    assert (cs.sink_frames, cs.rope_at_read) == (1, 1)


def test_binding_rejects_cpu_tensors():
    import torch
    cache = vm.LatentCache(torch.zeros(1, 72, 224, dtype=torch.bfloat16), 3, 4, 6)
    x = torch.zeros(1, 24, 1536, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        vm.vmla_cache_append(cache, x, torch.zeros(1536, 192, dtype=torch.bfloat16),
                             torch.zeros(1536, 32, dtype=torch.bfloat16), 0, 1)


def test_peak_probe_library():
    # the matrix-core peak probe that bench.py times next to the published peak
    path = os.path.join(ROOT, "latent_kv_attention_cache_amd", "libvmla_probe.so")
    probe = ctypes.CDLL(path)
    probe.vmla_probe_sink_floats.restype = ctypes.c_int64
    probe.vmla_probe_mfma_flops.argtypes = [ctypes.c_int32]
    probe.vmla_probe_mfma_flops.restype = ctypes.c_double
    probe.vmla_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    assert probe.vmla_probe_sink_floats() == 1024 * 256
    # 1024 blocks x 4 waves x 4 MFMAs of 2 * 32 * 32 * 16 flops per trip
    assert probe.vmla_probe_mfma_flops(1) == 1024 * 4 * 4 * 32768
    assert probe.vmla_probe_mfma_bf16(None, 1, None) == -1
    assert probe.vmla_probe_mfma_bf16(A, 0, None) == -1
    probe.vmla_probe_read_sink_words.restype = ctypes.c_int64
    probe.vmla_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert probe.vmla_probe_read_sink_words() == 2048 * 256
    assert probe.vmla_probe_hbm_read(A, 24, B, None) == -1          # not a multiple of 16
    assert probe.vmla_probe_hbm_read(MIS, 32, B, None) == -1        # 8-byte aligned only
    assert probe.vmla_probe_hbm_read(None, 32, B, None) == -1
