"""ctypes binding of ``libvmla.so`` (the C ABI in include/vmla.h).

Argument marshalling only: torch tensors supply device pointers, shapes and the
current HIP stream; every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is missing, or a tensor is not
on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import LIB_PATH

VMLA_OK = 0
VMLA_ERR_NULL = -1
VMLA_ERR_SHAPE = -2
VMLA_ERR_DTYPE = -3
VMLA_ERR_ALIGN = -4
VMLA_ERR_RANGE = -5
VMLA_ERR_WORKSPACE = -6
VMLA_ERR_HIP = -7
VMLA_ERR_OVERLAP = -8

VMLA_F32 = 0
VMLA_BF16 = 1

_TORCH_DTYPE = {VMLA_F32: torch.float32, VMLA_BF16: torch.bfloat16}
_VMLA_DTYPE = {torch.float32: VMLA_F32, torch.bfloat16: VMLA_BF16}


class vmla_dims(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_nope", ctypes.c_int32),
        ("d_rope", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("rope_pairs", ctypes.c_int32 * 3), ("rope_axis_dims", ctypes.c_int32 * 3),
        ("rope_theta", ctypes.c_float), ("scale", ctypes.c_float),
    ]


class vmla_cache(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("window_frames", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
        ("sink_frames", ctypes.c_int32), ("rope_at_read", ctypes.c_int32),
    ]


class VmlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {vmla_status_string(status)} (status {status})")


_LIB = None

EXPORTED = ("vmla_default_dims", "vmla_cache_append", "vmla_attention_workspace_bytes",
            "vmla_chunk_attention", "vmla_query_prologue", "vmla_latent_attention",
            "vmla_fold_query_weights", "vmla_fold_output_weights", "vmla_layer_workspace_bytes",
            "vmla_chunk_attention_layer", "vmla_layer_query_prologue", "vmla_layer_attention",
            "vmla_output_projection", "vmla_pack_kv_weights", "vmla_explicit_workspace_bytes",
            "vmla_chunk_attention_explicit", "vmla_chunk_causal_attention",
            "vmla_chunk_causal_latent_attention", "vmla_chunk_causal_attention_explicit",
            "vmla_chunk_attention_noalloc", "vmla_status_string", "vmla_abi_version")

# Size of the library-owned scratch array of vmla_chunk_attention_noalloc.
VMLA_NOALLOC_SCRATCH_BYTES = 32 << 20


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libvmla.so once; raise if it has not been built.

    ``VMLA_LIBRARY`` in the environment names another build of the same ABI
    (the CPU tests use it for the host-only sanitizer build)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or os.environ.get("VMLA_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m latent_kv_attention_cache_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    lib.vmla_default_dims.argtypes = [ctypes.POINTER(vmla_dims)]
    lib.vmla_default_dims.restype = None
    lib.vmla_cache_append.argtypes = [ctypes.POINTER(vmla_dims), ctypes.POINTER(vmla_cache), I32,
                                      P, P, P, I32, I32, P]
    lib.vmla_cache_append.restype = I32
    lib.vmla_attention_workspace_bytes.argtypes = [ctypes.POINTER(vmla_dims), I32, I32]
    lib.vmla_attention_workspace_bytes.restype = ctypes.c_size_t
    lib.vmla_chunk_attention.argtypes = [ctypes.POINTER(vmla_dims), ctypes.POINTER(vmla_cache), I32,
                                         P, P, P, P, I32, I32, I32, P, P, ctypes.c_size_t, P]
    lib.vmla_chunk_attention.restype = I32
    lib.vmla_chunk_attention_noalloc.argtypes = [ctypes.POINTER(vmla_dims), ctypes.POINTER(vmla_cache), I32,
                                                 P, P, P, P, I32, I32, I32, P, P]
    lib.vmla_chunk_attention_noalloc.restype = I32
    lib.vmla_query_prologue.argtypes = [ctypes.POINTER(vmla_dims), ctypes.POINTER(vmla_cache), I32,
                                        P, P, P, I32, I32, I32, P, ctypes.c_size_t, P]
    lib.vmla_query_prologue.restype = I32
    lib.vmla_latent_attention.argtypes = [ctypes.POINTER(vmla_dims), ctypes.POINTER(vmla_cache), I32,
                                          P, I32, I32, I32, P, P, ctypes.c_size_t, P]
    lib.vmla_latent_attention.restype = I32
    D, C, SZ = ctypes.POINTER(vmla_dims), ctypes.POINTER(vmla_cache), ctypes.c_size_t
    lib.vmla_fold_query_weights.argtypes = [D, I32, I32, P, P, P, P]
    lib.vmla_fold_query_weights.restype = I32
    lib.vmla_fold_output_weights.argtypes = [D, I32, P, P, P, P]
    lib.vmla_fold_output_weights.restype = I32
    lib.vmla_layer_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.vmla_layer_workspace_bytes.restype = SZ
    lib.vmla_chunk_attention_layer.argtypes = [D, C, I32, P, P, I32, P, P, I32, I32, I32, P, P, SZ, P]
    lib.vmla_chunk_attention_layer.restype = I32
    lib.vmla_layer_query_prologue.argtypes = [D, C, I32, P, P, I32, P, I32, I32, I32, P, SZ, P]
    lib.vmla_layer_query_prologue.restype = I32
    lib.vmla_layer_attention.argtypes = [D, C, I32, I32, P, I32, I32, I32, P, P, SZ, P]
    lib.vmla_layer_attention.restype = I32
    lib.vmla_output_projection.argtypes = [D, I32, ctypes.c_int64, P, P, P, P]
    lib.vmla_output_projection.restype = I32
    lib.vmla_pack_kv_weights.argtypes = [D, I32, P, P, P, P]
    lib.vmla_pack_kv_weights.restype = I32
    lib.vmla_explicit_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.vmla_explicit_workspace_bytes.restype = SZ
    lib.vmla_chunk_attention_explicit.argtypes = [D, C, I32, P, P, P, I32, I32, I32, P, P, SZ, P]
    lib.vmla_chunk_attention_explicit.restype = I32
    lib.vmla_chunk_causal_attention.argtypes = [D, C, I32, P, P, P, P, I32, I32, I32, P, P, SZ, P]
    lib.vmla_chunk_causal_attention.restype = I32
    lib.vmla_chunk_causal_latent_attention.argtypes = [D, C, I32, P, I32, I32, I32, P, P, SZ, P]
    lib.vmla_chunk_causal_latent_attention.restype = I32
    lib.vmla_chunk_causal_attention_explicit.argtypes = [D, C, I32, P, P, P, I32, I32, I32, P, P, SZ, P]
    lib.vmla_chunk_causal_attention_explicit.restype = I32
    lib.vmla_status_string.argtypes = [I32]
    lib.vmla_status_string.restype = ctypes.c_char_p
    lib.vmla_abi_version.argtypes = []
    lib.vmla_abi_version.restype = I32
    _LIB = lib
    return lib


def vmla_status_string(status: int) -> str:
    return load_library().vmla_status_string(int(status)).decode()


def default_dims(**overrides) -> vmla_dims:
    d = vmla_dims()
    load_library().vmla_default_dims(ctypes.byref(d))
    for k, v in overrides.items():
        if k in ("rope_pairs", "rope_axis_dims"):
            getattr(d, k)[:] = list(v)
        else:
            setattr(d, k, v)
    return d


@dataclass
class LatentCache:
    """Cache of latent frames: ``data`` [batch, (sink_frames + window_frames) *
    grid_h * grid_w, d_c + d_rope]: the sink frame (if any), then the ring of the
    most recent ``window_frames`` frames. ``rope_at_read``: k_R is kept before
    RoPE and rotated in the active context at attention time."""
    data: torch.Tensor
    window_frames: int
    grid_h: int
    grid_w: int
    sink_frames: int = 0
    rope_at_read: bool = False

    @staticmethod
    def empty(batch: int, window_frames: int, grid_h: int, grid_w: int, dtype=torch.bfloat16,
              device="cuda", dims: vmla_dims | None = None, fill: float | None = None,
              sink_frames: int = 0, rope_at_read: bool = False) -> "LatentCache":
        d = dims or default_dims()
        t = torch.empty((batch, (sink_frames + window_frames) * grid_h * grid_w, d.d_c + d.d_rope),
                        dtype=dtype, device=device)
        if fill is not None:
            t.fill_(fill)
        return LatentCache(t, window_frames, grid_h, grid_w, sink_frames, rope_at_read)

    def n_valid_frames(self, t_first: int, n_frames: int) -> int:
        """Frames of the active context once frames t_first .. t_first + n_frames - 1 are in."""
        return min(t_first + n_frames, self.sink_frames + self.window_frames)

    def slot_frame(self, t: int) -> int:
        """Slot frame (slots [s * T, (s + 1) * T)) that latent frame t is stored in."""
        if t < self.sink_frames:
            return t
        return self.sink_frames + (t - self.sink_frames) % self.window_frames

    @property
    def batch(self) -> int:
        return self.data.shape[0]

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    def c_struct(self) -> vmla_cache:
        return vmla_cache(self.data.data_ptr(), _dtype_code(self.data), self.data.shape[0],
                          self.window_frames, self.grid_h, self.grid_w, int(self.sink_frames),
                          int(bool(self.rope_at_read)))


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _VMLA_DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32") from None


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _expect_shape(t: torch.Tensor, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def vmla_cache_append(cache: LatentCache, x: torch.Tensor, w_down: torch.Tensor, w_kr: torch.Tensor,
                      t_first: int, n_frames: int, dims: vmla_dims | None = None, stream=None) -> None:
    """Write frames t_first .. t_first + n_frames - 1 of every batch element into the ring."""
    lib = load_library()
    d = dims or default_dims()
    B, T = cache.batch, cache.tokens_per_frame
    _expect_shape(x, (B, n_frames * T, d.d_model), "x")
    _expect_shape(w_down, (d.d_model, d.d_c), "w_down")
    _expect_shape(w_kr, (d.d_model, d.d_rope), "w_kr")
    code = _dtype_code(cache.data)
    for t, n in ((x, "x"), (w_down, "w_down"), (w_kr, "w_kr")):
        if t.dtype != cache.data.dtype:
            raise TypeError(f"{n} dtype {t.dtype} differs from the cache's {cache.data.dtype}")
    _dev(cache.data, "cache")
    cs = cache.c_struct()
    st = lib.vmla_cache_append(ctypes.byref(d), ctypes.byref(cs), code, _dev(x, "x"),
                               _dev(w_down, "w_down"), _dev(w_kr, "w_kr"), int(t_first),
                               int(n_frames), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_cache_append")


def vmla_attention_workspace_bytes(batch: int, n_q: int, dims: vmla_dims | None = None) -> int:
    d = dims or default_dims()
    return int(load_library().vmla_attention_workspace_bytes(ctypes.byref(d), int(batch), int(n_q)))


def vmla_chunk_attention(cache: LatentCache, x: torch.Tensor, w_q: torch.Tensor, w_k_up: torch.Tensor,
                         w_v_up: torch.Tensor, t_first: int, n_frames: int, n_valid_frames: int,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """Attention of the chunk's queries over ring slots [0, n_valid_frames * T).

    Returns ``out`` [batch, n_frames * T, n_heads, d_v] in the cache dtype.
    """
    lib = load_library()
    d = dims or default_dims()
    B, T = cache.batch, cache.tokens_per_frame
    n_q = n_frames * T
    _expect_shape(x, (B, n_q, d.d_model), "x")
    _expect_shape(w_q, (d.d_model, d.n_heads * (d.d_nope + d.d_rope)), "w_q")
    _expect_shape(w_k_up, (d.n_heads, d.d_c, d.d_nope), "w_k_up")
    _expect_shape(w_v_up, (d.n_heads, d.d_c, d.d_v), "w_v_up")
    code = _dtype_code(cache.data)
    for t, n in ((x, "x"), (w_q, "w_q"), (w_k_up, "w_k_up"), (w_v_up, "w_v_up")):
        if t.dtype != cache.data.dtype:
            raise TypeError(f"{n} dtype {t.dtype} differs from the cache's {cache.data.dtype}")
    if out is None:
        out = torch.empty((B, n_q, d.n_heads, d.d_v), dtype=cache.data.dtype, device=x.device)
    _expect_shape(out, (B, n_q, d.n_heads, d.d_v), "out")
    need = vmla_attention_workspace_bytes(B, n_q, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _dev(cache.data, "cache")
    cs = cache.c_struct()
    st = lib.vmla_chunk_attention(ctypes.byref(d), ctypes.byref(cs), code, _dev(x, "x"),
                                  _dev(w_q, "w_q"), _dev(w_k_up, "w_k_up"), _dev(w_v_up, "w_v_up"),
                                  int(t_first), int(n_frames), int(n_valid_frames),
                                  _dev(out, "out"), _dev(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_chunk_attention")
    return out


def vmla_chunk_attention_noalloc(cache: LatentCache, x: torch.Tensor, w_q: torch.Tensor,
                                 w_k_up: torch.Tensor, w_v_up: torch.Tensor, t_first: int,
                                 n_frames: int, n_valid_frames: int, out: torch.Tensor,
                                 dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """vmla_chunk_attention with the library's own scratch array instead of a
    workspace: the call allocates nothing (``out`` is the caller's). Calls that
    overlap in time on one GPU race on that array."""
    lib = load_library()
    d = dims or default_dims()
    B, T = cache.batch, cache.tokens_per_frame
    n_q = n_frames * T
    _expect_shape(x, (B, n_q, d.d_model), "x")
    _expect_shape(w_q, (d.d_model, d.n_heads * (d.d_nope + d.d_rope)), "w_q")
    _expect_shape(w_k_up, (d.n_heads, d.d_c, d.d_nope), "w_k_up")
    _expect_shape(w_v_up, (d.n_heads, d.d_c, d.d_v), "w_v_up")
    _expect_shape(out, (B, n_q, d.n_heads, d.d_v), "out")
    for t, n in ((x, "x"), (w_q, "w_q"), (w_k_up, "w_k_up"), (w_v_up, "w_v_up"), (out, "out")):
        if t.dtype != cache.data.dtype:
            raise TypeError(f"{n} dtype {t.dtype} differs from the cache's {cache.data.dtype}")
    _dev(cache.data, "cache")
    cs = cache.c_struct()
    st = lib.vmla_chunk_attention_noalloc(ctypes.byref(d), ctypes.byref(cs), _dtype_code(cache.data),
                                          _dev(x, "x"), _dev(w_q, "w_q"), _dev(w_k_up, "w_k_up"),
                                          _dev(w_v_up, "w_v_up"), int(t_first), int(n_frames),
                                          int(n_valid_frames), _dev(out, "out"), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_chunk_attention_noalloc")
    return out


def _attn_common(cache, x, w_q, w_k_up, w_v_up, n_frames, out, workspace, d):
    B, T = cache.batch, cache.tokens_per_frame
    n_q = n_frames * T
    if x is not None:
        _expect_shape(x, (B, n_q, d.d_model), "x")
    if w_q is not None:
        _expect_shape(w_q, (d.d_model, d.n_heads * (d.d_nope + d.d_rope)), "w_q")
    if w_k_up is not None:
        _expect_shape(w_k_up, (d.n_heads, d.d_c, d.d_nope), "w_k_up")
    if w_v_up is not None:
        _expect_shape(w_v_up, (d.n_heads, d.d_c, d.d_v), "w_v_up")
    for t, n in ((x, "x"), (w_q, "w_q"), (w_k_up, "w_k_up"), (w_v_up, "w_v_up"), (out, "out")):
        if t is not None and t.dtype != cache.data.dtype:
            raise TypeError(f"{n} dtype {t.dtype} differs from the cache's {cache.data.dtype}")
    if out is not None:
        _expect_shape(out, (B, n_q, d.n_heads, d.d_v), "out")
    need = vmla_attention_workspace_bytes(B, n_q, d)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    _dev(cache.data, "cache")
    return cache.c_struct(), _dtype_code(cache.data)


def vmla_query_prologue(cache: LatentCache, x, w_q, w_k_up, t_first: int, n_frames: int,
                        n_valid_frames: int, workspace: torch.Tensor, dims: vmla_dims | None = None,
                        stream=None) -> None:
    """First stage of vmla_chunk_attention: absorbed, pre-scaled queries into ``workspace``."""
    lib = load_library()
    d = dims or default_dims()
    cs, code = _attn_common(cache, x, w_q, w_k_up, None, n_frames, None, workspace, d)
    st = lib.vmla_query_prologue(ctypes.byref(d), ctypes.byref(cs), code, _dev(x, "x"),
                                 _dev(w_q, "w_q"), _dev(w_k_up, "w_k_up"), int(t_first),
                                 int(n_frames), int(n_valid_frames), _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_query_prologue")


def vmla_latent_attention(cache: LatentCache, w_v_up, t_first: int, n_frames: int,
                          n_valid_frames: int, out: torch.Tensor, workspace: torch.Tensor,
                          dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """Second stage of vmla_chunk_attention: attention over the window from ``workspace``."""
    lib = load_library()
    d = dims or default_dims()
    cs, code = _attn_common(cache, None, None, None, w_v_up, n_frames, out, workspace, d)
    st = lib.vmla_latent_attention(ctypes.byref(d), ctypes.byref(cs), code, _dev(w_v_up, "w_v_up"),
                                   int(t_first), int(n_frames), int(n_valid_frames),
                                   _dev(out, "out"), _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_latent_attention")
    return out


# ---------------------------------------------------------------------------
# The whole attention layer: query latent and folded output mixer
# ---------------------------------------------------------------------------

def _same_dtype(ref: torch.Tensor, **tensors):
    for n, t in tensors.items():
        if t.dtype != ref.dtype:
            raise TypeError(f"{n} dtype {t.dtype} differs from {ref.dtype}")


def vmla_fold_query_weights(w_uq: torch.Tensor, w_k_up: torch.Tensor, d_q: int,
                            out: torch.Tensor | None = None, dims: vmla_dims | None = None,
                            stream=None) -> torch.Tensor:
    """bf16 [d_q, n_heads * (d_c + d_rope)]: per head [A_h | W_UQ^rope[h]]."""
    lib = load_library()
    d = dims or default_dims()
    _expect_shape(w_uq, (d_q, d.n_heads * (d.d_nope + d.d_rope)), "w_uq")
    _expect_shape(w_k_up, (d.n_heads, d.d_c, d.d_nope), "w_k_up")
    _same_dtype(w_uq, w_k_up=w_k_up)
    if out is None:
        out = torch.empty((d_q, d.n_heads * (d.d_c + d.d_rope)), dtype=torch.bfloat16,
                          device=w_uq.device)
    _expect_shape(out, (d_q, d.n_heads * (d.d_c + d.d_rope)), "w_qa")
    if out.dtype != torch.bfloat16:
        raise TypeError("w_qa must be bfloat16")
    st = lib.vmla_fold_query_weights(ctypes.byref(d), _dtype_code(w_uq), int(d_q), _dev(w_uq, "w_uq"),
                                     _dev(w_k_up, "w_k_up"), _dev(out, "w_qa"), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_fold_query_weights")
    return out


def vmla_fold_output_weights(w_v_up: torch.Tensor, w_o: torch.Tensor, out: torch.Tensor | None = None,
                             dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """bf16 [n_heads * d_c, d_model]: per head B_h W_O[h]."""
    lib = load_library()
    d = dims or default_dims()
    _expect_shape(w_v_up, (d.n_heads, d.d_c, d.d_v), "w_v_up")
    _expect_shape(w_o, (d.n_heads * d.d_v, d.d_model), "w_o")
    _same_dtype(w_v_up, w_o=w_o)
    if out is None:
        out = torch.empty((d.n_heads * d.d_c, d.d_model), dtype=torch.bfloat16, device=w_o.device)
    _expect_shape(out, (d.n_heads * d.d_c, d.d_model), "w_vo")
    if out.dtype != torch.bfloat16:
        raise TypeError("w_vo must be bfloat16")
    st = lib.vmla_fold_output_weights(ctypes.byref(d), _dtype_code(w_o), _dev(w_v_up, "w_v_up"),
                                      _dev(w_o, "w_o"), _dev(out, "w_vo"), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_fold_output_weights")
    return out


def vmla_layer_workspace_bytes(batch: int, n_q: int, d_q: int, dims: vmla_dims | None = None) -> int:
    d = dims or default_dims()
    return int(load_library().vmla_layer_workspace_bytes(ctypes.byref(d), int(d_q), int(batch),
                                                         int(n_q)))


def _layer_common(cache, x, w_dq, d_q, w_qa, w_vo, n_frames, out, workspace, d):
    B, T = cache.batch, cache.tokens_per_frame
    n_q = n_frames * T
    if x is not None:
        _expect_shape(x, (B, n_q, d.d_model), "x")
        _same_dtype(cache.data, x=x)
    if w_dq is not None:
        _expect_shape(w_dq, (d.d_model, d_q), "w_dq")
        _same_dtype(cache.data, w_dq=w_dq)
    if w_qa is not None:
        _expect_shape(w_qa, (d_q, d.n_heads * (d.d_c + d.d_rope)), "w_qa")
        if w_qa.dtype != torch.bfloat16:
            raise TypeError("w_qa must be bfloat16")
    if w_vo is not None:
        _expect_shape(w_vo, (d.n_heads * d.d_c, d.d_model), "w_vo")
        if w_vo.dtype != torch.bfloat16:
            raise TypeError("w_vo must be bfloat16")
    if out is not None:
        _expect_shape(out, (B, n_q, d.d_model), "out")
        _same_dtype(cache.data, out=out)
    need = vmla_layer_workspace_bytes(B, n_q, d_q, d)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    _dev(cache.data, "cache")
    return cache.c_struct(), _dtype_code(cache.data)


def vmla_chunk_attention_layer(cache: LatentCache, x: torch.Tensor, w_dq: torch.Tensor,
                               w_qa: torch.Tensor, w_vo: torch.Tensor, t_first: int, n_frames: int,
                               n_valid_frames: int, out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None, dims: vmla_dims | None = None,
                               stream=None) -> torch.Tensor:
    """One chunk step of the whole layer; returns ``out`` [batch, n_q, d_model]."""
    lib = load_library()
    d = dims or default_dims()
    d_q = w_dq.shape[1]
    B, n_q = cache.batch, n_frames * cache.tokens_per_frame
    if out is None:
        out = torch.empty((B, n_q, d.d_model), dtype=cache.data.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty(vmla_layer_workspace_bytes(B, n_q, d_q, d), dtype=torch.uint8,
                                device=x.device)
    cs, code = _layer_common(cache, x, w_dq, d_q, w_qa, w_vo, n_frames, out, workspace, d)
    st = lib.vmla_chunk_attention_layer(ctypes.byref(d), ctypes.byref(cs), code, _dev(x, "x"),
                                        _dev(w_dq, "w_dq"), int(d_q), _dev(w_qa, "w_qa"),
                                        _dev(w_vo, "w_vo"), int(t_first), int(n_frames),
                                        int(n_valid_frames), _dev(out, "out"),
                                        _dev(workspace, "workspace"),
                                        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_chunk_attention_layer")
    return out


def vmla_layer_query_prologue(cache: LatentCache, x, w_dq, w_qa, t_first: int, n_frames: int,
                              n_valid_frames: int, workspace: torch.Tensor,
                              dims: vmla_dims | None = None, stream=None) -> None:
    """First stage of vmla_chunk_attention_layer: query latent and Qhat rows into ``workspace``."""
    lib = load_library()
    d = dims or default_dims()
    d_q = w_dq.shape[1]
    cs, code = _layer_common(cache, x, w_dq, d_q, w_qa, None, n_frames, None, workspace, d)
    st = lib.vmla_layer_query_prologue(ctypes.byref(d), ctypes.byref(cs), code, _dev(x, "x"),
                                       _dev(w_dq, "w_dq"), int(d_q), _dev(w_qa, "w_qa"), int(t_first),
                                       int(n_frames), int(n_valid_frames), _dev(workspace, "workspace"),
                                       workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_layer_query_prologue")


def vmla_layer_attention(cache: LatentCache, d_q: int, w_vo, t_first: int, n_frames: int,
                         n_valid_frames: int, out: torch.Tensor, workspace: torch.Tensor,
                         dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """Second stage of vmla_chunk_attention_layer: attention and folded output mixer."""
    lib = load_library()
    d = dims or default_dims()
    cs, code = _layer_common(cache, None, None, d_q, None, w_vo, n_frames, out, workspace, d)
    st = lib.vmla_layer_attention(ctypes.byref(d), ctypes.byref(cs), code, int(d_q), _dev(w_vo, "w_vo"),
                                  int(t_first), int(n_frames), int(n_valid_frames), _dev(out, "out"),
                                  _dev(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_layer_attention")
    return out


def vmla_output_projection(heads: torch.Tensor, w_o: torch.Tensor, out: torch.Tensor | None = None,
                           dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """Unfolded output mixer: ``heads`` [..., n_heads, d_v] (vmla_chunk_attention's
    output) times w_o [n_heads * d_v, d_model] -> [..., d_model]."""
    lib = load_library()
    d = dims or default_dims()
    if tuple(heads.shape[-2:]) != (d.n_heads, d.d_v):
        raise ValueError(f"heads has shape {tuple(heads.shape)}, expected [..., {d.n_heads}, {d.d_v}]")
    _expect_shape(w_o, (d.n_heads * d.d_v, d.d_model), "w_o")
    _same_dtype(heads, w_o=w_o)
    m = heads.numel() // (d.n_heads * d.d_v)
    if out is None:
        out = torch.empty(tuple(heads.shape[:-2]) + (d.d_model,), dtype=heads.dtype, device=heads.device)
    _expect_shape(out, tuple(heads.shape[:-2]) + (d.d_model,), "out")
    _same_dtype(heads, out=out)
    st = lib.vmla_output_projection(ctypes.byref(d), _dtype_code(heads), int(m), _dev(heads, "heads"),
                                    _dev(w_o, "w_o"), _dev(out, "out"), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_output_projection")
    return out


# ---------------------------------------------------------------------------
# Explicit reconstruction (comparison point of the latent form)
# ---------------------------------------------------------------------------

def vmla_pack_kv_weights(w_k_up: torch.Tensor, w_v_up: torch.Tensor, out: torch.Tensor | None = None,
                         dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """[d_c, n_heads * (d_nope + d_v)]: per head [W_K_up[h] | W_V_up[h]] (dtype of the inputs)."""
    lib = load_library()
    d = dims or default_dims()
    _expect_shape(w_k_up, (d.n_heads, d.d_c, d.d_nope), "w_k_up")
    _expect_shape(w_v_up, (d.n_heads, d.d_c, d.d_v), "w_v_up")
    _same_dtype(w_k_up, w_v_up=w_v_up)
    if out is None:
        out = torch.empty((d.d_c, d.n_heads * (d.d_nope + d.d_v)), dtype=w_k_up.dtype,
                          device=w_k_up.device)
    _expect_shape(out, (d.d_c, d.n_heads * (d.d_nope + d.d_v)), "w_kv")
    _same_dtype(w_k_up, w_kv=out)
    st = lib.vmla_pack_kv_weights(ctypes.byref(d), _dtype_code(w_k_up), _dev(w_k_up, "w_k_up"),
                                  _dev(w_v_up, "w_v_up"), _dev(out, "w_kv"), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_pack_kv_weights")
    return out


def vmla_explicit_workspace_bytes(batch: int, n_q: int, n_k: int, dims: vmla_dims | None = None) -> int:
    d = dims or default_dims()
    return int(load_library().vmla_explicit_workspace_bytes(ctypes.byref(d), int(batch), int(n_q),
                                                            int(n_k)))


def vmla_chunk_attention_explicit(cache: LatentCache, x: torch.Tensor, w_q: torch.Tensor,
                                  w_kv: torch.Tensor, t_first: int, n_frames: int, n_valid_frames: int,
                                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                  dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """Chunk attention through explicit per-head K/V reconstruction; returns
    ``out`` [batch, n_q, n_heads, d_v] (the same result as vmla_chunk_attention)."""
    lib = load_library()
    d = dims or default_dims()
    B, T = cache.batch, cache.tokens_per_frame
    n_q = n_frames * T
    _expect_shape(x, (B, n_q, d.d_model), "x")
    _expect_shape(w_q, (d.d_model, d.n_heads * (d.d_nope + d.d_rope)), "w_q")
    _expect_shape(w_kv, (d.d_c, d.n_heads * (d.d_nope + d.d_v)), "w_kv")
    _same_dtype(cache.data, x=x, w_q=w_q, w_kv=w_kv)
    if out is None:
        out = torch.empty((B, n_q, d.n_heads, d.d_v), dtype=cache.data.dtype, device=x.device)
    _expect_shape(out, (B, n_q, d.n_heads, d.d_v), "out")
    _same_dtype(cache.data, out=out)
    need = vmla_explicit_workspace_bytes(B, n_q, n_valid_frames * T, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    _dev(cache.data, "cache")
    cs = cache.c_struct()
    st = lib.vmla_chunk_attention_explicit(ctypes.byref(d), ctypes.byref(cs), _dtype_code(cache.data),
                                           _dev(x, "x"), _dev(w_q, "w_q"), _dev(w_kv, "w_kv"),
                                           int(t_first), int(n_frames), int(n_valid_frames),
                                           _dev(out, "out"), _dev(workspace, "workspace"),
                                           workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_chunk_attention_explicit")
    return out


# ---------------------------------------------------------------------------
# A whole clip under the chunk-causal block mask
# ---------------------------------------------------------------------------

def _clip_out(cache, x, n_frames, out, d):
    B, T = cache.batch, cache.tokens_per_frame
    n_q = n_frames * T
    if x is not None:
        _expect_shape(x, (B, n_q, d.d_model), "x")
    if out is None:
        out = torch.empty((B, n_q, d.n_heads, d.d_v), dtype=cache.data.dtype, device=cache.data.device)
    _expect_shape(out, (B, n_q, d.n_heads, d.d_v), "out")
    _same_dtype(cache.data, out=out)
    _dev(cache.data, "cache")
    return out, n_q


def vmla_chunk_causal_attention(cache: LatentCache, x: torch.Tensor, w_q: torch.Tensor,
                                w_k_up: torch.Tensor, w_v_up: torch.Tensor, n_frames: int,
                                chunk_frames: int, mask_window_frames: int,
                                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """Every token of frames 0 .. n_frames - 1 attends under the chunk-causal
    block mask (chunks of ``chunk_frames``, a window of ``mask_window_frames``);
    ``cache`` holds the clip's rows at slots t * T + n. Returns ``out``
    [batch, n_frames * T, n_heads, d_v]."""
    lib = load_library()
    d = dims or default_dims()
    _expect_shape(w_q, (d.d_model, d.n_heads * (d.d_nope + d.d_rope)), "w_q")
    _expect_shape(w_k_up, (d.n_heads, d.d_c, d.d_nope), "w_k_up")
    _expect_shape(w_v_up, (d.n_heads, d.d_c, d.d_v), "w_v_up")
    _same_dtype(cache.data, x=x, w_q=w_q, w_k_up=w_k_up, w_v_up=w_v_up)
    out, n_q = _clip_out(cache, x, n_frames, out, d)
    need = vmla_attention_workspace_bytes(cache.batch, n_q, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    cs = cache.c_struct()
    st = lib.vmla_chunk_causal_attention(ctypes.byref(d), ctypes.byref(cs), _dtype_code(cache.data),
                                         _dev(x, "x"), _dev(w_q, "w_q"), _dev(w_k_up, "w_k_up"),
                                         _dev(w_v_up, "w_v_up"), int(n_frames), int(chunk_frames),
                                         int(mask_window_frames), _dev(out, "out"),
                                         _dev(workspace, "workspace"),
                                         workspace.numel() * workspace.element_size(), _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_chunk_causal_attention")
    return out


def vmla_chunk_causal_latent_attention(cache: LatentCache, w_v_up: torch.Tensor, n_frames: int,
                                       chunk_frames: int, mask_window_frames: int, out: torch.Tensor,
                                       workspace: torch.Tensor, dims: vmla_dims | None = None,
                                       stream=None) -> torch.Tensor:
    """Second stage of vmla_chunk_causal_attention: reads the Qhat rows that
    vmla_query_prologue (t_first = 0, n_frames, n_valid_frames = n_frames) left
    in ``workspace``."""
    lib = load_library()
    d = dims or default_dims()
    _expect_shape(w_v_up, (d.n_heads, d.d_c, d.d_v), "w_v_up")
    _same_dtype(cache.data, w_v_up=w_v_up)
    out, n_q = _clip_out(cache, None, n_frames, out, d)
    need = vmla_attention_workspace_bytes(cache.batch, n_q, d)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    cs = cache.c_struct()
    st = lib.vmla_chunk_causal_latent_attention(ctypes.byref(d), ctypes.byref(cs),
                                                _dtype_code(cache.data), _dev(w_v_up, "w_v_up"),
                                                int(n_frames), int(chunk_frames),
                                                int(mask_window_frames), _dev(out, "out"),
                                                _dev(workspace, "workspace"),
                                                workspace.numel() * workspace.element_size(),
                                                _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_chunk_causal_latent_attention")
    return out


def vmla_chunk_causal_attention_explicit(cache: LatentCache, x: torch.Tensor, w_q: torch.Tensor,
                                         w_kv: torch.Tensor, n_frames: int, chunk_frames: int,
                                         mask_window_frames: int, out: torch.Tensor | None = None,
                                         workspace: torch.Tensor | None = None,
                                         dims: vmla_dims | None = None, stream=None) -> torch.Tensor:
    """vmla_chunk_causal_attention through explicit per-head K/V of the whole
    clip (``w_kv`` from vmla_pack_kv_weights)."""
    lib = load_library()
    d = dims or default_dims()
    _expect_shape(w_q, (d.d_model, d.n_heads * (d.d_nope + d.d_rope)), "w_q")
    _expect_shape(w_kv, (d.d_c, d.n_heads * (d.d_nope + d.d_v)), "w_kv")
    _same_dtype(cache.data, x=x, w_q=w_q, w_kv=w_kv)
    out, n_q = _clip_out(cache, x, n_frames, out, d)
    need = vmla_explicit_workspace_bytes(cache.batch, n_q, n_q, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    cs = cache.c_struct()
    st = lib.vmla_chunk_causal_attention_explicit(ctypes.byref(d), ctypes.byref(cs),
                                                  _dtype_code(cache.data), _dev(x, "x"),
                                                  _dev(w_q, "w_q"), _dev(w_kv, "w_kv"),
                                                  int(n_frames), int(chunk_frames),
                                                  int(mask_window_frames), _dev(out, "out"),
                                                  _dev(workspace, "workspace"),
                                                  workspace.numel() * workspace.element_size(),
                                                  _stream(stream))
    if st != VMLA_OK:
        raise VmlaError(st, "vmla_chunk_causal_attention_explicit")
    return out
