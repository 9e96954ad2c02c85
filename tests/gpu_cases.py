"""Helpers for GPU parity tests: build seeded device inputs, drive the HIP path
through the C ABI binding, and compare with the CPU oracle.

The device side and the oracle side share only the seeded generators of
``workloads``; no expected value ever comes from the HIP path.
"""
from __future__ import annotations

import numpy as np
import torch

import latent_kv_attention_cache_amd as vm
import oracle.vmla_oracle as orc
from workloads import mixer_weights, weights, x_frame

REL_FROB = 1e-2     # ||gpu - ref||_F / ||ref||_F, pooled and per head
MAX_ABS = 3e-2      # max |gpu - ref|, absolute and relative to max |ref|


def tdtype(w):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def to_dev(a, w, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(tdtype(w))


def dev_weights(w, wts, device="cuda"):
    return {k: to_dev(v, w, device) for k, v in wts.items()}


def compare(gpu, ref, what, rel_frob=REL_FROB, max_abs=MAX_ABS, per_head_axis=None):
    """Assert the acceptance bar and return the error summary.

    The bar applies three ways: to the pooled relative Frobenius error, to
    each head's own relative Frobenius error (when ``per_head_axis`` names
    the head axis), and to the max error both in absolute terms and relative
    to max |ref|. At tens of thousands of keys |o| is about 0.01, so the
    absolute bound alone could not fail; the per-head and relative forms
    keep one wrong head or row block from hiding in the pooled norm."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values in GPU output"
    err = gpu - ref
    rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
    mx = float(np.abs(err).max())
    summary = {"rel_frob": rel, "max_abs": mx, "max_abs_over_max_ref": mx / float(np.abs(ref).max())}
    if per_head_axis is not None:
        e = np.moveaxis(err, per_head_axis, 0).reshape(err.shape[per_head_axis], -1)
        r = np.moveaxis(ref, per_head_axis, 0).reshape(ref.shape[per_head_axis], -1)
        summary["worst_head_rel_frob"] = float((np.linalg.norm(e, axis=1) / np.linalg.norm(r, axis=1)).max())
    print(f"[parity] {what}: {summary}", flush=True)
    assert rel <= rel_frob, f"{what}: rel Frobenius {rel:.3e} > {rel_frob}"
    assert mx <= max_abs, f"{what}: max abs {mx:.3e} > {max_abs}"
    assert summary["max_abs_over_max_ref"] <= max_abs, \
        f"{what}: max abs / max|ref| {summary['max_abs_over_max_ref']:.3e} > {max_abs}"
    if per_head_axis is not None:
        assert summary["worst_head_rel_frob"] <= rel_frob, \
            f"{what}: worst head rel Frobenius {summary['worst_head_rel_frob']:.3e} > {rel_frob}"
    return summary


class Run:
    """One batch of seeded inputs driven through the HIP path for workload ``w``."""

    def __init__(self, w, layer=0, step_of_frame=None, device="cuda", fill=None, batch_x=None):
        self.w = w
        self.layer = layer
        self.step_of_frame = step_of_frame or (lambda t: 0)
        self.wts = weights(w, layer)
        self.dw = dev_weights(w, self.wts, device)
        self.dims = vm.default_dims(d_model=w.d_model, n_heads=w.n_heads, d_c=w.d_c, d_nope=w.d_nope,
                                    d_rope=w.d_rope, rope_pairs=w.rope_pairs,
                                    rope_axis_dims=w.rope_axis_dims)
        self.cache = vm.LatentCache.empty(w.batch, w.window_frames, w.grid_h, w.grid_w,
                                          dtype=tdtype(w), device=device, dims=self.dims, fill=fill,
                                          sink_frames=w.sink_frames, rope_at_read=w.rope_at_read)
        self.device = device
        self._xcache = {}
        self.batch_x = batch_x   # optional fn(t, b) -> device tensor [T, D] (bulk inputs)

    def x_host(self, t, b=0):
        key = (t, b, self.step_of_frame(t))
        if key not in self._xcache:
            self._xcache[key] = x_frame(self.w, t, b=b, step=key[2], layer=self.layer)
        return self._xcache[key]

    def x_dev(self, frames):
        rows = []
        for b in range(self.w.batch):
            per = []
            for t in frames:
                if self.batch_x is not None:
                    per.append(self.batch_x(t, b))
                else:
                    per.append(to_dev(self.x_host(t, b), self.w, self.device))
            rows.append(torch.cat(per, 0))
        return torch.stack(rows, 0).contiguous()

    def append(self, t_first, n_frames):
        x = self.x_dev(range(t_first, t_first + n_frames))
        vm.vmla_cache_append(self.cache, x, self.dw["w_down"], self.dw["w_kr"], t_first, n_frames,
                             dims=self.dims)
        return x

    def fill_window(self):
        """Append the frames that precede the query chunk: each run of consecutive
        frames in pieces of at most W frames."""
        prior = list(self.w.prior_frames)
        i = 0
        while i < len(prior):
            n = 1
            while (i + n < len(prior) and prior[i + n] == prior[i] + n
                   and n < self.w.window_frames):
                n += 1
            self.append(prior[i], n)
            i += n

    def attention(self, t_first=None, n_frames=None):
        w = self.w
        t_first = w.t_first if t_first is None else t_first
        n_frames = w.chunk_frames if n_frames is None else n_frames
        x = self.x_dev(range(t_first, t_first + n_frames))
        n_valid = self.cache.n_valid_frames(t_first, n_frames)
        return vm.vmla_chunk_attention(self.cache, x, self.dw["w_q"], self.dw["w_k_up"],
                                       self.dw["w_v_up"], t_first, n_frames, n_valid,
                                       dims=self.dims)

    def chunk_step(self):
        """Fill the window, append the chunk, attend. Returns out [B, N_q, H, d_v]."""
        self.fill_window()
        self.append(self.w.t_first, self.w.chunk_frames)
        return self.attention()

    # ---- the whole layer: query latent and folded output mixer

    def _mixer(self):
        if not hasattr(self, "mix"):
            self.mix = mixer_weights(self.w, self.layer)
            self.dmix = dev_weights(self.w, self.mix, self.device)
            self.w_qa = vm.vmla_fold_query_weights(self.dmix["w_uq"], self.dw["w_k_up"], self.w.d_q,
                                                   dims=self.dims)
            self.w_vo = vm.vmla_fold_output_weights(self.dw["w_v_up"], self.dmix["w_o"], dims=self.dims)

    def layer_call(self, t_first=None, n_frames=None):
        """vmla_chunk_attention_layer for the chunk; returns out [B, N_q, d_model]."""
        self._mixer()
        w = self.w
        t_first = w.t_first if t_first is None else t_first
        n_frames = w.chunk_frames if n_frames is None else n_frames
        x = self.x_dev(range(t_first, t_first + n_frames))
        n_valid = self.cache.n_valid_frames(t_first, n_frames)
        return vm.vmla_chunk_attention_layer(self.cache, x, self.dmix["w_dq"], self.w_qa, self.w_vo,
                                             t_first, n_frames, n_valid, dims=self.dims)

    def layer_step(self):
        """Fill the window, append the chunk, run the whole layer."""
        self.fill_window()
        self.append(self.w.t_first, self.w.chunk_frames)
        return self.layer_call()

    def layer_reference(self, b=0, query_tokens=None, t_first=None, n_frames=None):
        self._mixer()
        w = self.w
        if t_first is not None:
            w = w.with_(t_first=t_first, chunk_frames=n_frames or w.chunk_frames)
        return orc.chunk_layer_reference(w, self.wts, self.mix, lambda t: self.x_host(t, b),
                                         query_tokens)

    def reference(self, b=0, query_tokens=None, t_first=None, n_frames=None):
        w = self.w
        if t_first is not None:
            w = w.with_(t_first=t_first, chunk_frames=n_frames or w.chunk_frames)
        ref = orc.chunk_attention_reindexed_reference if w.rope_at_read else orc.chunk_attention_reference
        return ref(w, self.wts, lambda t: self.x_host(t, b), query_tokens)

    def append_reference(self, t_first, n_frames, b=0):
        x = np.concatenate([self.x_host(t, b) for t in range(t_first, t_first + n_frames)])
        if self.w.rope_at_read:
            return orc.append_reference_raw(self.w, self.wts, x)
        return orc.append_reference(self.w, self.wts, x, t_first, n_frames)

    def cache_rows(self, t_first, n_frames, b=0):
        T = self.w.tokens_per_frame
        rows = []
        data = self.cache.data[b].float().cpu().numpy()
        for t in range(t_first, t_first + n_frames):
            s = self.cache.slot_frame(t) * T
            rows.append(data[s:s + T])
        return np.concatenate(rows)
