"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against something the pages print, a closed form,
an invariant, a library routine, or brute force on tiny inputs. The last
group plants plausible mistakes into a copy of the oracle and shows that some
pin fails for each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.vmla_oracle as orc
from workloads import config, custom, split_variant, weights, x_frame

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------------------
# Storage figures printed on the pages
# ---------------------------------------------------------------------------

def test_storage_figures_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "storage_figures.json")))
    d = g["dims"]["value"]
    lat = orc.cached_scalars_per_token(d["d_c"], d["d_rope"])
    dense = orc.dense_scalars_per_token(d["n_heads"], d["d_head"])
    assert lat == g["latent_scalars_per_token"]["value"]
    assert dense == g["dense_scalars_per_token"]["value"]
    assert round(100.0 * (1.0 - lat / dense), 1) == g["reduction_percent"]["value"]
    assert round(dense / lat, 1) == g["reduction_factor"]["value"]
    ct = g["clip_tokens"]
    assert ct["frames"] * ct["tokens_per_frame"] == ct["value"]
    w = config(2)
    assert w.window_frames * w.tokens_per_frame == ct["value"]
    total = ct["value"] * d["n_layers"] * dense
    assert round(total / 1e9, 2) == g["dense_cache_scalars_billions"]["value"]
    assert round(total * g["dense_cache_gb_bf16"]["bytes_per_scalar"] / 1e9, 1) == \
        g["dense_cache_gb_bf16"]["value"]
    # the workload dims agree with the printed model dims
    assert (w.d_model, w.n_heads, w.d_head, w.d_c, w.d_rope) == \
        (d["d_model"], d["n_heads"], d["d_head"], d["d_c"], d["d_rope"])
    assert w.cache_row == lat


# ---------------------------------------------------------------------------
# 3D-RoPE
# ---------------------------------------------------------------------------

OMEGA = orc.rope_frequencies()


def _rope_complex(v, pos):
    """Independent route: RoPE as multiplication of complex pairs by e^{i phi}."""
    axes = [0] * 6 + [1] * 5 + [2] * 5
    out = np.empty_like(v, dtype=np.float64)
    for j in range(16):
        z = complex(v[2 * j], v[2 * j + 1]) * complex(math.cos(pos[axes[j]] * OMEGA[j]),
                                                      math.sin(pos[axes[j]] * OMEGA[j]))
        out[2 * j], out[2 * j + 1] = z.real, z.imag
    return out


def test_rope_is_complex_rotation():
    for _ in range(20):
        v = RNG.standard_normal(32)
        pos = RNG.integers(0, 300, size=3)
        np.testing.assert_allclose(orc.rope3d(v, pos, OMEGA), _rope_complex(v, pos),
                                   rtol=0, atol=1e-12)


def test_rope_basis_vector_closed_form():
    # pair 0 is on the t axis with omega = 1: (1, 0) at t -> (cos t, sin t)
    v = np.zeros(32)
    v[0] = 1.0
    out = orc.rope3d(v, np.array([3, 0, 0]), OMEGA)
    np.testing.assert_allclose(out[:2], [math.cos(3.0), math.sin(3.0)], atol=1e-15)
    np.testing.assert_allclose(out[2:], 0.0, atol=0)


def test_rope_norm_identity_group_law():
    v = RNG.standard_normal((50, 32))
    p = RNG.integers(0, 500, size=(50, 3))
    p2 = RNG.integers(0, 500, size=(50, 3))
    r = orc.rope3d(v, p, OMEGA)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(v, axis=1), rtol=1e-13)
    np.testing.assert_allclose(orc.rope3d(v, np.zeros((50, 3), int), OMEGA), v, atol=0)
    np.testing.assert_allclose(orc.rope3d(r, p2, OMEGA), orc.rope3d(v, p + p2, OMEGA),
                               rtol=0, atol=1e-11)


def test_rope_relative_position_invariance():
    q = RNG.standard_normal((40, 32))
    k = RNG.standard_normal((40, 32))
    pq = RNG.integers(0, 200, size=(40, 3))
    pk = RNG.integers(0, 200, size=(40, 3))
    shift = RNG.integers(-100, 100, size=(40, 3))
    a = np.sum(orc.rope3d(q, pq, OMEGA) * orc.rope3d(k, pk, OMEGA), axis=1)
    b = np.sum(orc.rope3d(q, pq + shift, OMEGA) * orc.rope3d(k, pk + shift, OMEGA), axis=1)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_rope_axis_split_6_5_5_and_highest_bands():
    # [PL] App. D.3: 16 complex pairs split (6, 5, 5) over t, h, w, using each
    # axis group's highest-frequency bands.
    assert list(orc.rope_pair_axes()) == [0] * 6 + [1] * 5 + [2] * 5
    assert OMEGA.shape == (16,)
    for lo, hi in ((0, 6), (6, 11), (11, 16)):
        assert OMEGA[lo] == 1.0                          # highest band of the group
        assert np.all(np.diff(OMEGA[lo:hi]) < 0)         # bands decrease within a group
    v = RNG.standard_normal(32)
    for axis, (lo, hi) in enumerate(((0, 6), (6, 11), (11, 16))):
        pos = np.zeros(3, int)
        pos[axis] = 7
        out = orc.rope3d(v, pos, OMEGA)
        moved = np.flatnonzero(np.abs(out - v).reshape(16, 2).max(axis=1) > 1e-12)
        assert list(moved) == list(range(lo, hi))


def _standard_rope_inv_freq(dim, theta):
    """Inverse frequencies of plain (unscaled) RoPE over a head of width
    ``dim``, as the transformers library computes them: its linear-scaling
    routine at factor 1.0 is the original RoPE law."""
    transformers = pytest.importorskip("transformers")
    from transformers import modeling_rope_utils
    cfg = transformers.LlamaConfig(hidden_size=dim, num_attention_heads=1, head_dim=dim,
                                   rope_parameters={"rope_type": "linear", "factor": 1.0,
                                                    "rope_theta": float(theta)})
    inv_freq, _ = modeling_rope_utils._compute_linear_scaling_rope_parameters(cfg)
    return inv_freq.double().numpy()


def test_rope_frequency_law_matches_standard_rope_per_axis():
    # [PL] App. C.1: the t, h and w axes are rotated separately and the results
    # concatenated; [PL] App. D.3: 16 pairs split (6, 5, 5). Reading R1: each
    # axis group of width D_a = 12 / 10 / 10 is an ordinary RoPE subspace, so
    # its pair rates are exactly those of standard RoPE over a D_a-wide head at
    # theta = 10^4. The split variants' groups (6/6/4, 24/20/20, 36/30/30) too.
    from workloads import SPLIT_ROPE
    tables = [((6, 5, 5), (12, 10, 10))] + [tuple(v) for v in SPLIT_ROPE.values()]
    for pairs, dims in tables:
        om = orc.rope_frequencies(pairs, dims)
        assert om.shape == (sum(pairs),)
        lo = 0
        for n_pairs, dim in zip(pairs, dims):
            ref = _standard_rope_inv_freq(dim, 10000.0)[:n_pairs]
            # transformers computes in fp32: a few ulps of 2^-24
            np.testing.assert_allclose(om[lo:lo + n_pairs], ref, rtol=1e-6, atol=0,
                                       err_msg=f"axis group {dim} of {pairs}/{dims}")
            lo += n_pairs


def test_frame_positions_token_order():
    p = orc.frame_positions(5, 3, 4)
    assert p.shape == (12, 3)
    for n in range(12):
        assert tuple(p[n]) == (5, n // 4, n % 4)


# ---------------------------------------------------------------------------
# Attention core
# ---------------------------------------------------------------------------

def _rand_heads(nq, nk, H=3, dn=5, dr=4, dv=6, scale_q=1.0):
    q_nope = RNG.standard_normal((nq, H, dn)) * scale_q
    q_rope = RNG.standard_normal((nq, H, dr)) * scale_q
    k_nope = RNG.standard_normal((nk, H, dn))
    k_r = RNG.standard_normal((nk, dr))
    v = RNG.standard_normal((nk, H, dv))
    return q_nope, q_rope, k_nope, k_r, v


def test_attention_matches_torch_sdpa_fp64():
    q_nope, q_rope, k_nope, k_r, v = _rand_heads(7, 33)
    H = q_nope.shape[1]
    d = q_nope.shape[2] + q_rope.shape[2]
    out = orc.attention_explicit(q_nope, q_rope, k_nope, k_r, v, 1.0 / math.sqrt(d))
    Q = torch.from_numpy(np.concatenate([q_nope, q_rope], -1)).permute(1, 0, 2)[None]
    K = torch.from_numpy(np.concatenate([k_nope, np.repeat(k_r[:, None], H, 1)], -1)).permute(1, 0, 2)[None]
    V = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)   # default scale 1/sqrt(d)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_attention_closed_forms():
    q_nope, q_rope, k_nope, k_r, v = _rand_heads(4, 9)
    # zero queries -> uniform weights -> mean of the values
    out = orc.attention_explicit(0 * q_nope, 0 * q_rope, k_nope, k_r, v, 0.3)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-14)
    # one key -> that key's value
    out1 = orc.attention_explicit(q_nope, q_rope, k_nope[:1], k_r[:1], v[:1], 0.3)
    np.testing.assert_allclose(out1, np.broadcast_to(v[0], out1.shape), atol=1e-14)
    # a dominant key takes all the weight
    k2 = k_nope.copy()
    out2 = orc.attention_explicit(np.ones_like(q_nope), 0 * q_rope, np.where(
        np.arange(9)[:, None, None] == 4, 50.0, 0.0) + 0 * k2, 0 * k_r, v, 1.0)
    np.testing.assert_allclose(out2, np.broadcast_to(v[4], out2.shape), atol=1e-12)


def test_softmax_rows_sum_to_one():
    s = RNG.standard_normal((20, 300)) * 30
    p = orc.softmax_rows(s)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(orc.softmax_rows(s + 1234.5), p, atol=1e-14)   # shift invariance


def test_absorbed_equals_explicit():
    # [PL] App. E: latent-form inference keeps the training-time computation.
    H, dn, dr, dc, dv = 3, 6, 4, 7, 5
    c = RNG.standard_normal((41, dc))
    k_r = RNG.standard_normal((41, dr))
    w_k_up = RNG.standard_normal((H, dc, dn))
    w_v_up = RNG.standard_normal((H, dc, dv))
    q_nope = RNG.standard_normal((11, H, dn))
    q_rope = RNG.standard_normal((11, H, dr))
    k_nope, v = orc.reconstruct_heads(c, w_k_up, w_v_up)
    a = orc.attention_explicit(q_nope, q_rope, k_nope, k_r, v, 0.4)
    b = orc.attention_absorbed(q_nope, q_rope, c, k_r, w_k_up, w_v_up, 0.4)
    assert rel(b, a) < 1e-12


def test_mla_reduces_to_dense_mha_with_selection_up_projections():
    # d_c = H (d_nope + d_v): W_down holds every head's dense key and value
    # weights side by side; W_K_up / W_V_up select a head's block. MLA is then
    # exactly a dense MHA whose positional key is shared by all heads.
    D, H, dn, dr, dv = 10, 2, 3, 4, 5
    dc = H * (dn + dv)
    wk = [RNG.standard_normal((D, dn)) for _ in range(H)]
    wv = [RNG.standard_normal((D, dv)) for _ in range(H)]
    w_down = np.concatenate(wk + wv, axis=1)
    w_k_up = np.zeros((H, dc, dn))
    w_v_up = np.zeros((H, dc, dv))
    for h in range(H):
        w_k_up[h, h * dn:(h + 1) * dn, :] = np.eye(dn)
        w_v_up[h, H * dn + h * dv:H * dn + (h + 1) * dv, :] = np.eye(dv)
    w_kr = RNG.standard_normal((D, dr * 8))[:, :dr]
    w_q = RNG.standard_normal((D, H * (dn + dr)))
    xk = RNG.standard_normal((13, D))
    xq = RNG.standard_normal((6, D))
    # dr = 4 means 2 complex pairs: one on t, one on h
    pairs, dims = (1, 1, 0), (2, 2, 2)
    om = orc.rope_frequencies(pairs, dims)
    pk = RNG.integers(0, 20, size=(13, 3))
    pq = RNG.integers(0, 20, size=(6, 3))

    c, k_r = orc.latent_entry(xk, w_down, w_kr, pk, om, pairs)
    k_nope, v = orc.reconstruct_heads(c, w_k_up, w_v_up)
    q_nope, q_rope = orc.queries(xq, w_q, pq, om, H, dn, dr, pairs)
    out = orc.attention_explicit(q_nope, q_rope, k_nope, k_r, v, 1 / math.sqrt(dn + dr))

    # dense MHA built directly, RoPE by complex multiplication, SDPA from torch
    def crot(a, p):
        z = a[..., 0::2] + 1j * a[..., 1::2]
        phi = np.stack([p[..., 0] * om[0], p[..., 1] * om[1]], -1)
        z = z * np.exp(1j * phi)
        r = np.empty_like(a)
        r[..., 0::2], r[..., 1::2] = z.real, z.imag
        return r
    krot = crot(xk @ w_kr, pk)
    Qs, Ks, Vs = [], [], []
    for h in range(H):
        qh = xq @ w_q[:, h * (dn + dr):(h + 1) * (dn + dr)]
        Qs.append(np.concatenate([qh[:, :dn], crot(qh[:, dn:], pq)], 1))
        Ks.append(np.concatenate([xk @ wk[h], krot], 1))
        Vs.append(xk @ wv[h])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.stack(Qs))[None], torch.from_numpy(np.stack(Ks))[None],
        torch.from_numpy(np.stack(Vs))[None])[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)


def test_mla_equals_dense_mha_with_composed_weights_real_dims():
    # At the real widths: W_K,h := W_down W_K_up[h], W_V,h := W_down W_V_up[h].
    w = custom(2, 3, window_frames=2, chunk_frames=1, t_first=1, dtype="f32")
    wt = weights(w)
    xs = {t: x_frame(w, t) for t in range(2)}
    out = orc.chunk_attention_reference(w, wt, lambda t: xs[t])
    om = orc.rope_frequencies()
    H, dn = w.n_heads, w.d_nope
    xk = np.concatenate([xs[0], xs[1]]).astype(np.float64)
    pk = np.concatenate([orc.frame_positions(t, 2, 3) for t in (0, 1)])
    xq = xs[1].astype(np.float64)
    pq = orc.frame_positions(1, 2, 3)
    krot = np.stack([_rope_complex(r, p) for r, p in zip(xk @ wt["w_kr"].astype(np.float64), pk)])
    Qs, Ks, Vs = [], [], []
    for h in range(H):
        WK = wt["w_down"].astype(np.float64) @ wt["w_k_up"][h].astype(np.float64)
        WV = wt["w_down"].astype(np.float64) @ wt["w_v_up"][h].astype(np.float64)
        qh = xq @ wt["w_q"][:, h * 128:(h + 1) * 128].astype(np.float64)
        qr = np.stack([_rope_complex(r, p) for r, p in zip(qh[:, dn:], pq)])
        Qs.append(np.concatenate([qh[:, :dn], qr], 1))
        Ks.append(np.concatenate([xk @ WK, krot], 1))
        Vs.append(xk @ WV)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.stack(Qs))[None], torch.from_numpy(np.stack(Ks))[None],
        torch.from_numpy(np.stack(Vs))[None])[0].permute(1, 0, 2).numpy()
    assert rel(out, ref) < 1e-12


def test_oracle_at_wan_geometry_equals_dense_mha_with_composed_weights():
    # The benchmark geometry: a 30x52 grid (h up to 29, w up to 51) and t up to
    # 20, the real widths, a 3-frame window of 4680 keys; sampled query rows of
    # the last frame, corner tokens included. Reference: a dense MHA whose head
    # h uses W_K,h = W_down W_K_up[h] and W_V,h = W_down W_V_up[h] (the other
    # association of the products), RoPE by complex multiplication with the
    # per-axis standard-RoPE rates of transformers, torch SDPA in fp64.
    w = custom(30, 52, window_frames=3, chunk_frames=1, t_first=20, dtype="f32")
    wt = weights(w)
    frames = (18, 19, 20)
    xs = {t: x_frame(w, t) for t in frames}
    rows = np.array([0, 51, 52, 777, 1508, 1559])
    out = orc.chunk_attention_reference(w, wt, lambda t: xs[t], rows)
    om = np.concatenate([_standard_rope_inv_freq(d, 10000.0)[:n]
                         for n, d in zip(w.rope_pairs, w.rope_axis_dims)])

    def rot(v, p):
        ang = np.concatenate([np.full(n, float(p[a])) for a, n in enumerate(w.rope_pairs)]) * om
        z = (v[0::2] + 1j * v[1::2]) * np.exp(1j * ang)
        o = np.empty_like(v)
        o[0::2], o[1::2] = z.real, z.imag
        return o

    H, dn = w.n_heads, w.d_nope
    xk = np.concatenate([xs[t] for t in frames]).astype(np.float64)
    pk = [(t, n // 52, n % 52) for t in frames for n in range(1560)]
    krot = np.stack([rot(r, p) for r, p in zip(xk @ wt["w_kr"].astype(np.float64), pk)])
    xq = xs[20][rows].astype(np.float64)
    pq = [(20, n // 52, n % 52) for n in rows]
    wdown = wt["w_down"].astype(np.float64)
    Qs, Ks, Vs = [], [], []
    for h in range(H):
        qh = xq @ wt["w_q"][:, h * 128:(h + 1) * 128].astype(np.float64)
        Qs.append(np.concatenate([qh[:, :dn], np.stack([rot(r, p) for r, p in zip(qh[:, dn:], pq)])], 1))
        Ks.append(np.concatenate([xk @ (wdown @ wt["w_k_up"][h].astype(np.float64)), krot], 1))
        Vs.append(xk @ (wdown @ wt["w_v_up"][h].astype(np.float64)))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.stack(Qs))[None], torch.from_numpy(np.stack(Ks))[None],
        torch.from_numpy(np.stack(Vs))[None])[0].permute(1, 0, 2).numpy()
    # fp32 rates from transformers: angles up to ~50 rad carry ~1e-5 relative error
    assert rel(out, ref) < 1e-5


def _rope_complex_split(v, pos, pairs, axis_dims, theta=10000.0):
    """RoPE of a d_rope vector as multiplication of complex pairs by e^{i phi},
    the frequencies written out from theta^(-2 i / D_a) per axis group."""
    out = np.empty(len(v), dtype=np.float64)
    j = 0
    for ax in range(3):
        for i in range(pairs[ax]):
            om = theta ** (-2.0 * i / axis_dims[ax])
            z = complex(v[2 * j], v[2 * j + 1]) * complex(math.cos(pos[ax] * om), math.sin(pos[ax] * om))
            out[2 * j], out[2 * j + 1] = z.real, z.imag
            j += 1
    assert 2 * j == len(v)
    return out


@pytest.mark.parametrize("d_rope", [16, 64, 96])
def test_split_variants_equal_dense_mha_with_composed_weights(d_rope):
    # [PL] App. F NoPE/RoPE split variants at the real widths: the oracle with
    # the (128 - d_rope) / d_rope split equals a dense MHA whose head h has
    # W_K,h = W_down W_K_up[h] on its first 128 - d_rope columns and the shared,
    # rotated k_R on the rest (SDPA from torch, RoPE as complex multiplication).
    w = split_variant(custom(2, 3, window_frames=2, chunk_frames=1, t_first=1, dtype="f32"), d_rope)
    wt = weights(w)
    assert wt["w_kr"].shape == (1536, d_rope) and wt["w_k_up"].shape == (12, 192, 128 - d_rope)
    xs = {t: x_frame(w, t) for t in range(2)}
    out = orc.chunk_attention_reference(w, wt, lambda t: xs[t])
    dn = w.d_nope
    xk = np.concatenate([xs[0], xs[1]]).astype(np.float64)
    pk = np.concatenate([orc.frame_positions(t, 2, 3) for t in (0, 1)])
    xq = xs[1].astype(np.float64)
    pq = orc.frame_positions(1, 2, 3)
    rot = lambda a, p: _rope_complex_split(a, p, w.rope_pairs, w.rope_axis_dims)  # noqa: E731
    krot = np.stack([rot(r, p) for r, p in zip(xk @ wt["w_kr"].astype(np.float64), pk)])
    Qs, Ks, Vs = [], [], []
    for h in range(w.n_heads):
        WK = wt["w_down"].astype(np.float64) @ wt["w_k_up"][h].astype(np.float64)
        WV = wt["w_down"].astype(np.float64) @ wt["w_v_up"][h].astype(np.float64)
        qh = xq @ wt["w_q"][:, h * 128:(h + 1) * 128].astype(np.float64)
        Qs.append(np.concatenate([qh[:, :dn], np.stack([rot(r, p) for r, p in zip(qh[:, dn:], pq)])], 1))
        Ks.append(np.concatenate([xk @ WK, krot], 1))
        Vs.append(xk @ WV)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.stack(Qs))[None], torch.from_numpy(np.stack(Ks))[None],
        torch.from_numpy(np.stack(Vs))[None])[0].permute(1, 0, 2).numpy()
    assert rel(out, ref) < 1e-12


def test_split_rope_allocation():
    # the variants' t/h/w pair counts sum to d_rope / 2 and keep 6:5:5 (R17)
    from workloads import SPLIT_ROPE
    for d_rope, (pairs, dims) in SPLIT_ROPE.items():
        assert 2 * sum(pairs) == d_rope and tuple(2 * p for p in pairs) == tuple(dims)
    assert SPLIT_ROPE[32] == ((6, 5, 5), (12, 10, 10))


def test_brute_force_scalar_loops_tiny():
    # Tiny dims, every sum written as a scalar loop with math.cos / math.exp.
    D, H, dn, dr, dc, dv = 3, 2, 2, 4, 3, 2
    pairs, dims = (1, 1, 0), (2, 2, 2)
    om = orc.rope_frequencies(pairs, dims)
    w_q = RNG.standard_normal((D, H * (dn + dr)))
    w_down = RNG.standard_normal((D, dc))
    w_kr = RNG.standard_normal((D, dr))
    w_k_up = RNG.standard_normal((H, dc, dn))
    w_v_up = RNG.standard_normal((H, dc, dv))
    xk = RNG.standard_normal((5, D))
    xq = RNG.standard_normal((2, D))
    pk = RNG.integers(0, 9, size=(5, 3))
    pq = RNG.integers(0, 9, size=(2, 3))
    scale = 1 / math.sqrt(dn + dr)

    def mv(x, W, j):
        return sum(x[i] * W[i][j] for i in range(len(x)))

    def rot(vec, p):
        ang = [p[0] * om[0], p[1] * om[1]]
        o = list(vec)
        for j in range(2):
            a, b = vec[2 * j], vec[2 * j + 1]
            o[2 * j] = a * math.cos(ang[j]) - b * math.sin(ang[j])
            o[2 * j + 1] = a * math.sin(ang[j]) + b * math.cos(ang[j])
        return o

    ref = np.zeros((2, H, dv))
    for qi in range(2):
        qfull = [mv(xq[qi], w_q, j) for j in range(H * (dn + dr))]
        for h in range(H):
            qn = qfull[h * (dn + dr):h * (dn + dr) + dn]
            qr = rot(qfull[h * (dn + dr) + dn:(h + 1) * (dn + dr)], pq[qi])
            s, vals = [], []
            for k in range(5):
                c = [mv(xk[k], w_down, j) for j in range(dc)]
                kr = rot([mv(xk[k], w_kr, j) for j in range(dr)], pk[k])
                kn = [sum(c[i] * w_k_up[h][i][j] for i in range(dc)) for j in range(dn)]
                vv = [sum(c[i] * w_v_up[h][i][j] for i in range(dc)) for j in range(dv)]
                s.append(scale * (sum(qn[j] * kn[j] for j in range(dn)) +
                                  sum(qr[j] * kr[j] for j in range(dr))))
                vals.append(vv)
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for j in range(dv):
                ref[qi, h, j] = sum(e[k] / z * vals[k][j] for k in range(5))

    c, k_r = orc.latent_entry(xk, w_down, w_kr, pk, om, pairs)
    k_nope, v = orc.reconstruct_heads(c, w_k_up, w_v_up)
    q_nope, q_rope = orc.queries(xq, w_q, pq, om, H, dn, dr, pairs)
    out = orc.attention_explicit(q_nope, q_rope, k_nope, k_r, v, scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Positional caching and the ring
# ---------------------------------------------------------------------------

def test_absolute_rotation_equals_window_local_rotation():
    # [PL] App. D.5 / App. E rotate cached keys at read time with window-local
    # t; rotating at append time with absolute t gives the same scores when
    # queries use the same origin (no sink frame).
    w = custom(2, 3, window_frames=4, chunk_frames=2, t_first=7, dtype="f32")
    wt = weights(w)
    xs = {t: x_frame(w, t) for t in range(3, 9)}
    absolute = orc.chunk_attention_reference(w, wt, lambda t: xs[t])
    t0 = 5   # oldest frame of the window
    wl = w.with_(t_first=w.t_first - t0)
    local = orc.chunk_attention_reference(wl, wt, lambda t: xs[t + t0])
    assert rel(local, absolute) < 1e-12


# ---------------------------------------------------------------------------
# Long-horizon context: sink frame + window, RoPE at read time ([PL] App. D.4-D.5)
# ---------------------------------------------------------------------------

def test_reindexed_context_without_eviction_is_the_whole_history():
    # Before any frame is evicted the context is frames 0 .. t_end - 1 and their
    # local coordinates are the absolute ones: plain attention over all frames.
    w = custom(2, 3, window_frames=6, chunk_frames=3, t_first=2,
               dtype="f32").with_(sink_frames=1, rope_at_read=True)
    wt = weights(w)
    xs = {t: x_frame(w, t) for t in range(0, 5)}
    re = orc.chunk_attention_reindexed_reference(w, wt, lambda t: xs[t])
    plain = orc.chunk_attention_reference(
        w.with_(window_frames=5, sink_frames=0, rope_at_read=False), wt, lambda t: xs[t])
    assert rel(re, plain) < 1e-12


def test_reindexed_window_without_sink_equals_append_time_rotation():
    # Without a sink the local coordinates are a uniform shift of the absolute
    # ones, so the scores equal those of keys rotated when they were cached.
    w = custom(2, 3, window_frames=4, chunk_frames=2, t_first=7, dtype="f32")
    wt = weights(w)
    xs = {t: x_frame(w, t) for t in range(5, 9)}
    plain = orc.chunk_attention_reference(w, wt, lambda t: xs[t])
    re = orc.chunk_attention_reindexed_reference(w.with_(rope_at_read=True), wt, lambda t: xs[t])
    assert rel(re, plain) < 1e-12


def test_reindexed_sink_context_brute_force_tiny():
    # One sink frame (frame 0), a window of 2 frames, chunk = frame 4: the
    # context is frames 0, 3, 4 at local t 0, 1, 2. Every sum a scalar loop.
    D, H, dn, dr, dc, dv = 3, 2, 2, 4, 3, 2
    pairs, dims = (1, 1, 0), (2, 2, 2)
    w = custom(1, 2, window_frames=2, chunk_frames=1, t_first=4, dtype="f32").with_(
        d_model=D, n_heads=H, d_nope=dn, d_rope=dr, d_c=dc, d_v=dv, rope_pairs=pairs,
        rope_axis_dims=dims, sink_frames=1, rope_at_read=True)
    wt = {"w_q": RNG.standard_normal((D, H * (dn + dr))), "w_down": RNG.standard_normal((D, dc)),
          "w_kr": RNG.standard_normal((D, dr)), "w_k_up": RNG.standard_normal((H, dc, dn)),
          "w_v_up": RNG.standard_normal((H, dc, dv))}
    xs = {t: RNG.standard_normal((2, D)) for t in range(5)}
    om = orc.rope_frequencies(pairs, dims)
    scale = 1 / math.sqrt(dn + dr)

    def mv(x, W, j):
        return sum(x[i] * W[i][j] for i in range(len(x)))

    def rot(vec, t, h):
        ang = [t * om[0], h * om[1]]
        o = list(vec)
        for j in range(2):
            a, b = vec[2 * j], vec[2 * j + 1]
            o[2 * j] = a * math.cos(ang[j]) - b * math.sin(ang[j])
            o[2 * j + 1] = a * math.sin(ang[j]) + b * math.cos(ang[j])
        return o

    keys = [(xs[t][n], tl, n // 2) for t, tl in ((0, 0), (3, 1), (4, 2)) for n in range(2)]
    ref = np.zeros((2, H, dv))
    for qi in range(2):
        qfull = [mv(xs[4][qi], wt["w_q"], j) for j in range(H * (dn + dr))]
        for h in range(H):
            qn = qfull[h * (dn + dr):h * (dn + dr) + dn]
            qr = rot(qfull[h * (dn + dr) + dn:(h + 1) * (dn + dr)], 2, qi // 2)
            s, vals = [], []
            for xk, tl, hk in keys:
                c = [mv(xk, wt["w_down"], j) for j in range(dc)]
                kr = rot([mv(xk, wt["w_kr"], j) for j in range(dr)], tl, hk)
                kn = [sum(c[i] * wt["w_k_up"][h][i][j] for i in range(dc)) for j in range(dn)]
                vv = [sum(c[i] * wt["w_v_up"][h][i][j] for i in range(dc)) for j in range(dv)]
                s.append(scale * (sum(qn[j] * kn[j] for j in range(dn)) +
                                  sum(qr[j] * kr[j] for j in range(dr))))
                vals.append(vv)
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for j in range(dv):
                ref[qi, h, j] = sum(e[k] / z * vals[k][j] for k in range(len(keys)))
    out = orc.chunk_attention_reindexed_reference(w, wt, lambda t: xs[t])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_reindexing_sees_relative_coordinates_only(monkeypatch):
    # After eviction: adding a constant to every local coordinate leaves the
    # output unchanged (RoPE's relative invariance), while keeping the window
    # frames at their absolute t next to the sink at 0 changes it.
    w = custom(2, 3, window_frames=3, chunk_frames=2, t_first=9,
               dtype="f32").with_(sink_frames=1, rope_at_read=True)
    wt = weights(w)
    xs = {t: x_frame(w, t) for t in range(0, 11)}
    base = orc.chunk_attention_reindexed_reference(w, wt, lambda t: xs[t])
    orig = orc.active_context
    monkeypatch.setattr(orc, "active_context", lambda *a: [(t, tl + 5) for t, tl in orig(*a)])
    shifted = orc.chunk_attention_reindexed_reference(w, wt, lambda t: xs[t])
    monkeypatch.setattr(orc, "active_context", lambda *a: [(t, t) for t, _ in orig(*a)])
    absolute = orc.chunk_attention_reindexed_reference(w, wt, lambda t: xs[t])
    assert rel(shifted, base) < 1e-12
    assert rel(absolute, base) > 1e-3


# ---------------------------------------------------------------------------
# The whole layer: query latent and output mixer ([PL] §4, App. E)
# ---------------------------------------------------------------------------

def test_layer_with_identity_query_latent_and_mixer_is_the_attention_reference():
    # d_q = d_model with W_DQ = I and W_UQ = W_Q, and W_O = I: the layer is the
    # pinned single-projection reference with the heads concatenated in order,
    # for the plain window and for the re-indexed sink-plus-window context.
    for kw, ref_fn in (({}, orc.chunk_attention_reference),
                       (dict(sink_frames=1, rope_at_read=True),
                        orc.chunk_attention_reindexed_reference)):
        w = custom(2, 3, window_frames=3, chunk_frames=2, t_first=5, dtype="f32").with_(
            d_q=1536, **kw)
        wt = weights(w)
        xs = {t: x_frame(w, t) for t in range(0, 7)}
        eye = np.eye(w.d_model)
        mix = {"w_dq": eye, "w_uq": wt["w_q"], "w_o": eye}
        y = orc.chunk_layer_reference(w, wt, mix, lambda t: xs[t])
        ref = ref_fn(w, wt, lambda t: xs[t])
        assert rel(y, ref.reshape(ref.shape[0], -1)) < 1e-12


def _tiny_layer(D=7, dq=5, H=3, dn=4, dr=4, dc=6, dv=5):
    pairs, dims = (1, 1, 0), (2, 2, 2)
    return dict(D=D, dq=dq, H=H, dn=dn, dr=dr, dc=dc, dv=dv, pairs=pairs,
                om=orc.rope_frequencies(pairs, dims),
                w_dq=RNG.standard_normal((D, dq)), w_uq=RNG.standard_normal((dq, H * (dn + dr))),
                w_down=RNG.standard_normal((D, dc)), w_kr=RNG.standard_normal((D, dr)),
                w_k_up=RNG.standard_normal((H, dc, dn)), w_v_up=RNG.standard_normal((H, dc, dv)),
                w_o=RNG.standard_normal((H * dv, D)))


def test_layer_folded_latent_form_equals_explicit():
    # [PL] App. E: with A_h on the query latent and B_h folded into W_O, the
    # layer needs no per-head key or value and changes nothing but rounding.
    L = _tiny_layer()
    xk, xq = RNG.standard_normal((9, L["D"])), RNG.standard_normal((4, L["D"]))
    pk, pq = RNG.integers(0, 9, size=(9, 3)), RNG.integers(0, 9, size=(4, 3))
    scale = 1 / math.sqrt(L["dn"] + L["dr"])
    c, k_r = orc.latent_entry(xk, L["w_down"], L["w_kr"], pk, L["om"], L["pairs"])
    k_nope, v = orc.reconstruct_heads(c, L["w_k_up"], L["w_v_up"])
    q_nope, q_rope = orc.query_latent_queries(xq, L["w_dq"], L["w_uq"], pq, L["om"], L["H"],
                                              L["dn"], L["dr"], L["pairs"])
    explicit = orc.output_mixer(orc.attention_explicit(q_nope, q_rope, k_nope, k_r, v, scale),
                                L["w_o"])
    w_qa = orc.fold_query_weights(L["w_uq"], L["w_k_up"], L["H"], L["dn"], L["dr"])
    w_vo = orc.fold_output_weights(L["w_v_up"], L["w_o"])
    assert w_qa.shape == (L["dq"], L["H"] * (L["dc"] + L["dr"]))
    assert w_vo.shape == (L["H"] * L["dc"], L["D"])
    folded = orc.layer_latent_folded(xq @ L["w_dq"], pq, c, k_r, w_qa, w_vo, L["om"], L["H"],
                                     L["dc"], L["dr"], scale, L["pairs"])
    assert rel(folded, explicit) < 1e-12


def test_layer_brute_force_scalar_loops_tiny():
    # Grid 1x2, window of 2 frames, chunk = frame 3: keys of frames 2 and 3 at
    # their absolute t, queries of frame 3. Every sum a scalar loop. W_O is
    # square (H d_v = d_model), as in the real layer.
    D, dq, H, dn, dr, dc, dv = 4, 3, 2, 2, 4, 3, 2
    pairs, dims = (1, 1, 0), (2, 2, 2)
    w = custom(1, 2, window_frames=2, chunk_frames=1, t_first=3, dtype="f32").with_(
        d_model=D, d_q=dq, n_heads=H, d_nope=dn, d_rope=dr, d_c=dc, d_v=dv, rope_pairs=pairs,
        rope_axis_dims=dims)
    wt = {"w_down": RNG.standard_normal((D, dc)), "w_kr": RNG.standard_normal((D, dr)),
          "w_k_up": RNG.standard_normal((H, dc, dn)), "w_v_up": RNG.standard_normal((H, dc, dv))}
    mix = {"w_dq": RNG.standard_normal((D, dq)), "w_uq": RNG.standard_normal((dq, H * (dn + dr))),
           "w_o": RNG.standard_normal((H * dv, D))}
    xs = {t: RNG.standard_normal((2, D)) for t in range(4)}
    om = orc.rope_frequencies(pairs, dims)
    scale = 1 / math.sqrt(dn + dr)

    def mv(x, W, j):
        return sum(x[i] * W[i][j] for i in range(len(x)))

    def rot(vec, t, h):
        ang = [t * om[0], h * om[1]]
        o = list(vec)
        for j in range(2):
            a, b = vec[2 * j], vec[2 * j + 1]
            o[2 * j] = a * math.cos(ang[j]) - b * math.sin(ang[j])
            o[2 * j + 1] = a * math.sin(ang[j]) + b * math.cos(ang[j])
        return o

    keys = [(xs[t][n], t, n // 2) for t in (2, 3) for n in range(2)]
    ref = np.zeros((2, D))
    for qi in range(2):
        cq = [mv(xs[3][qi], mix["w_dq"], j) for j in range(dq)]
        qfull = [mv(cq, mix["w_uq"], j) for j in range(H * (dn + dr))]
        heads = []
        for h in range(H):
            qn = qfull[h * (dn + dr):h * (dn + dr) + dn]
            qr = rot(qfull[h * (dn + dr) + dn:(h + 1) * (dn + dr)], 3, qi // 2)
            s, vals = [], []
            for xk, tk, hk in keys:
                c = [mv(xk, wt["w_down"], j) for j in range(dc)]
                kr = rot([mv(xk, wt["w_kr"], j) for j in range(dr)], tk, hk)
                kn = [sum(c[i] * wt["w_k_up"][h][i][j] for i in range(dc)) for j in range(dn)]
                vv = [sum(c[i] * wt["w_v_up"][h][i][j] for i in range(dc)) for j in range(dv)]
                s.append(scale * (sum(qn[j] * kn[j] for j in range(dn)) +
                                  sum(qr[j] * kr[j] for j in range(dr))))
                vals.append(vv)
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            heads += [sum(e[k] / z * vals[k][j] for k in range(len(keys))) for j in range(dv)]
        for j in range(D):
            ref[qi, j] = mv(heads, mix["w_o"], j)
    out = orc.chunk_layer_reference(w, wt, mix, lambda t: xs[t])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_append_reference_raw_rows():
    w = custom(2, 3, window_frames=4, chunk_frames=2, t_first=7, dtype="f32")
    wt = weights(w)
    x = np.concatenate([x_frame(w, t) for t in (7, 8)])
    raw = orc.append_reference_raw(w, wt, x)
    rot = orc.append_reference(w, wt, x, 7, 2)
    assert rel(raw[:, :w.d_c], rot[:, :w.d_c]) < 1e-15
    pos = np.concatenate([orc.frame_positions(t, 2, 3) for t in (7, 8)])
    om = orc.rope_frequencies(w.rope_pairs, w.rope_axis_dims, w.rope_theta)
    assert rel(orc.rope3d(raw[:, w.d_c:], pos, om, w.rope_pairs), rot[:, w.d_c:]) < 1e-13


def test_ring_after_wrap_equals_linear_window_and_slot_order_is_irrelevant():
    w = custom(2, 2, window_frames=3, chunk_frames=1, t_first=0, dtype="f32")
    wt = weights(w)
    om = orc.rope_frequencies()
    ring = orc.LatentRing(1, 3, 2, 2, w.d_c, w.d_rope)
    xs = {}
    for t in range(8):                      # wraps twice; frames 5, 6, 7 remain
        xs[t] = x_frame(w, t)
        ring.append_frame(0, t, xs[t], wt["w_down"], wt["w_kr"], om)
    c, k_r = ring.valid(0, 3)
    # slots: frame 6 -> 0, frame 7 -> 1, frame 5 -> 2
    assert [orc.ring_slot(t, 0, 4, 3) for t in (5, 6, 7)] == [8, 0, 4]
    lin_c, lin_kr = [], []
    for t in (5, 6, 7):
        cc, kk = orc.latent_entry(xs[t], wt["w_down"], wt["w_kr"], orc.frame_positions(t, 2, 2), om)
        lin_c.append(cc)
        lin_kr.append(kk)
    order = np.concatenate([np.arange(8, 12), np.arange(0, 4), np.arange(4, 8)])
    np.testing.assert_array_equal(c[order], np.concatenate(lin_c))
    np.testing.assert_array_equal(k_r[order], np.concatenate(lin_kr))
    # attention in ring order equals attention in frame order
    wl = w.with_(t_first=7)
    ref = orc.chunk_attention_reference(wl, wt, lambda t: xs[t])
    q_nope, q_rope = orc.queries(xs[7], wt["w_q"], orc.frame_positions(7, 2, 2), om,
                                 w.n_heads, w.d_nope, w.d_rope)
    kn, vv = orc.reconstruct_heads(c, wt["w_k_up"], wt["w_v_up"])
    ring_out = orc.attention_explicit(q_nope, q_rope, kn, k_r, vv, 1 / math.sqrt(128))
    assert rel(ring_out, ref) < 1e-13


def test_key_permutation_invariance():
    q_nope, q_rope, k_nope, k_r, v = _rand_heads(5, 40)
    perm = RNG.permutation(40)
    a = orc.attention_explicit(q_nope, q_rope, k_nope, k_r, v, 0.5)
    b = orc.attention_explicit(q_nope, q_rope, k_nope[perm], k_r[perm], v[perm], 0.5)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_reappend_overwrites_in_place():
    w = custom(1, 3, window_frames=2, chunk_frames=1, t_first=0, dtype="f32")
    wt = weights(w)
    om = orc.rope_frequencies()
    ring = orc.LatentRing(1, 2, 1, 3, w.d_c, w.d_rope)
    for step in range(3):
        ring.append_frame(0, 1, x_frame(w, 1, step=step), wt["w_down"], wt["w_kr"], om)
    c, _ = ring.valid(0, 2)
    cc, _ = orc.latent_entry(x_frame(w, 1, step=2), wt["w_down"], wt["w_kr"],
                             orc.frame_positions(1, 1, 3), om)
    np.testing.assert_array_equal(c[3:6], cc)
    assert np.isnan(c[:3]).all()            # frame 0 never written


def test_append_reference_rows_layout():
    w = custom(2, 3, window_frames=2, chunk_frames=2, t_first=4, dtype="f32")
    wt = weights(w)
    x = np.concatenate([x_frame(w, 4), x_frame(w, 5)])
    rows = orc.append_reference(w, wt, x, 4, 2)
    assert rows.shape == (12, 224)
    np.testing.assert_allclose(rows[:, :192], x.astype(np.float64) @ wt["w_down"], rtol=1e-13, atol=1e-13)
    kr = x.astype(np.float64) @ wt["w_kr"]
    pos = np.concatenate([orc.frame_positions(4, 2, 3), orc.frame_positions(5, 2, 3)])
    for i in range(12):
        np.testing.assert_allclose(rows[i, 192:], _rope_complex(kr[i], pos[i]), atol=1e-12)


# ---------------------------------------------------------------------------
# A whole clip under the chunk-causal block mask ([PL] App. D.4; §3
# "Integration with causal attention")
# ---------------------------------------------------------------------------

def test_chunk_causal_mask_hand_derived():
    # 7 frames in chunks of 3 (the last chunk is frame 6 alone), a 5-frame
    # window: chunk 0 sees frames 0-2; chunk 1 ends at frame 5 and sees 1-5;
    # chunk 2 ends at frame 6 and sees 2-6. Written out by hand.
    expect = {0: {0, 1, 2}, 1: {0, 1, 2}, 2: {0, 1, 2}, 3: {1, 2, 3, 4, 5},
              4: {1, 2, 3, 4, 5}, 5: {1, 2, 3, 4, 5}, 6: {2, 3, 4, 5, 6}}
    m = orc.chunk_causal_frame_mask(7, 3, 5)
    for fq, keys in expect.items():
        assert set(np.flatnonzero(m[fq]).tolist()) == keys
    # a window as long as the clip: block lower triangular, full diagonal blocks
    m = orc.chunk_causal_frame_mask(8, 2, 8)
    for fq in range(8):
        assert set(np.flatnonzero(m[fq]).tolist()) == set(range(2 * (fq // 2) + 2))
    # one-frame chunks and a full window: ordinary frame-causal masking
    assert np.array_equal(orc.chunk_causal_frame_mask(5, 1, 5), np.tril(np.ones((5, 5), bool)))


def test_masked_attention_matches_torch_sdpa_bool_mask():
    q_nope, q_rope, k_nope, k_r, v = _rand_heads(10, 13)
    H = q_nope.shape[1]
    d = q_nope.shape[2] + q_rope.shape[2]
    allowed = RNG.random((10, 13)) < 0.4
    allowed[np.arange(10), RNG.integers(0, 13, 10)] = True     # every row keeps a key
    out = orc.masked_attention(q_nope, q_rope, k_nope, k_r, v, 1.0 / math.sqrt(d), allowed)
    Q = torch.from_numpy(np.concatenate([q_nope, q_rope], -1)).permute(1, 0, 2)[None]
    K = torch.from_numpy(np.concatenate([k_nope, np.repeat(k_r[:, None], H, 1)], -1)).permute(1, 0, 2)[None]
    V = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(allowed))
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def _clip_rows_equal_rollout(F, C, W):
    # The block mask gives chunk c the frames the rolling cache holds once c is
    # appended, so its rows equal the chunk step at t_first = c C ([PL] App. D.4).
    w = custom(2, 3, window_frames=W, chunk_frames=C, t_first=0, dtype="f32")
    wt = weights(w)
    xs = {t: x_frame(w, t) for t in range(F)}
    clip = orc.clip_chunk_causal_reference(w, wt, lambda t: xs[t], F, W)
    T = w.tokens_per_frame
    for c0 in range(0, F, C):
        n = min(C, F - c0)
        step = orc.chunk_attention_reference(w.with_(t_first=c0, chunk_frames=n), wt, lambda t: xs[t])
        assert rel(clip[c0 * T:(c0 + n) * T], step) < 1e-12


def test_clip_chunk_rows_equal_rollout_steps():
    for F, C, W in [(7, 3, 5), (6, 6, 6), (5, 1, 5), (7, 3, 7), (8, 2, 3)]:
        _clip_rows_equal_rollout(F, C, W)


def test_clip_chunk_causal_brute_force_tiny():
    # Tiny dims. The keys each chunk may see come from a simulated FIFO of W
    # frames filled chunk by chunk (the cache right after the chunk is
    # appended); every sum is a scalar loop.
    from collections import deque
    F, C, W, gh, gw = 5, 2, 3, 1, 2
    T = gh * gw
    D, H, dn, dr, dc, dv = 3, 2, 2, 4, 3, 2
    pairs, dims = (1, 1, 0), (2, 2, 2)
    w = custom(gh, gw, window_frames=W, chunk_frames=C, t_first=0, dtype="f32").with_(
        d_model=D, n_heads=H, d_nope=dn, d_rope=dr, d_c=dc, d_v=dv, rope_pairs=pairs,
        rope_axis_dims=dims)
    om = orc.rope_frequencies(pairs, dims)
    wt = {"w_q": RNG.standard_normal((D, H * (dn + dr))), "w_down": RNG.standard_normal((D, dc)),
          "w_kr": RNG.standard_normal((D, dr)), "w_k_up": RNG.standard_normal((H, dc, dn)),
          "w_v_up": RNG.standard_normal((H, dc, dv))}
    xs = RNG.standard_normal((F, T, D))
    fifo, visible = deque(maxlen=W), {}
    for c0 in range(0, F, C):
        for f in range(c0, min(c0 + C, F)):
            fifo.append(f)
        for f in range(c0, min(c0 + C, F)):
            visible[f] = list(fifo)
    scale = 1 / math.sqrt(dn + dr)

    def mv(x, W_, j):
        return sum(x[i] * W_[i][j] for i in range(len(x)))

    def rot(vec, p):
        o = list(vec)
        for j in range(2):
            ang = p[j] * om[j]
            a, b = vec[2 * j], vec[2 * j + 1]
            o[2 * j] = a * math.cos(ang) - b * math.sin(ang)
            o[2 * j + 1] = a * math.sin(ang) + b * math.cos(ang)
        return o

    def position(f, n):
        return (f, n // gw, n % gw)

    ref = np.zeros((F * T, H, dv))
    for qi in range(F * T):
        fq, nq = divmod(qi, T)
        qfull = [mv(xs[fq][nq], wt["w_q"], j) for j in range(H * (dn + dr))]
        for h in range(H):
            qn = qfull[h * (dn + dr):h * (dn + dr) + dn]
            qr = rot(qfull[h * (dn + dr) + dn:(h + 1) * (dn + dr)], position(fq, nq))
            s, vals = [], []
            for fk in visible[fq]:
                for nk in range(T):
                    c = [mv(xs[fk][nk], wt["w_down"], j) for j in range(dc)]
                    kr = rot([mv(xs[fk][nk], wt["w_kr"], j) for j in range(dr)], position(fk, nk))
                    kn = [sum(c[i] * wt["w_k_up"][h][i][j] for i in range(dc)) for j in range(dn)]
                    vals.append([sum(c[i] * wt["w_v_up"][h][i][j] for i in range(dc)) for j in range(dv)])
                    s.append(scale * (sum(qn[j] * kn[j] for j in range(dn)) +
                                      sum(qr[j] * kr[j] for j in range(dr))))
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for j in range(dv):
                ref[qi, h, j] = sum(e[k] / z * vals[k][j] for k in range(len(e)))

    out = orc.clip_chunk_causal_reference(w, wt, lambda t: xs[t], F, W)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Planted mistakes: every one of them must trip at least one pin
# ---------------------------------------------------------------------------

def _wrong_sign_rope(v, pos, omega, pairs=(6, 5, 5)):
    v = np.asarray(v, dtype=np.float64)
    phi = np.asarray(pos, dtype=np.float64)[..., orc.rope_pair_axes(pairs)] * omega
    out = np.empty(np.broadcast_shapes(v.shape, phi.shape[:-1] + (v.shape[-1],)))
    a, b = v[..., 0::2], v[..., 1::2]
    out[..., 0::2] = a * np.cos(phi) + b * np.sin(phi)
    out[..., 1::2] = -a * np.sin(phi) + b * np.cos(phi)
    return out


def _attention_no_rope_term(q_nope, q_rope, k_nope, k_r, v, scale, row_block=256):
    return _ORIG_ATT(q_nope, 0 * q_rope, k_nope, k_r, v, scale, row_block)


def _attention_wrong_scale(q_nope, q_rope, k_nope, k_r, v, scale, row_block=256):
    return _ORIG_ATT(q_nope, q_rope, k_nope, k_r, v, scale * math.sqrt(2.0), row_block)


def _reconstruct_transposed_value(c, w_k_up, w_v_up):
    k, v = _ORIG_REC(c, w_k_up, w_v_up)
    return k, v[:, ::-1, :]          # heads' values swapped


def _positions_hw_swapped(t, grid_h, grid_w):
    p = _ORIG_POS(t, grid_h, grid_w)
    return p[:, [0, 2, 1]]


def _context_absolute(t_first, chunk_frames, window, sink):
    return [(t, t) for t, _ in _ORIG_CTX(t_first, chunk_frames, window, sink)]


def _context_without_sink(t_first, chunk_frames, window, sink):
    return [(t, i) for i, (t, _) in enumerate(
        [c for c in _ORIG_CTX(t_first, chunk_frames, window, sink) if c[0] >= sink])]


def _mixer_head_minor(o, w_o):
    o = np.asarray(o, dtype=np.float64)
    return o.transpose(0, 2, 1).reshape(o.shape[0], -1) @ np.asarray(w_o, dtype=np.float64)


def _mixer_transposed(o, w_o):
    # a square W_O (H d_v = d_model, as in the real layer) read transposed
    o = np.asarray(o, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    return o.reshape(o.shape[0], -1) @ (w_o.T if w_o.shape[0] == w_o.shape[1] else w_o)


def _fold_query_rope_from_nope(w_uq, w_k_up, n_heads, d_nope, d_rope):
    w3 = np.asarray(w_uq, dtype=np.float64).reshape(-1, n_heads, d_nope + d_rope)
    return np.concatenate([np.concatenate([w3[:, h, :d_nope] @ np.asarray(w_k_up[h]).T,
                                           w3[:, h, :d_rope]], axis=1)
                           for h in range(n_heads)], axis=1)


def _fold_output_wrong_head(w_v_up, w_o):
    d_v, H = w_v_up.shape[2], w_v_up.shape[0]
    return np.concatenate([np.asarray(w_v_up[h]) @ np.asarray(w_o)[(H - 1 - h) * d_v:(H - h) * d_v]
                           for h in range(H)], axis=0)


def _mask_frame_causal(n_frames, chunk_frames, window):
    f = np.arange(n_frames)
    end = np.minimum((f // chunk_frames + 1) * chunk_frames, n_frames)
    return (f[None, :] <= f[:, None]) & (f[None, :] >= end[:, None] - window)


def _mask_window_from_chunk_start(n_frames, chunk_frames, window):
    f = np.arange(n_frames)
    start = (f // chunk_frames) * chunk_frames
    end = np.minimum(start + chunk_frames, n_frames)
    return (f[None, :] < end[:, None]) & (f[None, :] >= start[:, None] - window)


def _mask_without_window(n_frames, chunk_frames, window):
    return _ORIG_MASK(n_frames, chunk_frames, n_frames)


def _masked_attention_weights_not_renormalised(q_nope, q_rope, k_nope, k_r, v, scale, allowed,
                                               row_block=256):
    nq, nh, _ = q_nope.shape
    out = np.empty((nq, nh, v.shape[-1]))
    for h in range(nh):
        kh = np.concatenate([k_nope[:, h, :], k_r], axis=1)
        qh = np.concatenate([q_nope[:, h, :], q_rope[:, h, :]], axis=1)
        out[:, h, :] = (orc.softmax_rows((qh @ kh.T) * scale) * allowed) @ v[:, h, :]
    return out


def _rope_frequencies_no_factor_two(pairs=(6, 5, 5), axis_dims=(12, 10, 10), theta=10000.0):
    # theta^(-i / D_a): the exponent misses its factor 2
    return np.array([float(theta) ** (-i / d) for n, d in zip(pairs, axis_dims) for i in range(n)])


def _rope_frequencies_width_is_pair_count(pairs=(6, 5, 5), axis_dims=(12, 10, 10), theta=10000.0):
    # D_a taken as the group's pair count instead of its channel width
    return np.array([float(theta) ** (-2.0 * i / n) for n in pairs for i in range(n)])


_ORIG_CTX = orc.active_context
_ORIG_MASK = orc.chunk_causal_frame_mask
_ORIG_ATT = orc.attention_explicit
_ORIG_REC = orc.reconstruct_heads
_ORIG_POS = orc.frame_positions

PINS = [test_rope_is_complex_rotation, test_rope_frequency_law_matches_standard_rope_per_axis,
        test_attention_matches_torch_sdpa_fp64,
        test_mla_reduces_to_dense_mha_with_selection_up_projections,
        test_mla_equals_dense_mha_with_composed_weights_real_dims,
        test_oracle_at_wan_geometry_equals_dense_mha_with_composed_weights,
        test_brute_force_scalar_loops_tiny, test_append_reference_rows_layout,
        test_frame_positions_token_order, test_absorbed_equals_explicit,
        test_reindexed_sink_context_brute_force_tiny,
        test_layer_with_identity_query_latent_and_mixer_is_the_attention_reference,
        test_layer_folded_latent_form_equals_explicit, test_layer_brute_force_scalar_loops_tiny,
        test_chunk_causal_mask_hand_derived, test_masked_attention_matches_torch_sdpa_bool_mask,
        test_clip_chunk_rows_equal_rollout_steps, test_clip_chunk_causal_brute_force_tiny]


@pytest.mark.parametrize("name,patch", [
    ("rope rotation sign", ("rope3d", _wrong_sign_rope)),
    ("dropped positional score term", ("attention_explicit", _attention_no_rope_term)),
    ("wrong softmax scale", ("attention_explicit", _attention_wrong_scale)),
    ("values of the wrong head", ("reconstruct_heads", _reconstruct_transposed_value)),
    ("h and w swapped in positions", ("frame_positions", _positions_hw_swapped)),
    ("window frames not re-indexed", ("active_context", _context_absolute)),
    ("sink evicted with the window", ("active_context", _context_without_sink)),
    ("head outputs mixed head-minor", ("output_mixer", _mixer_head_minor)),
    ("output mixer transposed", ("output_mixer", _mixer_transposed)),
    ("A_h fold takes rope columns from the nope block", ("fold_query_weights", _fold_query_rope_from_nope)),
    ("B_h folded with another head's W_O rows", ("fold_output_weights", _fold_output_wrong_head)),
    ("frame-causal instead of chunk-causal", ("chunk_causal_frame_mask", _mask_frame_causal)),
    ("window counted from the chunk start", ("chunk_causal_frame_mask", _mask_window_from_chunk_start)),
    ("window ignored", ("chunk_causal_frame_mask", _mask_without_window)),
    ("masked weights not renormalised", ("masked_attention", _masked_attention_weights_not_renormalised)),
    ("RoPE exponent without its factor 2", ("rope_frequencies", _rope_frequencies_no_factor_two)),
    ("RoPE axis width taken as the pair count", ("rope_frequencies", _rope_frequencies_width_is_pair_count)),
])
def test_planted_mistake_is_caught(monkeypatch, name, patch):
    attr, fn = patch
    monkeypatch.setattr(orc, attr, fn)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin catches: {name}"
