"""The closed-form capacity model against the figures the pages print."""
import pytest

from latent_kv_attention_cache_amd import capacity as cap


def test_scalars_per_token_match_the_pages():
    # [PL] App. D.2: 224 cached scalars per token per layer against 3072
    assert cap.latent_scalars_per_token() == 224
    assert cap.dense_scalars_per_token() == 3072


def test_dense_window_matches_the_printed_scalar_count():
    # 21 frames x 1560 tokens x 30 layers x 3072 scalars = 3.02 B scalars ([PL] §3),
    # about 6.0 GB in bf16
    b = cap.cache_bytes_per_request(cap.dense_scalars_per_token())
    assert b == 2 * 3_019_161_600
    assert abs(b / cap.GB - 6.04) < 0.01


def test_measured_slopes_exceed_the_cache_by_a_similar_residual():
    # [PL] §4 "Batch Scaling Under Fixed Memory": 6.26 GB per request (dense) and
    # 0.57 / 1.43 GB per request at d_c = 64 / 512. The model's cache-only slope
    # sits below every measured one, and the residual (per-request activations
    # the pages do not itemise) is a few hundred MB in each case.
    measured = {"mha": 6.26, 64: 0.57, 512: 1.43}
    model = {"mha": cap.cache_bytes_per_request(3072) / cap.GB,
             64: cap.cache_bytes_per_request(cap.latent_scalars_per_token(64)) / cap.GB,
             512: cap.cache_bytes_per_request(cap.latent_scalars_per_token(512)) / cap.GB}
    for k in measured:
        residual = measured[k] - model[k]
        assert 0.1 < residual < 0.45, (k, residual)
    # the pages' 77-91 % reduction of the slope follows from their own numbers
    assert round(100 * (1 - 1.43 / 6.26)) == 77 and round(100 * (1 - 0.57 / 6.26)) == 91


def test_max_batch_and_sweep():
    assert cap.max_batch(100.0, 30.0) == 3
    assert cap.max_batch(100.0, 30.0, fixed_bytes=20.0) == 2
    assert cap.max_batch(10.0, 30.0) == 0
    with pytest.raises(ValueError):
        cap.max_batch(1.0, 0.0)
    s = cap.sweep(budget_bytes=288 * cap.GB)
    assert s["mha"]["max_batch"] == 47                  # 288 GB / 6.04 GB
    assert s["d_c=192"]["max_batch"] == 654             # 288 GB / 0.440 GB
    assert s["d_c=64"]["cache_bytes"] < s["d_c=192"]["cache_bytes"] < s["d_c=512"]["cache_bytes"]
    # a sink frame adds one frame of slots per layer
    assert cap.cache_bytes_per_request(224, frames=6, sink_frames=1) == 30 * 7 * 1560 * 224 * 2


def test_one_budget_reproduces_the_pages_batch_limits():
    # [PL] §4 "Batch Scaling Under Fixed Memory": dense MHA reaches the memory
    # limit at B = 28; d_c = 64 stays within budget at B = 320; 4.6x to at
    # least 11.4x larger batches (8.0x at d_c = 192, [PL] "Key results").
    # Reading: B = 28 is the largest dense batch that fits. Per request the
    # model holds its closed-form cache plus one common overhead taken from the
    # pages' slopes; the dense limit then fixes a budget window.
    r = cap.overhead_from_slopes()
    assert 0.25 * cap.GB < r < 0.40 * cap.GB            # ~0.32 GB of activations per request
    mha = cap.cache_bytes_per_request(cap.dense_scalars_per_token()) + r
    lo, hi = cap.budget_window(28, mha)
    assert 178.0 * cap.GB < lo < 178.1 * cap.GB and 184.4 * cap.GB < hi < 184.5 * cap.GB
    for budget in (lo + 1, 180 * cap.GB, hi - 1):
        s = cap.sweep(budget_bytes=budget, overhead_per_request=r)
        b = {k: v["max_batch"] for k, v in s.items()}
        assert b["mha"] == 28                           # a 29th dense request runs out of memory
        assert b["d_c=64"] >= 320                       # d_c = 64 still fits at B = 320
        assert b["d_c=64"] / b["mha"] >= 11.4
        assert round(b["d_c=512"] / b["mha"], 1) in (4.6, 4.7)   # the low end, 4.6x
        assert 7.5 < b["d_c=192"] / b["mha"] < 8.7      # 8.0x at the default width
    # at 180 GB: 28 dense requests against 352 / 236 / 129 at d_c = 64 / 192 / 512
    s = cap.sweep(budget_bytes=180 * cap.GB, overhead_per_request=r)
    assert [s[k]["max_batch"] for k in ("mha", "d_c=64", "d_c=192", "d_c=512")] == [28, 352, 236, 129]
