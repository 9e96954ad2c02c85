"""The algorithmic work bench.py reports, checked against counts written out
by hand (CPU only): flops per (query, key, head) of the absorbed form are
2 (d_c + d_rope) for the scores plus 2 d_c for P c; the explicit route's are
2 x 128 + 2 x 128; the chunk-causal clip sums each chunk's own key range."""
import bench
from workloads import config, split_variant


def test_chunk_step_work_config2():
    w = config(2)
    wk = bench.work(w)
    assert wk["core"] == 832 * 4680 * 32760 * 12
    assert wk["epilogue"] == 4680 * 12 * 2 * 192 * 128
    assert wk["prologue"] == 4680 * (2 * 1536 * 12 * 128 + 12 * 2 * 96 * 192)
    assert wk["append"] == 4680 * 2 * 1536 * 224
    assert wk["attn_kernel"] == 1533475307520                 # the roofline's flops per launch
    # bytes of the append: x read, weights read, cache rows written
    assert wk["bytes_append"] == 4680 * 1536 * 2 + 1536 * 224 * 2 + 4680 * 448


def test_explicit_route_work_config2():
    wk = bench.work(config(2), explicit=True)
    assert wk["core"] == (2 * 128 + 2 * 128) * 4680 * 32760 * 12
    # queries x W_Q plus the per-head K/V rebuild of every valid slot
    assert wk["prologue"] == 4680 * 2 * 1536 * 12 * 128 + 32760 * 2 * 192 * 12 * (96 + 128)


def test_split_and_width_variants_work():
    for d_rope in (16, 64, 96):
        wk = bench.work(split_variant(config(2), d_rope))
        assert wk["core"] == (2 * (192 + d_rope) + 2 * 192) * 4680 * 32760 * 12
    for d_c in (64, 512):
        wk = bench.work(config(2).with_(d_c=d_c))
        assert wk["core"] == (2 * (d_c + 32) + 2 * d_c) * 4680 * 32760 * 12


def test_chunk_causal_clip_work():
    w = config(2).with_(window_frames=21, chunk_frames=3, t_first=0)
    wk = bench.clip_work(w, 21, 21)
    assert wk["core"] == 832 * 4680 * 4680 * 12 * (1 + 2 + 3 + 4 + 5 + 6 + 7)
    # a 6-frame window: chunk 0 sees 3 frames, every later chunk 6
    wk6 = bench.clip_work(w, 21, 6)
    assert wk6["core"] == 832 * 4680 * 1560 * 12 * (3 + 6 * 6)
    # 20 frames: the last chunk has 2 frames and sees 20 (window = clip)
    wk20 = bench.clip_work(w, 20, 20)
    per_q_key = 832 * 12
    assert wk20["core"] == per_q_key * (sum(4680 * 4680 * (c + 1) for c in range(6)) + 3120 * 20 * 1560)
    # the sampled rows of the CPU baseline: the last chunk only
    assert bench.clip_work(w, 21, 21, rows=[6])["core"] == 832 * 4680 * 32760 * 12
