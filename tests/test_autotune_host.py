"""The autotuner's table-writing logic on recorded timings (no GPU)."""
from dense_gemm_12_amd import autotune


def _line(n, cfg):
    import gemm_inputs as gi
    w = gi.WORKLOADS[n]
    return f"{w['in_dtype']} {w['c_dtype']} {w['ta']} {w['tb']} {w['M']} {w['N']} {w['K']} {cfg}"


def _run(picks):
    lines = [_line(n, r[0][1]) for n, _, r in picks]
    out = autotune._prefer_consistent(lines, picks, log=lambda s: None)
    return [l.split()[7] for l in out]


W4, W2 = "dma_f16_256x256x64_s2_w2x4", "dma_f16_256x256x64_s2_w2x2"
S3 = "dma_f16_128x128x64_s3_w2x2"


def test_near_tie_does_not_follow_a_peer_that_was_itself_a_near_tie():
    # 4096 picks w2x2 by 0.2 %, 8192 picks w2x4 by 1.7 %: neither pick is
    # decisive, so neither may pull the other across.
    picks = [("fp16_tn_2048", "", [(0.0250, S3, 0), (0.0292, W2, 0)]),
             ("fp16_tn_4096", "", [(0.1137, W2, 0), (0.1139, W4, 0)]),
             ("fp16_tn_8192", "", [(0.8543, W4, 0), (0.8692, W2, 0)]),
             ("fp16_tn_16384", "", [(7.036, W4, 0), (7.642, W2, 0)])]
    assert _run(picks) == [S3, W2, W4, W4]


def test_near_tie_follows_agreeing_decisive_peers():
    # 8192 is a near-tie whose runner-up is what both equally near decisive
    # peers (4096 and 16384) chose.
    picks = [("fp16_tn_4096", "", [(0.113, W4, 0), (0.120, W2, 0)]),
             ("fp16_tn_8192", "", [(0.854, W2, 0), (0.858, W4, 0)]),
             ("fp16_tn_16384", "", [(7.04, W4, 0), (7.64, W2, 0)])]
    assert _run(picks) == [W4, W4, W4]


def test_near_tie_kept_when_nearest_decisive_peers_disagree():
    picks = [("fp16_tn_4096", "", [(0.113, S3, 0), (0.120, W2, 0)]),
             ("fp16_tn_8192", "", [(0.854, W2, 0), (0.858, W4, 0)]),
             ("fp16_tn_16384", "", [(7.04, W4, 0), (7.64, W2, 0)])]
    assert _run(picks) == [S3, W2, W4]


def test_runner_up_with_other_split_count_is_not_taken():
    picks = [("fp16_tn_4096", "", [(0.113, W4, 0), (0.120, W2, 0)]),
             ("fp16_tn_8192", "", [(0.854, W2, 0), (0.858, W4, 8)])]
    assert _run(picks) == [W4, W2]
