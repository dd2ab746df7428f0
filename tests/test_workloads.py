"""The seeded input generators: chunked / per-expert weight draws equal the full draw."""
import numpy as np

from workloads import CONFIGS, expert_weights, iter_expert_weights, make_workload, small_case


def test_chunked_weight_draw_equals_full_draw():
    wl = small_case([3, 0, 40, 7, 1], 64, 32, seed=11)
    cfg = wl.config
    got1, got2 = [], []
    for idx, a, b in iter_expert_weights(cfg, 11, chunk=2, threads=3):
        assert idx == list(range(idx[0], idx[0] + len(idx)))
        got1.append(a)
        got2.append(b)
    assert np.array_equal(np.concatenate(got1), wl.w1) and np.array_equal(np.concatenate(got2), wl.w2)
    a, b = expert_weights(cfg, 11, [3])
    assert np.array_equal(a[0], wl.w1[3]) and np.array_equal(b[0], wl.w2[3])


def test_config_shapes_and_splits():
    for name, rows in (("tiny", 192), ("mid", 32768), ("nvfp4", 24576), ("zipf", 49152), ("large", 65536)):
        wl = make_workload(CONFIGS[name], with_weights=False) if name != "tiny" else make_workload("tiny")
        assert int(wl.m_splits.sum()) == rows and wl.x.shape == (rows, CONFIGS[name].hidden)
        assert wl.probs.shape == (rows,) and wl.probs.dtype == np.float32
    assert make_workload("tiny").m_splits.tolist() == [64, 128]
    assert (make_workload(CONFIGS["zipf"], with_weights=False).m_splits == 0).sum() == 4
