"""The seeded input generator: determinism, chunk independence and the shapes and
statistics of the synthetic LLaMA-shaped layers."""
import numpy as np

from gen import synth


def test_counter_based_slices_agree():
    a = synth.u64(1001, 1, 0, 5000)
    b = np.concatenate([synth.u64(1001, 1, 0, 1234), synth.u64(1001, 1, 1234, 3766)])
    assert np.array_equal(a, b)
    assert not np.array_equal(synth.u64(1001, 1, 0, 100), synth.u64(1001, 2, 0, 100))
    n = synth.normal(5, 1, 10001)
    assert np.array_equal(n[3:9], synth._normal_chunk(5, 1, 3, 6))


def test_normal_and_t_moments():
    z = synth.normal(3, 1, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    t = synth.student_t3(3, 1, 6, 1 << 20)
    # Student-t(3): median 0, interquartile range 2 * 0.7649
    q1, q3 = np.percentile(t, [25, 75])
    assert abs(q3 - q1 - 1.5298) < 0.02


def test_configs_table():
    c = synth.CONFIGS
    assert (c["tiny"].M, c["tiny"].K, c["tiny"].N, c["tiny"].nb8) == (16, 512, 512, 1)
    assert (c["q_proj_7b"].nb, c["q_proj_7b"].nb8) == (32, 4)
    assert (c["down_7b"].nb, c["down_7b"].nb8) == (86, 22)
    assert (c["prefill_down_70b"].nb, c["prefill_down_70b"].nb8) == (224, 67)
    assert (c["prefill_up_70b"].nb, c["prefill_up_70b"].nb8) == (64, 7)
    assert c["decode_70b_n28672_m16"].nb8 == 7
    for cfg in c.values():
        assert cfg.K % 128 == 0 and cfg.N % 128 == 0 and 0 <= cfg.nb8 <= cfg.nb


def test_layer_draw_is_deterministic_and_shaped():
    cfg = synth.CONFIGS["tiny"]
    a, b = synth.make_layer(cfg), synth.make_layer(cfg)
    for k in ("X", "W", "score"):
        assert np.array_equal(a[k], b[k])
    assert a["X"].shape == (16, 512) and a["X"].dtype == np.uint16
    assert a["W"].shape == (512, 512)
    w = synth.fp16_bits_to_f32(a["W"])
    assert abs(w.std() - 0.02) < 1e-3
    ch, mu = synth.outlier_plan(cfg)
    assert len(ch) == 51 and len(set(ch.tolist())) == 51 and np.all(mu == 50)
    # the planted channels carry the largest calibration scores
    top = np.argsort(-a["score"], kind="stable")[:51]
    assert set(top.tolist()) == set(ch.tolist())


def test_first_rows_match_full_draw():
    cfg = synth.CONFIGS["q_proj_7b"]
    assert np.array_equal(synth.make_x(cfg, rows=8), synth.make_x(cfg)[:8])
