"""The seeded input generator: determinism, ranges and bf16 rounding."""
import numpy as np
import torch

from rnnt_inputs import WORKLOADS, make_inputs, poison_padding, round_bf16, workload_inputs


def test_deterministic_per_seed():
    a = workload_inputs("small-bf16")
    b = workload_inputs("small-bf16")
    c = workload_inputs("small-bf16", seed=99)
    for k in ("T_len", "U_len", "labels", "hA", "hL", "WA", "WL", "WO"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert not np.array_equal(a.hA, c.hA)


def test_length_and_label_ranges():
    for cfg in ("small-bf16", "20s-bf16", "vocab4096-bf16"):
        w = WORKLOADS[cfg]
        inp = workload_inputs(cfg)
        assert inp.T_len.min() >= w.t_range[0] and inp.T_len.max() <= w.t_range[1]
        assert inp.U_len.min() >= w.u_range[0] and inp.U_len.max() <= w.u_range[1]
        assert np.all(inp.labels[:, 0] == 0)
        for b in range(w.B):
            lab = inp.labels[b, 1:inp.U_len[b] + 1]
            assert lab.min() >= 1 and lab.max() <= w.V - 1
            assert np.all(inp.labels[b, inp.U_len[b] + 1:] == 0)
    assert WORKLOADS["20s-bf16"].t_range == (300, 500) and WORKLOADS["20s-bf16"].u_range == (72, 120)
    assert WORKLOADS["40s-b256-bf16"].t_range == (500, 1000) and WORKLOADS["40s-b256-bf16"].u_range == (100, 200)


def test_zipf_labels_are_skewed():
    inp = workload_inputs("vocab4096-bf16")
    lab = np.concatenate([inp.labels[b, 1:inp.U_len[b] + 1] for b in range(16)])
    # P(1) / P(2) = 2^1.1 for Zipf(1.1); id 1 is by far the most frequent
    c1, c2 = np.sum(lab == 1), np.sum(lab == 2)
    assert c1 > c2 > 0 and c1 > 0.05 * len(lab)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 3, 100000).astype(np.float32)
    # exact ties: bf16 value + half an ulp
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32) * 1.0
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16(x), ref)


def test_bf16_values_are_representable():
    inp = workload_inputs("small-bf16")
    for k in ("hA", "hL", "WA", "WL", "WO"):
        v = getattr(inp, k)
        assert np.array_equal(v, round_bf16(v))


def test_xavier_bounds():
    inp = make_inputs(1, 4, 2, 1024, 512, 512, 640, dtype="f32", seed=1)
    assert np.abs(inp.WO).max() <= np.sqrt(6 / (640 + 1024))
    assert np.abs(inp.WA).max() <= np.sqrt(6 / (512 + 640))


def test_poison_padding_touches_only_padding():
    inp = make_inputs(3, 8, 4, 9, 4, 4, 4, seed=5, t_range=(2, 8), u_range=(0, 4))
    p = poison_padding(inp)
    for b in range(3):
        Tb, U1 = inp.T_len[b], inp.U_len[b] + 1
        assert np.array_equal(p.hA[b, :Tb], inp.hA[b, :Tb]) and np.all(np.isnan(p.hA[b, Tb:]))
        assert np.array_equal(p.hL[b, :U1], inp.hL[b, :U1]) and np.all(np.isnan(p.hL[b, U1:]))
        assert np.array_equal(p.labels[b, :U1], inp.labels[b, :U1])
