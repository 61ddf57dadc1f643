"""The seeded input generator (no GPU)."""

import hashlib
import json
import os

import numpy as np
import pytest

from causal_flash_attention_amd import inputs as I
from causal_flash_attention_amd.workloads import BY_NAME, WORKLOADS

HERE = os.path.dirname(os.path.abspath(__file__))


def test_deterministic_and_thread_invariant():
    shape = (3, 700_001)  # spans several chunks with a ragged tail
    a = I.normal(shape, 1.0, 0, 0, "bf16", threads=1)
    b = I.normal(shape, 1.0, 0, 0, "bf16", threads=7)
    assert a.dtype == np.uint16 and a.shape == shape
    assert np.array_equal(a, b)
    f1 = I.normal(shape, 0.5, 3, 1, "f32", threads=1)
    f2 = I.normal(shape, 0.5, 3, 1, "f32", threads=5)
    assert f1.dtype == np.float32 and np.array_equal(f1, f2)


def test_bf16_is_rounded_f32():
    f = I.normal((5000,), 1.0, 0, 0, "f32")
    b = I.normal((5000,), 1.0, 0, 0, "bf16")
    assert np.array_equal(I.f32_to_bf16_bits(f), b)


def test_streams_and_seeds_differ():
    a = I.normal((4096,), 1.0, 0, 0, "f32")
    b = I.normal((4096,), 1.0, 0, 1, "f32")
    c = I.normal((4096,), 1.0, 1, 0, "f32")
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    # independent draws: sample correlation near 0
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.06


def test_prefix_stability():
    # element i does not depend on the total size (chunks are keyed by index)
    small = I.normal((1000,), 1.0, 0, 0, "f32")
    big = I.normal((I.CHUNK + 10,), 1.0, 0, 0, "f32")
    assert np.array_equal(small, big[:1000])


@pytest.mark.parametrize("std", [1.0, 0.01])
def test_moments(std):
    x = I.to_float64(I.normal((2_000_000,), std, 0, 0, "f32"), "f32") / std
    n = x.size
    assert abs(x.mean()) < 5 / np.sqrt(n)
    assert abs(x.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    # fraction inside one standard deviation of a normal: erf(1/sqrt 2)
    frac = np.mean(np.abs(x) < 1.0)
    assert abs(frac - 0.6826894921370859) < 5 * np.sqrt(0.6827 * 0.3173 / n)


def test_bf16_round_to_nearest_even():
    u = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF,
                  0xBF808000, 0x7F7FFFFF, 0x7FC00001, 0x00008000, 0x00018000],
                 dtype=np.uint32)
    got = I.f32_to_bf16_bits(u.view(np.float32))
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x3F80,
            0xBF80, 0x7F80, 0x7FC0, 0x0000, 0x0002]
    assert [int(x) for x in got] == want
    # widening is exact
    back = I.bf16_bits_to_f32(np.array([0x3F82, 0xC0A0], dtype=np.uint16))
    assert back.tolist() == [1.015625, -5.0]


def test_checksums_frozen():
    with open(os.path.join(HERE, "golden", "input_checksums.json")) as f:
        want = json.load(f)
    assert "tiny_f32_b1_h2_t64" in want
    for name, d in want.items():
        w = BY_NAME[name]
        qkv, dout = I.attention_inputs(w.B, w.T, w.n_head, w.head_dim, w.dtype,
                                       w.qkv_std, w.dout_std, seed=0)
        assert hashlib.sha256(qkv.tobytes()).hexdigest() == d["qkv"], name
        assert hashlib.sha256(dout.tobytes()).hexdigest() == d["dout"], name


def test_workloads_table():
    assert [w.name for w in WORKLOADS][0] == "tiny_f32_b1_h2_t64"
    w = BY_NAME["gpt2_124m_b16_t1024"]
    assert (w.B, w.T, w.n_head, w.head_dim, w.C) == (16, 1024, 12, 64, 768)
    assert w.counted_flops()["total"] == pytest.approx(90.19e9, rel=1e-3)
