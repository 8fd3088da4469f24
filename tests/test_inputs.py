"""The seeded input generator: splitmix64 against its published reference values, the normal
distribution, bf16 rounding, determinism and the workload shapes."""
import math

import numpy as np
import pytest
import scipy.stats
import torch

import moe_inputs as mi


def test_splitmix64_published_vectors():
    # Reference outputs of splitmix64 (Steele, Lea, Flood 2014; Vigna's splitmix64.c) for seeds 1234567 and 0.
    assert mi.splitmix64_seq(1234567, 5).tolist() == [6457827717110365317, 3203168211198807973,
                                                       9817491932198370423, 4593380528125082431,
                                                       16408922859458223821]
    assert mi.splitmix64_seq(0, 3).tolist() == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_streams_deterministic_and_distinct():
    a = mi.raw_u64(7, 1, 1000)
    assert (a == mi.raw_u64(7, 1, 1000)).all()
    assert not (a == mi.raw_u64(7, 2, 1000)).any()
    assert not (a == mi.raw_u64(8, 1, 1000)).any()
    # counter-based: a prefix of a longer draw is the shorter draw
    assert (mi.normal_f32(3, 5, (10,)) == mi.normal_f32(3, 5, (100,))[:10]).all()


def test_normal_distribution():
    z = mi.normal_f32(11, 3, (200000,)).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1.0) < 0.01
    assert scipy.stats.kstest(z, "norm").pvalue > 1e-3
    s = mi.normal_f32(11, 4, (200000,), 0.0, 1.0 / 8.0).astype(np.float64)
    assert abs(s.std() - 0.125) < 0.002


def test_bf16_is_rne_of_fp32():
    f = mi.normal_f32(5, 9, (50000,))
    b = mi.normal_bf16(5, 9, (50000,))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (b == ref).all()
    assert (mi.bf16_bits_to_f32(b) == torch.from_numpy(f).to(torch.bfloat16).float().numpy()).all()


@pytest.mark.parametrize("name", mi.CONFIG_NAMES)
def test_config_shapes(name):
    s = mi.spec(name)
    assert s.G % s.E_l == 0 and s.k <= s.G and s.d % 64 == 0 and s.f % 64 == 0 and s.M % 16 == 0
    lg = mi.logits(mi.spec(name, T_o=4)) if s.T_o > 4 else mi.logits(s)
    assert lg.dtype == np.float32 and lg.shape[1] == s.G


def test_zipf_bias_placement():
    s = mi.spec("skew")
    b = mi.expert_bias(s)
    # popularity rank q(e) = (e mod E_l) * R + e // E_l: expert 0 is hottest, local experts are spread
    assert b[0] == 0.0
    assert math.isclose(b[1], -1.2 * math.log(5.0))
    assert math.isclose(b[s.E_l], -1.2 * math.log(2.0))
    assert np.argsort(-b, kind="stable")[:4].tolist() == [0, 16, 32, 48]
