"""The bf16 comparison helper: contract tolerance, storage floor and its
one-ulp allowance (checked on synthetic data, no GPU)."""
import numpy as np
import pytest

from synthetic import bf16_round_f32
from tests._helpers import assert_close_bf16, bf16_storage_floor, bf16_ulp


def test_ulp_values():
    assert bf16_ulp(1.0) == 2.0 ** -7
    assert bf16_ulp(1.5) == 2.0 ** -7
    assert bf16_ulp(-3.0) == 2.0 ** -6
    assert bf16_ulp(0.25) == 2.0 ** -9


def test_perfectly_rounded_outputs_pass_even_when_heavy_tailed():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(10000) * rng.standard_normal(10000) ** 3   # heavy tail
    assert bf16_storage_floor(ref) > 1e-2
    assert_close_bf16(bf16_round_f32(ref.astype(np.float32)), ref)


def test_wrong_results_fail():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal(10000)
    bad = ref.copy()
    bad[17] += 0.05 * np.sqrt(np.mean(ref ** 2))
    with pytest.raises(AssertionError):
        assert_close_bf16(bad, ref)
    heavy = rng.standard_normal(10000) * rng.standard_normal(10000) ** 3
    bad = bf16_round_f32(heavy.astype(np.float32)).astype(np.float64)
    bad[5] += 0.05 * np.sqrt(np.mean(heavy ** 2))
    with pytest.raises(AssertionError):
        assert_close_bf16(bad, heavy)
