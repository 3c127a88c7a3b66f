"""Pins of the seeded input generator (SplitMix64 + Box-Muller, bf16 rounding)."""
import numpy as np
import pytest

from top_routing_expert_router_amd import synth
from top_routing_expert_router_amd.synth import recipes


def test_splitmix64_published_vector():
    # First outputs of splitmix64 started at state 0 (the published reference
    # implementation's well-known sequence).
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [synth.splitmix64(0, j) for j in range(3)] == want


def test_counter_slices_match_full_stream():
    for dt in ("f64", "f32", "bf16"):
        full = synth.normal(77, 10001, 0.5, dt)
        for first, n in ((0, 1), (1, 7), (5000, 1001), (9999, 2)):
            assert np.array_equal(synth.normal(77, n, 0.5, dt, first=first), full[first:first + n])


def test_normal_moments():
    a = synth.normal(123, 2_000_000, 1.0, "f64")
    assert abs(a.mean()) < 4e-3
    assert abs(a.var() - 1.0) < 5e-3
    assert abs((a ** 3).mean()) < 1.5e-2
    assert abs((a ** 4).mean() - 3.0) < 3e-2
    # the tails exist (Box-Muller is exact in distribution, not truncated)
    assert (np.abs(a) > 4.5).sum() > 0


def _bf16_nearest_even(f32):
    """Independent RNE of float32 -> bf16: choose between truncation and the next bf16 up in magnitude."""
    u = f32.view(np.uint32).astype(np.uint64)
    lo = (u >> 16).astype(np.uint64)
    hi = lo + 1
    vlo = (lo << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    vhi = (hi << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    x = f32.astype(np.float64)
    dlo, dhi = np.abs(x - vlo), np.abs(vhi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def test_bf16_rounding_is_nearest_even():
    f = synth.normal(9, 300_000, 3.0, "f32")
    b = synth.normal(9, 300_000, 3.0, "bf16")
    assert np.array_equal(b, _bf16_nearest_even(f))


@pytest.mark.parametrize("name,bytes_expected", [
    # "Expert-parallel MoE training" explainer, memory calculator: 8 gated experts
    # of 3 x 4096 x 14336 bf16 = 2,818,572,288 B per card, and 64 of them
    # 22,548,578,304 B; the DeepSeek-shaped run (256 experts of 3 x 7168 x 2048)
    # holds exactly that many bytes too.
    ("4", 2_818_572_288),
    ("5", 22_548_578_304),
])
def test_expert_weight_bytes_match_memory_calculator(name, bytes_expected):
    r = recipes.RUNS[name]
    assert r.E * r.m * r.H * r.F * r.elem_bytes == bytes_expected


def test_expert_slices_match_full_tensor():
    r = recipes.SMALL["5"]
    full = recipes.gen_expert_weight(r, "w2")
    part = recipes.gen_expert_weight(r, "w2", experts=[0, 17, 255])
    for e, w in part.items():
        assert np.array_equal(w, full[e])
