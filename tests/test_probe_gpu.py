"""The hardware bf16 conversion the LDS-tiled prefill epilogue relies on.

That epilogue rounds its fp32 sums to bf16 with the hardware's packed
conversion (v_cvt_pk_bf16_f32) where every other kernel uses an integer
round-to-nearest-even helper; the two must give the same bits for every fp32
pattern (finite, infinite and NaN), which one launch over all 2^32 patterns
checks (include/w4a16_probe.h).
"""
import pytest

torch = pytest.importorskip("torch")


@pytest.mark.gpu
def test_hardware_bf16_conversion_equals_the_rounding_helper():
    from decode_w4a16_affine_amd import profiling
    print("probe: bf16 conversion of all 2^32 fp32 patterns", flush=True)
    mismatches, first = profiling.bf16_round_check(torch)
    assert mismatches == 0, f"{mismatches} patterns differ, the smallest 0x{first:08x}"
    assert first == 0xFFFFFFFF
