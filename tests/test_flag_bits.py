"""The integer outlier test of the one-launch steps 1-2 (k_rows), checked
exhaustively on the host: for every fp16 value x and a spread of
thresholds, |x| >= thr compared in fp32 (reading R1 of the oracle, the
"exceeds about 6" test of step 1 in the Hugging Face summary's "LLM.int8()
の核心アイデア") equals the carry into bit 15 of (bits(x) & 0x7fff) +
(0x8000 - t16), t16 being the bits of the smallest fp16 value >= thr (the
largest finite fp16 value and beyond: the bits of infinity).  This pins
the arithmetic argument the kernel relies on; the GPU tests pin the kernel
against the oracle at the same thresholds."""
import numpy as np
import pytest


def ceil_bits(thr: float) -> int:
    # smallest fp16 value >= thr, as bits (thr > 0)
    if not thr <= 65504.0:
        return 0x7C00
    h = np.float16(np.float32(thr))
    b = int(h.view(np.uint16))
    if np.float32(h) < np.float32(thr):
        b += 1
    return b


THRESHOLDS = [6.0, 6.1, 5.999, 1.0, 0.5, 1e-4, 6.1e-5, 3e-8, 1e-10, 2.0 ** -24, 1000.3, 65504.0,
              65504.5, 65519.0, 65520.0, 1e30, float("inf")]


@pytest.mark.parametrize("thr", THRESHOLDS)
def test_integer_flag_test_matches_fp32_compare(thr):
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = bits.astype(np.uint16).view(np.float16)
    finite = np.isfinite(x)
    want = np.abs(x.astype(np.float32)) >= np.float32(thr)
    t16 = ceil_bits(thr)
    got = (((bits & 0x7FFF) + (0x8000 - t16)) >> 15) & 1
    assert np.array_equal(got[finite].astype(bool), want[finite])
    # two values a 32-bit word: no carry from the low half into the high one
    lo, hi = bits[:4096], bits[-4096:]
    word = (lo | (hi << 16)) & 0x7FFF7FFF
    s = word + (0x8000 - t16) * 0x10001
    assert np.array_equal((s >> 15) & 1, (((lo & 0x7FFF) + 0x8000 - t16) >> 15) & 1)
    assert np.array_equal((s >> 31) & 1, (((hi & 0x7FFF) + 0x8000 - t16) >> 15) & 1)
