"""The oracle against its pins (CPU only)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()


def test_encoder_exhaustive_fp32():
    """The oracle's E2M1 encoder on every finite fp32 in [-6, 6] (both signs of all 1.09e9 bit
    patterns from +0 to 6.0), against the textbook rule: the nearest value of the E2M1 grid, ties
    to the even code (reading of the forward-quantization paragraph's 'nearest FP4 value').  Kept
    out of the mutant runs for its length; the sampled encoder pins above cover those."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    mags2 = np.full(13, 255, dtype=np.uint8)  # 2*value -> magnitude code
    for code, v in enumerate((0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)):
        mags2[int(v * 2)] = code
    top = int(np.array(6.0, dtype=np.float32).view(np.uint32))
    step = 1 << 22

    def chunk(lo: int) -> int:
        bits = np.arange(lo, min(lo + step, top + 1), dtype=np.uint32)
        x = bits.view(np.float32)
        # round half to even on the grid: spacing 0.5 below 2, 1 below 4, 2 above (all exact)
        s = np.where(x < 2, np.float32(0.5), np.where(x < 4, np.float32(1.0), np.float32(2.0)))
        v = np.minimum(np.rint(x / s) * s, np.float32(6.0))
        ref = mags2[(v * 2).astype(np.int64)]
        assert not np.any(ref == 255)
        got = oracle.e2m1_encode(x)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"x={x[bad[0]]!r}: got {got[bad[0]]}, nearest-even {ref[bad[0]]}"
        neg = oracle.e2m1_encode(-x)
        bad = np.nonzero(neg != (ref | 8))[0]
        assert bad.size == 0, f"x={-x[bad[0]]!r}: got {neg[bad[0]]}, nearest-even {ref[bad[0]] | 8}"
        return int(bits.size)

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        done = sum(ex.map(chunk, range(0, top + 1, step)))
    assert done == top + 1
