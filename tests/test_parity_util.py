"""CPU checks of the parity helpers themselves: the per-(sequence, head) bar catches an
error that the whole-tensor bar lets through, packed slices follow cu_seqlens, and the
float32 floor only forgives values below float32's normal range."""
import numpy as np
import pytest

from tests.parity_util import Accum, check


def _tokens(seed=0, B=2, T=50, H=3, d=4, head_scale=(100.0, 1.0, 0.01)):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal((B, T, H, d)) * np.asarray(head_scale)[None, None, :, None]
    return ref


def test_per_slice_bar_catches_small_head_error():
    ref = _tokens()
    got = ref.copy()
    got[1, 7, 2, 0] += 0.5  # huge for head 2 (RMS 0.01), invisible next to head 0 (RMS 100)
    whole_rms = np.sqrt(np.mean(ref * ref))
    assert 0.5 / whole_rms < 2e-2  # the whole-tensor bar alone would pass
    with pytest.raises(AssertionError, match=r"slice \(1, 2\)"):
        check(got, ref, 2e-2, "planted", "tokens")


def test_clean_result_passes_both_bars():
    ref = _tokens(1)
    got = ref * (1 + 1e-3)
    assert check(got, ref, 2e-2, "clean", "tokens") < 2e-2


def test_packed_slices_follow_cu_seqlens():
    ref = _tokens(2, B=1, T=30, head_scale=(1.0, 1.0, 1.0))
    ref[:, 10:12] *= 1e-3  # a short sequence with tiny values
    got = ref.copy()
    got[0, 11, 1, 3] += 1e-3
    cu = np.array([0, 10, 12, 30])
    check(got, ref, 2e-2, "as one row", "tokens")  # one (row, head) slice: the error hides
    with pytest.raises(AssertionError, match=r"slice \(1, 1\)"):
        check(got, ref, 2e-2, "packed", "tokens", cu=cu)


def test_state_and_row_layouts():
    rng = np.random.default_rng(3)
    st = rng.standard_normal((3, 2, 4, 5))
    st[2, 1] *= 1e-6
    bad = st.copy()
    bad[2, 1, 0, 0] += 1e-5
    with pytest.raises(AssertionError, match=r"slice \(2, 1\)"):
        check(bad, st, 2e-2, "states", "states")
    rows = rng.standard_normal((4, 3, 8))
    rows[3, 0] *= 1e-6
    badr = rows.copy()
    badr[3, 0, 5] += 1e-5
    with pytest.raises(AssertionError, match=r"slice \(3, 0\)"):
        check(badr, rows, 2e-2, "rows", "rows")


def test_float32_floor():
    ref = np.full((1, 2, 1, 3), 1e-87)  # not representable in float32
    got = np.zeros_like(ref)            # what a float32 result holds
    check(got, ref, 1e-4, "underflow", "tokens")
    got2 = np.full_like(ref, 1e-30)     # a normal float32 value where the exact one is 1e-87
    with pytest.raises(AssertionError):
        check(got2, ref, 1e-4, "not underflow", "tokens")


def test_streamed_accumulation_equals_one_shot():
    ref = _tokens(4, B=3)
    got = ref * (1 + 1e-4 * np.random.default_rng(5).standard_normal(ref.shape))
    acc = Accum("streamed")
    for b in range(3):
        acc.add_tokens(got[b:b + 1], ref[b:b + 1], row0=b)
    assert acc.finish(2e-2) == pytest.approx(check(got, ref, 2e-2, "one shot", "tokens"))
    assert sorted(acc.slices) == [(b, h) for b in range(3) for h in range(3)]
