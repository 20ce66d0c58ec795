"""The C build of the input generator against its numpy reference (inputs only; no method
arithmetic lives in synth)."""
import numpy as np

import synth


def test_words_bit_exact():
    for seed, stream, start, count in ((1, 0, 0, 1000), (0x5EED0003, 7, 123456789, 5000),
                                       (2**63 + 5, 2**40, 2**33, 257)):
        assert np.array_equal(synth.words(seed, stream, start, count),
                              synth.words_native(seed, stream, start, count))


def test_normal_matches_reference():
    seed, stream = synth.seed_for(3), synth.weight_stream(5, "w1")
    start, count = 3_000_000, 200_000
    ref = synth.normal_f64_reference(seed, stream, start, count)
    full = synth.normal_f16(seed, stream, (start + count,), 1.0)[start:]
    # libm and numpy may differ in the last bit of log/cos: allow one binary16 step
    refh = ref.astype(np.float16)
    diff = np.abs(full.astype(np.float64) - refh.astype(np.float64))
    ulp = np.spacing(np.abs(refh)).astype(np.float64)
    assert (diff <= ulp).all()
    assert (full == refh).mean() > 0.999


def test_normal_moments_and_slices():
    x = synth.normal_f16(synth.seed_for(9), 1, (1 << 20,), 0.02).astype(np.float64)
    assert abs(x.mean()) < 0.02 * 5e-3 and abs(x.std() / 0.02 - 1) < 5e-3
    a = synth.normal_f16(1, 2, (3, 1000))
    b = synth.normal_f16(1, 2, (3000,))
    assert np.array_equal(a.ravel(), b)
