"""Checks of the pages' printed figure and of the seeded input generator (CPU)."""
import os

import numpy as np

import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_logits_memory_figure():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "logits_memory.txt"))
            if l.strip() and not l.startswith("#")]
    for tokens, vocab, min_logits, bpe, gib, tol in rows:
        n = int(tokens) * int(vocab)
        assert n > int(min_logits)
        assert abs(n * int(bpe) / 2**30 - float(gib)) < float(tol)
        assert n == 1_050_673_152


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-7 + 2**-9,
                     3.0e38, 1e-40], dtype=np.float32)
    bits = si.round_to_bf16_bits(vals)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6)
    expect = [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]
    assert bits[:5].tolist() == expect
    back = si.bf16_bits_to_f32(bits)
    assert np.isfinite(back[5]) and back[6] >= 0


def test_generator_is_seeded_and_shaped():
    a = si.make_inputs(64, 16, 100, bias_std=0.1, ignore_frac=0.25, reduction="none", seed=7)
    b = si.make_inputs(64, 16, 100, bias_std=0.1, ignore_frac=0.25, reduction="none", seed=7)
    for k in ("hidden", "weight", "bias", "targets", "grad_loss"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["hidden"].dtype == np.uint16 and a["hidden"].shape == (64, 16)
    assert (a["targets"] == si.IGNORE_INDEX).sum() == 16
    t = a["targets"][a["targets"] != si.IGNORE_INDEX]
    assert t.min() >= 0 and t.max() < 100
    z = si.make_inputs(4096, 8, 1000, targets="zipf", seed=1)["targets"]
    # Zipf(1.1): id 0 is the most frequent and frequencies fall with the id
    counts = np.bincount(z, minlength=1000)
    assert counts[0] > counts[1] > counts[10] and z.max() < 1000
    f = si.make_inputs(8, 4, 5, dtype="f32", weight_std=0.05, seed=0)
    assert f["weight"].dtype == np.float32 and abs(f["weight"].std() - 0.05) < 0.05
