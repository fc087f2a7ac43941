"""Oracle pins: storage arithmetic, the worked scale example, binary16 rounding,
hand-derived group parameters and the packed layout.  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import storage


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_storage_printed_values(golden_dir):
    g = _load(golden_dir, "storage_group_size_page.json")
    for G, printed in g["overhead_4bit"].items():
        ov = oracle.bits_per_weight(4, int(G)) - 4
        assert storage.round_half_up(ov, 3) == printed
    for G, printed in g["bpw_4bit"].items():
        G = int(G)
        if G == -1:
            # "~0 -> 4.000": the limit of a long row; at d_in = 4096 the exact
            # overhead is 20/4096 = 0.0049 bit.
            bpw = oracle.bits_per_weight(4, -1, d_in=4096)
            assert bpw - 4 < 0.01
            assert storage.round_half_up(bpw, 2) == "4.00"
            assert storage.round_half_up(oracle.bits_per_weight(4, -1, d_in=10**7), 3) == printed
        else:
            assert storage.round_half_up(oracle.bits_per_weight(4, G), 3) == printed
    for G, printed in g["gb_7e9"].items():
        gb = oracle.model_gigabytes(7.0e9, oracle.bits_per_weight(4, int(G)))
        assert storage.round_half_up(gb, 2) == printed
    g128 = oracle.model_gigabytes(7.0e9, oracle.bits_per_weight(4, 128))
    g32 = oracle.model_gigabytes(7.0e9, oracle.bits_per_weight(4, 32))
    assert storage.round_half_up(g32 - g128, 2) == g["span_gb_7b"]
    assert round(100 * (g32 - g128) / g128) == g["span_percent_7b"]
    span_bpw = oracle.bits_per_weight(4, 32) - oracle.bits_per_weight(4, 128)
    assert storage.round_half_up(span_bpw, 3) == g["span_bpw"]
    assert storage.round_half_up(oracle.model_gigabytes(70e9, span_bpw), 1) == g["span_gb_70b"]
    # sym=True: no zero point, numerator 16
    sym_ov = oracle.bits_per_weight(4, 128, sym=True) - 4
    assert sym_ov * 128 == g["sym_numerator_bits"]
    assert oracle.bits_per_weight(4, 128, sym=True) == 4.125
    # 7e9 weights in FP16
    assert oracle.model_gigabytes(7e9, 16) == g["fp16_7b_gb"]
    for b, lv in g["levels"].items():
        assert oracle.maxq_for(int(b)) + 1 == lv


def test_round_half_up_matches_page_not_half_even():
    assert storage.round_half_up(4.3125, 3) == "4.313"
    assert f"{4.3125:.3f}" == "4.312"  # why the page's printing needs half-up


def test_scale_worked_example(golden_dir):
    g = _load(golden_dir, "scale_worked_example_page.json")
    clean = np.array([g["clean_group"]])
    out = np.array([g["outlier_group"]])
    for sym in (False, True):
        s, _ = oracle.group_params(clean, g["bits"], sym)
        assert round(float(s[0]), 4) == g["clean_step_printed"]
    s_out, _ = oracle.group_params(out, g["bits"], True)
    assert round(float(s_out[0]), 3) == g["outlier_step_printed"]
    s_clean, _ = oracle.group_params(clean, g["bits"], True)
    assert round(float(s_out[0] / s_clean[0])) == g["ratio_printed"]
    # asymmetric reading of the merged group gives a different step (0.52/15)
    s_asym, _ = oracle.group_params(out, g["bits"], False)
    assert abs(float(s_asym[0]) - 0.52 / 15) < 1e-4


def test_fp16_single_rounding_from_float64():
    # midpoint between 1 and 1+2^-10 rounds to even (1.0)
    assert oracle.fp16_rne(1 + 2.0**-11) == 1.0
    # just above the midpoint rounds up -- a float32 detour would double-round to 1.0
    assert oracle.fp16_rne(1 + 2.0**-11 + 2.0**-30) == 1 + 2.0**-10
    assert oracle.fp16_rne(1 + 3 * 2.0**-11) == 1 + 2 * 2.0**-10
    assert oracle.fp16_rne(65504.0) == 65504.0
    assert oracle.fp16_rne(2.0**-24) == 2.0**-24          # smallest subnormal
    assert oracle.fp16_rne(2.0**-26) == 0.0               # below half of it


def test_group_params_hand(golden_dir):
    g = _load(golden_dir, "group_params_hand.json")
    for c in g["cases"]:
        v = np.array([c["v"]])
        s, z = oracle.group_params(v, c["bits"], c["sym"])
        assert float(s[0]) == c["scale"], c
        assert float(z[0]) == c["zero"], c
        q, wh = oracle.quantize_values(v[0], s[0], z[0], oracle.maxq_for(c["bits"]))
        assert q.astype(int).tolist() == c["codes"], c
        np.testing.assert_array_equal(wh, s[0] * (q - z[0]))


def test_pack_hand(golden_dir):
    g = _load(golden_dir, "pack_hand.json")
    for c in g["cases"]:
        codes = np.array([c["codes"]], dtype=np.uint8)
        words = oracle.pack_rows(codes, c["bits"])
        assert [f"0x{int(w):08x}" for w in words[0]] == c["words"], c
        assert words.shape[1] == oracle.words_per_row(len(c["codes"]), c["bits"])
        np.testing.assert_array_equal(oracle.unpack_rows(words, c["bits"], codes.shape[1]), codes)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d_in", [32, 96, 128, 1000, 4096])
def test_pack_roundtrip_and_sizes(bits, d_in):
    rng = np.random.default_rng(bits * 10000 + d_in)
    codes = rng.integers(0, 1 << bits, size=(5, d_in), dtype=np.uint8)
    words = oracle.pack_rows(codes, bits)
    assert words.shape == (5, (d_in * bits + 31) // 32)
    np.testing.assert_array_equal(oracle.unpack_rows(words, bits, d_in), codes)
    if bits == 3 and d_in % 32 == 0:
        assert words.shape[1] == 3 * d_in // 32   # 32 codes per 3 words


def test_fp16_bits():
    b = oracle.fp16_bits(np.array([1.0, 0.066650390625, 8.0, 0.0]))
    assert b.tolist() == [0x3C00, 0x2C44, 0x4800, 0x0000]
    with pytest.raises(ValueError):
        oracle.fp16_bits(np.array([0.1]))
