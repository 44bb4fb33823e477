"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that at least one pin catches each of them.  This shows the pins constrain
every part of the oracle: the transform's normalization, order and signs,
the code bit order, the group indexing, the bias, and the embedding."""
import os
import types

import pytest

from oracle_pins import PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "reference.py")

MUTANTS = {
    "fold_uses_inverse": ("return fwht_signed(w, signs, block)",
                          "return fwht_signed(w, signs, block, inverse=True)"),
    "no_normalization": ("return a.reshape(*lead, K) / math.sqrt(block)",
                         "return a.reshape(*lead, K)"),
    "butterfly_swapped_halves": ("a = np.stack((lo + hi, lo - hi), axis=3)",
                                 "a = np.stack((lo + hi, hi - lo), axis=3)"),
    "signs_after_forward": ("return fwht_blocks(x * s, block)",
                            "return fwht_blocks(x, block) * s"),
    "signs_before_inverse": ("return fwht_blocks(x, block) * s\n    return",
                             "return fwht_blocks(x * s, block)\n    return"),
    "code_bit_order_reversed": ("c = (codes[:, :, None] >> shifts[None, None, :]) & np.uint32(3)",
                                "c = (codes[:, :, None] >> (30 - shifts)[None, None, :]) & np.uint32(3)"),
    "pack_bit_order_reversed": ("words = np.bitwise_or.reduce(c << shifts[None, None, :], axis=2)",
                                "words = np.bitwise_or.reduce(c << (30 - shifts)[None, None, :], axis=2)"),
    "bias_dropped": ("return sc[rows][:, g] * c + bi[rows][:, g]",
                     "return sc[rows][:, g] * c"),
    "bias_sign_flipped": ("return sc[rows][:, g] * c + bi[rows][:, g]",
                          "return sc[rows][:, g] * c - bi[rows][:, g]"),
    "group_of_64": ("g = np.arange(K) // GROUP", "g = np.arange(K) // 64 % (K // GROUP)"),
    "code_is_t": ("c = (t.astype(np.int64) + 1).astype(np.uint32)",
                  "c = (t.astype(np.int64) % 4).astype(np.uint32)"),
    "bias_equals_scale": ("return words, sc.copy(), (-sc).astype(np.float16)",
                          "return words, sc.copy(), sc.copy()"),
    "signs_wrap_per_block": ("return s.astype(np.float64)",
                             "return np.tile(s[:1024], K // 1024 + 1)[:K].astype(np.float64) if K >= 1024 else s.astype(np.float64)"),
    "transposed_operand": ("out[:, i:i + _ROW_CHUNK] = xr @ w.T",
                           "out[:, i:i + _ROW_CHUNK] = (w @ xr.T[::-1]).T"),
    "whole_vector_transform": ("return fwht_blocks(x * s, block)",
                               "return fwht_blocks(x * s, x.shape[-1]) if x.shape[-1] & (x.shape[-1] - 1) == 0 else fwht_blocks(x * s, block)"),
    "embed_skips_inverse": ("out[ok] = fwht_signed(rows, signs, block, inverse=True)",
                            "out[ok] = fwht_signed(rows, signs, block)"),
    "embed_wrong_row": ("rows = dequantize_rows(codes, scales, biases, K, ids[ok])",
                        "rows = dequantize_rows(codes, scales, biases, K, (ids[ok] + 1) % V)"),
    "unpack_accepts_code3": ("if (c == 3).any():", "if False:"),
}


def _mutant(old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) == 1, f"mutation site not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError) as e:  # any failure counts
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


# --- the PQ2_0 / PTQ1_0 oracle (oracle/formats.py) -------------------------
from oracle_pins_formats import PINS_FORMATS  # noqa: E402

FORMATS_PATH = os.path.join(os.path.dirname(SRC_PATH), "formats.py")

MUTANTS_FORMATS = {
    "pq2_scale_after_codes": ("out = np.concatenate([_scale_bytes(s), qs], axis=2)",
                              "out = np.concatenate([qs, _scale_bytes(s)], axis=2)"),
    "pq2_codes_high_bits_first": ("qs = cb[..., 0] | (cb[..., 1] << 2) | (cb[..., 2] << 4) | (cb[..., 3] << 6)",
                                  "qs = cb[..., 3] | (cb[..., 2] << 2) | (cb[..., 1] << 4) | (cb[..., 0] << 6)"),
    "pq2_decode_reads_high_bits_first": ("c = np.stack([(qs >> (2 * j)) & 3 for j in range(4)], axis=-1)",
                                         "c = np.stack([(qs >> (6 - 2 * j)) & 3 for j in range(4)], axis=-1)"),
    "pq2_decode_without_offset": ("return d[:, np.arange(K) // GROUP] * (c - 1.0)",
                                  "return d[:, np.arange(K) // GROUP] * c"),
    "pq2_accepts_any_bias": ("if not np.array_equal(b, s ^ np.uint16(0x8000)):", "if False:"),
    "pq2_scale_bytes_swapped": ("return (lo | (hi << 8)).view(np.float16)", "return (hi | (lo << 8)).view(np.float16)"),
    "ptq1_first_code_highest_digit": ("for j in reversed(range(TRITS_PER_BYTE)):", "for j in range(TRITS_PER_BYTE):"),
    "ptq1_decode_highest_digit_first": (
        "c = np.stack(digits, axis=-1).reshape(bl.shape[0], bl.shape[1], -1)[:, :, :GROUP]",
        "c = np.stack(digits[::-1], axis=-1).reshape(bl.shape[0], bl.shape[1], -1)[:, :, :GROUP]"),
    "ptq1_last_byte_unchecked": ("if (q > 242).any() or (q[:, :, -1] > 26).any():", "if (q > 242).any():"),
    "ptq1_codes_not_shifted": ("c = (t.astype(np.int64) + 1).reshape(N, G, GROUP)",
                               "c = (t.astype(np.int64) % 3).reshape(N, G, GROUP)"),
    "ptq1_group_of_64": ("return f16_to_f64(d)[:, np.arange(K) // GROUP] * t.astype(np.float64)",
                         "return f16_to_f64(d)[:, np.arange(K) // 64 % (K // GROUP)] * t.astype(np.float64)"),
}


def _mutant_formats(old, new):
    src = open(FORMATS_PATH).read()
    assert src.count(old) == 1, f"mutation site not unique/present: {old!r}"
    mod = types.ModuleType("formats_mutant")
    exec(compile(src.replace(old, new), "formats_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS_FORMATS))
def test_formats_mutant_is_caught(name):
    mod = _mutant_formats(*MUTANTS_FORMATS[name])
    caught = []
    for pin in PINS_FORMATS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
