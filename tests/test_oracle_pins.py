"""The oracle against what the pages and mathematics fix (CPU only).

Also builds copies of oracle.c with one plausible mistake planted in each and
checks that at least one pin fails for every copy."""

import pytest

import oracle
from oracle import build as obuild

from . import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.default())


# (name, original text, planted mistake) -- each replacement must exist in oracle.c
MUTANTS = [
    ("ssq_hi_lo_swapped_in_dot",
     "double wa = da * (double)(int8_t)(uint8_t)(slot >> 8);\n            double wb = db * (double)(int8_t)(uint8_t)(slot & 0xff);",
     "double wa = da * (double)(int8_t)(uint8_t)(slot & 0xff);\n            double wb = db * (double)(int8_t)(uint8_t)(slot >> 8);"),
    ("ssq_scales_swapped", "double da = orc_f16_to_f64(rd16(blk + 0));\n        double db = orc_f16_to_f64(rd16(blk + 2));",
     "double da = orc_f16_to_f64(rd16(blk + 2));\n        double db = orc_f16_to_f64(rd16(blk + 0));"),
    ("q8_scale_dropped", "double w = d * (double)(int8_t)blk[2 + j];", "double w = (double)(int8_t)blk[2 + j];"),
    ("q8_unsigned_weights", "double w = d * (double)(int8_t)blk[2 + j];", "double w = d * (double)(uint8_t)blk[2 + j];"),
    ("q8_x_index_off", "double xv = (double)x[k * ORC_BLOCK + j];", "double xv = (double)x[k * ORC_BLOCK + (j ^ 1)];"),
    ("q8_block_offset_off", "const uint8_t *blk = row + k * ORC_Q8_BYTES;", "const uint8_t *blk = row + k * ORC_Q8_BYTES + (k > 0);"),
    ("q8_streams_share_x", "x + (int64_t)s * cols, y + (int64_t)s * rows + r", "x, y + (int64_t)s * rows + r"),
    ("f16_subnormal_exponent", "v = ldexp((double)fr, -24);", "v = ldexp((double)fr, -25);"),
    ("f16_bias", "v = ldexp((double)(1024 + fr), ex - 25);", "v = ldexp((double)(1024 + fr), ex - 24);"),
    ("pack_b_in_high_byte", "uint16_t slot = (uint16_t)(((uint8_t)a[r * cols + c] << 8) | (uint8_t)b[r * cols + c]);",
     "uint16_t slot = (uint16_t)(((uint8_t)b[r * cols + c] << 8) | (uint8_t)a[r * cols + c]);"),
    ("argmax_last_tie_wins", "if (v[i] > v[best])", "if (v[i] >= v[best])"),
    ("accept_counts_all_matches", "if (tokens_in[i] != argmax[i - 1])\n            break;",
     "if (tokens_in[i] != argmax[i - 1])\n            continue;"),
    ("accept_compares_same_stream", "if (tokens_in[i] != argmax[i - 1])", "if (tokens_in[i] != argmax[i])"),
    ("magnitude_signed", "mag += fabs(w) * fabs(xv);", "mag += w * xv;"),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, orig, bad, tmp_path):
    src = open(obuild.SRC).read()
    assert orig in src, f"mutation anchor for {name} not found in oracle.c"
    lib = obuild.build_variant(src.replace(orig, bad, 1), str(tmp_path / f"lib_{name}.so"))
    failed = pins.run_all(oracle.Oracle(lib))
    assert failed, f"no pin caught the planted mistake {name}"
