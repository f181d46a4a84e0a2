"""The conv1d + SiLU oracle against its pins, and planted mistakes that the pins catch."""
import os

import pytest

import oracle
from oracle_conv_pins import PINS


@pytest.fixture(scope="module")
def conv_orc():
    return oracle.load_conv()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_conv_pin(conv_orc, pin):
    pin(conv_orc)


# (name, [(original text, replacement), ...]) edits of oracle/oracle_conv.c
MUTANTS = [
    ("weights_reversed", [("acc += w[d * K + k] * v;", "acc += w[d * K + (K - 1 - k)] * v;")]),
    ("tap_off_by_one", [("const int64_t s = t - S + k; /* input time of tap k */",
                         "const int64_t s = t - S + k - 1; /* input time of tap k */")]),
    ("bias_dropped", [("double acc = bias ? bias[d] : 0.0;\n                for",
                       "double acc = 0.0;\n                for")]),
    ("no_silu", [("u[(b * L + t) * D + d] = conv_silu(acc);", "u[(b * L + t) * D + d] = acc;")]),
    ("state_ignored", [("v = state_in ? state_in[(b * D + d) * S + (S + s)] : 0.0;\n"
                        "                    acc",
                        "v = 0.0;\n                    acc")]),
    ("state_reversed", [("v = state_in ? state_in[(b * D + d) * S + (S + s)] : 0.0;\n"
                         "                    acc",
                         "v = state_in ? state_in[(b * D + d) * S + (-1 - s)] : 0.0;\n"
                         "                    acc")]),
    ("state_out_offset", [("const int64_t s = L - S + j;", "const int64_t s = L - S + j - 1;")]),
    ("step_no_shift", [("st[k] = st[k + 1];", "st[k] = st[k];")]),
    ("step_newest_tap", [("acc += w[d * K + S] * xn;", "acc += w[d * K] * xn;")]),
    ("silu_sign", [("return p / (1.0 + exp(-p));", "return p / (1.0 + exp(p));")]),
]


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_conv_mutant_is_caught(tmp_path, name, edits):
    src = open(oracle.CONV_SOURCE).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"{name}: edit target not found: {old!r}"
        src = src.replace(old, new)
    cpath = os.path.join(str(tmp_path), f"{name}.c")
    with open(cpath, "w") as f:
        f.write(src)
    orc = oracle.ConvOracle(oracle.build(cpath, os.path.join(str(tmp_path), f"lib{name}.so")))
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
