"""Mutation check of the pins: plant plausible mistakes in a copy of the
oracle's C source, build it on the CPU, and require that the pins reject
every mutant.  The committed oracle is untouched."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import workload
from pins import (check_matmul_exact, check_pack, check_quantize_invariants,
                  check_quantize_row)
from test_oracle_pins import EXAMPLES, as_input, brute_rows

SRC = os.path.join(os.path.dirname(oracle.__file__), "dq_oracle.c")

# (name, text in dq_oracle.c, replacement)
MUTANTS = [
    ("bias_minus_one", "const uint32_t bias = 1u << (bits - 1);",
     "const uint32_t bias = (1u << (bits - 1)) - 1;"),
    ("code_msb_first", "uint32_t bit = (u >> j) & 1u;", "uint32_t bit = (u >> (bits - 1 - j)) & 1u;"),
    ("word_msb_first", "words[pos / 32] |= bit << (pos % 32);",
     "words[pos / 32] |= bit << (31 - pos % 32);"),
    ("round_half_away", "float r = rintf(t);", "float r = roundf(t);"),
    ("reciprocal_multiply", "float t = v / s;", "float t = v * (1.0f / s);"),
    ("scale_by_qmax_plus_one", "float s = (a == 0.0f ? 1.0f : a) / (float)qmax;",
     "float s = (a == 0.0f ? 1.0f : a) / (float)(qmax + 1);"),
    ("absmax_signed", "} else if (fabsf(v) > a) {", "} else if (v > a) {"),
    ("clip_symmetric_low", "if (r > hi)\n            r = hi;", "if (r > hi - 1)\n            r = hi - 1;"),
    ("zero_row_scale_one", "float s = (a == 0.0f ? 1.0f : a) / (float)qmax;",
     "float s = (a == 0.0f ? (float)qmax : a) / (float)qmax;"),
    ("nonfinite_ignored", "if (!isfinite(v)) {", "if (0) {"),
    ("unpack_bias_kept", "q[k] = (int32_t)u - bias;", "q[k] = (int32_t)u;"),
    ("matmul_no_scale", "y[m * N + n] = (double)scales[n] * acc;", "y[m * N + n] = acc;"),
    ("matmul_transposed", "double p = (double)bf16_bits_to_float(x[m * K + k]) * (double)q[k];\n"
     "                acc += p;\n                mag += fabs(p);\n            }\n            y[m * N + n]",
     "double p = (double)bf16_bits_to_float(x[k * M + m]) * (double)q[k];\n"
     "                acc += p;\n                mag += fabs(p);\n            }\n            y[m * N + n]"),
    ("bound_signed", "mag += fabs(p);\n            }\n            y[m * N + n]",
     "mag += p;\n            }\n            y[m * N + n]"),
    ("dequant_dropped_scale", "w_out[n * K + k] = (float)q[k] * scales[n];",
     "w_out[n * K + k] = (float)q[k];"),
]


def run_pins(orc: oracle.Oracle) -> list[str]:
    bad = []
    for ex in EXAMPLES:
        bits = int(ex["bits"])
        w_in, w_f32 = as_input([float(v) for v in ex["w"].split()], ex["dtype"])
        packed, scales, q = orc.quantize_pack(w_in, bits)
        want = [int(v) for v in ex["words"].split()]
        if packed[0, :len(want)].tolist() != want or packed[0, len(want):].any():
            bad.append("golden %s words" % ex["name"])
        bad += check_quantize_row(w_f32[0], bits, q[0], scales[0])
    for bits in (2, 5, 6, 15):
        rng = np.random.default_rng(bits)
        for w in brute_rows(bits, rng):
            packed, scales, q = orc.quantize_pack(w[None, :], bits)
            bad += check_quantize_row(w, bits, q[0], scales[0])
        nanrow = np.array([[1.0, np.nan, 0.5]], np.float32)
        packed, scales, q = orc.quantize_pack(nanrow, bits)
        bad += check_quantize_row(nanrow[0], bits, q[0], scales[0])
        w = workload.weights(95, bits, 16, 200, dtype="f32")
        packed, scales, q = orc.quantize_pack(w, bits)
        bad += check_quantize_invariants(w, bits, q, scales)
        lim = 1 << (bits - 1)
        qr = rng.integers(-lim, lim, size=(2, 37), dtype=np.int32)
        pr = orc.pack(qr, bits)
        bad += check_pack(qr, bits, pr)
        q2, _ = orc.unpack(pr, None, 2, 37, bits)
        if not np.array_equal(q2, qr):
            bad.append("round trip b=%d" % bits)
        wf = workload.weights(94, bits, 3, 9, dtype="f32")
        packed, scales, q = orc.quantize_pack(wf, bits)
        _, w_hat = orc.unpack(packed, scales, 3, 9, bits)
        if not np.array_equal(w_hat, q.astype(np.float32) * scales[:, None]):
            bad.append("dequant b=%d" % bits)
        x = workload.activations(94, bits, 2, 9)
        y, bound = orc.matmul(x, packed, scales, 3, 9, bits)
        bad += check_matmul_exact(workload.bf16_to_f32(x), q, scales, y, bound)
    return bad


def test_pins_accept_the_oracle():
    assert run_pins(oracle.default()) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not unique/found: %s" % name
    mut = tmp_path / ("oracle_%s.c" % name)
    mut.write_text(src.replace(old, new))
    path = oracle.build(force=True, src=str(mut), out=str(tmp_path / ("lib_%s.so" % name)))
    try:
        bad = run_pins(oracle.Oracle(path))
    except Exception as e:  # a mutant may also crash a check outright
        bad = ["raised %r" % e]
    assert bad, "mutant %s passed every pin" % name
