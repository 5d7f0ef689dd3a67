"""The oracle's pins are strong enough to catch plausible slips.

Each case rewrites one spot of a private copy of oracle/oracle.c (a transposed
operand, a dropped term, a wrong rounding tie, an unstable order, ...),
compiles it with gcc into a temporary directory, and runs every pin from
oracle_pins.py against it in a subprocess (a slip that reads out of bounds
may crash; a crash counts as caught).  At least one pin must fail for every
mutant, and all pins must pass on the unmodified source.
"""
import json
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")

# (name, text in oracle.c, replacement); the first occurrence is replaced
MUTANTS = [
    ("W transposed", "oracle_bf16_to_f64(W[n * K + k]);", "oracle_bf16_to_f64(W[k * N + n]);"),
    ("x row stride", "oracle_bf16_to_f64(x[m * K + k]) *", "oracle_bf16_to_f64(x[m + k]) *"),
    ("last k dropped", "for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k + 1 < K; ++k) {"),
    ("term sign", "sum += term;", "sum -= term;"),
    ("scale without abs", "abs_sum += fabs(term);", "abs_sum += term;"),
    ("ties away from zero", "(frac == 0.5 && fmod(lo, 2.0) != 0.0)", "(frac == 0.5)"),
    ("ties to odd", "fmod(lo, 2.0) != 0.0", "fmod(lo, 2.0) == 0.0"),
    ("subnormal spacing", "? -133 : E - 7", "? -134 : E - 7"),
    ("mantissa width", "? -133 : E - 7", "? -133 : E - 8"),
    ("overflow threshold", "if (rounded > ldexp(", "if (rounded >= ldexp("),
    ("decode shift", "(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    ("split-K unaligned chunk", "int64_t chunk = 64 * ((K + 64 * S - 1) / (64 * S));",
     "int64_t chunk = (K + S - 1) / S;"),
    ("split-K 16-byte chunk", "int64_t chunk = 64 * ((K + 64 * S - 1) / (64 * S));",
     "int64_t chunk = 8 * ((K + 8 * S - 1) / (8 * S));"),
    ("split-K floor chunk", "int64_t chunk = 64 * ((K + 64 * S - 1) / (64 * S));",
     "int64_t chunk = 64 * (K / (64 * S));"),
    ("split-K chunk overlap", "int64_t k_begin = s * chunk;", "int64_t k_begin = s * chunk - (s > 0);"),
    ("split-K descending sum", "for (int64_t s = 0; s < S; ++s)\n            sum += P[s * MN + i];",
     "for (int64_t s = S - 1; s >= 0; --s)\n            sum += P[s * MN + i];"),
    ("residual sign", "oracle_bf16_to_f64(r[i]) + y[i]", "oracle_bf16_to_f64(r[i]) - y[i]"),
    ("moe unstable segment", "for (int64_t p = 0; p < pairs; ++p) {\n            if (ids[p] == e)",
     "for (int64_t p = pairs - 1; p >= 0; --p) {\n            if (ids[p] == e)"),
    ("moe offsets not scanned", "offsets[e + 1] = offsets[e] + counts[e];", "offsets[e + 1] = counts[e];"),
    ("moe accepts id E", "if (e < 0 || e >= E)\n            ++invalid;", "if (e < 0 || e > E)\n            ++invalid;"),
    ("moe tail not -1", "sorted_pairs[p] = -1;", "sorted_pairs[p] = 0;"),
    ("grouped expert stride", "W + (int64_t)e * N * K", "W + (int64_t)e * K"),
    ("grouped token row", "x + t * K, W", "x + j * K, W"),
    ("grouped invalid ids kept", "if (e < 0 || e >= E) {\n                for", "if (e < 0) {\n                for"),
    ("topk ties to higher id", "    return ia < ib;", "    return ia > ib;"),
    ("topk ascending", "        return da > db;", "        return da < db;"),
    ("topk nan as +inf", "isnan(a) ? -INFINITY", "isnan(a) ? INFINITY"),
    ("topk retakes experts", "if (taken[e])", "if (0)"),
    ("mxfp4 nibble order", "(k % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
     "(k % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    ("mxfp4 one scale a row", "Ws[n * (K / 32) + k / 32]", "Ws[n * (K / 32)]"),
    ("e2m1 exponent bias", "ldexp(1.0 + m * 0.5, e - 1)", "ldexp(1.0 + m * 0.5, e)"),
    ("e2m1 mantissa weight", "ldexp(1.0 + m * 0.5, e - 1)", "ldexp(1.0 + m * 0.25, e - 1)"),
    ("e2m1 subnormal", "mag = m * 0.5;", "mag = m * 1.0;"),
    ("e2m1 sign dropped", "return sign ? -mag : mag;", "return mag;"),
    ("e4m3 exponent bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3 mantissa width", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 16.0, e - 7)"),
    ("e4m3 subnormal exponent", "ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    ("e4m3 NaN code finite", "if (e == 15 && m == 7)\n        return NAN;", "if (0)\n        return NAN;"),
    ("e4m3 sign dropped", "    return sign ? -mag : mag;\n}\n\nvoid oracle_projection_fp8",
     "    return mag;\n}\n\nvoid oracle_projection_fp8"),
    ("fp8 64-column scale blocks", "Ws[(n / 128) * KB + k / 128]", "Ws[(n / 128) * KB + k / 64 % KB]"),
    ("fp8 scale per row block only", "Ws[(n / 128) * KB + k / 128]", "Ws[(n / 128) * KB]"),
    ("fp8 scale blocks transposed", "Ws[(n / 128) * KB + k / 128]",
     "Ws[((k / 128) * ((N + 127) / 128) + n / 128) % (KB * ((N + 127) / 128))]"),
    ("e8m0 bias", "ldexp(1.0, (int)s - 127)", "ldexp(1.0, (int)s - 128)"),
    ("e8m0 nan code finite", "if (s == 255)\n        return NAN;", "if (0)\n        return NAN;"),
]


def _run(src_text: str, workdir: str) -> dict | None:
    """Compile a copy of the oracle and run every pin; None if the run crashed."""
    src = os.path.join(workdir, "oracle.c")
    with open(src, "w") as f:
        f.write(src_text)
    hdr = os.path.join(os.path.dirname(SRC), "oracle.h")
    with open(hdr) as f, open(os.path.join(workdir, "oracle.h"), "w") as g:
        g.write(f.read())
    lib = oracle.build(os.path.join(workdir, "liboracle.so"), src)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                          capture_output=True, text=True, timeout=300)
    if proc.returncode != 0:
        return None
    return json.loads(proc.stdout.strip().splitlines()[-1])


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_unmodified_oracle_passes_every_pin(source, tmp_path):
    res = _run(source, str(tmp_path))
    assert res is not None
    assert all(v is None for v in res.values()), res


def test_every_mutant_is_caught(source, tmp_path):
    for name, old, new in MUTANTS:
        assert old in source, f"mutation site for {name!r} not found in oracle.c"

    def one(i_case):
        i, (name, old, new) = i_case
        d = tmp_path / f"m{i}"
        d.mkdir()
        res = _run(source.replace(old, new, 1), str(d))
        if res is None:
            return name, "crashed"
        failed = [k for k, v in res.items() if v is not None]
        return name, failed

    with ThreadPoolExecutor(max_workers=4) as pool:
        outcomes = list(pool.map(one, enumerate(MUTANTS)))
    survivors = [name for name, failed in outcomes if not failed]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
