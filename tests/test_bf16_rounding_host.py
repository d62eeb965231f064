"""The library's bf16 narrowing (d2bf for doubles, f2bf for floats; both in
csrc/msa_internal.h), built for the host, against the oracle's rounding from
the definition (O.f64_to_bf16), bit for bit.

d2bf narrows to float rounding toward zero and sets the last bit when inexact
(round to odd), then rounds that float to bf16 to nearest even; f2bf is the
nearest-even float -> bf16 step. Cases: random doubles over every binade,
exact bf16 midpoints (ties), midpoints nudged by one double ulp either way
(which a double rounding through float would get wrong), values next to
powers of two, the float and bf16 subnormal ranges and below, the edge of the
finite range and beyond FLT_MAX, +-0, +-inf and NaN."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import msa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "support", "bf16_round_host.cpp")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def tool(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    exe = str(tmp_path_factory.mktemp("bf16") / "bf16_round_host")
    subprocess.run([HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I",
                    os.path.join(ROOT, "routed_sparse_attention_amd", "csrc"), SRC, "-o", exe],
                   check=True, capture_output=True)
    return exe


def _run(exe, mode, values):
    with tempfile.TemporaryDirectory() as d:
        src, dst = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(src, "wb") as f:
            f.write(mode.encode())
            f.write(values.tobytes())
        subprocess.run([exe, src, dst], check=True)
        return np.fromfile(dst, dtype=np.uint16)


def _double_cases(rng):
    parts = []
    # every binade of double that matters for bf16 (and well past it)
    e = rng.integers(-160, 140, size=200_000)
    parts.append(rng.uniform(1.0, 2.0, size=e.size) * np.ldexp(1.0, e) *
                 rng.choice([-1.0, 1.0], size=e.size))
    # exact midpoints between neighbouring bf16 values, and one double ulp off
    b = rng.integers(0x0001, 0x7F7F, size=50_000).astype(np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    sign = rng.choice([-1.0, 1.0], size=mid.size)
    for m in (mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)):
        parts.append(m * sign)
    # next to powers of two (a round-up there changes the exponent)
    p = np.ldexp(1.0, np.arange(-140, 129))
    for q in (p, np.nextafter(p, 0), np.nextafter(p, np.inf), p * (1 - 2.0 ** -9),
              p * (1 - 2.0 ** -9 - 2.0 ** -30), p * (1 - 2.0 ** -9 + 2.0 ** -30)):
        parts += [q, -q]
    # subnormals: float's and bf16's, and below bf16's smallest
    parts.append(rng.uniform(0, 2.0 ** -126, size=20_000) * rng.choice([-1.0, 1.0], size=20_000))
    parts.append(np.ldexp(rng.uniform(0.5, 1.0, size=5_000), rng.integers(-160, -130, size=5_000)))
    # the top of the finite range and beyond FLT_MAX
    top = (2.0 - 2.0 ** -7) * 2.0 ** 127
    parts.append(np.array([top, np.nextafter(top, np.inf), top * (1 + 2.0 ** -9),
                           top * (1 + 2.0 ** -9) * (1 - 2.0 ** -40), top * (1 + 2.0 ** -8),
                           3.4028234663852886e38, 3.5e38, 1e39, 1e300, np.inf]))
    parts.append(-parts[-1])
    parts.append(np.array([0.0, -0.0, np.nan, -np.nan]))
    return np.concatenate(parts)


def test_d2bf_matches_the_rounding_definition(tool):
    x = _double_cases(np.random.default_rng(70))
    got = _run(tool, "d", x.astype(np.float64))
    with np.errstate(invalid="ignore"):
        want = O.f64_to_bf16(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{bad.size} of {x.size} differ, e.g. x={x[bad[:4]].tolist()} "
                           f"got={[hex(v) for v in got[bad[:4]]]} "
                           f"want={[hex(v) for v in want[bad[:4]]]}")


def test_f2bf_matches_the_rounding_definition(tool):
    rng = np.random.default_rng(71)
    bits = np.concatenate([rng.integers(0, 1 << 32, size=300_000, dtype=np.uint64),
                           # ties: low half exactly 0x8000, either parity of bit 16
                           (rng.integers(0, 1 << 16, size=20_000, dtype=np.uint64) << 16) | 0x8000,
                           np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000, 0x00000001,
                                     0x00008000, 0x80000000, 0x7FC00000, 0x7F800001],
                                    dtype=np.uint64)]).astype(np.uint32)
    f = bits.view(np.float32)
    got = _run(tool, "f", f)
    with np.errstate(invalid="ignore"):
        want = O.f64_to_bf16(f.astype(np.float64))
    nan = np.isnan(f)
    # a float NaN keeps its sign and payload bits in f2bf (quiet bit set); the
    # oracle writes the canonical NaN. Both must be NaN patterns.
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x007F) != 0)
    bad = np.flatnonzero((got != want) & ~nan)
    assert bad.size == 0, (f"{bad.size} differ, e.g. bits={[hex(v) for v in bits[bad[:4]]]} "
                           f"got={[hex(v) for v in got[bad[:4]]]} "
                           f"want={[hex(v) for v in want[bad[:4]]]}")
