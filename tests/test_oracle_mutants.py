"""Planted mistakes in the oracle, on the CPU: each test below rebuilds the
oracle module with one plausible slip written into its source (a dropped
term, a wrong sign, bias, index order or rounding point) and checks that at
least one pin of tests/test_oracle_pins.py fails against it.  A mistake no
pin catches is a hole in the oracle's pinning.

The pins are run against the mutant by pointing the `oracle` package's
names at the mutant module's functions for the duration of one test."""

import inspect

import pytest

import oracle
import oracle.qmm_oracle as qo
import test_oracle_pins as pins

SRC = inspect.getsource(qo)

# (name, text in the oracle's source, the planted mistake)
MUTANTS = [
    ("nibble order", "lo = codes & 0xF\n    hi = codes >> 4", "hi = codes & 0xF\n    lo = codes >> 4"),
    ("Q6_K high-bit crumb order", "parts = [(b >> (2 * i)) & 3 for i in range(4)]",
     "parts = [(b >> (6 - 2 * i)) & 3 for i in range(4)]"),
    ("E4M3 exponent bias", "np.ldexp(1.0, ex - 7)", "np.ldexp(1.0, ex - 8)"),
    ("E4M3 subnormal step", "m * 2.0 ** -9", "m * 2.0 ** -10"),
    ("E8M0 bias", "np.ldexp(1.0, e - 127))", "np.ldexp(1.0, e - 128))"),
    ("E2M1 sign dropped", "return np.where(c & 8, -1.0, 1.0) * mag", "return mag"),
    ("E2M1 magnitudes 1.5 and 2 swapped", "E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)",
     "E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 2.0, 1.5, 3.0, 4.0, 6.0)"),
    ("affine scale and bias swapped",
     "s = np.repeat(sb[..., 0], 64, axis=-1)\n        b = np.repeat(sb[..., 1], 64, axis=-1)",
     "s = np.repeat(sb[..., 1], 64, axis=-1)\n        b = np.repeat(sb[..., 0], 64, axis=-1)"),
    ("affine bias dropped", "return s * q + b", "return s * q"),
    ("NVFP4 tensor scale dropped", "return v * sc * g", "return v * sc"),
    ("Q6_K zero point 31", "return d * sc * (q - 32)", "return d * sc * (q - 31)"),
    ("Q6_K high bits shifted by 3", "q = lo | (hi << 4)", "q = lo | (hi << 3)"),
    ("Q6_K sub-block scale unsigned", "astype(np.int8).astype(np.float64), 16",
     "astype(np.uint8).astype(np.float64), 16"),
    ("residual dropped", "        y = y + r\n        mag = mag + np.abs(r)\n    return y, mag\n\n\ngemm = gemv",
     "        mag = mag + np.abs(r)\n    return y, mag\n\n\ngemm = gemv"),
    ("silu sign", "return g / (1.0 + np.exp(-g))", "return g / (1.0 + np.exp(g))"),
    ("gate and up swapped", "h32 = (silu(gu[:inter]) * gu[inter:])", "h32 = (silu(gu[inter:]) * gu[:inter])"),
    ("combine weight dropped", "y += wt * (wd @ h)", "y += (wd @ h)"),
    ("router ties to the higher id", "key=lambda e: (-lg[t, e], e)", "key=lambda e: (-lg[t, e], -e)"),
    ("router softmax not renormalised", "wts[t] = z / z.sum()",
     "wts[t] = z / np.exp(lg[t] - top.max()).sum()"),
    ("shared expert gets no rows", "counts[E + s] = T", "counts[E + s] = 0"),
    ("last tile not cut", "min(tile_rows, counts[e] - r)", "tile_rows"),
    ("MXFP4 shared exponent off by one", "shared = (e - 1) - 2", "shared = e - 2"),
    ("MXFP4 ties to the lower code",
     "idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))",
     "idx = cand.argmax(axis=-1)"),
    ("W4A4 activations not quantized", "xq = mxfp4_dequantize_activations(codes, scales)",
     "xq = bf16(x_bits)"),
    ("Hadamard not normalised", "h = sylvester_hadamard(HADAMARD_BLOCK) / np.sqrt(HADAMARD_BLOCK)",
     "h = sylvester_hadamard(HADAMARD_BLOCK)"),
    ("Sylvester blocks in the wrong places", "h = np.block([[h, h], [h, -h]])",
     "h = np.block([[h, -h], [h, h]])"),
    ("prepare transforms before scaling", "v = x * s\n    y = _blocks_transform(v)",
     "v = x * s\n    y = _blocks_transform(x) * s"),
    ("finish scales before transforming", "out = _blocks_transform(v) * s", "out = _blocks_transform(v * s)"),
    ("bf16 rounding ties away from zero", "r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16", "r = (u + 0x8000) >> 16"),
    ("bf16 half ulp one binade off", "np.ldexp(1.0, e - 9)", "np.ldexp(1.0, e - 8)"),
]


def _mutant_module(old, new):
    assert SRC.count(old) == 1, f"mutation site not unique: {old!r}"
    code = compile(SRC.replace(old, new), "qmm_oracle_mutant.py", "exec")
    ns = {"__name__": "qmm_oracle_mutant"}
    exec(code, ns)
    return ns


def _pin_cases():
    """Every pin of test_oracle_pins.py with its parameter sets, cheapest
    first (the routing statistics at T = 8192 last)."""
    cases = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            cases.append((name, fn, {}))
            continue
        assert len(marks) == 1
        argnames, values = marks[0].args[0], marks[0].args[1]
        names = [a.strip() for a in argnames.split(",")]
        for v in values:
            v = v if len(names) > 1 else (v,)
            cases.append((name, fn, dict(zip(names, v))))
    cases.sort(key=lambda c: c[0] == "test_routing_statistics_against_printed_values")
    return cases


CASES = _pin_cases()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(monkeypatch, name, old, new):
    ns = _mutant_module(old, new)
    for attr in dir(qo):
        if not attr.startswith("__") and attr in ns and hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, ns[attr])
    caught = []
    for pin, fn, kw in CASES:
        try:
            fn(**kw)
        except Exception as e:  # an assertion or any error the slip causes
            caught.append(f"{pin}{kw or ''}: {type(e).__name__}")
            break
    assert caught, f"no pin fails with the planted mistake '{name}'"


def test_unmutated_oracle_passes_every_pin():
    """The harness itself: the pins all pass on the oracle as it is."""
    for pin, fn, kw in CASES:
        fn(**kw)
