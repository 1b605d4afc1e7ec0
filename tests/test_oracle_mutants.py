"""Every plausible mistake planted in a copy of the oracle is caught by a pin.

Each mutant is the oracle's C source with one textual change, built with gcc
into a temporary directory; the pins of ``oracle_pins`` are run against it and
at least one of them must fail.  This shows that the pins would notice a
dropped term, a wrong sign, a wrong index or stride, a transposed operand, or
a wrong rounding rule in the oracle."""
import importlib.util
import os
import shutil
import sys
import tempfile

import pytest

import oracle as oracle_pkg
import oracle_pins as pins

MUTANTS = {
    "drop_last_term": ("k < K; ++k", "k < K - 1; ++k"),
    "skip_first_term": ("int64_t k = 0; k < K", "int64_t k = (K > 1); k < K"),
    "wrong_sign": ("s += decode_bf16", "s -= decode_bf16"),
    "wrong_sign_rowmajor": ("acc[j] += a *", "acc[j] -= a *"),
    "transposed_b": ("decode_bf16(B[k * ldb + j])", "decode_bf16(B[j * ldb + k])"),
    "lda_ignored": ("A[i * lda + k]", "A[i * K + k]"),
    "ldb_off_by_one_nk": ("decode_bf16(B[j * ldb + k])", "decode_bf16(B[j * (ldb - 1) + k])"),
    "ldb_off_by_one_kn": ("decode_bf16(B[k * ldb + j])", "decode_bf16(B[k * (ldb - 1) + j])"),
    "double_rounding": ("    if (isnan(x))\n        return 0x7FC0;",
                        "    x = (double)(float)x;\n    if (isnan(x))\n        return 0x7FC0;"),
    "round_down_above_half": ("r = fl + 1.0;\n    else if", "r = fl;\n    else if"),
    "ties_away": ("r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "r = fl + 1.0;"),
    "ties_down": ("r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "r = fl;"),
    "no_subnormal_quantum": ("(E < -126) ? -133 : (E - 7)", "(E - 7)"),
    "lose_sign": ("uint16_t sign = signbit(x) ? 0x8000 : 0x0000;", "uint16_t sign = 0;"),
    "noncanonical_nan": ("return 0x7FC0;", "return 0x7FFF;"),
    "overflow_saturates": ("return (uint16_t)(sign | 0x7F80);\n\n    float",
                           "return (uint16_t)(sign | 0x7F7F);\n\n    float"),
    "c_decode_shift_15": ("uint32_t w = (uint32_t)h << 16;", "uint32_t w = (uint32_t)h << 15;"),
}

# Mistakes in the Python decoder (oracle.bf16_bits_to_f64), which every GPU
# tolerance check uses: each is planted in a copy of the oracle package that
# loads the real C library.
PY_MUTANTS = {
    "py_decode_no_shift": ("(bits.astype(np.uint32) << 16)", "(bits.astype(np.uint32))"),
    "py_decode_shift_15": ("(bits.astype(np.uint32) << 16)", "(bits.astype(np.uint32) << 15)"),
    "py_decode_drops_sign": ("bits = np.asarray(bits, dtype=np.uint16)\n",
                             "bits = np.asarray(bits, dtype=np.uint16) & 0x7FFF\n"),
}


def _first_failure(o):
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError as e:
            return pin.__name__, str(e)[:200]
    return None


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    src = open(oracle_pkg.SOURCE).read()
    assert src.count(old) >= 1, "mutation site for %s not found" % name
    mutated = src.replace(old, new)
    path_c = os.path.join(workdir, name + ".c")
    with open(path_c, "w") as f:
        f.write(mutated)
    so = oracle_pkg.build(path_c, os.path.join(workdir, "lib" + name + ".so"))
    caught = _first_failure(oracle_pkg.load(so))
    assert caught is not None, "mutant %s passed every pin" % name


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_decoder_mutant_is_caught(name, workdir):
    old, new = PY_MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle_pkg.SOURCE), "__init__.py")).read()
    assert src.count(old) == 1, "mutation site for %s not found" % name
    pkg_dir = os.path.join(workdir, "oracle_" + name)
    os.makedirs(pkg_dir, exist_ok=True)
    path = os.path.join(pkg_dir, "__init__.py")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    mod_name = "oracle_mutant_" + name
    spec = importlib.util.spec_from_file_location(mod_name, path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[mod_name] = mod
    try:
        spec.loader.exec_module(mod)
        o = mod.load(oracle_pkg.load().path)          # the real C library, the mutated decoder
        assert type(o).__module__ == mod_name
        assert _first_failure(o) is not None, "mutant %s passed every pin" % name
    finally:
        del sys.modules[mod_name]


def test_pins_use_the_decoder_gpu_checks_use():
    """The Python decoder the pins check is the very function the GPU tests
    and the smoke check decode with."""
    import oracle_pins
    assert oracle_pins._module_decoder(oracle_pkg.load()) is oracle_pkg.bf16_bits_to_f64
