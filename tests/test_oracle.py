"""The CPU oracle against what the mathematics fixes (runs without a GPU)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle, pin):
    pin(oracle)


def test_oracle_uses_threads(oracle):
    assert oracle.num_threads() >= 1


def test_stale_library_is_rebuilt(tmp_path):
    """load() rebuilds the default library when oracle_gemm.c is newer than
    it (or it is missing), so an edited oracle is never run from an old build."""
    import os

    import oracle as oracle_pkg
    src = tmp_path / "oracle_gemm.c"
    lib = tmp_path / "liboracle_gemm.so"
    src.write_text(open(oracle_pkg.SOURCE).read())
    assert oracle_pkg._stale(str(lib), str(src))             # missing
    oracle_pkg.build(str(src), str(lib))
    os.utime(src, (1_000_000, 1_000_000))
    os.utime(lib, (2_000_000, 2_000_000))
    assert not oracle_pkg._stale(str(lib), str(src))
    os.utime(src, (3_000_000, 3_000_000))                    # source edited after the build
    assert oracle_pkg._stale(str(lib), str(src))
