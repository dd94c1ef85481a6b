"""C-ABI checks that need no GPU: exports, configuration checks, layouts and
the host-side budget allocator (against the oracle's statement of it)."""
import ctypes
import os
import re

import numpy as np
import pytest

import predictive_kv_block_amd as spin
from oracle import spin_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spin.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(spin_\w+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    lib = spin.load()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(spin.EXPORTS) == names


def test_config_validation_and_layout():
    cfg = spin.make_config(1, 96, 524288, 2048)
    n = spin.spin_state_bytes(cfg)
    lay = spin.spin_state_layout_of(cfg)
    assert lay["total"] == n and lay["max_blocks"] == 8192
    assert lay["D"] - lay["V"] >= 96 * 524288 * 4
    for k in ("V", "D", "VB", "step", "request_id", "error", "q8", "wq", "qexp", "bscore", "ukey"):
        assert lay[k] % 256 == 0
    bad = spin.make_config(1, 4, 1024, 64)
    bad.block_size = 32
    with pytest.raises(spin.SpinError) as e:
        spin.spin_state_bytes(bad)
    assert e.value.status == spin.SPIN_EUNSUPPORTED
    bad = spin.make_config(0, 4, 1024, 64)
    with pytest.raises(spin.SpinError) as e:
        spin.spin_state_bytes(bad)
    assert e.value.status == spin.SPIN_EINVAL
    bad = spin.make_config(1, 4, 1024, 64, max_rows=5)
    with pytest.raises(spin.SpinError):
        spin.spin_state_bytes(bad)
    small = spin.make_config(1, 1, 4096, 256, heads=4, head_dim=32)      # predictor-only shape
    assert spin.spin_state_bytes(small) > 0


def test_null_and_range_arguments_rejected_before_any_launch():
    lib = spin.load()
    cfg = spin.make_config(1, 2, 1024, 64)
    out = ctypes.c_void_p()
    assert lib.spin_state_init(ctypes.byref(cfg), None, 0, None, ctypes.byref(out)) == spin.SPIN_EINVAL
    assert lib.spin_state_destroy(None) == spin.SPIN_EINVAL
    assert lib.spin_predict_blocks(None, 0, None, 5000, None, None, None, None) == spin.SPIN_EINVAL
    assert lib.spin_update(None, 0, None, None, None, None, None) == spin.SPIN_EINVAL
    b = spin.SpinBatch(1, 1, 16, 0, None, None)
    assert lib.spin_topk_scores(ctypes.byref(b), 64, None, None, None, None, None, None, 0,
                                None) == spin.SPIN_EINVAL
    # a row long enough for several top-k levels needs a workspace
    big = spin.SpinBatch(2, 1, 8192, 0, None, ctypes.c_void_p(16))
    n = ctypes.c_size_t()
    assert lib.spin_topk_workspace_bytes(ctypes.byref(big), 2048, ctypes.byref(n)) == spin.SPIN_OK
    assert n.value >= 2 * 32 * 2048 * 8
    assert lib.spin_topk_scores(ctypes.byref(big), 2048, ctypes.c_void_p(256), None,
                                ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                                None, 0, None) == spin.SPIN_EINVAL
    assert lib.spin_topk_workspace_bytes(ctypes.byref(big), 2050, ctypes.byref(n)) == spin.SPIN_EINVAL
    assert lib.spin_measure_miss(ctypes.byref(b), 0, None, None, None, None) == spin.SPIN_EINVAL
    p = ctypes.c_void_p(256)
    assert lib.spin_slot_scores(None, 0, ctypes.byref(big), p, None) == spin.SPIN_EINVAL
    assert lib.spin_estimate_miss(ctypes.byref(big), 0, p, p, p, p, p, p, None) == spin.SPIN_EINVAL
    assert lib.spin_estimate_miss(ctypes.byref(big), 8192, p, p, p, p, p, p,
                                  None) == spin.SPIN_EINVAL
    assert lib.spin_estimate_miss(ctypes.byref(big), 2048, p, p, None, p, p, p,
                                  None) == spin.SPIN_EINVAL
    assert lib.spin_estimate_miss(ctypes.byref(b), 64, p, p, p, p, p, p, None) == spin.SPIN_EINVAL
    assert lib.spin_predictor_fidelity(ctypes.byref(big), 2048, p, p, p, p, None,
                                       None) == spin.SPIN_EINVAL
    assert lib.spin_predictor_fidelity(ctypes.byref(big), 0, p, p, p, p, p, None) == spin.SPIN_EINVAL
    assert "invalid" in spin.spin_status_string(spin.SPIN_EINVAL)


@pytest.mark.parametrize("L,mean", [(4, 5000), (1, 6000), (7, 7000), (3, 9500)])
def test_allocate_budgets_matches_oracle(L, mean):
    rng = np.random.default_rng(L * 31 + mean)
    for trial in range(20):
        m = rng.random(L) * (0.5 if trial % 2 else 0.05)
        if trial == 0:
            m[:] = 0.0
        got = spin.spin_allocate_budgets(list(m), mean)
        exp = O.allocate_budgets(m, mean)
        assert got == [int(x) for x in exp]
        assert sum(got) == L * mean
    with pytest.raises(spin.SpinError):
        spin.spin_allocate_budgets([0.1, 1.5], 5000)


@pytest.mark.parametrize("L,G", [(1, 1), (4, 7), (9, 5), (61, 12)])
def test_allocate_budgets_curve_matches_oracle(L, G):
    rng = np.random.default_rng(L * 97 + G)
    for trial in range(25):
        steps = rng.integers(1, 2500, size=G)
        grid = np.cumsum(steps) - steps[0] + int(rng.integers(0, 2500))
        grid = np.minimum(grid, 10000 - (G - 1 - np.arange(G)))     # ascending, <= 10000
        if trial % 3 == 0:
            curve = np.sort(rng.random((L, G)), axis=1)[:, ::-1]   # falling with the keep
        else:
            curve = rng.random((L, G))
        if trial == 1:
            curve = np.round(curve * 4) / 4                           # many equal gains
        mean = int(rng.integers(grid[0], 10001))
        got = spin.spin_allocate_budgets_curve(curve.tolist(), grid.tolist(), mean)
        exp = O.allocate_budgets_curve(curve, grid, mean)
        assert got == [int(x) for x in exp]
    with pytest.raises(spin.SpinError):
        spin.spin_allocate_budgets_curve([[0.1, 0.2]], [5000, 4000], 5000)    # not ascending
    with pytest.raises(spin.SpinError):
        spin.spin_allocate_budgets_curve([[0.1, 0.2]], [6000, 8000], 5000)    # floor above mean
    with pytest.raises(spin.SpinError):
        spin.spin_allocate_budgets_curve([[0.1, 1.5]], [4000, 8000], 5000)    # miss outside [0, 1]


def test_header_is_plain_c_and_links():
    """include/spin.h compiles as C11, and a C program that takes the address
    of every entry point links against libspin.so (the boundary is a C ABI)."""
    import shutil
    import subprocess
    import tempfile

    cc = shutil.which("gcc")
    if cc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    src = "#include \"spin.h\"\n#include <stdio.h>\nint main(void) {\n  void* fns[] = {\n"
    src += ",\n".join(f"    (void*)&{name}" for name in spin.EXPORTS)
    src += "\n  };\n  printf(\"%d\\n\", (int)(sizeof(fns) / sizeof(fns[0])));\n  return 0;\n}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "abi_check.c")
        exe = os.path.join(d, "abi_check")
        with open(c, "w") as f:
            f.write(src)
        lib_dir = os.path.dirname(spin.LIB_PATH)
        r = subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                            "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                            c, "-o", exe, "-L", lib_dir, "-l:libspin.so",
                            "-Wl,--allow-shlib-undefined"],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
