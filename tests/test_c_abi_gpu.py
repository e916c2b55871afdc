"""tri_score and tri_select_compact from a plain C program on the GPU.

tests/c/score_from_c.c includes triattn.h and the HIP runtime C API,
allocates every buffer itself with hipMalloc and calls the library with no
Python or torch in its process.  It reads the inputs this test writes as
raw arrays and writes the scores and kept indices back.  Scores must
match the oracle within the usual bar (1e-4 * max(1, |ref|), floored at the
fp32 resolution of the raw scores); kept indices must equal the oracle's
top-B of the GPU's own scores, bit for bit.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
import rope_aware_key_amd as R
import synth
from harness import check_scores, oracle_unit, units_of, z_floor

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_score_and_select_from_c(tmp_path):
    shape = synth.Shape(128, 8, 2, 2)
    lens, budgets = [300, 1000, 77, 0], [64, 500, 100, 5]
    case = synth.build_case("c_abi", shape, lens, budgets, device="cpu", seed=31)
    d, Hq, Hkv, L, S = 128, 8, 2, 2, len(lens)
    files = {
        "cu_len.bin": np.asarray(case.cu_len, np.int64),
        "cur_pos.bin": np.asarray(case.cur_pos, np.int32),
        "budget.bin": np.asarray(case.budget, np.int32),
        "k.bin": case.k.numpy().view(np.uint16),
        "k_pos.bin": case.k_pos.numpy().astype(np.int32),
        "centre.bin": case.q_centre.numpy().astype(np.float32),
        "absmean.bin": case.q_absmean.numpy().astype(np.float32),
        "R.bin": case.q_R.numpy().astype(np.float32),
    }
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(tmp_path / name)

    exe = tmp_path / "score_from_c"
    lib_dir = os.path.dirname(R.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "c", "score_from_c.c"),
                    "-L", lib_dir, "-ltriattn", "-L", "/opt/rocm/lib", "-lamdhip64",
                    f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    print(f"running the C caller on {S} sequences", flush=True)
    r = subprocess.run([str(exe), str(tmp_path), str(d), str(Hq), str(Hkv), str(L), str(S)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    scores = np.fromfile(tmp_path / "scores.bin", dtype=np.float32)
    kept = np.fromfile(tmp_path / "kept.bin", dtype=np.int32)
    assert scores.shape[0] == case.total_rows() and kept.shape[0] == case.total_out_rows()
    for (s, l, g) in units_of(case):
        if case.seq_len(s) == 0:
            continue
        start, n, ref, Sref, mu, sigma = oracle_unit(case, s, l, g)
        check_scores(scores[start:start + n], ref, f"unit {(s, l, g)}", z_floor(Sref, sigma))
        ostart, b = case.unit_out_rows(s, l, g)
        np.testing.assert_array_equal(kept[ostart:ostart + b],
                                      O.select_topb(scores[start:start + n], int(case.budget[s])),
                                      err_msg=f"kept of unit {(s, l, g)}")
