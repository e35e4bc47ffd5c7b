"""The C ABI used from plain C (needs an MI355X): tests/c_abi_check.c, built next to
libdg.so by the package's build step, runs the sampler head, acceptance, renoise,
self-conditioning and the stop test on device buffers it allocates itself, and checks
them against closed forms (all-zero embeddings: entropy ln V, argmax 0, nothing
accepted, z = 0) and two refused calls."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "block_ar_canvas_amd",
                   "c_abi_check")


def test_c_program_runs_a_step_through_the_c_abi():
    assert os.path.exists(EXE), "c_abi_check is built with libdg.so by the package's build step"
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and "c_abi_check: ok" in res.stdout, res.stdout + res.stderr
