"""The C ABI driven from plain C: tests/c_abi/gdn_c_check.c allocates device
memory with the HIP runtime's C API, calls gdn_verify and
gdn_commit_all_layers through include/gdn_replay.h (no Python or PyTorch in
that process) and checks outputs and committed states against the CPU oracle
(1e-5 normwise), untouched slots bit for bit and the padding row."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "gdn_c_check")


@pytest.mark.gpu
def test_c_program_verify_and_commit_match_the_oracle():
    assert os.path.exists(EXE), "C check not built: python -c 'import __graft_entry__ as g; g.build()'"
    print("running", EXE, flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "c-abi check:" in r.stdout and r.stdout.strip().endswith("ok")
