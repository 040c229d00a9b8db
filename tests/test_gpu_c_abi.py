"""The C ABI from plain C: tests/c_abi/abi_check.c (built by build(); no
Python or torch in that process) allocates with hipMalloc, sizes the prefill
workspace with the query, runs kda_chunk_fwd (fp32, two packed sequences, an
initial state), kda_decode_step on its final state, kda_decode_replay with
ragged counts and an in-place commit, and kda_chunk_fwd with unbounded decay set
through kda_fused_opts, and checks each result against the fp64 oracle
(normwise 1e-4, fp32).  It runs as a child process under a time limit.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "c_abi"))
import build_abi_check  # noqa: E402


def test_plain_c_consumer():
    print("case C consumer: chunk_fwd + decode_step + decode_replay + unbounded chunk_fwd, fp32", flush=True)
    exe = build_abi_check.BIN
    if not os.path.exists(exe):
        exe = build_abi_check.build()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=100)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
