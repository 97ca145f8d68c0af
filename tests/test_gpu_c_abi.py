"""The library driven from plain C (tests/c/abi_client.c, built by __graft_entry__.build()):
GDN and KDA plans, fused and split, encode / unpack / identity step (readout = S_hat^T q) /
regular step / status, with device memory from the HIP runtime API and no Python in the
process."""
import os
import subprocess

import pytest

import paritylib as P

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c", "abi_client")


def test_c_client_runs_the_path():
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c/abi_client is not built; run __graft_entry__.build() first")
    P.log("[c-abi] running tests/c/abi_client")
    res = subprocess.run([CLIENT], capture_output=True, text=True, timeout=120)
    P.log(res.stdout.strip())
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c-abi: ok" in res.stdout
    assert res.stdout.count("identity-step readout") == 4
