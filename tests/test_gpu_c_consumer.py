"""The C ABI used from a plain-C program (tests/c_consumer/vsa_c_example.c):
no Python or torch in the process that calls vsa_forward.  The program draws
the inputs with the seeded generator, runs the forward pass on a stream of its
own, and checks every selection row and every output row against the CPU
oracle (max-abs 2e-2, mean-abs 2e-3, relative RMS 5e-3), on the tiny workload
(1 head, 64 + 1,024 + 64 tokens) and on 3 heads with 2 / 37 / 3 tiles."""
import os
import subprocess

import pytest

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_consumer", "vsa_c_example")


def _exe():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built; run __graft_entry__.build()")
    return EXE


def test_c_consumer_is_built_and_links():
    """Host-only: every library the program needs resolves (ldd)."""
    r = subprocess.run(["ldd", _exe()], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "not found" not in r.stdout, r.stdout
    for lib in ("libvsa.so", "liboracle_vsa.so", "libsynth.so", "libamdhip64.so"):
        assert lib in r.stdout, (lib, r.stdout)


@pytest.mark.gpu
def test_c_consumer_forward_matches_oracle():
    print("[c consumer] tiny and ragged cases", flush=True)
    r = subprocess.run([_exe(), "8"], capture_output=True, text=True, timeout=240)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.count(" ok\n") == 2, r.stdout
