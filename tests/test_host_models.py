"""Host programs that check the kernels' host-side logic, no GPU needed:

* tests/ring_model.cpp replays the vector-memory issue and wait sequence of
  every wave of the persistent forward and dK+dV kernels (their own static
  schedule, loader constants and wait formulas) and checks that each tile is
  complete and the expected one when it is consumed; each planted mistake in
  it must be caught.
* tests/abi_check.cpp drives the C ABI's argument validation (attn_api.hip)
  with rejected arguments, the kernel launchers replaced by stubs that abort.
* tests/sched_check.cpp checks the static schedule builder.
* tests/tile_check.cpp checks the LDS tile layouts: each a permutation of a
  row's chunks, bank-conflict-free column reads for the second product, the
  single-base addresses of the k-slot layout, and that every direct load of
  the stage loaders lands where the tile layout places its chunk.

The ring model, the ABI check, the schedule check and the tile check are
also built with AddressSanitizer and UndefinedBehaviorSanitizer on their
host code."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_forward_backward_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-g"]


def _hipcc():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    return hipcc


def _build(tmp_path, name, sources, extra=()):
    exe = str(tmp_path / name)
    cmd = [_hipcc(), "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", *extra,
           "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(ROOT, s) for s in sources], "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=300, env=env)


def test_ring_model_and_planted_mistakes(tmp_path):
    exe = _build(tmp_path, "ring_model", ["tests/ring_model.cpp"])
    r = _run(exe)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
    for plant in range(1, 7):
        r = _run(exe, str(plant))
        assert r.returncode != 0 and "FAIL" in r.stdout, (plant, r.stdout[-500:])


def test_tile_layouts(tmp_path):
    exe = _build(tmp_path, "tile_check", ["tests/tile_check.cpp"])
    r = _run(exe)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr


@pytest.mark.parametrize("name,sources", [
    ("ring_model", ["tests/ring_model.cpp"]),
    ("tile_check", ["tests/tile_check.cpp"]),
    ("abi_check", ["tests/abi_check.cpp", "attention_forward_backward_amd/csrc/attn_api.hip"]),
    ("sched_check", ["tests/sched_check.cpp"]),
])
def test_host_code_under_sanitizers(tmp_path, name, sources):
    exe = _build(tmp_path, name + "_san", sources, SAN)
    r = _run(exe)
    print(r.stdout[-2000:])
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout[-2000:] + r.stderr[-3000:]
