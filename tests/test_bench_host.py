"""Host-side checks of the benchmark driver and its workload generators."""

import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout


@pytest.mark.parametrize("tokens", [1, 447, 448, 449, 16384, 65536, 100003])
def test_request_runs_slots(tokens):
    slots, num_slots = workloads.request_runs_slots(tokens)
    assert slots.dtype == np.int64 and slots.shape == (tokens,)
    assert num_slots % 512 == 0 and slots.min() >= 0 and slots.max() < num_slots
    assert np.unique(slots).size == tokens
    # split into runs of consecutive slots: each starts a 512-slot chunk,
    # holds 448..511 tokens (the last may be shorter), one run per chunk
    breaks = np.flatnonzero(np.diff(slots) != 1) + 1
    starts = np.concatenate([[0], breaks])
    lengths = np.diff(np.concatenate([starts, [tokens]]))
    assert (slots[starts] % 512 == 0).all()
    assert (lengths[:-1] >= 448).all() and (lengths <= 511).all()
    assert np.unique(slots[starts] // 512).size == starts.size == num_slots // 512


def test_cpu_threads_capped():
    sys.path.insert(0, ROOT)
    import bench

    threads, nproc = bench.cpu_threads()
    assert 1 <= threads <= min(16, nproc)


def test_unknown_companion_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--only", "no_such_kernel"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "unknown companion" in r.stderr and not r.stdout


def test_probe_library_exports():
    """The benchmark's probe library builds for gfx950 and exports its
    launchers (no device work here)."""
    import ctypes

    from mxfp4_paged_cache_store_amd import build

    if not os.path.exists(build.PROBE_LIB_PATH):
        build.build_probes()
    lib = ctypes.CDLL(build.PROBE_LIB_PATH)
    for name in ("probe_read", "probe_write", "probe_copy_rows", "probe_copy_wide", "probe_copy_expand",
                 "probe_scatter_dwords", "probe_lds", "probe_lds_pattern", "probe_empty"):
        assert hasattr(lib, name), name
