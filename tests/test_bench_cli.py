"""CPU checks of bench.py's contract that need no GPU: it measures one GPU
only (more is refused with exit code 2 before anything touches a device), and
its algorithmic byte counts -- the numerators of every GB/s and roofline
figure -- are the documented ones."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from combine_get_dispatch_02_amd.workloads import CONFIGS  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_algorithmic_bytes_dsv3():
    wl = CONFIGS["dsv3"]
    T, H, k, E, R = wl.T, wl.H, wl.k, wl.E, wl.R
    N = T * k
    b = bench.algorithmic_bytes(wl)
    # combine: token_row and weights read, k rows gathered per token, one row written
    assert b["combine"] == 528_744_448 == 4 * T * k + 4 * T * k + 2 * N * H + 2 * T * H
    # dispatch: ids and weights read, x read once, N rows written, source index,
    # weight and token_row per slot, expert and rank offsets
    assert b["dispatch"] == 529_269_800
    assert b["dispatch"] - b["combine"] == (12 * T * k + 4 * N + 4 * N + 4 * T * k + 4 * (E + 1) + 4 * (R + 1)) \
        - (8 * T * k)
    # the FP8 rows: one code byte per channel plus one fp32 scale per 128 channels
    assert b["dispatch"] - b["dispatch_fp8"] == 2 * N * H - (N * H + 4 * N * (H // 128))
    # the payload convention of the page's own benchmark: one bf16 row per (token, expert) pair each way
    assert 2 * 2 * N * H == 939_524_096


def test_algorithmic_bytes_deduplicated_and_padded():
    wl = CONFIGS["tiny"]
    T, H, k, E, R = wl.T, wl.H, wl.k, wl.E, wl.R
    n, m = 200, T * k - 5
    b = bench.algorithmic_bytes(wl, n_ht=n, n_ll=m)
    assert b["combine_ht"] == 4 * T * R + 2 * n * H + 2 * T * H
    assert b["combine_ll"] == 8 * T * k + 2 * m * H + 2 * T * H
    assert b["dispatch_ll"] - b["dispatch_ll_fp8"] == 2 * m * H - (m * H + 4 * m * (H // 128))
