"""The call-epoch bookkeeping of the lookback workspaces (csrc/call_epoch.hpp), on the CPU.

tests/epoch_model.hip builds the header's own functions for the host and runs simulated
workgroups through them one atomic step at a time, in random interleavings (deterministic per
seed).  After every call all counts must be back at zero, every slot line must hold the next
epoch, and every wave of the call must have read the call's epoch, over grids of 1 to
thousands of workgroups (fewer and more than the 256 slot lines), 1 to 4 reading waves per
workgroup, and epochs that wrap at 2^30.  The order the kernels follow (every read of a
workgroup before its count_done, behind a barrier) must hold in every run; the order without
that barrier must be caught."""
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "linear_recurrence_scan_linrec_amd" / "csrc"
EPOCH_WRAP = (1 << 30) - 2   # two calls before the 30-bit epoch wraps to 0
GRIDS = ["1", "2", "3", "5", "37", "255", "256", "257", "511", "600", "2344"]


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(hipcc).exists():
        pytest.skip("hipcc not found")
    exe = tmp_path_factory.mktemp("epoch_model") / "epoch_model"
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", f"-I{CSRC}",
           str(ROOT / "tests" / "epoch_model.hip"), "-o", str(exe), "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    return exe


def run(exe, order, seed, waves, resident, calls, start, grids):
    args = [str(exe), order, str(seed), str(waves), str(resident), str(calls), str(start), *grids]
    return subprocess.run(args, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("waves,resident,start,seed", [
    (1, 16, 0, 11),            # one carry wave (the one-tile plans' common case)
    (2, 16, 0, 12),            # two carry waves (128-channel slabs)
    (4, 64, 0, 13),            # four carry waves, many resident workgroups
    (2, 8, EPOCH_WRAP, 14),    # through the wrap of the 30-bit epoch
])
def test_kernel_order_keeps_every_call_on_its_epoch(model, waves, resident, start, seed):
    r = run(model, "ordered", seed, waves, resident, 2, start, GRIDS)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]
    # every call of every grid ran, each with one read per wave per workgroup
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("grid ")]
    assert len(lines) == 2 * len(GRIDS)
    for ln, grid in zip(lines, [g for g in GRIDS for _ in range(2)]):
        assert ln.split()[4] == str(int(grid) * waves), ln


def test_order_without_the_barrier_is_caught(model):
    """count_done straight after the count, with a second wave's read after it: some
    interleaving lets that read return the next call's epoch, and the model must find it."""
    caught = 0
    for seed in range(1, 7):
        r = run(model, "unordered", seed, 2, 16, 3, 0, GRIDS[:8])
        if r.returncode == 1 and "a wave read epoch" in r.stdout:
            caught += 1
        else:
            assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert caught >= 3, caught
