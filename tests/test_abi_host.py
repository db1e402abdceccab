"""The C-ABI library on the host: it loads, exports every declared symbol, and its host-side
logic (status strings, plans, argument checks that return before any HIP call) behaves.
No kernel runs here."""
import ctypes
import os
import re
from pathlib import Path

import pytest

from linear_recurrence_scan_linrec_amd import linrec as binding

INCLUDE = Path(__file__).resolve().parent.parent / "include"
HEADER = INCLUDE / "linrec.h"
STREAM_HEADER = INCLUDE / "linrec_stream.h"


def declared_functions(header=HEADER):
    text = re.sub(r"/\*.*?\*/", "", header.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(linrec_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert names, "no declarations parsed from include/linrec.h"
    lib = ctypes.CDLL(str(binding.LIBRARY))
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"
    assert sorted(binding.EXPORTED) == names


def test_every_header_is_covered():
    """Each header under include/ belongs to one of the two libraries checked here."""
    assert sorted(p.name for p in INCLUDE.glob("*.h")) == ["linrec.h", "linrec_stream.h"]


def test_stream_ceiling_library_exports_and_checks_arguments():
    from linear_recurrence_scan_linrec_amd import stream_ceiling as sc

    names = declared_functions(STREAM_HEADER)
    lib = sc.library()
    assert names == sorted(sc.EXPORTED) and all(hasattr(lib, n) for n in names)
    f = lib.linrec_stream_r2w1
    # checks that return before any HIP call
    assert f(None, None, None, 0, 1, 4, 2, None) == 0                       # empty: no-op
    assert f(None, None, None, 1024, 1, 3, 2, None) == 1                    # unroll
    assert b"unroll" in lib.linrec_stream_last_error()
    assert f(None, None, None, 1024, 1, 4, 0, None) == 1                    # groups per CU
    assert f(None, None, None, 1000, 1, 1, 2, None) == 1                    # not whole segments
    assert f(None, None, None, 1024, 3, 1, 2, None) == 1                    # rows do not divide it
    assert f(None, None, None, 1024, 1, 1, 2, None) == 1                    # null buffers
    base = 1 << 32
    assert f(base, base + 8192, base + 16, 1024, 1, 1, 2, None) == 1         # z overlaps x
    assert b"overlaps" in lib.linrec_stream_last_error()
    assert f(base + 4, base + 8192, base + 65536, 1024, 1, 1, 2, None) == 1  # misaligned
    assert b"aligned" in lib.linrec_stream_last_error()

    c = lib.linrec_stream_column_walk
    assert c(None, None, None, 0, 4096, 256, 8, 2, 8, None) == 0             # empty: no-op
    assert c(None, None, None, 32, 4096, 256, 4, 2, 8, None) == 1            # lanes
    assert b"lanes" in lib.linrec_stream_last_error()
    assert c(None, None, None, 32, 4096, 256, 8, 3, 8, None) == 1            # waves
    assert c(None, None, None, 32, 4096, 256, 8, 2, 16, None) == 1           # steps per lane
    assert c(None, None, None, 32, 4096, 100, 8, 2, 8, None) == 1            # D not whole slabs
    assert c(None, None, None, 1, 1 << 20, 1024, 8, 2, 8, None) == 1         # a batch row past 2 GiB
    assert b"2 GiB" in lib.linrec_stream_last_error()
    assert c(None, None, None, 32, 4096, 256, 8, 2, 8, None) == 1            # null buffers
    n = 32 * 4096 * 256 * 4
    assert c(base, base + 2 * n, base + 16, 32, 4096, 256, 8, 2, 8, None) == 1   # z overlaps x
    assert b"overlaps" in lib.linrec_stream_last_error()
    assert c(base + 4, base + 2 * n, base + 4 * n, 32, 4096, 256, 8, 2, 8, None) == 1   # misaligned
    assert b"aligned" in lib.linrec_stream_last_error()


def test_status_strings():
    assert binding.linrec_status_string(0) == "success"
    assert binding.linrec_status_string(2) == "output overlaps another buffer"
    assert binding.linrec_status_string(99) == "unknown status"


def test_empty_problems_are_noops_without_touching_the_device():
    for shape in ((0, 10, 10), (10, 0, 10), (10, 10, 0)):
        assert binding.linrec_scan_raw(0, 0, 0, *shape, 0) == binding.LINREC_OK


def test_invalid_sizes_and_null_buffers():
    assert binding.linrec_scan_raw(0, 0, 0, -1, 4, 4, 0) == binding.LINREC_ERR_INVALID_ARGUMENT
    assert "must be >= 0" in binding.linrec_last_error_message()
    assert binding.linrec_scan_raw(0, 0, 0, 1, 4, 4, 0) == binding.LINREC_ERR_INVALID_ARGUMENT
    assert "non-null" in binding.linrec_last_error_message()
    big = 1 << 40
    assert binding.linrec_scan_raw(64, 128, 256, big, big, 4, 0) == binding.LINREC_ERR_INVALID_ARGUMENT
    assert "overflow" in binding.linrec_last_error_message() and "63 bits" in binding.linrec_last_error_message()


def test_overlap_is_rejected_before_any_hip_call():
    # fake addresses: the overlap check runs before the buffers are looked up
    base = 1 << 32
    n = 2 * 8 * 16
    assert binding.linrec_scan_raw(base, base + 4 * n, base + 8, 2, 8, 16, 0) == binding.LINREC_ERR_OVERLAP
    assert binding.linrec_scan_raw(base, base + 4 * n, base + 4 * n + 4, 2, 8, 16, 0) == binding.LINREC_ERR_OVERLAP


def test_default_tiles_are_supported_for_many_shapes():
    for B in (1, 2, 7, 32):
        for L in (1, 100, 5000):
            for D in (1, 3, 4, 64, 256, 1000, 8192):
                binding.linrec_scan_plan(B, L, D)
                binding.linrec_scan_plan(B, L, D, aligned16=False)


def test_plans_for_the_named_workloads():
    p = binding.linrec_scan_plan(32, 4096, 256)
    assert p["vec"] == 4 and p["lanes_per_row"] <= 64
    assert p["chunks"] * p["steps_per_tile"] >= 4096
    slabs = -(-256 // (p["lanes_per_row"] * p["vec"]))
    assert p["tiles"] == 32 * slabs * p["chunks"]
    p = binding.linrec_scan_plan(2, 262144, 64)
    assert p["lanes_per_row"] <= 16            # several rows of 64 channels per wave instruction
    p = binding.linrec_scan_plan(1, 64, 8)
    assert p["chunks"] == 1 and p["workspace_bytes"] == 0
    p = binding.linrec_scan_plan(3, 100, 7)
    assert p["vec"] == 1                       # D % 4 != 0 takes the 32-bit form
    p = binding.linrec_scan_plan(3, 100, 8, aligned16=False)
    assert p["vec"] == 1
    p = binding.linrec_scan_plan(0, 100, 8)
    assert p["tiles"] == 0 and p["workspace_bytes"] == 0


def test_plan_workspace_covers_status_arrays():
    p = binding.linrec_scan_plan(8, 16384, 1024)
    # four 8-byte status words per (tile, channel): the tile pair's product of decays as an
    # fp32 hi + lo pair, its B, and the inclusive state
    per_entry = 4 * 8
    entries = p["tiles"] * p["lanes_per_row"] * p["vec"]
    header, completion_counters = 512, 256 * 128
    assert p["workspace_bytes"] == header + completion_counters + per_entry * entries


@pytest.fixture
def tile_env():
    old = os.environ.get("LINREC_TILE")
    yield
    if old is None:
        os.environ.pop("LINREC_TILE", None)
    else:
        os.environ["LINREC_TILE"] = old


def test_tile_override(tile_env):
    os.environ["LINREC_TILE"] = "t=8,w=2"
    p = binding.linrec_scan_plan(32, 4096, 256)
    assert (p["steps_per_lane"], p["waves"], p["vec"]) == (8, 2, 4)
    os.environ["LINREC_TILE"] = "vec=1"
    assert binding.linrec_scan_plan(32, 4096, 256)["vec"] == 1
    os.environ["LINREC_TILE"] = "p=8,t=8,w=4,q=2"
    p = binding.linrec_scan_plan(32, 4096, 256)
    assert p["lanes_per_row"] == 8 and p["steps_per_tile"] == 8 * 4 * (64 // 8)
    os.environ["LINREC_TILE"] = "m=1,vec=4,t=16,w=2"
    p = binding.linrec_scan_plan(32, 4096, 256)
    assert (p["mode"], p["steps_per_lane"], p["waves"]) == (1, 16, 2)
    os.environ["LINREC_TILE"] = "w=15,p=32"        # 15 data waves + 2 carry waves > 1024 threads
    with pytest.raises(binding.LinrecError):
        binding.linrec_scan_plan(32, 4096, 256)
    os.environ["LINREC_TILE"] = "w=15,p=16,t=4"
    assert binding.linrec_scan_plan(32, 4096, 256)["waves"] == 15
    # the relay (m=2): at most 2 data waves and one carry wave, else the plan runs as m=0
    os.environ["LINREC_TILE"] = "m=2,t=4,w=2"
    p = binding.linrec_scan_plan(32, 4096, 256)
    assert (p["mode"], p["steps_per_lane"], p["waves"], p["lanes_per_row"]) == (2, 4, 2, 8)
    for demoted in ("m=2,w=4", "m=2,t=8,w=8", "w=4", "p=32"):   # the last two on the default m=2
        os.environ["LINREC_TILE"] = demoted
        assert binding.linrec_scan_plan(32, 4096, 256)["mode"] == 0, demoted
    os.environ["LINREC_TILE"] = "m=2,vec=1,p=64,t=8,w=1"   # 64 channels: one carry wave
    assert binding.linrec_scan_plan(32, 4096, 256)["mode"] == 2
    for bad in ("t=5", "w=3", "w=16", "w=5", "vec=2", "t=16", "m=3", "m=2,vec=4,t=16", "w=14,t=8", "m=-1", "m=0,vec=4,t=16", "x=2", "t", "t=abc", "p=3", "p=128", "p=0",
                "q=-1", "q=65", "d=1"):
        os.environ["LINREC_TILE"] = bad
        with pytest.raises(binding.LinrecError) as err:
            binding.linrec_scan_plan(32, 4096, 256)
        assert err.value.status == binding.LINREC_ERR_INVALID_ARGUMENT
    os.environ["LINREC_TILE"] = "vec=4"
    with pytest.raises(binding.LinrecError):
        binding.linrec_scan_plan(3, 100, 7)   # vec=4 cannot serve D % 4 != 0


# ----------------------------------------------------------------------------- linrec_scan_ex on the host

def desc(B, L, D, dtype=0, reverse=0, base=1 << 32, strides=None, h_init=None, h_final=None):
    """A linrec_scan_desc over fake, well separated addresses (no kernel runs)."""
    es = 4 if dtype == 0 else 2
    n = max(B * L * D, 1)
    st = strides or [(L * D, D)] * 3
    ops = [binding.linrec_operand(base + k * 4 * n * es, *st[k]) for k in range(3)]
    return binding.linrec_scan_desc(B, L, D, dtype, reverse, *ops, h_init, h_final)


def ex_plan(d):
    plan = binding.linrec_plan()
    status = binding.library().linrec_scan_ex_plan(ctypes.byref(d), ctypes.byref(plan))
    return status, {name: getattr(plan, name) for name, _ in binding.linrec_plan._fields_}


def test_ex_plan_of_contiguous_f32_is_linrec_scan_plan():
    for shape in ((32, 4096, 256), (2, 262144, 64), (3, 100, 7), (1, 64, 8)):
        st, p = ex_plan(desc(*shape))
        assert st == binding.LINREC_OK
        assert p == binding.linrec_scan_plan(*shape)


def test_ex_plan_vector_form_needs_aligned_strides():
    assert ex_plan(desc(4, 100, 64, dtype=1))[1]["vec"] == 4
    assert ex_plan(desc(4, 100, 64, dtype=2))[1]["vec"] == 4
    # a time stride that is not a multiple of 4 elements, or an operand 2 elements in
    st = [(100 * 66, 66), (100 * 64, 64), (100 * 64, 64)]
    assert ex_plan(desc(4, 100, 64, strides=st))[1]["vec"] == 1
    d = desc(4, 100, 64, dtype=1)
    d.b.ptr += 4
    assert ex_plan(d)[1]["vec"] == 1
    # broadcast a over batch rows and time (strides 0) keeps the vector form
    st = [(0, 0), (100 * 64, 64), (100 * 64, 64)]
    assert ex_plan(desc(4, 100, 64, strides=st))[1]["vec"] == 4


def test_ex_rejects_bad_descriptors():
    bad = binding.LINREC_ERR_INVALID_ARGUMENT
    lib = binding.library()
    assert lib.linrec_scan_ex(None, None) == bad
    assert lib.linrec_scan_ex(ctypes.byref(desc(2, 8, 16, dtype=3)), None) == bad
    assert "dtype" in binding.linrec_last_error_message()
    for mode in (3, -1):       # 0 forward, 1 reverse, 2 reverse with the decays one step ahead
        assert lib.linrec_scan_ex(ctypes.byref(desc(2, 8, 16, reverse=mode)), None) == bad
        assert "reverse" in binding.linrec_last_error_message()
    assert lib.linrec_scan_ex(ctypes.byref(desc(2, 8, 16, strides=[(128, -16), (128, 16), (128, 16)])), None) == bad
    assert "strides" in binding.linrec_last_error_message()
    # rows of h overlap: time stride below D, or batch rows on top of each other
    assert lib.linrec_scan_ex(ctypes.byref(desc(2, 8, 16, strides=[(128, 16), (128, 16), (128, 8)])), None) == bad
    assert "overlap one another" in binding.linrec_last_error_message()
    assert lib.linrec_scan_ex(ctypes.byref(desc(2, 8, 16, strides=[(128, 16), (128, 16), (64, 16)])), None) == bad
    # time-major h (batch stride D, time stride B*D) is fine
    assert ex_plan(desc(2, 8, 16, strides=[(128, 16), (128, 16), (16, 32)]))[0] == binding.LINREC_OK
    # an operand not aligned to its element size, a state not aligned to 4 bytes
    d = desc(2, 8, 16, dtype=1)
    d.a.ptr += 1
    assert lib.linrec_scan_ex(ctypes.byref(d), None) == bad
    assert "aligned" in binding.linrec_last_error_message()
    assert lib.linrec_scan_ex(ctypes.byref(desc(2, 8, 16, h_init=(1 << 40) + 2)), None) == bad
    assert lib.linrec_scan_ex(ctypes.byref(desc(2, 8, 16, h_final=(1 << 40) + 6)), None) == bad
    # a time stride so large that one tile would span 1 GiB or more
    assert ex_plan(desc(2, 8000, 16, strides=[(0, 1 << 22), (128000, 16), (128000, 16)]))[0] == bad
    assert "1 GiB" in binding.linrec_last_error_message()


def test_ex_overlaps_are_rejected_before_any_hip_call():
    lib = binding.library()
    over = binding.LINREC_ERR_OVERLAP
    d = desc(2, 8, 16)
    d.h.ptr = d.a.ptr + 64
    assert lib.linrec_scan_ex(ctypes.byref(d), None) == over
    d = desc(2, 8, 16, h_final=None)
    d.h_final = d.b.ptr + 4
    assert lib.linrec_scan_ex(ctypes.byref(d), None) == over
    d = desc(2, 8, 16)
    d.h_init = d.h.ptr
    assert lib.linrec_scan_ex(ctypes.byref(d), None) == over
    d = desc(2, 8, 16, h_init=1 << 44)
    d.h_final = d.h_init
    assert lib.linrec_scan_ex(ctypes.byref(d), None) == over
    # a and b may alias, and h_init may alias an input
    d = desc(2, 8, 16)
    d.b.ptr = d.a.ptr
    d.h_init = d.a.ptr
    assert ex_plan(d)[0] == binding.LINREC_OK


def test_ex_empty_problems_without_a_final_state_are_noops():
    lib = binding.library()
    for shape in ((0, 10, 10), (10, 0, 10), (10, 10, 0)):
        d = desc(*shape)
        d.a.ptr = d.b.ptr = d.h.ptr = None
        assert lib.linrec_scan_ex(ctypes.byref(d), None) == binding.LINREC_OK


# The plans the tile rules pick for the named workloads (on the 256-CU part the plan entry points
# assume), as measured and chosen: a change to the rules shows up here first.
DEFAULT_PLANS = {
    # (B, L, D, dtype): (vec, steps_per_lane, waves, lanes_per_row, mode)
    (32, 4096, 256, 0): (4, 8, 1, 8, 2),        # fp32 pages shape: the relay over 128-byte rows, 64-step tiles
    (16, 512, 8192, 0): (4, 8, 4, 32, 0),       # wide_channels: local carry, 4 sequences per workgroup
    (8, 16384, 1024, 0): (4, 8, 1, 8, 2),       # near_unit_resets: the relay
    (2, 262144, 64, 0): (4, 8, 7, 8, 1),        # long_sequence: one tile per workgroup, two per CU
    (32, 4096, 256, 1): (4, 16, 7, 16, 1),      # bf16 pages shape: one tile per workgroup (1280 tiles)
    (16, 512, 8192, 1): (4, 8, 8, 64, 0),       # bf16 wide_channels: local carry over 64-lane slabs
    (8, 16384, 1024, 1): (4, 8, 8, 32, 0),      # bf16 near_unit_resets: persistent lookback
    (2, 262144, 64, 1): (4, 16, 7, 16, 1),      # bf16 long_sequence: one tile per workgroup
}


@pytest.mark.parametrize("key", sorted(DEFAULT_PLANS), ids=lambda k: f"{'f32' if k[3] == 0 else 'bf16'}-{k[0]}x{k[1]}x{k[2]}")
def test_default_plans_of_the_named_workloads(key):
    B, L, D, dtype = key
    status, p = ex_plan(desc(B, L, D, dtype=dtype))
    assert status == binding.LINREC_OK
    assert (p["vec"], p["steps_per_lane"], p["waves"], p["lanes_per_row"], p["mode"]) == DEFAULT_PLANS[key]


def test_workspace_sizes_without_a_device():
    """The workspace-size entry points are host arithmetic (on a host without a GPU they assume a
    256-CU part, like the plan entry points)."""
    lib = binding.library()
    for shape in ((8, 16384, 1024), (2, 262144, 64), (32, 4096, 256), (3, 100, 7), (1, 64, 8)):
        need = lib.linrec_scan_workspace_bytes(*shape)
        # the larger of the aligned and unaligned plans' needs
        assert need == max(binding.linrec_scan_plan(*shape, aligned16=al)["workspace_bytes"] for al in (True, False))
    assert binding.linrec_scan_plan(1, 64, 8)["workspace_bytes"] == 0   # one chunk: no carry to pass on
    assert lib.linrec_scan_workspace_bytes(-1, 64, 8) == 0
    d = desc(2, 262144, 64)
    out = ctypes.c_size_t(7)
    assert lib.linrec_scan_ex_workspace_bytes(ctypes.byref(d), ctypes.byref(out)) == binding.LINREC_OK
    assert out.value == ex_plan(d)[1]["workspace_bytes"] > 0
    assert lib.linrec_scan_ex_workspace_bytes(ctypes.byref(d), None) == binding.LINREC_ERR_INVALID_ARGUMENT
    assert lib.linrec_scan_ex_workspace_bytes(None, ctypes.byref(out)) == binding.LINREC_ERR_INVALID_ARGUMENT


def test_caller_workspace_entry_points_check_sizes_before_any_hip_call():
    lib = binding.library()
    assert lib.linrec_scan_ws(None, None, None, 0, 5, 5, None, 0, None) == binding.LINREC_OK
    assert lib.linrec_scan_ws(None, None, None, -1, 5, 5, None, 0, None) == binding.LINREC_ERR_INVALID_ARGUMENT
    d = desc(0, 10, 10)
    d.a.ptr = d.b.ptr = d.h.ptr = None
    assert lib.linrec_scan_ex_ws(ctypes.byref(d), None, 0, None) == binding.LINREC_OK
    assert lib.linrec_scan_ex_ws(None, None, 0, None) == binding.LINREC_ERR_INVALID_ARGUMENT


def test_decays_ahead_needs_the_reverse_scan():
    """a_ahead selects the reverse form whose decays are one time step ahead; the binding
    refuses it for a forward scan before touching any buffer."""
    import torch
    x = torch.zeros(1, 4, 4)
    with pytest.raises(ValueError, match="reverse"):
        binding.linrec_scan(x, x, a_ahead=True)
    d = binding.make_desc(x, x, x, reverse=True, a_ahead=True)
    assert d.reverse == 2
    assert binding.make_desc(x, x, x, reverse=True).reverse == 1
