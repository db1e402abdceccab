"""linrec_scan_ex_noalloc through the C ABI: the same results as linrec_scan_ex (its kernels, its
plans) with the lookback workspace in the library's static scratch, on calls in a row whose
second is smaller, in 16-bit storage with both states and reverse time, under graph capture with
no warm-up, and a clear error past the scratch's 16 MiB.  Bars: the fp32 bar
|h - ref| <= 1e-4 * (1 + |ref|) against the float64 oracle for both entry points, and the same
bar between the two entry points' outputs."""
import ctypes
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linrec_inputs as li  # noqa: E402
import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def lr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrence_scan_linrec_amd import linrec as binding
    return binding


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def ratio(x, ref):
    return float(np.max(np.abs(x - ref) / (1.0 + np.abs(ref))))


def run_both(lr, a, b, **kw):
    """(h from linrec_scan_ex_noalloc, h from linrec_scan_ex), same inputs, same stream."""
    lib = lr.library()
    s = torch.cuda.current_stream().cuda_stream
    out = []
    for fn in (lib.linrec_scan_ex_noalloc, lib.linrec_scan_ex):
        h = torch.full_like(a, float("nan"))
        hf = torch.empty((a.shape[0], a.shape[2]), device="cuda") if "h_init" in kw else None
        d = lr.make_desc(a, b, h, kw.get("h_init"), hf, kw.get("reverse", False))
        status = fn(ctypes.byref(d), s)
        assert status == lr.LINREC_OK, lr.linrec_last_error_message()
        out.append((h, hf))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("first,second", [((2, 65536, 64), (1, 20000, 64)), ((4, 30000, 24), (2, 5000, 24))],
                         ids=["long", "narrow"])
def test_noalloc_matches_linrec_scan_ex_on_calls_in_a_row(lr, first, second):
    for k, shape in enumerate((first, second)):
        plan = lr.linrec_scan_plan(*shape)
        assert plan["chunks"] > 1 and plan["workspace_bytes"] > 0      # looks back: uses the scratch
        a_np, b_np = li.make_inputs(*shape, seed=3000 + k, a_lo=0.9, a_hi=1.0)
        a, b = torch.from_numpy(a_np).cuda(), torch.from_numpy(b_np).cuda()
        (h_na, _), (h_ex, _) = run_both(lr, a, b)
        ref = oracle.linrec_oracle_f64(a_np, b_np)
        r_na, r_ex, r_pair = ratio(host(h_na), ref), ratio(host(h_ex), ref), ratio(host(h_na), host(h_ex))
        say(f"[noalloc] call {k} {shape}: noalloc {r_na:.3e}, ex {r_ex:.3e}, between {r_pair:.3e}")
        assert r_na <= TOL and r_ex <= TOL and r_pair <= TOL


def test_noalloc_half_storage_states_and_reverse(lr):
    B, L, D = 3, 20000, 64
    a_np, b_np = li.make_inputs(B, L, D, seed=3100, a_lo=0.9, a_hi=1.0)
    a = torch.from_numpy(a_np).cuda().to(torch.bfloat16)
    b = torch.from_numpy(b_np).cuda().to(torch.bfloat16)
    a32, b32 = a.float().cpu().numpy(), b.float().cpu().numpy()
    h0_np = np.random.default_rng(3101).standard_normal((B, D)).astype(np.float32)
    h0 = torch.from_numpy(h0_np).cuda()
    for reverse in (False, True):
        (h_na, f_na), (h_ex, f_ex) = run_both(lr, a, b, h_init=h0, reverse=reverse)
        fn = oracle.linrec_oracle_rev_f64 if reverse else oracle.linrec_oracle_f64
        ref = fn(a32, b32, h_init=h0_np)
        e = TOL * (1.0 + np.abs(ref))
        bar = e + 2.0 ** -8 * (np.abs(ref) + e)                  # one bf16 rounding of each output
        worst = float(np.max(np.abs(host(h_na) - ref) / bar))
        last = ref[:, 0, :] if reverse else ref[:, -1, :]
        say(f"[noalloc] bf16 reverse={reverse}: {worst:.3f} of the bar")
        assert worst <= 1.0
        assert ratio(host(f_na), last) <= TOL and ratio(host(f_na), host(f_ex)) <= TOL
        assert float(np.max(np.abs(host(h_na) - host(h_ex)) / bar)) <= 1.0


def test_noalloc_local_carry_touches_no_scratch_and_is_bitwise_equal(lr):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    shape = (cus // 8, 2048, 256)        # 8-lane slabs: one sequence per CU, the carry stays local
    a_np, b_np = li.make_inputs(*shape, seed=3200)
    a, b = torch.from_numpy(a_np).cuda(), torch.from_numpy(b_np).cuda()
    (h_na, _), (h_ex, _) = run_both(lr, a, b)
    assert torch.equal(h_na, h_ex)
    assert ratio(host(h_na), oracle.linrec_oracle_f64(a_np, b_np)) <= TOL


def test_noalloc_under_capture_without_warm_up(lr):
    lib = lr.library()
    shape = B, L, D = (2, 40000, 64)
    a = torch.empty(shape, device="cuda")
    b = torch.empty(shape, device="cuda")
    h = torch.empty(shape, device="cuda")
    d = lr.make_desc(a, b, h)
    fresh = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=fresh):
        assert lib.linrec_scan_ex_noalloc(ctypes.byref(d), fresh.cuda_stream) == lr.LINREC_OK
    for k in range(3):
        a_np, b_np = li.make_inputs(B, L, D, seed=3300 + k, a_lo=0.9, a_hi=1.0)
        a.copy_(torch.from_numpy(a_np))
        b.copy_(torch.from_numpy(b_np))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.linrec_oracle_f64(a_np, b_np)
        r = ratio(host(h), ref)
        say(f"[noalloc] capture replay {k}: {r:.3e}")
        assert r <= TOL
        # an eager call of the same entry point in between (shares the scratch, ordered)
        h2 = torch.empty_like(h)
        d2 = lr.make_desc(a, b, h2)
        assert lib.linrec_scan_ex_noalloc(ctypes.byref(d2), torch.cuda.current_stream().cuda_stream) == lr.LINREC_OK
        torch.cuda.synchronize()
        assert ratio(host(h2), ref) <= TOL


def test_noalloc_rejects_plans_beyond_the_scratch(lr):
    lib = lr.library()
    old = os.environ.get("LINREC_TILE")
    os.environ["LINREC_TILE"] = "m=1,t=4,w=1,p=16"          # 16-step tiles: 32768 tiles of 64 channels
    try:
        shape = (2, 262144, 64)
        a = torch.rand(shape, device="cuda")
        b = torch.randn(shape, device="cuda")
        h = torch.full_like(a, float("nan"))
        d = lr.make_desc(a, b, h)
        need = ctypes.c_size_t(0)
        assert lib.linrec_scan_ex_workspace_bytes(ctypes.byref(d), ctypes.byref(need)) == lr.LINREC_OK
        assert need.value > 16 << 20
        status = lib.linrec_scan_ex_noalloc(ctypes.byref(d), torch.cuda.current_stream().cuda_stream)
        message = lr.linrec_last_error_message()
        torch.cuda.synchronize()
        assert status == lr.LINREC_ERR_INVALID_ARGUMENT and "static scratch" in message, message
        assert torch.isnan(h).all()                            # nothing was enqueued
    finally:
        if old is None:
            os.environ.pop("LINREC_TILE", None)
        else:
            os.environ["LINREC_TILE"] = old
