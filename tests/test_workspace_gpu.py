"""Lookback workspaces on the GPU, through the C ABI: one per stream for the library's own, the
caller's through linrec_scan_ws / linrec_scan_ex_ws, concurrent streams, and graph capture
without a warm-up call.  Every output is compared with the float64 oracle at the fp32 bar
|h - ref| <= 1e-4 * (1 + |ref|)."""
import ctypes
import sys
import warnings

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linrec_inputs as li  # noqa: E402
import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-4
# few channels and a long L: the default plan is one tile per workgroup, looking back
LOOKBACK_SHAPE = (2, 40000, 64)


@pytest.fixture(scope="module")
def lr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrence_scan_linrec_amd import linrec as binding
    return binding


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def worst_ratio(h, ref):
    got = h.detach().float().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))


def cases(n, shape, seed):
    out = []
    for k in range(n):
        a_np, b_np = li.make_inputs(*shape, seed=seed + k, a_lo=0.9, a_hi=1.0)
        out.append((a_np, b_np, torch.from_numpy(a_np).cuda(), torch.from_numpy(b_np).cuda(),
                    torch.empty(shape, device="cuda")))
    return out


def test_lookback_shape_needs_a_workspace(lr):
    plan = lr.linrec_scan_plan(*LOOKBACK_SHAPE)
    assert plan["mode"] == 1 and plan["chunks"] > 1 and plan["workspace_bytes"] > 0
    need = lr.library().linrec_scan_workspace_bytes(*LOOKBACK_SHAPE)
    assert need >= plan["workspace_bytes"]
    a = torch.empty(LOOKBACK_SHAPE, device="cuda")
    assert lr.workspace_bytes(a, a) == plan["workspace_bytes"]


@pytest.mark.parametrize("own", [True, False], ids=["library_workspaces", "caller_workspaces"])
def test_two_streams_run_lookback_scans_concurrently(lr, own):
    """Two streams (default priority) each get eight lookback scans enqueued alternately with no
    synchronisation in between, so their kernels overlap on the device.  With the library's
    workspaces each stream has its own; with caller workspaces each stream passes its own.  Every
    output must match the oracle (shared status words would mix the two streams' carries)."""
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    work = [cases(8, LOOKBACK_SHAPE, 2000 + 100 * s) for s in range(2)]
    need = lr.library().linrec_scan_workspace_bytes(*LOOKBACK_SHAPE)
    ws = [torch.zeros(need, dtype=torch.uint8, device="cuda") for _ in streams]
    torch.cuda.synchronize()
    say(f"[streams] {'library' if own else 'caller'} workspaces: 2 streams x 8 scans of {LOOKBACK_SHAPE}")
    for k in range(8):
        for s, stream in enumerate(streams):
            _, _, a, b, h = work[s][k]
            lr.linrec_scan(a, b, h, stream=stream, workspace=None if own else ws[s])
    torch.cuda.synchronize()
    for s in range(2):
        for k, (a_np, b_np, _, _, h) in enumerate(work[s]):
            worst = worst_ratio(h, oracle.linrec_oracle_f64(a_np, b_np))
            assert worst <= TOL, (s, k, worst)
    say(f"[streams] all 16 outputs within the bar; recomputed waits on the device: {lr.linrec_device_timeouts()}")


def test_fresh_workspaces_are_cleared_before_their_first_scan(lr):
    """The first lookback call on a stream allocates that stream's workspace and must clear it
    before its scan reads the slot lines.  Each round releases every workspace (so new ones may
    reuse memory that held an earlier workspace's lines and status words), then enqueues the first
    scan on each of three side streams at once, with no synchronisation.  torch's side streams do
    not wait for the null stream, so a clear issued there could still be running when the scan
    reads the lines; the library clears on the call's own stream.  Every output must match the
    oracle with no predecessor recomputed (a scan that read uncleared lines would see mixed
    epochs and fall back to recomputing)."""
    work = cases(3, LOOKBACK_SHAPE, 2600)
    refs = [oracle.linrec_oracle_f64(a_np, b_np) for a_np, b_np, *_ in work]
    for r in range(4):
        torch.cuda.synchronize()
        lr.linrec_release()
        streams = [torch.cuda.Stream() for _ in work]
        for (_, _, a, b, h), stream in zip(work, streams):
            lr.linrec_scan(a, b, h, stream=stream)
        torch.cuda.synchronize()
        waits = lr.linrec_device_timeouts()
        worst = max(worst_ratio(h, ref) for (*_, h), ref in zip(work, refs))
        say(f"[fresh] round {r}: worst {worst:.2e}, recomputed waits {waits}")
        assert worst <= TOL and waits == 0, (r, worst, waits)


def test_caller_workspace_argument_checks(lr):
    lib = lr.library()
    B, L, D = LOOKBACK_SHAPE
    a = torch.rand(LOOKBACK_SHAPE, device="cuda")
    b = torch.randn(LOOKBACK_SHAPE, device="cuda")
    h = torch.empty(LOOKBACK_SHAPE, device="cuda")
    need = lr.workspace_bytes(a, b, h)            # exactly what these buffers' plan needs
    assert 0 < need <= lib.linrec_scan_workspace_bytes(B, L, D)
    ws = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    args = (a.data_ptr(), b.data_ptr(), h.data_ptr(), B, L, D)
    s = torch.cuda.current_stream().cuda_stream
    assert lib.linrec_scan_ws(*args, None, 0, s) == lr.LINREC_ERR_INVALID_ARGUMENT
    assert "needs a workspace" in lr.linrec_last_error_message()
    assert lib.linrec_scan_ws(*args, ws.data_ptr(), need - 8, s) == lr.LINREC_ERR_INVALID_ARGUMENT
    assert lib.linrec_scan_ws(*args, ws.data_ptr() + 16, need, s) == lr.LINREC_ERR_INVALID_ARGUMENT
    assert "aligned" in lr.linrec_last_error_message()
    assert lib.linrec_scan_ws(*args, h.data_ptr() + 256, need, s) == lr.LINREC_ERR_OVERLAP
    host = ctypes.create_string_buffer(need + 256)
    aligned = (ctypes.addressof(host) + 255) // 256 * 256
    assert lib.linrec_scan_ws(*args, aligned, need, s) == lr.LINREC_ERR_INVALID_ARGUMENT
    assert "workspace" in lr.linrec_last_error_message()
    # a plan that needs no workspace accepts none
    small = torch.rand(1, 64, 8, device="cuda")
    assert lib.linrec_scan_ws(small.data_ptr(), small.data_ptr(), torch.empty_like(small).data_ptr(), 1, 64, 8,
                              None, 0, s) == lr.LINREC_OK
    # and the real call with the caller's workspace meets the bar
    assert lib.linrec_scan_ws(*args, ws.data_ptr(), need, s) == lr.LINREC_OK
    torch.cuda.synchronize()
    assert worst_ratio(h, oracle.linrec_oracle_f64(a.cpu().numpy(), b.cpu().numpy())) <= TOL


def test_capture_without_warm_up(lr):
    """A fresh stream has no library workspace: a raw C call captured on it returns an error (it
    would have to allocate), the binding's call under torch.cuda.graph brings a workspace from the
    graph's pool, and a raw call with a caller workspace (cleared once before capture) replays.
    Every replay, with new inputs and eager calls in between, must match the oracle."""
    lib = lr.library()
    B, L, D = LOOKBACK_SHAPE
    a = torch.empty(LOOKBACK_SHAPE, device="cuda")
    b = torch.empty(LOOKBACK_SHAPE, device="cuda")
    h1 = torch.empty(LOOKBACK_SHAPE, device="cuda")
    h2 = torch.empty(LOOKBACK_SHAPE, device="cuda")
    need = lib.linrec_scan_workspace_bytes(B, L, D)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    fresh = torch.cuda.Stream()
    g_err = torch.cuda.CUDAGraph()
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")     # the refused call leaves the captured graph empty
        with torch.cuda.graph(g_err, stream=fresh):
            status = lib.linrec_scan(a.data_ptr(), b.data_ptr(), h1.data_ptr(), B, L, D, fresh.cuda_stream)
            message = lr.linrec_last_error_message()
    assert status == lr.LINREC_ERR_INVALID_ARGUMENT and "captured" in message, (status, message)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lr.linrec_scan(a, b, h1)                                     # binding: workspace from the pool
        st = torch.cuda.current_stream().cuda_stream
        assert lib.linrec_scan_ws(a.data_ptr(), b.data_ptr(), h2.data_ptr(), B, L, D, ws.data_ptr(), need,
                                  st) == lr.LINREC_OK
    for k in range(3):
        a_np, b_np = li.make_inputs(B, L, D, seed=2300 + k, a_lo=0.9, a_hi=1.0)
        a.copy_(torch.from_numpy(a_np))
        b.copy_(torch.from_numpy(b_np))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.linrec_oracle_f64(a_np, b_np)
        w1, w2 = worst_ratio(h1, ref), worst_ratio(h2, ref)
        say(f"[capture] replay {k}: pool workspace {w1:.3e}, caller workspace {w2:.3e}")
        assert w1 <= TOL and w2 <= TOL
        # eager calls in between, on the current stream and with the caller's workspace
        h_e = lr.linrec_scan(a, b)
        h_w = lr.linrec_scan(a, b, workspace=ws)
        torch.cuda.synchronize()
        assert worst_ratio(h_e, ref) <= TOL and worst_ratio(h_w, ref) <= TOL
        say(f"[capture] recomputed waits in the library's workspaces: {lr.linrec_device_timeouts()}")


def test_epoch_bookkeeping_across_grids_of_every_size(lr):
    """Thirty lookback calls in a row on one stream and one workspace, with grids from 1 to
    thousands of workgroups (one-tile and persistent plans, fewer and more workgroups than slot
    lines).  Each call counts its workgroups into slot lines that depend on its grid, and the last
    one advances the epoch; a count left over, or an epoch advanced early, would let a later call
    accept stale status words.  Every output must match the oracle, and no call may fall back to
    recomputing a predecessor (a call that read another call's epoch would have to)."""
    import os
    old = os.environ.get("LINREC_TILE")
    say(f"[epochs] recomputed waits before the release: {lr.linrec_device_timeouts()}")
    lr.linrec_release()                  # the count of recomputed waits runs from here
    rng = np.random.default_rng(2400)
    # (shape, tile override): grids of 1, 2, 5, 37, 255, 256, 257 and ~2000+ workgroups
    cases = [((1, 3000, 64), "m=1,t=4,w=1,p=16"), ((2, 9000, 64), "m=0,t=4,w=8,p=32,l=0,q=1"),
             ((1, 700, 8), "m=1,t=4,w=1,p=2"), ((3, 20000, 24), ""), ((2, 40000, 64), ""),
             ((32, 2048, 256), "m=0,t=4,w=8,p=32,l=0"), ((5, 12000, 136), "m=0,t=8,w=2,p=8,l=0,q=2"),
             ((4, 30000, 64), "m=1,t=8,w=7,p=8")]
    try:
        for k in range(30):
            shape, tile = cases[int(rng.integers(len(cases)))]
            if tile:
                os.environ["LINREC_TILE"] = tile
            else:
                os.environ.pop("LINREC_TILE", None)
            plan = lr.linrec_scan_plan(*shape)
            a_np, b_np = li.make_inputs(*shape, seed=2400 + k, a_lo=0.9, a_hi=1.0)
            h = lr.linrec_scan(torch.from_numpy(a_np).cuda(), torch.from_numpy(b_np).cuda())
            torch.cuda.synchronize()
            worst = worst_ratio(h, oracle.linrec_oracle_f64(a_np, b_np))
            waits = lr.linrec_device_timeouts()
            say(f"[epochs] call {k}: {shape} {tile or 'default'} tiles={plan['tiles']}: {worst:.2e}, "
                f"recomputed waits so far {waits}")
            assert worst <= TOL, (k, shape, tile, worst)
            assert waits == 0, (k, shape, tile, waits)
    finally:
        if old is None:
            os.environ.pop("LINREC_TILE", None)
        else:
            os.environ["LINREC_TILE"] = old
