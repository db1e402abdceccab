"""GPU parity: the HIP path (through the C ABI) against the float64 oracle, element by element.

Bar: |h_gpu - h_ref| <= 1e-4 * (1 + |h_ref|) for every element (the acceptance rule of the
harness the POPCORNBENCH transcripts were written for: fp32 compared with atol = rtol = 1e-4,
as restated in the "Kimi-K2.6 l2_p1" transcript's correctness discussion).  Exact
invariants (h == b where a == 0, L == 1) are checked bitwise.
"""
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


def error_ratio(h_gpu, ref):
    """max over elements of |h - ref| / (1 + |ref|), and its (i, t, d) index."""
    h = h_gpu.detach().cpu().numpy().reshape(-1)
    r = ref.reshape(-1)
    worst, where = -1.0, 0
    step = 1 << 24
    for s in range(0, h.size, step):
        hc = h[s:s + step].astype(np.float64)
        rc = r[s:s + step]
        ratio = np.abs(hc - rc) / (1.0 + np.abs(rc))
        ratio[np.isnan(ratio)] = np.inf
        k = int(np.argmax(ratio))
        if ratio[k] > worst:
            worst, where = float(ratio[k]), s + k
    return worst, np.unravel_index(where, ref.shape) if ref.size else None


def run_gpu(lr, a_np, b_np, stream=None):
    a = torch.from_numpy(a_np).cuda()
    b = torch.from_numpy(b_np).cuda()
    h = lr.linrec_scan(a, b, stream=stream)
    torch.cuda.synchronize()
    return h


def check_case(lr, a_np, b_np, label):
    say(f"[parity] {label} shape={a_np.shape}")
    h = run_gpu(lr, a_np, b_np)
    ref = oracle.linrec_oracle_f64(a_np, b_np)
    worst, where = error_ratio(h, ref)
    say(f"[parity] {label}: max ratio {worst:.3e} at {where}")
    assert worst <= TOL, f"{label}: max |h-ref|/(1+|ref|) = {worst:.3e} at {where}"
    return worst


# ----------------------------------------------------------------------------- small cases first

def test_tiny_workload(lr):
    w = li.WORKLOADS["tiny"]
    for seed in w.seeds:
        a, b = li.workload_inputs("tiny", seed)
        check_case(lr, a, b, f"tiny seed={seed}")


EDGE_SHAPES = [
    (1, 1, 1), (1, 1, 8), (2, 2, 3), (1, 3, 4), (3, 63, 5), (2, 65, 8), (1, 64, 1), (4, 17, 2),
    (2, 257, 256), (1, 1000, 3), (5, 129, 260), (1, 4097, 64), (2, 300, 1024), (1, 70, 4100),
]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes(lr, shape):
    B, L, D = shape
    a, b = li.make_inputs(B, L, D, seed=1000 + B * 7 + L * 3 + D)
    check_case(lr, a, b, f"edge {shape}")


def test_length_one_is_exact(lr):
    a, b = li.make_inputs(3, 1, 40, seed=77)
    a[:] = np.float32(np.inf)         # a_0 never contributes
    h = run_gpu(lr, a, b).cpu().numpy()
    assert np.array_equal(h, b)


def supported_tiles():
    """(vec, t, w, m) of every kernel instantiation; m = 0 persistent, m = 1 one tile per workgroup."""
    out = []
    for m in (0, 1):
        for vec in (1, 4):
            for t in (4, 8, 16):
                for w in (1, 2, 4, 7, 8, 15):
                    if m == 0 and vec == 4 and t == 16:
                        continue
                    if w == 15 and vec * t > 16:
                        continue
                    out.append((vec, t, w, m))
    return out


@pytest.fixture
def tile_env():
    old = os.environ.get("LINREC_TILE")
    yield
    if old is None:
        os.environ.pop("LINREC_TILE", None)
    else:
        os.environ["LINREC_TILE"] = old


@pytest.mark.parametrize("m", [0, 1])
@pytest.mark.parametrize("p", [1, 2, 4, 8, 16, 32, 64])
def test_lanes_per_row(lr, p, m, tile_env):
    """Narrower channel slabs (fewer lanes per row, more rows per wave instruction)."""
    os.environ["LINREC_TILE"] = f"p={p},m={m},w=8"
    for shape in ((3, 2999, 136), (2, 1501, 256), (1, 777, 24)):
        a, b = li.make_inputs(*shape, seed=shape[1] + p, a_lo=0.5, a_hi=1.0)
        plan = lr.linrec_scan_plan(*shape)
        assert plan["lanes_per_row"] <= p and plan["mode"] == m
        check_case(lr, a, b, f"p={p} m={m} {shape} chunks={plan['chunks']}")


@pytest.mark.parametrize("tile", supported_tiles(), ids=lambda t: f"vec{t[0]}_t{t[1]}_w{t[2]}_m{t[3]}")
def test_every_tile_shape(lr, tile, tile_env):
    """Each kernel instantiation on ragged shapes that span many tiles along L."""
    vec, t, w, m = tile
    p = ",p=16" if w == 15 and vec == 4 else ""
    os.environ["LINREC_TILE"] = f"vec={vec},t={t},w={w},m={m}{p}"
    for shape in ((3, 2999, 136), (2, 3001, 24), (1, 1500, 1 if vec == 1 else 4)):
        a, b = li.make_inputs(*shape, seed=shape[1] + vec + t + w, a_lo=0.5, a_hi=1.0)
        plan = lr.linrec_scan_plan(*shape)
        assert (plan["vec"], plan["steps_per_lane"], plan["waves"], plan["mode"]) == (vec, t, w, m)
        check_case(lr, a, b, f"tile {tile} {shape} chunks={plan['chunks']}")


def test_modes_and_grids_alternate_on_one_workspace(lr, tile_env):
    """Consecutive calls with different kernels and grid sizes share the device workspace; each
    call's status words must carry a fresh epoch (a stale word accepted as current would show up
    as a wrong carry); calls that keep the carry local in between leave the workspace alone."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cases = [("m=0", (4, 3000, 256)), ("m=1", (4, 3000, 256)), ("m=1,t=8,w=2", (2, 9000, 64)),
             ("m=0,w=2", (2, 9000, 64)), ("m=1", (4, 3000, 256)), ("m=0", (1, 70000, 8)),
             ("m=0,p=64,w=8,l=0", (3, 5000, 256)), ("m=1,p=64,w=8", (3, 5000, 256)),
             ("m=0,p=8,q=1,w=4", (cus // 8, 3000, 256)), ("m=0", (4, 3000, 256)),
             ("m=0,p=8,q=1,w=2,t=8", (cus // 8, 3100, 256)), ("m=0,w=4,t=8", (2, 9000, 64))]
    for k, (spec, shape) in enumerate(cases):
        os.environ["LINREC_TILE"] = spec
        a, b = li.make_inputs(*shape, seed=500 + k, a_lo=0.9, a_hi=1.0)
        plan = lr.linrec_scan_plan(*shape)
        assert plan["chunks"] > 1
        check_case(lr, a, b, f"call {k} {spec} {shape} tiles={plan['tiles']}")


def test_misaligned_buffers_take_the_scalar_form(lr):
    B, L, D = 2, 700, 64
    a_np, b_np = li.make_inputs(B, L, D, seed=31)
    n = B * L * D
    a_flat = torch.empty(n + 1, dtype=torch.float32, device="cuda")
    b_flat = torch.empty(n + 1, dtype=torch.float32, device="cuda")
    h_flat = torch.empty(n + 1, dtype=torch.float32, device="cuda")
    a = a_flat[1:].view(B, L, D)
    b = b_flat[1:].view(B, L, D)
    h = h_flat[1:].view(B, L, D)
    a.copy_(torch.from_numpy(a_np))
    b.copy_(torch.from_numpy(b_np))
    assert a.data_ptr() % 16 != 0
    lr.linrec_scan(a, b, h)
    torch.cuda.synchronize()
    worst, where = error_ratio(h, oracle.linrec_oracle_f64(a_np, b_np))
    assert worst <= TOL, (worst, where)


def test_normal_a_at_the_pages_shape(lr):
    """The pages draw both inputs with randn; a ~ N(0,1) has |a| > 1 and negative a."""
    a, b = li.make_inputs(32, 4096, 256, seed=105, a_dist="normal")
    check_case(lr, a, b, "pages shape, a~N(0,1)")


# ----------------------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["tiny", "pages_shape", "long_sequence", "wide_channels", "near_unit_resets"])
def test_named_workload_all_seeds(lr, name):
    w = li.WORKLOADS[name]
    for seed in w.seeds:
        a, b = li.workload_inputs(name, seed)
        check_case(lr, a, b, f"{name} seed={seed} ({w.describe()})")
        del a, b


def test_resets_give_b_exactly(lr):
    a, b = li.workload_inputs("near_unit_resets", 5)
    h = run_gpu(lr, a, b).cpu().numpy()
    mask = a == 0
    assert mask.sum() > 0
    assert np.array_equal(h[mask], b[mask])


# Workloads whose default plan keeps the carry local (persistent workgroups that own whole
# sequences): every output then has one fixed evaluation order.  The one-tile plan of
# long_sequence looks back, and which predecessor has published its inclusive state when a tile
# reads it depends on timing, so its bracketing may differ from run to run.
LOCAL_CARRY_WORKLOADS = ("pages_shape", "wide_channels", "near_unit_resets")


@pytest.mark.parametrize("name", LOCAL_CARRY_WORKLOADS + ("long_sequence",))
def test_run_to_run(lr, name):
    """Local-carry plans are bitwise equal from run to run; lookback plans agree within the bar."""
    a_np, b_np = li.workload_inputs(name)
    a = torch.from_numpy(a_np).cuda()
    b = torch.from_numpy(b_np).cuda()
    del a_np, b_np
    h1 = lr.linrec_scan(a, b)
    h2 = lr.linrec_scan(a, b)
    h3 = lr.linrec_scan(a, b)
    torch.cuda.synchronize()
    diff = max(((h1 - h).abs() / (1 + h1.abs())).max().item() for h in (h2, h3))
    equal = torch.equal(h1, h2) and torch.equal(h1, h3)
    say(f"[determinism] {name}: max run-to-run ratio {diff:.3e}, bitwise equal {equal}")
    if name in LOCAL_CARRY_WORKLOADS:
        assert equal, f"{name}: local-carry plan not bitwise reproducible (max ratio {diff:.3e})"
    assert diff <= TOL


def test_non_default_stream(lr):
    a_np, b_np = li.make_inputs(4, 5000, 256, seed=44)
    ref = oracle.linrec_oracle_f64(a_np, b_np)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = torch.from_numpy(a_np).cuda(non_blocking=False)
        b = torch.from_numpy(b_np).cuda(non_blocking=False)
        a2 = a * 1.0            # produced on s, consumed by the scan on s
        h = lr.linrec_scan(a2, b, stream=s)
        h2 = h * 1.0            # consumed on s after the scan
    s.synchronize()
    worst, where = error_ratio(h2, ref)
    assert worst <= TOL, (worst, where)


# ----------------------------------------------------------------------------- failure handling

@pytest.fixture
def spin_env():
    old = os.environ.get("LINREC_SPIN_LIMIT")
    yield
    if old is None:
        os.environ.pop("LINREC_SPIN_LIMIT", None)
    else:
        os.environ["LINREC_SPIN_LIMIT"] = old


@pytest.mark.parametrize("m", [0, 1])
def test_spin_limit_zero_recomputes_and_stays_exact(lr, spin_env, tile_env, m):
    """With the wait for a predecessor forced to zero polls, every tile that finds its predecessor's
    status not yet published recomputes that predecessor's pair from a and b.  The output must not
    change beyond the bar, and every kernel exits normally."""
    os.environ["LINREC_TILE"] = f"m={m}"
    # (2, 40000, 64) with one tile per workgroup: 90 chunks per sequence, the long-chain window
    for shape, lo in (((2, 8192, 64), 0.9), ((4, 2048, 256), 0.0), ((2, 40000, 64), 0.9)):
        a_np, b_np = li.make_inputs(*shape, seed=9, a_lo=lo, a_hi=1.0)
        ref = oracle.linrec_oracle_f64(a_np, b_np)
        before = lr.linrec_device_timeouts()
        os.environ["LINREC_SPIN_LIMIT"] = "0"
        h = run_gpu(lr, a_np, b_np)
        os.environ.pop("LINREC_SPIN_LIMIT")
        recomputed = lr.linrec_device_timeouts() - before
        worst, where = error_ratio(h, ref)
        say(f"[recompute] m={m} {shape}: {recomputed} tiles recomputed a predecessor; max ratio {worst:.3e}")
        assert worst <= TOL, (worst, where)
        # the normal path afterwards
        h = run_gpu(lr, a_np, b_np)
        assert error_ratio(h, ref)[0] <= TOL


def test_bad_buffers_are_rejected(lr):
    a = torch.zeros(2, 8, 16, device="cuda")
    h = torch.zeros_like(a)
    host = np.zeros((2, 8, 16), np.float32)
    st = lr.linrec_scan_raw(host.ctypes.data, a.data_ptr(), h.data_ptr(), 2, 8, 16, 0)
    assert st == lr.LINREC_ERR_INVALID_ARGUMENT
    # a claimed size far beyond the allocations: refused (as too small, or as overlapping h)
    st = lr.linrec_scan_raw(a.data_ptr(), a.data_ptr(), h.data_ptr(), 2, 8, 1 << 36, 0)
    assert st in (lr.LINREC_ERR_INVALID_ARGUMENT, lr.LINREC_ERR_OVERLAP), lr.linrec_last_error_message()
    with pytest.raises(ValueError):
        lr.linrec_scan(a.double(), a)
    with pytest.raises(ValueError):
        lr.linrec_scan(a.transpose(1, 2), a.transpose(1, 2))
    torch.cuda.synchronize()


@pytest.mark.parametrize("local", [0, 1])
def test_local_carry(lr, tile_env, local):
    """Persistent workgroups whose grid (one per CU here) divides the (batch row, channel slab)
    sequences into 1, 2 or 4 per workgroup keep the carry in LDS instead of looking back; l=0
    forces the lookback on the same shapes."""
    m = 0
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for k, (rows, L, D) in enumerate(((cus // 8, 3001, 256), (cus // 4, 1501, 256), (cus // 8, 777, 1024))):
        os.environ["LINREC_TILE"] = f"p=8,q=1,w=8,m={m},l={local}"
        a, b = li.make_inputs(rows, L, D, seed=900 + k, a_lo=0.5, a_hi=1.0)
        plan = lr.linrec_scan_plan(rows, L, D)
        assert plan["chunks"] > 1 and plan["lanes_per_row"] == 8
        check_case(lr, a, b, f"local={local} m={m} {(rows, L, D)} sequences={rows * D // 32}")


def local_tiles():
    """(vec, t, w) of every persistent instantiation."""
    return [(vec, t, w) for vec in (1, 4) for t in (4, 8, 16) for w in (1, 2, 4, 7, 8, 15)
            if not (vec == 4 and t == 16) and not (w == 15 and vec * t > 16)]


@pytest.mark.parametrize("tile", local_tiles(), ids=lambda t: f"vec{t[0]}_t{t[1]}_w{t[2]}")
def test_every_local_tile_shape(lr, tile_env, tile):
    """Each persistent instantiation with a local carry, on a ragged shape whose 8-lane slabs give
    one sequence per CU (so the grid of one workgroup per CU takes whole sequences)."""
    vec, t, w = tile
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    D = 256 if vec == 4 else 64
    rows = cus // 8
    os.environ["LINREC_TILE"] = f"vec={vec},t={t},w={w},p=8,q=1,m=0"
    for L in (2 * 8 * t * w + 5, 1001):
        a, b = li.make_inputs(rows, L, D, seed=1200 + vec + t + w + L, a_lo=0.5, a_hi=1.0)
        plan = lr.linrec_scan_plan(rows, L, D)
        assert plan["lanes_per_row"] == 8 and plan["vec"] == vec
        check_case(lr, a, b, f"local tile {tile} {(rows, L, D)} chunks={plan['chunks']}")


@pytest.mark.parametrize("shape", [(32, 4096, 256), (4, 3000, 256), (2, 20000, 64)],
                         ids=["local_carry", "lookback_persistent", "lookback_one_tile"])
def test_graph_capture_and_replay(lr, shape):
    """linrec_scan captured into a HIP graph (after a first call has sized the workspace) and
    replayed with new inputs each time, with eager work and synchronisation between replays;
    every replay must match the oracle.  The call records only kernel launches (no memset, no
    allocation), and a lookback's call epoch advances inside the kernel, so replays stay valid."""
    B, L, D = shape
    a = torch.empty(shape, device="cuda")
    b = torch.empty(shape, device="cuda")
    h = torch.empty(shape, device="cuda")
    a0, b0 = li.make_inputs(B, L, D, seed=1700, a_lo=0.5, a_hi=1.0)
    a.copy_(torch.from_numpy(a0))
    b.copy_(torch.from_numpy(b0))
    lr.linrec_scan(a, b, h)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lr.linrec_scan(a, b, h)
    for k in range(3):
        a_np, b_np = li.make_inputs(B, L, D, seed=1701 + k, a_lo=0.5, a_hi=1.0)
        a.copy_(torch.from_numpy(a_np))
        b.copy_(torch.from_numpy(b_np))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        worst, where = error_ratio(h, oracle.linrec_oracle_f64(a_np, b_np))
        say(f"[graph] {shape} replay {k}: max ratio {worst:.3e}")
        assert worst <= TOL, (k, worst, where)
        # eager use of the library between replays
        h_eager = lr.linrec_scan(a, b)
        torch.cuda.synchronize()
        assert error_ratio(h_eager, oracle.linrec_oracle_f64(a_np, b_np))[0] <= TOL


def recurrence_residual(a, b, h, steps=1 << 16):
    """Largest |h_t - (a_t h_{t-1} + b_t)| / (1 + |h_t|) over every element, evaluated on the
    device in float64 from the stored fp32 values, a batch row and a stretch of time steps at a
    time; and whether h_0 = b_0 holds exactly.  Away from the hand-overs between lanes this is
    one fp32 rounding (2^-24); where a lane starts from its carried state it is that state's
    distance from the previous lane's last output, a few fp32 roundings of the replay.  A wrong
    carry or a misplaced row shows up as a residual of the order of |h|."""
    worst = 0.0
    first_exact = True
    B, L, _ = h.shape
    for i in range(B):
        first_exact &= bool(torch.equal(h[i, 0], b[i, 0]))
        for t0 in range(1, L, steps):
            t1 = min(L, t0 + steps)
            ht = h[i, t0:t1].double()
            r = (ht - (a[i, t0:t1].double() * h[i, t0 - 1:t1 - 1].double() + b[i, t0:t1].double())).abs_()
            worst = max(worst, float((r / (1.0 + ht.abs())).max()))
            del ht, r
    return worst, first_exact


@pytest.mark.parametrize("shape", [(2, 1 << 20, 1028), (16, 1 << 17, 1028)], ids=["one_tile", "persistent"])
def test_more_than_2_31_elements(lr, shape):
    """B*L*D above 2^31 elements, with batch rows more than 2^32 bytes apart: 64-bit row and
    status indexing.  Inputs are drawn on the device from a seeded generator (26 GB per case).
    Every element is checked against the recurrence itself (the residual of each step from the
    stored values, far below the bar), and the oracle checks a few channels, including the last
    slab's ragged edge, over every step."""
    B, L, D = shape
    assert B * L * D > 2 ** 31
    say(f"[large] {shape}: {B * L * D} elements")
    gen = torch.Generator(device="cuda").manual_seed(31 + B)
    a = torch.rand(shape, device="cuda", generator=gen)
    a.mul_(0.5).add_(0.5)                                   # U(0.5, 1)
    b = torch.randn(shape, device="cuda", generator=gen)
    h = lr.linrec_scan(a, b)
    torch.cuda.synchronize()
    residual, first_exact = recurrence_residual(a, b, h)
    say(f"[large] {shape}: largest step residual {residual:.3e}, h_0 = b_0: {first_exact}")
    assert first_exact
    assert residual <= TOL / 4, residual
    cols = [0, 5, 511, D - 4, D - 1]
    a_s = np.ascontiguousarray(a[:, :, cols].cpu().numpy())
    b_s = np.ascontiguousarray(b[:, :, cols].cpu().numpy())
    h_s = h[:, :, cols].cpu().numpy()
    del a, b, h
    torch.cuda.empty_cache()
    ref = oracle.linrec_oracle_f64(a_s, b_s)
    ratio = np.abs(h_s - ref) / (1.0 + np.abs(ref))
    worst = float(ratio.max())
    say(f"[large] {shape}: channels {cols}, max ratio {worst:.3e}")
    assert worst <= TOL, (worst, np.unravel_index(int(np.argmax(ratio)), ratio.shape))


def test_release_then_reallocate_and_grow(lr):
    """linrec_release frees the per-device workspace (a no-op when there is none).  The next call
    that looks back allocates and clears a new one, and a larger shape grows it.  Every result
    meets the bar, and the timeout count reads zero again after a release."""
    lr.linrec_release()
    lr.linrec_release()
    assert lr.linrec_device_timeouts() == 0
    shapes = ((2, 3000, 64), (2, 3000, 64), (4, 20000, 256))   # the last needs a larger workspace
    for k, shape in enumerate(shapes):
        a_np, b_np = li.make_inputs(*shape, seed=1800 + k, a_lo=0.5, a_hi=1.0)
        h = run_gpu(lr, a_np, b_np)
        worst, where = error_ratio(h, oracle.linrec_oracle_f64(a_np, b_np))
        say(f"[release] {shape} call {k}: max ratio {worst:.3e}")
        assert worst <= TOL, (shape, worst, where)
        if k == 0:
            lr.linrec_release()
            assert lr.linrec_device_timeouts() == 0
    assert lr.linrec_scan_plan(4, 20000, 256)["workspace_bytes"] > lr.linrec_scan_plan(2, 3000, 64)["workspace_bytes"]


def test_concurrent_host_threads_on_one_stream(lr):
    """Four host threads enqueue lookback scans on one stream at once (ctypes releases the GIL, so
    the library's host code runs concurrently): the workspace bookkeeping is shared under a lock,
    and the calls, ordered by the stream, all meet the bar."""
    import threading
    shape = (2, 6000, 64)
    cases = []
    for k in range(4):
        a_np, b_np = li.make_inputs(*shape, seed=1900 + k, a_lo=0.5, a_hi=1.0)
        cases.append((a_np, b_np, torch.from_numpy(a_np).cuda(), torch.from_numpy(b_np).cuda(),
                      torch.empty(shape, device="cuda")))
    stream = torch.cuda.current_stream()
    errors = []

    def worker(k):
        try:
            _, _, a, b, h = cases[k]
            for _ in range(10):
                lr.linrec_scan(a, b, h, stream=stream)
        except Exception as e:   # reported below: an exception in a thread would be lost
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k, (a_np, b_np, _, _, h) in enumerate(cases):
        worst, where = error_ratio(h, oracle.linrec_oracle_f64(a_np, b_np))
        say(f"[threads] case {k}: max ratio {worst:.3e}")
        assert worst <= TOL, (k, worst, where)


@pytest.mark.parametrize("tile", ["", "l=0", "m=1"], ids=["default", "lookback", "one_tile"])
def test_non_finite_first_decay_is_ignored(lr, tile, tile_env, spin_env):
    """a at t = 0 multiplies the zero state before the first step, so it never contributes: an
    infinite or NaN a_0 leaves every output finite and equal to the oracle's, also when the
    lookback recomputes predecessors (chunk 0 included) from the inputs."""
    if tile:
        os.environ["LINREC_TILE"] = tile
    B, L, D = 4, 5000, 64
    a_np, b_np = li.make_inputs(B, L, D, seed=2000, a_lo=0.5, a_hi=1.0)
    a_np[:, 0, 0::2] = np.float32(np.inf)
    a_np[:, 0, 1::2] = np.float32(np.nan)
    ref = oracle.linrec_oracle_f64(a_np, b_np)
    assert np.isfinite(ref).all()
    for spin in (None, "0"):
        if spin is not None:
            os.environ["LINREC_SPIN_LIMIT"] = spin
        h = run_gpu(lr, a_np, b_np)
        os.environ.pop("LINREC_SPIN_LIMIT", None)
        assert bool(torch.isfinite(h).all())
        worst, where = error_ratio(h, ref)
        say(f"[a0] {tile or 'default'} spin={spin}: max ratio {worst:.3e}")
        assert worst <= TOL, (worst, where)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_default_plans_resolve_every_carry_from_status(lr, dtype):
    """At the four large workloads, the default plans (several of which look back across
    workgroups) resolve every carry from the status their predecessors publish: the recompute
    fallback, correct but slow, is never taken.  A persistent grid larger than what the device
    runs at once, or a tile that waits on one not yet started, would show up here.  The count
    runs from the workspace's allocation (growing it starts a new one), so each workload starts
    from a released workspace."""
    for name in ("pages_shape", "long_sequence", "wide_channels", "near_unit_resets"):
        a_np, b_np = li.workload_inputs(name)
        a = torch.from_numpy(a_np).cuda().to(dtype)
        b = torch.from_numpy(b_np).cuda().to(dtype)
        plan = lr.plan_for(a, b)
        say(f"[timeouts] {name} {dtype}: mode {plan['mode']}, {plan['tiles']} tiles, {plan['chunks']} chunks")
        lr.linrec_release()
        for _ in range(3):
            h = lr.linrec_scan(a, b)
        torch.cuda.synchronize()
        assert lr.linrec_device_timeouts() == 0, name
        assert torch.isfinite(h.float()).all()
        del a, b, h
        torch.cuda.empty_cache()
