"""GPU parity of the relay kernel (LINREC_TILE m=2) against the float64 oracle.

The relay runs only where the persistent grid gives every workgroup whole (batch row, channel
slab) sequences, so each shape here has B * (channel slabs) equal to 1, 2 or 4 times the CU count
with q=1 (one workgroup per CU).  The carry wave folds each tile's lane pairs in fp64, one tile
behind the data waves; these tests cover every relay instantiation, ragged lengths and channel
counts, narrow and wide slabs (1 to 64 lanes per row, so 64 down to 1 lane pairs per wave and
channel), 2 and 4 sequences per workgroup, an initial and a final state, the reverse recurrence
and its form with the decays one step ahead, 16-bit storage, decays close to 1, and the
fallback to the lookback kernel where no grid keeps the carry local.

Bar (as for every fp32 path): |h - ref| <= 1e-4 * (1 + |ref|) per element; 16-bit storage adds
one rounding to the storage type (see test_parity_ex_gpu).
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests.test_parity_ex_gpu import check, decays_ahead, device_inputs, say  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrence_scan_linrec_amd import linrec as binding
    return binding


@pytest.fixture(scope="module")
def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.fixture
def tile_env():
    old = os.environ.get("LINREC_TILE")
    yield
    if old is None:
        os.environ.pop("LINREC_TILE", None)
    else:
        os.environ["LINREC_TILE"] = old


def relay_tiles():
    """(vec, t, w) of every relay instantiation for 4-byte registers (vec * t * 4 <= 128 bytes)."""
    return [(vec, t, w) for vec in (1, 4) for t in (4, 8, 16) for w in (1, 2) if vec * t * 4 <= 128]


def run_relay(lr, spec, a, b, **kw):
    os.environ["LINREC_TILE"] = spec
    plan = lr.plan_for(a, b, **{k: v for k, v in kw.items() if k in ("h_init", "reverse", "a_ahead")})
    assert plan["mode"] == 2 and plan["chunks"] > 1, plan
    out = lr.linrec_scan(a, b, **kw)
    torch.cuda.synchronize()
    return out, plan


@pytest.mark.parametrize("tile", relay_tiles(), ids=lambda t: f"vec{t[0]}_t{t[1]}_w{t[2]}")
def test_every_relay_tile_shape(lr, cus, tile_env, tile):
    """Each instantiation over 8-lane slabs, one sequence per workgroup; lengths with a ragged last
    tile and with exactly two tiles."""
    vec, t, w = tile
    D = 256 if vec == 4 else 64          # 8 slabs of 8 lanes per batch row
    B = cus // 8
    rows = w * 8 * t                      # 8 groups of 8 lanes per wave
    for L in (2 * rows, 2 * rows + 5, 1001):
        a, b, a_np, b_np = device_inputs((B, L, D), seed=1300 + vec + t + w + L, a_lo=0.5, a_hi=1.0)
        h, plan = run_relay(lr, f"vec={vec},t={t},w={w},p=8,q=1,m=2", a, b)
        check(h, oracle.linrec_oracle_f64(a_np, b_np), torch.float32,
              f"relay {tile} {(B, L, D)} chunks={plan['chunks']}")


@pytest.mark.parametrize("p,vec", [(1, 4), (2, 4), (4, 4), (16, 4), (64, 1), (32, 1)])
def test_relay_lanes_per_row(lr, cus, tile_env, p, vec):
    """Slabs of 1 to 64 lanes (64 down to 1 lane pairs per wave and channel for the carry wave);
    8 slabs per batch row, and with more than one lane per row also a last slab that is ragged
    (channels past D read as zero and are never stored)."""
    slab = p * vec
    B = cus // 8
    for D in (8 * slab, 8 * slab - vec) if p > 1 else (8 * slab,):
        L = 700
        a, b, a_np, b_np = device_inputs((B, L, D), seed=1400 + p + D, a_lo=0.5, a_hi=1.0)
        h, plan = run_relay(lr, f"vec={vec},t=8,w=1,p={p},q=1,m=2", a, b)
        assert plan["lanes_per_row"] == p
        check(h, oracle.linrec_oracle_f64(a_np, b_np), torch.float32, f"relay p={p} vec={vec} {(B, L, D)}")


@pytest.mark.parametrize("per_group", [2, 4])
def test_relay_several_sequences_per_workgroup(lr, cus, tile_env, per_group):
    """2 or 4 sequences per workgroup: tiles alternate between them, each with its own carry cell."""
    B = cus * per_group // 8
    for L, t, w in ((1001, 8, 1), (515, 4, 2)):
        a, b, a_np, b_np = device_inputs((B, L, 256), seed=1500 + per_group + L, a_lo=0.5, a_hi=1.0)
        h, plan = run_relay(lr, f"t={t},w={w},p=8,q=1,m=2", a, b)
        check(h, oracle.linrec_oracle_f64(a_np, b_np), torch.float32,
              f"relay {per_group} sequences per workgroup {(B, L, 256)} t={t} w={w}")


@pytest.mark.parametrize("reverse", [False, True], ids=["forward", "reverse"])
def test_relay_states(lr, cus, tile_env, reverse):
    """An initial state in and the final state out, forward and in reverse, on a ragged length."""
    B, L, D = cus // 8, 1003, 256
    a, b, a_np, b_np = device_inputs((B, L, D), seed=1600 + reverse, a_lo=0.5, a_hi=1.0)
    h0_np = np.random.default_rng(1601).standard_normal((B, D)).astype(np.float32)
    h0 = torch.from_numpy(h0_np).cuda()
    (h, hf), _ = run_relay(lr, "t=8,w=1,p=8,q=1,m=2", a, b, h_init=h0, return_final=True, reverse=reverse)
    fn = oracle.linrec_oracle_rev_f64 if reverse else oracle.linrec_oracle_f64
    ref = fn(a_np, b_np, h_init=h0_np)
    tag = "reverse" if reverse else "forward"
    check(h, ref, torch.float32, f"relay states {tag}")
    check(hf, ref[:, 0 if reverse else -1, :], torch.float32, f"relay states {tag} h_final")


def test_relay_decays_ahead(lr, cus, tile_env):
    """The reverse form with each decay one step ahead, with and without an initial state."""
    B, L, D = cus // 8, 777, 256
    a, b, a_np, b_np = device_inputs((B, L, D), seed=1700, a_lo=0.5, a_hi=1.0)
    h, _ = run_relay(lr, "t=8,w=1,p=8,q=1,m=2", a, b, reverse=True, a_ahead=True)
    check(h, oracle.linrec_oracle_rev_f64(decays_ahead(a_np, 0.0), b_np), torch.float32, "relay ahead")
    h0_np = np.random.default_rng(1701).standard_normal((B, D)).astype(np.float32)
    h0 = torch.from_numpy(h0_np).cuda()
    (h, hf), _ = run_relay(lr, "t=4,w=2,p=8,q=1,m=2", a, b, h_init=h0, return_final=True, reverse=True,
                           a_ahead=True)
    ref = oracle.linrec_oracle_rev_f64(decays_ahead(a_np, 1.0), b_np, h_init=h0_np)
    check(h, ref, torch.float32, "relay ahead with h_init")
    check(hf, ref[:, 0, :], torch.float32, "relay ahead h_final")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("t", [8, 16])
def test_relay_16_bit_storage(lr, cus, tile_env, dtype, t):
    """16-bit storage: 4 channels per lane stay packed in registers, so 16 steps per lane fit."""
    B, L, D = cus // 8, 1100, 256
    a, b, a_np, b_np = device_inputs((B, L, D), seed=1800 + t, dtype=dtype, a_lo=0.5, a_hi=1.0)
    h, _ = run_relay(lr, f"t={t},w=1,p=8,q=1,m=2", a, b)
    check(h, oracle.linrec_oracle_f64(a_np, b_np), dtype, f"relay {dtype} t={t}")


def test_relay_near_unit_decays_at_the_pages_shape(lr, tile_env):
    """Decays 0.99999 constant in time over B=32 L=4096 D=256: h is close to a running sum of
    up to 4096 standard normal steps, and the carry wave's fp64 state keeps every element within
    the bar."""
    B, L, D = 32, 4096, 256
    a_np = np.full((B, L, D), 0.99999, dtype=np.float32)
    b_np = np.random.default_rng(1900).standard_normal((B, L, D)).astype(np.float32)
    a = torch.from_numpy(a_np).cuda()
    b = torch.from_numpy(b_np).cuda()
    os.environ.pop("LINREC_TILE", None)
    plan = lr.linrec_scan_plan(B, L, D)
    assert plan["mode"] == 2, plan
    h = lr.linrec_scan(a, b)
    torch.cuda.synchronize()
    worst = check(h, oracle.linrec_oracle_f64(a_np, b_np), torch.float32, "relay near-unit pages shape")
    say(f"[relay] near-unit worst/bar {worst:.3f}")


def test_relay_falls_back_to_lookback(lr, tile_env):
    """m=2 on shapes whose sequences no grid can divide into whole ones per workgroup: the tiles
    look back through the m=0 kernel of the same shape."""
    for k, shape in enumerate(((3, 2999, 136), (1, 20000, 64))):
        a, b, a_np, b_np = device_inputs(shape, seed=2000 + k, a_lo=0.5, a_hi=1.0)
        os.environ["LINREC_TILE"] = "t=8,w=1,m=2"
        plan = lr.linrec_scan_plan(*shape)
        assert plan["mode"] == 2 and plan["chunks"] > 1
        h = lr.linrec_scan(a, b)
        torch.cuda.synchronize()
        check(h, oracle.linrec_oracle_f64(a_np, b_np), torch.float32, f"relay fallback {shape}")


def test_relay_graph_capture_and_replay(lr, tile_env):
    """The default relay plan at B=32 L=4096 D=256 captured into a HIP graph: no workspace, and
    each replay (with eager work between them) matches the eager result bit for bit."""
    B, L, D = 32, 4096, 256
    a, b, a_np, b_np = device_inputs((B, L, D), seed=2100, a_lo=0.5, a_hi=1.0)
    os.environ.pop("LINREC_TILE", None)
    assert lr.linrec_scan_plan(B, L, D)["mode"] == 2
    eager = lr.linrec_scan(a, b)
    torch.cuda.synchronize()
    check(eager, oracle.linrec_oracle_f64(a_np, b_np), torch.float32, "relay eager")
    h = torch.empty_like(a)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lr.linrec_scan(a, b, h)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lr.linrec_scan(a, b, h)
    for r in range(3):
        h.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, eager), f"replay {r} differs from the eager result"
        (a * 2.0).sum().item()   # eager work between replays
