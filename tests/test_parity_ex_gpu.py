"""GPU parity of linrec_scan_ex (through the C ABI) against the float64 oracle: strided and
broadcast operands, bf16/fp16 storage, an initial and a final state, pieces chained through
them, and the reverse-time recurrence.

Bars:
* fp32 storage: |h - ref| <= 1e-4 * (1 + |ref|) per element, as for linrec_scan.
* 16-bit storage: the inputs are the 16-bit values (they widen to fp32 exactly, and the oracle
  consumes exactly those values); the kernel computes in fp32 and rounds each output once to
  the storage type, to nearest.  So the output is within u * |y| of an fp32 result y that meets
  the fp32 bar, u = 2^-8 (bf16, 8 significant bits) or 2^-11 (fp16, 11 bits), which gives
  |h - ref| <= e + u * (|ref| + e) with e = 1e-4 * (1 + |ref|).
* h_final is fp32 (never rounded to the storage type): the fp32 bar against the oracle's state
  after the last step.
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
UNIT_ROUNDOFF = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}

# tile overrides: the default choice, one tile per workgroup, the 32-bit form, a deep
# narrow tile, and short tiles with narrow slabs (many chunks, long carry chains)
TILES = ["", "m=1", "vec=1", "m=1,vec=1,t=8,w=2", "t=8,w=4,p=8", "m=1,t=4,w=1,p=16", "t=4,w=8,p=32,l=0"]


@pytest.fixture(scope="module")
def lr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrence_scan_linrec_amd import linrec as binding
    return binding


@pytest.fixture
def tile_env():
    old = os.environ.get("LINREC_TILE")
    yield
    if old is None:
        os.environ.pop("LINREC_TILE", None)
    else:
        os.environ["LINREC_TILE"] = old


def set_tile(spec):
    if spec:
        os.environ["LINREC_TILE"] = spec
    else:
        os.environ.pop("LINREC_TILE", None)


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def host(t):
    """A device tensor's values as a float64 numpy array (16-bit values widen exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(h, ref, dtype, label):
    """Assert the storage-type bar element by element; returns the worst |h-ref| / bar."""
    got = host(h)
    e = TOL * (1.0 + np.abs(ref))
    bar = e + UNIT_ROUNDOFF[dtype] * (np.abs(ref) + e)
    ratio = np.abs(got - ref) / bar
    ratio[np.isnan(ratio)] = np.inf
    worst = float(ratio.max()) if ratio.size else 0.0
    where = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else None
    say(f"[ex] {label}: worst |h-ref|/bar = {worst:.3f} at {where}")
    assert worst <= 1.0, f"{label}: |h-ref| exceeds the bar by {worst:.3f}x at {where}"
    return worst


def device_inputs(shape, seed, dtype=torch.float32, a_lo=0.0, a_hi=1.0):
    """Seeded inputs on the GPU in the storage type, and the fp32 host copies of those exact values."""
    a_np, b_np = li.make_inputs(*shape, seed=seed, a_lo=a_lo, a_hi=a_hi)
    a = torch.from_numpy(a_np).cuda().to(dtype)
    b = torch.from_numpy(b_np).cuda().to(dtype)
    return a, b, a.float().cpu().numpy(), b.float().cpu().numpy()


SHAPES = [(3, 2999, 136), (2, 3001, 24), (1, 1500, 7), (2, 257, 1)]


# ----------------------------------------------------------------------------- strides

@pytest.mark.parametrize("tile", TILES)
def test_strided_operands(lr, tile, tile_env):
    """a every other time step of a larger tensor, b time-major, h inside a wider padded row."""
    set_tile(tile)
    for k, (B, L, D) in enumerate(SHAPES):
        a_np, b_np = li.make_inputs(B, L, D, seed=200 + k, a_lo=0.5, a_hi=1.0)
        big_a = torch.full((B, 2 * L, D), float("nan"), device="cuda")
        a = big_a[:, ::2, :]
        a.copy_(torch.from_numpy(a_np))
        b_tm = torch.from_numpy(np.ascontiguousarray(b_np.transpose(1, 0, 2))).cuda()
        b = b_tm.transpose(0, 1)                      # strides (D, B*D, 1)
        pad = 8
        h_big = torch.full((B, L, D + 2 * pad), float("nan"), device="cuda")
        h = h_big[:, :, pad:pad + D]
        lr.linrec_scan(a, b, h)
        torch.cuda.synchronize()
        check(h, oracle.linrec_oracle_f64(a_np, b_np), torch.float32, f"strided {tile or 'default'} {(B, L, D)}")
        # nothing outside h was written
        assert torch.isnan(h_big[:, :, :pad]).all() and torch.isnan(h_big[:, :, pad + D:]).all()


def test_strided_pages_shape(lr):
    """Strided operands at the pages' full shape: b stored time-major, h written inside a wider
    padded row (the padding must stay untouched)."""
    a_np, b_np = li.workload_inputs("pages_shape")
    B, L, D = a_np.shape
    a = torch.from_numpy(a_np).cuda()
    b = torch.from_numpy(np.ascontiguousarray(b_np.transpose(1, 0, 2))).cuda().transpose(0, 1)
    pad = 4
    h_big = torch.full((B, L, D + 2 * pad), float("nan"), device="cuda")
    h = h_big[:, :, pad:pad + D]
    lr.linrec_scan(a, b, h)
    torch.cuda.synchronize()
    check(h, oracle.linrec_oracle_f64(a_np, b_np), torch.float32, "strided pages_shape")
    assert torch.isnan(h_big[:, :, :pad]).all() and torch.isnan(h_big[:, :, pad + D:]).all()


@pytest.mark.parametrize("tile", TILES[:3])
def test_broadcast_decay(lr, tile, tile_env):
    """One decay row shared by every batch row (batch stride 0), and a decay constant over time
    (time stride 0) whose per-channel constants run from 0.5 to 0.99999."""
    set_tile(tile)
    B, L, D = 4, 2500, 64
    a_np, b_np = li.make_inputs(1, L, D, seed=301, a_lo=0.9, a_hi=1.0)
    _, b_np = li.make_inputs(B, L, D, seed=302)
    a = torch.from_numpy(a_np).cuda().expand(B, L, D)
    b = torch.from_numpy(b_np).cuda()
    h = lr.linrec_scan(a, b)
    torch.cuda.synchronize()
    check(h, oracle.linrec_oracle_f64(np.broadcast_to(a_np, (B, L, D)), b_np), torch.float32,
          f"batch-broadcast a {tile or 'default'}")
    # 1 - c log-spaced from 0.5 down to 1e-5 across the channels
    c_np = (1.0 - np.logspace(np.log10(0.5), -5.0, D)).astype(np.float32).reshape(1, 1, D)
    a_t = torch.from_numpy(c_np).cuda().expand(B, L, D)      # time stride 0
    h = lr.linrec_scan(a_t, b)
    torch.cuda.synchronize()
    check(h, oracle.linrec_oracle_f64(np.broadcast_to(c_np, (B, L, D)), b_np), torch.float32,
          f"time-broadcast a {tile or 'default'}")


# the default plan (local carry at this shape), one tile per workgroup (lookback over long
# chains), the 32-bit form, and persistent workgroups that look back
CARRY_TILES = ["", "m=1", "vec=1", "t=4,w=8,p=32,l=0"]


@pytest.mark.parametrize("decay", [0.999, 0.9999, 0.99999])
def test_constant_decay_near_one(lr, decay, tile_env):
    """A decay that is the same at every step and close to 1, at the pages' shape (B=32, L=4096,
    D=256, b ~ N(0,1), so |h| grows to 80-200 and crosses zero many times), passed both as a
    time-broadcast operand (time stride 0) and as a materialised tensor, under every carry form.

    Every lane, wave and tile then multiplies the same decays, so a product of decays rounded
    in fp32 has the same error everywhere and the carry would add those errors up along the
    sequence; the kernel keeps the products on the carry path in fp64, and the outputs stay
    within the unchanged bar 1e-4 * (1 + |h|) element by element."""
    B, L, D = 32, 4096, 256
    _, b_np = li.make_inputs(B, L, D, seed=310)
    a_np = np.full((B, L, D), decay, dtype=np.float32)
    ref = oracle.linrec_oracle_f64(a_np, b_np)
    say(f"[ex] constant decay {decay}: max |h| = {np.abs(ref).max():.1f}")
    b = torch.from_numpy(b_np).cuda()
    a_full = torch.from_numpy(a_np).cuda()
    a_bcast = torch.full((1, 1, D), decay, dtype=torch.float32, device="cuda").expand(B, L, D)
    for tile in CARRY_TILES:
        set_tile(tile)
        for name, a in (("materialised", a_full), ("time-broadcast", a_bcast)):
            h = lr.linrec_scan(a, b)
            torch.cuda.synchronize()
            check(h, ref, torch.float32, f"constant decay {decay} {name} {tile or 'default'}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_half_storage_constant_decay_long_chain(lr, dtype, tile_env):
    """16-bit storage publishes each tile's product of decays as one fp32 word, rounded once per
    tile; with a constant decay those roundings repeat along the chain.  Over 586 chunks per
    sequence at (2, 262144, 64), with the closest decay below 1 that the storage type holds
    (1 - 2^-8 for bf16, 1 - 2^-11 for fp16), time-broadcast and materialised, one tile per
    workgroup and persistent lookback: every output within the storage type's bar.

    A decay of exactly 1 is left out at this length: rounding errors made while |h| is in the
    hundreds then never fade, and a plain sequential fp32 loop misses the bar by 4x (bf16
    outputs), 11x (fp16) and 85x (fp32) where the running sum comes back near zero."""
    B, L, D = 2, 262144, 64
    decay = 1.0 - 2.0 ** (-8 if dtype == torch.bfloat16 else -11)
    _, b32 = li.make_inputs(B, L, D, seed=330)
    b = torch.from_numpy(b32).cuda().to(dtype)
    b_np = b.float().cpu().numpy()
    a_np = np.full((B, L, D), decay, dtype=np.float32)
    ref = oracle.linrec_oracle_f64(a_np, b_np)
    say(f"[ex] {dtype} constant decay {decay}: max |h| = {np.abs(ref).max():.1f}")
    a_full = torch.from_numpy(a_np).cuda().to(dtype)
    a_bcast = torch.full((1, 1, D), decay, dtype=dtype, device="cuda").expand(B, L, D)
    for tile in ("", "m=0,t=8,w=8,p=16,l=0"):
        set_tile(tile)
        for name, a in (("materialised", a_full), ("time-broadcast", a_bcast)):
            h = lr.linrec_scan(a, b)
            torch.cuda.synchronize()
            check(h, ref, dtype, f"{dtype} constant decay {decay} {name} {tile or 'default'}")


# ----------------------------------------------------------------------------- 16-bit storage

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("tile", TILES)
def test_half_storage(lr, dtype, tile, tile_env):
    set_tile(tile)
    for k, shape in enumerate(SHAPES):
        a, b, a_np, b_np = device_inputs(shape, 400 + k, dtype, a_lo=0.5, a_hi=1.0)
        h = lr.linrec_scan(a, b)
        torch.cuda.synchronize()
        assert h.dtype == dtype
        check(h, oracle.linrec_oracle_f64(a_np, b_np), dtype, f"{dtype} {tile or 'default'} {shape}")


# tiles that exist only because 16-bit values stay packed in registers (4 channels per lane):
# one tile per workgroup with 15 waves of 8 positions, and persistent tiles of 16 positions
HALF_TILES = ["m=1,t=8,w=15,p=16", "t=16,w=4,p=32", "t=16,w=2,p=16", "t=16,w=4,p=32,l=0"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("tile", HALF_TILES)
def test_half_storage_packed_tiles(lr, dtype, tile, tile_env):
    """Packed 16-bit register tiles on ragged shapes: plain, with an initial and a final state
    (positions past L become identity steps in the packed words), and in reverse time."""
    set_tile(tile)
    for k, shape in enumerate(SHAPES):
        B, L, D = shape
        a, b, a_np, b_np = device_inputs(shape, 800 + k, dtype, a_lo=0.5, a_hi=1.0)
        label = f"{dtype} {tile} {shape}"
        h = lr.linrec_scan(a, b)
        torch.cuda.synchronize()
        check(h, oracle.linrec_oracle_f64(a_np, b_np), dtype, label)
        h0_np = np.random.default_rng(900 + k).standard_normal((B, D)).astype(np.float32)
        h0 = torch.from_numpy(h0_np).cuda()
        for reverse in (False, True):
            h, hf = lr.linrec_scan(a, b, h_init=h0, return_final=True, reverse=reverse)
            torch.cuda.synchronize()
            fn = oracle.linrec_oracle_rev_f64 if reverse else oracle.linrec_oracle_f64
            ref = fn(a_np, b_np, h_init=h0_np)
            tag = f"{label} state{' reverse' if reverse else ''}"
            check(h, ref, dtype, tag)
            check(hf, ref[:, 0 if reverse else -1, :], torch.float32, tag + " h_final")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_half_storage_named_workloads(lr, dtype):
    """The named workloads at full size, stored in 16 bits: one tile per workgroup (the pages'
    shape, long_sequence), persistent lookback (near_unit_resets, with resets) and a local carry
    (wide_channels)."""
    for name in ("pages_shape", "near_unit_resets", "long_sequence", "wide_channels"):
        a_np32, b_np32 = li.workload_inputs(name)
        a = torch.from_numpy(a_np32).cuda().to(dtype)
        b = torch.from_numpy(b_np32).cuda().to(dtype)
        del a_np32, b_np32
        a_np, b_np = a.float().cpu().numpy(), b.float().cpu().numpy()
        h = lr.linrec_scan(a, b)
        torch.cuda.synchronize()
        check(h, oracle.linrec_oracle_f64(a_np, b_np), dtype, f"{dtype} {name}")
        if name == "near_unit_resets":
            mask = torch.from_numpy(a_np == 0).cuda()
            assert bool(mask.any())
            assert torch.equal(h[mask], b[mask])          # a reset gives b, exactly
        del a, b, h


# ----------------------------------------------------------------------------- line groups

# tiles whose slab rows are narrower than a 128-byte line, on shapes where whole line groups fill
# each batch row and the sequences fill whole blocks of 8 groups: the slabs sharing a line are
# then mapped to slots equal modulo 8 (x=1).  The first five keep the carry local on a 256-CU
# part: 256 sequences, one per persistent workgroup, or 512, two per workgroup.
LINE_GROUP_CASES = [
    (torch.float32, "p=4", (16, 1500, 256)),                 # 64-byte rows, 2 slabs per line
    (torch.float32, "vec=1,p=8", (8, 1500, 256)),            # 32-byte rows, 4 slabs per line
    (torch.bfloat16, "p=8", (32, 1500, 256)),                # 64-byte rows
    (torch.float16, "p=4", (16, 1500, 256)),                 # 32-byte rows
    (torch.float32, "p=4,w=2", (32, 1500, 256)),             # 512 sequences: 2 per workgroup, local
    (torch.float32, "p=4,l=0", (4, 1500, 256)),              # the same slabs with a lookback
    (torch.bfloat16, "p=8,m=1,t=4,w=4", (8, 1500, 256)),     # one tile per workgroup
]


@pytest.mark.parametrize("dtype,tile,shape", LINE_GROUP_CASES,
                         ids=[f"{str(d).split('.')[-1]}-{t}" for d, t, _ in LINE_GROUP_CASES])
def test_line_groups(lr, dtype, tile, shape, tile_env):
    """Sequences permuted so that slabs sharing a cache line run on one XCD give the oracle's
    result; with a local carry the result is bitwise that of dispatch order (x=0), since each
    sequence is evaluated the same way whichever workgroup runs it."""
    a, b, a_np, b_np = device_inputs(shape, 750, dtype, a_lo=0.5, a_hi=1.0)
    ref = oracle.linrec_oracle_f64(a_np, b_np)
    out = {}
    for x in (1, 0):
        set_tile(f"{tile},x={x}")
        plan = lr.plan_for(a, b)
        h = lr.linrec_scan(a, b)
        torch.cuda.synchronize()
        check(h, ref, dtype, f"line groups {tile} x={x} {tuple(shape)} (lanes {plan['lanes_per_row']})")
        out[x] = h
    if "l=0" not in tile and "m=1" not in tile:
        assert torch.equal(out[1], out[0])


# ----------------------------------------------------------------------------- initial / final state

@pytest.mark.parametrize("tile", TILES)
def test_initial_and_final_state(lr, tile, tile_env):
    set_tile(tile)
    for k, shape in enumerate(SHAPES):
        B, L, D = shape
        a, b, a_np, b_np = device_inputs(shape, 500 + k, a_lo=0.5, a_hi=1.0)
        h0_np = np.random.default_rng(600 + k).standard_normal((B, D)).astype(np.float32)
        h0 = torch.from_numpy(h0_np).cuda()
        h, hf = lr.linrec_scan(a, b, h_init=h0, return_final=True)
        torch.cuda.synchronize()
        ref = oracle.linrec_oracle_f64(a_np, b_np, h_init=h0_np)
        check(h, ref, torch.float32, f"h_init {tile or 'default'} {shape}")
        check(hf, ref[:, -1, :], torch.float32, f"h_final {tile or 'default'} {shape}")
        # without an initial state the final state is still the last row
        h, hf = lr.linrec_scan(a, b, return_final=True)
        torch.cuda.synchronize()
        assert torch.equal(hf, h[:, -1, :])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_pieces_chained_through_the_state(lr, dtype):
    """A long scan run as ragged pieces, each piece's final state the next one's initial state,
    matches the whole sequence; the final state stays fp32 between pieces."""
    B, L, D = 2, 20000, 64
    a, b, a_np, b_np = device_inputs((B, L, D), 700, dtype, a_lo=0.9, a_hi=1.0)
    cuts = [0, 1, 130, 4099, 4100, 13000, 19999, L]
    h = torch.empty_like(a)
    state = None
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        _, state = lr.linrec_scan(a[:, lo:hi], b[:, lo:hi], h[:, lo:hi], h_init=state, return_final=True)
    torch.cuda.synchronize()
    ref = oracle.linrec_oracle_f64(a_np, b_np)
    check(h, ref, dtype, f"pieces {dtype}")
    check(state, ref[:, -1, :], torch.float32, f"pieces final state {dtype}")


def test_zero_length_passes_the_state(lr):
    B, D = 3, 40
    a = torch.empty((B, 0, D), device="cuda")
    h0 = torch.randn(B, D, device="cuda")
    _, hf = lr.linrec_scan(a, a.clone(), h_init=h0, return_final=True)
    torch.cuda.synchronize()
    assert torch.equal(hf, h0)
    hf = torch.full((B, D), 7.0, device="cuda")
    lr.linrec_scan(a, a.clone(), h_final=hf)
    torch.cuda.synchronize()
    assert torch.equal(hf, torch.zeros_like(hf))


@pytest.fixture
def spin_env():
    old = os.environ.get("LINREC_SPIN_LIMIT")
    yield
    if old is None:
        os.environ.pop("LINREC_SPIN_LIMIT", None)
    else:
        os.environ["LINREC_SPIN_LIMIT"] = old


@pytest.mark.parametrize("reverse", [False, True], ids=["forward", "reverse"])
@pytest.mark.parametrize("tile", ["m=0,l=0", "m=1"])
def test_recompute_with_initial_state(lr, tile, reverse, tile_env, spin_env):
    """Lookback with the wait for a predecessor forced to zero polls: tiles recompute their
    predecessors' pairs from a and b, and a walk that passes chunk 0 applies the initial state
    itself.  Decays near 1 keep h_init visible over several tiles, so a walk that dropped it
    would fail the bar."""
    set_tile(tile)
    B, L, D = 2, 8192, 64
    a, b, a_np, b_np = device_inputs((B, L, D), 710, a_lo=0.995, a_hi=1.0)
    h0_np = (10.0 * np.random.default_rng(711).standard_normal((B, D))).astype(np.float32)
    before = lr.linrec_device_timeouts()
    os.environ["LINREC_SPIN_LIMIT"] = "0"
    h, hf = lr.linrec_scan(a, b, h_init=torch.from_numpy(h0_np).cuda(), return_final=True, reverse=reverse)
    torch.cuda.synchronize()
    os.environ.pop("LINREC_SPIN_LIMIT")
    recomputed = lr.linrec_device_timeouts() - before
    ref = (oracle.linrec_oracle_rev_f64 if reverse else oracle.linrec_oracle_f64)(a_np, b_np, h_init=h0_np)
    label = f"recompute h_init {tile} {'reverse' if reverse else 'forward'} ({recomputed} tiles recomputed)"
    check(h, ref, torch.float32, label)
    check(hf, ref[:, 0 if reverse else -1, :], torch.float32, label + " h_final")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16], ids=["f32", "bf16", "f16"])
def test_recompute_on_long_chains(lr, dtype, tile_env, spin_env):
    """The long-chain lookback window (one tile per workgroup, 90 chunks per sequence: 3
    predecessors per round trip in fp32, 2 then 4 in 16 bits) with the wait forced to zero polls,
    with an initial state that decays near 1 keep visible over many tiles, so that recomputed
    pairs and walks past chunk 0 both reach the output."""
    set_tile("")
    B, L, D = 2, 40000, 64
    a, b, a_np, b_np = device_inputs((B, L, D), 720, dtype, a_lo=0.995, a_hi=1.0)
    h0_np = (10.0 * np.random.default_rng(721).standard_normal((B, D))).astype(np.float32)
    h0 = torch.from_numpy(h0_np).cuda()
    plan = lr.plan_for(a, b, h_init=h0)
    assert plan["mode"] == 1 and plan["chunks"] > 64, plan
    before = lr.linrec_device_timeouts()
    os.environ["LINREC_SPIN_LIMIT"] = "0"
    h, hf = lr.linrec_scan(a, b, h_init=h0, return_final=True)
    torch.cuda.synchronize()
    os.environ.pop("LINREC_SPIN_LIMIT")
    recomputed = lr.linrec_device_timeouts() - before
    ref = oracle.linrec_oracle_f64(a_np, b_np, h_init=h0_np)
    label = f"long-chain recompute {dtype} ({recomputed} tiles recomputed)"
    check(h, ref, dtype, label)
    check(hf, ref[:, -1, :], torch.float32, label + " h_final")
    assert recomputed > 0


# ----------------------------------------------------------------------------- reverse time

@pytest.mark.parametrize("tile", TILES)
def test_reverse(lr, tile, tile_env):
    set_tile(tile)
    for k, shape in enumerate(SHAPES):
        B, L, D = shape
        a, b, a_np, b_np = device_inputs(shape, 800 + k, a_lo=0.5, a_hi=1.0)
        h = lr.linrec_scan(a, b, reverse=True)
        torch.cuda.synchronize()
        check(h, oracle.linrec_oracle_rev_f64(a_np, b_np), torch.float32, f"reverse {tile or 'default'} {shape}")
        h0_np = np.random.default_rng(900 + k).standard_normal((B, D)).astype(np.float32)
        h, hf = lr.linrec_scan(a, b, reverse=True, h_init=torch.from_numpy(h0_np).cuda(), return_final=True)
        torch.cuda.synchronize()
        ref = oracle.linrec_oracle_rev_f64(a_np, b_np, h_init=h0_np)
        check(h, ref, torch.float32, f"reverse h_init {tile or 'default'} {shape}")
        check(hf, ref[:, 0, :], torch.float32, f"reverse h_final {tile or 'default'} {shape}")


@pytest.mark.parametrize("name", ["pages_shape", "long_sequence"])
def test_reverse_named_workloads(lr, name):
    """Reverse time at full size: the local-carry plan of the pages' shape and the long lookback
    chains of long_sequence, run backwards, with a final state."""
    a_np, b_np = li.workload_inputs(name)
    a = torch.from_numpy(a_np).cuda()
    b = torch.from_numpy(b_np).cuda()
    h, hf = lr.linrec_scan(a, b, reverse=True, return_final=True)
    torch.cuda.synchronize()
    ref = oracle.linrec_oracle_rev_f64(a_np, b_np)
    check(h, ref, torch.float32, f"reverse {name}")
    check(hf, ref[:, 0, :], torch.float32, f"reverse {name} h_final")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_reverse_half_strided(lr, dtype):
    """Reverse time with 16-bit storage and a time-major gradient operand."""
    B, L, D = 4, 3001, 128
    a, _, a_np, _ = device_inputs((B, L, D), 1000, dtype, a_lo=0.5, a_hi=1.0)
    _, g_np32 = li.make_inputs(B, L, D, seed=1001)
    g_tm = torch.from_numpy(np.ascontiguousarray(g_np32.transpose(1, 0, 2))).cuda().to(dtype)
    g = g_tm.transpose(0, 1)
    g_np = g.float().cpu().numpy()
    h = lr.linrec_scan(a, g, reverse=True)
    torch.cuda.synchronize()
    check(h, oracle.linrec_oracle_rev_f64(a_np, g_np), dtype, f"reverse {dtype} time-major b")


def test_reverse_gives_the_gradient_of_the_forward_scan(lr):
    """dLoss/db of loss = sum(g * scan(a, b)) from float64 autograd of the plain recurrence on
    the CPU equals the GPU reverse scan over g with a shifted one step (a[t+1] at position t),
    and dLoss/da[t] = dLoss/db[t] * h[t-1] (zero at t = 0)."""
    B, L, D = 2, 300, 12
    a_np, b_np = li.make_inputs(B, L, D, seed=1100, a_lo=0.5, a_hi=1.0)
    _, g_np = li.make_inputs(B, L, D, seed=1101)
    a64 = torch.from_numpy(a_np).double().requires_grad_(True)
    b64 = torch.from_numpy(b_np).double().requires_grad_(True)
    state = torch.zeros(B, D, dtype=torch.float64)
    rows = []
    for t in range(L):
        state = (a64[:, t] * state if t > 0 else 0.0) + b64[:, t]
        rows.append(state)
    loss = (torch.stack(rows, dim=1) * torch.from_numpy(g_np).double()).sum()
    loss.backward()
    a_shift = np.zeros_like(a_np)
    a_shift[:, :-1] = a_np[:, 1:]
    a = torch.from_numpy(a_shift).cuda()
    g = torch.from_numpy(g_np).cuda()
    db = lr.linrec_scan(a, g, reverse=True)
    h = lr.linrec_scan(torch.from_numpy(a_np).cuda(), torch.from_numpy(b_np).cuda())
    torch.cuda.synchronize()
    check(db, b64.grad.numpy(), torch.float32, "gradient in b")
    da = torch.zeros_like(db)
    da[:, 1:] = db[:, 1:] * h[:, :-1]
    check(da, a64.grad.numpy(), torch.float32, "gradient in a")


def decays_ahead(a_np, last):
    """a taken one time step ahead: a'[t] = a[t+1], and a'[L-1] = last (the decay that
    multiplies h_init in the reverse scan: 1 when one is given; unused without one)."""
    s = np.empty_like(a_np)
    s[:, :-1] = a_np[:, 1:]
    s[:, -1] = last
    return s


@pytest.mark.parametrize("tile", TILES)
def test_reverse_with_decays_ahead(lr, tile, tile_env):
    """reverse=True, a_ahead=True reads a one time step ahead inside the kernel: equal to the
    plain reverse scan over a shifted copy of a, with and without an initial state (which enters
    with decay 1), on ragged shapes in every tile form."""
    set_tile(tile)
    for k, shape in enumerate(SHAPES):
        B, L, D = shape
        a, b, a_np, b_np = device_inputs(shape, 1200 + k, a_lo=0.5, a_hi=1.0)
        h = lr.linrec_scan(a, b, reverse=True, a_ahead=True)
        torch.cuda.synchronize()
        check(h, oracle.linrec_oracle_rev_f64(decays_ahead(a_np, 0.0), b_np), torch.float32,
              f"decays ahead {tile or 'default'} {shape}")
        h0_np = np.random.default_rng(1300 + k).standard_normal((B, D)).astype(np.float32)
        h, hf = lr.linrec_scan(a, b, reverse=True, a_ahead=True, h_init=torch.from_numpy(h0_np).cuda(),
                               return_final=True)
        torch.cuda.synchronize()
        ref = oracle.linrec_oracle_rev_f64(decays_ahead(a_np, 1.0), b_np, h_init=h0_np)
        check(h, ref, torch.float32, f"decays ahead h_init {tile or 'default'} {shape}")
        check(hf, ref[:, 0, :], torch.float32, f"decays ahead h_final {tile or 'default'} {shape}")


@pytest.mark.parametrize("tile", ["m=0,t=4,w=8,p=32,l=0", "m=1"])
def test_decays_ahead_through_recomputed_predecessors(lr, tile, tile_env, spin_env):
    """With the wait for a predecessor forced to zero polls, tiles recompute their predecessors'
    pairs from a and b: that path must take the decays one step ahead too, and a walk past
    chunk 0 must apply h_init with decay 1.  Decays near 1 keep h_init visible over many tiles."""
    set_tile(tile)
    B, L, D = 2, 8192, 64
    a, b, a_np, b_np = device_inputs((B, L, D), 1400, a_lo=0.995, a_hi=1.0)
    h0_np = (10.0 * np.random.default_rng(1401).standard_normal((B, D))).astype(np.float32)
    os.environ["LINREC_SPIN_LIMIT"] = "0"
    h = lr.linrec_scan(a, b, reverse=True, a_ahead=True, h_init=torch.from_numpy(h0_np).cuda())
    torch.cuda.synchronize()
    os.environ.pop("LINREC_SPIN_LIMIT")
    check(h, oracle.linrec_oracle_rev_f64(decays_ahead(a_np, 1.0), b_np, h_init=h0_np), torch.float32,
          f"decays ahead, recomputed predecessors, {tile}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_gradient_from_the_forward_decays(lr, dtype):
    """dLoss/db of loss = sum(g * scan(a, b)), from float64 autograd of the plain recurrence on
    the CPU, equals reverse=True, a_ahead=True over g with the forward scan's own a (no shifted
    copy), here with a time-major a; dLoss/da[t] = dLoss/db[t] * h[t-1]."""
    B, L, D = 2, 300, 12
    a_np32, b_np32 = li.make_inputs(B, L, D, seed=1500, a_lo=0.5, a_hi=1.0)
    _, g_np32 = li.make_inputs(B, L, D, seed=1501)
    a_tm = torch.from_numpy(np.ascontiguousarray(a_np32.transpose(1, 0, 2))).cuda().to(dtype)
    a = a_tm.transpose(0, 1)
    b = torch.from_numpy(b_np32).cuda().to(dtype)
    g = torch.from_numpy(g_np32).cuda().to(dtype)
    a_np, b_np, g_np = (x.float().cpu().numpy() for x in (a, b, g))
    a64 = torch.from_numpy(a_np).double().requires_grad_(True)
    b64 = torch.from_numpy(b_np).double().requires_grad_(True)
    state = torch.zeros(B, D, dtype=torch.float64)
    rows = []
    for t in range(L):
        state = (a64[:, t] * state if t > 0 else 0.0) + b64[:, t]
        rows.append(state)
    (torch.stack(rows, dim=1) * torch.from_numpy(g_np).double()).sum().backward()
    db = lr.linrec_scan(a, g, reverse=True, a_ahead=True)
    h = lr.linrec_scan(a, b)
    torch.cuda.synchronize()
    check(db, b64.grad.numpy(), dtype, f"gradient in b, {dtype}")
    da = torch.zeros(B, L, D, dtype=torch.float32, device="cuda")
    da[:, 1:] = db[:, 1:].float() * h[:, :-1].float()
    if dtype == torch.float32:
        check(da, a64.grad.numpy(), dtype, "gradient in a")


def test_decays_ahead_at_full_size_and_in_pieces(lr):
    """long_sequence run backwards with the decays one step ahead (its long lookback chains),
    whole and in three ragged pieces taken from the last: each piece starts from
    h_init = a[:, start of the next piece] * (the next piece's result at its first step)."""
    a_np, b_np = li.workload_inputs("long_sequence")
    a = torch.from_numpy(a_np).cuda()
    b = torch.from_numpy(b_np).cuda()
    ref = oracle.linrec_oracle_rev_f64(decays_ahead(a_np, 0.0), b_np)
    whole = lr.linrec_scan(a, b, reverse=True, a_ahead=True)
    torch.cuda.synchronize()
    check(whole, ref, torch.float32, "decays ahead, long_sequence")
    L = a.shape[1]
    cuts = [0, 70001, 200003, L]
    pieces, state = [], None
    for lo, hi in reversed(list(zip(cuts[:-1], cuts[1:]))):
        h = lr.linrec_scan(a[:, lo:hi], b[:, lo:hi], reverse=True, a_ahead=True, h_init=state)
        pieces.append(h)
        state = (a[:, lo] * h[:, 0]).contiguous()
    torch.cuda.synchronize()
    check(torch.cat(pieces[::-1], dim=1), ref, torch.float32, "decays ahead, long_sequence in pieces")


def test_local_carry_with_every_operand_form(lr, tile_env):
    """Persistent workgroups that keep the carry local (8-lane slabs, one workgroup per CU taking
    whole sequences), with strided operands, bf16 storage, an initial and a final state, and
    reverse time."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, L, D = cus // 8, 1999, 256
    set_tile("p=8,q=1,w=4,m=0,l=1")
    a, b, a_np, b_np = device_inputs((B, L, D), 1300, a_lo=0.5, a_hi=1.0)
    h0_np = np.random.default_rng(1301).standard_normal((B, D)).astype(np.float32)
    h0 = torch.from_numpy(h0_np).cuda()
    for reverse in (False, True):
        fn = oracle.linrec_oracle_rev_f64 if reverse else oracle.linrec_oracle_f64
        ref = fn(a_np, b_np, h_init=h0_np)
        b_tm = b.transpose(0, 1).contiguous().transpose(0, 1)          # time-major b
        h_big = torch.full((B, L, D + 8), float("nan"), device="cuda")
        h = h_big[:, :, 4:4 + D]
        _, hf = lr.linrec_scan(a, b_tm, h, h_init=h0, return_final=True, reverse=reverse)
        torch.cuda.synchronize()
        check(h, ref, torch.float32, f"local carry strided reverse={reverse}")
        check(hf, ref[:, 0 if reverse else -1, :], torch.float32, f"local carry h_final reverse={reverse}")
        assert torch.isnan(h_big[:, :, :4]).all() and torch.isnan(h_big[:, :, 4 + D:]).all()
    ab, bb, ab_np, bb_np = device_inputs((B, L, D), 1302, torch.bfloat16, a_lo=0.5, a_hi=1.0)
    h = lr.linrec_scan(ab, bb)
    torch.cuda.synchronize()
    check(h, oracle.linrec_oracle_f64(ab_np, bb_np), torch.bfloat16, "local carry bf16")
