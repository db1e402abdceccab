"""GPU parity on seeded combinations of the options that the other parity tests take one at a
time: each case draws a shape (ragged L and D included), a storage type, the direction of time,
an initial and a final state, a layout per operand (contiguous, time-major, every other time
step of a larger tensor, broadcast over batch rows, an output inside padded rows), a tile
override and, for reverse scans, the decays one time step ahead, and compares every output
element with the float64 oracle.  Same bars as the other
linrec_scan_ex parity tests; an output's padding must stay untouched.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import linrec_inputs as li  # noqa: E402
import oracle  # noqa: E402
from tests.test_parity_ex_gpu import HALF_TILES, TILES, check, say  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = 96
DTYPES = [torch.float32, torch.bfloat16, torch.float16]
IN_LAYOUTS = ["contiguous", "time_major", "every_other_step", "broadcast_rows"]


@pytest.fixture(scope="module")
def lr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrence_scan_linrec_amd import linrec as binding
    return binding


def draw_case(k):
    rng = np.random.default_rng(31000 + k)
    B = int(rng.integers(1, 5))
    L = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 5000))]))
    D = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 300)), 4 * int(rng.integers(1, 65))]))
    dtype = DTYPES[int(rng.integers(len(DTYPES)))]
    tiles = TILES + (HALF_TILES if dtype != torch.float32 else [])
    case = {
        "shape": (B, L, D),
        "dtype": dtype,
        "reverse": bool(rng.integers(2)),
        "h_init": bool(rng.integers(2)),
        "h_final": bool(rng.integers(2)),
        "a_layout": IN_LAYOUTS[int(rng.integers(len(IN_LAYOUTS)))],
        "b_layout": IN_LAYOUTS[int(rng.integers(len(IN_LAYOUTS)))],
        "h_padded": bool(rng.integers(2)),
        "a_lo": float(rng.choice([0.0, 0.5, 0.9])),
        "tile": tiles[int(rng.integers(len(tiles)))],
        "seed": 32000 + k,
    }
    # drawn last, so the earlier draws of every case stay as they were
    case["a_ahead"] = case["reverse"] and bool(rng.integers(2))
    return case


def lay_out(values, layout, dtype):
    """A (B, L, D) device view holding `values` (rows broadcast from row 0 for broadcast_rows)."""
    B, L, D = values.shape
    v = torch.from_numpy(values).to(dtype)
    if layout == "contiguous":
        return v.cuda()
    if layout == "time_major":
        return v.transpose(0, 1).contiguous().cuda().transpose(0, 1)
    if layout == "every_other_step":
        big = torch.full((B, 2 * L, D), float("nan"), dtype=dtype, device="cuda")
        big[:, ::2, :] = v.cuda()
        return big[:, ::2, :]
    if layout == "broadcast_rows":
        return v[:1].cuda().expand(B, L, D)
    raise ValueError(layout)


@pytest.mark.parametrize("k", range(CASES))
def test_seeded_combination(lr, k, monkeypatch):
    c = draw_case(k)
    B, L, D = c["shape"]
    dtype = c["dtype"]
    if c["tile"]:
        monkeypatch.setenv("LINREC_TILE", c["tile"])   # restored when the test ends
    else:
        monkeypatch.delenv("LINREC_TILE", raising=False)
    label = (f"combo {k}: {c['shape']} {str(dtype).split('.')[-1]} tile='{c['tile']}' reverse={c['reverse']} "
             f"h_init={c['h_init']} h_final={c['h_final']} a={c['a_layout']} b={c['b_layout']} "
             f"h_padded={c['h_padded']} a_ahead={c['a_ahead']}")
    say(label)
    a_np, b_np = li.make_inputs(B, L, D, seed=c["seed"], a_lo=c["a_lo"], a_hi=1.0)
    a = lay_out(a_np, c["a_layout"], dtype)
    b = lay_out(b_np, c["b_layout"], dtype)
    # the values the GPU consumes, as the oracle sees them (16-bit values widen exactly)
    a_ref = a.float().cpu().numpy()
    b_ref = b.float().cpu().numpy()
    pad = 3
    if c["h_padded"]:
        h_big = torch.full((B, L, D + 2 * pad), float("nan"), dtype=dtype, device="cuda")
        h = h_big[:, :, pad:pad + D]
    else:
        h_big, h = None, torch.empty((B, L, D), dtype=dtype, device="cuda")
    h0_np = (np.random.default_rng(c["seed"] + 1).standard_normal((B, D)).astype(np.float32)
             if c["h_init"] else None)
    h0 = torch.from_numpy(h0_np).cuda() if c["h_init"] else None
    out = lr.linrec_scan(a, b, h, h_init=h0, return_final=c["h_final"], reverse=c["reverse"],
                         a_ahead=c["a_ahead"])
    torch.cuda.synchronize()
    if c["a_ahead"]:
        # the decays one time step ahead; the first step's decay multiplies h_init: 1
        shifted = np.empty_like(a_ref)
        shifted[:, :-1] = a_ref[:, 1:]
        shifted[:, -1] = 1.0
        a_ref = shifted
    fn = oracle.linrec_oracle_rev_f64 if c["reverse"] else oracle.linrec_oracle_f64
    ref = fn(a_ref, b_ref, h_init=h0_np)
    if c["h_final"]:
        h_out, hf = out
        last = 0 if c["reverse"] else L - 1
        if L > 0:
            check(hf, ref[:, last, :], torch.float32, label + " h_final")
    else:
        h_out = out
    assert h_out.data_ptr() == h.data_ptr()
    check(h, ref, dtype, label)
    if h_big is not None:
        assert torch.isnan(h_big[:, :, :pad].float()).all() and torch.isnan(h_big[:, :, pad + D:].float()).all()
