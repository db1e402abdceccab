"""The streaming-ceiling kernels compute what their timings claim: every element of z is x + y,
for every launch shape, walk order and tile walk, ragged lengths included.  z starts as NaN, so
an element the kernel skips fails the comparison."""
import itertools

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sc():
    from linear_recurrence_scan_linrec_amd import stream_ceiling
    return stream_ceiling


def operands(n, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(n, generator=g).cuda()
    y = torch.randn(n, generator=g).cuda()
    z = torch.full((n,), float("nan"), device="cuda")
    return x, y, z


@pytest.mark.parametrize("rows,unroll,groups", [(1, 1, 1), (1, 4, 8), (32, 2, 2), (32, 4, 8), (7, 1, 16)])
def test_r2w1_writes_every_sum(sc, rows, unroll, groups):
    n = rows * 256 * unroll * 37
    x, y, z = operands(n, rows * 100 + unroll)
    print(f"stream_r2w1 n={n} rows={rows} unroll={unroll} groups_per_cu={groups}", flush=True)
    sc.stream_r2w1(x, y, z, rows, unroll, groups)
    torch.cuda.synchronize()
    assert torch.equal(z, x + y)


WALKS = list(itertools.product((8, 16, 32, 64), (1, 2, 4, 8), (4, 8)))


@pytest.mark.parametrize("lanes,waves,t", WALKS, ids=lambda v: str(v))
def test_column_walk_writes_every_sum(sc, lanes, waves, t):
    # L ragged against every tile height (tiles of 16 to 512 rows), D two slabs wide
    B, L, D = 3, 1000 + 3 * waves + t, 8 * lanes
    x, y, z = operands(B * L * D, lanes * 1000 + waves * 10 + t)
    print(f"column_walk B={B} L={L} D={D} lanes={lanes} waves={waves} steps_per_lane={t}", flush=True)
    sc.column_walk(x, y, z, B, L, D, lanes, waves, t)
    torch.cuda.synchronize()
    assert torch.equal(z, x + y)


def test_column_walk_at_the_pages_shape(sc):
    B, L, D = 32, 4096, 256
    x, y, z = operands(B * L * D, 7)
    print("column_walk B=32 L=4096 D=256 lanes=8 waves=2 steps_per_lane=8", flush=True)
    sc.column_walk(x, y, z, B, L, D, 8, 2, 8)
    torch.cuda.synchronize()
    assert torch.equal(z, x + y)
