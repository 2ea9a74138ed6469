"""The launch planners, on the host (no GPU): q8_0_gemv_plan and
q8_0_chain_plan report the plans q8_0_gemv and q8_0_chain_create use, and
these tests check them against properties that define a correct plan --
every op computed by exactly one launch, in an order that respects the
dependencies between ops, every (op, tile) item of a fused launch done by
exactly one workgroup, tiles of legal shapes whose LDS fits a CU."""
import itertools
import random

import pytest

# fake, aligned device addresses: the planners compare them, never read them
BASE = 0x100000000

KIB = 1024
W_STAGE = 64 * 272          # one weight column of a wave: 64 lanes x one 272-byte group
X_SLICE = 1024 + 16         # one x slice (256 floats) plus 16 bytes of bank offset
LDS_PER_CU = 160 * KIB


@pytest.fixture(scope="module")
def q8():
    import q8_block_quantized_gemv_amd as mod
    return mod


def wbytes(n, p):
    return p * (n // 32) * 34


def groups(n):
    return n // 256


def tiles(p, lanes):
    return -(-p // (64 // lanes))


# ------------------------------------------------------------------ q8_0_gemv_plan
@pytest.mark.parametrize("cus", [256, 64, 1])
@pytest.mark.parametrize("n", [256, 512, 1024, 2048, 3072, 3584, 18944, 1 << 20, 96, 160, 896, 4864])
def test_gemv_plan_is_a_legal_shape(q8, n, cus):
    for p in (1, 7, 63, 64, 300, 3584, 4608, 18944, 152064, (1 << 22) + 3):
        c, w, st, tr, g = q8.gemv_plan(n, p, cus)
        if n % 256:
            assert (c, st, tr) == (0, 0, 0) and w in (1, 4) and g >= 1
            continue
        assert c in (1, 2, 4) and w in (1, 2, 4) and st in (1, 2)
        assert (16 // c) % w == 0                   # every group slot has exactly one owner wave
        lds = w * (st * W_STAGE + 2 * c * X_SLICE)
        assert lds <= LDS_PER_CU
        assert 1 <= tr <= 64 // c and g == -(-p // tr)
        if tr < 64 // c:
            # shorter tiles only to even out CUs that hold two or more whole
            # tiles: still all resident, no more tiles a CU than whole tiles
            # would give, and the fewest rows a tile that allows
            whole = tiles(p, c)
            k = -(-whole // cus)
            assert k >= 2 and whole <= cus * (LDS_PER_CU // lds)
            assert -(-g // cus) == k and tr == -(-p // (k * cus))


def test_gemv_plan_row_poor_ops_use_small_tiles(q8):
    """Ops with few rows (every projection of a 0.6B or 7B model but gate, up
    and the lm_head) take 16-row tiles and split each tile's group columns
    over as many waves as there are columns, up to 4: all rows in one round
    of workgroups."""
    for n, p in ((3584, 3584), (18944, 3584), (1024, 2048), (3072, 1024), (2048, 1024)):
        c, w, _, tr, g = q8.gemv_plan(n, p, 256)
        assert c == 4 and tr == 16 and g == -(-p // 16) and g <= 256
        assert w == min(4, -(-groups(n) // 4)) or (w == 4 and groups(n) > 8)


def test_gemv_plan_evens_out_resident_tiles(q8):
    """The 7B gate (3584 -> 18944): 592 two-wave tiles of 32 rows would come
    two or three to a CU of 256; 758 tiles of 25 rows come at most three to
    a CU, all resident (three 42 KiB workgroups a CU)."""
    assert q8.gemv_plan(3584, 18944, 256) == (2, 2, 1, 25, 758)
    # an lm_head (many rounds of tiles) keeps whole tiles
    c, _, _, tr, _ = q8.gemv_plan(3584, 152064, 256)
    assert tr == 64 // c


@pytest.mark.parametrize("args,code", [((0, 64, 256), -2), ((48, 64, 256), -2), ((256, 0, 256), -2),
                                       ((256, 64, 0), -1), ((256, 64, 5000), -1)])
def test_gemv_plan_refuses(q8, args, code):
    with pytest.raises(q8.Q8Error) as e:
        q8.gemv_plan(*args)
    assert e.value.code == code


# ------------------------------------------------------------------ q8_0_chain_plan
class Pool:
    """Non-overlapping fake buffers, 1 MiB apart."""

    def __init__(self):
        self.next = BASE

    def take(self, nbytes):
        a = self.next
        self.next += (nbytes + (1 << 20) + 255) // 256 * 256
        return a


def reads(op):
    x, w, y, n, p = op
    return [(x, 4 * n), (w, wbytes(n, p))]


def writes(op):
    x, w, y, n, p = op
    return [(y, 4 * p)]


def overlap(a, b):
    return a[0] < b[0] + b[1] and b[0] < a[0] + a[1]


def depends(a, b):
    """b must wait for a: a write of either touches what the other reads or writes."""
    return (any(overlap(wb, r) for wb in writes(b) for r in reads(a) + writes(a)) or
            any(overlap(wa, r) for wa in writes(a) for r in reads(b)))


def check_plan(q8, ops, flags, cus=256):
    launches, top, tid = q8.chain_plan(ops, flags, cus)
    # every op in exactly one launch, launches in op order
    at = 0
    for L in launches:
        assert L["first_op"] == at and L["n_ops"] >= 1
        at += L["n_ops"]
    assert at == len(ops)
    per_op = bool(flags & q8.Q8_CHAIN_PER_OP)
    for k, L in enumerate(launches):
        members = ops[L["first_op"]:L["first_op"] + L["n_ops"]]
        # no op of a launch waits for another of the same launch
        for a, b in itertools.combinations(members, 2):
            assert not depends(a, b)
        if per_op:
            assert L["n_ops"] == 1
        elif k + 1 < len(launches):
            # a launch ends only where the next op has to wait for it
            nxt = ops[launches[k + 1]["first_op"]]
            assert any(depends(a, nxt) for a in members)
        if L["n_ops"] == 1:
            n, p = members[0][3], members[0][4]
            c, w, st, tr, g = q8.gemv_plan(n, p, cus)
            if n % 256 == 0:
                assert L["kind"] == q8.LAUNCH_ROWS
                assert (L["lanes_per_row"], L["waves"], L["stages"], L["tile_rows"], L["workgroups"]) == \
                    (c, w, st, tr, g)
            else:
                assert L["kind"] == q8.LAUNCH_SUPERROWS and L["workgroups"] == g
            assert L["first_tile"] == -1
            continue
        # a fused launch: every (op, tile) item exactly once, tile ids dense
        items = list(zip(top[L["first_tile"]:L["first_tile"] + L["workgroups"]],
                         tid[L["first_tile"]:L["first_tile"] + L["workgroups"]]))
        assert len(items) == len(set(items)) == L["workgroups"]
        by_op = {}
        for o, t in items:
            assert L["first_op"] <= o < L["first_op"] + L["n_ops"]
            by_op.setdefault(o, []).append(t)
        assert sorted(by_op) == list(range(L["first_op"], L["first_op"] + L["n_ops"]))
        whole = all(m[3] % 256 == 0 for m in members)
        if whole:
            assert L["kind"] == q8.LAUNCH_FUSED and L["tile_rows"] == 64 // L["lanes_per_row"]
            for o, ts in by_op.items():
                assert sorted(ts) == list(range(tiles(ops[o][4], L["lanes_per_row"])))
            same_width = len({m[3] for m in members}) == 1
            if flags & q8.Q8_CHAIN_SPLIT_K and same_width:
                # the latency plan of all the launch's rows (whole tiles:
                # where one op's plan would even out shorter tiles, the
                # launch keeps the whole-tile rules), tiles in op order
                c, w, st, tr, _ = q8.gemv_plan(members[0][3], sum(m[4] for m in members), cus)
                if tr == 64 // c:
                    assert (L["lanes_per_row"], L["waves"], L["stages"]) == (c, w, st)
                assert items == sorted(items)
            else:
                # steady-state tiles, largest tiles first: float x, one-wave
                # 16-row tiles, four lanes per row, one weight stage; x
                # quantized per column, two lanes per row, two weight stages
                # when rows are long, one when they are short
                if flags & q8.Q8_CHAIN_XQ:
                    b = [wbytes(m[3], m[4]) for m in members]
                    mean = sum(bb * groups(m[3]) for bb, m in zip(b, members)) / sum(b)
                    assert (L["lanes_per_row"], L["waves"], L["stages"]) == (2, 1, (2 if mean >= 8 else 1))
                else:
                    assert (L["lanes_per_row"], L["waves"], L["stages"]) == (4, 1, 1)
                rows = 64 // L["lanes_per_row"]
                sizes = [rows * (ops[o][3] // 32) * 34 for o, _ in items]
                assert sizes == sorted(sizes, reverse=True)
        else:
            assert L["kind"] == q8.LAUNCH_FUSED_MIXED
            for o, ts in by_op.items():
                fast = sorted(t for t in ts if not t & q8.TAIL_BIT)
                tail = sorted(t & ~q8.TAIL_BIT for t in ts if t & q8.TAIL_BIT)
                assert fast == list(range(len(fast))) and tail == list(range(len(tail)))
                assert fast or tail
                n, p = ops[o][3], ops[o][4]
                if n % 256 == 0:   # rows of whole groups: 32-row tiles (two lanes per row)
                    assert len(fast) == -(-p // 32) and not tail
    return launches


def decoder_layer(pool, hidden, q, kv, inter, x=None):
    """q, k, v from x; o from the attention output; gate, up from the norm of
    the new stream; down from their product -- real dependencies."""
    x = x or pool.take(4 * hidden)
    hn = pool.take(4 * hidden)
    ops = []
    for p in (q, kv, kv):
        ops.append((x, pool.take(wbytes(hidden, p)), pool.take(4 * p), hidden, p))
    # (attention's output stands in as q's output, silu(gate) * up as gate's)
    ops.append((ops[0][2], pool.take(wbytes(q, hidden)), hn, q, hidden))
    g, u = pool.take(4 * inter), pool.take(4 * inter)
    ops.append((hn, pool.take(wbytes(hidden, inter)), g, hidden, inter))
    ops.append((hn, pool.take(wbytes(hidden, inter)), u, hidden, inter))
    ops.append((g, pool.take(wbytes(inter, hidden)), x, inter, hidden))   # writes back into x
    return ops


@pytest.mark.parametrize("flags", [0, 1, 2, 4, 6])
@pytest.mark.parametrize("shape", [(1024, 2048, 1024, 3072), (3584, 3584, 512, 18944), (896, 896, 128, 4864),
                                   (512, 512, 256, 1376)])
def test_decoder_chain_plans(q8, shape, flags):
    pool = Pool()
    ops = []
    x = pool.take(4 * shape[0])
    for _ in range(3):
        ops += decoder_layer(pool, *shape, x=x)
    launches = check_plan(q8, ops, flags)
    if not flags & q8.Q8_CHAIN_PER_OP:
        # q|k|v and gate|up fuse; o and down wait for what came before
        assert [L["n_ops"] for L in launches][:4] == [3, 1, 2, 1]


def test_independent_ops_fuse_into_one_launch(q8):
    pool = Pool()
    ops = [(pool.take(4 * n), pool.take(wbytes(n, p)), pool.take(4 * p), n, p)
           for n, p in ((3584, 3584), (3584, 18944), (18944, 3584), (1024, 151936), (256, 1))]
    launches = check_plan(q8, ops, 0)
    assert len(launches) == 1 and launches[0]["kind"] == q8.LAUNCH_FUSED


@pytest.mark.parametrize("seed", range(12))
def test_random_chains(q8, seed):
    """Random ops over a small pool of buffers (so that many read or write
    what others touched), random widths, every flag combination."""
    rng = random.Random(seed)
    pool = Pool()
    widths = [256, 512, 1024, 3584, 96, 160, 896]
    bufs = {}
    ops = []
    for i in range(rng.randint(1, 40)):
        n = rng.choice(widths)
        p = rng.choice([1, 5, 64, 65, 300, 1024, 4099])
        # x and y from a few shared buffers, sized for the largest use
        xi, yi = rng.randrange(6), rng.randrange(6)
        while yi == xi:
            yi = rng.randrange(6)
        for k in (xi, yi):
            if k not in bufs:
                bufs[k] = pool.take(4 * 8192)
        ops.append((bufs[xi], pool.take(wbytes(n, p)), bufs[yi], n, p))
    for flags in (0, 1, 2, 4, 6):
        check_plan(q8, ops, flags, cus=rng.choice([256, 80, 8]))


def test_chain_plan_validates_like_create(q8):
    pool = Pool()
    x, w = pool.take(4 * 256), pool.take(wbytes(256, 4))
    with pytest.raises(q8.Q8Error) as e:
        q8.chain_plan([(x, w, x + 8, 256, 4)])        # y overlaps x
    assert e.value.code == q8.Q8_ERR_ALIAS
    with pytest.raises(q8.Q8Error) as e:
        q8.chain_plan([(x, w, pool.take(16), 250, 4)])
    assert e.value.code == q8.Q8_ERR_SHAPE
    with pytest.raises(q8.Q8Error) as e:
        q8.chain_plan([(x, w, pool.take(16), 256, 4)], flags=8)
    assert e.value.code == q8.Q8_ERR_INVALID_ARG
