"""GPU parity: libsbd (through its C ABI) against the CPU oracle, bit for bit.

Tolerance is zero everywhere: the path is integer and bit work, so nnz, the
order of the indices and the value bits must be identical.  Sizes span
several 32768-element tiles, ragged tails, unaligned views, empty and
all-changed inputs, signed zeros and NaN payloads, and tiles whose change
counts sit on each side of the compaction's staging limits (512 and 8192
changes per tile, and 1024 and 4096, the limits of earlier layouts).  No oracle input or expected value comes from the GPU
path.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

TILE = 32768  # elements per compaction tile (the sizes below also straddle 16K and 64K)
SIZES = [0, 1, 7, 8, 9, 63, 64, 65, 511, 512, 513, 2047, 2048, 2049, 16383, 16385,
         TILE - 1, TILE, TILE + 1, 2 * TILE + 3, 65535, 65537, 5 * TILE - 8, 100_003,
         (1 << 20) + 5]
FRACS = [0.0, 0.01, 0.5, 1.0]


@pytest.fixture(scope="module")
def sbd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_bf16_delta_amd as m

    m.load()
    return m


def np_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def gpu_bits(a: np.ndarray, pad_front: int = 0) -> torch.Tensor:
    """Device bf16 tensor holding the bits of `a`; with pad_front > 0 the
    returned view starts pad_front elements into its allocation (unaligned)."""
    buf = torch.zeros(a.size + pad_front, dtype=torch.int16)
    buf[pad_front:] = torch.from_numpy(a.view(np.int16).copy())
    return buf.cuda().view(torch.bfloat16)[pad_front:]


def rand_case(seed, n, frac, special=True):
    rng = np.random.default_rng(seed)
    old = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    new = old.copy()
    k = int(round(frac * n))
    if k:
        pos = rng.choice(n, size=k, replace=False)
        off = rng.integers(1, 1 << 16, size=k, dtype=np.uint32).astype(np.uint16)
        new[pos] = (old[pos].astype(np.uint32) + off).astype(np.uint16)
    if special and n >= 8:
        old[:8] = [0x0000, 0x7FC0, 0x7FC0, 0x7F80, 0x8000, 0x0001, 0xFF80, 0x3F80]
        new[:8] = [0x8000, 0x7FC0, 0x7FC1, 0x7F80, 0x0000, 0x0001, 0x7F80, 0x3F80]
    return old, new


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("frac", FRACS)
def test_diff_matches_oracle(sbd, oracle_mod, n, frac):
    old, new = rand_case(n * 7 + int(frac * 1000), n, frac)
    ri, rv = oracle_mod.diff(old, new)
    gi, gv = sbd.diff(gpu_bits(old), gpu_bits(new))
    assert gi.numel() == ri.size
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)


@pytest.mark.parametrize("pad_old,pad_new", [(1, 1), (3, 0), (0, 5), (7, 2)])
@pytest.mark.parametrize("n", [TILE + 77, 3 * TILE])
def test_diff_unaligned_views(sbd, oracle_mod, pad_old, pad_new, n):
    old, new = rand_case(99 + pad_old + 10 * pad_new, n, 0.03)
    ri, rv = oracle_mod.diff(old, new)
    gi, gv = sbd.diff(gpu_bits(old, pad_old), gpu_bits(new, pad_new))
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)


# changes per tile, straddling the compact-slot (512) and staging (8192)
# limits, plus 1023-1025 and 4095-4097 (limits of earlier layouts); the last
# tile is ragged (5000 of 32768 elements, all changed)
TILE_COUNTS = [0, 1, 1023, 1024, 1025, 4095, 4096, 4097, TILE, 3, TILE // 2, 1027, 511, 512,
               513, 8191, 8192, 8193, 5000]


def tile_kinds_case(seed, counts=TILE_COUNTS, last_valid=5000):
    rng = np.random.default_rng(seed)
    n = (len(counts) - 1) * TILE + last_valid
    old = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    new = old.copy()
    for t, c in enumerate(counts):
        width = TILE if t < len(counts) - 1 else last_valid
        pos = t * TILE + rng.choice(width, size=min(c, width), replace=False)
        off = rng.integers(1, 1 << 16, size=pos.size, dtype=np.uint32).astype(np.uint16)
        new[pos] = (old[pos].astype(np.uint32) + off).astype(np.uint16)
    return old, new


@pytest.mark.parametrize("pad", [0, 3])
def test_diff_tile_kinds(sbd, oracle_mod, pad):
    """Every staging path -- compact slot, shared arena, dense re-read -- and their
    limits, aligned and unaligned, as one tensor and as a parameter list."""
    old, new = tile_kinds_case(11 + pad)
    ri, rv = oracle_mod.diff(old, new)
    per_tile = np.bincount(ri // TILE, minlength=len(TILE_COUNTS))
    assert per_tile.tolist() == TILE_COUNTS  # the fixture is what it claims
    gi, gv = sbd.diff(gpu_bits(old, pad), gpu_bits(new, pad))
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)
    # the same tiles as a list of one-tile parameters plus the whole tensor
    olds = [old[t * TILE:(t + 1) * TILE] for t in range(len(TILE_COUNTS))] + [old]
    news = [new[t * TILE:(t + 1) * TILE] for t in range(len(TILE_COUNTS))] + [new]
    ri2, rv2, rn2, ro2 = oracle_mod.diff_many(olds, news)
    gi2, gv2, gn2, go2 = sbd.diff_many([gpu_bits(o, pad) for o in olds],
                                       [gpu_bits(x, pad) for x in news])
    assert np.array_equal(gn2.cpu().numpy(), rn2)
    assert np.array_equal(go2.cpu().numpy(), ro2)
    assert np.array_equal(gi2.cpu().numpy(), ri2)
    assert np.array_equal(np_bits(gv2), rv2)


# (changes in the first half, changes in the second half) of each tile: the
# count kernel loads and stages a tile as two halves of 16384 elements, so a
# tile's entries may all sit in one half, or the first half may fill or
# overflow the 8192-entry stage alone
HALF = TILE // 2
HALF_COUNTS = [(0, 1), (1, 0), (4096, 0), (0, 4096), (4097, 0), (0, 4097), (4095, 1),
               (1, 4095), (2048, 2049), (2048, 2048), (512, 0), (0, 513), (HALF, 0), (0, HALF),
               (600, 600), (8192, 0), (8193, 0), (0, 8193), (8191, 1), (4096, 4097),
               (4096, 4096), (0, 0)]


def halves_case(seed, pairs=HALF_COUNTS, last_valid=20000):
    """Tiles with the given per-half counts; elements HALF - 1 and HALF of
    every tile with changes in both halves are among them (the seam); the
    last tile is ragged, its second half partial, all of it changed."""
    rng = np.random.default_rng(seed)
    n = len(pairs) * TILE + last_valid
    old = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    new = old.copy()
    for t, (a, b) in enumerate(pairs):
        pos = []
        if a:
            pa = rng.choice(HALF, size=a, replace=False)
            if b and (HALF - 1) not in pa:
                pa[0] = HALF - 1
            pos.append(pa)
        if b:
            pb = HALF + rng.choice(HALF, size=b, replace=False)
            if a and HALF not in pb:
                pb[0] = HALF
            pos.append(pb)
        if pos:
            q = t * TILE + np.concatenate(pos)
            off = rng.integers(1, 1 << 16, size=q.size, dtype=np.uint32).astype(np.uint16)
            new[q] = (old[q].astype(np.uint32) + off).astype(np.uint16)
    tail = np.arange(len(pairs) * TILE, n)
    new[tail] = (old[tail].astype(np.uint32) + 1).astype(np.uint16)
    return old, new


@pytest.mark.parametrize("pad", [0, 3])
def test_diff_tile_halves(sbd, oracle_mod, pad):
    """Tiles whose changes sit in one half only, fill or overflow the stage
    from one half, or meet at the seam between the halves, aligned and
    unaligned, as one tensor and as a parameter list."""
    old, new = halves_case(17 + pad)
    ri, rv = oracle_mod.diff(old, new)
    ntiles = len(HALF_COUNTS)
    first = np.bincount(ri[ri < ntiles * TILE] // HALF, minlength=2 * ntiles)
    assert first.tolist() == [c for ab in HALF_COUNTS for c in ab]  # the fixture is what it claims
    gi, gv = sbd.diff(gpu_bits(old, pad), gpu_bits(new, pad))
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)
    olds = [old[t * TILE:(t + 1) * TILE] for t in range(ntiles + 1)] + [old]
    news = [new[t * TILE:(t + 1) * TILE] for t in range(ntiles + 1)] + [new]
    ri2, rv2, rn2, ro2 = oracle_mod.diff_many(olds, news)
    gi2, gv2, gn2, go2 = sbd.diff_many([gpu_bits(o, pad) for o in olds],
                                       [gpu_bits(x, pad) for x in news])
    assert np.array_equal(gn2.cpu().numpy(), rn2)
    assert np.array_equal(go2.cpu().numpy(), ro2)
    assert np.array_equal(gi2.cpu().numpy(), ri2)
    assert np.array_equal(np_bits(gv2), rv2)


@pytest.mark.parametrize("seed", [41, 42])
def test_diff_arena_mixed_tiles_repeated(sbd, oracle_mod, seed):
    """Hundreds of tiles whose counts fall on both sides of every staging
    limit, so many tiles share the staging arena in whatever order they
    finish; two different inputs through one workspace in a row (the arena
    counter starts afresh each call), as one tensor and as a list."""
    from sparse_bf16_delta_amd.plan import DiffPlan

    rng = np.random.default_rng(seed)
    ntiles = 300
    counts = rng.choice([0, 5, 600, 1024, 1025, 2000, 3500, 4096, 4097, 8192, 8193, 9000],
                        size=ntiles)
    cases = [tile_kinds_case(seed, counts=list(counts), last_valid=TILE),
             tile_kinds_case(seed + 100, counts=list(rng.permutation(counts)), last_valid=TILE)]
    n = ntiles * TILE
    for old, new in cases:  # calls on one stream share the cached workspace
        ri, rv = oracle_mod.diff(old, new)
        gi, gv = sbd.diff(gpu_bits(old), gpu_bits(new))
        assert np.array_equal(gi.cpu().numpy(), ri)
        assert np.array_equal(np_bits(gv), rv)
    # the list form: parameters of uneven sizes cut across tiles, one plan run twice
    cuts = [0, 5 * TILE + 77, 40 * TILE, 41 * TILE + 3, 200 * TILE + 1000, n]
    for old, new in cases:
        olds = [gpu_bits(old[a:b]) for a, b in zip(cuts, cuts[1:])]
        news = [gpu_bits(new[a:b]) for a, b in zip(cuts, cuts[1:])]
        plan = DiffPlan(olds, news, capacity=n // 4)
        for _ in range(2):
            plan.run()
            idx, val, nnz, offsets = plan.result()
            ri2, rv2, rn2, ro2 = oracle_mod.diff_many([old[a:b] for a, b in zip(cuts, cuts[1:])],
                                                      [new[a:b] for a, b in zip(cuts, cuts[1:])])
            assert np.array_equal(offsets.cpu().numpy(), ro2)
            assert np.array_equal(idx.cpu().numpy(), ri2)
            assert np.array_equal(np_bits(val), rv2)


@pytest.mark.parametrize("arena", ["none", "some", "capacity"])
@pytest.mark.parametrize("seed", [51, 52])
def test_diff_arena_size_does_not_change_the_delta(sbd, oracle_mod, arena, seed):
    """The staging arena is whatever the workspace holds past its minimum:
    none at all, a few tiles' worth, or the size the capacity asks for.
    Tiles that find no room (staged or dense) are recomputed from both
    inputs; the delta equals the oracle's in every case, as one tensor and
    as a list, and a capacity cut still writes nothing past the capacity."""
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    rng = np.random.default_rng(seed)
    ntiles = 120
    counts = rng.choice([0, 5, 511, 512, 513, 800, 2000, 4096, 4097, 8192, 8193, 9000, TILE],
                        size=ntiles)
    old, new = tile_kinds_case(seed, counts=list(counts), last_valid=TILE)
    ri, rv = oracle_mod.diff(old, new)
    n = old.size
    lib = _abi.load()
    o, x = gpu_bits(old), gpu_bits(new)
    low = lib.delta_workspace_size_for(n, 1, 0)
    size = {"none": low, "some": low + 48 * 1024,
            "capacity": lib.delta_workspace_size_for(n, 1, ri.size)}[arena]
    ws = torch.empty(size, dtype=torch.uint8, device="cuda")
    for cap in (ri.size + 10, ri.size // 2):
        guard = 4096
        idx = torch.full((cap + guard,), -7, dtype=torch.int32, device="cuda")
        val = torch.full((cap + guard,), -7, dtype=torch.int16, device="cuda")
        nnz = torch.zeros(1, dtype=torch.int64, device="cuda")
        _abi.check(lib.delta_diff(_ptr(o), _ptr(x), n, _ptr(idx), _ptr(val), cap, _ptr(nnz),
                                  _ptr(ws), ws.numel(), _stream(o.device)))
        m = min(cap, ri.size)
        assert int(nnz.item()) == ri.size
        assert np.array_equal(idx[:m].cpu().numpy(), ri[:m])
        assert np.array_equal(np_bits(val[:m]), rv[:m])
        assert bool((idx[m:] == -7).all()) and bool((val[m:] == -7).all())
    # the list form, parameters cut across tiles, with the same arena budget
    cuts = [0, 7 * TILE + 5, 30 * TILE, 31 * TILE + 1, 90 * TILE + 333, n]
    olds = [gpu_bits(old[a:b]) for a, b in zip(cuts, cuts[1:])]
    news = [gpu_bits(new[a:b]) for a, b in zip(cuts, cuts[1:])]
    k = len(olds)
    lowk = lib.delta_workspace_size_for(n, k, 0)
    sizek = {"none": lowk, "some": lowk + 48 * 1024,
             "capacity": lib.delta_workspace_size_for(n, k, ri.size)}[arena]
    wsk = torch.empty(sizek, dtype=torch.uint8, device="cuda")
    import ctypes
    optrs = (ctypes.c_void_p * k)(*[t.data_ptr() for t in olds])
    nptrs = (ctypes.c_void_p * k)(*[t.data_ptr() for t in news])
    nums = (ctypes.c_int64 * k)(*[t.numel() for t in olds])
    idx = torch.full((ri.size,), -7, dtype=torch.int32, device="cuda")
    val = torch.full((ri.size,), -7, dtype=torch.int16, device="cuda")
    nnzk = torch.zeros(k, dtype=torch.int64, device="cuda")
    offk = torch.zeros(k + 1, dtype=torch.int64, device="cuda")
    _abi.check(lib.delta_diff_many(k, optrs, nptrs, nums, _ptr(idx), _ptr(val), ri.size,
                                   _ptr(nnzk), _ptr(offk), _ptr(wsk), wsk.numel(),
                                   _stream(o.device)))
    ri2, rv2, rn2, ro2 = oracle_mod.diff_many([old[a:b] for a, b in zip(cuts, cuts[1:])],
                                              [new[a:b] for a, b in zip(cuts, cuts[1:])])
    assert np.array_equal(offk.cpu().numpy(), ro2)
    assert np.array_equal(idx.cpu().numpy(), ri2)
    assert np.array_equal(np_bits(val), rv2)


@pytest.mark.parametrize("cut", [1024 + 1023 + 1, 1 + 1023 + 1024 + 1025 + 4095 + 7,
                                 sum(TILE_COUNTS[:8]) + 100, sum(TILE_COUNTS[:16]) + 4097,
                                 sum(TILE_COUNTS) - 1])
def test_diff_tile_kinds_capacity(sbd, oracle_mod, cut):
    """A capacity that ends inside a compact, a wide and a dense tile's run:
    the prefix is exact and nothing past the capacity is written."""
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    old, new = tile_kinds_case(23)
    ri, rv = oracle_mod.diff(old, new)
    n = old.size
    lib = _abi.load()
    o, x = gpu_bits(old), gpu_bits(new)
    guard = 4096
    idx = torch.full((cut + guard,), -7, dtype=torch.int32, device="cuda")
    val = torch.full((cut + guard,), -7, dtype=torch.int16, device="cuda")
    nnz = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(lib.delta_workspace_size(n, 1), dtype=torch.uint8, device="cuda")
    _abi.check(lib.delta_diff(_ptr(o), _ptr(x), n, _ptr(idx), _ptr(val), cut, _ptr(nnz),
                              _ptr(ws), ws.numel(), _stream(o.device)))
    assert int(nnz.item()) == ri.size
    assert np.array_equal(idx[:cut].cpu().numpy(), ri[:cut])
    assert np.array_equal(np_bits(val[:cut]), rv[:cut])
    assert bool((idx[cut:] == -7).all()) and bool((val[cut:] == -7).all())


@pytest.mark.parametrize("pad", [0, 3])
def test_diff_many_sharded_matches_oracle(sbd, oracle_mod, pad):
    """Global int64 positions: every tile kind, offsets past 2^31, unaligned."""
    old, new = tile_kinds_case(31 + pad)
    olds = [old[:TILE * 3], old, old[5:TILE + 9], old[:0], old[TILE:]]
    news = [new[:TILE * 3], new, new[5:TILE + 9], new[:0], new[TILE:]]
    offs = [0, (1 << 31) + 7, 5 * (1 << 33) + 3, 123, 1 << 40]
    ri, rv, rn, ro = oracle_mod.shard_delta_many(olds, news, offs)
    gi, gv, gn, go = sbd.diff_many([gpu_bits(o, pad) for o in olds],
                                   [gpu_bits(x, pad) for x in news], flat_offsets=offs)
    assert gi.dtype == torch.int64
    assert np.array_equal(gn.cpu().numpy(), rn)
    assert np.array_equal(go.cpu().numpy(), ro)
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)


@pytest.mark.parametrize("world", [1, 3, 8])
def test_sharded_ranks_concatenate_to_full_delta(sbd, oracle_mod, world):
    """Each rank diffs its Shard(0) rows of three parameters on the GPU; in
    rank order the global positions are the whole parameters' deltas."""
    rng = np.random.default_rng(world)
    shapes = [(1003, 64), (4096, 40), (7, 3, 11)]
    fulls = []
    for sh in shapes:
        o, x = rand_case(int(rng.integers(1 << 20)), int(np.prod(sh)), 0.04, special=False)
        fulls.append((o, x))
    got = {p: ([], []) for p in range(len(shapes))}
    for rank in range(world):
        lo, ln, offs = [], [], []
        for p, sh in enumerate(shapes):
            first, count = sbd.shard0_piece(sh[0], world, rank)
            inner = int(np.prod(sh[1:]))
            lo.append(gpu_bits(fulls[p][0][first * inner:(first + count) * inner]))
            ln.append(gpu_bits(fulls[p][1][first * inner:(first + count) * inner]))
            offs.append(sbd.flat_offset(sh, first))
        gi, gv, gn, go = sbd.diff_many(lo, ln, flat_offsets=offs)
        o_h = go.cpu().numpy()
        for p in range(len(shapes)):
            got[p][0].append(gi[o_h[p]:o_h[p + 1]].cpu().numpy())
            got[p][1].append(np_bits(gv[o_h[p]:o_h[p + 1]]))
    for p, (o, x) in enumerate(fulls):
        ri, rv = oracle_mod.diff(o, x)
        assert np.array_equal(np.concatenate(got[p][0]), ri.astype(np.int64))
        assert np.array_equal(np.concatenate(got[p][1]), rv)


def test_diff_many_sharded_capacity(sbd, oracle_mod):
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream
    import ctypes

    old, new = tile_kinds_case(41)
    ri, rv, rn, ro = oracle_mod.shard_delta_many([old], [new], [1 << 35])
    cut = 1024 + 1023 + 500
    lib = _abi.load()
    o, x = gpu_bits(old), gpu_bits(new)
    guard = 2048
    idx = torch.full((cut + guard,), -7, dtype=torch.int64, device="cuda")
    val = torch.full((cut + guard,), -7, dtype=torch.int16, device="cuda")
    nnz = torch.zeros(1, dtype=torch.int64, device="cuda")
    offsets = torch.zeros(2, dtype=torch.int64, device="cuda")
    ws = torch.empty(lib.delta_workspace_size(old.size, 1), dtype=torch.uint8, device="cuda")
    ptrs_o = (ctypes.c_void_p * 1)(o.data_ptr())
    ptrs_n = (ctypes.c_void_p * 1)(x.data_ptr())
    nums = (ctypes.c_int64 * 1)(old.size)
    fos = (ctypes.c_int64 * 1)(1 << 35)
    _abi.check(lib.delta_diff_many_sharded(1, ptrs_o, ptrs_n, nums, fos, _ptr(idx), _ptr(val),
                                           cut, _ptr(nnz), _ptr(offsets), _ptr(ws), ws.numel(),
                                           _stream(o.device)))
    assert int(offsets[1].item()) == ri.size
    assert np.array_equal(idx[:cut].cpu().numpy(), ri[:cut])
    assert np.array_equal(np_bits(val[:cut]), rv[:cut])
    assert bool((idx[cut:] == -7).all()) and bool((val[cut:] == -7).all())


def test_diff_capacity_protocol(sbd, oracle_mod):
    """Entries past `capacity` are never written; nnz still reports the truth."""
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    n = 5 * TILE + 11
    old, new = rand_case(5, n, 0.2)
    ri, rv = oracle_mod.diff(old, new)
    lib = _abi.load()
    o, x = gpu_bits(old), gpu_bits(new)
    cap = ri.size // 3
    guard = 4096
    idx = torch.full((cap + guard,), -7, dtype=torch.int32, device="cuda")
    val = torch.full((cap + guard,), -7, dtype=torch.int16, device="cuda")
    nnz = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(lib.delta_workspace_size(n, 1), dtype=torch.uint8, device="cuda")
    _abi.check(lib.delta_diff(_ptr(o), _ptr(x), n, _ptr(idx), _ptr(val), cap, _ptr(nnz),
                              _ptr(ws), ws.numel(), _stream(o.device)))
    assert int(nnz.item()) == ri.size
    assert np.array_equal(idx[:cap].cpu().numpy(), ri[:cap])
    assert np.array_equal(np_bits(val[:cap]), rv[:cap])
    assert bool((idx[cap:] == -7).all()) and bool((val[cap:] == -7).all())
    # the wrapper's retry path returns the full delta
    gi, gv = sbd.diff(o, x, capacity=cap)
    assert np.array_equal(gi.cpu().numpy(), ri)


def test_diff_deterministic_and_repeatable(sbd):
    old, new = rand_case(17, 40 * TILE + 5, 0.05)
    o, x = gpu_bits(old), gpu_bits(new)
    a = sbd.diff(o, x)
    for _ in range(3):
        b = sbd.diff(o, x)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int16),
                                                     b[1].view(torch.int16))


def _param_list(seed, sizes, frac):
    olds, news = [], []
    for i, s in enumerate(sizes):
        o, x = rand_case(seed * 1000 + i, s, frac, special=s >= 8)
        olds.append(o)
        news.append(x)
    return olds, news


MANY_SIZES = [128, 0, TILE, 1, TILE + 1, 1024, 0, 3 * TILE - 1, 128, 7, 65536, 33_000]


@pytest.mark.parametrize("frac", [0.0, 0.02, 0.6])
def test_diff_many_matches_oracle(sbd, oracle_mod, frac):
    olds, news = _param_list(3, MANY_SIZES, frac)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    gi, gv, gn, go = sbd.diff_many([gpu_bits(o) for o in olds], [gpu_bits(x) for x in news])
    assert np.array_equal(gn.cpu().numpy(), rn)
    assert np.array_equal(go.cpu().numpy(), ro)
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)


def test_diff_many_unaligned_and_capacity(sbd, oracle_mod):
    olds, news = _param_list(4, [TILE + 5, 300, 2 * TILE], 0.1)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    g_o = [gpu_bits(o, pad) for o, pad in zip(olds, (1, 0, 3))]
    g_n = [gpu_bits(x, pad) for x, pad in zip(news, (2, 5, 0))]
    gi, gv, gn, go = sbd.diff_many(g_o, g_n, capacity=int(ro[-1]) // 2)
    assert np.array_equal(go.cpu().numpy(), ro)
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)


@pytest.mark.parametrize("n,frac", [(1, 1.0), (513, 0.3), (TILE + 3, 0.01), (1 << 20, 0.08),
                                    (1 << 20, 1.0), (100_003, 0.0)])
def test_apply_matches_oracle(sbd, oracle_mod, n, frac):
    old, new = rand_case(n + 3, n, frac)
    ri, rv = oracle_mod.diff(old, new)
    want = old.copy()
    oracle_mod.apply_(want, ri, rv)
    snap = gpu_bits(old)
    sbd.apply_(snap, torch.from_numpy(ri).cuda(),
               torch.from_numpy(rv.view(np.int16)).cuda().view(torch.bfloat16),
               check_indices=True)
    assert np.array_equal(np_bits(snap), want)


def test_apply_unaligned_delta_arrays(sbd, oracle_mod):
    n = 3 * TILE + 9
    old, new = rand_case(8, n, 0.07)
    ri, rv = oracle_mod.diff(old, new)
    want = old.copy()
    oracle_mod.apply_(want, ri, rv)
    ib = torch.zeros(ri.size + 3, dtype=torch.int32)
    ib[3:] = torch.from_numpy(ri)
    vb = torch.zeros(rv.size + 1, dtype=torch.int16)
    vb[1:] = torch.from_numpy(rv.view(np.int16))
    snap = gpu_bits(old, 1)
    sbd.apply_(snap, ib.cuda()[3:], vb.cuda()[1:].view(torch.bfloat16))
    assert np.array_equal(np_bits(snap), want)


def test_apply_skips_out_of_range_indices(sbd, oracle_mod):
    """Entries outside [0, n) are counted and never written; the others are."""
    n = 1000
    snap0 = np.arange(n, dtype=np.uint16)
    idx = np.array([3, 5, 10, 40, 999, 1000, 4096, 2_000_000_000], dtype=np.int32)
    val = np.full(idx.size, 0xABCD, dtype=np.uint16)
    buf = gpu_bits(np.concatenate([snap0, np.full(64, 7, dtype=np.uint16)]))
    snap = buf[:n]
    with pytest.raises(sbd.DeltaError, match="3 delta entries"):
        sbd.apply_(snap, torch.from_numpy(idx).cuda(),
                   torch.from_numpy(val.view(np.int16)).cuda().view(torch.bfloat16),
                   check_indices=True)
    want = snap0.copy()
    oracle_mod.apply_(want, idx[:5], val[:5])
    got = np_bits(buf)
    assert np.array_equal(got[:n], want)
    assert np.all(got[n:] == 7)  # nothing past the snapshot


def test_apply_unsorted_is_flagged_and_stays_inside(sbd):
    """An unsorted or duplicated delta breaks the precondition: it is counted,
    the values at its positions are unspecified, and no other position of the
    snapshot (or memory beyond it) changes."""
    n = 1000
    snap0 = np.arange(n, dtype=np.uint16)
    idx = np.array([5, 3, 3, 999, 1000, -1, 2_000_000_000, 10], dtype=np.int32)
    val = np.full(idx.size, 0xABCD, dtype=np.uint16)
    buf = gpu_bits(np.concatenate([snap0, np.full(64, 7, dtype=np.uint16)]))
    snap = buf[:n]
    with pytest.raises(sbd.DeltaError, match="6 delta entries"):
        sbd.apply_(snap, torch.from_numpy(idx).cuda(),
                   torch.from_numpy(val.view(np.int16)).cuda().view(torch.bfloat16),
                   check_indices=True)
    got = np_bits(buf)
    touched = np.zeros(n, dtype=bool)
    touched[[3, 5, 10, 999]] = True
    assert np.array_equal(got[:n][~touched], snap0[~touched])
    assert np.all(np.isin(got[:n][touched], [0xABCD]) | (got[:n][touched] == snap0[touched]))
    assert np.all(got[n:] == 7)


@pytest.mark.parametrize("frac", [0.02, 0.05, 0.1, 0.3])
@pytest.mark.parametrize("pad", [0, 1, 8])
def test_apply_dense_runs_and_boundaries(sbd, oracle_mod, frac, pad):
    """Densities around the merge threshold, on a snapshot that is aligned or
    offset by 1 or 8 elements (64-byte segments then start inside the
    snapshot's first one); chunk edges share segments."""
    n = 9 * 2048 * 40 + 77
    old, new = rand_case(int(frac * 100) + pad, n, frac, special=False)
    ri, rv = oracle_mod.diff(old, new)
    snap = gpu_bits(old, pad)
    sbd.apply_(snap, torch.from_numpy(ri).cuda(),
               torch.from_numpy(rv.view(np.int16)).cuda().view(torch.bfloat16))
    assert np.array_equal(np_bits(snap), new)


# The segment rewrite of sparse workgroups runs only for deltas of at least
# 2^25 entries (below that, masked stores are cheaper): these cases are that
# large, so they check properties that hold at any size -- the result equals
# `new` -- with the delta taken by torch's own comparison, not by diff.
SEG_N = (1 << 30) + 12345


def _torch_delta(old_bits, new_bits):
    idx = torch.nonzero(old_bits != new_bits).reshape(-1).to(torch.int32)
    return idx, new_bits[idx.long()].view(torch.bfloat16)


def _sparse_pair(n, seed, percent=3.5):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    old = torch.randint(-(1 << 15), 1 << 15, (n,), dtype=torch.int16, device="cuda", generator=g)
    pick = torch.randint(0, 1000, (n,), dtype=torch.int16, device="cuda", generator=g)
    new = torch.where(pick < int(percent * 10), old ^ 0x1, old)
    del pick
    return old, new


@pytest.mark.parametrize("pad", [0, 3])
def test_apply_segment_rewrite_large(sbd, pad):
    """About 37.6 million entries at 3.5 % (span per entry above the merge
    threshold): sparse workgroups rewrite whole 64-byte segments; the
    snapshot starts `pad` elements into its allocation, with guard elements
    after it."""
    n = SEG_N
    old, new = _sparse_pair(n, 7 + pad)
    idx, val = _torch_delta(old, new)
    assert idx.numel() >= (1 << 25)
    buf = torch.full((pad + n + 64,), 7, dtype=torch.int16, device="cuda")
    buf[pad:pad + n] = old
    snap = buf[pad:pad + n].view(torch.bfloat16)
    sbd.apply_(snap, idx, val, check_indices=True)
    assert torch.equal(buf[pad:pad + n], new)
    assert bool((buf[:pad] == 7).all()) and bool((buf[pad + n:] == 7).all())
    sbd.apply_(snap, *_torch_delta(new, old))  # and back
    assert torch.equal(buf[pad:pad + n], old)


@pytest.mark.parametrize("cap_factor", [1, 3])
def test_apply_many_segment_rewrite_unaligned_params(sbd, cap_factor):
    """A list packed back to back at odd element offsets (each parameter's
    segments start at a different shift, edge segments shared with the
    neighbours), more than 2^25 entries in all.  With the exact count the
    large-delta kernel applies it (one entry per lane); with a buffer three
    times that size passed as the capacity, the density bound rules that
    kernel out and the 2048-entry-chunk kernel rewrites the segments."""
    sizes = [(1 << 29) + 7, 5, (1 << 28) + 3, 1000, (1 << 29) - 11]
    total = sum(sizes)
    old, new = _sparse_pair(total, 21)
    buf = torch.full((1 + total + 64,), 7, dtype=torch.int16, device="cuda")
    buf[1:1 + total] = old
    views, idxs, vals, counts, pos = [], [], [], [], 0
    for n in sizes:
        views.append(buf[1 + pos:1 + pos + n].view(torch.bfloat16))
        i, v = _torch_delta(old[pos:pos + n], new[pos:pos + n])
        idxs.append(i)
        vals.append(v)
        counts.append(i.numel())
        pos += n
    offsets = torch.tensor([0] + list(np.cumsum(counts)), dtype=torch.int64, device="cuda")
    m = int(offsets[-1])
    assert m >= (1 << 25)
    idx = torch.full((cap_factor * m,), -1, dtype=torch.int32, device="cuda")
    val = torch.zeros(cap_factor * m, dtype=torch.bfloat16, device="cuda")
    idx[:m] = torch.cat(idxs)
    val[:m] = torch.cat(vals)
    sbd.apply_many_(views, idx, val, offsets, max_nnz=cap_factor * m, check_indices=True)
    assert torch.equal(buf[1:1 + total], new)
    assert int(buf[0]) == 7 and bool((buf[1 + total:] == 7).all())


def test_apply_segment_rewrite_with_broken_precondition(sbd):
    """A large delta with an unsorted pair, a repeated index and an
    out-of-range entry in three workgroups' chunks: they are counted, those
    chunks are written entry by entry, every other position ends as in
    `new` (or keeps its old value where its entry was replaced), and nothing
    outside the snapshot changes."""
    n = SEG_N
    old, new = _sparse_pair(n, 33)
    idx, val = _torch_delta(old, new)
    k0, k1, k2 = 5_000_000, 12_000_000, 30_000_000
    orig1, orig2 = int(idx[k1]), int(idx[k2])
    idx2, val2 = idx.clone(), val.view(torch.int16).clone()
    idx2[[k0, k0 + 1]] = idx2[[k0 + 1, k0]]
    val2[[k0, k0 + 1]] = val2[[k0 + 1, k0]]
    idx2[k1] = idx2[k1 - 1]
    idx2[k2] = n + 5
    buf = torch.full((n + 64,), 7, dtype=torch.int16, device="cuda")
    buf[:n] = old
    with pytest.raises(sbd.DeltaError, match="delta entries"):
        sbd.apply_(buf[:n].view(torch.bfloat16), idx2, val2.view(torch.bfloat16),
                   check_indices=True)
    want = new.clone()
    want[orig1] = old[orig1]   # its entry now names another position
    want[orig2] = old[orig2]   # its entry is out of range
    dup = int(idx2[k1])
    got_dup = int(buf[dup])
    assert got_dup in (int(val2[k1 - 1]), int(val2[k1]))
    want[dup] = got_dup
    assert torch.equal(buf[:n], want)
    assert bool((buf[n:] == 7).all())


def test_apply_merge_with_broken_precondition_stays_inside(sbd):
    """A chunk dense enough for the line merge but holding unsorted, repeated
    and out-of-range entries: they are counted, only the broken entries'
    positions may differ, every well-formed entry lands, and nothing outside
    the snapshot changes (such a chunk is applied entry by entry)."""
    rng = np.random.default_rng(3)
    n = 40_000
    snap0 = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    idx = np.sort(rng.choice(np.arange(1000, 20_000), size=4096, replace=False)).astype(np.int32)
    idx[100:110] = idx[100:110][::-1]          # unsorted
    idx[500] = idx[499]                        # repeated
    idx[900] = n + 5                           # out of range
    idx[901] = -3                              # negative
    val = rng.integers(0, 1 << 16, size=idx.size, dtype=np.uint32).astype(np.uint16)
    buf = gpu_bits(np.concatenate([snap0, np.full(256, 7, dtype=np.uint16)]))
    snap = buf[:n]
    with pytest.raises(sbd.DeltaError, match="delta entries"):
        sbd.apply_(snap, torch.from_numpy(idx).cuda(),
                   torch.from_numpy(val.view(np.int16)).cuda().view(torch.bfloat16),
                   check_indices=True)
    got = np_bits(buf)
    inr = idx[(idx >= 0) & (idx < n)]
    touched = np.zeros(n, dtype=bool)
    touched[inr] = True
    assert np.array_equal(got[:n][~touched], snap0[~touched])
    for i in np.flatnonzero(touched):  # the entry's value or, if repeated or unsorted, another of its
        assert got[i] == snap0[i] or got[i] in set(val[idx == i].tolist())
    # positions whose only entry is well-formed (sorted neighbourhood) hold its value
    ok = np.ones(idx.size, dtype=bool)
    ok[95:115] = False
    ok[495:505] = False
    ok[900:902] = False
    good = idx[ok]
    assert np.array_equal(got[good], val[ok])
    assert np.all(got[n:] == 7)


@pytest.mark.parametrize("frac", [0.0, 0.03, 0.7])
def test_apply_many_matches_oracle(sbd, oracle_mod, frac):
    olds, news = _param_list(6, MANY_SIZES, frac)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    wants = []
    for p, o in enumerate(olds):
        w = o.copy()
        oracle_mod.apply_(w, ri[ro[p]:ro[p + 1]], rv[ro[p]:ro[p + 1]])
        wants.append(w)
    snaps = [gpu_bits(o) for o in olds]
    sbd.apply_many_(snaps, torch.from_numpy(ri).cuda(),
                    torch.from_numpy(rv.view(np.int16)).cuda().view(torch.bfloat16),
                    torch.from_numpy(ro).cuda(), check_indices=True)
    for s, w in zip(snaps, wants):
        assert np.array_equal(np_bits(s), w)


def test_apply_many_max_nnz_cuts_the_delta(sbd, oracle_mod):
    """Only entries j < min(offsets[nparams], max_nnz) are applied: cut at zero,
    inside the first chunk, inside a parameter, on a parameter boundary, one
    short of the total and past it; the oracle applies the same prefix."""
    olds, news = _param_list(21, MANY_SIZES, 0.3)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    total = int(ro[-1])
    boundary = int(ro[len(olds) // 2])
    gi = torch.from_numpy(ri).cuda()
    gv = torch.from_numpy(rv.view(np.int16)).cuda().view(torch.bfloat16)
    go = torch.from_numpy(ro).cuda()
    for cut in sorted({0, 1, 777, boundary, boundary + 1, total // 2 + 3, total - 1, total,
                       total + 5000}):
        want = []
        for p, o in enumerate(olds):
            w = o.copy()
            a, b = int(ro[p]), min(int(ro[p + 1]), cut)
            if b > a:
                oracle_mod.apply_(w, ri[a:b], rv[a:b])
            want.append(w)
        snaps = [gpu_bits(o) for o in olds]
        sbd.apply_many_(snaps, gi, gv, go, max_nnz=cut, check_indices=True)
        for s, w in zip(snaps, want):
            assert np.array_equal(np_bits(s), w), cut
        # a plan given a prefix of the delta and an unbounded max_nnz applies
        # exactly that prefix (it never reads past the buffers)
        from sparse_bf16_delta_amd.plan import ApplyPlan

        k = min(cut, total)
        snaps = [gpu_bits(o) for o in olds]
        ApplyPlan(snaps).run(gi[:k], gv[:k], go, max_nnz=1 << 40)
        torch.cuda.synchronize()
        for s, w in zip(snaps, want):
            assert np.array_equal(np_bits(s), w), ("plan", cut)


@pytest.mark.parametrize("frac", [0.05, 0.5, 1.0])
def test_apply_many_adjacent_unaligned_params(sbd, oracle_mod, frac):
    """Parameters packed back to back at odd element offsets share 64- and
    128-byte segments at their edges; each must be updated without touching
    its neighbours' bytes."""
    sizes = [37, 1000, 1, 4093, 64, 63, 65, 20_000, 5, 3 * TILE + 11]
    olds, news = _param_list(11 + int(frac * 10), sizes, frac)
    flat_old = np.concatenate(olds)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want = []
    for p, o in enumerate(olds):
        w = o.copy()
        oracle_mod.apply_(w, ri[ro[p]:ro[p + 1]], rv[ro[p]:ro[p + 1]])
        want.append(w)
    buf = gpu_bits(flat_old, 3)
    views, pos = [], 0
    for n in sizes:
        views.append(buf[pos:pos + n])
        pos += n
    sbd.apply_many_(views, torch.from_numpy(ri).cuda(),
                    torch.from_numpy(rv.view(np.int16)).cuda().view(torch.bfloat16),
                    torch.from_numpy(ro).cuda(), check_indices=True)
    assert np.array_equal(np_bits(buf), np.concatenate(want))


@pytest.mark.parametrize("frac", [0.01, 0.3])
def test_many_thousands_of_parameters(sbd, oracle_mod, frac):
    """20,000 parameters, mostly tiny or empty with a few spanning several
    tiles, back to back in one buffer: past the 4096 that one step of the
    parameter search covers.  diff_many and apply_many against the oracle."""
    rng = np.random.default_rng(int(frac * 1000) + 5)
    k = 20_000
    kind = rng.random(k)
    sizes = np.where(kind < 0.05, 0,
                     np.where(kind < 0.80, rng.integers(1, 300, k),
                              np.where(kind < 0.995, rng.integers(300, 5000, k),
                                       rng.integers(TILE, 3 * TILE, k)))).astype(np.int64)
    total = int(sizes.sum())
    old, new = rand_case(int(frac * 100) + 9, total, frac)
    bounds = np.concatenate([[0], np.cumsum(sizes)])
    olds = [old[a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    news = [new[a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    g_old, g_new = gpu_bits(old, 1), gpu_bits(new, 1)
    vo = [g_old[a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    vn = [g_new[a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    gi, gv, gn, go = sbd.diff_many(vo, vn)
    assert np.array_equal(gn.cpu().numpy(), rn)
    assert np.array_equal(go.cpu().numpy(), ro)
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)
    sbd.apply_many_(vo, gi, gv, go, check_indices=True)
    assert np.array_equal(np_bits(g_old), new)


def test_two_streams_at_once(sbd, oracle_mod):
    """Two parameter lists diffed and applied concurrently on two streams:
    each stream has its own cached workspace (and so its own staging arena
    and counters), and both results match the oracle."""
    cases = []
    for seed, frac in ((61, 0.02), (62, 0.15)):
        olds, news = _param_list(seed, MANY_SIZES + [9 * TILE + 5], frac)
        cases.append((olds, news, oracle_mod.diff_many(olds, news)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    out = []
    for (olds, news, _), st in zip(cases, streams):
        g_o = [gpu_bits(o) for o in olds]
        g_n = [gpu_bits(x) for x in news]
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            gi, gv, gn, go = sbd.diff_many(g_o, g_n)
            sbd.apply_many_(g_o, gi, gv, go)
        out.append((gi, gv, gn, go, g_o))
    torch.cuda.synchronize()
    for (olds, news, (ri, rv, rn, ro)), (gi, gv, gn, go, g_o) in zip(cases, out):
        assert np.array_equal(go.cpu().numpy(), ro)
        assert np.array_equal(gi.cpu().numpy(), ri)
        assert np.array_equal(np_bits(gv), rv)
        for s_, x in zip(g_o, news):
            assert np.array_equal(np_bits(s_), x)


def test_two_host_threads(sbd, oracle_mod):
    """Two host threads, each with its own stream (and so its own cached
    workspace), diff and apply their own parameter lists at the same time --
    the library calls run without the GIL -- five rounds each, every round
    against the oracle."""
    import threading

    cases = []
    for seed, frac in ((71, 0.03), (72, 0.2)):
        olds, news = _param_list(seed, MANY_SIZES + [5 * TILE + 9], frac)
        cases.append((olds, news, oracle_mod.diff_many(olds, news)))
    errors = []
    barrier = threading.Barrier(2)

    def worker(k):
        try:
            olds, news, (ri, rv, rn, ro) = cases[k]
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                g_n = [gpu_bits(x) for x in news]
                barrier.wait(timeout=60)
                for r in range(5):
                    g_o = [gpu_bits(o) for o in olds]
                    gi, gv, gn, go = sbd.diff_many(g_o, g_n)
                    sbd.apply_many_(g_o, gi, gv, go)
                    st.synchronize()
                    ok = (np.array_equal(go.cpu().numpy(), ro)
                          and np.array_equal(gi.cpu().numpy(), ri)
                          and np.array_equal(np_bits(gv), rv)
                          and all(np.array_equal(np_bits(s_), x) for s_, x in zip(g_o, news)))
                    if not ok:
                        errors.append((k, r))
                        return
        except Exception as e:  # reported by the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors


def test_diff_many_then_apply_many_without_host_sync(sbd):
    """The receiver can follow the sender on one stream: apply_many reads the
    device offsets written by diff_many; the result equals `new` bitwise."""
    olds, news = _param_list(7, MANY_SIZES, 0.05)
    g_o = [gpu_bits(o) for o in olds]
    g_n = [gpu_bits(x) for x in news]
    gi, gv, gn, go = sbd.diff_many(g_o, g_n)
    sbd.apply_many_(g_o, gi, gv, go)
    for a, b in zip(g_o, g_n):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1023, 4096 * 4 + 5, (1 << 20) + 3])
@pytest.mark.parametrize("pad", [0, 1])
def test_xor_matches_oracle(sbd, oracle_mod, n, pad):
    old, new = rand_case(n + 11, n, 0.05)
    want_mask = oracle_mod.xor_mask(old, new)
    g_o, g_n = gpu_bits(old, pad), gpu_bits(new, pad)
    mask = sbd.xor_mask(g_o, g_n)
    assert np.array_equal(np_bits(mask), want_mask)
    want_snap = old.copy()
    oracle_mod.xor_apply_(want_snap, want_mask)
    sbd.xor_apply_(g_o, mask)
    assert np.array_equal(np_bits(g_o), want_snap)
    sbd.xor_apply_(g_o, mask)
    assert np.array_equal(np_bits(g_o), old)


@pytest.mark.parametrize("frac", [0.0, 0.001, 0.02, 0.3, 1.0])
@pytest.mark.parametrize("n,pad", [(TILE * 3 + 5, 0), (TILE * 3 + 5, 1), (100_003, 3), (15, 0)])
def test_xor_apply_sparse_masks(sbd, oracle_mod, frac, n, pad):
    """xor_apply leaves the snapshot untouched where the mask is zero: masks
    from all-zero to all-nonzero, ragged tails and unaligned views."""
    old, new = rand_case(int(frac * 1e4) + n + pad, n, frac, special=False)
    want_mask = oracle_mod.xor_mask(old, new)
    want = old.copy()
    oracle_mod.xor_apply_(want, want_mask)
    g_snap, g_mask = gpu_bits(old, pad), gpu_bits(want_mask, pad)
    sbd.xor_apply_(g_snap, g_mask)
    assert np.array_equal(np_bits(g_snap), want)
    sbd.xor_apply_(g_snap, g_mask)
    assert np.array_equal(np_bits(g_snap), old)


def test_xor_apply_mask_aliasing_snapshot(sbd):
    """snapshot ^= snapshot clears it, zero and nonzero units alike."""
    old, _ = rand_case(5, 2 * TILE + 9, 0.0, special=False)
    old[: TILE] = 0  # a run of all-zero units
    g = gpu_bits(old)
    sbd.xor_apply_(g, g)
    assert not bool((g.view(torch.int16) != 0).any())


def test_xor_mask_may_alias_new(sbd, oracle_mod):
    old, new = rand_case(77, 3 * TILE + 1, 0.1)
    want = oracle_mod.xor_mask(old, new)
    g_o, g_n = gpu_bits(old), gpu_bits(new)
    sbd.xor_mask(g_o, g_n, out=g_n)
    assert np.array_equal(np_bits(g_n), want)


def test_aliased_inputs(sbd, oracle_mod):
    """old and new may be the very same buffer (an empty delta, also in a
    list), and the mask may overwrite old as well as new."""
    old, new = rand_case(78, 3 * TILE + 5, 0.1)
    g = gpu_bits(old)
    gi, gv = sbd.diff(g, g)
    assert gi.numel() == 0 and gv.numel() == 0
    gi, gv, nnz, offs = sbd.diff_many([g, g[:TILE + 3]], [g, g[:TILE + 3]])
    assert gi.numel() == 0 and int(offs[-1].item()) == 0 and int(nnz.sum().item()) == 0
    want = oracle_mod.xor_mask(old, new)
    g_o, g_n = gpu_bits(old), gpu_bits(new)
    sbd.xor_mask(g_o, g_n, out=g_o)
    assert np.array_equal(np_bits(g_o), want)


def test_c1_single_tensor_roundtrip(sbd, oracle_mod):
    """1024x1024 bf16, fp32-master step at lr 3e-6: diff, apply, XOR round trip."""
    cfg = workloads.CONFIGS["tensor1m"]
    sw, su = workloads.seeds(cfg.seed_family, 0)
    old, new = workloads.make_step_pair(1 << 20, sw, su, 3e-6, "fp32_master", device="cuda")
    o_np, n_np = np_bits(old), np_bits(new)
    ri, rv = oracle_mod.diff(o_np, n_np)
    gi, gv = sbd.diff(old, new)
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(np_bits(gv), rv)
    snap = old.clone()
    sbd.apply_(snap, gi, gv)
    assert torch.equal(snap.view(torch.int16), new.view(torch.int16))
    mask = sbd.xor_mask(old, new)
    assert np.array_equal(np_bits(mask), oracle_mod.xor_mask(o_np, n_np))
    snap2 = old.clone()
    sbd.xor_apply_(snap2, mask)
    assert torch.equal(snap2.view(torch.int16), new.view(torch.int16))
    print(f"1024x1024 tensor: realized density {ri.size / (1 << 20):.4%}")


def test_diff_many_empty_list_through_abi(sbd):
    """nparams == 0: only offsets[0] = 0 is written."""
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    lib = _abi.load()
    offsets = torch.full((4,), -9, dtype=torch.int64, device="cuda")
    ws = torch.empty(lib.delta_workspace_size(0, 0), dtype=torch.uint8, device="cuda")
    _abi.check(lib.delta_diff_many(0, None, None, None, None, None, 0, None, _ptr(offsets),
                                   _ptr(ws), ws.numel(), _stream(offsets.device)))
    assert offsets.cpu().tolist() == [0, -9, -9, -9]
