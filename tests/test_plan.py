"""The launch planner (host logic only; no GPU needed)."""
import json
import os

import numpy as np
import pytest

import sum_reduction_amd as rd
import workloads

CU = 256  # MI355X
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MAX_BLOCKS = 1 << 20


@pytest.fixture(autouse=True)
def _clear_tuning():
    rd.rd_tune_set(None)
    yield
    rd.rd_tune_set(None)


def check_invariants(p, outer, R, inner, cu=CU):
    d = p.as_dict()
    assert 1 <= p.blocks <= MAX_BLOCKS or d["path"] == "none", d
    if d["path"] in ("rows", "rows_short"):
        assert inner == 1
        if d["path"] == "rows":
            assert p.group in (64, 256) and p.split >= 1
            assert p.workspace_bytes == (4 * outer * p.split if p.split > 1 else 0)
            groups = outer * p.split
            assert p.blocks == min(-(-groups // (256 // p.group)), MAX_BLOCKS)
            # pieces of at most 4 rows (512 in all) are combined by the
            # last workgroup of the one launch, others by a second kernel
            one = outer <= 4 and outer * p.split <= 512
            assert d["combine"] == (("last_block" if one else "pass") if p.split > 1
                                    else "none")
            assert p.passes == (2 if p.split > 1 and not one else 1)
        else:
            assert p.passes == 1
    if d["path"] in ("cols", "cols_small"):
        # the slabs tile [0, R) with none empty
        assert p.split * p.rows_per_split >= R
        assert (p.split - 1) * p.rows_per_split < R
        assert p.workspace_bytes == (4 * p.split * outer * inner if p.split > 1 else 0)
        # a few slabs of one-wave tiles, every workgroup resident, are joined
        # by the last slab's workgroups in the one launch, others by a second
        # kernel
        one = False
        if d["path"] == "cols" and p.split > 1:
            tiles = -(-(-(-inner // 4)) // (64 * p.col_waves))
            one = (p.col_waves == 1 and p.row_waves > 1 and p.split <= 16
                   and p.blocks == tiles * outer * p.split <= cu
                   and (p.split - 1) * outer * inner <= 65536)
        assert d["combine"] == (("last_block" if one else "pass") if p.split > 1 else "none"), d
        assert p.passes == (2 if p.split > 1 and not one else 1)
        if d["path"] == "cols":
            assert inner > 128
            assert p.block_threads == 64 * p.col_waves * p.row_waves <= 1024
    if d["path"] == "cols_small":
        assert 2 <= inner <= 128
        blocks = -(-(p.split * outer) // 4)              # a wave per item
        rpw = 64 // -(-inner // 4)
        full_step_of_3 = inner == 3 and p.rows_per_split == rpw * p.unroll
        if p.rows_per_split <= rpw * p.unroll and not full_step_of_3:   # one load step per
            blocks = min(blocks, 64 * cu)                 # item: waves take several in turn
        assert p.blocks == min(blocks, MAX_BLOCKS)


def test_workload_plans():
    plans = {}
    for name, w in workloads.WORKLOADS.items():
        p = (rd.rd_plan_1d(CU, w.numel) if w.full_reduce
             else rd.rd_plan_dim(CU, w.outer, w.R, w.inner))
        check_invariants(p, w.outer, w.R, w.inner)
        plans[name] = p.as_dict()
    # the 1D reduce of 1e9: pieces of 32768 floats (8192 16-byte chunks, two
    # unrolled steps of a 256-lane group), one workgroup and one partial each
    assert plans["normal_1e9"]["path"] == "rows"
    assert plans["normal_1e9"]["split"] == -(-10**9 // 32768) == 30518
    assert plans["normal_1e9"]["blocks"] == 30518
    assert plans["normal_1e9"]["order"] == "blocked"
    assert plans["normal_1e9"]["combine"] == "pass"
    assert plans["normal_1e9"]["passes"] == 2
    # 1e6 floats: 256 pieces of depth 2 combined in the same launch; 1e8:
    # 3052 of depth 16, combined by the second kernel (its partial results
    # in the stream's scratch)
    for name, P, U, c, n in (("harmonic_1e6", 256, 2, "last_block", 1),
                             ("uniform_1e8", 3052, 16, "pass", 2)):
        d = plans[name]
        assert (d["split"], d["unroll"], d["combine"], d["passes"]) == (P, U, c, n), d
    assert all(p["nontemporal"] == 1 for p in plans.values())
    # the [128, 4096, 4095] reduce fills the chip without a split along R:
    # 8 waves side by side cover 512 lane-columns (2048 columns), 2 tiles
    # per outer index, 256 workgroups -- one per CU
    assert plans["cols_128x4096x4095"]["path"] == "cols"
    assert plans["cols_128x4096x4095"]["col_waves"] == 8
    assert plans["cols_128x4096x4095"]["unroll"] == 4
    assert plans["cols_128x4096x4095"]["blocks"] == 256
    assert plans["cols_128x4096x4095"]["split"] == 1
    assert plans["cols_128x4096x4095"]["workspace_bytes"] == 0
    # the row sum: one workgroup per row, written directly
    assert plans["rows_32768x32768"]["path"] == "rows"
    assert plans["rows_32768x32768"]["group"] == 256
    assert plans["rows_32768x32768"]["split"] == 1
    assert plans["rows_32768x32768"]["blocks"] == 32768


def test_row_pieces():
    """Long rows are cut into pieces of about 32768 floats: always when there
    are fewer rows than CUs, otherwise from 1 GB of input on; never below one
    full unrolled step (16 x 16 bytes) per lane -- except that a few rows
    which a step of 2 loads per lane lets give every CU a piece take the
    shallowest depth that does, and fewer rows than CUs of at most 128 MiB
    left at the default depth take 4 loads a step."""
    def P(outer, R):
        return rd.rd_plan_dim(CU, outer, R, 1).split
    assert P(1, 10**6) == 256                # depth 2 (16 would allow only 61)
    assert rd.rd_plan_dim(CU, 1, 10**6, 1).unroll == 2
    assert (P(1, 4 * 10**6), rd.rd_plan_dim(CU, 1, 4 * 10**6, 1).unroll) == (256, 8)
    assert (P(1, 300_000), rd.rd_plan_dim(CU, 1, 300_000, 1).unroll) == (73, 4)
    assert (P(1, 10**7), rd.rd_plan_dim(CU, 1, 10**7, 1).unroll) == (306, 4)
    assert (P(1, 4 * 10**7), rd.rd_plan_dim(CU, 1, 4 * 10**7, 1).unroll) == (1221, 16)
    assert rd.rd_plan_dim(CU, 5, 10**6, 1).unroll == 4       # more rows, under 128 MiB
    assert rd.rd_plan_dim(CU, 16, 4 * 10**6, 1).unroll == 16  # 256 MB: the default depth
    # the softmax denominator: its shallowest built depth, 8 (122 pieces)
    sm = rd.rd_plan_reduce(CU, 1, 10**6, 1, "softmax_denom")
    assert (sm.unroll, sm.split) == (8, 122)
    assert P(1, 10**7) == 306                # ceil(1e7 / 32768) > one per CU
    assert P(1, 10**8) == 3052
    assert P(100, 10**7) == 306
    assert P(1000, 100_000) == 1             # 400 MB, a row per workgroup already
    assert P(300, 10**6) == 31               # 1.2 GB
    assert P(8192, 131072) == 4
    assert P(32768, 32768) == 1              # the problem-91 rows are one piece each
    assert P(256, 1 << 22) == 128
    for outer, R in ((1, 3 * 10**9 // 4), (7, 10**8), (2000, 1 << 20)):
        p = rd.rd_plan_dim(CU, outer, R, 1)
        span = -(-(-(-(R // 4) // p.split)) // 256) * 256   # chunks per piece
        assert span * 4 <= 32768 and span >= 4096, (outer, R, p.split)


def test_softmax_row_pieces_are_twice_as_long():
    for outer, R in ((1, 10**9), (100, 10**7), (8192, 131072), (3, 5000)):
        s = rd.rd_plan_reduce(CU, outer, R, 1, "sum").as_dict()
        for op in ("sumsq", "max", "min"):
            assert rd.rd_plan_reduce(CU, outer, R, 1, op).as_dict() == s
        assert s == rd.rd_plan_dim(CU, outer, R, 1).as_dict()
    assert rd.rd_plan_reduce(CU, 1, 10**9, 1, "softmax_denom").split == -(-10**9 // 65536)
    assert rd.rd_plan_reduce(CU, 100, 10**7, 1, "softmax_denom").split == 153
    assert rd.rd_plan_reduce(CU, 8192, 131072, 1, "softmax_denom").split == 2
    with pytest.raises(ValueError):
        rd.rd_plan_reduce(CU, 1, 10, 1, "mean")


def test_problem47_lane_columns():
    """The trace's count: 4095 = 1023 * 4 + 3, so 1024 lane-columns per row,
    the last holding 3 columns; 128 * 4095 = 524160 outputs."""
    with open(os.path.join(GOLDEN, "problem47_shape_facts.json")) as f:
        facts = json.load(f)
    outer, R, inner = facts["shape"]
    lane_cols = -(-inner // 4)
    assert lane_cols == 1024 and inner - 4 * (lane_cols - 1) == 3
    assert outer * inner == facts["outputs"]
    p = rd.rd_plan_dim(CU, outer, R, inner)
    tiles = -(-lane_cols // (64 * p.col_waves))
    assert p.blocks == tiles * outer * p.split


def test_degenerate_plans():
    assert rd.rd_plan_dim(CU, 0, 5, 5).as_dict()["path"] == "none"
    assert rd.rd_plan_dim(CU, 5, 5, 0).as_dict()["path"] == "none"
    assert rd.rd_plan_dim(CU, 5, 0, 5).as_dict()["path"] == "zero"
    assert rd.rd_plan_1d(CU, 0).as_dict()["path"] == "zero"
    assert rd.rd_plan_1d(CU, 63).as_dict()["path"] == "rows_short"
    assert rd.rd_plan_1d(CU, 64).as_dict()["path"] == "rows"
    assert rd.rd_plan_dim(CU, 3, 9, 2).as_dict()["path"] == "cols_small"
    assert rd.rd_plan_dim(CU, 3, 9, 128).as_dict()["path"] == "cols_small"
    assert rd.rd_plan_dim(CU, 3, 9, 129).as_dict()["path"] == "cols"


def test_random_shapes_keep_invariants():
    rng = np.random.default_rng(0)
    for _ in range(3000):
        outer, R, inner = (int(v) for v in np.exp(rng.uniform(0, 14, 3)).astype(np.int64))
        if outer * R * inner > 2 ** 40:
            continue
        for cu in (1, 32, 80, 256, 304):
            p = rd.rd_plan_dim(cu, outer, R, inner)
            check_invariants(p, outer, R, inner, cu)


def test_column_tile_width():
    """Widest tile that still gives every CU a workgroup."""
    assert rd.rd_plan_dim(CU, 128, 4096, 4095).col_waves == 8
    assert rd.rd_plan_dim(CU, 64, 4096, 4095).col_waves == 4
    assert rd.rd_plan_dim(CU, 1000, 10, 200).col_waves == 1   # 50 lane-columns
    assert rd.rd_plan_dim(CU, 1000, 10, 1000).col_waves == 4  # 250 lane-columns
    p = rd.rd_plan_dim(CU, 256, 4096, 256)                    # 256 one-wave tiles:
    assert p.col_waves == 1 and p.row_waves == 1                # just reach the CUs


@pytest.mark.parametrize("op", ["sum", "sumsq", "max", "min", "softmax_denom"])
def test_column_slabs_of_one_tile(op):
    """Columns too few for one-wave tiles to reach every CU: one tile a block,
    8 waves taking turns on its rows, as many slabs of R as keep the grid
    within one block per CU (a grid just past the CU count pays for a second
    round), every row wave with at least one step of 4 rows per slab."""
    shapes = [(1, 1 << 16, 4095), (1, 4096, 10922), (1, 32768, 32768), (2, 65536, 1024),
              (1, 262144, 512), (4, 8192, 2048), (1, 1000000, 200), (3, 100000, 300),
              (1, 40, 4096), (2, 31, 1000), (1, 4096, 129)]
    for cu in (CU, 80, 304):
        for outer, R, inner in shapes:
            p = rd.rd_plan_reduce(cu, outer, R, inner, op)
            tiles = -(-(-(-inner // 4)) // 64)
            if tiles * outer >= cu:      # (fewer CUs) one-wave tiles reach them all
                assert p.row_waves == 1 and p.blocks >= cu, (outer, R, inner, cu)
                continue
            assert (p.col_waves, p.row_waves, p.unroll) == (1, 8, 4), (outer, R, inner, cu)
            want = max(1, min(cu // (tiles * outer), max(1, R // 32)))
            rps = -(-R // want)
            assert (p.rows_per_split, p.split) == (rps, -(-R // rps)), (outer, R, inner, cu)
            assert p.blocks == tiles * outer * p.split <= cu, (outer, R, inner, cu)
            if op != "softmax_denom":   # (its partial results are pairs)
                check_invariants(p, outer, R, inner, cu)
            # the slabs joined in the one launch, up to 16 of them and 65536
            # published words (the softmax pair: a second kernel)
            one = (op != "softmax_denom" and 1 < p.split <= 16
                   and (p.split - 1) * outer * inner <= 65536)
            assert p.as_dict()["combine"] == ("last_block" if one else
                                              "pass" if p.split > 1 else "none"), (outer, R, inner, cu)
            assert p.passes == (1 if one or p.split == 1 else 2)


def test_column_slab_combine_tuning():
    """combine = 1 keeps the second kernel for slabs the planner would join in
    one launch; 2 is taken only where the single launch is built (one-wave
    tiles with row waves, at most 16 slabs, the grid within the CUs);
    anything else is refused."""
    p = rd.rd_plan_dim(CU, 1, 4096, 10922)
    assert (p.as_dict()["combine"], p.passes, p.split) == ("last_block", 1, 5)
    with rd.tuning(combine=1):
        q = rd.rd_plan_dim(CU, 1, 4096, 10922)
        assert (q.as_dict()["combine"], q.passes) == ("pass", 2)
        assert (q.split, q.blocks, q.workspace_bytes) == (p.split, p.blocks, p.workspace_bytes)
    with rd.tuning(combine=2):
        assert rd.rd_plan_dim(CU, 4, 8192, 2048).as_dict()["combine"] == "last_block"
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 1, 1 << 20, 64)            # cols_small
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 1, 2_000_000, 512)         # 128 slabs of 2 tiles
    with rd.tuning(combine=2, split=4, col_waves=2, row_waves=1, unroll=4):
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 1, 4096, 10922)            # wide tiles
    with rd.tuning(combine=2, split=40, col_waves=1, row_waves=8, unroll=4):
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 1, 4096, 1024)             # more than 16 slabs
    with rd.tuning(combine=3):
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 1, 4096, 10922)
    with rd.tuning(combine=2, split=3):
        assert rd.rd_plan_reduce(CU, 1, 4096, 10922, "max").as_dict()["combine"] == "last_block"
        with pytest.raises(rd.RdError):
            rd.rd_plan_reduce(CU, 1, 4096, 10922, "softmax_denom")


def test_forced_column_path():
    with rd.tuning(path=4):
        assert rd.rd_plan_dim(CU, 3, 9, 64).as_dict()["path"] == "cols"
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 3, 9, 3)          # cols needs inner >= 4
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 3, 9, 1)          # no column path for rows
    with rd.tuning(path=5):
        assert rd.rd_plan_dim(CU, 3, 9, 256).as_dict()["path"] == "cols_small"
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 3, 9, 257)        # at most 64 lane-columns
    with rd.tuning(path=2):
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 3, 9, 64)


def test_small_problems_still_spread():
    """A small outer*inner is split along R so that the grid fills the chip."""
    p = rd.rd_plan_dim(CU, 1, 1 << 20, 64)
    assert p.split > 1 and p.blocks >= CU
    p = rd.rd_plan_dim(CU, 4, 1 << 24, 1)
    assert p.split > 1 and p.blocks >= CU


def test_plan_depends_only_on_cu_count_and_shape():
    a = rd.rd_plan_dim(CU, 7, 100_000, 33).as_dict()
    b = rd.rd_plan_dim(CU, 7, 100_000, 33).as_dict()
    assert a == b


def test_tuning_override():
    with rd.tuning(group=64, unroll=4, split=3):
        p = rd.rd_plan_1d(CU, 1000)
        assert (p.group, p.unroll, p.split) == (64, 4, 3)
    with rd.tuning(col_waves=2, row_waves=2, unroll=16, split=5):
        p = rd.rd_plan_dim(CU, 3, 100, 1000)
        assert (p.col_waves, p.row_waves, p.unroll, p.split) == (2, 2, 16, 5)
    with rd.tuning(col_waves=3, row_waves=3):
        with pytest.raises(rd.RdError):
            rd.rd_plan_dim(CU, 3, 100, 1000)
    with rd.tuning(group=128):
        with pytest.raises(rd.RdError):
            rd.rd_plan_1d(CU, 10000)
    assert rd.rd_tune_supported("rows", 256, 0, 8)
    assert not rd.rd_tune_supported("rows", 256, 0, 6)
    assert rd.rd_tune_supported("cols", 1, 4, 8)
    assert not rd.rd_tune_supported("cols", 8, 4, 8)
    # the other operators have the planner's default shapes
    for op in ("sumsq", "max", "min"):
        assert rd.rd_tune_supported("rows", 256, 0, 16, op)
        assert rd.rd_tune_supported("rows", 64, 0, 8, op)
        assert rd.rd_tune_supported("rows", 256, 0, 2, op)   # small inputs' shapes
        assert rd.rd_tune_supported("rows", 256, 0, 4, op)
        assert not rd.rd_tune_supported("rows", 64, 0, 4, op)
        for cw in (1, 2, 4, 8):
            assert rd.rd_tune_supported("cols", cw, 1, 4, op)
        assert not rd.rd_tune_supported("cols", 1, 4, 8, op)


def test_default_plans_are_built_for_every_operator():
    """Whatever the planner picks by default for an operator is built for it
    (the sum's small-inner slabs may take a depth the others do not have)."""
    rng = np.random.default_rng(1)
    ops = ("sum", "sumsq", "max", "min", "softmax_denom")
    for _ in range(1000):
        outer, R, inner = (int(v) for v in np.exp(rng.uniform(0, 12, 3)).astype(np.int64))
        for op in ops:
            p = rd.rd_plan_reduce(CU, outer, R, inner, op).as_dict()
            if p["path"] == "rows":
                assert rd.rd_tune_supported("rows", p["group"], 0, p["unroll"], op)
            if p["path"] == "cols":
                assert rd.rd_tune_supported("cols", p["col_waves"], p["row_waves"], p["unroll"],
                                            op)
            if p["path"] == "cols_small":
                assert rd.rd_tune_supported("cols_small", 0, 0, p["unroll"], op), (op, p)


def _scan_invariants(p, outer, R, inner, cu=CU):
    d = p.as_dict()
    assert d["path"] == ("scan_rows" if inner == 1 else
                         "scan_cols_small" if inner <= 128 else "scan_cols")
    # the pieces / slabs cover R exactly, none empty
    assert p.split >= 1 and p.rows_per_split >= 1
    assert p.split * p.rows_per_split >= R > (p.split - 1) * p.rows_per_split
    if inner == 1:
        assert p.rows_per_split % 4096 == 0           # whole tiles per piece
        few_long = outer < 4 * cu and R >= 1 << 20 and outer * R >= 1 << 24
        large = R >= 16384 and outer * R * 4 >= (1 << 29 if R % 32768 == 0 else 1 << 30)
        few = 3 * outer < cu and R >= 65536
        L = 32768 if few_long or R % 32768 == 0 else 16384
        if few and not large and outer * R <= 1 << 20:
            L = 16384                                   # small arrays: 8-wave pieces
        look = (few_long or large or few) and -(-R // L) <= (1 << 20) // outer
        assert (p.combine == 3) == look, (outer, R, cu, p.as_dict())
        if look:
            # one launch, a workgroup of 16 waves per 32768 positions (or 8
            # per 16384), the carries by look-back: ticket, chunk totals,
            # group totals
            assert (p.group, p.block_threads, p.rows_per_split, p.passes) == \
                (L // 32, L // 32, L, 1)
            assert p.split == -(-R // L) and p.blocks == outer * p.split
            assert p.workspace_bytes == 256 + 8 * outer * (p.split + -(-p.split // 64))
            return
        # pieces only for fewer rows than a third of the CUs, each of at
        # least 131072 positions (and of more than one tile)
        assert (p.split > 1) == (3 * outer < cu and R >= 131072), (outer, R, cu, p.split)
        # a workgroup per uncut row of more than 16384 -- 16 waves from 65536
        # on, else 8 --; among fewer than 4 rows a CU, 4 waves per uncut row
        # of more than a tile; else a wave per piece (4 to a workgroup)
        if p.split > 1:
            want = 64
        elif R > 16384:
            want = 1024 if R >= 65536 else 512
        else:
            want = 256 if R > 4096 and outer < 4 * cu else 64
        assert p.group == want, (outer, R, cu, p.group)
        if p.group == 64:
            assert p.block_threads == 256
            assert p.blocks == min(-(-outer * p.split // 4), 1 << 20)
        else:
            assert p.block_threads == p.group
            assert p.blocks == min(outer * p.split, 1 << 20)
        ws = 2 * outer * p.split * 4 if p.split > 1 else 0
    elif inner <= 128:
        assert p.unroll in (4, 8)
        assert p.blocks == min(-(-outer * p.split // 4), 1 << 20)   # a wave per slab
        ws = 2 * p.split * outer * inner * 4 if p.split > 1 else 0
    else:
        tiles = -(-(-(-inner // 4) if inner >= 4 else 1) // 64)
        bw, rw = p.col_waves, p.row_waves
        waves = tiles * outer
        assert bw in (1, 2, 4, 8, 16) and p.block_threads == 64 * bw * rw
        assert tiles >= bw
        if 2 * waves >= cu and waves < 2 * cu and inner >= 4:
            # between half and twice as many tiles as CUs: rw waves of a
            # block take turns on one tile's row groups, one pass, the
            # fewest (at most 8) that make 4 waves per CU
            assert p.split == 1 and bw == 1 and rw in (1, 2, 4, 8)
            assert waves * rw >= 4 * cu or rw == 8
            assert rw == 1 or waves * (rw // 2) < 4 * cu
            assert p.unroll in (4, 8) and p.blocks == min(waves, 1 << 20)
        elif 2 * waves < cu and inner >= 4:
            # fewer tiles than half the CUs: slabs, as many as keep the blocks
            # within one per CU, each a round of 8 waves x U rows at least;
            # the scan pass in row rounds of 8 waves a tile (single waves for
            # rows a multiple of 8 KB apart, from 16 KB), totals by the column
            # reduction
            S = max(1, min(cu // waves, max(1, R // 64)))
            rps = -(-R // S)
            assert (p.rows_per_split, p.split) == (rps, -(-R // rps)), p.as_dict()
            lock = inner >= 4096 and inner % 2048 == 0
            assert bw == 1 and rw == (1 if lock else 8), p.as_dict()
            assert p.unroll == (16 if lock and rps >= 1024 else 8), p.as_dict()
            assert p.blocks == waves * p.split <= cu
        else:
            # slabs only when fewer tiles than half the CUs; then the widest
            # block that still gives every CU one
            assert rw == 1
            assert (p.split > 1) == (waves < cu and R >= 128)
            blocks = -(-tiles // bw) * p.split * outer
            assert blocks >= cu or bw == 1
            assert bw == 16 or -(-tiles // (2 * bw)) * p.split * outer < cu or tiles < 2 * bw
            assert p.blocks == min(blocks, 1 << 20)
        ws = 2 * p.split * outer * inner * 4 if p.split > 1 else 0
    assert p.workspace_bytes == ws
    assert p.passes == (3 if p.split > 1 else 1)


def test_cumsum_row_widths_at_their_edges():
    """Uncut rows: a wave per row up to 16384 positions, a workgroup of 8
    waves above, of 16 from 65536 on (two of its 32768-position chunks);
    few long rows take the look-back's 32768-position pieces.  (1024 rows:
    under 1 GB, below the look-back kernel's arrays.)"""
    for R, group in ((4096, 64), (16384, 64), (16385, 512), (32768, 512), (65535, 512),
                     (65536, 1024), (100_000, 1024)):
        p = rd.rd_plan_cumsum(CU, 1024, R, 1)
        assert p.split == 1 and p.group == group, (R, p.as_dict())
        assert p.block_threads == max(group, 256)
    p = rd.rd_plan_cumsum(CU, 16, 1 << 19, 1)   # 16 rows of 2^19: look-back pieces
    assert p.split == 16 and p.group == 1024 and p.passes == 1
    p = rd.rd_plan_cumsum(CU, 16, 1 << 20, 1)   # 16 rows of 2^20: look-back pieces
    assert p.split == 32 and p.group == 1024 and p.passes == 1
    with rd.tuning(unroll=4):                    # 4-slice chunks: 4 waves
        assert rd.rd_plan_cumsum(CU, 4096, 65536, 1).group == 256


def test_cumsum_rows_streamed():
    """order = interleaved on the row scan: persistent workgroups (as many as
    the CUs hold at once), whole rows only, a workgroup per row only."""
    for group, unroll, per_cu in ((256, 8, 4), (512, 8, 2), (1024, 8, 1), (512, 4, 4)):
        with rd.tuning(group=group, unroll=unroll, order=1):
            p = rd.rd_plan_cumsum(CU, 32768, 32768, 1)
            assert (p.group, p.order, p.split) == (group, 1, 1)
            assert p.blocks == CU * per_cu and p.block_threads == group
        with rd.tuning(group=group, unroll=unroll, order=1, split=1):
            assert rd.rd_plan_cumsum(CU, 3, 50_000, 1).blocks == 3  # fewer rows than CUs
        with rd.tuning(group=group, unroll=unroll, order=1):
            with pytest.raises(rd.RdError):  # few long rows are cut into pieces
                rd.rd_plan_cumsum(CU, 3, 150_000, 1)
    with rd.tuning(group=64, order=1):
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum(CU, 32768, 32768, 1)
    with rd.tuning(group=512, order=1, split=2):
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum(CU, 32768, 32768, 1)
    with rd.tuning(group=512, order=2):
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum(CU, 32768, 32768, 1)
    assert rd.rd_plan_cumsum(CU, 32768, 32768, 1).order == 0


def test_cumsum_plans():
    """Rows: a workgroup of 8 waves per row (problem 91: 32768 rows, no pieces,
    two 16384-position chunks a row); few long rows
    are cut into pieces of whole 4096-element tiles, a wave each, other few
    rows take a workgroup each.
    Columns: a wave per 64 lane-columns, slabs of R when there are too few
    waves."""
    p = rd.rd_plan_cumsum(CU, 32768, 32768, 1)   # 4 GB: rows in ticket order
    assert p.as_dict()["path"] == "scan_rows" and p.split == 1 and p.blocks == 32768
    assert p.as_dict()["combine"] == "lookback" and p.rows_per_split == 32768
    assert p.group == 1024 and p.block_threads == 1024 and p.unroll == 8
    assert p.workspace_bytes == 256 + 8 * 32768 * 2
    p = rd.rd_plan_cumsum(CU, 4000, 32768, 1)    # under 512 MiB: a workgroup per row
    assert p.split == 1 and p.group == 512 and p.workspace_bytes == 0
    p = rd.rd_plan_cumsum(CU, 4096, 32768, 1)    # 512 MiB of whole pieces: ticket order
    assert p.as_dict()["combine"] == "lookback" and p.group == 1024
    p = rd.rd_plan_cumsum(CU, 8192, 16384, 1)    # 512 MiB, 16384: the workgroup per row
    assert p.as_dict()["combine"] == "none"
    p = rd.rd_plan_cumsum(CU, 30000, 35791, 1)   # a partial last piece: 8 waves
    assert (p.combine, p.group, p.split, p.rows_per_split) == (3, 512, 3, 16384)
    # few rows (fewer than a third of the CUs) of 65536 positions or more:
    # the look-back, 32768-position pieces of 16 waves (8 waves, 16384, for
    # rows not a multiple of 32768)
    p = rd.rd_plan_cumsum(CU, 1, 1 << 20, 1)                # 4 MB: 8-wave pieces
    assert p.as_dict()["combine"] == "lookback" and (p.split, p.group, p.passes) == (64, 512, 1)
    p = rd.rd_plan_cumsum(CU, 2, 1 << 20, 1)
    assert p.as_dict()["combine"] == "lookback" and (p.split, p.group, p.passes) == (32, 1024, 1)
    p = rd.rd_plan_cumsum(CU, 64, 131072, 1)              # 64 * 3 < 256 CUs
    assert p.as_dict()["combine"] == "lookback" and (p.split, p.blocks) == (4, 256)
    p = rd.rd_plan_cumsum(CU, 7, 777777, 1)
    assert (p.combine, p.group, p.split, p.rows_per_split) == (3, 512, 48, 16384)
    p = rd.rd_plan_cumsum(CU, 64, 65536, 1)
    assert p.as_dict()["combine"] == "lookback" and p.split == 2
    with rd.tuning(combine=1):                            # the three kernels instead
        p = rd.rd_plan_cumsum(CU, 1, 1 << 20, 1)
        assert p.split == 256 and p.rows_per_split == 4096 and p.passes == 3
        p = rd.rd_plan_cumsum(CU, 64, 131072, 1)
        assert p.split == 32 and p.group == 64 and p.passes == 3
        p = rd.rd_plan_cumsum(CU, 1, 1 << 28, 1)
        assert p.split == 4096 and p.passes == 3
        p = rd.rd_plan_cumsum(CU, 64, 65536, 1)           # rows too short to cut
        assert p.split == 1 and p.group == 1024 and p.passes == 1
    p = rd.rd_plan_cumsum(CU, 1, 1 << 28, 1)              # long rows: look-back
    assert p.as_dict()["combine"] == "lookback" and p.split == 8192 and p.blocks == 8192
    assert p.passes == 1 and p.workspace_bytes == 256 + 8 * (8192 + 128)
    p = rd.rd_plan_cumsum(CU, 86, 131072, 1)              # 86 * 3 >= 256: one pass
    assert p.split == 1 and p.group == 1024 and p.blocks == 86 and p.workspace_bytes == 0
    p = rd.rd_plan_cumsum(CU, 1, 32768, 1)                # one chunk: a workgroup
    assert p.split == 1 and p.passes == 1 and p.workspace_bytes == 0
    p = rd.rd_plan_cumsum(CU, 512, 16384, 1)              # few rows of 4 tiles
    assert p.split == 1 and p.group == 256 and p.block_threads == 256 and p.blocks == 512
    p = rd.rd_plan_cumsum(CU, 1024, 16384, 1)             # 4 rows a CU: a wave each
    assert p.split == 1 and p.group == 64 and p.blocks == 256
    p = rd.rd_plan_cumsum(CU, 128, 4096, 4095)
    assert p.as_dict()["path"] == "scan_cols" and p.split == 1
    assert p.col_waves == 8 and p.blocks == 256         # 16 tiles a row: 2 blocks of 8
    p = rd.rd_plan_cumsum(CU, 1, 65536, 4095)            # 16 tiles: 16 slabs in row rounds
    assert (p.split, p.row_waves, p.col_waves, p.unroll, p.blocks) == (16, 8, 1, 8, 256)
    assert p.passes == 3 and p.workspace_bytes == 2 * 16 * 4095 * 4
    for inner in (4096, 8192, 6144):                      # rows a multiple of 8 KB apart
        p = rd.rd_plan_cumsum(CU, 1, 65536, inner)
        assert p.row_waves == 1 and p.col_waves == 1 and p.unroll == 16, (inner, p.as_dict())
        assert p.blocks == -(-inner // 256) * p.split <= CU
    p = rd.rd_plan_cumsum(CU, 1, 65536, 2048)             # 8 KB apart: row rounds
    assert p.row_waves == 8 and p.split == 32
    rng = np.random.default_rng(5)
    for _ in range(3000):
        outer, R, inner = (int(v) for v in rng.integers(1, [3000, 200_000, 5000]))
        if rng.random() < 0.3:
            inner = 1
        if rng.random() < 0.2:
            outer = int(rng.integers(1, 8))
        cu = int(rng.integers(1, 300))
        _scan_invariants(rd.rd_plan_cumsum(cu, outer, R, inner), outer, R, inner, cu)


def test_lookback_workspace_indices_stay_inside():
    """Host-side bounds of the look-back kernel's workspace: piece (o, j)
    publishes chunk total o*P + j, reads those of its group before j, reads
    the group totals o*NG + h for h < j // 64 and, as the last piece of a
    group with a successor, publishes o*NG + j // 64; the ticket takes the
    first 256 bytes.  Every index must fall inside workspace_bytes."""
    rng = np.random.default_rng(17)
    cases = [(1, 1 << 28), (3, 64 * 32768), (2, 64 * 32768 + 1), (1, 4097 * 16384 + 3)]
    cases += [tuple(int(v) for v in rng.integers(1, [600, 1 << 24])) for _ in range(300)]
    for outer, R in cases:
        for group in (512, 1024):
            with rd.tuning(combine=3, group=group):
                p = rd.rd_plan_cumsum(CU, outer, R, 1)
            P, L = p.split, p.rows_per_split
            NG = -(-P // 64)
            assert L == group // 64 * 2048 and (P - 1) * L < R <= P * L
            assert p.blocks == outer * P
            agg_end = 256 + 8 * outer * P            # one past the chunk totals
            last_gsum = 256 + 8 * (outer * P + (outer - 1) * NG + (NG - 1))
            assert p.workspace_bytes == last_gsum + 8
            # the highest group total any piece publishes or reads: the last
            # row's group (P - 2) // 64, and only when P > 64
            if P > 64:
                g_pub = (P - 2) // 64
                assert 256 + 8 * (outer * P + (outer - 1) * NG + g_pub) < p.workspace_bytes
            # the highest chunk total read: row outer - 1, piece P - 2
            if P > 1:
                assert 256 + 8 * ((outer - 1) * P + P - 2) < agg_end


def test_cumsum_forced_split():
    with rd.tuning(split=5):
        p = rd.rd_plan_cumsum(CU, 2, 3 * 4096 + 1, 1)   # 4 tiles: at most 4 pieces
        assert p.split == 4 and p.rows_per_split == 4096
        p = rd.rd_plan_cumsum(CU, 2, 100, 7)
        assert p.split == 5 and p.rows_per_split == 20
        p = rd.rd_plan_cumsum(CU, 2, 3, 7)              # at most R slabs
        assert p.split == 3 and p.rows_per_split == 1


def test_cumsum_small_inner_plans():
    """inner <= 128: a wave per (outer index, slab); a forced path picks
    either column kernel (the small one up to inner = 256)."""
    p = rd.rd_plan_cumsum(CU, 4096, 4096, 4)
    assert p.as_dict()["path"] == "scan_cols_small" and p.split == 1 and p.blocks == 1024
    p = rd.rd_plan_cumsum(CU, 1, 1 << 24, 4)
    assert p.split > 1 and p.passes == 3
    with rd.tuning(path=7):
        assert rd.rd_plan_cumsum(CU, 3, 9, 2).as_dict()["path"] == "scan_cols"
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum(CU, 3, 9, 1)       # rows have one path
    with rd.tuning(path=8):
        assert rd.rd_plan_cumsum(CU, 3, 9, 256).as_dict()["path"] == "scan_cols_small"
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum(CU, 3, 9, 257)
    with rd.tuning(path=4):
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum(CU, 3, 9, 64)      # a reduction path
    with rd.tuning(unroll=16):
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum(CU, 3, 9, 64)      # small scan: 4 or 8


def test_cumsum_degenerate_plans():
    for shape in ((0, 5, 5), (5, 0, 5), (5, 5, 0)):
        assert rd.rd_plan_cumsum(CU, *shape).as_dict()["path"] == "none"
    with pytest.raises(rd.RdError):
        rd.rd_plan_cumsum(0, 1, 1, 1)
    with pytest.raises(rd.RdError):
        rd.rd_plan_cumsum(CU, -1, 1, 1)


def test_cumsum_contiguous_view_plans_like_the_array():
    for outer, R, inner in ((32768, 32768, 1), (128, 4096, 4095), (1, 1 << 20, 1),
                            (4096, 4096, 4), (3, 5, 7), (1, 100, 130), (7, 0, 3)):
        a = rd.rd_plan_cumsum(CU, outer, R, inner).as_dict()
        b = rd.rd_plan_cumsum_strided(CU, outer, R, inner, R * inner, inner, 1).as_dict()
        assert a == b, (outer, R, inner)


def test_cumsum_strided_view_plans():
    """The unit stride decides: inner axis -> column scans (any outer and R
    strides), R with inner == 1 -> row scan (any row stride), none -> a lane
    per output column, split into slabs of >= 32 rows when there are few."""
    # the [4096, 4096] array transposed: [4096, 4096], strides (1, 4096):
    # 64 blocks of 64 columns, cut into 8 slabs of 512 rows
    p = rd.rd_plan_cumsum_strided(CU, 4096, 4096, 1, 1, 4096, 1).as_dict()
    assert p["path"] == "scan_strided" and p["split"] == 8 and p["rows_per_split"] == 512
    assert p["workspace_bytes"] == 2 * 8 * 4096 * 4 and p["passes"] == 3
    assert p["nontemporal"] == 0 and p["blocks"] == 8 * 64
    # [32768, 32768] transposed: 512 blocks, one pass
    for v in ((32768, 32768, 1, 1, 32768, 1), (1, 32768, 32768, 0, 1, 32768)):
        p = rd.rd_plan_cumsum_strided(CU, *v).as_dict()
        assert p["path"] == "scan_strided" and p["split"] == 1 and p["blocks"] == 512
    # columns 0..1023 of [64, 512, 4096]: the column scan with sr = 4096
    p = rd.rd_plan_cumsum_strided(CU, 64, 512, 1024, 512 * 4096, 4096, 1).as_dict()
    assert p["path"] == "scan_cols"
    assert p == rd.rd_plan_cumsum(CU, 64, 512, 1024).as_dict()
    # every other row of a [8192, 8192] array: rows with so = 2*8192
    p = rd.rd_plan_cumsum_strided(CU, 4096, 8192, 1, 2 * 8192, 1, 1).as_dict()
    assert p == rd.rd_plan_cumsum(CU, 4096, 8192, 1).as_dict()
    # the inner axis strided, terms adjacent along R: inputs staged, enough
    # columns for no slabs
    p = rd.rd_plan_cumsum_strided(CU, 512, 100, 1024, 1024 * 100, 1, 100).as_dict()
    assert p["path"] == "scan_strided" and p["split"] == 1 and p["passes"] == 1
    assert p["blocks"] == 512 * 1024 // 64 and p["workspace_bytes"] == 0
    # one strided column (outputs staged): as many slabs as keep 128 rows each
    p = rd.rd_plan_cumsum_strided(CU, 1, 100_000, 1, 0, 7, 1).as_dict()
    assert p["path"] == "scan_strided" and p["rows_per_split"] == 196 and p["split"] == 511
    # neither side contiguous: a lane per column, slabs of at least 32 rows
    p = rd.rd_plan_cumsum_strided(CU, 100, 1000, 3, 7000, 7, 2).as_dict()
    assert p["path"] == "scan_strided" and p["rows_per_split"] >= 32 and p["split"] > 1
    assert p["blocks"] == p["split"] * -(-300 // 256)
    # length-1 axes: their strides are ignored
    assert rd.rd_plan_cumsum_strided(CU, 1, 9, 4, 12345, 4, 1).as_dict()["path"] == \
        "scan_cols_small"
    assert rd.rd_plan_cumsum_strided(CU, 9, 1, 1, 5, 3, 77).as_dict()["path"] == "scan_rows"
    rng = np.random.default_rng(9)
    for _ in range(2000):
        outer, R, inner = (int(v) for v in rng.integers(1, [500, 50_000, 600]))
        so, sr, si = (int(v) for v in rng.integers(0, [10**6, 5000, 40]))
        cu = int(rng.integers(1, 300))
        p = rd.rd_plan_cumsum_strided(cu, outer, R, inner, so, sr, si)
        d = p.as_dict()
        assert p.split * p.rows_per_split >= R > (p.split - 1) * p.rows_per_split
        unit_rows = inner == 1 and (sr == 1 or R == 1)
        unit_cols = inner > 1 and si == 1
        if not (unit_rows or unit_cols):
            assert d["path"] == "scan_strided"
            n = outer * inner
            staged = inner == 1 or sr == 1 or R == 1
            groups = -(-n // 64)
            if not staged and 2 * groups >= cu and n < cu * 1024:
                # one pass in row rounds: the fewest of 2, 4, 8 waves a group
                # of 64 columns that make 4 waves per CU
                rw = p.row_waves
                assert rw in (2, 4, 8) and p.split == 1 and p.passes == 1, d
                assert groups * rw >= 4 * cu or rw == 8
                assert rw == 2 or groups * (rw // 2) < 4 * cu
                assert p.blocks == min(groups, 1 << 20) and p.block_threads == 64 * rw
                assert p.workspace_bytes == 0
                continue
            assert p.row_waves == 0, d
            cols = 64 if staged else 256
            assert p.blocks == min(p.split * -(-n // cols), 1 << 20)
            assert p.split == 1 or p.rows_per_split >= (128 if staged else 32)
            if staged and -(-n // 64) >= 2 * cu:
                assert p.split == 1   # enough blocks: one pass, x read once
            assert p.workspace_bytes == (2 * p.split * outer * inner * 4 if p.split > 1 else 0)
        else:
            assert d == rd.rd_plan_cumsum(cu, outer, R, inner).as_dict()


def test_cumsum_strided_forced_path():
    """path = RD_PATH_SCAN_STRIDED is valid for every view (with split);
    a row or column path is refused where its unit stride is missing."""
    with rd.tuning(path=10):
        p = rd.rd_plan_cumsum_strided(CU, 3, 100, 5, 500, 5, 1).as_dict()
        assert p["path"] == "scan_strided"
        assert rd.rd_plan_cumsum(CU, 32768, 32768, 1).as_dict()["path"] == "scan_strided"
    with rd.tuning(path=10, split=3):
        p = rd.rd_plan_cumsum_strided(CU, 3, 100, 5, 500, 5, 1)
        assert p.split == 3 and p.rows_per_split == 34 and p.passes == 3
    with rd.tuning(path=10, unroll=4):
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum_strided(CU, 3, 100, 5, 500, 5, 1)
    with rd.tuning(path=6):
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum_strided(CU, 3, 100, 1, 1, 3, 1)   # rows, R strided
    with rd.tuning(path=7):
        with pytest.raises(rd.RdError):
            rd.rd_plan_cumsum_strided(CU, 3, 100, 5, 500, 1, 100)  # inner strided
    with pytest.raises(rd.RdError):
        rd.rd_plan_cumsum_strided(CU, 2, 2, 2, -1, 2, 1)


# ------------------------------------------------------------ strided views
def test_strided_contiguous_view_plans_like_the_array():
    for outer, R, inner in ((1, 10**9, 1), (128, 4096, 4095), (32768, 32768, 1), (3, 5, 7),
                            (4096, 4096, 4), (1, 100, 130), (7, 0, 3), (0, 4, 4)):
        a = rd.rd_plan_dim(CU, outer, R, inner).as_dict()
        b = rd.rd_plan_strided(CU, outer, R, inner, R * inner, inner, 1).as_dict()
        assert a == b, (outer, R, inner)


def test_strided_path_follows_the_unit_stride():
    P = lambda *v: rd.rd_plan_strided(CU, *v).as_dict()
    # reducing dim 1 of a transposed [N, M] array: outputs adjacent (so = 1),
    # terms M apart -> read as the columns of [1, R, outer]
    p = P(4096, 1000, 1, 1, 4096, 0)
    q = rd.rd_plan_dim(CU, 1, 1000, 4096).as_dict()
    assert p == q
    # reducing dim 0 of a transposed array: each output's terms contiguous
    # (sr = 1), outputs M apart -> rows
    p = P(1, 4096, 1000, 0, 1, 4096)
    assert p["path"] == "rows" and p == rd.rd_plan_dim(CU, 1000, 4096, 1).as_dict()
    # a row slice of a wider array: rows with a stride
    assert P(500, 98, 1, 300, 1, 1)["path"] == "rows_short" or P(500, 98, 1, 300, 1, 1)["path"] == "rows"
    # columns of an inner slice: the column kernels with a row stride
    assert P(8, 64, 4, 64 * 100, 100, 1)["path"] == "cols_small"
    assert P(2, 64, 1000, 10**6, 3000, 1)["path"] == "cols"
    # broadcast rows (stride 0) still have a unit stride
    assert P(1, 50, 300, 0, 0, 1)["path"] == "cols_small" or P(1, 50, 300, 0, 0, 1)["path"] == "cols"
    # no unit stride, terms more than 32 floats apart along the kept inner
    # axis (or a narrow span): the lane-per-output kernel
    p = P(3, 100, 50, 10**5, 700, 33)
    # 150 outputs: split along R into slabs of at least 32 rows (here 3)
    assert p["path"] == "strided" and p["split"] == 3 and p["rows_per_split"] == 34
    assert p["passes"] == 2 and p["workspace_bytes"] == 4 * 3 * 150
    assert p["blocks"] == -(-450 // 256)
    assert P(3, 100, 40, 10**5, 700, 3)["path"] == "strided"   # span 118 floats
    # many outputs: one slab, one pass
    p = P(300, 64, 1000, 10**6, 3000, 40)
    assert p["path"] == "strided" and p["split"] == 1 and p["passes"] == 1
    assert p["workspace_bytes"] == 0 and p["blocks"] == -(-300000 // 256)
    # the kept inner axis 2..32 floats apart, a span wider than 128 floats:
    # the column kernel over the dense span of each row, planned as the
    # columns of that span, with workspaces sized by the outputs
    p = P(1, 4096, 10923, 0, 262144, 3)          # x[::8, ::3] of [32768, 32768]
    q = rd.rd_plan_dim(CU, 1, 4096, 32767).as_dict()
    assert p["path"] == "cols" and p["split"] == q["split"] and p["blocks"] == q["blocks"]
    assert p["workspace_bytes"] == q["split"] * 10923 * 4 * (q["split"] > 1)
    p = P(3, 100, 50, 10**5, 700, 3)             # span 148 floats
    assert p["path"] == "cols" and p["col_waves"] == rd.rd_plan_dim(CU, 3, 100, 148).col_waves
    p = P(300, 64, 1000, 10**6, 32000, 32)
    assert p["path"] == "cols" and p["split"] == 1 and p["workspace_bytes"] == 0
    # length-1 axes lose their strides
    assert P(1, 1000, 1, 999, 1, 77) == rd.rd_plan_dim(CU, 1, 1000, 1).as_dict()
    assert P(5, 1, 6, 6, 12345, 1) == rd.rd_plan_dim(CU, 5, 1, 6).as_dict()


def test_strided_invalid_views():
    for v in ((-1, 2, 2, 4, 2, 1), (2, 2, 2, -4, 2, 1), (2, 2, 2, 4, -2, 1), (2, 2, 2, 4, 2, -1),
              (2, 2, 2, 2 ** 62, 1, 1), (2, 2 ** 40, 2, 0, 2 ** 30, 1)):
        with pytest.raises(rd.RdError):
            rd.rd_plan_strided(CU, *v)
    with rd.tuning(path=4):   # a column kernel cannot read a view without a unit stride
        with pytest.raises(rd.RdError):
            rd.rd_plan_strided(CU, 3, 100, 50, 10**5, 700, 33)
    with rd.tuning(path=5):   # nor the small-inner one a dense span
        with pytest.raises(rd.RdError):
            rd.rd_plan_strided(CU, 3, 100, 50, 10**5, 700, 3)


def test_view3_collapses_torch_layouts():
    import torch
    x = torch.empty(6, 7, 8, 9)
    cases = {
        (x, 1): (6, 7, 72, 504, 72, 1),
        (x.transpose(0, 1), 1): (7, 6, 72, 72, 504, 1),
        (x[:, :, 2:5, :], 1): (6, 7, 27, 504, 72, 1),   # rows 2..4 of each 8x9 block are adjacent
        (x[:, :, :, 2:5], 1): (6, 7, None, None, None, None),   # 8 runs of 3, 9 apart: no collapse
        (x[1:4], 2): (21, 8, 9, 72, 9, 1),
        (x[:, 1:4], 2): (6, 8, None, None, None, None),   # outer strides 504 and 72: no collapse
        (x.permute(3, 0, 1, 2), 0): (1, 9, 336, 0, 1, 9),
        (x.expand(2, 6, 7, 8, 9), 1): (2, 6, 504, 0, 504, 1),
    }
    for (t, d), want in cases.items():
        got = rd._view3(t, d)
        if want[2] is None:
            assert got is None, (t.shape, t.stride(), d)
        else:
            assert got == want, (t.shape, t.stride(), d, got)


def _workspace_extent(outer, R, inner, p):
    """Host-side index arithmetic of a split reduce: the largest float index
    the first kernel writes and the second one reads in the workspace, as
    the kernels compute them (rows: piece results at row * P + piece;
    columns: slab results at (s * outer + o) * inner + column), against the
    workspace's size in floats."""
    d = p.as_dict()
    if d["path"] == "rows":
        written = outer * p.split - 1                  # dst[seg], seg < outer * P
        read = (outer - 1) * p.split + p.split - 1      # combine_row: part[o * P + k], k < P
    else:
        # pass 1: the last slab (its first row r0 = s * rps < R), last outer
        # index, last column; pass 2 (slab_combine): slab[s * n + e]
        s_last = p.split - 1
        assert s_last * p.rows_per_split < R
        written = (s_last * outer + outer - 1) * inner + inner - 1
        read = s_last * (outer * inner) + outer * inner - 1
    return written, read, p.workspace_bytes // 4


def test_split_workspace_indices_stay_inside():
    """Every index the two kernels of a split plan touch lies inside its
    workspace -- among them the [3, 50000, 70] axis reduce (341 slabs of
    147 rows, 286,440 bytes: highest index 71,609 of 71,610 floats), whose
    graph-captured workspace once faulted on replay; the same arithmetic
    holds for every default split plan of a sweep of shapes."""
    p = rd.rd_plan_dim(CU, 3, 50_000, 70)
    assert p.as_dict()["path"] == "cols_small"
    assert (p.split, p.rows_per_split, p.workspace_bytes) == (341, 147, 286_440)
    assert _workspace_extent(3, 50_000, 70, p) == (71_609, 71_609, 71_610)
    rng = np.random.default_rng(77)
    checked = 0
    for _ in range(4000):
        outer, R, inner = (int(v) for v in np.exp(rng.uniform(0, 11, 3)).astype(np.int64))
        p = rd.rd_plan_dim(CU, outer, R, inner)
        if p.split == 1 or p.as_dict()["path"] not in ("rows", "cols", "cols_small"):
            continue
        if p.as_dict()["path"] == "rows" and inner != 1:
            continue
        written, read, floats = _workspace_extent(outer, R, inner, p)
        assert written < floats and read < floats, (outer, R, inner, p.as_dict())
        checked += 1
    assert checked > 100
