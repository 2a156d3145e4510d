"""CPU-side checks of the C-ABI library: it loads, exports what include/pa.h declares,
and its host functions (planner, validators, status strings, argument checks) behave.
No kernel is launched here."""
import ctypes

import numpy as np
import pytest

import paged_kv_attention_04_amd as pa
import synthetic


@pytest.fixture(scope="module")
def lib():
    return pa.lib()


def qwen(num_blocks=5461):
    return pa.Geometry.make(32, 8, num_blocks)


def test_exports_every_declared_symbol(lib):
    names = pa.header_functions()
    assert set(names) >= {"pa_plan", "pa_append_kv", "pa_attention_batch", "pa_validate_batch",
                          "pa_validate_append", "pa_query_num_cus", "pa_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_struct_sizes_match_header(lib):
    # int32 x 11 + 128 + 129, then 2 + 3 x 16 int32 of the prefix groups, then a uint64 at
    # an 8-byte boundary; the library reports the size its own compiler gives the struct
    assert ctypes.sizeof(pa.Geometry) == 24
    assert ctypes.sizeof(pa.Plan) == 8 * ((4 * (11 + 128 + 129 + 2 + 3 * 16 + 3) + 7) // 8) + 8
    lib.pa_plan_struct_bytes.restype = ctypes.c_size_t
    assert lib.pa_plan_struct_bytes() == ctypes.sizeof(pa.Plan)


def test_status_strings(lib):
    for code in pa.STATUS:
        assert lib.pa_status_string(code)
    assert lib.pa_status_string(12345) == b"unknown status"


def _split_ranges(plan, kv):
    nb = -(-int(kv) // 16)
    s = plan.split_blocks
    return [(b, min(nb, b + s)) for b in range(0, nb, s)]


@pytest.mark.parametrize("wl_fn", [synthetic.config_tiny, synthetic.config_decode, synthetic.config_mixed])
def test_plan_splits_tile_each_row_once(wl_fn):
    wl = wl_fn(poison=False) if wl_fn is not synthetic.config_tiny else wl_fn()
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256)
    assert plan.num_reqs == wl.num_reqs and plan.total_q == wl.total_q
    items = 0
    for r in range(wl.num_reqs):
        if wl.qo_len[r] != 1:
            continue
        ranges = _split_ranges(plan, wl.kv_len[r])
        covered = [b for lo, hi in ranges for b in range(lo, hi)]
        assert covered == list(range(-(-int(wl.kv_len[r]) // 16)))     # contiguous, once, block aligned
        assert all(hi > lo for lo, hi in ranges)                          # no empty split
        assert len(ranges) <= plan.max_splits
        items += len(ranges) * wl.num_kv_heads
    assert items == plan.decode_items
    assert 1 <= plan.split_blocks <= 512


def test_plan_is_pure_and_fills_cus():
    wl = synthetic.config_decode(poison=False)
    g = qwen()
    a = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256)
    b = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256)
    assert bytes(a) == bytes(b)
    assert a.decode_items >= 256                                        # a workgroup per CU
    assert a.max_splits == 1                                            # 32 x 8 pairs fill the CUs unsplit
    # fewer (row, KV head) pairs than CUs: rows are split over kv_len
    sp = synthetic.config_shared_prefix(poison=False)
    b = pa.pa_plan(g, sp.qo_len, sp.kv_len, 256)
    assert b.max_splits == 2 and b.decode_items == 256
    # batch 1 at 2K: splits stay >= 8 blocks but still spread over many CUs
    one = pa.pa_plan(g, [1], [2049], 256)
    assert one.split_blocks >= 8 and one.decode_items >= 8 * 16


def test_plan_prefill_rows_and_workspace():
    g = qwen()
    qo = [512] + [1] * 31
    kv = [4608] + [2048 + i for i in range(31)]
    plan = pa.pa_plan(g, qo, kv, 256)
    assert plan.num_prefill_rows == 1 and plan.num_decode_rows == 31
    assert plan.prefill_req[0] == 0 and plan.prefill_tiles == 512 // 32
    assert plan.prefill_tile_start[1] == 16
    # 16 tiles x 8 KV heads leave half the CUs idle: each tile's 36 key steps are split in two
    assert plan.prefill_splits == 2
    n_pf = 16 * 8 * 2
    need = n_pf * 128 * 129 * 4
    if plan.max_splits > 1:
        need += 32 * plan.max_splits * 32 * 129 * 4
    assert plan.workspace_bytes >= need
    # forced split of 1 block and one large split
    p1 = pa.pa_plan(g, qo, kv, 256, split_blocks=1)
    assert p1.split_blocks == 1 and p1.max_splits == -(-2078 // 16)
    p512 = pa.pa_plan(g, [1], [100], 256, split_blocks=1000)
    assert p512.split_blocks == 512 and p512.max_splits == 1 and p512.workspace_bytes == 0
    # rows longer than 512 blocks are always split
    long = pa.pa_plan(g, [1] * 64, [20000] * 64, 256)
    assert long.split_blocks <= 512 and long.max_splits == 3 and long.split_blocks * 3 >= 1250


def test_plan_prefill_splits():
    g = qwen()
    # enough tiles to fill the CUs: no split and no workspace
    big = pa.pa_plan(g, [2048] * 4, [2048] * 4, 256)
    assert big.prefill_tiles == 4 * 64 and big.prefill_splits == 1 and big.workspace_bytes == 0
    # short keys are never split below 4 steps per workgroup
    short = pa.pa_plan(g, [64], [300], 256)
    assert short.prefill_tiles == 2 and short.prefill_splits == 1
    # one long chunk: split over many workgroups
    one = pa.pa_plan(g, [256], [32768], 256)
    assert one.prefill_tiles == 8 and one.prefill_splits > 1
    assert 64 * one.prefill_splits <= 256 * 2
    # forced counts, including more splits than steps
    for s in (1, 3, 64):
        f = pa.pa_plan(g, [40], [100], 256, prefill_splits=s)
        assert f.prefill_splits == s and (f.workspace_bytes > 0) == (s > 1)
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(g, [40], [100], 256, prefill_splits=65)
    assert e.value.code == -2
    # decode-only batches carry no prefill split
    assert pa.pa_plan(g, [1] * 8, [100] * 8, 256).prefill_splits == 0


def _shared_tables(n_rows, shared, private, max_blocks, seed=0, split_at=None):
    """Block tables where every row starts with the same `shared` blocks (rows from
    split_at on use a different shared run) followed by private blocks."""
    rng = np.random.default_rng(seed)
    ids = rng.permutation(100000).astype(np.int32)
    bt = np.full((n_rows, max_blocks), -1, np.int32)
    nxt = 2 * shared
    for r in range(n_rows):
        base = 0 if split_at is None or r < split_at else shared
        bt[r, :shared] = ids[base:base + shared]
        bt[r, shared:shared + private[r]] = ids[nxt:nxt + private[r]]
        nxt += private[r]
    return bt


def test_plan_shared_prefix_groups():
    g = qwen(num_blocks=100000)
    sp = synthetic.config_shared_prefix(poison=False)
    plan = pa.pa_plan(g, sp.qo_len, sp.kv_len, 256)
    before = bytes(plan)
    pa.pa_plan_shared_prefix(g, plan, sp.qo_len, sp.kv_len, sp.block_tables, 256)
    assert plan.num_prefix_groups == 1
    assert (plan.prefix_first_req[0], plan.prefix_num_reqs[0], plan.prefix_blocks[0]) == (0, 16, 384)
    assert 1 <= plan.prefix_splits <= 64 and plan.prefix_splits * 2 <= 384 // 8
    # decode splits now cover only the private suffixes (2048 + U[0,255] tokens)
    assert plan.split_blocks * plan.max_splits >= -(-(int(sp.kv_len.max()) - 6144) // 16)
    assert plan.split_blocks < 263
    n = 16 * plan.prefix_splits * 32
    assert plan.workspace_bytes >= n * 129 * 4
    assert bytes(plan) != before
    # no shared run: the plan is left as it was
    dec = synthetic.config_decode(poison=False)
    p2 = pa.pa_plan(g, dec.qo_len, dec.kv_len, 256)
    b2 = bytes(p2)
    pa.pa_plan_shared_prefix(g, p2, dec.qo_len, dec.kv_len, dec.block_tables, 256)
    assert bytes(p2) == b2 and p2.num_prefix_groups == 0
    # a run shorter than the minimum is not a group
    p3 = pa.pa_plan(g, sp.qo_len, sp.kv_len, 256)
    pa.pa_plan_shared_prefix(g, p3, sp.qo_len, sp.kv_len, sp.block_tables, 256, min_shared_blocks=385)
    assert p3.num_prefix_groups == 0


def test_plan_shared_prefix_runs_and_limits():
    g = qwen(num_blocks=100000)
    # 40 rows sharing 20 blocks: cut into groups of at most 32 requests
    qo = [1] * 40
    priv = [3 + (r % 5) for r in range(40)]
    kv = [16 * (20 + priv[r]) - r % 7 for r in range(40)]
    bt = _shared_tables(40, 20, priv, 32)
    plan = pa.pa_plan(g, qo, kv, 256)
    pa.pa_plan_shared_prefix(g, plan, qo, kv, bt, 256)
    assert plan.num_prefix_groups == 2
    assert [plan.prefix_num_reqs[i] for i in range(2)] == [32, 8]
    assert [plan.prefix_blocks[i] for i in range(2)] == [20, 20]
    # a prefill row breaks a run; two different shared runs make two groups
    qo = [1, 1, 1, 9, 1, 1, 1, 1]
    priv = [4] * 8
    kv = [16 * 24] * 8
    bt = _shared_tables(8, 20, priv, 32, split_at=5)
    plan = pa.pa_plan(g, qo, kv, 256)
    pa.pa_plan_shared_prefix(g, plan, qo, kv, bt, 256)
    groups = [(plan.prefix_first_req[i], plan.prefix_num_reqs[i]) for i in range(plan.num_prefix_groups)]
    assert groups == [(0, 3), (5, 3)]
    # a row whose kv_len ends inside the shared run shares only whole blocks before its last
    qo = [1, 1]
    kv = [16 * 24, 16 * 18 + 1]
    bt = _shared_tables(2, 20, [4, 0], 32)
    plan = pa.pa_plan(g, qo, kv, 256)
    pa.pa_plan_shared_prefix(g, plan, qo, kv, bt, 256)
    assert plan.num_prefix_groups == 1 and plan.prefix_blocks[0] == 18
    # lengths whose total differs from the plan's are rejected and leave the plan alone
    before = bytes(plan)
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan_shared_prefix(g, plan, [1, 2], [16 * 24, 16 * 19], bt, 256)
    assert e.value.code == -2 and bytes(plan) == before


def test_plan_shared_prefix_fused_launch_choices():
    """On a bf16 pool the prefix key splits are one of 4, 6, 8, 12, 16 (clamped to the
    prefix's 128-key steps) and the decode split length one of the even cuts of the longest
    suffix into 1 .. 8 parts, the pair chosen by one simulated makespan.  Pinned choices,
    with their HIP-event times on MI355X from a grid of forced plans on the same kernels:
    16 requests at 8192 + U sharing 6144 tokens -> (6 splits, 48 blocks), 40.8 us (the
    grid's best 38.0 us); the 36-layer sweep's batch 8 (4 of the rows share the prefix) ->
    (16, 65), 26.8 us (best 25.5 us); batch 32 -> (16, 129), 58.5 us, the grid's best.  The
    workspace holds a decode partial for every group row (its result waits there for the
    prefix partials) and the prefix partials."""
    g = qwen(num_blocks=100000)
    sp = synthetic.config_shared_prefix(poison=False)
    plan = pa.pa_plan(g, sp.qo_len, sp.kv_len, 256)
    pa.pa_plan_shared_prefix(g, plan, sp.qo_len, sp.kv_len, sp.block_tables, 256)
    assert plan.prefix_splits == 6 and plan.split_blocks == 48 and plan.max_splits == 3
    longest = max(-(-int(L) // 16) - 384 for L in sp.kv_len)
    assert plan.split_blocks in {-(-longest // k) for k in range(1, 9)}
    R, S, Hq = 16, plan.max_splits, 32
    need = 65536 + R * S * Hq * 128 * 4 + R * S * Hq * 4 + R * plan.prefix_splits * Hq * 129 * 4
    assert plan.workspace_bytes >= need
    again = pa.pa_plan(g, sp.qo_len, sp.kv_len, 256)
    pa.pa_plan_shared_prefix(g, again, sp.qo_len, sp.kv_len, sp.block_tables, 256)
    assert bytes(again) == bytes(plan)                 # a pure function of its inputs
    # the same batch on a q8_0 pool, under the q8_0 costs (its 128-row prefix tile makes
    # a prefix workgroup dearer): unsplit decode rows and 16 prefix splits, 38.5 us in
    # the q8_0 grid (its best 37.3 us; the earlier choice (12, 48) 42.6 us)
    q8 = pa.pa_plan(g, sp.qo_len, sp.kv_len, 256)
    pa.pa_plan_shared_prefix(g, q8, sp.qo_len, sp.kv_len, sp.block_tables, 256, q8=True)
    assert (q8.prefix_splits, q8.split_blocks) == (16, 142)
    for batch, want in ((8, (16, 65)), (32, (16, 129))):
        wl = synthetic.config_sweep_decode(batch, 0, poison=False, fill_pools=False)
        gs = pa.Geometry.make(32, 8, wl.num_blocks)
        p = pa.pa_plan(gs, wl.qo_len, wl.kv_len, 256)
        pa.pa_plan_shared_prefix(gs, p, wl.qo_len, wl.kv_len, wl.block_tables, 256)
        assert (p.prefix_splits, p.split_blocks) == want, batch
    for shared in (20, 100, 200):
        qo = [1] * 6
        kv = [16 * (shared + 30) + r for r in range(6)]
        bt = _shared_tables(6, shared, [31] * 6, shared + 40)
        p2 = pa.pa_plan(g, qo, kv, 256)
        pa.pa_plan_shared_prefix(g, p2, qo, kv, bt, 256)
        steps = -(-shared * 16 // 128)
        assert p2.num_prefix_groups == 1 and p2.prefix_splits in {min(c, steps) for c in (4, 6, 8, 12, 16)}


def test_plan_shared_prefix_overrides():
    """Forced prefix split counts and split lengths are used as given (the split length
    clamped to 512 blocks); out-of-range values are PA_ERR_SHAPE and leave the plan as
    it was."""
    g = qwen(num_blocks=100000)
    sp = synthetic.config_shared_prefix(poison=False)
    for ps, sb in ((3, 0), (0, 36), (24, 18), (1, 1000)):
        plan = pa.pa_plan(g, sp.qo_len, sp.kv_len, 256)
        pa.pa_plan_shared_prefix(g, plan, sp.qo_len, sp.kv_len, sp.block_tables, 256, prefix_splits=ps,
                                 split_blocks=sb)
        if ps:
            assert plan.prefix_splits == ps
        if sb:
            assert plan.split_blocks == min(sb, 512)
            longest = max(-(-int(L) // 16) - 384 for L in sp.kv_len)
            assert plan.max_splits == -(-longest // plan.split_blocks)
    for ps, sb in ((-1, 0), (65, 0), (0, -3)):
        plan = pa.pa_plan(g, sp.qo_len, sp.kv_len, 256)
        before = bytes(plan)
        with pytest.raises(pa.PaError) as e:
            pa.pa_plan_shared_prefix(g, plan, sp.qo_len, sp.kv_len, sp.block_tables, 256, prefix_splits=ps,
                                     split_blocks=sb)
        assert e.value.code == -2 and bytes(plan) == before


@pytest.mark.parametrize("hq,hkv", [(32, 32), (32, 16), (24, 8), (48, 8), (64, 8), (8, 1)])
def test_plan_counts_virtual_kv_heads(hq, hkv):
    """Grouped-query ratios other than four: a KV head with G query heads is served by
    ceil(G / 4) workgroups of four head slots, so the decode workgroup count and the
    partials scale with that count of virtual KV heads, not with num_kv_heads."""
    vheads = hkv * -(-(hq // hkv) // 4)
    g = pa.Geometry.make(hq, hkv, 4096)
    kv = [700, 33, 1, 2048]
    plan = pa.pa_plan(g, [1] * 4, kv, split_blocks=8)
    splits = [-(-(-(-k // 16)) // 8) for k in kv]
    assert plan.max_splits == max(splits)
    assert plan.decode_items == sum(splits) * vheads
    # decode partials hold four head slots per virtual KV head: o and lse per (row, split, slot)
    n = 4 * plan.max_splits * vheads * 4
    assert plan.workspace_bytes >= 64 * 1024 + n * 128 * 4 + n * 4


def test_plan_errors():
    g = qwen()
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(g, [2], [1])
    assert e.value.code == -2
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(g, [0], [5])
    assert e.value.code == -2
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(pa.Geometry.make(32, 12, 10), [1], [5])              # KV heads do not divide query heads
    assert e.value.code == -5
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(pa.Geometry.make(32, 8, 10, head_dim=64), [1], [5])
    assert e.value.code == -5
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(g, [2] * 129, [2] * 129)                              # too many prefill rows
    assert e.value.code == -5
    empty = pa.pa_plan(g, [], [])
    assert empty.num_reqs == 0 and empty.workspace_bytes == 0


def test_validate_batch():
    wl = synthetic.config_tiny()
    g = pa.Geometry.make(8, 2, 64)
    assert pa.pa_validate_batch(g, wl.qo_len, wl.kv_len, wl.block_tables) == (0, -1)
    bt = wl.block_tables.copy()
    bt[2, 3] = 64                                                        # past the pool
    assert pa.pa_validate_batch(g, wl.qo_len, wl.kv_len, bt) == (-3, 2)
    bt = wl.block_tables.copy()
    bt[1, 0] = -1
    assert pa.pa_validate_batch(g, wl.qo_len, wl.kv_len, bt) == (-3, 1)
    # entries past ceil(kv_len/16) are not read, so -1 there is fine
    assert wl.block_tables[0, 5] == -1
    kv = wl.kv_len.copy()
    kv[3] = 0
    assert pa.pa_validate_batch(g, wl.qo_len, kv, wl.block_tables) == (-2, 3)
    kv = wl.kv_len.copy()
    kv[0] = 16 * wl.block_tables.shape[1] + 1                            # more blocks than the table has
    assert pa.pa_validate_batch(g, wl.qo_len, kv, wl.block_tables) == (-2, 0)


def test_validate_append():
    g = pa.Geometry.make(8, 2, 4)
    assert pa.pa_validate_append(g, [0, 5, -1, 63, -7]) == (0, -1)
    assert pa.pa_validate_append(g, [0, 64]) == (-3, 1)
    assert pa.pa_validate_append(g, [3, 9, 3]) == (-3, 2)


def test_q8_tile_bytes_agree():
    import oracle
    import synthetic
    text = open(pa.HEADER).read()
    assert "#define PA_Q8_TILE_BYTES (16 * 128 + 16 * (128 / 32) * 2)" in text
    assert pa.PA_Q8_TILE_BYTES == 2176 == synthetic.q8_tile_bytes() == oracle.q8_tile_bytes(128, 16)


def test_validate_copy():
    g = pa.Geometry.make(8, 2, 12)
    assert pa.pa_validate_copy(g, [3, 7, 3], [9, 1, 11]) == (0, -1)    # one source, several copies
    assert pa.pa_validate_copy(g, [], []) == (0, -1)
    assert pa.pa_validate_copy(g, [3, 12], [9, 1]) == (-3, 1)          # src out of range
    assert pa.pa_validate_copy(g, [3, 4], [-1, 1]) == (-3, 0)          # dst out of range
    assert pa.pa_validate_copy(g, [3, 4], [9, 9]) == (-3, 1)           # dst repeats
    assert pa.pa_validate_copy(g, [3, 4], [9, 3]) == (-3, 1)           # dst is also a src
    with pytest.raises(ValueError):
        pa.pa_validate_copy(g, [1, 2], [3])


def test_entry_points_reject_bad_arguments_before_launch(lib):
    g = qwen()
    plan = pa.pa_plan(g, [1], [100])
    # NULL pointers for a non-empty batch
    rc = lib.pa_attention_batch(ctypes.byref(g), ctypes.byref(plan), None, None, None, None, 7, None, None, None,
                                None, None, 0, None)
    assert rc == -1
    # geometry differs from the plan's
    g2 = pa.Geometry.make(16, 4, 5461)
    one = ctypes.c_void_p(16)
    rc = lib.pa_attention_batch(ctypes.byref(g2), ctypes.byref(plan), one, one, one, one, 7, one, one, one, one,
                                None, 0, None)
    assert rc == -5
    # a plan that needs a workspace, given none
    big = pa.pa_plan(g, [1] * 4, [8000] * 4)
    assert big.workspace_bytes > 0
    rc = lib.pa_attention_batch(ctypes.byref(g), ctypes.byref(big), one, one, one, one, 600, one, one, one, one,
                                None, 0, None)
    assert rc == -4
    # append: unsupported geometry, negative count, NULL pools
    rc = lib.pa_append_kv(ctypes.byref(pa.Geometry.make(32, 8, 10, head_dim=64)), one, one, one, one, one, 1, None)
    assert rc == -5
    assert lib.pa_append_kv(ctypes.byref(g), one, one, one, one, one, -1, None) == -2
    assert lib.pa_append_kv(ctypes.byref(g), None, one, one, one, one, 1, None) == -1
    assert lib.pa_append_kv(ctypes.byref(g), None, None, None, None, None, 0, None) == 0
    # q8_0 pool: the same argument checks
    mixed = pa.pa_plan(g, [1, 64], [100, 200])
    rc = lib.pa_attention_batch_q8(ctypes.byref(pa.Geometry.make(32, 8, 10, head_dim=64)), ctypes.byref(mixed), one,
                                   one, one, 16, one, one, one, one, None, 0, None)
    assert rc == -5
    rc = lib.pa_attention_batch_q8(ctypes.byref(g), ctypes.byref(plan), None, None, None, 7, None, None, None,
                                   None, None, 0, None)
    assert rc == -1
    assert lib.pa_append_kv_q8(ctypes.byref(g), None, one, one, one, 1, None) == -1
    assert lib.pa_append_kv_q8(ctypes.byref(g), one, one, one, one, -1, None) == -2
    assert lib.pa_append_kv_q8(ctypes.byref(g), None, None, None, None, 0, None) == 0
    assert lib.pa_copy_blocks_q8(ctypes.byref(g), None, one, one, 1, None) == -1
    assert lib.pa_copy_blocks_q8(ctypes.byref(g), one, one, one, -1, None) == -2
    assert lib.pa_copy_blocks_q8(None, one, one, one, 1, None) == -1
    assert lib.pa_append_kv_q8(None, one, one, one, one, 1, None) == -1
    # FP8 pools: the same checks, and scales that are not finite and > 0
    f = ctypes.c_float
    assert lib.pa_append_kv_fp8(ctypes.byref(g), None, one, one, one, one, 1, f(1), f(1), None) == -1
    assert lib.pa_append_kv_fp8(ctypes.byref(g), one, one, one, one, one, -1, f(1), f(1), None) == -2
    assert lib.pa_append_kv_fp8(ctypes.byref(g), one, one, one, one, one, 1, f(0), f(1), None) == -2
    assert lib.pa_append_kv_fp8(ctypes.byref(g), one, one, one, one, one, 1, f(1), f(float("nan")), None) == -2
    assert lib.pa_append_kv_fp8(ctypes.byref(g), None, None, None, None, None, 0, f(1), f(1), None) == 0
    assert lib.pa_append_kv_fp8(None, one, one, one, one, one, 1, f(1), f(1), None) == -1
    rc = lib.pa_attention_batch_fp8(ctypes.byref(g), ctypes.byref(plan), one, one, one, one, 7, one, one, one, one,
                                    None, 0, f(-1), f(1), None)
    assert rc == -2
    rc = lib.pa_attention_batch_fp8(ctypes.byref(g), ctypes.byref(plan), None, None, None, None, 7, None, None, None,
                                    None, None, 0, f(1), f(1), None)
    assert rc == -1
    assert lib.pa_copy_blocks_fp8(ctypes.byref(g), one, None, one, one, 1, None) == -1
    assert lib.pa_copy_blocks_fp8(ctypes.byref(g), one, one, one, one, -1, None) == -2
    # the fused steps (bf16, q8_0, FP8): NULL geometry or plan, missing new rows, a decode
    # step given chunk rows, bad FP8 scales -- all before anything is launched
    chunk = pa.pa_plan(g, [1, 5], [100, 40])
    for name, q8, fp8 in (("pa_decode_step", False, False), ("pa_attention_step", False, False),
                          ("pa_decode_step_q8", True, False), ("pa_attention_step_q8", True, False),
                          ("pa_decode_step_fp8", False, True), ("pa_attention_step_fp8", False, True)):
        fn = getattr(lib, name)
        pools = (one,) if q8 else (one, one)
        scales = (f(1), f(1)) if fp8 else ()

        def call(geo, pl, k_new, v_new, scales=scales):
            return fn(geo, pl, one, *pools, k_new, v_new, one, 7, one, one, one, one, None, 0, *scales, None)
        assert call(None, ctypes.byref(plan), one, one) == -1, name
        assert call(ctypes.byref(g), None, one, one) == -1, name
        assert call(ctypes.byref(g), ctypes.byref(plan), None, one) == -1, name
        if "decode" in name:
            assert call(ctypes.byref(g), ctypes.byref(chunk), one, one) == -5, name
        if fp8:
            assert call(ctypes.byref(g), ctypes.byref(plan), one, one, (f(0), f(1))) == -2, name
            assert call(ctypes.byref(g), ctypes.byref(plan), one, one, (f(1), f(float("inf")))) == -2, name
    # block copy: the same checks
    rc = lib.pa_copy_blocks(ctypes.byref(pa.Geometry.make(32, 8, 10, head_dim=64)), one, one, one, one, 1, None)
    assert rc == -5
    assert lib.pa_copy_blocks(ctypes.byref(g), one, one, one, one, -1, None) == -2
    assert lib.pa_copy_blocks(ctypes.byref(g), one, None, one, one, 1, None) == -1
    assert lib.pa_copy_blocks(None, one, one, one, one, 1, None) == -1
    assert lib.pa_copy_blocks(ctypes.byref(g), None, None, None, None, 0, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(pa, "_lib", None)
    monkeypatch.setattr(pa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        pa.lib()


def test_product_path_does_not_import_oracle():
    import subprocess
    import sys
    code = ("import sys, paged_kv_attention_04_amd as pa; pa.lib(); "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'")
    subprocess.check_call([sys.executable, "-c", code], cwd=pa.os.path.dirname(pa._PKG))
