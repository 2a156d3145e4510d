"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element
on the same seeded inputs.

Bars: pa_append_kv is bit-exact over the whole pool (untouched and poisoned slots
included); attention outputs agree within max |err| <= 2e-2 on the bf16 output and
<= 1e-3 on the fp32 LSE, the error of each output taken against the oracle's exact
(fp64) value.  Against the oracle's own bf16 rounding of that value two correctly
rounded results may differ by one unit in the last place, 2^-5 for outputs in [4, 8),
which no bar of 2e-2 could hold; that difference is printed as well.  Pool slots that
hold no token are NaN, so any read of them would show up as NaN in the output.
"""
import numpy as np
import pytest

import oracle
import synthetic
from synthetic import bf16_bits_to_f32

pytestmark = pytest.mark.gpu

TOL_O = 2e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_04_amd as pa
    pa.lib()
    yield


def _run_gpu(wl, split_blocks=0, prefill_splits=0, cascade=False, num_cus=256, prefix_splits=0):
    import paged_kv_attention_04_amd as pa
    return pa.run_workload(wl, split_blocks=split_blocks, prefill_splits=prefill_splits, cascade=cascade,
                           num_cus=num_cus, prefix_splits=prefix_splits)


def _errors(out, lse, ref, rows=None):
    """Largest |error| of the bf16 outputs and of the LSE against the oracle's exact values."""
    got, want = bf16_bits_to_f32(out).astype(np.float64), ref["out_f64"]
    l_got, l_want = lse.astype(np.float64), ref["lse_f64"]
    if rows is not None:
        got, want, l_got, l_want = got[rows], want[rows], l_got[rows], l_want[rows]
    assert not np.isnan(got).any(), "NaN in GPU output"
    return float(np.max(np.abs(got - want))), float(np.max(np.abs(l_got - l_want)))


def _rounded_difference(out, ref) -> float:
    """Largest |difference| between the GPU's and the oracle's bf16 outputs (reported only)."""
    return float(np.max(np.abs(bf16_bits_to_f32(out) - bf16_bits_to_f32(ref["out"]))))


def exact_error_report(out, lse, ref) -> str:
    """Error of the GPU result against the oracle's unrounded (fp64) values: the largest
    error in bf16 units in the last place of the exact value, the largest normwise
    relative error of a (row, head) output vector, and the largest LSE error.  Printed
    beside the bars, so that a regression that stays inside the absolute bar still shows."""
    got = bf16_bits_to_f32(out).astype(np.float64)
    exact = ref["out_f64"]
    mag = np.maximum(np.abs(exact), 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)              # bf16 keeps 8 significant bits
    ulps = np.abs(got - exact) / ulp
    norm = np.maximum(np.max(np.abs(exact), axis=-1), 1e-30)
    rel = np.max(np.abs(got - exact), axis=-1) / norm
    dl = np.abs(lse.astype(np.float64) - ref["lse_f64"])
    return (f"ulp max {ulps.max():.2f} p99.9 {np.quantile(ulps, 0.999):.2f}; normwise rel max {rel.max():.2e}; "
            f"|dLSE| vs fp64 {dl.max():.2e}")


def check(wl, split_blocks=0, label="", prefill_splits=0, cascade=False, num_cus=256, prefix_splits=0):
    print(f"[gpu] {wl.name} {label} R={wl.num_reqs} total_q={wl.total_q} split={split_blocks} "
          f"prefill_splits={prefill_splits} cascade={cascade} num_cus={num_cus} prefix_splits={prefix_splits}",
          flush=True)
    kp, vp, out, lse = _run_gpu(wl, split_blocks, prefill_splits, cascade, num_cus, prefix_splits)
    okp, ovp, ref = oracle.run_workload(wl, want_f64=True)
    assert np.array_equal(kp, okp) and np.array_equal(vp, ovp), "append is not bit-exact"
    eo, el = _errors(out, lse, ref)
    dec = np.concatenate([np.arange(a, b) for a, b, q in zip(wl.qo_indptr[:-1], wl.qo_indptr[1:], wl.qo_len) if q == 1]
                         or [np.zeros(0, int)]).astype(int)
    pre = np.setdiff1d(np.arange(wl.total_q), dec)
    parts = []
    if dec.size:
        parts.append("decode %.2e/%.2e" % _errors(out, lse, ref, dec))
    if pre.size:
        parts.append("prefill %.2e/%.2e" % _errors(out, lse, ref, pre))
    print(f"[gpu]   max|dO|={eo:.3e} max|dLSE|={el:.3e} ({', '.join(parts)}); {exact_error_report(out, lse, ref)}; "
          f"bf16 vs bf16 {_rounded_difference(out, ref):.3e}", flush=True)
    assert eo <= TOL_O, f"output error {eo}"
    assert el <= TOL_LSE, f"LSE error {el}"
    return out, lse


# ------------------------------------------------------------------ the five workloads

def test_tiny_decode():
    check(synthetic.config_tiny())


def test_tiny_decode_q_times_8():
    """Large scores force many online-softmax rescales."""
    check(synthetic.config_tiny(seed=31, q_scale=8.0), label="q*8")


def test_qwen3_decode_step():
    check(synthetic.config_decode())


def test_shared_prefix_decode():
    check(synthetic.config_shared_prefix())


def test_shared_prefix_decode_cascade():
    """The 384 shared blocks read once per KV head for all 16 rows, merged with each
    row's private suffix."""
    check(synthetic.config_shared_prefix(), cascade=True, label="cascade")


@pytest.mark.parametrize("num_cus", [8, 32, 256])
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_cascade_groups(num_cus, q_scale):
    """Every row shares its first 70 blocks (1120 tokens: the shared range ends inside a
    128-key step).  The prefill row in the middle splits the decode rows into two groups
    (rows 0-4 and 6-8); num_cus 8 / 32 / 256 gives 1 / 2 / 4 key splits of the shared
    blocks.  Row 3 holds exactly one token past the shared range."""
    wl = synthetic.build("cascade_groups", 71, 32, 8, qo_len=[1, 1, 1, 1, 1, 20, 1, 1, 1],
                         kv_len=[1125, 1300, 1500, 1121, 1700, 1250, 1136, 1400, 2000], num_blocks=700,
                         shared_prefix_blocks=70, q_scale=q_scale)
    check(wl, cascade=True, num_cus=num_cus, label=f"cascade q*{q_scale:g}")


def test_mixed_batch():
    check(synthetic.config_mixed())


@pytest.mark.parametrize("batch,long_only", [(1, False), (1, True), (8, False), (32, False), (64, False)])
def test_sweep_decode_layer(batch, long_only):
    check(synthetic.config_sweep_decode(batch, layer=batch % 36, long_only=long_only))


@pytest.mark.parametrize("q8", [False, True])
def test_cascade_prefix_workgroups_merge(q8):
    """32 rows share 125 blocks (2000 tokens) and have 1-20-token suffixes; with 20 prefix
    splits the decode workgroups are done long before the prefix ones, so the prefix
    workgroups are the last arrivals and merge the group's rows: eight passes of four rows,
    21-22 partials per row in two batches."""
    kv = [2001 + (i * 7) % 20 for i in range(32)]
    build = synthetic.build_q8 if q8 else synthetic.build
    wl = build("prefix_last", 73, 32, 8, qo_len=[1] * 32, kv_len=kv, num_blocks=125 + 2 * 32 + 16,
               shared_prefix_blocks=125)
    check(wl, cascade=True, prefix_splits=20, label="q8_0 prefix last" if q8 else "prefix last")


@pytest.mark.parametrize("batch", [8, 16, 32, 64])
def test_sweep_decode_layer_cascade(batch):
    """The sweep's layers with half the rows sharing a 6144-token prefix, on the
    one-launch cascade with the planner's choice of prefix splits and split length."""
    check(synthetic.config_sweep_decode(batch, layer=(batch + 1) % 36), cascade=True, label="cascade")


def test_prompt_chunks_match_oracle_and_one_shot():
    one, chunks = synthetic.prompt_chunks(seed=5, prompt_len=2048, chunk=512, num_blocks=256)
    o_one, l_one = check(one, label="one-shot")
    outs, lses = [], []
    for wl in chunks:
        o, l = check(wl, label="chunk")
        outs.append(o)
        lses.append(l)
    o_ch, l_ch = np.concatenate(outs), np.concatenate(lses)
    d_o = float(np.max(np.abs(bf16_bits_to_f32(o_ch) - bf16_bits_to_f32(o_one))))
    d_l = float(np.max(np.abs(l_ch - l_one)))
    print(f"[gpu]   chunked vs one-shot: {d_o:.3e} / {d_l:.3e}", flush=True)
    assert d_o <= TOL_O and d_l <= TOL_LSE


# ------------------------------------------------------------------ planner-independent results

@pytest.mark.parametrize("split", [1, 2, 3, 7, 64])
def test_split_sweep(split):
    check(synthetic.config_tiny(seed=41), split_blocks=split)
    check(synthetic.build("split_sweep", 42, 32, 8, qo_len=[1] * 6 + [20], kv_len=[1, 16, 17, 700, 1025, 3000, 300],
                          num_blocks=512), split_blocks=split)


@pytest.mark.parametrize("psplit", [1, 2, 3, 5, 64])
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_prefill_split_sweep(psplit, q_scale):
    """Forced key-split counts of the prefill tiles all match the oracle; 64 exceeds every
    tile's step count, so some key ranges are empty.  Rows: a 77-token chunk after 1023
    tokens (three tiles, the last ragged), a 33-token prompt from position 0 (a one-token
    tail tile), a 2-token chunk, and a decode row."""
    wl = synthetic.build("prefill_split", 61, 32, 8, qo_len=[77, 1, 33, 2], kv_len=[1100, 500, 33, 700],
                         num_blocks=400, q_scale=q_scale)
    check(wl, prefill_splits=psplit, label=f"q*{q_scale:g}")


# ------------------------------------------------------------------ invariants on the GPU

def _permuted(wl, seed):
    perm = np.random.default_rng(seed).permutation(wl.num_blocks).astype(np.int32)
    kp = np.empty_like(wl.k_pool)
    vp = np.empty_like(wl.v_pool)
    kp[perm] = wl.k_pool
    vp[perm] = wl.v_pool
    bt = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    sm = (perm[wl.slot_mapping // 16] * 16 + wl.slot_mapping % 16).astype(np.int32)
    import dataclasses
    return dataclasses.replace(wl, k_pool=kp, v_pool=vp, block_tables=bt, slot_mapping=sm, name=wl.name + "_perm")


@pytest.mark.parametrize("make", [synthetic.config_tiny, lambda: synthetic.build(
    "perm_mixed", 51, 32, 8, qo_len=[1, 70, 1, 3], kv_len=[300, 1000, 45, 3], num_blocks=300)])
def test_block_permutation_is_bit_exact(make):
    """Reduction order depends only on logical positions and the plan, never on where the
    blocks sit, so relabelling physical blocks leaves every output bit unchanged."""
    wl = make()
    _, _, out_a, lse_a = _run_gpu(wl)
    _, _, out_b, lse_b = _run_gpu(_permuted(wl, 3))
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


def test_shared_prefix_equals_duplicated_blocks_bit_exact():
    wl = synthetic.build("shared_gpu", 61, 32, 8, qo_len=[1, 1, 1, 40], kv_len=[600, 700, 513, 900], num_blocks=400,
                         shared_prefix_blocks=32)
    _, _, out_a, lse_a = _run_gpu(wl)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    bt = wl.block_tables.copy()
    free = sorted(set(range(wl.num_blocks)) - set(bt.ravel().tolist()))
    for r in range(1, wl.num_reqs):
        for b in range(32):
            new = free.pop()
            kp[new], vp[new] = kp[bt[r, b]], vp[bt[r, b]]
            bt[r, b] = new
    import dataclasses
    dup = dataclasses.replace(wl, k_pool=kp, v_pool=vp, block_tables=bt)
    _, _, out_b, lse_b = _run_gpu(dup)
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)
    check(wl, label="shared vs oracle")


# ------------------------------------------------------------------ edge shapes

@pytest.mark.parametrize("qo,kv", [
    ([1], [1]),                                  # a single key: O = V
    ([1, 1], [16, 32]),                          # whole blocks, no tail
    ([2], [2]),                                  # smallest prefill row, no context
    ([17], [17]),                                # ragged prefill tile
    ([33, 1], [1000, 1]),                        # prefill at an offset + single-key decode
    ([16], [16 * 64 + 1]),                       # context spanning many key tiles
    ([1], [16 * 64 * 3 + 5]),                    # several 64-block splits
    ([5, 1, 8, 1], [5, 2000, 200, 17]),          # short speculative-style rows mixed with decode
])
def test_edge_shapes(qo, kv):
    need = sum(-(-k // 16) for k in kv)
    check(synthetic.build("edge", 71 + len(qo), 8, 2, qo_len=qo, kv_len=kv, num_blocks=need + 3))


# ------------------------------------------------------------------ graph capture

def test_graph_replay_matches_eager():
    """The append and the attention captured into one graph and replayed several times,
    with eager work and synchronisations between the replays: every replay gives the
    eager result bit for bit (the split counters reset themselves; nothing is cleared
    with a memset)."""
    import torch
    import paged_kv_attention_04_amd as pa
    wl = synthetic.build("graph_mixed", 81, 32, 8, qo_len=[1, 40, 1, 1, 1], kv_len=[900, 1200, 1500, 2300, 1600],
                         num_blocks=600, shared_prefix_blocks=40, poison=False)
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256, split_blocks=20, prefill_splits=2)
    pa.pa_plan_shared_prefix(g, plan, wl.qo_len, wl.kv_len, wl.block_tables, 256)
    assert plan.max_splits > 1 and plan.num_prefix_groups == 1 and plan.prefill_splits == 2
    d = {k: pa.to_device(getattr(wl, k)) for k in ("k_pool", "v_pool", "q", "block_tables", "qo_indptr", "kv_len",
                                                   "slot_mapping", "k_new", "v_new")}
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    ws = pa.workspace_for(plan)

    def step():
        pa.pa_append_kv(g, d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], d["slot_mapping"])
        pa.pa_attention_batch(g, plan, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["qo_indptr"],
                              d["kv_len"], out, lse, ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    for i in range(4):
        out.fill_(0)
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[gpu] graph replay {i}", flush=True)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i} differs from the eager result"
        step()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


def _layer_workloads(num_layers, batch=8, seed=97):
    """``num_layers`` layers of the 36-layer sweep's batch shape (half the rows at 2048
    tokens, half at 8192 sharing a 6144-token prefix): one set of block tables and lengths
    for every layer (a block id names one page in each layer's pool), and per layer its
    own pool values, Q and new K / V.  Unused slots stay NaN in every layer."""
    import dataclasses
    base = synthetic.config_sweep_decode(batch, layer=0, num_blocks=1600)
    rng = np.random.default_rng(seed)
    layers = []
    for li in range(num_layers):
        def fresh(a):
            vals = synthetic.f32_to_bf16_bits(rng.standard_normal(a.shape, dtype=np.float32))
            return np.where(np.isnan(bf16_bits_to_f32(a)), a, vals).astype(np.uint16)
        layers.append(dataclasses.replace(
            base, name=f"sweep_b{batch}_stack_layer{li}", k_pool=fresh(base.k_pool), v_pool=fresh(base.v_pool),
            q=synthetic.f32_to_bf16_bits(rng.standard_normal(base.q.shape, dtype=np.float32)),
            k_new=synthetic.f32_to_bf16_bits(rng.standard_normal(base.k_new.shape, dtype=np.float32)),
            v_new=synthetic.f32_to_bf16_bits(rng.standard_normal(base.v_new.shape, dtype=np.float32))))
    return layers


def test_graph_captured_layer_stack_matches_oracle():
    """The form the 36-layer sweep times: one plan per step with shared-prefix groups, then
    per layer one pa_decode_step (append fused into the attention launch), all layers
    captured into one graph.  Four layers of the batch-8 shape; every replay (eager work and
    synchronisations between replays) is checked layer by layer against the oracle --
    pools bit-exact after the append, outputs within the bars -- and bit for bit against
    the first replay."""
    import torch
    import paged_kv_attention_04_amd as pa
    layers = _layer_workloads(4)
    wl0 = layers[0]
    g = pa.Geometry.make(wl0.num_q_heads, wl0.num_kv_heads, wl0.num_blocks, wl0.scale)
    plan = pa.pa_plan(g, wl0.qo_len, wl0.kv_len, 256)
    pa.pa_plan_shared_prefix(g, plan, wl0.qo_len, wl0.kv_len, wl0.block_tables, 256)
    assert plan.num_prefix_groups == 1
    ws = pa.workspace_for(plan)
    bt, indptr, kv = (pa.to_device(getattr(wl0, k)) for k in ("block_tables", "qo_indptr", "kv_len"))
    dev = [{k: pa.to_device(getattr(wl, k)) for k in ("k_pool", "v_pool", "q", "k_new", "v_new")} for wl in layers]
    outs = [torch.empty((wl0.total_q, wl0.num_q_heads, wl0.head_dim), dtype=torch.int16, device="cuda")
            for _ in layers]
    lses = [torch.empty((wl0.total_q, wl0.num_q_heads), dtype=torch.float32, device="cuda") for _ in layers]

    def step():
        for d, o, l in zip(dev, outs, lses):
            pa.pa_decode_step(g, plan, d["q"], d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], bt, indptr, kv, o, l,
                              ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                    # the append is idempotent: the same token to the same slot
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    refs = [oracle.run_workload(wl, want_f64=True) for wl in layers]
    first = None
    for rep in range(3):
        for o, l in zip(outs, lses):
            o.fill_(-1)
            l.fill_(-7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [(o.cpu().numpy().view(np.uint16), l.cpu().numpy()) for o, l in zip(outs, lses)]
        for li, ((out, lse), (okp, ovp, ref), d) in enumerate(zip(got, refs, dev)):
            assert np.array_equal(d["k_pool"].cpu().numpy().view(np.uint16), okp)
            assert np.array_equal(d["v_pool"].cpu().numpy().view(np.uint16), ovp)
            eo, el = _errors(out, lse, ref)
            print(f"[gpu] graph stack replay {rep} layer {li}: max|dO|={eo:.3e} max|dLSE|={el:.3e}; "
                  f"{exact_error_report(out, lse, ref)}", flush=True)
            assert eo <= TOL_O and el <= TOL_LSE
        if first is None:
            first = got
        assert all(np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) for a, b in zip(got, first))
        step()                                    # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ block copy (copy-on-write)

def _geometry(wl):
    import paged_kv_attention_04_amd as pa
    return pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale, wl.head_dim, wl.block_size)


@pytest.mark.parametrize("num_blocks,n_pairs", [(64, 1), (4096, 1500)])
def test_copy_blocks_bit_exact(num_blocks, n_pairs):
    """Whole pools compared bit for bit: copied blocks, every other block, and two
    out-of-range pairs that must be skipped.  Pool words are random bit patterns."""
    import torch
    import paged_kv_attention_04_amd as pa
    print(f"[gpu] copy_blocks num_blocks={num_blocks} pairs={n_pairs}", flush=True)
    rng = np.random.default_rng(num_blocks + n_pairs)
    Hkv, B, D = 8, 16, 128
    kp = rng.integers(0, 2**16, (num_blocks, Hkv, B, D), dtype=np.uint16)
    vp = rng.integers(0, 2**16, (num_blocks, Hkv, B, D), dtype=np.uint16)
    perm = rng.permutation(num_blocks)
    dst = perm[:n_pairs].astype(np.int32)
    src = rng.choice(perm[n_pairs:], n_pairs).astype(np.int32)      # sources may repeat
    src = np.concatenate([src, [-1, 3]]).astype(np.int32)
    dst = np.concatenate([dst, [5, num_blocks]]).astype(np.int32)
    wl_g = pa.Geometry.make(32, Hkv, num_blocks)
    assert pa.pa_validate_copy(wl_g, src, dst)[0] == -3       # PA_ERR_RANGE
    okp, ovp = oracle.copy_blocks(kp, vp, src, dst, Hkv, D, B, num_blocks)
    dk, dv = pa.to_device(kp), pa.to_device(vp)
    pa.pa_copy_blocks(wl_g, dk, dv, pa.to_device(src), pa.to_device(dst))
    pa.pa_copy_blocks(wl_g, dk, dv, pa.to_device(src[:0]), pa.to_device(dst[:0]))    # empty list: no-op
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy().view(np.uint16), okp)
    assert np.array_equal(dv.cpu().numpy().view(np.uint16), ovp)


def _forked_workload(seed, n_fork, prompt):
    """n_fork decode rows forked from one prompt of ``prompt`` tokens: every block is
    shared, the last one partly filled, so each row's next token lands in one slot."""
    nb = -(-prompt // 16)
    assert prompt % 16, "the shared tail must be partly filled"
    wl = synthetic.build("forked", seed, 32, 8, qo_len=[1] * n_fork, kv_len=[prompt + 1] * n_fork,
                         num_blocks=nb + n_fork + 8, shared_prefix_blocks=nb)
    assert len(set(wl.slot_mapping.tolist())) == 1
    return wl


def _copy_on_write(wl):
    """Book section 8.3.2: every row but the first gets a private copy of the shared tail
    block before it writes.  Returns (src, dst, new block tables, new slot mapping)."""
    bt = wl.block_tables.copy()
    used = set(bt[bt >= 0].ravel().tolist())
    free = [b for b in range(wl.num_blocks) if b not in used]
    tail = (int(wl.kv_len[0]) - 1) // wl.block_size
    src, dst = [], []
    for r in range(1, wl.num_reqs):
        src.append(int(bt[r, tail]))
        dst.append(free[r - 1])
        bt[r, tail] = free[r - 1]
    slots = np.array([synthetic.slot_of(bt[r], int(wl.kv_len[r]) - 1, wl.block_size) for r in range(wl.num_reqs)],
                     dtype=np.int32)
    return np.array(src, np.int32), np.array(dst, np.int32), bt, slots


@pytest.mark.parametrize("cascade", [False, True])
def test_copy_on_write_fork_step(cascade):
    """Rows forked from one prompt: copy the shared tail, repoint the tables, append each
    row's token and attend, all on the device; the oracle takes the same steps.  Pools
    bit-exact, attention within the bars, and each row sees its own token."""
    import torch
    import paged_kv_attention_04_amd as pa
    wl = _forked_workload(41, 8, 16 * 37 + 5)
    src, dst, bt, slots = _copy_on_write(wl)
    g = _geometry(wl)
    assert pa.pa_validate_copy(g, src, dst) == (0, -1)
    assert pa.pa_validate_append(g, slots) == (0, -1)
    print(f"[gpu] copy-on-write fork rows={wl.num_reqs} kv={int(wl.kv_len[0])} cascade={cascade}", flush=True)
    okp, ovp = oracle.copy_blocks(wl.k_pool, wl.v_pool, src, dst, wl.num_kv_heads, wl.head_dim, wl.block_size,
                                  wl.num_blocks)
    okp, ovp = oracle.append(okp, ovp, wl.k_new, wl.v_new, slots, wl.num_kv_heads, wl.head_dim, wl.block_size,
                             wl.num_blocks)
    ref = oracle.attention(wl.q, okp, ovp, bt, wl.qo_len, wl.kv_len, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.block_size, wl.num_blocks, wl.scale, want_f64=True)

    dk, dv = pa.to_device(wl.k_pool), pa.to_device(wl.v_pool)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len)
    if cascade:
        pa.pa_plan_shared_prefix(g, plan, wl.qo_len, wl.kv_len, bt)
        assert plan.num_prefix_groups == 1
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    pa.pa_copy_blocks(g, dk, dv, pa.to_device(src), pa.to_device(dst))
    pa.pa_append_kv(g, dk, dv, pa.to_device(wl.k_new), pa.to_device(wl.v_new), pa.to_device(slots))
    pa.pa_attention_batch(g, plan, pa.to_device(wl.q), dk, dv, pa.to_device(bt), pa.to_device(wl.qo_indptr),
                          pa.to_device(wl.kv_len), out, lse, pa.workspace_for(plan))
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy().view(np.uint16), okp)
    assert np.array_equal(dv.cpu().numpy().view(np.uint16), ovp)
    eo, el = _errors(out.cpu().numpy().view(np.uint16), lse.cpu().numpy(), ref)
    print(f"[gpu]   max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE
    # the rows' outputs differ: each attended to its own newest token
    o = bf16_bits_to_f32(out.cpu().numpy().view(np.uint16))
    assert all(not np.array_equal(o[0], o[r]) for r in range(1, wl.num_reqs))


# ------------------------------------------------------------------ q8_0 pool

def test_q8_tiny_decode():
    """Append quantises the new rows bit-exactly as the oracle does (whole pools compared,
    poisoned slots included); attention over the represented values within the bars."""
    check(synthetic.config_tiny_q8(), label="q8_0")


def test_q8_tiny_decode_q_times_8():
    check(synthetic.config_tiny_q8(seed=13, q_scale=8.0), label="q8_0 q*8")


def test_q8_qwen3_decode_step():
    check(synthetic.config_decode_q8(), label="q8_0")


@pytest.mark.parametrize("split", [1, 2, 7, 64])
def test_q8_split_sweep(split):
    wl = synthetic.build_q8("q8_split", 14, 32, 8, qo_len=[1] * 6, kv_len=[1, 16, 17, 300, 1000, 2500],
                            num_blocks=400)
    check(wl, split_blocks=split, label=f"q8_0 split {split}")


@pytest.mark.parametrize("kv", [[1], [15], [16], [33], [4096]])
def test_q8_edge_lengths(kv):
    wl = synthetic.build_q8("q8_edge", 15, 32, 8, qo_len=[1] * len(kv), kv_len=kv, num_blocks=300)
    check(wl, label=f"q8_0 kv {kv}")


def test_q8_chunk_row_small():
    """A 40-token chunk at offset 60 beside a decode row (8 q / 2 kv heads) on a q8_0 pool:
    the chunk's new rows are quantised by the append and read back as codes."""
    wl = synthetic.build_q8("q8_prefill", 16, 8, 2, qo_len=[1, 40], kv_len=[20, 100], num_blocks=32)
    check(wl, label="q8_0 chunk")


@pytest.mark.parametrize("q_scale", [1.0, 8.0])
@pytest.mark.parametrize("psplit", [0, 1, 3, 16])
def test_q8_chunk_rows(psplit, q_scale):
    """Chunk rows on a q8_0 pool: chunks at position 0 (2 and 129 tokens), ragged tails,
    a 77-token chunk at 2036 spanning three 32-token tiles, decode rows beside them, with
    the planner's or 1 / 3 / 16 key splits; q*8 makes the softmax peaked, so the LSE
    follows single scores (their K scales are applied in fp32, not rounded)."""
    wl = synthetic.build_q8("q8_chunks", 17, 32, 8, qo_len=[2, 31, 129, 1, 77, 16],
                            kv_len=[2, 1000, 129, 500, 2113, 300], num_blocks=300, q_scale=q_scale)
    check(wl, prefill_splits=psplit, label=f"q8_0 chunks psplit {psplit} q*{q_scale:g}")


def test_q8_mixed_batch():
    """The mixed batch (512-token chunk at 4096 + 31 decode rows) on a q8_0 pool."""
    check(synthetic.config_mixed_q8(), label="q8_0")


def test_q8_shared_prefix_cascade():
    """The shared-prefix decode on a q8_0 pool through the one-launch cascade: the shared
    blocks' codes read once per KV head by the matrix-unit tile."""
    check(synthetic.config_shared_prefix_q8(), cascade=True, label="q8_0 cascade")


@pytest.mark.parametrize("num_cus", [8, 256])
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_q8_cascade_groups(num_cus, q_scale):
    """test_cascade_groups' batch (two groups split by a chunk row, a shared range ending
    inside a step, a one-token suffix) on a q8_0 pool."""
    wl = synthetic.build_q8("q8_cascade_groups", 72, 32, 8, qo_len=[1, 1, 1, 1, 1, 20, 1, 1, 1],
                            kv_len=[1125, 1300, 1500, 1121, 1700, 1250, 1136, 1400, 2000], num_blocks=700,
                            shared_prefix_blocks=70, q_scale=q_scale)
    check(wl, cascade=True, num_cus=num_cus, label=f"q8_0 cascade q*{q_scale:g}")


def test_q8_copy_blocks_bit_exact():
    import torch
    import paged_kv_attention_04_amd as pa
    rng = np.random.default_rng(17)
    nb, Hkv = 300, 8
    pool = rng.integers(0, 256, pa.q8_pool_shape(nb, Hkv), dtype=np.uint8)
    perm = rng.permutation(nb)
    src, dst = perm[:40].astype(np.int32), perm[40:80].astype(np.int32)
    src = np.concatenate([src, [-1, 3]]).astype(np.int32)
    dst = np.concatenate([dst, [5, nb]]).astype(np.int32)
    g = pa.Geometry.make(32, Hkv, nb)
    dp = pa.to_device(pool)
    pa.pa_copy_blocks_q8(g, dp, pa.to_device(src), pa.to_device(dst))
    torch.cuda.synchronize()
    want = pool.copy()
    want[dst[:40]] = pool[src[:40]]
    assert np.array_equal(dp.cpu().numpy(), want)


@pytest.mark.parametrize("prefill_splits,split_blocks", [(3, 7), (64, 2)])
def test_split_results_are_bitwise_reproducible(prefill_splits, split_blocks):
    """Split partials are merged in split order, not in the order the splits finish, so
    repeated runs of one batch give identical bits."""
    import paged_kv_attention_04_amd as pa
    wl = synthetic.build("repro", 82, 32, 8, qo_len=[1, 96, 1], kv_len=[700, 1500, 1300], num_blocks=300,
                         poison=False)
    print(f"[gpu] reproducibility prefill_splits={prefill_splits} split_blocks={split_blocks}", flush=True)
    first = pa.run_workload(wl, split_blocks=split_blocks, prefill_splits=prefill_splits)
    for _ in range(5):
        again = pa.run_workload(wl, split_blocks=split_blocks, prefill_splits=prefill_splits)
        assert np.array_equal(again[2], first[2]) and np.array_equal(again[3], first[3])


# ------------------------------------------------------------------ block allocator

def test_deferred_release_waits_for_the_stream():
    """A block whose last reference goes while queued device work may still read it
    returns to the free pool only after that work: here a bounded sleep kernel."""
    import torch
    import paged_kv_attention_04_amd as pa
    a = pa.BlockAllocator(16)
    b = a.alloc(4)
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)                    # a few tens of ms of queued work
    a.release(b, stream=torch.cuda.current_stream())
    free, waiting = a.num_free()
    assert (free, waiting) == (12, 4)
    with pytest.raises(pa.PaError):
        a.alloc(13)                                   # the four are not reusable yet
    torch.cuda.synchronize()
    assert a.num_free() == (16, 0)
    c = a.alloc(2)
    torch.cuda._sleep(200_000_000)
    a.release(c, stream=torch.cuda.current_stream())
    a.sync()                                          # waits for that work
    assert a.num_free() == (16, 0)


def test_allocator_drives_fork_copy_on_write():
    """The forked decode step with its copy-on-write decisions taken by the allocator:
    every row holds a reference to the shared blocks; each writer but the last to ask
    gets a fresh tail (the last one finds the tail unshared and writes in place).  The
    pools and outputs equal the oracle's for the same tables."""
    import torch
    import paged_kv_attention_04_amd as pa
    wl = _forked_workload(43, 6, 16 * 20 + 9)
    nb = wl.num_blocks
    alloc = pa.BlockAllocator(nb)
    ids = alloc.alloc(nb)                             # take every block, give back the unused ones
    used = sorted(set(wl.block_tables[wl.block_tables >= 0].ravel().tolist()))
    alloc.release([x for x in ids if x not in used], deferred=False)
    shared = wl.block_tables[0, :21]
    for _ in range(wl.num_reqs - 1):
        alloc.retain(shared)                          # every forked row references the prompt
    bt = wl.block_tables.copy()
    src, dst = [], []
    for r in range(1, wl.num_reqs):                   # rows 1.. ask first; row 0 asks last
        t = alloc.cow(int(bt[r, 20]))
        if t != bt[r, 20]:
            src.append(int(bt[r, 20]))
            dst.append(t)
            bt[r, 20] = t
    assert alloc.cow(int(bt[0, 20])) == bt[0, 20]     # the last holder writes in place
    assert all(alloc.refcount(int(x)) == wl.num_reqs for x in shared[:20])
    src, dst = np.array(src, np.int32), np.array(dst, np.int32)
    slots = np.array([synthetic.slot_of(bt[r], int(wl.kv_len[r]) - 1, 16) for r in range(wl.num_reqs)], np.int32)
    g = _geometry(wl)
    assert pa.pa_validate_copy(g, src, dst) == (0, -1) and pa.pa_validate_append(g, slots) == (0, -1)
    okp, ovp = oracle.copy_blocks(wl.k_pool, wl.v_pool, src, dst, wl.num_kv_heads, 128, 16, nb)
    okp, ovp = oracle.append(okp, ovp, wl.k_new, wl.v_new, slots, wl.num_kv_heads, 128, 16, nb)
    ref = oracle.attention(wl.q, okp, ovp, bt, wl.qo_len, wl.kv_len, wl.num_q_heads, wl.num_kv_heads, 128, 16, nb,
                           wl.scale, want_f64=True)
    dk, dv = pa.to_device(wl.k_pool), pa.to_device(wl.v_pool)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len)
    out = torch.empty((wl.total_q, wl.num_q_heads, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    pa.pa_copy_blocks(g, dk, dv, pa.to_device(src), pa.to_device(dst))
    pa.pa_append_kv(g, dk, dv, pa.to_device(wl.k_new), pa.to_device(wl.v_new), pa.to_device(slots))
    pa.pa_attention_batch(g, plan, pa.to_device(wl.q), dk, dv, pa.to_device(bt), pa.to_device(wl.qo_indptr),
                          pa.to_device(wl.kv_len), out, lse, pa.workspace_for(plan))
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy().view(np.uint16), okp)
    assert np.array_equal(dv.cpu().numpy().view(np.uint16), ovp)
    eo, el = _errors(out.cpu().numpy().view(np.uint16), lse.cpu().numpy(), ref)
    assert eo <= TOL_O and el <= TOL_LSE
    for r in range(wl.num_reqs):                      # every request ends
        alloc.release(bt[r, :21], stream=torch.cuda.current_stream())
    alloc.sync()
    assert alloc.num_free() == (nb, 0)


# ------------------------------------------------------------------ PA_VALIDATE=1

def test_validate_mode_rejects_bad_content_before_launch(monkeypatch):
    """With PA_VALIDATE=1 the entry points copy the index arrays to the host and run the
    validators first: a table entry outside the pool, a repeated slot or lengths that
    disagree return an error with nothing launched; a valid batch gives the same result
    as without the checks."""
    import torch
    import paged_kv_attention_04_amd as pa
    wl = synthetic.config_tiny(poison=False)
    ref = pa.run_workload(wl, validate=False)
    monkeypatch.setenv("PA_VALIDATE", "1")
    got = pa.run_workload(wl, validate=False)
    assert all(np.array_equal(a, b) for a, b in zip(ref, got))
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len)
    kp, vp = pa.to_device(wl.k_pool), pa.to_device(wl.v_pool)
    out = torch.zeros((wl.total_q, wl.num_q_heads, 128), dtype=torch.int16, device="cuda")
    lse = torch.zeros((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    bad_bt = wl.block_tables.copy()
    bad_bt[2, 1] = wl.num_blocks + 5
    with pytest.raises(pa.PaError, match="RANGE"):
        pa.pa_attention_batch(g, plan, pa.to_device(wl.q), kp, vp, pa.to_device(bad_bt), pa.to_device(wl.qo_indptr),
                              pa.to_device(wl.kv_len), out, lse, pa.workspace_for(plan))
    bad_kv = wl.kv_len.copy()
    bad_kv[0] = 0                                      # kv_len < qo_len
    with pytest.raises(pa.PaError, match="SHAPE"):
        pa.pa_attention_batch(g, plan, pa.to_device(wl.q), kp, vp, pa.to_device(wl.block_tables),
                              pa.to_device(wl.qo_indptr), pa.to_device(bad_kv), out, lse, pa.workspace_for(plan))
    # lengths that keep the total but move the 2-token row: the plan's row classes no
    # longer match the device's (a row the plan takes for a decode row would be left
    # unwritten), so validation rejects the call
    wl2 = synthetic.build("validate_classes", 19, 8, 2, qo_len=[2, 1, 1], kv_len=[40, 50, 60], num_blocks=32,
                          poison=False)
    g2 = pa.Geometry.make(wl2.num_q_heads, wl2.num_kv_heads, wl2.num_blocks, wl2.scale)
    plan2 = pa.pa_plan(g2, [1, 2, 1], wl2.kv_len)
    out2 = torch.zeros((wl2.total_q, wl2.num_q_heads, 128), dtype=torch.int16, device="cuda")
    lse2 = torch.zeros((wl2.total_q, wl2.num_q_heads), dtype=torch.float32, device="cuda")
    with pytest.raises(pa.PaError, match="SHAPE"):
        pa.pa_attention_batch(g2, plan2, pa.to_device(wl2.q), pa.to_device(wl2.k_pool), pa.to_device(wl2.v_pool),
                              pa.to_device(wl2.block_tables), pa.to_device(wl2.qo_indptr), pa.to_device(wl2.kv_len),
                              out2, lse2, pa.workspace_for(plan2))
    torch.cuda.synchronize()
    assert not out2.any()
    slots = wl.slot_mapping.copy()
    slots[1] = slots[0]
    before = kp.clone()
    with pytest.raises(pa.PaError, match="RANGE"):
        pa.pa_append_kv(g, kp, vp, pa.to_device(wl.k_new), pa.to_device(wl.v_new), pa.to_device(slots))
    torch.cuda.synchronize()
    assert torch.equal(kp, before) and not out.any()   # nothing was launched


# ------------------------------------------------------------------ fused decode step

def _decode_step_gpu(wl, split_blocks=0, cascade=False):
    """pa_decode_step on device copies of the workload; returns host (k_pool, v_pool, out, lse)."""
    import torch
    import paged_kv_attention_04_amd as pa
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256, split_blocks)
    if cascade:
        pa.pa_plan_shared_prefix(g, plan, wl.qo_len, wl.kv_len, wl.block_tables)
    kp, vp = pa.to_device(wl.k_pool), pa.to_device(wl.v_pool)
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    pa.pa_decode_step(g, plan, pa.to_device(wl.q), kp, vp, pa.to_device(wl.k_new), pa.to_device(wl.v_new),
                      pa.to_device(wl.block_tables), pa.to_device(wl.qo_indptr), pa.to_device(wl.kv_len), out, lse,
                      pa.workspace_for(plan))
    torch.cuda.synchronize()
    return (kp.cpu().numpy().view(np.uint16), vp.cpu().numpy().view(np.uint16), out.cpu().numpy().view(np.uint16),
            lse.cpu().numpy())


@pytest.mark.parametrize("case", ["tiny", "qwen3", "qwen3_full", "split7", "split1", "cascade"])
def test_fused_decode_step_matches_append_then_attention(case):
    """Writing each row's new token inside the attention launch gives the pools the
    oracle's append gives, and the same output bits as pa_append_kv followed by
    pa_attention_batch on the GPU."""
    split = {"split7": 7, "split1": 1}.get(case, 0)
    cascade = case == "cascade"
    wl = {"tiny": lambda: synthetic.config_tiny(),
          "qwen3": lambda: synthetic.config_decode(num_reqs=12, num_blocks=2000),
          "qwen3_full": lambda: synthetic.config_decode(),        # the bench's step, full size
          "split7": lambda: synthetic.config_tiny(seed=45),
          "split1": lambda: synthetic.build("fused_split1", 46, 32, 8, qo_len=[1] * 3, kv_len=[1, 17, 300],
                                            num_blocks=40),
          "cascade": lambda: synthetic.build("fused_cascade", 47, 32, 8, qo_len=[1] * 5, kv_len=[700, 820, 990, 640, 777],
                                             num_blocks=400, shared_prefix_blocks=30)}[case]()
    print(f"[gpu] fused decode step {case}", flush=True)
    kp, vp, out, lse = _decode_step_gpu(wl, split, cascade)
    okp, ovp, ref = oracle.run_workload(wl, want_f64=True)
    assert np.array_equal(kp, okp) and np.array_equal(vp, ovp)
    eo, el = _errors(out, lse, ref)
    print(f"[gpu]   max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE
    _, _, out2, lse2 = _run_gpu(wl, split, cascade=cascade)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def _attention_step_gpu(wl, prefill_splits=0, cascade=False, one_launch=None, split_blocks=0):
    """pa_attention_step on device copies of the workload; returns host (k_pool, v_pool, out, lse)."""
    import torch
    import paged_kv_attention_04_amd as pa
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256, split_blocks, prefill_splits)
    if cascade:
        pa.pa_plan_shared_prefix(g, plan, wl.qo_len, wl.kv_len, wl.block_tables)
        assert plan.num_prefix_groups >= 1
    if one_launch is not None:
        plan.one_launch = one_launch
    kp, vp = pa.to_device(wl.k_pool), pa.to_device(wl.v_pool)
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    pa.pa_attention_step(g, plan, pa.to_device(wl.q), kp, vp, pa.to_device(wl.k_new), pa.to_device(wl.v_new),
                         pa.to_device(wl.block_tables), pa.to_device(wl.qo_indptr), pa.to_device(wl.kv_len), out, lse,
                         pa.workspace_for(plan))
    torch.cuda.synchronize()
    return (kp.cpu().numpy().view(np.uint16), vp.cpu().numpy().view(np.uint16), out.cpu().numpy().view(np.uint16),
            lse.cpu().numpy())


@pytest.mark.parametrize("case", ["tiny_mixed", "mixed", "chunk_at_0", "chunk_at_1536", "spec", "psplit3",
                                  "cascade_mixed"])
def test_fused_attention_step_matches_append_then_attention(case):
    """Any batch with the append fused into the attention launches (chunk rows read their
    new tokens from the new rows, one workgroup per tile and KV head writes them): the
    pools the oracle's append gives, outputs within tolerance of the oracle, and the same
    output bits as pa_append_kv followed by pa_attention_batch on the GPU."""
    psplit = 3 if case == "psplit3" else 0
    cascade = case == "cascade_mixed"
    chunks = None
    if case.startswith("chunk_at"):
        _, chunks = synthetic.prompt_chunks(seed=5, prompt_len=2048, chunk=512, num_blocks=256)
    wl = {"tiny_mixed": lambda: synthetic.build("fused_mixed", 48, 8, 2, qo_len=[1, 40], kv_len=[20, 100],
                                                num_blocks=32),
          "mixed": lambda: synthetic.config_mixed(),
          "chunk_at_0": lambda: chunks[0],
          "chunk_at_1536": lambda: chunks[3],
          "spec": lambda: synthetic.build("spec_verify_fused", 93, 32, 8, qo_len=[8] * 16, kv_len=[2048 + 8] * 16,
                                          num_blocks=16 * 130 + 32),
          "psplit3": lambda: synthetic.build("fused_psplit", 49, 32, 8, qo_len=[1, 40, 1, 70, 2], kv_len=[300, 500, 17, 70, 33],
                                             num_blocks=200),
          "cascade_mixed": lambda: synthetic.build("fused_cascade_mixed", 50, 32, 8, qo_len=[1, 1, 1, 1, 33],
                                                   kv_len=[700, 820, 990, 640, 900], num_blocks=400,
                                                   shared_prefix_blocks=30)}[case]()
    print(f"[gpu] fused attention step {case} R={wl.num_reqs} total_q={wl.total_q}", flush=True)
    kp, vp, out, lse = _attention_step_gpu(wl, psplit, cascade)
    okp, ovp, ref = oracle.run_workload(wl, want_f64=True)
    assert np.array_equal(kp, okp) and np.array_equal(vp, ovp)
    eo, el = _errors(out, lse, ref)
    print(f"[gpu]   max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE
    _, _, out2, lse2 = _run_gpu(wl, 0, psplit, cascade=cascade)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_validate_mode_attention_step(monkeypatch):
    """With PA_VALIDATE=1 pa_attention_step checks the slots its fused append writes,
    chunk rows included: a valid mixed batch gives the same bytes as without the checks,
    and tables that send a chunk token and another row's new token to one slot return
    PA_ERR_RANGE with nothing launched."""
    import torch
    import paged_kv_attention_04_amd as pa
    wl = synthetic.build("validate_step", 51, 8, 2, qo_len=[1, 40, 3], kv_len=[20, 100, 35], num_blocks=40,
                         poison=False)
    plain = _attention_step_gpu(wl)
    monkeypatch.setenv("PA_VALIDATE", "1")
    checked = _attention_step_gpu(wl)
    assert all(np.array_equal(a, b) for a, b in zip(plain, checked))
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len)
    bad_bt = wl.block_tables.copy()
    bad_bt[2, 2] = bad_bt[1, 6]          # row 2's new positions 32..34 land on row 1's positions 96..98
    kp, vp = pa.to_device(wl.k_pool), pa.to_device(wl.v_pool)
    before = kp.clone()
    out = torch.zeros((wl.total_q, wl.num_q_heads, 128), dtype=torch.int16, device="cuda")
    lse = torch.zeros((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    with pytest.raises(pa.PaError, match="RANGE"):
        pa.pa_attention_step(g, plan, pa.to_device(wl.q), kp, vp, pa.to_device(wl.k_new), pa.to_device(wl.v_new),
                             pa.to_device(bad_bt), pa.to_device(wl.qo_indptr), pa.to_device(wl.kv_len), out, lse,
                             pa.workspace_for(plan))
    torch.cuda.synchronize()
    assert torch.equal(kp, before) and not out.any()   # nothing was launched


@pytest.mark.parametrize("case", ["mixed", "tiny_mixed", "psplit3_split5", "chunks_only_one_decode", "many_decode"])
def test_one_launch_mixed_batch(case):
    """Chunk tiles and decode workgroups in one launch (chunk tiles first, or interleaved):
    the same output bits as the two launches (prefill, then decode), with and without the
    fused append, pools bit-exact against the oracle's append, outputs within the bars of
    the oracle."""
    wl, psplit, split = {
        "mixed": lambda: (synthetic.config_mixed(), 0, 0),
        "tiny_mixed": lambda: (synthetic.build("one_launch_tiny", 52, 8, 2, qo_len=[1, 40, 1], kv_len=[20, 100, 7],
                                               num_blocks=40), 0, 0),
        "psplit3_split5": lambda: (synthetic.build("one_launch_splits", 53, 32, 8, qo_len=[1, 40, 1, 70, 2, 1],
                                                   kv_len=[300, 500, 17, 700, 33, 900], num_blocks=300), 3, 5),
        "chunks_only_one_decode": lambda: (synthetic.build("one_launch_more_tiles", 54, 32, 8, qo_len=[200, 1, 130],
                                                           kv_len=[1200, 64, 900], num_blocks=200), 0, 0),
        "many_decode": lambda: (synthetic.build("one_launch_many_decode", 55, 32, 8, qo_len=[33] + [1] * 40,
                                                kv_len=[40] + [300 + 13 * i for i in range(40)],
                                                num_blocks=3 + sum(-(-(300 + 13 * i) // 16) for i in range(40)) + 8),
                           0, 0),
    }[case]()
    print(f"[gpu] one-launch mixed {case} R={wl.num_reqs} total_q={wl.total_q}", flush=True)
    two = _run_gpu(wl, split, psplit)
    import paged_kv_attention_04_amd as pa
    one = pa.run_workload(wl, split_blocks=split, prefill_splits=psplit, one_launch=1)
    assert np.array_equal(one[2], two[2]) and np.array_equal(one[3], two[3]), "one launch differs from two"
    mix = pa.run_workload(wl, split_blocks=split, prefill_splits=psplit, one_launch=2)      # interleaved order
    assert np.array_equal(mix[2], two[2]) and np.array_equal(mix[3], two[3]), "interleaved launch differs"
    okp, ovp, ref = oracle.run_workload(wl, want_f64=True)
    assert np.array_equal(one[0], okp) and np.array_equal(one[1], ovp)
    eo, el = _errors(one[2], one[3], ref)
    print(f"[gpu]   max|dO|={eo:.3e} max|dLSE|={el:.3e}; {exact_error_report(one[2], one[3], ref)}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE
    fk, fv, fo, fl = _attention_step_gpu(wl, psplit, one_launch=1, split_blocks=split)      # the fused append too
    assert np.array_equal(fk, okp) and np.array_equal(fv, ovp)
    assert np.array_equal(fo, two[2]) and np.array_equal(fl, two[3])


def test_fused_decode_step_rejects_chunk_rows():
    import paged_kv_attention_04_amd as pa
    wl = synthetic.build("fused_mixed", 48, 8, 2, qo_len=[1, 40], kv_len=[20, 100], num_blocks=32)
    with pytest.raises(pa.PaError, match="UNSUPPORTED"):
        _decode_step_gpu(wl)


def test_spec_verify_rows():
    """Speculative verification (small qo_len rows): 16 requests x 8 new tokens, causal,
    at 2056 tokens of context, through the chunked-prefill path."""
    wl = synthetic.build("spec_verify_2k", 92, 32, 8, qo_len=[8] * 16, kv_len=[2048 + 8] * 16,
                         num_blocks=16 * 130 + 32)
    check(wl, label="spec verify")


# ------------------------------------------------------------------ grouped-query ratios

# (query heads, KV heads): G = 1, 2, 3, 5, 6, 8 query heads per KV head, and one KV head
# for all query heads.  Workgroups serve four head slots of one KV head, so G = 1, 2, 3
# leave slots empty, 5 and 6 take two slices with the second partly empty, 8 two full ones.
GQA_RATIOS = [(8, 8), (16, 8), (24, 8), (40, 8), (48, 8), (64, 8), (8, 1)]


def _gqa(case, hq, hkv, q8=False, fp8=False):
    seed = 4000 + 17 * hq + hkv + (500 if q8 else 0) + (900 if fp8 else 0)
    make = synthetic.build_q8 if q8 else synthetic.build_fp8 if fp8 else synthetic.build
    name = f"gqa{hq}x{hkv}_{case}" + ("_q8" if q8 else "") + ("_fp8" if fp8 else "")
    if case == "mixed":        # split decode rows, a one-token row, 32-token chunk tiles
        return make(name, seed, hq, hkv, qo_len=[1, 70, 1, 1, 33], kv_len=[900, 300, 17, 1, 33], num_blocks=100)
    if case == "chunks8":      # rows of at most 8 tokens: 32-row tiles
        return make(name, seed, hq, hkv, qo_len=[8] * 5 + [3], kv_len=[520] * 5 + [40], num_blocks=180)
    if case == "chunks16":     # rows of at most 16 tokens: 64-row tiles
        return make(name, seed, hq, hkv, qo_len=[16, 12, 1, 16], kv_len=[700, 90, 300, 16], num_blocks=90)
    if case == "cascade":      # decode rows sharing 30 blocks
        return make(name, seed, hq, hkv, qo_len=[1] * 6, kv_len=[700, 820, 990, 640, 777, 1000], num_blocks=200,
                    shared_prefix_blocks=30)
    raise ValueError(case)


@pytest.mark.parametrize("hq,hkv", GQA_RATIOS)
@pytest.mark.parametrize("case", ["mixed", "chunks8", "chunks16", "cascade"])
def test_gqa_ratios(hq, hkv, case):
    """Other query-head-per-KV-head ratios through every path: decode rows (split and not),
    chunk tiles of 128 / 64 / 32 rows with and without key splits, the shared-prefix
    cascade, the fused append (both steps) and the one-launch mixed batch, each within the
    bars of the oracle, and the fused and one-launch forms bit-identical to the plain ones."""
    wl = _gqa(case, hq, hkv)
    if case == "cascade":
        check(wl, cascade=True, label=f"G={hq // hkv} cascade")
        check(wl, split_blocks=3, label=f"G={hq // hkv} split 3")
        kp, vp, out, lse = _decode_step_gpu(wl, cascade=True)
        _, _, out2, lse2 = _run_gpu(wl, cascade=True)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
        okp, ovp, _ = oracle.run_workload(wl)
        assert np.array_equal(kp, okp) and np.array_equal(vp, ovp)
        return
    out, lse = check(wl, split_blocks=5, label=f"G={hq // hkv} split 5")
    check(wl, prefill_splits=3, label=f"G={hq // hkv} psplit 3")
    kp, vp, fo, fl = _attention_step_gpu(wl, split_blocks=5)
    assert np.array_equal(fo, out) and np.array_equal(fl, lse), "fused step differs"
    okp, ovp, _ = oracle.run_workload(wl)
    assert np.array_equal(kp, okp) and np.array_equal(vp, ovp)
    if case == "mixed":
        import paged_kv_attention_04_amd as pa
        for mode in (1, 2):
            one = pa.run_workload(wl, split_blocks=5, one_launch=mode)
            assert np.array_equal(one[2], out) and np.array_equal(one[3], lse), f"one launch {mode} differs"


@pytest.mark.parametrize("hq,hkv", [(8, 8), (24, 8), (48, 8), (8, 1)])
@pytest.mark.parametrize("case", ["mixed", "cascade"])
def test_gqa_ratios_q8(hq, hkv, case):
    """The q8_0 pool at other grouped-query ratios: decode rows, chunk rows, cascade."""
    wl = _gqa(case, hq, hkv, q8=True)
    check(wl, split_blocks=5, cascade=case == "cascade", label=f"G={hq // hkv} q8_0")


# ------------------------------------------------------------------ FP8 pools

def test_fp8_tiny_decode():
    """Append encodes the new rows bit-exactly as the oracle does (both whole pools compared,
    NaN-coded poison slots included); attention over the represented values within the bars."""
    check(synthetic.config_tiny_fp8(), label="fp8")


def test_fp8_tiny_decode_q_times_8():
    check(synthetic.config_tiny_fp8(seed=23, q_scale=8.0), label="fp8 q*8")


def test_fp8_qwen3_decode_step():
    check(synthetic.config_decode_fp8(), label="fp8")


@pytest.mark.parametrize("split", [1, 2, 7, 64])
def test_fp8_split_sweep(split):
    wl = synthetic.build_fp8("fp8_split", 24, 32, 8, qo_len=[1] * 6, kv_len=[1, 16, 17, 300, 1000, 2500],
                             num_blocks=400)
    check(wl, split_blocks=split, label=f"fp8 split {split}")


@pytest.mark.parametrize("kv", [[1], [15], [16], [33], [4096]])
def test_fp8_edge_lengths(kv):
    wl = synthetic.build_fp8("fp8_edge", 25, 32, 8, qo_len=[1] * len(kv), kv_len=kv, num_blocks=300)
    check(wl, label=f"fp8 kv {kv}")


@pytest.mark.parametrize("q_scale", [1.0, 8.0])
@pytest.mark.parametrize("psplit", [0, 1, 3, 16])
def test_fp8_chunk_rows(psplit, q_scale):
    """Chunk rows on FP8 pools (128-row tiles): chunks at position 0 (2 and 129 tokens),
    ragged tails, a 77-token chunk at 2036 spanning three 32-token tiles, decode rows beside
    them, with the planner's or 1 / 3 / 16 key splits."""
    wl = synthetic.build_fp8("fp8_chunks", 27, 32, 8, qo_len=[2, 31, 129, 1, 77, 16],
                             kv_len=[2, 1000, 129, 500, 2113, 300], num_blocks=300, q_scale=q_scale)
    check(wl, prefill_splits=psplit, label=f"fp8 chunks psplit {psplit} q*{q_scale:g}")


@pytest.mark.parametrize("k_scale,v_scale", [(2.0 ** -8, 2.0 ** -7), (7.3, 0.0173), (1.0, 1.0)])
def test_fp8_scales(k_scale, v_scale):
    """Scales that make the append saturate (|x| / scale beyond 448 for most new values),
    that make it produce subnormal codes (x / 7.3), and the unit scale, through decode,
    split decode and chunk rows."""
    wl = synthetic.build_fp8("fp8_scales", 28, 32, 8, qo_len=[1, 40, 1, 9], kv_len=[700, 300, 33, 1200],
                             num_blocks=200, k_scale=k_scale, v_scale=v_scale)
    check(wl, label=f"fp8 scales {k_scale:g}/{v_scale:g}")
    check(wl, split_blocks=3, prefill_splits=2, label=f"fp8 scales {k_scale:g}/{v_scale:g} split")


def test_fp8_mixed_batch():
    """The mixed batch (512-token chunk at 4096 + 31 decode rows) on FP8 pools."""
    check(synthetic.config_mixed_fp8(), label="fp8")


def test_fp8_shared_prefix_cascade():
    """The shared-prefix decode on FP8 pools through the one-launch cascade."""
    check(synthetic.config_shared_prefix_fp8(), cascade=True, label="fp8 cascade")


@pytest.mark.parametrize("num_cus", [8, 256])
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_fp8_cascade_groups(num_cus, q_scale):
    """test_cascade_groups' batch (two groups split by a chunk row, a shared range ending
    inside a step, a one-token suffix) on FP8 pools."""
    wl = synthetic.build_fp8("fp8_cascade_groups", 73, 32, 8, qo_len=[1, 1, 1, 1, 1, 20, 1, 1, 1],
                             kv_len=[1125, 1300, 1500, 1121, 1700, 1250, 1136, 1400, 2000], num_blocks=700,
                             shared_prefix_blocks=70, q_scale=q_scale)
    check(wl, cascade=True, num_cus=num_cus, label=f"fp8 cascade q*{q_scale:g}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (24, 8), (48, 8), (8, 1)])
@pytest.mark.parametrize("case", ["mixed", "chunks8", "chunks16", "cascade"])
def test_gqa_ratios_fp8(hq, hkv, case):
    """FP8 pools at other grouped-query ratios: decode rows, chunk tiles of 128 / 64 / 32
    rows, the cascade with its 32 / 64-row prefix tiles."""
    wl = _gqa(case, hq, hkv, fp8=True)
    check(wl, split_blocks=5, cascade=case == "cascade", label=f"G={hq // hkv} fp8")
    if case != "cascade":
        check(wl, prefill_splits=3, label=f"G={hq // hkv} fp8 psplit 3")


def _represented_bf16(wl, kp8, vp8):
    """The bf16 workload that holds what FP8 pools kp8 / vp8 (after the append) represent:
    pools of code * scale, and new rows equal to the represented values at their slots, so
    that its own append leaves exactly those pools."""
    import dataclasses
    from synthetic import f32_to_bf16_bits
    kb = f32_to_bf16_bits((oracle.decode_e4m3(kp8) * wl.k_scale).astype(np.float32)).reshape(kp8.shape)
    vb = f32_to_bf16_bits((oracle.decode_e4m3(vp8) * wl.v_scale).astype(np.float32)).reshape(vp8.shape)
    blk, off = wl.slot_mapping // wl.block_size, wl.slot_mapping % wl.block_size
    return dataclasses.replace(wl, name=wl.name + "_as_bf16", kv_format="bf16", k_pool=kb, v_pool=vb,
                               k_new=np.ascontiguousarray(kb[blk, :, off]),
                               v_new=np.ascontiguousarray(vb[blk, :, off]), k_scale=1.0, v_scale=1.0)


@pytest.mark.parametrize("case", ["decode", "chunks8", "chunks16", "chunks128", "cascade"])
def test_fp8_equals_bf16_on_represented_values_bit_exact(case):
    """With power-of-two scales every represented value is a bf16 number and scaling by the
    scale is exact, so the FP8 path (codes widened to bf16, K scale folded into the score
    scale, V scale into the normalisation) must give the bf16 path's bits over pools of the
    represented values: decode rows split and not, chunk tiles of 32 / 64 / 128 rows with
    and without key splits, the cascade."""
    kw = dict(num_blocks=300, k_scale=0.5, v_scale=0.125)
    chunk_runs = [dict(), dict(prefill_splits=3, split_blocks=2)]
    if case == "decode":
        wl = synthetic.build_fp8("fp8_eq", 41, 32, 8, qo_len=[1] * 5, kv_len=[1, 17, 300, 1000, 2500], **kw)
        runs = [dict(), dict(split_blocks=3)]
    elif case == "chunks8":
        wl = synthetic.build_fp8("fp8_eq", 42, 32, 8, qo_len=[1, 8, 5, 8], kv_len=[500, 800, 100, 8], **kw)
        runs = chunk_runs
    elif case == "chunks16":
        wl = synthetic.build_fp8("fp8_eq", 43, 32, 8, qo_len=[16, 1, 11], kv_len=[700, 90, 1100], **kw)
        runs = chunk_runs
    elif case == "chunks128":
        wl = synthetic.build_fp8("fp8_eq", 44, 32, 8, qo_len=[1, 100, 3, 40], kv_len=[500, 900, 3, 1300], **kw)
        runs = chunk_runs
    else:
        wl = synthetic.build_fp8("fp8_eq", 45, 32, 8, qo_len=[1] * 6, kv_len=[700, 820, 990, 640, 777, 1000],
                                 num_blocks=200, shared_prefix_blocks=30, k_scale=2.0, v_scale=0.25)
        runs = [dict(cascade=True), dict(cascade=True, num_cus=8)]
    for kw_run in runs:
        print(f"[gpu] fp8 == bf16 {case} {kw_run}", flush=True)
        kp8, vp8, out8, lse8 = _run_gpu(wl, **kw_run)
        okp, ovp, _ = oracle.run_workload(wl)
        assert np.array_equal(kp8, okp) and np.array_equal(vp8, ovp), "append is not bit-exact"
        bw = _represented_bf16(wl, kp8, vp8)
        kpb, vpb, outb, lseb = _run_gpu(bw, **kw_run)
        assert np.array_equal(outb, out8), f"outputs differ in {np.count_nonzero(outb != out8)} places"
        assert np.array_equal(lseb.view(np.uint32), lse8.view(np.uint32))


def test_fp8_append_special_values_bit_exact():
    """The append on special inputs: NaN (stored as the NaN code 0x7F), +-inf and values
    far past 448 * scale (saturated to +-448), +-0, values in the subnormal range and
    exact midpoints between codes (ties to even), both pools compared whole."""
    import torch
    import paged_kv_attention_04_amd as pa
    from synthetic import f32_to_bf16_bits
    rng = np.random.default_rng(23)
    nb, Hkv, B, D, n = 40, 2, 16, 128, 37
    kp = rng.integers(0, 256, (nb, Hkv, B, D), dtype=np.uint8)
    vp = rng.integers(0, 256, (nb, Hkv, B, D), dtype=np.uint8)
    special = np.array([np.nan, -np.nan, np.inf, -np.inf, 1e30, -1e30, 0.0, -0.0, 2.0**-12, -2.0**-10,
                        3 * 2.0**-11, 2.5, 2.75, 448.0, 480.0], np.float32)
    vals = rng.standard_normal((n, Hkv, D)).astype(np.float32) * 50.0
    vals.reshape(-1)[rng.choice(vals.size, 800, replace=False)] = np.resize(special, 800)
    k_new = f32_to_bf16_bits(vals)
    v_new = f32_to_bf16_bits(vals[::-1].copy())
    slots = rng.choice(nb * B, n, replace=False).astype(np.int32)
    slots[3] = -1                                         # skipped
    g = pa.Geometry.make(8, Hkv, nb)
    for k_scale, v_scale in ((1.0, 1.0), (0.25, 3.0)):
        okp, ovp = oracle.append_fp8(kp, vp, k_new, v_new, slots, Hkv, D, B, nb, k_scale, v_scale)
        dk, dv = pa.to_device(kp), pa.to_device(vp)
        pa.pa_append_kv_fp8(g, dk, dv, pa.to_device(k_new), pa.to_device(v_new), pa.to_device(slots), k_scale, v_scale)
        torch.cuda.synchronize()
        assert np.array_equal(dk.cpu().numpy(), okp) and np.array_equal(dv.cpu().numpy(), ovp)


def _fp8_step_gpu(wl, split_blocks=0, prefill_splits=0, cascade=False):
    """pa_decode_step_fp8 (decode-only batches) or pa_attention_step_fp8 on device copies of
    an FP8 workload; returns host (k_pool, v_pool, out, lse)."""
    import torch
    import paged_kv_attention_04_amd as pa
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256, split_blocks, prefill_splits)
    if cascade:
        pa.pa_plan_shared_prefix(g, plan, wl.qo_len, wl.kv_len, wl.block_tables)
        assert plan.num_prefix_groups >= 1
    kp, vp = pa.to_device(wl.k_pool), pa.to_device(wl.v_pool)
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    step = pa.pa_decode_step_fp8 if plan.num_prefill_rows == 0 else pa.pa_attention_step_fp8
    step(g, plan, pa.to_device(wl.q), kp, vp, pa.to_device(wl.k_new), pa.to_device(wl.v_new),
         pa.to_device(wl.block_tables), pa.to_device(wl.qo_indptr), pa.to_device(wl.kv_len), out, lse,
         pa.workspace_for(plan), wl.k_scale, wl.v_scale)
    torch.cuda.synchronize()
    return kp.cpu().numpy(), vp.cpu().numpy(), out.cpu().numpy().view(np.uint16), lse.cpu().numpy()


@pytest.mark.parametrize("case", ["tiny", "qwen3", "split7", "split1", "cascade", "mixed", "chunks8", "chunks16",
                                  "psplit3", "cascade_mixed", "special"])
def test_fp8_fused_steps_match_append_then_attention(case):
    """The FP8 steps with the append fused into the attention launches: the pools the
    oracle's append gives (bit for bit, NaN-coded poison included) and the same output and
    LSE bits as pa_append_kv_fp8 followed by pa_attention_batch_fp8, on decode rows (split
    and not, the cascade) and chunk rows of every tile shape (key splits, a shared-prefix
    group beside them); 'special' puts NaN-free extremes (saturating and tiny values) in
    the new rows."""
    split = {"split7": 7, "split1": 1}.get(case, 0)
    psplit = 3 if case == "psplit3" else 0
    cascade = case in ("cascade", "cascade_mixed")
    b = synthetic.build_fp8
    wl = {"tiny": lambda: synthetic.config_tiny_fp8(seed=61),
          "qwen3": lambda: synthetic.config_decode_fp8(num_reqs=12),
          "split7": lambda: synthetic.config_tiny_fp8(seed=62),
          "split1": lambda: b("fp8_fused_split1", 63, 32, 8, qo_len=[1] * 3, kv_len=[1, 17, 300], num_blocks=40),
          "cascade": lambda: b("fp8_fused_cascade", 64, 32, 8, qo_len=[1] * 5, kv_len=[700, 820, 990, 640, 777],
                               num_blocks=400, shared_prefix_blocks=30),
          "mixed": lambda: b("fp8_fused_mixed", 65, 32, 8, qo_len=[1, 77, 1, 33], kv_len=[300, 2113, 17, 33],
                             num_blocks=300),
          "chunks8": lambda: b("fp8_fused_c8", 66, 32, 8, qo_len=[8, 3, 1, 8], kv_len=[520, 40, 100, 8], num_blocks=90),
          "chunks16": lambda: b("fp8_fused_c16", 67, 32, 8, qo_len=[16, 12, 1], kv_len=[700, 90, 300], num_blocks=90),
          "psplit3": lambda: b("fp8_fused_psplit", 68, 32, 8, qo_len=[1, 40, 1, 70, 2], kv_len=[300, 500, 17, 70, 33],
                               num_blocks=200),
          "cascade_mixed": lambda: b("fp8_fused_cascade_mixed", 69, 32, 8, qo_len=[1, 1, 1, 1, 33],
                                     kv_len=[700, 820, 990, 640, 900], num_blocks=400, shared_prefix_blocks=30),
          "special": lambda: b("fp8_fused_special", 70, 32, 8, qo_len=[1, 20, 1], kv_len=[300, 400, 50],
                               num_blocks=80, k_scale=2.0 ** -8, v_scale=7.3)}[case]()
    print(f"[gpu] fp8 fused step {case} R={wl.num_reqs} total_q={wl.total_q}", flush=True)
    kp, vp, out, lse = _fp8_step_gpu(wl, split, psplit, cascade)
    okp, ovp, ref = oracle.run_workload(wl, want_f64=True)
    assert np.array_equal(kp, okp) and np.array_equal(vp, ovp), "fused append is not bit-exact"
    eo, el = _errors(out, lse, ref)
    print(f"[gpu]   max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE
    _, _, out2, lse2 = _run_gpu(wl, split, psplit, cascade=cascade)
    assert np.array_equal(out, out2), f"outputs differ in {np.count_nonzero(out != out2)} places"
    assert np.array_equal(lse.view(np.uint32), lse2.view(np.uint32))


def _q8_step_gpu(wl, split_blocks=0, prefill_splits=0, cascade=False):
    """pa_decode_step_q8 (decode-only batches) or pa_attention_step_q8 on a device copy of
    a q8_0 workload; returns host (kv_pool, out, lse)."""
    import torch
    import paged_kv_attention_04_amd as pa
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256, split_blocks, prefill_splits)
    if cascade:
        pa.pa_plan_shared_prefix(g, plan, wl.qo_len, wl.kv_len, wl.block_tables, q8=True)
        assert plan.num_prefix_groups >= 1
    kvp = pa.to_device(wl.kv_pool)
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    step = pa.pa_decode_step_q8 if plan.num_prefill_rows == 0 else pa.pa_attention_step_q8
    step(g, plan, pa.to_device(wl.q), kvp, pa.to_device(wl.k_new), pa.to_device(wl.v_new),
         pa.to_device(wl.block_tables), pa.to_device(wl.qo_indptr), pa.to_device(wl.kv_len), out, lse,
         pa.workspace_for(plan))
    torch.cuda.synchronize()
    return kvp.cpu().numpy(), out.cpu().numpy().view(np.uint16), lse.cpu().numpy()


@pytest.mark.parametrize("case", ["tiny", "qwen3", "split7", "split1", "cascade", "mixed", "chunks", "psplit3",
                                  "cascade_mixed", "gqa"])
def test_q8_fused_steps_match_append_then_attention(case):
    """The q8_0 steps with the append fused into the attention launches: the pool the
    oracle's append gives (codes and scales, bit for bit, poisoned slots included) and the
    same output and LSE bits as pa_append_kv_q8 followed by pa_attention_batch_q8, on
    decode rows (split and not, the cascade) and chunk rows (key splits, a shared-prefix
    group beside them, other query-head ratios)."""
    split = {"split7": 7, "split1": 1}.get(case, 0)
    psplit = 3 if case == "psplit3" else 0
    cascade = case in ("cascade", "cascade_mixed")
    b = synthetic.build_q8
    wl = {"tiny": lambda: synthetic.config_tiny_q8(seed=81),
          "qwen3": lambda: synthetic.config_decode_q8(num_reqs=12),
          "split7": lambda: synthetic.config_tiny_q8(seed=82),
          "split1": lambda: b("q8_fused_split1", 83, 32, 8, qo_len=[1] * 3, kv_len=[1, 17, 300], num_blocks=40),
          "cascade": lambda: b("q8_fused_cascade", 84, 32, 8, qo_len=[1] * 5, kv_len=[700, 820, 990, 640, 777],
                               num_blocks=400, shared_prefix_blocks=30),
          "mixed": lambda: b("q8_fused_mixed", 85, 32, 8, qo_len=[1, 77, 1, 33], kv_len=[300, 2113, 17, 33],
                             num_blocks=300),
          "chunks": lambda: b("q8_fused_chunks", 86, 32, 8, qo_len=[8, 3, 1, 16, 2], kv_len=[520, 40, 100, 700, 2],
                              num_blocks=120),
          "psplit3": lambda: b("q8_fused_psplit", 87, 32, 8, qo_len=[1, 40, 1, 70, 2], kv_len=[300, 500, 17, 70, 33],
                               num_blocks=200),
          "cascade_mixed": lambda: b("q8_fused_cascade_mixed", 88, 32, 8, qo_len=[1, 1, 1, 1, 33],
                                     kv_len=[700, 820, 990, 640, 900], num_blocks=400, shared_prefix_blocks=30),
          "gqa": lambda: b("q8_fused_gqa", 89, 24, 8, qo_len=[1, 20, 1], kv_len=[300, 400, 50], num_blocks=80)}[case]()
    print(f"[gpu] q8_0 fused step {case} R={wl.num_reqs} total_q={wl.total_q}", flush=True)
    kvp, out, lse = _q8_step_gpu(wl, split, psplit, cascade)
    okvp, _, ref = oracle.run_workload(wl, want_f64=True)
    assert np.array_equal(kvp, okvp), "fused append is not bit-exact"
    eo, el = _errors(out, lse, ref)
    print(f"[gpu]   max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE
    _, _, out2, lse2 = _run_gpu(wl, split, psplit, cascade=cascade)
    assert np.array_equal(out, out2), f"outputs differ in {np.count_nonzero(out != out2)} places"
    assert np.array_equal(lse.view(np.uint32), lse2.view(np.uint32))


def test_fp8_copy_blocks_bit_exact():
    import torch
    import paged_kv_attention_04_amd as pa
    rng = np.random.default_rng(19)
    nb, Hkv, B, D = 300, 8, 16, 128
    kp = rng.integers(0, 256, (nb, Hkv, B, D), dtype=np.uint8)
    vp = rng.integers(0, 256, (nb, Hkv, B, D), dtype=np.uint8)
    perm = rng.permutation(nb)
    src = np.concatenate([perm[:40], [-1, 3]]).astype(np.int32)
    dst = np.concatenate([perm[40:80], [5, nb]]).astype(np.int32)
    g = pa.Geometry.make(32, Hkv, nb)
    okp, ovp = oracle.copy_blocks_fp8(kp, vp, src, dst, Hkv, D, B, nb)
    dk, dv = pa.to_device(kp), pa.to_device(vp)
    pa.pa_copy_blocks_fp8(g, dk, dv, pa.to_device(src), pa.to_device(dst))
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), okp) and np.array_equal(dv.cpu().numpy(), ovp)


# ------------------------------------------------------------------ randomised batches

def _random_batch(seed):
    """A seeded random batch: 1-24 rows, a mix of decode rows and chunk rows (2-100 new
    tokens), contexts up to ~2600 tokens, sometimes a shared prefix, random split
    overrides, and which path runs it."""
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.integers(1, 25))
    decode_only = rng.random() < 0.5
    qo = [1 if (decode_only or rng.random() < 0.6) else int(rng.integers(2, 101)) for _ in range(R)]
    shared = int(rng.choice([0, 0, 17, 40])) if R > 1 else 0
    kv = [int(max(q, shared * 16 + 1 + rng.integers(0, 2600 - shared * 16))) for q in qo]
    kv = [max(k, q + shared * 16) for k, q in zip(kv, qo)]     # new tokens never land in shared blocks
    nb = sum(-(-k // 16) for k in kv) + 16
    wl = synthetic.build(f"random{seed}", 2000 + seed, 32, 8, qo_len=qo, kv_len=kv, num_blocks=nb,
                         shared_prefix_blocks=shared, poison=True)
    split = int(rng.choice([0, 0, 1, 3, 16]))
    psplit = int(rng.choice([0, 0, 1, 2, 5]))
    cascade = bool(shared and decode_only and rng.random() < 0.7)
    return wl, split, psplit, cascade, decode_only, rng


@pytest.mark.parametrize("seed", range(16))
def test_random_batches(seed):
    wl, split, psplit, cascade, decode_only, rng = _random_batch(seed)
    print(f"[gpu] random batch {seed}: R={wl.num_reqs} qo={list(wl.qo_len)[:6]}.. kv_max={int(wl.kv_len.max())} "
          f"shared={wl.shared_prefix_blocks} split={split} psplit={psplit} cascade={cascade}", flush=True)
    check(wl, split_blocks=split, prefill_splits=psplit, cascade=cascade, label=f"random {seed}")
    if decode_only:
        kp, vp, out, lse = _decode_step_gpu(wl, split, cascade)          # the fused step, same bits
        _, _, out2, lse2 = _run_gpu(wl, split, cascade=cascade)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    q8 = synthetic.build_q8(f"random{seed}_q8", 3000 + seed, 32, 8, qo_len=list(wl.qo_len), kv_len=list(wl.kv_len),
                            num_blocks=wl.num_blocks, shared_prefix_blocks=wl.shared_prefix_blocks)
    check(q8, split_blocks=split, prefill_splits=psplit, cascade=cascade, label=f"random {seed} q8_0")
    f8 = synthetic.build_fp8(f"random{seed}_fp8", 5000 + seed, 32, 8, qo_len=list(wl.qo_len), kv_len=list(wl.kv_len),
                             num_blocks=wl.num_blocks, shared_prefix_blocks=wl.shared_prefix_blocks,
                             k_scale=float(rng.choice([0.03, 0.375, 2.5])), v_scale=float(rng.choice([0.05, 0.5])))
    check(f8, split_blocks=split, prefill_splits=psplit, cascade=cascade, label=f"random {seed} fp8")
