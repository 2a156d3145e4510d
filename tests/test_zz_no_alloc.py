"""pa_attention_batch_noalloc against pa_attention_batch (with a caller workspace) and the
oracle: two calls in a row on the library's per-device scratch array, the second with a
smaller batch, so the second call runs on what the first one left behind."""
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


def _run_both(wl, split_blocks, prefill_splits, cascade):
    """Append the new tokens, then attend twice on the same inputs: through the caller-
    workspace entry and through the scratch entry.  Returns host (out, lse) of each and
    the plan."""
    import torch
    import paged_kv_attention_04_amd as pa
    g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
    plan = pa.pa_plan(g, wl.qo_len, wl.kv_len, 256, split_blocks, prefill_splits)
    if cascade:
        pa.pa_plan_shared_prefix(g, plan, wl.qo_len, wl.kv_len, wl.block_tables, 256)
    d = {k: pa.to_device(getattr(wl, k)) for k in ("k_pool", "v_pool", "q", "block_tables", "qo_indptr", "kv_len",
                                                   "slot_mapping", "k_new", "v_new")}
    pa.pa_append_kv(g, d["k_pool"], d["v_pool"], d["k_new"], d["v_new"], d["slot_mapping"])
    res = []
    for noalloc in (False, True):
        out = torch.full((wl.total_q, wl.num_q_heads, wl.head_dim), -1, dtype=torch.int16, device="cuda")
        lse = torch.full((wl.total_q, wl.num_q_heads), -7.0, dtype=torch.float32, device="cuda")
        if noalloc:
            pa.pa_attention_batch_noalloc(g, plan, d["q"], d["k_pool"], d["v_pool"], d["block_tables"],
                                          d["qo_indptr"], d["kv_len"], out, lse)
        else:
            pa.pa_attention_batch(g, plan, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["qo_indptr"],
                                  d["kv_len"], out, lse, pa.workspace_for(plan))
        torch.cuda.synchronize()
        res.append((out.cpu().numpy().view(np.uint16), lse.cpu().numpy()))
    return res, plan


def _check_against_oracle(wl, out, lse):
    """The bars against the oracle's exact (fp64) outputs and LSE."""
    _, _, ref = oracle.run_workload(wl, want_f64=True)
    got = bf16_bits_to_f32(out).astype(np.float64)
    assert not np.isnan(got).any()
    eo = float(np.max(np.abs(got - ref["out_f64"])))
    el = float(np.max(np.abs(lse.astype(np.float64) - ref["lse_f64"])))
    print(f"[gpu]   vs oracle max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE


def test_noalloc_two_calls_match_workspace_entry():
    import paged_kv_attention_04_amd as pa
    # call 1: decode splits, prefill key splits and a shared-prefix group all use the scratch
    big = synthetic.build("noalloc_big", 85, 32, 8, qo_len=[1, 40, 1, 1, 1, 1], kv_len=[900, 1200, 1500, 2300, 1600, 700],
                          num_blocks=700, shared_prefix_blocks=40)
    # call 2: a smaller batch (8 query / 2 KV heads, split decode rows only)
    small = synthetic.config_tiny(seed=86)
    for wl, split, psplit, cascade in ((big, 20, 2, True), (small, 3, 0, False)):
        print(f"[gpu] noalloc {wl.name} R={wl.num_reqs} split={split} psplit={psplit} cascade={cascade}", flush=True)
        (ref, got), plan = _run_both(wl, split, psplit, cascade)
        assert 0 < plan.workspace_bytes <= pa.PA_NOALLOC_SCRATCH_BYTES
        assert plan.max_splits > 1
        if cascade:
            assert plan.num_prefix_groups == 1 and plan.prefill_splits == 2
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), \
            "scratch entry differs from the workspace entry"
        _check_against_oracle(wl, *got)


def test_noalloc_rejects_plans_beyond_the_scratch():
    """A plan whose partials exceed the scratch array returns PA_ERR_WORKSPACE before any
    launch (the outputs keep their sentinel values)."""
    import torch
    import paged_kv_attention_04_amd as pa
    g = pa.Geometry.make(32, 8, 64)
    plan = pa.pa_plan(g, [512], [4608], 256, 0, 64)        # 16 tiles x 8 heads x 64 splits of 64 KiB
    assert plan.workspace_bytes > pa.PA_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.int16, device="cuda")
    ints = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    out = torch.full((512, 32, 128), -1, dtype=torch.int16, device="cuda")
    lse = torch.full((512, 32), -7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(pa.PaError, match="WORKSPACE"):
        pa.pa_attention_batch_noalloc(g, plan, dummy, dummy, dummy, ints, ints, ints, out, lse)
    torch.cuda.synchronize()
    assert bool((out == -1).all()) and bool((lse == -7.0).all())
