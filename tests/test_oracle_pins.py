"""Pins for the CPU oracle: checks against what the pages print and what the
mathematics fixes, never against the oracle's own formula retyped.

Page A = AI-infra book ch. 8 "Inference optimisation"; page B = serving tutorial,
section "PagedAttention: KV cache in pages".  Printed values live in
tests/golden/pages_worked_examples.json with their citations.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from synthetic import bf16_bits_to_f32, f32_to_bf16_bits

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_examples.json")))
rng = np.random.default_rng(12345)


def _bf16(shape, scale=1.0, gen=None):
    g = gen or rng
    return f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32) * np.float32(scale))


def _contiguous_case(Hq, Hkv, D, qo, kv, B=16, seed=0, scale=None):
    """A single request whose blocks are physical blocks 0..n-1 in order (no paging),
    so that dense attention over the first kv positions is the reference."""
    g = np.random.default_rng(seed)
    nb = -(-kv // B)
    kp = np.full((nb + 1, Hkv, B, D), synthetic.BF16_NAN, np.uint16)   # one spare poisoned block
    kd, vd = _bf16((kv, Hkv, D), gen=g), _bf16((kv, Hkv, D), gen=g)
    vp = kp.copy()
    for j in range(kv):
        kp[j // B, :, j % B] = kd[j]
        vp[j // B, :, j % B] = vd[j]
    q = _bf16((qo, Hq, D), gen=g)
    bt = np.arange(nb, dtype=np.int32)[None, :]
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    return dict(q=q, kd=kd, vd=vd, kp=kp, vp=vp, bt=bt, scale=sc, nblocks=nb + 1)


def _run(c, Hq, Hkv, D, qo, kv, B=16, want_f64=True):
    return oracle.attention(c["q"], c["kp"], c["vp"], c["bt"], [qo], [kv], Hq, Hkv, D, B, c["nblocks"],
                            c["scale"], want_f64=want_f64)


# ---------------------------------------------------------------- geometry / capacity pins

def test_kv_bytes_per_token_closed_form():
    """k = 2 x 36 x 8 x 128 x 2 = 147,456 bytes (page A, section 8.1.2), measured as the
    bytes one oracle append changes in a one-layer pool, times the layer count."""
    g = GOLD["kv_bytes_per_token"]
    geo = synthetic.QWEN3_8B
    assert (geo["num_layers"], geo["num_kv_heads"], geo["head_dim"], geo["dtype_bytes"]) == \
        (g["layers"], g["kv_heads"], g["head_dim"], g["bytes"])
    Hkv, D, B = geo["num_kv_heads"], geo["head_dim"], 16
    kp = np.zeros((4, Hkv, B, D), np.uint16)
    vp = np.zeros_like(kp)
    kn = np.full((1, Hkv, D), 0xFFFF, np.uint16)
    k2, v2 = oracle.append(kp, vp, kn, kn, [2 * B + 5], Hkv, D, B, 4)
    changed = int((k2 != kp).sum() + (v2 != vp).sum()) * geo["dtype_bytes"]
    assert changed == 4096
    assert changed * geo["num_layers"] == g["value"] == 147456


def test_pool_blocks_for_12gib():
    # 12 GiB / (36 layers x 16 tokens x 4096 B per token-layer) blocks per layer
    assert synthetic.POOL_BLOCKS_12GIB == 5461
    assert synthetic.POOL_BLOCKS_12GIB * 16 == 87376


def test_capacity_table():
    """Page A, section 8.1.2 table and section 8.3.2: allocation in 16-token blocks at
    144 KiB per token; shared 6144-token prefix stored once."""
    c = GOLD["capacity"]
    kib = GOLD["kv_bytes_per_token"]["value"] // 1024
    nb = lambda L: -(-L // 16)
    assert c["short_in"] + c["out"] - 1 == c["short_tokens"]
    assert nb(c["short_tokens"]) * 16 == c["short_alloc_tokens"]
    assert nb(c["long_tokens"]) * 16 == c["long_alloc_tokens"]
    assert c["short_in"] * kib // 1024 == c["short_mib_after_prefill"]
    assert c["long_in"] * kib // 1024 == c["long_mib_after_prefill"]
    assert c["short_alloc_tokens"] * kib // 1024 == c["short_mib"]
    assert c["long_alloc_tokens"] * kib // 1024 == c["long_mib"]
    assert c["pool_mib"] // c["short_mib"] == c["fit_short"]
    assert c["pool_mib"] // c["long_mib"] == c["fit_long"]
    # Shared prefix through the harness allocator: 16 long requests whose first 384
    # blocks alias one set of physical blocks.
    prefix_blocks = c["prefix_tokens"] // 16
    bt = synthetic.place_blocks(np.random.default_rng(0), 6000, [nb(c["long_tokens"])] * 16, prefix_blocks)
    unique = len(set(bt.ravel().tolist()) - {-1})
    assert prefix_blocks * 16 * kib // 1024 == c["prefix_mib"]
    assert unique * 16 * kib // 1024 == c["shared_total_mib_16"]
    per_req = (nb(c["long_tokens"]) - prefix_blocks) * 16 * kib // 1024
    assert (c["pool_mib"] - c["prefix_mib"]) // per_req == c["fit_long_shared"]


def test_paging_example_and_sharing():
    """Page A, section 8.3.1: lengths 9, 13, 5, 15 in 4-token pages -> 52 slots (waste 22 -> 10);
    A and B sharing their first 8 tokens -> 44 slots."""
    e = GOLD["paging_example"]
    p = e["page"]
    nbs = [-(-L // p) for L in e["lengths"]]
    bt = synthetic.place_blocks(np.random.default_rng(1), 64, nbs)
    assert len(set(bt.ravel().tolist()) - {-1}) * p == e["paged_slots"]
    assert e["max_len"] * len(e["lengths"]) - sum(e["lengths"]) == e["waste_whole"]
    assert e["paged_slots"] - sum(e["lengths"]) == e["waste_paged"]
    # only A and B share: alias their first two blocks
    shared = e["shared_tokens_AB"] // p
    btab = synthetic.place_blocks(np.random.default_rng(2), 64, nbs[:2], shared)
    btcd = synthetic.place_blocks(np.random.default_rng(3), 64, nbs[2:])
    used = len(set(btab.ravel().tolist()) - {-1}) + len(set(btcd.ravel().tolist()) - {-1})
    assert used * p == e["paged_slots_shared"]
    assert e["reserved_whole"] == e["max_len"] * 4


def test_four_branches():
    """Page A, section 8.3.2: 4 x (95 + 9) = 416 references to 95 + 4 x 9 = 131 physical blocks."""
    b = GOLD["branches"]
    bt = synthetic.place_blocks(np.random.default_rng(4), 1000, [b["shared_blocks"] + b["own_blocks"]] * b["branches"],
                                b["shared_blocks"])
    assert int((bt >= 0).sum()) == b["references"]
    assert len(set(bt.ravel().tolist()) - {-1}) == b["physical"]


# ---------------------------------------------------------------- indexing pins

def test_tutorial_request_a_slots():
    """Page B diagram: request A has 40 tokens in blocks 7, 1, 3 (last one 8 of 16 used);
    so token 39 is slot 3*16 + 7 and tokens 0..15 live in block 7, which B also uses."""
    e = GOLD["tutorial_request_A"]
    bt = np.array(e["block_table"], np.int32)
    B = e["block_size"]
    slots = [oracle.slot(bt, p, B) for p in range(e["tokens"])]
    assert slots[:16] == list(range(7 * 16, 8 * 16))
    assert slots[16:32] == list(range(16, 32))
    assert slots[32:] == list(range(48, 48 + e["last_block_used"]))
    assert slots[-1] == 55
    assert -(-e["tokens"] // B) == len(bt)
    # oracle append of token 39 lands in physical block 3 at offset 7, nothing else changes
    kp = np.zeros((8, 2, B, 4), np.uint16)
    kn = np.arange(8, dtype=np.uint16).reshape(1, 2, 4) + 1
    k2, _ = oracle.append(kp, kp, kn, kn, [slots[-1]], 2, 4, B, 8)
    assert np.array_equal(k2[3, :, 7], kn[0])
    k2[3, :, 7] = 0
    assert not k2.any()


def test_append_skips_negative_slots_and_keeps_bytes():
    B, Hkv, D, nb = 16, 2, 8, 6
    kp = _bf16((nb, Hkv, B, D))
    vp = _bf16((nb, Hkv, B, D))
    kn, vn = _bf16((3, Hkv, D)), _bf16((3, Hkv, D))
    k2, v2 = oracle.append(kp, vp, kn, vn, [5, -1, 4 * B + 15], Hkv, D, B, nb)
    assert np.array_equal(k2[0, :, 5], kn[0]) and np.array_equal(v2[4, :, 15], vn[2])
    mask = np.ones(kp.shape, bool)
    mask[0, :, 5] = False
    mask[4, :, 15] = False
    assert np.array_equal(k2[mask], kp[mask]) and np.array_equal(v2[mask], vp[mask])
    with pytest.raises(ValueError):
        oracle.append(kp, vp, kn, vn, [nb * B], Hkv, D, B, nb)   # slot past the pool


def test_generator_chunks_consistent_with_oracle_append():
    one, chunks = synthetic.prompt_chunks(seed=9, prompt_len=96, chunk=32, num_q_heads=4, num_kv_heads=2,
                                          num_blocks=16)
    for a, b in zip(chunks[:-1], chunks[1:]):
        kp, vp = oracle.append(a.k_pool, a.v_pool, a.k_new, a.v_new, a.slot_mapping, 2, 128, 16, 16)
        assert np.array_equal(kp, b.k_pool) and np.array_equal(vp, b.v_pool)


# ---------------------------------------------------------------- causal-mask pins

@pytest.mark.parametrize("case", GOLD["causal_pairs"], ids=lambda c: f"c{c['c']}_h{c['h']}")
def test_causal_pair_count(case):
    """N_pair = ch + c(c+1)/2 (page A, section 8.2.3), counted by the oracle's own loop."""
    c, h = case["c"], case["h"]
    D = 8
    kv = c + h
    nb = -(-kv // 16)
    q = np.zeros((c, 1, D), np.uint16)
    kp = np.zeros((nb, 1, 16, D), np.uint16)
    bt = np.arange(nb, dtype=np.int32)[None]
    res = oracle.attention(q, kp, kp, bt, [c], [kv], 1, 1, D, 16, nb, 1.0)
    assert res["pairs"] == case["pairs"]


def test_chunked_pairs_sum_to_prompt_triangle():
    # four 512-token chunks of a 2048 prompt visit 2048*2049/2 pairs, as one shot does
    D, total = 4, 0
    for k in range(4):
        c, h = 512, 512 * k
        nb = (c + h) // 16
        res = oracle.attention(np.zeros((c, 1, D), np.uint16), np.zeros((nb, 1, 16, D), np.uint16),
                               np.zeros((nb, 1, 16, D), np.uint16), np.arange(nb, dtype=np.int32)[None],
                               [c], [c + h], 1, 1, D, 16, nb, 1.0)
        total += res["pairs"]
    assert total == 2048 * 2049 // 2 == 2098176


# ---------------------------------------------------------------- softmax / output pins

@pytest.mark.parametrize("Hq,Hkv,qo,kv", [(8, 2, 1, 17), (8, 2, 5, 40), (4, 4, 33, 33), (6, 3, 7, 70), (8, 1, 16, 16)])
def test_matches_torch_sdpa_dense(Hq, Hkv, qo, kv):
    """Brute force: with the blocks laid out in order, paged attention is dense scaled
    dot-product attention with a bottom-right causal mask and KV heads repeated over
    contiguous groups of query heads; torch's SDPA in float64 is the reference, and
    scipy's logsumexp of the masked scores pins the LSE."""
    from scipy.special import logsumexp
    D = 128
    c = _contiguous_case(Hq, Hkv, D, qo, kv, seed=Hq * 100 + kv)
    res = _run(c, Hq, Hkv, D, qo, kv)
    q = torch.from_numpy(bf16_bits_to_f32(c["q"]).astype(np.float64)).permute(1, 0, 2)      # [Hq][qo][D]
    k = torch.from_numpy(bf16_bits_to_f32(c["kd"]).astype(np.float64)).permute(1, 0, 2)     # [Hkv][kv][D]
    v = torch.from_numpy(bf16_bits_to_f32(c["vd"]).astype(np.float64)).permute(1, 0, 2)
    g = Hq // Hkv
    k = k.repeat_interleave(g, dim=0)
    v = v.repeat_interleave(g, dim=0)
    mask = torch.ones(qo, kv, dtype=torch.bool).tril(diagonal=kv - qo)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=c["scale"])
    got = torch.from_numpy(res["out_f64"]).permute(1, 0, 2)
    assert torch.allclose(got, ref, rtol=0, atol=1e-12)
    scores = (q @ k.transpose(1, 2)).numpy() * c["scale"]
    scores = np.where(mask.numpy()[None], scores, -np.inf)
    lse_ref = logsumexp(scores, axis=-1).T                                                   # [qo][Hq]
    assert np.allclose(res["lse_f64"], lse_ref, rtol=0, atol=1e-12)
    # the bf16 output is the double output rounded to nearest even
    assert np.array_equal(res["out"], oracle.round_bf16(res["out_f64"].ravel()).reshape(res["out"].shape))
    assert np.array_equal(res["lse"], res["lse_f64"].astype(np.float32))


def test_single_key_gives_v_and_scaled_dot():
    """kv_len = 1: the softmax weight is 1, so O = V exactly and LSE = scale * q.k."""
    Hq, Hkv, D = 4, 2, 128
    c = _contiguous_case(Hq, Hkv, D, 1, 1, seed=3)
    res = _run(c, Hq, Hkv, D, 1, 1)
    for h in range(Hq):
        kvh = h // (Hq // Hkv)
        assert np.array_equal(res["out"][0, h], c["vd"][0, kvh])
        qk = float(np.dot(bf16_bits_to_f32(c["q"][0, h]).astype(np.float64),
                          bf16_bits_to_f32(c["kd"][0, kvh]).astype(np.float64)))
        assert abs(res["lse_f64"][0, h] - c["scale"] * qk) < 1e-12


def test_identical_keys_give_mean_v():
    """All keys equal: uniform weights, O = mean(V) and LSE = scale*q.k + ln(n)."""
    Hq, Hkv, D, n = 2, 1, 128, 37
    c = _contiguous_case(Hq, Hkv, D, 1, n, seed=4)
    for j in range(n):
        c["kp"][j // 16, :, j % 16] = c["kd"][0]
    res = _run(c, Hq, Hkv, D, 1, n)
    mean_v = bf16_bits_to_f32(c["vd"]).astype(np.float64).mean(axis=0)          # [Hkv][D]
    for h in range(Hq):
        assert np.allclose(res["out_f64"][0, h], mean_v[0], rtol=0, atol=1e-13)
        qk = float(np.dot(bf16_bits_to_f32(c["q"][0, h]).astype(np.float64),
                          bf16_bits_to_f32(c["kd"][0, 0]).astype(np.float64)))
        assert abs(res["lse_f64"][0, h] - (c["scale"] * qk + math.log(n))) < 1e-12


def test_zero_scale_gives_mean_v():
    Hq, Hkv, D, n = 4, 2, 128, 50
    c = _contiguous_case(Hq, Hkv, D, 1, n, seed=5, scale=0.0)
    res = _run(c, Hq, Hkv, D, 1, n)
    mean_v = bf16_bits_to_f32(c["vd"]).astype(np.float64).mean(axis=0)
    for h in range(Hq):
        assert np.allclose(res["out_f64"][0, h], mean_v[h // 2], rtol=0, atol=1e-13)
        assert abs(res["lse_f64"][0, h] - math.log(n)) < 1e-12


def test_dominant_key_selects_its_value():
    """One key aligned with q and far larger than the rest takes all the weight."""
    Hq, Hkv, D, n = 1, 1, 128, 40
    c = _contiguous_case(Hq, Hkv, D, 1, n, seed=6)
    j0 = 23
    c["kp"][j0 // 16, 0, j0 % 16] = f32_to_bf16_bits(bf16_bits_to_f32(c["q"][0, 0]) * np.float32(4.0))
    res = _run(c, Hq, Hkv, D, 1, n)
    v0 = bf16_bits_to_f32(c["vp"][j0 // 16, 0, j0 % 16]).astype(np.float64)
    assert np.allclose(res["out_f64"][0, 0], v0, atol=1e-6)


# ---------------------------------------------------------------- invariants

def test_fig_8_10_block_table_equals_contiguous():
    """Page A fig. 8-10: logical blocks 0,1,2 in physical blocks 2,0,3 (block 1 free).
    Reading through the table gives the same result as reading the blocks in order;
    the free block holds NaN and is never read."""
    f = GOLD["fig_8_10"]
    Hq, Hkv, D, qo, kv = 4, 2, 128, 3, 40
    c = _contiguous_case(Hq, Hkv, D, qo, kv, seed=7)
    ref = _run(c, Hq, Hkv, D, qo, kv)
    kp = np.full((4, Hkv, 16, D), synthetic.BF16_NAN, np.uint16)
    vp = kp.copy()
    for logical, phys in enumerate(f["block_table"]):
        kp[phys] = c["kp"][logical]
        vp[phys] = c["vp"][logical]
    got = oracle.attention(c["q"], kp, vp, np.array([f["block_table"]], np.int32), [qo], [kv], Hq, Hkv, D, 16, 4,
                           c["scale"])
    assert f["free_block"] not in f["block_table"]
    assert np.array_equal(got["out"], ref["out"]) and np.array_equal(got["lse"], ref["lse"])


def test_block_permutation_invariance():
    wl = synthetic.config_tiny(seed=11)
    _, _, ref = oracle.run_workload(wl)
    perm = np.random.default_rng(5).permutation(wl.num_blocks).astype(np.int32)   # old -> new id
    kp = np.empty_like(wl.k_pool)
    vp = np.empty_like(wl.v_pool)
    kp[perm] = wl.k_pool
    vp[perm] = wl.v_pool
    bt = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    sm = (perm[wl.slot_mapping // 16] * 16 + wl.slot_mapping % 16).astype(np.int32)
    k2, v2 = oracle.append(kp, vp, wl.k_new, wl.v_new, sm, wl.num_kv_heads, 128, 16, wl.num_blocks)
    got = oracle.attention(wl.q, k2, v2, bt, wl.qo_len, wl.kv_len, wl.num_q_heads, wl.num_kv_heads, 128, 16,
                           wl.num_blocks, wl.scale)
    assert np.array_equal(got["out"], ref["out"]) and np.array_equal(got["lse"], ref["lse"])


def test_shared_prefix_equals_duplicated_blocks():
    """Page A section 8.3.2 (note on the four-branch run: shared branches give the same
    outputs): aliasing prefix blocks equals storing a private copy per request."""
    wl = synthetic.build("shared", 21, 8, 2, qo_len=[1, 1, 3], kv_len=[70, 90, 67], num_blocks=64,
                         shared_prefix_blocks=3)
    _, _, ref = oracle.run_workload(wl)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    bt = wl.block_tables.copy()
    free = sorted(set(range(wl.num_blocks)) - set(bt.ravel().tolist()))
    for r in range(1, wl.num_reqs):            # give requests 1.. their own copy of the prefix
        for b in range(3):
            new = free.pop()
            kp[new], vp[new] = kp[bt[r, b]], vp[bt[r, b]]
            bt[r, b] = new
    assert len(set(bt[:, :3].ravel().tolist())) == 3 * wl.num_reqs
    k2, v2 = oracle.append(kp, vp, wl.k_new, wl.v_new, wl.slot_mapping, 2, 128, 16, 64)
    got = oracle.attention(wl.q, k2, v2, bt, wl.qo_len, wl.kv_len, 8, 2, 128, 16, 64, wl.scale)
    assert np.array_equal(got["out"], ref["out"]) and np.array_equal(got["lse"], ref["lse"])


def test_shared_block_rows_coincide():
    """Page B diagram: B's table is [7], A's is [7, 1, 3].  The same prompt in block 7 gives B
    exactly A's first 16 outputs."""
    Hq, Hkv, D = 4, 2, 128
    g = np.random.default_rng(8)
    kp, vp = _bf16((8, Hkv, 16, D), gen=g), _bf16((8, Hkv, 16, D), gen=g)
    qa = _bf16((40, Hq, D), gen=g)
    q = np.concatenate([qa, qa[:16]])
    bt = np.array([[7, 1, 3], [7, -1, -1]], np.int32)
    res = oracle.attention(q, kp, vp, bt, [40, 16], [40, 16], Hq, Hkv, D, 16, 8, 1 / math.sqrt(D))
    assert np.array_equal(res["out"][40:], res["out"][:16])
    assert np.array_equal(res["lse"][40:], res["lse"][:16])


def test_chunked_prefill_equals_one_shot():
    """Page A section 8.2.3: a prompt processed in chunks attends exactly as in one shot."""
    one, chunks = synthetic.prompt_chunks(seed=10, prompt_len=200, chunk=64, num_q_heads=8, num_kv_heads=2,
                                          num_blocks=32)
    _, _, ref = oracle.run_workload(one)
    outs, lses = [], []
    for wl in chunks:
        _, _, r = oracle.run_workload(wl)
        outs.append(r["out"])
        lses.append(r["lse"])
    assert np.array_equal(np.concatenate(outs), ref["out"])
    assert np.array_equal(np.concatenate(lses), ref["lse"])


def test_poisoned_slots_never_read():
    wl = synthetic.config_tiny(seed=12)
    assert np.isnan(bf16_bits_to_f32(wl.k_pool)).any()
    _, _, res = oracle.run_workload(wl)
    assert not np.isnan(bf16_bits_to_f32(res["out"])).any()
    assert np.isfinite(res["lse"]).all()


def test_row_select_computes_only_selected():
    wl = synthetic.config_tiny(seed=13)
    _, _, full = oracle.run_workload(wl)
    sel = np.array([0, 1, 0, 1], np.uint8)
    _, _, part = oracle.run_workload(wl, row_select=sel)
    assert np.array_equal(part["out"][[1, 3]], full["out"][[1, 3]])
    assert not part["out"][[0, 2]].any()
    assert part["pairs"] == int(wl.kv_len[1] + wl.kv_len[3])


# ---------------------------------------------------------------- rounding pin

def test_round_bf16_matches_torch_on_float32_values():
    """For values exactly representable in float32, torch's float32 -> bfloat16 cast is a
    single round-to-nearest-even; the oracle's double -> bf16 must agree bit for bit."""
    g = np.random.default_rng(99)
    x = np.concatenate([g.standard_normal(20000), g.standard_normal(2000) * 1e-38, g.standard_normal(2000) * 1e30,
                        np.ldexp(1.0, np.arange(-140, 128)).astype(np.float64)]).astype(np.float32)
    bits = x.view(np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)                          # exact halfway cases
    x = np.concatenate([x, ties, -ties]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_double_only_cases():
    # 1 + 2^-8 is a tie -> even (1.0); a hair above rounds up; 1 + 3*2^-8 ties up to even
    assert oracle.round_bf16(1 + 2.0 ** -8)[0] == 0x3F80
    assert oracle.round_bf16(1 + 2.0 ** -8 + 2.0 ** -40)[0] == 0x3F81
    assert oracle.round_bf16(1 + 3 * 2.0 ** -8)[0] == 0x3F82
    assert oracle.round_bf16(-0.0)[0] == 0x8000
    assert oracle.round_bf16(2.0 ** -133)[0] == 0x0001
    assert oracle.round_bf16(2.0 ** 128)[0] == 0x7F80
    assert oracle.round_bf16(float("nan"))[0] == 0x7FC0


# ------------------------------------------------------------------ block copy (copy-on-write)

def test_copy_blocks_moves_whole_blocks_only():
    """Block src -> dst for every KV head, K and V; nothing else changes; an out-of-range
    pair is skipped; the inputs are not modified (checked with numpy indexing)."""
    rng = np.random.default_rng(3)
    nb, Hkv, B, D = 12, 2, 16, 128
    kp = rng.integers(0, 2**16, (nb, Hkv, B, D), dtype=np.uint16)
    vp = rng.integers(0, 2**16, (nb, Hkv, B, D), dtype=np.uint16)
    kp0, vp0 = kp.copy(), vp.copy()
    src, dst = np.array([3, 7, 0, 5], np.int32), np.array([9, 1, 11, 99], np.int32)
    k2, v2 = oracle.copy_blocks(kp, vp, src, dst, Hkv, D, B, nb)
    ek, ev = kp0.copy(), vp0.copy()
    for s_, d_ in zip(src[:3], dst[:3]):
        ek[d_], ev[d_] = kp0[s_], vp0[s_]
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
    assert np.array_equal(kp, kp0) and np.array_equal(vp, vp0)


def _cow_workload():
    # two decode rows share all three blocks; the third is partly filled (positions 32..38)
    # and both rows' new token (position 39) maps to the same slot of it
    wl = synthetic.build("cow", 9, 8, 2, qo_len=[1, 1], kv_len=[40, 40], num_blocks=16,
                         shared_prefix_blocks=3, poison=False)
    assert np.array_equal(wl.block_tables[0, :3], wl.block_tables[1, :3])
    assert wl.slot_mapping[0] == wl.slot_mapping[1]
    return wl


def _attend(wl, kp, vp, bt):
    return oracle.attention(wl.q, kp, vp, bt, wl.qo_len, wl.kv_len, wl.num_q_heads, wl.num_kv_heads,
                            wl.head_dim, wl.block_size, wl.num_blocks, wl.scale)


def _unshared_reference(wl):
    """Each request owns private blocks holding the same context; each appends its own token."""
    used = set(wl.block_tables[wl.block_tables >= 0].ravel().tolist())
    spare = [b for b in range(wl.num_blocks) if b not in used]
    kp, vp, bt = wl.k_pool.copy(), wl.v_pool.copy(), wl.block_tables.copy()
    for r in range(2):
        mine = spare[3 * r: 3 * r + 3]
        kp[mine], vp[mine] = wl.k_pool[bt[r, :3]], wl.v_pool[bt[r, :3]]
        bt[r, :3] = mine
        s = synthetic.slot_of(bt[r], 39, wl.block_size)
        kp[s // wl.block_size, :, s % wl.block_size] = wl.k_new[r]
        vp[s // wl.block_size, :, s % wl.block_size] = wl.v_new[r]
    return _attend(wl, kp, vp, bt)


def test_copy_on_write_gives_each_branch_its_own_token():
    """Book section 8.3.2: before a request writes into a physical block it shares, the
    block is copied and that request's table is pointed at the copy.  After the copy and
    both appends, each request's attention equals the one over a layout where nothing was
    shared; appending without the copy makes the two requests' tokens collide."""
    wl = _cow_workload()
    ref = _unshared_reference(wl)
    bt = wl.block_tables.copy()
    used = set(bt[bt >= 0].ravel().tolist())
    free = [b for b in range(wl.num_blocks) if b not in used][-1]
    kp, vp = oracle.copy_blocks(wl.k_pool, wl.v_pool, [int(bt[1, 2])], [free], wl.num_kv_heads, wl.head_dim,
                                wl.block_size, wl.num_blocks)
    bt[1, 2] = free
    slots = [synthetic.slot_of(bt[r], 39, wl.block_size) for r in range(2)]
    kp, vp = oracle.append(kp, vp, wl.k_new, wl.v_new, slots, wl.num_kv_heads, wl.head_dim, wl.block_size,
                           wl.num_blocks)
    res = _attend(wl, kp, vp, bt)
    assert np.array_equal(res["out"], ref["out"]) and np.array_equal(res["lse"], ref["lse"])
    # without the copy the second append overwrites the first request's token
    kp, vp = oracle.append(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping, wl.num_kv_heads,
                           wl.head_dim, wl.block_size, wl.num_blocks)
    bad = _attend(wl, kp, vp, wl.block_tables)
    assert not np.array_equal(bad["out"][0], ref["out"][0])


# ------------------------------------------------------------------ q8_0 KV pool

QWEN_KV_BYTES_PER_TOKEN_BF16 = 2 * 36 * 8 * 128 * 2      # K and V, 36 layers, 8 KV heads, d = 128, bf16


def test_q8_bytes_reproduce_the_pages_figures():
    """Book section 8.4.2 / fig. 8-23: a q8_0 group is 34 bytes against 64 for bf16.  The
    long request (8192 + 256 tokens, 1188 MiB in bf16) takes 631.125 MiB; an 8K context
    saves 540 MiB; 16 long requests take about 9.86 GiB."""
    tile = oracle.q8_tile_bytes(128, 16)
    assert tile == 2176 and synthetic.q8_tile_bytes(128, 16) == tile
    per_token_q8 = 2 * 36 * 8 * tile // 16
    assert per_token_q8 * 64 == QWEN_KV_BYTES_PER_TOKEN_BF16 * 34
    MiB = 2**20
    assert 8448 * QWEN_KV_BYTES_PER_TOKEN_BF16 == 1188 * MiB
    assert 8448 * per_token_q8 == 631.125 * MiB
    assert 8192 * QWEN_KV_BYTES_PER_TOKEN_BF16 - 8192 * per_token_q8 == 540 * MiB
    assert round(16 * 8448 * per_token_q8 / 2**30, 2) == 9.86


def test_float_to_half_matches_numpy():
    """binary32 -> binary16 to nearest even, against numpy's conversion: random finite bit
    patterns over the whole range, every tie between neighbouring halves, subnormals and
    the overflow edge."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    halves = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    ties = ((halves[:-1].astype(np.float64) + halves[1:].astype(np.float64)) / 2).astype(np.float32)
    edge = np.array([65504, 65519.996, 65520, 65536, 2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-14,
                     2.0**-14 - 2.0**-25, -0.0, 1e-30], np.float32)
    allv = np.concatenate([vals[:4000], ties, edge, -ties[:200]])
    with np.errstate(over="ignore"):
        want = allv.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(v) for v in allv], np.uint16)
    assert np.array_equal(got, want)


def test_half_to_double_matches_numpy():
    h = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16).astype(np.float64)
    for i in range(0, 2**16, 37):
        g = oracle.half_to_double(int(h[i]))
        assert (np.isnan(g) and np.isnan(f[i])) or g == f[i]


def test_q8_quantise_recovers_exact_groups():
    """A group whose values are integers c times 2^-5 with max |c| = 127 has scale exactly
    2^-5 and codes exactly c."""
    rng = np.random.default_rng(6)
    c = rng.integers(-127, 128, (50, 128))
    c[:, ::32] = np.where(rng.random((50, 4)) < 0.5, 127, -127)
    x = f32_to_bf16_bits((c * 2.0**-5).astype(np.float32))
    codes, scales = oracle.quantize_q8_rows(x, 128)
    assert np.array_equal(codes.astype(np.int64), c)
    assert np.all(scales == 0x2800)                    # binary16 of 2^-5


def test_q8_quantise_error_bound_and_edges():
    """Every value is within half a scale step of code * d; the largest magnitude of a
    group maps to +-127; an all-zero group has scale 0 and codes 0; a group beyond the
    binary16 range saturates at scale 65504."""
    rng = np.random.default_rng(7)
    mag = 10.0 ** rng.uniform(-3, 3, (400, 4, 1))
    x32 = (rng.standard_normal((400, 4, 32)) * mag).astype(np.float32).reshape(400, 128)
    x = f32_to_bf16_bits(x32)
    xv = bf16_bits_to_f32(x).astype(np.float64).reshape(400, 4, 32)
    codes, scales = oracle.quantize_q8_rows(x, 128)
    d = scales.view(np.float16).astype(np.float64)[..., None]
    rec = codes.reshape(400, 4, 32).astype(np.float64) * d
    assert np.all(np.abs(rec - xv) <= d / 2 + 1e-12 * np.abs(xv))
    assert np.all(np.abs(codes.reshape(400, 4, 32)).max(axis=2) == 127)
    z, zs = oracle.quantize_q8_rows(np.zeros(128, np.uint16), 128)
    assert not z.any() and not zs.any()
    big = f32_to_bf16_bits(np.full(128, 3e9, np.float32))
    bc, bs = oracle.quantize_q8_rows(big, 128)
    assert np.all(bs == 0x7BFF) and np.all(bc == 127)


def _dequantise(pool, which, Hkv, D=128, B=16):
    """numpy reading of the layout: pool [nb][Hkv][2][tile], `which` 0 = K, 1 = V; a tile is
    [B][D] int8 codes, then [B][D/32] binary16 scales."""
    nb = pool.shape[0]
    t = np.ascontiguousarray(pool.reshape(nb, Hkv, 2, -1)[:, :, which])
    codes = t[:, :, :B * D].reshape(nb, Hkv, B, D).view(np.int8).astype(np.float64)
    sc = np.ascontiguousarray(t[:, :, B * D:]).view(np.float16).reshape(nb, Hkv, B, D // 32).astype(np.float64)
    return codes * np.repeat(sc, 32, axis=3)


def test_q8_attention_equals_dense_softmax_on_dequantised_values():
    """Append (quantise) then attend, against a dense numpy softmax over the values the
    codes represent, gathered through the block table."""
    wl = synthetic.config_tiny_q8(poison=True)
    pool, _, res = oracle.run_workload(wl, want_f64=True)
    K, V = _dequantise(pool, 0, wl.num_kv_heads), _dequantise(pool, 1, wl.num_kv_heads)
    q = bf16_bits_to_f32(wl.q).astype(np.float64)
    g = wl.num_q_heads // wl.num_kv_heads
    for r in range(wl.num_reqs):
        L = int(wl.kv_len[r])
        blocks = wl.block_tables[r, :-(-L // 16)]
        for h in range(wl.num_q_heads):
            Kr = K[blocks, h // g].reshape(-1, 128)[:L]
            Vr = V[blocks, h // g].reshape(-1, 128)[:L]
            s = Kr @ q[r, h] * wl.scale
            lse = np.log(np.sum(np.exp(s - s.max()))) + s.max()
            o = np.exp(s - lse) @ Vr
            assert abs(res["lse_f64"][r, h] - lse) < 1e-12
            assert np.max(np.abs(res["out_f64"][r, h] - o)) < 1e-12


def test_q8_append_writes_exactly_the_quantised_rows():
    wl = synthetic.config_tiny_q8(poison=True)
    got = oracle.append_q8(wl.kv_pool, wl.k_new, wl.v_new, wl.slot_mapping, wl.num_kv_heads, 128, 16, wl.num_blocks)
    want = wl.kv_pool.copy()
    for which, new in ((0, wl.k_new), (1, wl.v_new)):
        codes, scales = oracle.quantize_q8_rows(new, 128)
        for t, s in enumerate(wl.slot_mapping):
            blk, off = divmod(int(s), 16)
            want[blk, :, which, off * 128:(off + 1) * 128] = codes[t].view(np.uint8)
            want[blk, :, which, 2048 + off * 8:2048 + off * 8 + 8] = scales[t].view(np.uint8).reshape(wl.num_kv_heads, 8)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ FP8 (E4M3) pool

def test_e4m3_decode_matches_torch_for_every_code():
    """All 256 codes against torch's float8_e4m3fn (the OCP E4M3 format): 448 at 0x7E, NaN at
    S.1111.111, subnormals k * 2^-9."""
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode_e4m3(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0**-9 and got[0x08] == 2.0**-6 and got[0x38] == 1.0


def test_e4m3_encode_matches_torch_and_saturates():
    """Encoding rounds to nearest with ties to even (torch's float -> float8_e4m3fn on every
    value up to 464, where torch's result is still finite, including every midpoint between
    neighbouring codes); magnitudes above 448 saturate to 448 (torch gives NaN past 464)."""
    rng = np.random.default_rng(21)
    vals = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.4, 20000),
                           np.linspace(-464, 464, 4001)])
    finite = oracle.decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (finite[:-1] + finite[1:]) / 2
    vals = np.concatenate([vals, mids, -mids, [0.0, -0.0, 448.0, -448.0, 2.0**-10, 3 * 2.0**-11]])
    vals = vals[np.abs(vals) <= 464]
    got = oracle.encode_e4m3(vals)
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    big = oracle.encode_e4m3([464.5, 500.0, 1e6, -1e30, np.inf, -np.inf])
    assert list(big) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    # a NaN (either sign) is stored as the NaN code 0x7F, which decodes to NaN
    nan_codes = oracle.encode_e4m3([np.nan, -np.nan, np.copysign(np.nan, -1.0)])
    assert list(nan_codes) == [0x7F, 0x7F, 0x7F]
    assert np.isnan(oracle.decode_e4m3(nan_codes)).all()


def test_fp8_bytes_are_half_of_bf16():
    """Book section 8.4.2: one byte per value against two; per token and layer of Qwen3-8B
    (8 KV heads x 128 dims, K and V) 4096 bytes against 8192, the byte ratio behind the
    pages' smaller per-token slope of the FP8 fit (2.37e-5 against 4.37e-5 ms per token)."""
    wl = synthetic.config_decode_fp8(poison=False)
    assert wl.k_pool.dtype == np.uint8 and wl.k_pool.shape == (synthetic.POOL_BLOCKS_12GIB, 8, 16, 128)
    per_token = 2 * 8 * 128
    assert per_token * 2 == QWEN_KV_BYTES_PER_TOKEN_BF16 // 36


def test_fp8_attention_equals_bf16_attention_on_the_represented_values():
    """With power-of-two scales every represented value code * scale is a bf16 value, so
    attention over the FP8 pools must equal the (pinned) bf16 definition over pools that hold
    those values, to the last bit of the fp64 result."""
    wl = synthetic.build_fp8("fp8_pin", 31, 8, 2, qo_len=[1, 5, 1], kv_len=[40, 70, 129], num_blocks=40,
                             poison=False, k_scale=0.5, v_scale=0.25)
    kp, vp, res = oracle.run_workload(wl, want_f64=True)
    kb = f32_to_bf16_bits((oracle.decode_e4m3(kp) * 0.5).astype(np.float32)).reshape(kp.shape)
    vb = f32_to_bf16_bits((oracle.decode_e4m3(vp) * 0.25).astype(np.float32)).reshape(vp.shape)
    ref = oracle.attention(wl.q, kb, vb, wl.block_tables, wl.qo_len, wl.kv_len, wl.num_q_heads, wl.num_kv_heads,
                           128, 16, wl.num_blocks, wl.scale, want_f64=True)
    assert np.array_equal(res["out_f64"], ref["out_f64"]) and np.array_equal(res["lse_f64"], ref["lse_f64"])


def test_fp8_append_stores_the_encoded_quotients():
    """Each new value x lands as encode(float32(x / scale)) at its slot; every other byte of
    the pools is unchanged; a value that is already code * scale round-trips exactly."""
    wl = synthetic.build_fp8("fp8_append", 32, 8, 2, qo_len=[1, 3], kv_len=[30, 50], num_blocks=12,
                             poison=True, k_scale=0.375, v_scale=3.0)
    kp, vp = oracle.append_fp8(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping, 2, 128, 16, 12,
                               wl.k_scale, wl.v_scale)
    wk, wv = wl.k_pool.copy(), wl.v_pool.copy()
    for t, s in enumerate(wl.slot_mapping):
        blk, off = divmod(int(s), 16)
        for new, want, sc in ((wl.k_new, wk, wl.k_scale), (wl.v_new, wv, wl.v_scale)):
            q = (bf16_bits_to_f32(new[t]) / np.float32(sc)).astype(np.float32)
            want[blk, :, off] = oracle.encode_e4m3(q.astype(np.float64).ravel()).reshape(2, 128)
    assert np.array_equal(kp, wk) and np.array_equal(vp, wv)
    # round trip of representable values (scale a power of two keeps them in bf16)
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    x = f32_to_bf16_bits((oracle.decode_e4m3(codes) * 2.0).astype(np.float32))
    x = np.concatenate([x, np.zeros(128 - x.size, np.uint16)])[None, None, :].repeat(2, axis=1)
    kp2, _ = oracle.append_fp8(np.zeros((1, 2, 16, 128), np.uint8), np.zeros((1, 2, 16, 128), np.uint8), x, x,
                               [0], 2, 128, 16, 1, 2.0, 2.0)
    assert np.array_equal(kp2[0, 0, 0, :codes.size], codes)
