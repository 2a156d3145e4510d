"""Seeded synthetic inputs for paged-KV attention workloads.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds none of the attention arithmetic: it only draws random numbers,
rounds them to bf16 bit patterns, places logical KV blocks in a physical
pool, and builds the block tables and slot mappings that an engine's KV
manager would hand to the attention layer.

Vocabulary follows the pages:
  * a sequence is cut into fixed-size blocks of ``block_size`` tokens; a
    per-request block table maps logical block -> physical block, and a new
    physical block may come from anywhere in the free pool (AI-infra book,
    ch. 8 "Inference optimisation", section 8.3.1, fig. 8-10; serving
    tutorial, section "PagedAttention: KV cache in pages", 16-token blocks);
  * a shared prefix is stored once and several block tables point at the
    same physical blocks (book section 8.3.1, fig. 8-13; section 8.3.2);
  * ``qo_len`` is the number of new (query) tokens of a row and ``kv_len``
    the number of KV entries it attends over, counted after this step's
    append (Perplexity blog on disaggregated prefill/decode, section on
    prefill vs decode performance: decode rows have qo_len = 1);
  * the pool is laid out HND inside a block: [block][kv_head][token][dim]
    (same blog, paragraph on NHD vs HND page layout).

Recipe (stated once, used everywhere): ``numpy.random.SeedSequence(seed)``
spawns independent PCG64 streams for lengths, placement, K/V context, new
tokens and Q; values are ``standard_normal`` float32 rounded to bf16 with
round-to-nearest-even; ``U[0,255]`` is an integer drawn uniformly from
0..255 inclusive.  Pool slots that hold no context token are poisoned with a
bf16 NaN when ``poison`` is set, so that any read of them shows up.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (round to nearest even).

    Only used to turn drawn normals into input bit patterns; the inputs never
    contain NaN or infinity, so no special case is needed for them.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One layer's worth of inputs for a mixed decode / chunked-prefill batch.

    Arrays hold bf16 data as uint16 bit patterns.
      q            [total_q][num_q_heads][head_dim]        rows ordered by request
      k_pool/v_pool [num_blocks][num_kv_heads][block_size][head_dim]  state BEFORE the append
      k_new/v_new  [n_new][num_kv_heads][head_dim]          the K/V of this step's new tokens
      slot_mapping [n_new] int32: block_id * block_size + offset of each new token
      block_tables [R][max_blocks] int32, -1 past a request's last block
    """

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    qo_len: np.ndarray
    kv_len: np.ndarray
    block_tables: np.ndarray
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    shared_prefix_blocks: int = 0
    notes: dict = field(default_factory=dict)
    kv_format: str = "bf16"
    # q8_0 only (k_pool / v_pool are then None): uint8 [num_blocks][num_kv_heads][2][q8_tile_bytes],
    # each (block, KV head) holding its K tile, then its V tile
    kv_pool: Optional[np.ndarray] = None
    # fp8 only: k_pool / v_pool are uint8 E4M3 codes in the bf16 layout; a value is code * scale
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_reqs(self) -> int:
        return int(self.qo_len.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.qo_len.sum())

    @property
    def qo_indptr(self) -> np.ndarray:
        out = np.zeros(self.num_reqs + 1, dtype=np.int32)
        np.cumsum(self.qo_len, out=out[1:])
        return out

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def unique_blocks(self) -> int:
        """Number of distinct physical blocks referenced (a shared prefix counts once)."""
        used = set()
        for r in range(self.num_reqs):
            nb = -(-int(self.kv_len[r]) // self.block_size)
            used.update(int(b) for b in self.block_tables[r, :nb])
        return len(used)


def _streams(seed: int, n: int = 6):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def slot_of(block_table_row: np.ndarray, pos: int, block_size: int) -> int:
    """Pool slot of logical position ``pos`` (engine bookkeeping, not attention)."""
    return int(block_table_row[pos // block_size]) * block_size + pos % block_size


def place_blocks(rng, num_blocks: int, blocks_per_req: List[int], shared_prefix_blocks: int = 0,
                 max_blocks: Optional[int] = None) -> np.ndarray:
    """Random physical placement: a random permutation of the pool hands out
    blocks; the first ``shared_prefix_blocks`` logical blocks of every request
    alias one common set of physical blocks."""
    need = shared_prefix_blocks + sum(max(0, n - shared_prefix_blocks) for n in blocks_per_req)
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need} blocks")
    perm = rng.permutation(num_blocks).astype(np.int32)
    mb = max_blocks if max_blocks is not None else max(blocks_per_req)
    bt = np.full((len(blocks_per_req), mb), -1, dtype=np.int32)
    shared = perm[:shared_prefix_blocks]
    cur = shared_prefix_blocks
    for r, n in enumerate(blocks_per_req):
        p = min(shared_prefix_blocks, n)
        bt[r, :p] = shared[:p]
        own = n - p
        bt[r, p:n] = perm[cur:cur + own]
        cur += own
    return bt


def build(name: str, seed: int, num_q_heads: int, num_kv_heads: int, qo_len, kv_len,
          num_blocks: int, head_dim: int = 128, block_size: int = 16, shared_prefix_blocks: int = 0,
          poison: bool = True, q_scale: float = 1.0, scale: Optional[float] = None,
          max_blocks: Optional[int] = None) -> Workload:
    qo_len = np.asarray(qo_len, dtype=np.int32)
    kv_len = np.asarray(kv_len, dtype=np.int32)
    R = qo_len.shape[0]
    if np.any(qo_len < 1) or np.any(kv_len < qo_len):
        raise ValueError("need 1 <= qo_len <= kv_len")
    s_len, s_place, s_k, s_v, s_new, s_q = _streams(seed)
    B, D, Hkv, Hq = block_size, head_dim, num_kv_heads, num_q_heads
    nb = [-(-int(L) // B) for L in kv_len]
    bt = place_blocks(s_place, num_blocks, nb, shared_prefix_blocks, max_blocks)

    fill = BF16_NAN if poison else np.uint16(0)
    k_pool = np.full((num_blocks, Hkv, B, D), fill, dtype=np.uint16)
    v_pool = np.full((num_blocks, Hkv, B, D), fill, dtype=np.uint16)
    filled = set()
    for r in range(R):
        ctx = int(kv_len[r] - qo_len[r])          # tokens already in the cache before this step
        nctx_blocks = -(-ctx // B)
        if nctx_blocks == 0:
            continue
        kd = f32_to_bf16_bits(s_k.standard_normal((nctx_blocks, Hkv, B, D), dtype=np.float32))
        vd = f32_to_bf16_bits(s_v.standard_normal((nctx_blocks, Hkv, B, D), dtype=np.float32))
        for b in range(nctx_blocks):
            phys = int(bt[r, b])
            if phys in filled:       # an aliased (shared) block is written once
                continue
            n = min(B, ctx - b * B)
            k_pool[phys, :, :n, :] = kd[b, :, :n, :]
            v_pool[phys, :, :n, :] = vd[b, :, :n, :]
            if n == B:
                filled.add(phys)

    n_new = int(qo_len.sum())
    k_new = f32_to_bf16_bits(s_new.standard_normal((n_new, Hkv, D), dtype=np.float32))
    v_new = f32_to_bf16_bits(s_new.standard_normal((n_new, Hkv, D), dtype=np.float32))
    slots = np.empty(n_new, dtype=np.int32)
    t = 0
    for r in range(R):
        for pos in range(int(kv_len[r] - qo_len[r]), int(kv_len[r])):
            slots[t] = slot_of(bt[r], pos, B)
            t += 1
    q = f32_to_bf16_bits(s_q.standard_normal((n_new, Hq, D), dtype=np.float32) * np.float32(q_scale))
    return Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                    num_blocks=num_blocks, scale=(1.0 / np.sqrt(D)) if scale is None else scale,
                    qo_len=qo_len, kv_len=kv_len, block_tables=bt, q=q, k_pool=k_pool, v_pool=v_pool,
                    k_new=k_new, v_new=v_new, slot_mapping=slots,
                    shared_prefix_blocks=shared_prefix_blocks)


def q8_tile_bytes(head_dim: int = 128, block_size: int = 16) -> int:
    """q8_0 (block, KV head) tile: [B][D] int8 codes followed by [B][D/32] binary16 scales."""
    return block_size * head_dim + block_size * (head_dim // 32) * 2


HALF_NAN = np.uint16(0x7E00)


def build_q8(name: str, seed: int, num_q_heads: int, num_kv_heads: int, qo_len, kv_len, num_blocks: int,
             head_dim: int = 128, block_size: int = 16, shared_prefix_blocks: int = 0, poison: bool = True,
             q_scale: float = 1.0) -> Workload:
    """Like ``build`` with a q8_0 pool.  Context tokens already in the cache are drawn in the
    storage format itself: codes round(N(0,1) * 42) clipped to [-127, 127] (about what
    quantising N(0,1) data gives) and one binary16 scale per 32 dims from U[0.018, 0.03].
    Slots that hold no context token keep random code bytes and NaN scales when ``poison``
    is set.  The new tokens' K/V are bf16 N(0,1), to be quantised by the append."""
    qo_len = np.asarray(qo_len, dtype=np.int32)
    kv_len = np.asarray(kv_len, dtype=np.int32)
    R = qo_len.shape[0]
    if np.any(qo_len < 1) or np.any(kv_len < qo_len):
        raise ValueError("need 1 <= qo_len <= kv_len")
    s_len, s_place, s_k, s_v, s_new, s_q = _streams(seed)
    B, D, Hkv, Hq = block_size, head_dim, num_kv_heads, num_q_heads
    G = D // 32
    nb = [-(-int(L) // B) for L in kv_len]
    bt = place_blocks(s_place, num_blocks, nb, shared_prefix_blocks, None)
    tile = q8_tile_bytes(D, B)
    kv_pool = np.zeros((num_blocks, Hkv, 2, tile), np.uint8)
    if poison:
        for which, s_x in ((0, s_k), (1, s_v)):
            kv_pool[:, :, which, :B * D] = s_x.integers(0, 256, (num_blocks, Hkv, B * D), dtype=np.uint8)
        kv_pool[:, :, :, B * D:].view(np.uint16)[...] = HALF_NAN
    filled = set()
    for r in range(R):
        ctx = int(kv_len[r] - qo_len[r])
        for b in range(-(-ctx // B)):
            phys = int(bt[r, b])
            n = min(B, ctx - b * B)
            if phys in filled:
                continue
            for which, s_x in ((0, s_k), (1, s_v)):
                codes = np.clip(np.rint(s_x.standard_normal((Hkv, n, D)) * 42.0), -127, 127).astype(np.int8)
                scales = s_x.uniform(0.018, 0.03, (Hkv, n, G)).astype(np.float16).view(np.uint16)
                t = kv_pool[phys, :, which]                       # [Hkv][tile bytes], a view
                t[:, :B * D].reshape(Hkv, B, D)[:, :n, :] = codes.view(np.uint8)
                t[:, B * D:].reshape(Hkv, B, G * 2)[:, :n, :] = scales.view(np.uint8).reshape(Hkv, n, G * 2)
            if n == B:
                filled.add(phys)
    n_new = int(qo_len.sum())
    k_new = f32_to_bf16_bits(s_new.standard_normal((n_new, Hkv, D), dtype=np.float32))
    v_new = f32_to_bf16_bits(s_new.standard_normal((n_new, Hkv, D), dtype=np.float32))
    slots = np.empty(n_new, dtype=np.int32)
    t = 0
    for r in range(R):
        for pos in range(int(kv_len[r] - qo_len[r]), int(kv_len[r])):
            slots[t] = slot_of(bt[r], pos, B)
            t += 1
    q = f32_to_bf16_bits(s_q.standard_normal((n_new, Hq, D), dtype=np.float32) * np.float32(q_scale))
    return Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                    num_blocks=num_blocks, scale=1.0 / np.sqrt(D), qo_len=qo_len, kv_len=kv_len,
                    block_tables=bt, q=q, k_pool=None, v_pool=None, k_new=k_new, v_new=v_new,
                    slot_mapping=slots, shared_prefix_blocks=shared_prefix_blocks, kv_format="q8_0",
                    kv_pool=kv_pool)


FP8_NAN = np.uint8(0x7F)


def build_fp8(name: str, seed: int, num_q_heads: int, num_kv_heads: int, qo_len, kv_len, num_blocks: int,
              head_dim: int = 128, block_size: int = 16, shared_prefix_blocks: int = 0, poison: bool = True,
              q_scale: float = 1.0, k_scale: float = 0.375, v_scale: float = 0.3125) -> Workload:
    """Like ``build`` with FP8 pools (OCP E4M3 codes, one byte per value, the bf16 layout)
    and per-pool scales.  Context tokens already in the cache are drawn in the storage
    format itself: a random sign, exponent field 3..8 (magnitudes 2^-4 .. 3.75) and fraction
    field 0..7, so every code is finite.  Slots that hold no context token keep the NaN
    code when ``poison`` is set.  The new tokens' K/V are bf16 N(0,1), stored by the append."""
    qo_len = np.asarray(qo_len, dtype=np.int32)
    kv_len = np.asarray(kv_len, dtype=np.int32)
    R = qo_len.shape[0]
    if np.any(qo_len < 1) or np.any(kv_len < qo_len):
        raise ValueError("need 1 <= qo_len <= kv_len")
    s_len, s_place, s_k, s_v, s_new, s_q = _streams(seed)
    B, D, Hkv, Hq = block_size, head_dim, num_kv_heads, num_q_heads
    nb = [-(-int(L) // B) for L in kv_len]
    bt = place_blocks(s_place, num_blocks, nb, shared_prefix_blocks, None)
    fill = FP8_NAN if poison else np.uint8(0)
    k_pool = np.full((num_blocks, Hkv, B, D), fill, dtype=np.uint8)
    v_pool = np.full((num_blocks, Hkv, B, D), fill, dtype=np.uint8)
    filled = set()
    for r in range(R):
        ctx = int(kv_len[r] - qo_len[r])
        for b in range(-(-ctx // B)):
            phys = int(bt[r, b])
            n = min(B, ctx - b * B)
            if phys in filled:
                continue
            for pool, s_x in ((k_pool, s_k), (v_pool, s_v)):
                sign = s_x.integers(0, 2, (Hkv, n, D), dtype=np.uint8) << 7
                expo = s_x.integers(3, 9, (Hkv, n, D), dtype=np.uint8) << 3
                frac = s_x.integers(0, 8, (Hkv, n, D), dtype=np.uint8)
                pool[phys, :, :n, :] = sign | expo | frac
            if n == B:
                filled.add(phys)
    n_new = int(qo_len.sum())
    k_new = f32_to_bf16_bits(s_new.standard_normal((n_new, Hkv, D), dtype=np.float32))
    v_new = f32_to_bf16_bits(s_new.standard_normal((n_new, Hkv, D), dtype=np.float32))
    slots = np.empty(n_new, dtype=np.int32)
    t = 0
    for r in range(R):
        for pos in range(int(kv_len[r] - qo_len[r]), int(kv_len[r])):
            slots[t] = slot_of(bt[r], pos, B)
            t += 1
    q = f32_to_bf16_bits(s_q.standard_normal((n_new, Hq, D), dtype=np.float32) * np.float32(q_scale))
    wl = Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                  num_blocks=num_blocks, scale=1.0 / np.sqrt(D), qo_len=qo_len, kv_len=kv_len,
                  block_tables=bt, q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
                  slot_mapping=slots, shared_prefix_blocks=shared_prefix_blocks, kv_format="fp8",
                  k_scale=float(k_scale), v_scale=float(v_scale))
    return wl


def config_tiny_fp8(seed: int = 12, poison: bool = True, q_scale: float = 1.0) -> Workload:
    """config_tiny's shape (4 decode rows, 8 q / 2 kv heads) on FP8 pools."""
    return build_fp8("tiny_fp8", seed, 8, 2, qo_len=[1] * 4, kv_len=[17, 64, 100, 250], num_blocks=64,
                     poison=poison, q_scale=q_scale)


def config_decode_fp8(seed: int = 2, num_reqs: int = 32, poison: bool = True) -> Workload:
    """The Qwen3-8B decode step (32 rows, kv_len 2048 + U[0,255]) on FP8 pools of as many
    blocks as the bf16 one; the default seed gives config_decode's lengths and tables."""
    kv = 2048 + _uniform_extra(seed, num_reqs)
    return build_fp8("qwen3_8b_decode_step_fp8", seed, 32, 8, qo_len=[1] * num_reqs, kv_len=kv,
                     num_blocks=POOL_BLOCKS_12GIB, poison=poison)


def config_tiny_q8(seed: int = 11, poison: bool = True, q_scale: float = 1.0) -> Workload:
    """The tiny decode case (4 rows, kv_len 17 / 64 / 100 / 250, 8 q / 2 kv heads) on a q8_0 pool."""
    return build_q8("tiny_decode_q8", seed, 8, 2, qo_len=[1, 1, 1, 1], kv_len=[17, 64, 100, 250],
                    num_blocks=64, poison=poison, q_scale=q_scale)


def config_decode_q8(seed: int = 2, num_reqs: int = 32, poison: bool = True) -> Workload:
    """The Qwen3-8B decode step (32 rows, kv_len 2048 + U[0,255]) on a q8_0 pool of as many
    blocks as the bf16 one; the default seed gives config_decode's lengths and tables."""
    kv = 2048 + _uniform_extra(seed, num_reqs)
    return build_q8("qwen3_8b_decode_step_q8", seed, 32, 8, qo_len=[1] * num_reqs, kv_len=kv,
                    num_blocks=POOL_BLOCKS_12GIB, poison=poison)


# Qwen3-8B attention geometry (book section 8.1.2: 36 layers, 8 KV heads of size 128, bf16).
QWEN3_8B = dict(num_layers=36, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype_bytes=2)
# A 12 GiB pool spread over 36 layers, in 16-token blocks of one layer's K+V for all KV heads.
POOL_BLOCKS_12GIB = (12 * 2**30) // (36 * 16 * 2 * 8 * 128 * 2)


def _uniform_extra(seed: int, n: int) -> np.ndarray:
    """U[0,255] per request, from its own stream so lengths do not depend on other draws."""
    return np.random.default_rng(np.random.SeedSequence([seed, 0xA11])).integers(0, 256, size=n)


def config_tiny(seed: int = 1, poison: bool = True, q_scale: float = 1.0) -> Workload:
    """Tiny paged decode: 8 Q / 2 KV heads, 4 decode rows, blocks permuted in a 64-block pool."""
    return build("tiny_decode", seed, 8, 2, qo_len=[1, 1, 1, 1], kv_len=[17, 64, 100, 250],
                 num_blocks=64, poison=poison, q_scale=q_scale)


def config_decode(seed: int = 2, num_reqs: int = 32, poison: bool = True,
                  num_blocks: int = POOL_BLOCKS_12GIB, q_scale: float = 1.0) -> Workload:
    """Qwen3-8B single-layer decode step: kv_len = 2048 + U[0,255], random scattered blocks."""
    kv = 2048 + _uniform_extra(seed, num_reqs)
    return build("qwen3_8b_decode", seed, 32, 8, qo_len=np.ones(num_reqs, np.int32), kv_len=kv,
                 num_blocks=num_blocks, poison=poison, q_scale=q_scale)


def config_shared_prefix(seed: int = 3, num_reqs: int = 16, poison: bool = True,
                         num_blocks: int = POOL_BLOCKS_12GIB) -> Workload:
    """Long-context decode, kv_len = 8192 + U[0,255]; the first 384 blocks (6144 tokens)
    of every block table alias the same physical blocks."""
    kv = 8192 + _uniform_extra(seed, num_reqs)
    return build("shared_prefix_decode", seed, 32, 8, qo_len=np.ones(num_reqs, np.int32), kv_len=kv,
                 num_blocks=num_blocks, shared_prefix_blocks=384, poison=poison)


def config_mixed(seed: int = 4, poison: bool = True, num_blocks: int = POOL_BLOCKS_12GIB) -> Workload:
    """Mixed continuous batch: one 512-token prefill chunk at kv offset 4096 (4608 kv total)
    followed by 31 decode rows with kv_len = 2048 + U[0,255]; 543 new tokens in all."""
    kv = np.concatenate([[4608], 2048 + _uniform_extra(seed, 31)]).astype(np.int32)
    qo = np.concatenate([[512], np.ones(31, np.int32)]).astype(np.int32)
    return build("mixed_batch", seed, 32, 8, qo_len=qo, kv_len=kv, num_blocks=num_blocks, poison=poison)


def config_mixed_q8(seed: int = 4, poison: bool = True, num_blocks: int = POOL_BLOCKS_12GIB) -> Workload:
    """config_mixed's rows (one 512-token chunk at kv offset 4096, 31 decode rows) on a
    q8_0 pool."""
    kv = np.concatenate([[4608], 2048 + _uniform_extra(seed, 31)]).astype(np.int32)
    qo = np.concatenate([[512], np.ones(31, np.int32)]).astype(np.int32)
    return build_q8("mixed_batch_q8", seed, 32, 8, qo_len=qo, kv_len=kv, num_blocks=num_blocks, poison=poison)


def config_shared_prefix_q8(seed: int = 3, num_reqs: int = 16, poison: bool = True,
                            num_blocks: int = POOL_BLOCKS_12GIB) -> Workload:
    """config_shared_prefix's rows (kv_len 8192 + U[0,255], 384 shared blocks) on a q8_0 pool."""
    kv = 8192 + _uniform_extra(seed, num_reqs)
    return build_q8("shared_prefix_decode_q8", seed, 32, 8, qo_len=np.ones(num_reqs, np.int32), kv_len=kv,
                    num_blocks=num_blocks, shared_prefix_blocks=384, poison=poison)


def config_mixed_fp8(seed: int = 4, poison: bool = True, num_blocks: int = POOL_BLOCKS_12GIB) -> Workload:
    """config_mixed's rows (one 512-token chunk at kv offset 4096, 31 decode rows) on FP8 pools."""
    kv = np.concatenate([[4608], 2048 + _uniform_extra(seed, 31)]).astype(np.int32)
    qo = np.concatenate([[512], np.ones(31, np.int32)]).astype(np.int32)
    return build_fp8("mixed_batch_fp8", seed, 32, 8, qo_len=qo, kv_len=kv, num_blocks=num_blocks, poison=poison)


def config_shared_prefix_fp8(seed: int = 3, num_reqs: int = 16, poison: bool = True,
                             num_blocks: int = POOL_BLOCKS_12GIB) -> Workload:
    """config_shared_prefix's rows (kv_len 8192 + U[0,255], 384 shared blocks) on FP8 pools."""
    kv = 8192 + _uniform_extra(seed, num_reqs)
    return build_fp8("shared_prefix_decode_fp8", seed, 32, 8, qo_len=np.ones(num_reqs, np.int32), kv_len=kv,
                     num_blocks=num_blocks, shared_prefix_blocks=384, poison=poison)


def config_sweep_decode(batch: int, layer: int, seed: int = 5, poison: bool = True,
                        num_blocks: Optional[int] = None, long_only: bool = False,
                        fill_pools: bool = True) -> Workload:
    """One layer of the 36-layer decode sweep: half the rows have a 2048-token context and
    half an 8192-token context whose first 6144 tokens are a shared prefix; the step
    appends one token per row (kv_len 2049 / 8193).  Batch 1 is short unless ``long_only``.
    ``fill_pools=False`` leaves the pools empty (zero-size arrays): tables, lengths, slots,
    Q and new K/V only, for callers that fill device pools themselves."""
    if batch == 1:
        kv = [8193] if long_only else [2049]
    else:
        kv = [2049] * (batch // 2) + [8193] * (batch - batch // 2)
    kv = np.asarray(kv, np.int32)
    nshort = int((kv == 2049).sum())
    nlong = batch - nshort
    shared = 384 if nlong > 0 else 0
    # Long rows come after short rows; the shared prefix applies to long rows only, so build
    # their placement with aliasing and the short rows without it.
    need = nshort * 129 + (384 + nlong * (513 - 384) if nlong else 0)
    nblocks = num_blocks if num_blocks is not None else max(POOL_BLOCKS_12GIB, need)
    wl = _build_short_long(f"sweep_b{batch}_layer{layer}", [seed, layer, batch], kv, shared, nblocks,
                           poison, fill_pools)
    return wl


def _build_short_long(name, seed_words, kv, shared_blocks, num_blocks, poison, fill_pools=True):
    """Placement where only the rows longer than the shared prefix alias it."""
    seed = int(np.random.SeedSequence(seed_words).generate_state(1)[0])
    s_len, s_place, s_k, s_v, s_new, s_q = _streams(seed)
    B, D, Hkv, Hq = 16, 128, 8, 32
    R = len(kv)
    qo = np.ones(R, np.int32)
    nb = [-(-int(L) // B) for L in kv]
    mb = max(nb)
    perm = s_place.permutation(num_blocks).astype(np.int32)
    bt = np.full((R, mb), -1, np.int32)
    shared = perm[:shared_blocks]
    cur = shared_blocks
    for r in range(R):
        p = shared_blocks if nb[r] > shared_blocks else 0
        bt[r, :p] = shared[:p]
        bt[r, p:nb[r]] = perm[cur:cur + nb[r] - p]
        cur += nb[r] - p
    if cur > num_blocks:
        raise ValueError("pool too small")
    fill = BF16_NAN if poison else np.uint16(0)
    pool_shape = (num_blocks, Hkv, B, D) if fill_pools else (0, Hkv, B, D)
    k_pool = np.full(pool_shape, fill, np.uint16)
    v_pool = np.full(pool_shape, fill, np.uint16)
    filled = set()
    for r in range(R if fill_pools else 0):
        ctx = int(kv[r]) - 1
        ncb = -(-ctx // B)
        kd = f32_to_bf16_bits(s_k.standard_normal((ncb, Hkv, B, D), dtype=np.float32))
        vd = f32_to_bf16_bits(s_v.standard_normal((ncb, Hkv, B, D), dtype=np.float32))
        for b in range(ncb):
            phys = int(bt[r, b])
            if phys in filled:
                continue
            n = min(B, ctx - b * B)
            k_pool[phys, :, :n] = kd[b, :, :n]
            v_pool[phys, :, :n] = vd[b, :, :n]
            if n == B:
                filled.add(phys)
    k_new = f32_to_bf16_bits(s_new.standard_normal((R, Hkv, D), dtype=np.float32))
    v_new = f32_to_bf16_bits(s_new.standard_normal((R, Hkv, D), dtype=np.float32))
    slots = np.array([slot_of(bt[r], int(kv[r]) - 1, B) for r in range(R)], np.int32)
    q = f32_to_bf16_bits(s_q.standard_normal((R, Hq, D), dtype=np.float32))
    return Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                    num_blocks=num_blocks, scale=1.0 / np.sqrt(D), qo_len=qo, kv_len=np.asarray(kv, np.int32),
                    block_tables=bt, q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
                    slot_mapping=slots, shared_prefix_blocks=shared_blocks)


def prompt_chunks(seed: int = 5, prompt_len: int = 2048, chunk: int = 512, num_q_heads: int = 32,
                  num_kv_heads: int = 8, num_blocks: int = 256, poison: bool = True, layer: int = 0):
    """A causal prompt processed one-shot and in chunks of ``chunk`` tokens.

    Returns (one_shot, [chunk_0, chunk_1, ...]).  All share one block table and one set of
    per-position Q/K/V; chunk k has context h = k*chunk and qo_len = chunk, and its pool
    holds the K/V of every earlier position (book section 8.2.3: chunk c at context h)."""
    one = build(f"prompt{prompt_len}_layer{layer}", int(np.random.SeedSequence([seed, layer, 77]).generate_state(1)[0]),
                num_q_heads, num_kv_heads, qo_len=[prompt_len], kv_len=[prompt_len],
                num_blocks=num_blocks, poison=poison)
    chunks = []
    B = one.block_size
    k_pool = one.k_pool.copy()
    v_pool = one.v_pool.copy()
    for c0 in range(0, prompt_len, chunk):
        c1 = min(prompt_len, c0 + chunk)
        sl = slice(c0, c1)
        wl = Workload(name=f"{one.name}_chunk{c0 // chunk}", num_q_heads=num_q_heads,
                      num_kv_heads=num_kv_heads, head_dim=one.head_dim, block_size=B,
                      num_blocks=num_blocks, scale=one.scale, qo_len=np.array([c1 - c0], np.int32),
                      kv_len=np.array([c1], np.int32), block_tables=one.block_tables.copy(),
                      q=one.q[sl].copy(), k_pool=k_pool.copy(), v_pool=v_pool.copy(),
                      k_new=one.k_new[sl].copy(), v_new=one.v_new[sl].copy(),
                      slot_mapping=one.slot_mapping[sl].copy())
        chunks.append(wl)
        for t in range(c0, c1):       # the next chunk sees this chunk's K/V in the pool
            s = int(one.slot_mapping[t])
            k_pool[s // B, :, s % B, :] = one.k_new[t]
            v_pool[s // B, :, s % B, :] = one.v_new[t]
    return one, chunks
