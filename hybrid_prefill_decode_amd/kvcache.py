"""Paged KV pool plumbing for callers: allocate the two pools in the page layout the C ABI
uses and place already-computed K/V rows into their slots (torch indexing; no layer math).

K pool [num_blocks][Hkv][d/8][16][8] (chunk-major pages: chunk c of the 16 tokens is one
contiguous 256-byte run), V pool [num_blocks][Hkv][d][16] (dim-major pages); position p of a
sequence lives in block table_row[p // 16], slot p % 16.
"""
from __future__ import annotations

import torch

BLOCK = 16


def k_pool_shape(num_blocks: int, n_kv_heads: int, head_dim: int):
    return (num_blocks, n_kv_heads, head_dim // 8, BLOCK, 8)


def v_pool_shape(num_blocks: int, n_kv_heads: int, head_dim: int):
    return (num_blocks, n_kv_heads, head_dim, BLOCK)


def alloc_pools(num_blocks: int, n_kv_heads: int, head_dim: int, device="cuda",
                fill: float = float("nan")):
    k = torch.full(k_pool_shape(num_blocks, n_kv_heads, head_dim), fill, dtype=torch.bfloat16,
                   device=device)
    v = torch.full(v_pool_shape(num_blocks, n_kv_heads, head_dim), fill, dtype=torch.bfloat16,
                   device=device)
    return k, v


def k_slots(k_pool):
    """A view of the K pool indexed [block, head, slot, chunk, 8] (no copy): k_slots(k)[b, h, t]
    is token t's row of page (b, h) as [d/8, 8]."""
    return k_pool.permute(0, 1, 3, 2, 4)


def k_rows_of(k_pool, blk, slot):
    """K rows [n, Hkv, d] of the (block, slot) pairs (a copy)."""
    r = k_slots(k_pool)[blk, :, slot]
    return r.reshape(r.shape[0], r.shape[1], -1)


def k_token_major(k_pool):
    """The whole K pool as [num_blocks, Hkv, 16, d] (a copy): the logical layout of a page."""
    nb, h, c, t, e = k_pool.shape
    return k_slots(k_pool).reshape(nb, h, t, c * e)


def k_from_token_major(k_tm):
    """Inverse of k_token_major: [num_blocks, Hkv, 16, d] -> a K pool tensor (a copy)."""
    nb, h, t, d = k_tm.shape
    return k_tm.reshape(nb, h, t, d // 8, 8).permute(0, 1, 3, 2, 4).contiguous()


def write_positions(k_pool, v_pool, table_row, positions, k_rows, v_rows) -> None:
    """k_rows / v_rows [len(positions), Hkv, d] -> their pages."""
    dev = k_pool.device
    pos = torch.as_tensor(positions, device=dev).long()
    row = torch.as_tensor(table_row, device=dev).long()
    blk = row[pos // BLOCK]
    slot = pos % BLOCK
    n, h, d = k_rows.shape
    k_slots(k_pool)[blk, :, slot] = k_rows.to(dev, torch.bfloat16).reshape(n, h, d // 8, 8)
    v_pool[blk, :, :, slot] = v_rows.to(dev, torch.bfloat16)


def read_positions(k_pool, v_pool, table_row, positions):
    """Inverse of write_positions: ([n, Hkv, d], [n, Hkv, d])."""
    dev = k_pool.device
    pos = torch.as_tensor(positions, device=dev).long()
    row = torch.as_tensor(table_row, device=dev).long()
    blk = row[pos // BLOCK]
    slot = pos % BLOCK
    return k_rows_of(k_pool, blk, slot), v_pool[blk, :, :, slot]
