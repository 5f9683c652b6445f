"""Paged KV pool plumbing for callers: allocate the two pools in the page layout the C ABI
uses and place already-computed K/V rows into their slots (torch indexing; no layer math).

K pool [num_blocks][Hkv][16][d] (token-major pages), V pool [num_blocks][Hkv][d][16]
(dim-major pages); position p of a sequence lives in block table_row[p // 16], slot p % 16.
"""
from __future__ import annotations

import torch

BLOCK = 16


def alloc_pools(num_blocks: int, n_kv_heads: int, head_dim: int, device="cuda",
                fill: float = float("nan")):
    k = torch.full((num_blocks, n_kv_heads, BLOCK, head_dim), fill, dtype=torch.bfloat16,
                   device=device)
    v = torch.full((num_blocks, n_kv_heads, head_dim, BLOCK), fill, dtype=torch.bfloat16,
                   device=device)
    return k, v


def write_positions(k_pool, v_pool, table_row, positions, k_rows, v_rows) -> None:
    """k_rows / v_rows [len(positions), Hkv, d] -> their pages."""
    dev = k_pool.device
    pos = torch.as_tensor(positions, device=dev).long()
    row = torch.as_tensor(table_row, device=dev).long()
    blk = row[pos // BLOCK]
    slot = pos % BLOCK
    k_pool[blk, :, slot, :] = k_rows.to(dev, torch.bfloat16)
    v_pool[blk, :, :, slot] = v_rows.to(dev, torch.bfloat16)


def read_positions(k_pool, v_pool, table_row, positions):
    """Inverse of write_positions: ([n, Hkv, d], [n, Hkv, d])."""
    dev = k_pool.device
    pos = torch.as_tensor(positions, device=dev).long()
    row = torch.as_tensor(table_row, device=dev).long()
    blk = row[pos // BLOCK]
    slot = pos % BLOCK
    return k_pool[blk, :, slot, :], v_pool[blk, :, :, slot]
