"""Plain reference of moving one request's paged K/V into the transfer layout and back.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU-baseline leg.

What it computes. A prefill instance hands a finished prompt's KV cache to a decode instance as
one tensor of shape [L, 2, T, n_kv_heads, head_dim] (layer, K then V, token, KV head, dim); the
decode instance places it into its own paged cache ("7.8 Disaggregated Prefill/Decode & Chunked
Prefill", "Lifecycle of a Request", step 3 and 4). The copy goes layer by layer, each layer's
slice as soon as that layer has appended its K/V rows ("Layer-Wise Pipelining"). Pages use the
head-before-token layout, so one (block, head) page is contiguous ("Gescheiden Prefill en Decode",
section on sharded KV cache transfers):
    K pool [num_blocks][n_kv_heads][16 tokens][head_dim]
    V pool [num_blocks][n_kv_heads][head_dim][16 tokens]
and position p of a request lives in slot (table_row[p // 16], p % 16).

So export is the gather  out[layer, 0, i, h, :] = K[table_row[p // 16], h, p % 16, :]  and
                         out[layer, 1, i, h, :] = V[table_row[p // 16], h, :, p % 16]
for p = start + i, i < count; import is the matching scatter into another pool and table.
Values are copied, never rounded: the reference works on whatever dtype it is given.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def export_layer(kpool: np.ndarray, vpool: np.ndarray, table_row: np.ndarray, start: int,
                 count: int, layer: int, out: np.ndarray) -> None:
    """Writes out[layer, 0/1, i] for tokens start .. start + count - 1, one token at a time."""
    for i in range(count):
        p = start + i
        b, s = int(table_row[p // BLOCK]), p % BLOCK
        out[layer, 0, i] = kpool[b, :, s, :]
        out[layer, 1, i] = vpool[b, :, :, s]


def import_layer(src: np.ndarray, table_row: np.ndarray, start: int, count: int, layer: int,
                 kpool: np.ndarray, vpool: np.ndarray) -> None:
    """Scatters src[layer, 0/1, i] into the slots of positions start .. start + count - 1."""
    for i in range(count):
        p = start + i
        b, s = int(table_row[p // BLOCK]), p % BLOCK
        kpool[b, :, s, :] = src[layer, 0, i]
        vpool[b, :, :, s] = src[layer, 1, i]
