"""Plain, slow, obviously-correct fp64 reference of one transformer-layer step over a hybrid batch.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU-baseline leg.

What it computes. A hybrid batch concatenates prompt-chunk tokens and single decode tokens; the
linear layers treat every token row on its own, attention runs per request over that request's own
keys and values ("ConfluxServe" summary, "The big picture: what happens inside one Transformer
layer" and "Why can linear layers be batched but attention cannot?"). Each request arrives with
(start position = tokens already cached, n new tokens) and the pass is one ragged forward over the
flattened tokens: prompt chunks write K/V into the paged cache and attend causally to everything
cached for their request; decodes append one token ("Chunked prefill (stall-free batching),
explained", "How it works, step by step"). A query at absolute position p sees keys 0..p inclusive
("7.8 Disaggregated Prefill/Decode & Chunked Prefill", "Attention on Partial KV Caches" and its GQA
exercise, which repeats each KV head over its group of query heads).

So the oracle is the plain definition: run each request's new tokens through a pre-norm decoder
layer with causal attention over its whole context. Nothing is blocked, fused or reordered; every
intermediate stays in fp64 (inputs are bf16 values upcast exactly by the caller).

Readings where the pages are silent (each is a parameter or a documented convention):
  * block: h1 = RMSNorm(x); qkv = h1 W_qkv^T; RoPE on q, k; attention; h2 = x + o W_o^T;
    out = h2 + (silu(h3 W_gate^T) * (h3 W_up^T)) W_down^T with h3 = RMSNorm(h2); no biases.
  * RMSNorm: x / sqrt(mean(x^2) + eps) * gain.
  * RoPE: rotate-half pairs (j, j + d/2) with angle p * theta^(-2j/d); q and k only, never v.
  * cached K is stored after RoPE; a new token sits at position num_cached + i.
  * the K/V slot of position p of sequence s is (block_table[s][p // B], p % B).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """Per row: x / sqrt(mean_j x_j^2 + eps) * gain."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T with W stored [out_features, in_features]."""
    return x @ w.T


def rope(v: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding of v [n, heads, d] at absolute positions [n]: each pair (j, j + d/2),
    j < d/2, turns by angle p * theta^(-2j/d)."""
    d = v.shape[-1]
    half = d // 2
    j = np.arange(half, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * j / d)
    ang = positions.astype(np.float64)[:, None] * omega[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    a = v[..., :half]
    b = v[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
                     scale: float) -> np.ndarray:
    """softmax(q k^T * scale) v per query head, keys j <= q_pos only.

    q [n, Hq, d] at absolute positions q_pos [n]; k, v [L, Hkv, d] hold positions 0..L-1.
    Query head h reads KV head h // (Hq / Hkv)."""
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    group = hq // hkv
    visible = np.arange(L)[None, :] <= q_pos[:, None]
    out = np.empty((n, hq, d), dtype=np.float64)
    for h in range(hq):
        kh = k[:, h // group, :]
        vh = v[:, h // group, :]
        s = (q[:, h, :] @ kh.T) * scale
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vh
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(h: np.ndarray, w_gate_up: np.ndarray, d_ff: int) -> np.ndarray:
    """silu(h W_gate^T) * (h W_up^T); W_gate_up holds the d_ff gate rows, then the d_ff up rows."""
    gate = linear(h, w_gate_up[:d_ff])
    up = linear(h, w_gate_up[d_ff:])
    return silu(gate) * up


def kv_slot_addresses(block_table_row: np.ndarray, positions: np.ndarray,
                      block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Paged-cache slot of each position: (physical block, slot within the block)."""
    positions = np.asarray(positions, dtype=np.int64)
    return block_table_row[positions // block_size].astype(np.int64), positions % block_size


def sequence_step(shape, x_seq: np.ndarray, w: Dict[str, np.ndarray], num_cached: int,
                  cached_k: np.ndarray, cached_v: np.ndarray,
                  rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """The layer applied to one request's n new tokens x_seq [n, H] at positions
    num_cached .. num_cached + n - 1, with cached (post-RoPE) K/V [num_cached, Hkv, d].

    `rows` (default: all) selects which of the n rows to finish through attention, the output
    projection and the MLP; K/V are still computed for every row up to the last selected one,
    since later rows attend to them. Returns fp64 arrays for the selected rows plus the new
    (rotated) K and V rows for positions num_cached .. num_cached + last."""
    n = x_seq.shape[0]
    hq, hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    sel = np.arange(n) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    last = int(sel.max()) + 1 if sel.size else 0
    x_kv = x_seq[:last]
    pos_all = num_cached + np.arange(last)

    h1 = rmsnorm(x_kv, w["attn_norm"], shape.rms_eps)
    w_qkv = w["w_qkv"]
    q_w = w_qkv[: hq * d]
    k_w = w_qkv[hq * d: (hq + hkv) * d]
    v_w = w_qkv[(hq + hkv) * d:]
    k_new = rope(linear(h1, k_w).reshape(last, hkv, d), pos_all, shape.rope_theta)
    v_new = linear(h1, v_w).reshape(last, hkv, d)
    k_full = np.concatenate([cached_k.reshape(num_cached, hkv, d), k_new], axis=0)
    v_full = np.concatenate([cached_v.reshape(num_cached, hkv, d), v_new], axis=0)

    pos = num_cached + sel
    q = linear(h1[sel], q_w).reshape(sel.size, hq, d)
    q_rot = rope(q, pos, shape.rope_theta)
    scale = 1.0 / np.sqrt(d) if getattr(shape, "softmax_scale", 0.0) in (0.0, None) \
        else float(shape.softmax_scale)
    attn = causal_attention(q_rot, k_full, v_full, pos, scale).reshape(sel.size, hq * d)
    h2 = x_seq[sel] + linear(attn, w["w_o"])
    h3 = rmsnorm(h2, w["mlp_norm"], shape.rms_eps)
    out = h2 + linear(swiglu(h3, w["w_gate_up"], shape.d_ff), w["w_down"])
    return {"rows": sel, "out": out, "q_rot": q_rot, "attn_out": attn, "h2": h2,
            "k_new": k_new, "v_new": v_new}


def layer_step(shape, x: np.ndarray, w: Dict[str, np.ndarray],
               seqs: Sequence[Tuple[int, int]], cached: Sequence[Tuple[np.ndarray, np.ndarray]],
               block_table: np.ndarray) -> Dict[str, np.ndarray]:
    """The whole hybrid batch: rows of x [T, H] belong to the sequences in order, sequence s
    owning seqs[s] = (num_cached, q_len) rows. Returns out / q_rot / attn_out / h2 for all T rows,
    and the new K/V rows with their paged addresses (seq, position, block, slot)."""
    T = x.shape[0]
    hq, hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    out = np.empty((T, shape.hidden))
    q_rot = np.empty((T, hq, d))
    attn = np.empty((T, hq * d))
    h2 = np.empty((T, shape.hidden))
    new_k: List[np.ndarray] = []
    new_v: List[np.ndarray] = []
    addr: List[np.ndarray] = []
    row = 0
    for s, (c, n) in enumerate(seqs):
        r = sequence_step(shape, x[row:row + n], w, c, cached[s][0], cached[s][1])
        out[row:row + n] = r["out"]
        q_rot[row:row + n] = r["q_rot"]
        attn[row:row + n] = r["attn_out"]
        h2[row:row + n] = r["h2"]
        pos = c + np.arange(n)
        blk, slot = kv_slot_addresses(block_table[s], pos, shape.block_size)
        addr.append(np.stack([np.full(n, s), pos, blk, slot], axis=1))
        new_k.append(r["k_new"])
        new_v.append(r["v_new"])
        row += n
    return {
        "out": out, "q_rot": q_rot, "attn_out": attn, "h2": h2,
        "k_new": np.concatenate(new_k) if new_k else np.zeros((0, hkv, d)),
        "v_new": np.concatenate(new_v) if new_v else np.zeros((0, hkv, d)),
        "kv_addr": np.concatenate(addr) if addr else np.zeros((0, 4), dtype=np.int64),
    }
