"""Plain fp64 reference of one model iteration over a hybrid batch: embedding, the layer stack,
the final norm, the LM head on each sequence's last row, and the greedy pick.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU-baseline leg.

What it computes. One iteration of chunked prefill runs the forward pass over the flattened
tokens of all scheduled requests, and a request whose last prompt chunk completes samples its
first token in that same pass ("Chunked prefill (stall-free batching), explained", "How it works,
step by step", steps 4 and 5); the prefill worker of chapter 7.8 computes logits for the last
position only and takes their argmax ("7.8 Disaggregated Prefill/Decode & Chunked Prefill", the
prefill worker's listing). Decodes take their next token the same way.

Readings: the layer is oracle.layer's (each layer with its own weights and its own cached K/V,
one block table for all layers); a final RMSNorm with its own gain precedes the LM head (the pages
print none; standard for the pre-norm stacks whose shapes the workloads use); greedy = the first
index of the largest logit.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

from oracle import layer as OL


def embed(table: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """Row tokens[t] of the embedding table for each token t."""
    return table[np.asarray(tokens, dtype=np.int64)]


def last_rows(seqs: Sequence[Tuple[int, int]]) -> np.ndarray:
    """Row index of the last new token of each sequence in the flattened batch."""
    return np.cumsum([n for _, n in seqs]) - 1


def lm_logits(h: np.ndarray, final_norm: np.ndarray, lm_head: np.ndarray, eps: float) -> np.ndarray:
    """Logits of rows h: RMSNorm(h) with the final gain, times the LM head [vocab, hidden]^T."""
    return OL.linear(OL.rmsnorm(h, final_norm, eps), lm_head)


def greedy(logits: np.ndarray) -> np.ndarray:
    """First index of the largest value of each row."""
    return np.argmax(logits, axis=-1)


def model_step(shape, tokens: np.ndarray, embed_table: np.ndarray,
               layers: Sequence[Dict[str, np.ndarray]], final_norm: np.ndarray,
               lm_head: np.ndarray, seqs: Sequence[Tuple[int, int]],
               caches: Sequence[Sequence[Tuple[np.ndarray, np.ndarray]]],
               block_table: np.ndarray) -> Dict[str, np.ndarray]:
    """caches[l][s] = (K, V) already cached for sequence s in layer l. Returns the hidden rows
    after the last layer [T, hidden] and the logits of each sequence's last row [S, vocab]."""
    x = embed(embed_table, tokens)
    for l, w in enumerate(layers):
        x = OL.layer_step(shape, x, w, seqs, caches[l], block_table)["out"]
    logits = lm_logits(x[last_rows(seqs)], final_norm, lm_head, shape.rms_eps)
    return {"hidden": x, "logits": logits}
