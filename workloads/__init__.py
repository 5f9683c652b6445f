"""Seeded synthetic hybrid batches: shapes, contexts, block tables and random values.

This module only draws random inputs. It holds none of the layer's arithmetic, so both the
fp64 oracle (through the tests) and the GPU path can consume the very same arrays.

Shapes follow the five workloads the layer step is measured on:
  1  tiny layer (hidden 256, 4/2 heads, head_dim 64, d_ff 512): one 64-token chunk at prefix 64
     plus decodes at contexts 32, 57, 96, 128;
  2  Qwen3-8B shape: 1024-token chunk at prefix 0 plus 16 decodes at context 8192;
  3  Qwen3-14B shape: 2048-token chunk at prefix 16384 plus 96 decodes, contexts uniform in
     [2048, 8192];
  4  Qwen3-8B shape: 4096-token prompt at prefix 0 plus 64 decodes at context 1125
     (also split into a prefill-only and a decode-only batch);
  5  70B shape: 512-token chunk at prefix 8192 plus 512 decodes, contexts log-uniform in
     [1024, 32768].
The contexts of the decodes in 1-5 are the scenarios of the ConfluxServe summary ("What problem
is it actually solving?": 16 decodes at 8K context) and of "Chunked prefill (stall-free
batching), explained" ("Worked example": 64 decodes at 1,125 tokens with a 4,096-token prompt).

Value recipe: hidden states and cached K/V ~ N(0, 1), linear weights ~ N(0, 0.02^2), norm gains
= 1, each drawn in fp32 and rounded to bf16 (round-to-nearest-even). Contexts and block ids come
from numpy PCG64(SeedSequence(1000 + config)); bulk values come from torch generators seeded
from the same SeedSequence, on the device the caller names (CPU and GPU streams differ, each is
deterministic).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    block_size: int = BLOCK_SIZE
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def qkv_cols(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def weight_params(self) -> int:
        h, f = self.hidden, self.d_ff
        return h * self.qkv_cols + h * self.n_q_heads * self.head_dim + 2 * f * h + h * f


SHAPES: Dict[str, LayerShape] = {
    "tiny": LayerShape(256, 4, 2, 64, 512),
    "qwen3_8b": LayerShape(4096, 32, 8, 128, 12288),
    "qwen3_14b": LayerShape(5120, 40, 8, 128, 17408),
    "llama_70b": LayerShape(8192, 64, 8, 128, 28672),
}


@dataclasses.dataclass
class BatchSpec:
    """One hybrid batch: per sequence (num_cached, q_len); prefill chunks first, then decodes."""
    name: str
    shape: LayerShape
    seqs: List[Tuple[int, int]]
    seed: int
    pool_slack: float = 1.25

    @property
    def num_seqs(self) -> int:
        return len(self.seqs)

    @property
    def num_tokens(self) -> int:
        return sum(n for _, n in self.seqs)

    @property
    def q_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([n for _, n in self.seqs])]).astype(np.int32)

    @property
    def num_cached(self) -> np.ndarray:
        return np.array([c for c, _ in self.seqs], dtype=np.int32)


def _seq_streams(seed: int) -> List[np.random.SeedSequence]:
    # streams: 0 contexts, 1 block permutation, 2 weights, 3 hidden states, 4 per-sequence KV
    return np.random.SeedSequence(seed).spawn(5)


def make_spec(cfg: int, variant: str = "mixed") -> BatchSpec:
    """Build the batch of workload `cfg` (1..5). `variant` is "mixed", "prefill_only" or
    "decode_only" (the same data as the mixed batch, split; workload 4 names the split runs)."""
    seed = 1000 + cfg
    ctx_rng = np.random.Generator(np.random.PCG64(_seq_streams(seed)[0]))
    if cfg == 1:
        shape = SHAPES["tiny"]
        seqs = [(64, 64)] + [(c, 1) for c in (32, 57, 96, 128)]
        slack = 1.0
    elif cfg == 2:
        shape = SHAPES["qwen3_8b"]
        seqs = [(0, 1024)] + [(8192, 1)] * 16
        slack = 1.25
    elif cfg == 3:
        shape = SHAPES["qwen3_14b"]
        ctx = ctx_rng.integers(2048, 8192, size=96, endpoint=True)
        seqs = [(16384, 2048)] + [(int(c), 1) for c in ctx]
        slack = 1.25
    elif cfg == 4:
        shape = SHAPES["qwen3_8b"]
        seqs = [(0, 4096)] + [(1125, 1)] * 64
        slack = 1.25
    elif cfg == 5:
        shape = SHAPES["llama_70b"]
        u = ctx_rng.random(512)
        ctx = np.rint(1024.0 * np.power(32.0, u)).astype(np.int64)
        seqs = [(8192, 512)] + [(int(c), 1) for c in ctx]
        slack = 1.25
    else:
        raise ValueError(f"no workload {cfg}")
    spec = BatchSpec(f"cfg{cfg}", shape, seqs, seed, slack)
    if variant == "mixed":
        return spec
    if variant == "prefill_only":
        return BatchSpec(f"cfg{cfg}_prefill_only", shape, seqs[:1], seed, slack)
    if variant == "decode_only":
        return BatchSpec(f"cfg{cfg}_decode_only", shape, seqs[1:], seed, slack)
    raise ValueError(variant)


def named_spec(name: str) -> BatchSpec:
    """cfgN, cfgN_prefill_only, cfgN_decode_only, or "p1_16dec_8k": the decode-only scenario the
    ConfluxServe page times on a full model (16 decodes at 8K context, Qwen3-14B-shaped)."""
    if name == "p1_16dec_8k":
        return BatchSpec(name, SHAPES["qwen3_14b"], [(8192, 1)] * 16, 1100, 1.25)
    if "_" in name:
        return make_spec(int(name[3:name.index("_")]), name[name.index("_") + 1:])
    return make_spec(int(name[3:]))


def custom_spec(shape: LayerShape, seqs: Sequence[Tuple[int, int]], seed: int,
                name: str = "custom", pool_slack: float = 1.25) -> BatchSpec:
    return BatchSpec(name, shape, list(seqs), seed, pool_slack)


def blocks_needed(spec: BatchSpec) -> List[int]:
    b = spec.shape.block_size
    return [-(-(c + n) // b) for c, n in spec.seqs]


def block_table(spec: BatchSpec, permute_seed: Optional[int] = None) -> Tuple[np.ndarray, int]:
    """Physical block ids: the first sum(needed) entries of a seeded permutation of the pool,
    handed to the sequences in order. Returns (table [S, maxB] int32 padded with -1, pool size)."""
    need = blocks_needed(spec)
    total = sum(need)
    pool = max(total, int(math.ceil(total * spec.pool_slack)))
    ss = _seq_streams(spec.seed)[1] if permute_seed is None else np.random.SeedSequence(permute_seed)
    rng = np.random.Generator(np.random.PCG64(ss))
    perm = rng.permutation(pool)[:total].astype(np.int32)
    max_b = max(need) if need else 1
    table = np.full((max(len(need), 1), max_b), -1, dtype=np.int32)
    off = 0
    for s, nb in enumerate(need):
        table[s, :nb] = perm[off:off + nb]
        off += nb
    return table, pool


def _torch_seed(ss: np.random.SeedSequence, index: int = 0) -> int:
    return int(ss.spawn(index + 1)[index].generate_state(1, dtype=np.uint64)[0] & ((1 << 62) - 1))


def _randn_bf16(shape, std: float, seed: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def hidden_states(spec: BatchSpec, device="cpu"):
    """x [T, hidden] bf16 ~ N(0, 1)."""
    seed = _torch_seed(_seq_streams(spec.seed)[3])
    return _randn_bf16((spec.num_tokens, spec.shape.hidden), 1.0, seed, device)


def weights(spec: BatchSpec, device="cpu", gain_jitter: float = 0.0) -> Dict[str, "object"]:
    """Layer weights, bf16. Linear matrices ~ N(0, 0.02^2) in [out, in] (row = output feature)
    layout; w_gate_up stacks the d_ff gate rows, then the d_ff up rows. Norm gains are 1 (or
    1 + N(0, gain_jitter^2) when a test wants the gain to matter)."""
    import torch
    s = spec.shape
    ws = _seq_streams(spec.seed)[2]
    dims = {
        "w_qkv": (s.qkv_cols, s.hidden),
        "w_o": (s.hidden, s.n_q_heads * s.head_dim),
        "w_gate_up": (2 * s.d_ff, s.hidden),
        "w_down": (s.hidden, s.d_ff),
    }
    out = {}
    for i, (k, shp) in enumerate(dims.items()):
        out[k] = _randn_bf16(shp, 0.02, _torch_seed(ws, i), device)
    for i, k in enumerate(("attn_norm", "mlp_norm")):
        if gain_jitter > 0.0:
            g = _randn_bf16((s.hidden,), gain_jitter, _torch_seed(ws, 4 + i), device).float() + 1.0
            out[k] = g.to(torch.bfloat16)
        else:
            out[k] = torch.ones(s.hidden, dtype=torch.bfloat16, device=device)
    return out


def cached_kv(spec: BatchSpec, seq: int, device="cpu"):
    """Already-cached K and V of sequence `seq` for positions 0..c-1: two [c, Hkv, d] bf16 tensors
    ~ N(0, 1). Cached K is taken to be stored after the rotary embedding."""
    s = spec.shape
    c = spec.seqs[seq][0]
    base = _seq_streams(spec.seed)[4]
    seed = int(np.random.SeedSequence([int(x) for x in base.generate_state(2)] + [seq])
               .generate_state(1, dtype=np.uint64)[0] & ((1 << 62) - 1))
    kv = _randn_bf16((2, c, s.n_kv_heads, s.head_dim), 1.0, seed, device)
    return kv[0], kv[1]


def describe(spec: BatchSpec) -> dict:
    s = spec.shape
    dec = [c for c, n in spec.seqs if n == 1]
    pre = [(c, n) for c, n in spec.seqs if n > 1]
    shape_name = next((k for k, v in SHAPES.items() if v == s), "custom")
    parts = [f"{n}-token chunk at prefix {c}" for c, n in pre]
    if dec:
        parts.append(f"{len(dec)} decodes at mean context {float(np.mean(dec)):.0f}")
    label = f"{spec.name}: {shape_name} layer, " + " + ".join(parts)
    return {
        "workload": label, "name": spec.name, "hidden": s.hidden, "n_q_heads": s.n_q_heads,
        "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim, "d_ff": s.d_ff,
        "tokens": spec.num_tokens, "prefill_chunks": [list(p) for p in pre],
        "decodes": len(dec), "decode_ctx_mean": (float(np.mean(dec)) if dec else 0.0),
        "block_size": s.block_size,
    }


# ---------------------------------------------------------------------- layer stacks (model step)

def layer_spec(spec: BatchSpec, layer: int) -> BatchSpec:
    """The same batch for layer `layer` of a stack: its own seed for that layer's weights and
    cached K/V (the contexts, the block table and the tokens stay those of `spec`)."""
    return BatchSpec(f"{spec.name}/L{layer}", spec.shape, list(spec.seqs),
                     spec.seed * 1000 + 1 + layer, spec.pool_slack)


def model_tensors(spec: BatchSpec, vocab: int, device="cpu") -> Dict[str, "object"]:
    """Token ids [T] (uniform in [0, vocab)), embedding [vocab, hidden] ~ N(0, 1) (so embedded
    activations are N(0, 1) like the layer workloads), LM head [vocab, hidden] ~ N(0, 0.02^2),
    final norm gain 1."""
    import torch
    s = spec.shape
    ss = np.random.SeedSequence([spec.seed, vocab, 77])
    rng = np.random.default_rng(ss.spawn(1)[0])
    tokens = rng.integers(0, vocab, spec.num_tokens).astype(np.int32)
    return {
        "tokens": tokens,
        "embed": _randn_bf16((vocab, s.hidden), 1.0, _torch_seed(ss, 1), device),
        "lm_head": _randn_bf16((vocab, s.hidden), 0.02, _torch_seed(ss, 2), device),
        "final_norm": torch.ones(s.hidden, dtype=torch.bfloat16, device=device),
    }


# ---------------------------------------------------------------------- serving-loop inputs

def prompt_token(rid: int, pos: np.ndarray, vocab: int) -> np.ndarray:
    """Synthetic prompt token ids: a fixed function of request id and position."""
    return ((rid * 1000003 + pos * 7919) % vocab).astype(np.int32)


def engine_model(shape: LayerShape, layers: int, vocab: int, num_blocks: int, device="cuda",
                 seed: int = 2024, pool_fill: float = 0.0) -> dict:
    """Random-init model of `layers` layers for the serving loop: per-layer weights (each layer
    its own seed), KV pools of `num_blocks` pages per layer, embedding, final norm and LM head
    (keyword arguments of serving.Engine)."""
    import torch
    base = custom_spec(shape, [(0, 1)], seed)
    layer_w = [weights(layer_spec(base, l), device) for l in range(layers)]
    pools = []
    for _ in range(layers):
        # K pages chunk-major [d/8][16][8], V pages dim-major [d][16] (the library's page layout)
        k = torch.full((num_blocks, shape.n_kv_heads, shape.head_dim // 8, BLOCK_SIZE, 8),
                       pool_fill, dtype=torch.bfloat16, device=device)
        v = torch.full((num_blocks, shape.n_kv_heads, shape.head_dim, BLOCK_SIZE), pool_fill,
                       dtype=torch.bfloat16, device=device)
        pools.append((k, v))
    t = model_tensors(base, vocab, device)
    return {"layer_weights": layer_w, "pools": pools, "embed": t["embed"],
            "final_norm": t["final_norm"], "lm_head": t["lm_head"], "num_blocks": num_blocks,
            "prompt_tokens": lambda rid, pos: prompt_token(rid, pos, vocab)}
