"""Iteration loop of a serving instance: the native token-budget scheduler forms each hybrid
batch, hl_model_step runs it on the GPU, the greedy tokens go back to the scheduler.

The loop is the chunked-prefill iteration ("Chunked prefill (stall-free batching), explained",
"How it works, step by step"): schedule within the budget, one forward pass over the flattened
tokens, completed prompts take their first token and decode from the next iteration. Everything
numeric happens in the library; this module moves host arrays to the device and back, and keeps
the clock. The caller provides the model (weights, KV pools, embedding, final norm, LM head) and
the prompts' token ids.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np
import torch

from . import binding as B


@dataclass
class IterationRecord:
    ms: float                 # GPU time of the model step (events around it)
    tokens: int
    decodes: int
    prefill_tokens: int
    visible_pairs: int        # causal (query, key) pairs of the iteration, summed over requests
    cached_tokens: int        # already-cached keys the iteration reads (sum of num_cached)
    seqs: int = 0
    emitted: List[int] = field(default_factory=list)   # request ids that took a token


class Engine:
    """shape: the layer dimensions (hidden, n_q_heads, n_kv_heads, head_dim, d_ff, rms_eps,
    rope_theta); layer_weights / pools: per layer, the weight dict and the (K, V) pools of
    `num_blocks` pages each; embed / lm_head [vocab, hidden], final_norm [hidden];
    prompt_tokens(request id, positions) -> int32 token ids of those prompt positions."""

    def __init__(self, shape, layer_weights: Sequence[Dict[str, torch.Tensor]],
                 pools: Sequence, embed: torch.Tensor, final_norm: torch.Tensor,
                 lm_head: torch.Tensor, num_blocks: int, max_blocks_per_seq: int,
                 prompt_tokens: Callable[[int, np.ndarray], np.ndarray], device: str = "cuda",
                 **sched):
        vocab = int(embed.shape[0])
        self.shape, self.vocab, self.dev = shape, vocab, device
        self.cfg = B.layer_cfg(shape)
        self.num_blocks, self.mb = num_blocks, max_blocks_per_seq
        self.prompt_tokens = prompt_tokens
        self.reset(**sched)
        self.layer_w, self.pools = list(layer_weights), list(pools)
        self.tensors = {"embed": embed, "final_norm": final_norm, "lm_head": lm_head}
        self.model = B.ModelHandle(self.layer_w, self.pools, embed, final_norm, lm_head)
        self.ws = torch.empty(256, dtype=torch.uint8, device=device)
        self.logits = torch.empty(1, vocab, dtype=torch.bfloat16, device=device)
        self.next = torch.empty(1, dtype=torch.int32, device=device)
        self.ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def reset(self, **sched) -> None:
        """A fresh scheduler (all blocks free, no requests) over the same weights and pools."""
        self.sched = B.Scheduler(num_blocks=self.num_blocks, max_blocks_per_seq=self.mb, **sched)

    def submit(self, rid: int, prompt_len: int, max_new: int) -> None:
        self.sched.submit(rid, prompt_len, max_new)

    def step(self) -> Optional[IterationRecord]:
        b = self.sched.next()
        self.last = b
        S = len(b["request_ids"])
        if S == 0:
            return None
        qs, nc = b["q_start"], b["num_cached"]
        toks = np.empty(int(qs[-1]), dtype=np.int32)
        vis = ctx = pre = dec = 0
        for s in range(S):
            c, n = int(nc[s]), int(qs[s + 1] - qs[s])
            ctx += c
            if b["decode_tokens"][s] >= 0:
                toks[qs[s]] = b["decode_tokens"][s]
                dec += 1
            else:
                toks[qs[s]:qs[s + 1]] = self.prompt_tokens(int(b["request_ids"][s]),
                                                           c + np.arange(n))
                pre += n
            vis += n * c + n * (n + 1) // 2
        batch = B.Batch(qs, nc, b["table"], self.dev)
        need = B.model_workspace_bytes(self.cfg, batch, self.model)
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.dev)
        if S > self.next.numel():
            self.logits = torch.empty(S, self.vocab, dtype=torch.bfloat16, device=self.dev)
            self.next = torch.empty(S, dtype=torch.int32, device=self.dev)
        tokens = torch.from_numpy(toks).to(self.dev)
        self.ev[0].record()
        B.model_step(self.cfg, batch, self.model, tokens, toks, self.logits[:S], self.next[:S],
                     self.ws)
        self.ev[1].record()
        nxt = self.next[:S].cpu().numpy()  # synchronises
        ms = self.ev[0].elapsed_time(self.ev[1])
        emitted = [int(r) for r, e in zip(b["request_ids"], b["emits"]) if e]
        self.sched.complete(nxt)
        return IterationRecord(ms, int(qs[-1]), dec, pre, vis, ctx, S, emitted)


def step_time_model(recs: List[IterationRecord], layer_params: float, head_params: float,
                    hidden: int, layers: int, kv_bytes_per_token: float, flops: float, bw: float,
                    fixed_ms: float, overlap: bool = True) -> np.ndarray:
    """Step times (ms) of the chunked-prefill page's roofline step-time model ("Chunked prefill
    (stall-free batching), explained", "The bottleneck: prefill-decode interference" and "What
    chunking costs"). Compute: 2 flops per weight per token plus 4 d_model L flops per causal
    (query, key) pair. Memory: one read of the 16-bit weights plus the K/V of every already-cached
    token the iteration attends to (decode contexts and the cached prefix of prompt chunks). With
    overlap the step takes the larger of the two (the page's optimistic model); without, the K/V
    time is added after the larger of compute and weight time (its pessimistic model). A fixed cost
    is added per iteration; 0.5 ms reproduces the page's printed step times. The LM head runs on
    one row per sequence, so its flops count once per sequence rather than per token."""
    tok = np.array([r.tokens for r in recs], dtype=np.float64)
    seqs = np.array([r.seqs for r in recs], dtype=np.float64)
    vis = np.array([r.visible_pairs for r in recs], dtype=np.float64)
    ctx = np.array([r.cached_tokens for r in recs], dtype=np.float64)
    t_comp = (2 * layer_params * tok + 2 * head_params * seqs
              + 4.0 * hidden * layers * vis) / flops
    t_w = 2 * (layer_params + head_params) / bw
    t_kv = kv_bytes_per_token * ctx / bw
    t = np.maximum(t_comp, t_w + t_kv) if overlap else np.maximum(t_comp, t_w) + t_kv
    return 1000.0 * t + fixed_ms


def fit_step_model(recs: List[IterationRecord], overlap: bool = True, **kw) -> Dict[str, float]:
    """Achievable compute, bandwidth and fixed cost of step_time_model that minimise the median
    relative error against measured step times (grid search)."""
    ms = np.array([r.ms for r in recs], dtype=np.float64)
    best = None
    for f in np.linspace(0.1e15, 2.5e15, 49):
        for bw in np.linspace(0.5e12, 8.0e12, 31):
            base = step_time_model(recs, flops=f, bw=bw, fixed_ms=0.0, overlap=overlap, **kw)
            for fx in np.linspace(0.0, 4.0, 41):
                err = float(np.median(np.abs(base + fx - ms) / ms))
                if best is None or err < best[0]:
                    best = (err, f, bw, fx)
    return {"tflops": round(best[1] / 1e12, 1), "tb_per_s": round(best[2] / 1e12, 2),
            "fixed_ms": round(best[3], 2), "median_rel_err": round(best[0], 4)}
