"""Plain reference of the token-budget scheduler of chunked prefill.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU-baseline leg.

Each iteration fills a token budget in the order the chunked-prefill page gives ("Chunked prefill
(stall-free batching), explained", "How it works, step by step", and its schedule listing):
  1. one token for every running decode;
  2. the next chunk of each prompt already being prefilled: min(budget left, p - p_done) tokens
     starting at p_done;
  3. waiting requests in arrival order while budget, sequence slots and KV blocks remain, each
     given as many prompt tokens as fit (the first one that does not fit stops admission);
  4. one forward pass over the flattened tokens;
  5. a request whose last prompt chunk completes takes its first token from that pass and
     decodes from the next iteration.
With the adaptive policy the prompt tokens an iteration may carry follow chapter 7.8's dynamic
chunk sizing ("7.8 Disaggregated Prefill/Decode & Chunked Prefill", "Priority and Preemption
Policies"): the largest chunk while nothing decodes, the smallest once the number of decoding
requests reaches a pressure threshold, and a straight line from the base chunk down to the
smallest in between, rounded down to whole tokens. That chunk is the iteration's whole prompt
share: decode tokens come on top of it, however many prompts the share is spread over.
Reading of "can allocate": a request is admitted only if blocks for its whole lifetime (prompt +
outputs, 16 tokens per block) are free; it takes them at admission (lowest free ids first) and
returns them when its outputs are complete.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional


class Request:
    def __init__(self, rid: int, prompt_len: int, max_new: int):
        self.rid, self.prompt_len, self.max_new = rid, prompt_len, max_new
        self.prefilled = 0
        self.generated = 0
        self.last_token = -1
        self.blocks: List[int] = []


def lifetime_blocks(r: Request) -> int:
    return math.ceil((r.prompt_len + r.max_new - 1) / 16)


def adaptive_chunk(d: int, lo: int, base: int, hi: int, threshold: int) -> int:
    """Prompt share under decode load d: hi when d == 0, lo when d >= threshold, otherwise the
    line from base (as d -> 0) to lo (at d = threshold), rounded down:
    floor(base - d (base - lo) / threshold) = base - ceil(d (base - lo) / threshold), exact in
    integers."""
    if d <= 0:
        return hi
    if d >= threshold:
        return lo
    drop = -(-d * (base - lo) // threshold)  # ceiling division
    return base - drop


class Scheduler:
    def __init__(self, budget=0, max_seqs=1, num_blocks=1, adaptive=False, min_chunk=128,
                 base_chunk=512, max_chunk=4096, pressure_threshold=16):
        self.budget, self.max_seqs = budget, max_seqs
        self.adaptive = adaptive
        self.min_chunk, self.base_chunk = min_chunk, base_chunk
        self.max_chunk, self.threshold = max_chunk, pressure_threshold
        self.num_blocks = num_blocks
        self.free = list(range(num_blocks))  # sorted: lowest id first
        self.waiting: List[Request] = []
        self.prefilling: List[Request] = []
        self.running: List[Request] = []
        self.last: List[tuple] = []

    def submit(self, rid: int, prompt_len: int, max_new: int) -> None:
        r = Request(rid, prompt_len, max_new)
        if lifetime_blocks(r) > self.num_blocks:
            raise ValueError("request needs more KV blocks than the pool holds")
        self.waiting.append(r)

    def prompt_share(self) -> int:
        """Prompt tokens the next iteration may carry once every decode has its token."""
        d = len(self.running)
        if self.adaptive:
            return adaptive_chunk(d, self.min_chunk, self.base_chunk, self.max_chunk,
                                  self.threshold)
        return self.budget - d

    def _admit(self, r: Request) -> bool:
        """Take r off the waiting queue if a sequence slot and its lifetime blocks are free."""
        busy = len(self.running) + len(self.prefilling)
        need = lifetime_blocks(r)
        if busy >= self.max_seqs or need > len(self.free):
            return False
        self.waiting.pop(0)
        r.blocks, self.free = self.free[:need], self.free[need:]
        self.prefilling.append(r)
        return True

    def next(self) -> List[Dict]:
        """The iteration's sequences: dicts with rid, num_cached, q_len, decode_token, emits,
        blocks (the request's block list)."""
        share = self.prompt_share()
        picked = [(r, 1) for r in self.running]                 # 1. a token per decode
        queue = list(self.prefilling)                           # 2. prompts in progress
        while share > 0:
            if not queue:                                       # 3. arrivals, in order
                if not self.waiting or not self._admit(self.waiting[0]):
                    break
                queue.append(self.prefilling[-1])
            r = queue.pop(0)
            take = min(share, r.prompt_len - r.prefilled)
            picked.append((r, take))
            share -= take
        self.last = picked
        out = []
        for r, n in picked:
            dec = r in self.running
            out.append({"rid": r.rid,
                        "num_cached": r.prompt_len + r.generated - 1 if dec else r.prefilled,
                        "q_len": n, "decode_token": r.last_token if dec else -1,
                        "emits": 1 if dec or r.prefilled + n == r.prompt_len else 0,
                        "blocks": list(r.blocks)})
        return out

    def complete(self, next_tokens: List[int]) -> List[int]:
        """Advance after the pass; returns the ids of requests that finished."""
        done = []
        for (r, n), tok in zip(self.last, next_tokens):
            if r in self.prefilling:
                r.prefilled += n
                if r.prefilled < r.prompt_len:
                    continue
                r.generated, r.last_token = 1, tok                # 5. first token
                self.prefilling.remove(r)
                self.running.append(r)
            else:
                r.generated += 1
                r.last_token = tok
            if r.generated >= r.max_new:
                self.running.remove(r)
                self.free = sorted(self.free + r.blocks)
                r.blocks = []
                done.append(r.rid)
        self.last = []
        return done
