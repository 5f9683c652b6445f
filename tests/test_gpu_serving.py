"""GPU test of the serving loop: the native token-budget scheduler forms each hybrid batch,
hl_model_step runs it, the greedy tokens go back to the scheduler ("Chunked prefill (stall-free
batching), explained", "How it works, step by step"). Each request's logits, whenever it takes a
token, are checked against the fp64 oracle run on that request's whole token sequence in one
shot: a prompt split into chunks over several iterations, with its K/V written to and read back
from the paged cache in between, and the decodes that follow must give the logits of the
unsplit sequence. Tolerance as for the model step: 1e-2 * max|ref| on the logits; the greedy
pick is checked on the GPU's own bf16 logits, exactly."""
import numpy as np
import pytest
import torch

import oracle.model as OM
import workloads
from hybrid_prefill_decode_amd import serving as SV
from tests._gpu import assert_close, say
from tests._util import f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def oracle_logits(eng, layers, tokens):
    """fp64 logits of the last position of one fresh sequence holding `tokens`"""
    s, n = eng.shape, len(tokens)
    empty = np.zeros((0, s.n_kv_heads, s.head_dim))
    table = np.arange((n + 15) // 16, dtype=np.int32)[None, :]
    return OM.model_step(s, np.asarray(tokens, np.int32), f64(eng.tensors["embed"]), layers,
                         f64(eng.tensors["final_norm"]), f64(eng.tensors["lm_head"]), [(0, n)],
                         [[(empty, empty)] for _ in layers], table)["logits"][0]


def test_engine_chunked_requests_vs_oracle():
    shape = workloads.LayerShape(256, 4, 2, 64, 512)
    L, vocab = 2, 512
    eng = SV.Engine(shape, **workloads.engine_model(shape, L, vocab, 48, DEV, seed=7,
                                                    pool_fill=float("nan")),
                    max_blocks_per_seq=16, device=DEV, budget=48, max_seqs=3)
    reqs = {0: (150, 4), 1: (100, 3), 2: (23, 2)}  # prompt length, tokens to generate
    late = {5: 2}  # request 2 arrives before iteration 5
    for rid in (0, 1):
        eng.submit(rid, *reqs[rid])
    layers = [{k: f64(v) for k, v in w.items()} for w in eng.layer_w]
    gen = {rid: [] for rid in reqs}
    it = hybrid = 0
    while True:
        if it in late:
            eng.submit(late[it], *reqs[late[it]])
        r = eng.step()
        if r is None:
            break
        b = eng.last
        say(f"iteration {it}: requests {b['request_ids'].tolist()}, q_start "
            f"{b['q_start'].tolist()}, cached {b['num_cached'].tolist()}")
        hybrid += int(r.decodes > 0 and r.prefill_tokens > 0)
        logits = eng.logits[:len(b["request_ids"])]
        picks = eng.next[:len(b["request_ids"])].cpu().numpy()
        assert np.array_equal(picks, OM.greedy(logits.float().cpu().numpy()))
        for s, rid in enumerate(b["request_ids"].tolist()):
            if not b["emits"][s]:
                continue
            p = reqs[rid][0]
            seq = list(workloads.prompt_token(rid, np.arange(p), vocab)) + gen[rid]
            assert_close(f64(logits[s]), oracle_logits(eng, layers, seq),
                         f"logits of request {rid} token {len(gen[rid])}")
            gen[rid].append(int(picks[s]))
        it += 1
        assert it < 64
    assert hybrid >= 1, "no iteration mixed decodes with a prompt chunk"
    for rid, (_, n) in reqs.items():
        assert len(gen[rid]) == n, (rid, gen[rid])
    assert eng.sched.counts() == (0, 0, 0, 48)
