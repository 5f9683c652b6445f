"""The token-budget scheduler: the oracle against a hand-worked trace and the invariants the
chunked-prefill page states, then the native scheduler (hl_sched_*) against the oracle batch by
batch on random arrivals (integer work: bit-exact). CPU only."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.scheduler as OS
from hybrid_prefill_decode_amd import binding as B

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scheduler_trace.txt")


def _fmt(batch, names):
    return " ".join(f"{names[e['rid']]}:{e['num_cached']}+{e['q_len']}{'*' if e['emits'] else ''}"
                    for e in batch)


def test_oracle_hand_worked_trace():
    want = [l.split(": ", 1)[1].strip() for l in open(GOLDEN) if l[0].isdigit()]
    s = OS.Scheduler(budget=8, max_seqs=2, num_blocks=40)
    names = {0: "A", 1: "B", 2: "C"}
    for rid, p, o in [(0, 10, 3), (1, 5, 1), (2, 3, 2)]:
        s.submit(rid, p, o)
    got = []
    for it in range(len(want)):
        b = s.next()
        got.append(_fmt(b, names))
        s.complete([100 + it] * len(b))
    assert got == want
    assert not s.waiting and not s.prefilling and not s.running and len(s.free) == 40


def _drive(sched_next, sched_complete, submit, reqs, arrivals, iters, rng):
    """Run a scheduler: requests arrive at their iteration; returns the batches."""
    out, k = [], 0
    for it in range(iters):
        while k < len(reqs) and arrivals[k] <= it:
            submit(*reqs[k])
            k += 1
        b = sched_next()
        out.append(b)
        toks = rng.integers(0, 1000, len(b["rid"]) if isinstance(b, dict) else len(b)).tolist()
        sched_complete(toks)
    return out


def _random_workload(seed, n=60):
    rng = np.random.default_rng(seed)
    prompts = np.minimum(np.maximum(1, rng.lognormal(4.0, 1.0, n).astype(int)), 700)
    outs = np.maximum(1, rng.lognormal(2.0, 1.0, n).astype(int))
    arrivals = np.sort(rng.integers(0, 150, n))
    return [(i, int(p), int(o)) for i, (p, o) in enumerate(zip(prompts, outs))], arrivals


@pytest.mark.parametrize("params", [dict(budget=64, max_seqs=8, num_blocks=300),
                                    dict(budget=256, max_seqs=32, num_blocks=120),
                                    dict(budget=17, max_seqs=3, num_blocks=1000),
                                    dict(adaptive=True, max_seqs=16, num_blocks=400, min_chunk=16,
                                         base_chunk=96, max_chunk=400, pressure_threshold=6)])
def test_oracle_invariants(params):
    """Decodes never stall; the budget holds; admission is in arrival order; slots and blocks
    hold; every prompt is processed exactly once in order and yields its outputs."""
    reqs, arrivals = _random_workload(sum(map(ord, str(params))))
    s = OS.Scheduler(**params)
    rng = np.random.default_rng(0)
    byid = {r[0]: r for r in reqs}
    seen_prompt = {r[0]: 0 for r in reqs}
    outputs = {r[0]: 0 for r in reqs}
    admitted = []
    k = 0
    for it in range(2000):
        while k < len(reqs) and arrivals[k] <= it:
            s.submit(*reqs[k])
            k += 1
        running = [r.rid for r in s.running]
        b = s.next()
        if params.get("adaptive"):
            # the prompt share, computed exactly with rationals, plus one token per decode
            d = len(running)
            lo, base, thr = params["min_chunk"], params["base_chunk"], params["pressure_threshold"]
            if d == 0:
                chunk = params["max_chunk"]
            elif d >= thr:
                chunk = lo
            else:
                chunk = math.floor(base - Fraction(d, thr) * (base - lo))
            cap = chunk + d
        else:
            cap = params["budget"]
        assert sum(e["q_len"] for e in b) <= cap
        assert [e["rid"] for e in b[:len(running)]] == running          # decodes first, all of them
        assert all(e["q_len"] == 1 for e in b[:len(running)])
        assert len(b) <= params["max_seqs"]
        blocks = [x for e in b for x in e["blocks"]]
        assert len(blocks) == len(set(blocks))                           # no page shared
        for e in b[len(running):]:
            if e["num_cached"] == 0:
                admitted.append(e["rid"])
            assert e["num_cached"] == seen_prompt[e["rid"]]              # chunks in order
            seen_prompt[e["rid"]] += e["q_len"]
            assert seen_prompt[e["rid"]] <= byid[e["rid"]][1]
            assert e["emits"] == (seen_prompt[e["rid"]] == byid[e["rid"]][1])
        for e in b:
            assert len(e["blocks"]) * 16 >= e["num_cached"] + e["q_len"]
            outputs[e["rid"]] += e["emits"]
        s.complete(rng.integers(0, 1000, len(b)).tolist())
        if k == len(reqs) and not (s.waiting or s.prefilling or s.running):
            break
    assert admitted == sorted(admitted)                                  # arrival order
    assert all(seen_prompt[r[0]] == r[1] for r in reqs)
    assert all(outputs[r[0]] == r[2] for r in reqs)
    assert len(s.free) == params["num_blocks"]


@pytest.mark.parametrize("params", [dict(budget=64, max_seqs=8, num_blocks=300),
                                    dict(budget=512, max_seqs=40, num_blocks=2000),
                                    dict(budget=19, max_seqs=4, num_blocks=90),
                                    dict(adaptive=True, max_seqs=16, num_blocks=500, min_chunk=16,
                                         base_chunk=96, max_chunk=400, pressure_threshold=6)])
def test_native_scheduler_matches_oracle(params):
    reqs, arrivals = _random_workload(7 + params["max_seqs"], n=80)
    mb = 64
    nat = B.Scheduler(max_blocks_per_seq=mb, **params)
    ora = OS.Scheduler(**params)
    rng = np.random.default_rng(1)
    k = 0
    for it in range(3000):
        while k < len(reqs) and arrivals[k] <= it:
            nat.submit(*reqs[k])
            ora.submit(*reqs[k])
            k += 1
        o = ora.next()
        n = nat.next()
        S = len(o)
        assert len(n["request_ids"]) == S, it
        assert n["request_ids"].tolist() == [e["rid"] for e in o]
        assert n["num_cached"].tolist() == [e["num_cached"] for e in o]
        assert np.diff(n["q_start"]).tolist() == [e["q_len"] for e in o]
        assert n["decode_tokens"].tolist() == [e["decode_token"] for e in o]
        assert n["emits"].tolist() == [e["emits"] for e in o]
        for i, e in enumerate(o):
            assert n["table"][i, :len(e["blocks"])].tolist() == e["blocks"]
        toks = rng.integers(0, 1000, S).tolist()
        assert sorted(nat.complete(toks)) == sorted(ora.complete(toks))
        if k == len(reqs) and not (ora.waiting or ora.prefilling or ora.running):
            break
    assert nat.counts() == (0, 0, 0, params["num_blocks"])


def test_native_scheduler_rejects():
    with pytest.raises(B.HLError):
        B.Scheduler(budget=0, max_seqs=1, num_blocks=1, max_blocks_per_seq=1)
    s = B.Scheduler(budget=8, max_seqs=1, num_blocks=10, max_blocks_per_seq=2)
    with pytest.raises(B.HLError):
        s.submit(1, 30, 4)   # 33 tokens need 3 blocks > 2
    with pytest.raises(B.HLError):
        s.submit(2, 0, 4)
    # more blocks than the whole pool holds: refused at submission (it could never be admitted,
    # and arrival-order admission would hold every later request behind it)
    small = B.Scheduler(budget=8, max_seqs=2, num_blocks=3, max_blocks_per_seq=8)
    with pytest.raises(B.HLError):
        small.submit(1, 60, 4)   # 63 tokens: 4 blocks > 3
    small.submit(2, 40, 4)       # 43 tokens: 3 blocks
    with pytest.raises(ValueError):
        OS.Scheduler(budget=8, max_seqs=2, num_blocks=3).submit(1, 60, 4)


def test_native_adaptive_two_prompt_trace():
    """The native scheduler on the hand-worked adaptive trace of tests/golden."""
    path = os.path.join(os.path.dirname(__file__), "golden", "scheduler_adaptive_trace.txt")
    want = [l.split(":", 1)[1].strip() for l in open(path) if l[0].isdigit()]
    s = B.Scheduler(adaptive=True, max_seqs=4, num_blocks=40, min_chunk=4, base_chunk=8,
                    max_chunk=12, pressure_threshold=4, max_blocks_per_seq=8)
    names = {0: "C", 1: "A", 2: "B"}
    for rid, p, o in [(0, 3, 4), (1, 20, 2), (2, 20, 2)]:
        s.submit(rid, p, o)
    got = []
    for it in range(len(want)):
        n = s.next()
        qlen = np.diff(n["q_start"]).tolist()
        got.append(" ".join(f"{names[r]}:{c}+{q}{'*' if e else ''}" for r, c, q, e in
                            zip(n["request_ids"].tolist(), n["num_cached"].tolist(), qlen,
                                n["emits"].tolist())))
        s.complete([100 + it] * len(qlen))
    assert got == want, got
    assert s.counts() == (0, 0, 0, 40)
