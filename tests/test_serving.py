"""Host-side pieces of the serving loop: the roofline step-time model that measured iterations are
compared with, checked against the step times the chunked-prefill page prints for its H100-class
example ("Chunked prefill (stall-free batching), explained": "The bottleneck: prefill-decode
interference", "What chunking costs" and "Worked example"). The page's formula is lost in the
extracted text; these printed numbers fix the reading (compute 2N per token + 4 d L per causal
pair, memory 2N + kappa per cached key, 0.5 ms per iteration)."""
import numpy as np
import pytest

from hybrid_prefill_decode_amd.serving import IterationRecord, step_time_model

# an 8B Llama-3.1 shape at 60 % of 989 TFLOP/s and 80 % of 3.35 TB/s
KW = dict(layer_params=8.0e9, head_params=0.0, hidden=4096, layers=32,
          kv_bytes_per_token=131072, flops=0.6 * 989e12, bw=0.8 * 3.35e12, fixed_ms=0.5)


def rec(decodes=0, ctx=0, chunk=0, prefix=0):
    """one iteration: `decodes` decodes at context `ctx` plus one prompt chunk after `prefix`"""
    pairs = decodes * (ctx + 1) + chunk * prefix + chunk * (chunk + 1) // 2
    return IterationRecord(0.0, decodes + chunk, decodes, chunk, pairs,
                           decodes * ctx + (prefix if chunk else 0),
                           decodes + (1 if chunk else 0))


def prompt_ms(p, c):
    return float(step_time_model([rec(chunk=c, prefix=k * c) for k in range(p // c)], **KW).sum())


def test_page_decode_and_prefill_steps():
    assert step_time_model([rec(decodes=64, ctx=1125)], **KW)[0] == pytest.approx(10.0, abs=0.05)
    assert step_time_model([rec(chunk=4096)], **KW)[0] == pytest.approx(118, abs=0.5)


def test_page_worked_example_mixed_iterations():
    t = step_time_model([rec(64, 1125, 512, 512 * k) for k in range(8)], **KW)
    assert t[0] == pytest.approx(16.2, abs=0.05) and t[-1] == pytest.approx(17.8, abs=0.05)
    assert np.all(np.diff(t) > 0)                  # rising with the cached prefix
    assert t.sum() == pytest.approx(136, abs=1.0)  # the eight chunks finish the prompt


def test_page_chunking_overheads():
    one = prompt_ms(8192, 8192)
    assert one == pytest.approx(251, abs=0.5)
    assert prompt_ms(8192, 128) == pytest.approx(427, abs=1.0)
    for c, ovh in ((256, 0.062), (512, 0.030), (2048, 0.006)):
        assert prompt_ms(8192, c) / one - 1.0 == pytest.approx(ovh, abs=0.0015)


def test_serial_model_adds_kv_time():
    r = [rec(64, 1125, 512, 0)]
    kv_ms = 1000 * KW["kv_bytes_per_token"] * 64 * 1125 / KW["bw"]
    ser = step_time_model(r, overlap=False, **KW)[0]
    comp_ms = 1000 * (2 * 8e9 * 576 + 4 * 4096 * 32 * (64 * 1126 + 512 * 513 // 2)) / KW["flops"]
    assert ser == pytest.approx(max(comp_ms, 1000 * 16e9 / KW["bw"]) + kv_ms + 0.5, rel=1e-9)
    assert ser > step_time_model(r, **KW)[0]
