"""hybrid_layer_step_noalloc (the step with its workspace in the library's fixed per-device
array, for callers that cannot allocate) against hybrid_layer_step with a caller workspace:
out and both pools bit-identical, on two calls in a row, the second with a smaller batch (the
array keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from hybrid_prefill_decode_amd import binding as B
from tests._gpu import DeviceCase, assert_close, bits, say
from tests._util import f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _noalloc(case):
    d = B._desc(case.cfg, case.batch, case.x, None, None)
    wt = B._weights(case.w)
    kv = B._pages(case.kp, case.vp)
    bt = B._table(case.batch)
    return B.lib().hybrid_layer_step_noalloc(ctypes.byref(d), ctypes.byref(wt), ctypes.byref(kv),
                                             ctypes.byref(bt), B._ptr(case.out))


def _compare(spec, label):
    ref = DeviceCase(spec, DEV)
    k0, v0 = ref.kp.clone(), ref.vp.clone()
    ref.step(taps=False)
    torch.cuda.synchronize()
    case = DeviceCase(spec, DEV)
    case.out.fill_(float("nan"))
    assert torch.equal(bits(case.kp), bits(k0)) and torch.equal(bits(case.vp), bits(v0))
    rc = _noalloc(case)
    assert rc == B.HL_OK, B.strerror(rc)
    torch.cuda.synchronize()
    assert_close(f64(case.out), f64(ref.out), f"{label} out vs hybrid_layer_step")
    assert torch.equal(bits(case.out), bits(ref.out)), f"{label}: out not bit-identical"
    assert torch.equal(bits(case.kp), bits(ref.kp)) and torch.equal(bits(case.vp), bits(ref.vp))


def test_noalloc_step_matches_step_twice_second_smaller():
    assert torch.cuda.is_available()
    big = workloads.make_spec(1)
    say(f"noalloc call 1: {big.seqs} (T={big.num_tokens})")
    _compare(big, "call 1")
    small = workloads.custom_spec(workloads.SHAPES["tiny"], [(5, 20), (40, 1), (16, 1)], 9)
    assert small.num_tokens < big.num_tokens
    say(f"noalloc call 2: {small.seqs} (T={small.num_tokens})")
    _compare(small, "call 2")
