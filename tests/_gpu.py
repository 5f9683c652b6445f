"""GPU-side test plumbing: seeded workloads packed into device buffers in the layout
include/hybrid_layer.h documents, plus comparison helpers. Values come only from `workloads`;
the oracle sees host fp64 copies of the same arrays."""
import sys

import numpy as np
import torch

import workloads
from hybrid_prefill_decode_amd import binding as B
from hybrid_prefill_decode_amd import kvcache as KC
from tests._util import f64

SENTINEL = 0x7FC0  # bf16 quiet NaN: every slot that holds no valid K/V


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


def make_pools(spec, table, pool, device="cuda"):
    """K pool [pool][Hkv][d/8][16][8] and V pool [pool][Hkv][d][16], NaN everywhere except the
    cached positions 0..c-1 of every sequence, which get that sequence's seeded K/V."""
    s = spec.shape
    kp, vp = KC.alloc_pools(pool, s.n_kv_heads, s.head_dim, device)
    for si, (c, _) in enumerate(spec.seqs):
        if c == 0:
            continue
        k, v = workloads.cached_kv(spec, si, device)
        KC.write_positions(kp, vp, table[si], range(c), k, v)
    return kp, vp


def k_rows(kp, blk, slot):
    """K rows [n, Hkv, d] at (block, slot) pairs given as device index tensors."""
    return KC.k_rows_of(kp, blk, slot)


class DeviceCase:
    """One workload on the GPU: inputs, pools, descriptor and output buffers."""

    def __init__(self, spec, device="cuda", permute_seed=None, gain_jitter=0.0, table=None):
        self.spec = spec
        s = self.shape = spec.shape
        if table is None:
            self.table, self.pool = workloads.block_table(spec, permute_seed)
        else:
            self.table, self.pool = table
        self.cfg = B.layer_cfg(s)
        self.batch = B.Batch(spec.q_start, spec.num_cached, self.table, device)
        self.x = workloads.hidden_states(spec, device)
        self.w = workloads.weights(spec, device, gain_jitter=gain_jitter)
        self.kp, self.vp = make_pools(spec, self.table, self.pool, device)
        T = spec.num_tokens
        self.out = torch.empty(T, s.hidden, dtype=torch.bfloat16, device=device)
        self.taps = {
            "q_rot": torch.empty(T, s.n_q_heads * s.head_dim, dtype=torch.bfloat16, device=device),
            "attn_out": torch.empty(T, s.n_q_heads * s.head_dim, dtype=torch.bfloat16, device=device),
            "h2": torch.empty(T, s.hidden, dtype=torch.bfloat16, device=device),
        }
        self.ws = B.alloc_workspace(self.cfg, self.batch, device)

    def step(self, taps=True, events=None):
        B.hybrid_layer_step(self.cfg, self.batch, self.x, self.w, self.kp, self.vp, self.out,
                            self.ws, taps=self.taps if taps else None, events=events)

    def cached_host(self, si):
        """fp64 host copies of sequence si's cached K and V [c, Hkv, d]."""
        k, v = workloads.cached_kv(self.spec, si, self.x.device)
        return f64(k), f64(v)

    def oracle_host(self, seqs=None):
        """fp64 host copies for the oracle: x, weights, cached K/V of `seqs` (default all)."""
        idx = range(self.spec.num_seqs) if seqs is None else seqs
        cached = {}
        for si in idx:
            k, v = workloads.cached_kv(self.spec, si, self.x.device)
            cached[si] = (f64(k), f64(v))
        return f64(self.x), {k: f64(v) for k, v in self.w.items()}, cached


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


TOL = 1e-2  # max|gpu - ref| <= 1e-2 * max|ref| per output tensor (bf16 data, fp32 accumulation)


def assert_close(got, ref, what, tol=TOL):
    e = rel_err(got, ref)
    say(f"  {what}: rel max err {e:.3e}")
    assert e <= tol, f"{what}: rel max err {e:.3e} > {tol}"


def changed_slots(before_k, after_k, before_v, after_v):
    """(block, head, slot) triples whose K or V bytes differ between two pool snapshots."""
    dk = (bits(before_k) != bits(after_k)).any(dim=-1).any(dim=2)  # [pool, Hkv, 16]
    dv = (bits(before_v) != bits(after_v)).any(dim=-2)            # [pool, Hkv, 16]
    idx = torch.nonzero(dk | dv).cpu().numpy()
    return set(map(tuple, idx.tolist()))
