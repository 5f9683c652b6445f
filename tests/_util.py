"""Test-side helpers: marshal the seeded workloads into fp64 numpy arrays for the oracle."""
import numpy as np
import torch

import workloads


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16/float tensor (any device) to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_inputs(spec, device="cpu", gain_jitter=0.0, seqs_for_cache=None):
    """Host fp64 copies of x, the weights and the cached K/V of the sequences listed
    (default: all), drawn by `workloads` on `device`."""
    x = workloads.hidden_states(spec, device)
    w = workloads.weights(spec, device, gain_jitter=gain_jitter)
    idx = range(spec.num_seqs) if seqs_for_cache is None else seqs_for_cache
    cached = {}
    for s in idx:
        k, v = workloads.cached_kv(spec, s, device)
        cached[s] = (f64(k), f64(v))
    table, pool = workloads.block_table(spec)
    return {
        "x": f64(x), "w": {k: f64(v) for k, v in w.items()}, "cached": cached,
        "block_table": table, "pool": pool,
    }
