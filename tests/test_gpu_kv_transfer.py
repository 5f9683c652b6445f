"""GPU parity of the KV transfer entry points (hl_kv_export / hl_kv_import) against the oracle's
gather / scatter, bit for bit on raw bf16 bits (NaN payloads included): the exported layer slice,
every byte of the transfer buffer outside it, and after an import every byte of both pools.
"""
import numpy as np
import pytest
import torch

import oracle.kv_transfer as OKV
from hybrid_prefill_decode_amd import binding as B
from hybrid_prefill_decode_amd import kvcache as KC
from tests._gpu import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def _kbits(k_pool):
    """Raw bits of a K pool in the logical page layout [blocks, Hkv, 16 tokens, d] the oracle
    uses (the device pages are chunk-major; the permutation moves bits, no arithmetic)."""
    return KC.k_token_major(k_pool.view(torch.int16)).cpu().numpy()


def _rand_bits(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randint(-32768, 32767, shape, generator=g, device=DEV, dtype=torch.int16).view(torch.bfloat16)


CASES = [  # (Hkv, d, pool blocks, start, count)
    (8, 128, 300, 0, 4096),      # a 4096-token prompt of a Qwen3-8B-shaped layer, whole pages
    (8, 128, 300, 37, 1000),     # ragged on both ends
    (2, 64, 40, 15, 1),          # one token at the end of a page
    (4, 128, 40, 16, 16),        # exactly one page
    (3, 64, 60, 5, 300),
    (1, 128, 9, 0, 17),
]


@pytest.mark.parametrize("hkv,d,nblk,start,count", CASES)
def test_kv_export_import_bit_exact(hkv, d, nblk, start, count):
    say(f"kv transfer hkv={hkv} d={d} start={start} count={count}")
    L, layer = 3, 1
    npages = (start + count + 15) // 16 + 2
    rng = np.random.default_rng(count + d)
    row_a = rng.permutation(nblk)[:npages].astype(np.int32)
    kA, vA = _rand_bits(KC.k_pool_shape(nblk, hkv, d), 1), _rand_bits((nblk, hkv, d, 16), 2)
    dst = _rand_bits((L, 2, count, hkv, d), 3)  # other layers must keep these bits
    dst0 = _bits(dst)
    ta = torch.from_numpy(row_a).to(DEV)
    B.kv_export(kA, vA, ta, row_a, start, count, layer, dst)
    torch.cuda.synchronize()
    want = dst0.copy()
    OKV.export_layer(_kbits(kA), _bits(vA), row_a, start, count, layer, want)
    got = _bits(dst)
    assert np.array_equal(got, want), "export differs from the oracle gather"

    # import into another pool under another table: every byte equals the oracle scatter
    nblk_b = nblk + 11
    row_b = rng.permutation(nblk_b)[:npages].astype(np.int32)
    kB, vB = _rand_bits(KC.k_pool_shape(nblk_b, hkv, d), 4), _rand_bits((nblk_b, hkv, d, 16), 5)
    kB_ref, vB_ref = _kbits(kB), _bits(vB)
    OKV.import_layer(got, row_b, start, count, layer, kB_ref, vB_ref)
    tb = torch.from_numpy(row_b).to(DEV)
    B.kv_import(dst, tb, row_b, start, count, layer, kB, vB)
    torch.cuda.synchronize()
    assert np.array_equal(_kbits(kB), kB_ref), "import K pool differs from the oracle scatter"
    assert np.array_equal(_bits(vB), vB_ref), "import V pool differs from the oracle scatter"

    # round trip: exporting the imported span gives the same slice
    again = _rand_bits((L, 2, count, hkv, d), 6)
    B.kv_export(kB, vB, tb, row_b, start, count, layer, again)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(again)[layer], got[layer])
