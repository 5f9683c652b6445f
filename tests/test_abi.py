"""C-ABI library: it loads without a GPU, exports every symbol the header declares, and rejects
invalid calls on the host before anything is launched (CPU only; no compute call is made).

A validation failure is detected on the host mirrors and returns its own code; had the call gone
on to launch a kernel on this GPU-less machine it would have come back as HL_ERR_HIP instead, so
each expected code also shows that nothing was launched.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest
import torch

import workloads
from hybrid_prefill_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hybrid_layer.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(hl_[a-z_0-9]+|hybrid_layer_step[a-z_0-9]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("hybrid_layer_step", "hl_workspace_bytes", "hl_strerror", "hl_version",
              "hl_rmsnorm", "hl_rms_scale", "hl_gemm_bf16_nt", "hl_qkv_rope_append",
              "hl_rope_kv_append", "hl_attention",
              "hl_prefill_attention", "hl_decode_attention"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), f"{n} declared in include/hybrid_layer.h but not exported"
    # the binding wraps the same set, under the same names
    assert set(_declared_functions()) == set(B._SIGS)


def test_version_and_strerror():
    assert B.lib().hl_version() == B.HL_VERSION
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -99):
        s = B.strerror(code)
        assert isinstance(s, str) and s


# ---------------------------------------------------------------------- host-forced failures

def _fake_batch(seqs, shape=None, table=None, pool=64):
    """Descriptor pieces backed by CPU memory: validation never dereferences device pointers."""
    shape = shape or workloads.SHAPES["tiny"]
    spec = workloads.custom_spec(shape, seqs, seed=1, pool_slack=1.0)
    if table is None:
        table, pool = workloads.block_table(spec)
    b = B.Batch(spec.q_start, spec.num_cached, table, device="cpu")
    return spec, b, pool


def _step(spec, b, pool, ws_bytes=None, cfg=None, x_off=0, out=None):
    cfg = cfg or B.layer_cfg(spec.shape)
    s = spec.shape
    x = torch.zeros(max(spec.num_tokens, 1) * s.hidden + 64, dtype=torch.bfloat16)
    kp = torch.zeros(pool * s.n_kv_heads * 16 * s.head_dim, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    need = B.workspace_bytes(cfg, b) if ws_bytes is None else ws_bytes
    ws = torch.zeros(max(need, 1) + 512, dtype=torch.uint8)
    # 256-byte aligned view of the workspace
    off = (-ws.data_ptr()) % 256
    d = B._desc(cfg, b, None, None, None, with_stream=False)
    d.x = x.data_ptr() + x_off
    d.workspace = ws.data_ptr() + off
    d.workspace_bytes = need
    w = torch.zeros(4096, dtype=torch.bfloat16)
    wt = B.Weights(*([w.data_ptr()] * 6))
    kv = B.KvPages(kp.data_ptr(), vp.data_ptr(), pool)
    bt = B.BlockTable(b.table.data_ptr(), b.h_table.ctypes.data_as(B._c_i32p), b.max_blocks)
    o = torch.zeros_like(x) if out is None else out
    return B.lib().hybrid_layer_step(ctypes.byref(d), ctypes.byref(wt), ctypes.byref(kv),
                                     ctypes.byref(bt), o.data_ptr())


def test_rejects_bad_block_id():
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    b.h_table[1, 0] = pool  # one past the pool
    assert _step(spec, b, pool) == B.HL_ERR_BLOCK
    b.h_table[1, 0] = -1
    assert _step(spec, b, pool) == B.HL_ERR_BLOCK


def test_rejects_row_too_short_for_context():
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    # sequence 0 needs ceil(24 / 16) = 2 pages; a 1-column table cannot hold it
    short = np.ascontiguousarray(b.h_table[:, :1])
    b2 = B.Batch(spec.q_start, spec.num_cached, short, device="cpu")
    assert _step(spec, b2, pool) == B.HL_ERR_BLOCK


def test_rejects_empty_query_and_bad_q_start():
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    b.h_q_start[:] = [0, 4, 4]  # q_len = 0 for sequence 1
    assert _step(spec, b, pool, ws_bytes=1 << 20) == B.HL_ERR_DESC
    b.h_q_start[:] = [1, 4, 5]  # does not start at 0
    assert _step(spec, b, pool, ws_bytes=1 << 20) == B.HL_ERR_DESC
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    b.h_num_cached[0] = -3
    assert _step(spec, b, pool, ws_bytes=1 << 20) == B.HL_ERR_DESC


def test_rejects_misaligned_pointer():
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    assert _step(spec, b, pool, x_off=2) == B.HL_ERR_ALIGN


def test_rejects_small_workspace():
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    need = B.workspace_bytes(B.layer_cfg(spec.shape), b)
    assert need > 0
    assert _step(spec, b, pool, ws_bytes=need - 256) == B.HL_ERR_WORKSPACE


def test_rejects_bad_shapes():
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    bad = [
        workloads.LayerShape(256, 5, 2, 64, 512),    # Hq % Hkv != 0
        workloads.LayerShape(256, 4, 2, 96, 512),    # head_dim not 64 / 128
        workloads.LayerShape(200, 4, 2, 64, 512),    # hidden % 128 != 0
        workloads.LayerShape(256, 4, 2, 64, 500),    # d_ff % 64 != 0
        workloads.LayerShape(256, 34, 2, 64, 512),   # group of 17 heads
    ]
    for s in bad:
        assert _step(spec, b, pool, cfg=B.layer_cfg(s), ws_bytes=1 << 24) == B.HL_ERR_SHAPE, s
    cfg = B.layer_cfg(spec.shape)
    cfg.block_size = 32
    assert _step(spec, b, pool, cfg=cfg, ws_bytes=1 << 24) == B.HL_ERR_SHAPE


def test_rejects_out_aliasing_x_and_null_weights():
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    cfg = B.layer_cfg(spec.shape)
    d = B._desc(cfg, b, None, None, None, with_stream=False)
    assert B.lib().hybrid_layer_step(ctypes.byref(d), None, None, None, None) in (
        B.HL_ERR_NULL, B.HL_ERR_WORKSPACE)


def test_empty_batch_is_a_no_op():
    cfg = B.layer_cfg(workloads.SHAPES["tiny"])
    b = B.Batch(np.array([0]), np.zeros(0), np.full((1, 1), -1), device="cpu")
    assert B.workspace_bytes(cfg, b) == 0
    d = B._desc(cfg, b, None, None, None, with_stream=False)
    assert B.lib().hybrid_layer_step(ctypes.byref(d), None, None, None, None) == B.HL_OK


def test_workspace_bytes_matches_plan_of_all_workloads():
    for cfgid in range(1, 6):
        spec = workloads.make_spec(cfgid)
        table, pool = workloads.block_table(spec)
        b = B.Batch(spec.q_start, spec.num_cached, table, device="cpu")
        n = B.workspace_bytes(B.layer_cfg(spec.shape), b)
        s = spec.shape
        T = spec.num_tokens
        floor = 2 * T * (2 * s.hidden + 2 * s.n_q_heads * s.head_dim + s.d_ff)
        assert floor <= n < floor + (1 << 30), (cfgid, n, floor)


def test_gemm_and_rmsnorm_argument_checks():
    t = torch.zeros(64 * 128, dtype=torch.bfloat16)
    p = t.data_ptr()
    L = B.lib()
    g = L.hl_gemm_bf16_nt
    assert g(p, p, p, None, None, 8, 100, 64, 0, None, 0, None) == B.HL_ERR_ARG  # n % 128
    assert g(p, p, p, None, None, 8, 128, 60, 0, None, 0, None) == B.HL_ERR_ARG  # k % 64
    assert g(p, p, p, None, None, 8, 128, 64, 7, None, 0, None) == B.HL_ERR_ARG  # epilogue
    assert g(p, p, p, None, None, 8, 128, 64, 1, None, 0, None) == B.HL_ERR_NULL  # residual
    assert g(p + 2, p, p, None, None, 8, 128, 64, 0, None, 0, None) == B.HL_ERR_ALIGN
    assert L.hl_rmsnorm(p, p, p, 4, 12, 1e-6, None) == B.HL_ERR_ARG
    assert L.hl_rmsnorm(None, p, p, 4, 16, 1e-6, None) == B.HL_ERR_NULL
    assert L.hl_rms_scale(p, p, p, None, 4, 16, 1e-6, None) == B.HL_ERR_NULL
    assert L.hl_rms_scale(p, p, p, p, 4, 12, 1e-6, None) == B.HL_ERR_ARG


def test_gemm_tiled_argument_checks():
    t = torch.zeros(64 * 128, dtype=torch.bfloat16)
    p = t.data_ptr()
    g = B.lib().hl_gemm_bf16_nt_tiled
    assert g(p, p, p, None, None, 8, 256, 64, 0, 96, 256, 0, None, 0, None) == B.HL_ERR_ARG  # tile
    assert g(p, p, p, None, None, 8, 384, 64, 0, 128, 256, 0, None, 0, None) == B.HL_ERR_ARG  # n % tile_n
    assert g(p, p, p, None, None, 8, 256, 64, 0, 128, 256, 1, None, 0, None) == B.HL_ERR_ARG  # no workspace
    assert g(p, p, p, None, None, 8, 256, 64, 2, 128, 256, 1, p, 1 << 30, None) == B.HL_ERR_ARG  # SwiGLU split
    assert g(p, p, p, None, None, 8, 256, 64, 0, 128, 256, 1, p, 1024, None) == B.HL_ERR_ARG  # small workspace
    assert g(p, p, p, None, None, 8, 256, 60, 0, 128, 256, 0, None, 0, None) == B.HL_ERR_ARG  # k % 64
    assert g(p, p, p, None, None, 0, 256, 64, 0, 128, 256, 0, None, 0, None) == B.HL_OK  # m == 0: nothing
    big = 1 << 30
    assert g(p, p, p, None, None, 8, 256, 256, 0, 128, 256, 5, p, big, None) == B.HL_ERR_ARG  # 5 ranges > 4 k-steps
    assert g(p, p, p, None, None, 8, 256, 64, 2, 128, 256, 2, p, big, None) == B.HL_ERR_ARG  # 2 ranges > 1 k-step
    assert g(p, p, p, None, None, 8, 256, 256, 2, 128, 256, 2, None, 0, None) == B.HL_ERR_ARG  # no workspace
    assert g(p, p, p, None, None, 8, 256, 256, 2, 128, 256, -1, p, big, None) == B.HL_ERR_ARG  # negative
    assert g(p, p, p, None, None, 8, 256, 256, 2, 128, 256, -9, p, big, None) == B.HL_ERR_ARG  # tail > 8
    assert g(p, p, p, None, None, 8, 256, 256, 2, 128, 256, -5, p, big, None) == B.HL_ERR_ARG  # 5 > 4 k-steps
    assert g(p, p, p, None, None, 8, 256, 256, 2, 128, 256, -2, None, 0, None) == B.HL_ERR_ARG  # no workspace
    # the 192-wide tiles: SwiGLU only, one tile per workgroup only, N a multiple of 192
    assert g(p, p, p, None, None, 8, 384, 256, 0, 256, 192, 0, None, 0, None) == B.HL_ERR_ARG  # plain
    assert g(p, p, p, p, None, 8, 384, 256, 1, 128, 192, 0, None, 0, None) == B.HL_ERR_ARG  # residual
    assert g(p, p, p, None, None, 8, 384, 256, 2, 256, 192, 2, p, big, None) == B.HL_ERR_ARG  # split
    assert g(p, p, p, None, None, 8, 384, 256, 2, 128, 192, -2, p, big, None) == B.HL_ERR_ARG  # tail
    assert g(p, p, p, None, None, 8, 640, 256, 2, 256, 192, 0, None, 0, None) == B.HL_ERR_ARG  # N % 192


def test_gemm_swiglu_192_wide_choice():
    """The 192-wide SwiGLU tiles are chosen where they make exactly one round of 256 tiles: the
    gate/up projection of the 8B-shaped layer (N = 2 x 12288, K = 4096) at 512 and 256 rows; not
    at 128 or 1040 rows, and never for a width they do not divide (2 x 28672)."""
    sw = B.HL_EPI_SWIGLU
    assert B.gemm_tile_choice(512, 24576, 4096, sw, True, 0)[:3] == (256, 192, 0)
    assert B.gemm_tile_choice(256, 24576, 4096, sw, True, 0)[:3] == (128, 192, 0)
    assert B.gemm_tile_choice(128, 24576, 4096, sw, True, 0)[1] != 192
    assert B.gemm_tile_choice(1040, 24576, 4096, sw, True, 0)[1] != 192
    assert B.gemm_tile_choice(512, 57344, 8192, sw, True, 0)[1] != 192
    assert B.gemm_tile_choice(512, 24576, 4096, B.HL_EPI_NONE, True, 0)[1] != 192


@pytest.mark.parametrize("epi", [B.HL_EPI_NONE, B.HL_EPI_RESIDUAL, B.HL_EPI_SWIGLU])
def test_gemm_tile_choice_is_valid(epi):
    """The chooser returns a compiled tile shape that divides N, splits only plain / residual
    GEMMs that have a workspace, and keeps whole heads per tile for the QKV projection."""
    rng = np.random.default_rng(epi)
    tiles = set(B.GEMM_TILES)
    for _ in range(300):
        m = int(rng.integers(0, 9000))
        n = 128 * int(rng.integers(1, 400))
        k = 64 * int(rng.integers(1, 500))
        ws = bool(rng.integers(0, 2))
        hd = int(rng.choice([0, 64, 128])) if epi == B.HL_EPI_NONE else 0
        bm, bn, sk, sp = B.gemm_tile_choice(m, n, k, epi, ws, hd)
        if sk == 2:  # weight-streaming path of few token rows
            assert ws and 0 < m <= 64 and bn == 64 and bm == 16 * ((m + 15) // 16), (m, n, k)
            continue
        swiglu_tile = epi == B.HL_EPI_SWIGLU and (bm, bn) in B.SWIGLU_TILES
        assert ((bm, bn) in tiles or swiglu_tile) and n % bn == 0, (m, n, k, bm, bn)
        assert not swiglu_tile or sk == 0, (m, n, k, bm, bn, sk)  # one tile per workgroup only
        assert (sp >= 2) == (sk in (3, 4)), (sk, sp)
        if sk == 1:
            assert ws and hd == 0 and epi != B.HL_EPI_SWIGLU and k >= 256, (m, n, k)
        if sk == 3:  # split-K with a workspace, at least 4 k-steps per range; SwiGLU and the
            # QKV projection split the 128-wide tiles only
            assert ws and k // 64 >= 4 * sp, (m, n, k, sp)
            assert bn == 128 or not (hd or epi == B.HL_EPI_SWIGLU), (m, n, k, bm, bn)
            tiles_n = -(-m // bm) * (n // bn)
            assert sp * tiles_n * bm * bn * 4 <= 256 * 2 * 256 * 256 * 4, (m, n, bm, bn, sp)
        if sk == 4:  # tail split: full rounds of whole tiles, at most half a round left over
            tiles_n = -(-m // bm) * (n // bn)
            rem = tiles_n % 256
            assert ws and tiles_n > 256 and 0 < 2 * rem <= 256 and k // 64 >= 4 * sp, (m, n, k, sp)
            assert sp * rem * bm * bn * 4 <= 256 * 2 * 256 * 256 * 4, (m, n, bm, bn, sp)
        if hd:
            assert bn % hd == 0
    with pytest.raises(RuntimeError):
        B.gemm_tile_choice(8, 100, 64, epi)


def test_gemm_tile_choice_fits_the_batch():
    """The tile-quantisation cliff: a 1040-token batch (1024-token chunk + 16 decodes) gets tiles
    whose row count wastes less than a 256-row tile would (5 x 256 = 1280 rows for 1040)."""
    for n, k, epi in [(4096, 4096, B.HL_EPI_RESIDUAL), (24576, 4096, B.HL_EPI_SWIGLU),
                      (4096, 12288, B.HL_EPI_RESIDUAL)]:
        bm, bn, sk, _ = B.gemm_tile_choice(1040, n, k, epi)
        assert sk or bm * math.ceil(1040 / bm) < 1280, (n, k, bm, bn, sk)


def test_kv_span_argument_checks():
    t = torch.zeros(4096, dtype=torch.bfloat16)
    p = t.data_ptr()
    row = np.array([3, 1, 7], dtype=np.int32)
    pages = B.KvPages(p, p, 8)

    def span(hkv=2, d=128, L=2, layer=1, start=0, count=20, table=row):
        return B.KvSpan(hkv, d, L, layer, start, count, p, table.ctypes.data_as(B._c_i32p),
                        int(table.shape[0]), None)
    L = B.lib()
    e = lambda s, buf=p: L.hl_kv_export(ctypes.byref(s), ctypes.byref(pages), buf)
    i = lambda s, buf=p: L.hl_kv_import(ctypes.byref(s), buf, ctypes.byref(pages))
    for f in (e, i):
        assert f(span(d=96)) == B.HL_ERR_ARG
        assert f(span(hkv=0)) == B.HL_ERR_ARG
        assert f(span(layer=2)) == B.HL_ERR_ARG
        assert f(span(start=40, count=9)) == B.HL_ERR_ARG        # past 16 * table_len
        assert f(span(start=-1)) == B.HL_ERR_ARG
        assert f(span(table=np.array([3, 9, 7], dtype=np.int32), start=10, count=20)) == B.HL_ERR_BLOCK
        assert f(span(table=np.array([3, -1, 7], dtype=np.int32), start=10, count=20)) == B.HL_ERR_BLOCK
        assert f(span(), p + 8) == B.HL_ERR_ALIGN
        assert f(span(), None) == B.HL_ERR_NULL
        assert f(span(count=0)) == B.HL_OK                       # empty span: nothing launched
        # a span whose pages are all valid is accepted up to the launch (which fails here: no GPU)
        assert f(span(table=np.array([3, 9, 7], dtype=np.int32), start=0, count=16)) == B.HL_ERR_HIP


def _plan(shape, seqs):
    spec = workloads.custom_spec(shape, seqs, seed=1)
    table, _ = workloads.block_table(spec)
    return B.attention_plan(B.layer_cfg(shape), B.Batch(spec.q_start, spec.num_cached, table,
                                                       device="cpu"))


def _key_tiles(c, n):
    return [(c + r0 + min(128, n - r0) + 63) // 64 for r0 in range(0, n, 128)]


@pytest.mark.parametrize("name,shape,seqs,splits", [
    # a short chunk after a long prefix: one tile, a long key range -> split
    ("chunk128_at_8064", "qwen3_8b", [(8064, 128)], True),
    # a causal chunk alone with few tiles x heads: its long tiles (> 8 key tiles) split
    ("causal_1500_d128", "small_d128", [(0, 1500)], True),
    # config 2's 1024-token chunk: tiles of at most 16 key tiles, half the slots -> whole tiles
    ("cfg2", "qwen3_8b", [(0, 1024)] + [(8192, 1)] * 16, False),
    # config 3's 2048-token chunk at 16K alone: 640 even items, just above the 512 resident
    # slots, would leave a last round three-quarters idle -> split
    ("cfg3_prefill", "qwen3_14b", [(16384, 2048)], True),
    # the same chunk with config 3's decodes runs fused: decode units fill the prefill tail, so
    # tiles split only when there are fewer prefill items than compute units -> whole tiles
    ("cfg3", "qwen3_14b", [(16384, 2048)] + [(3000, 1)] * 96, False),
    # config 5's 512-token chunk at 8K with 512 decodes: fused, 256 items -> whole tiles
    ("cfg5", "llama_70b", [(8192, 512)] + [(4000, 1)] * 512, False),
    # config 4's 4096-token causal chunk: 1024 uneven items, dispatched longest first -> whole
    ("cfg4", "qwen3_8b", [(0, 4096)] + [(1125, 1)] * 64, False),
    ("tiny_chunk", "tiny", [(64, 64), (32, 1)], False),
])
def test_attention_plan_prefill_parts(name, shape, seqs, splits):
    """Prefill tiles are cut into parts where a few long tiles or a nearly empty last round would
    idle the launch (in a fused launch only below one item per compute unit); the counts agree
    with the parts the split size implies (host-only, on a host without a GPU the library assumes
    256 compute units)."""
    shape = workloads.LayerShape(1024, 8, 2, 128, 512) if shape == "small_d128" else \
        workloads.SHAPES[shape]
    p = _plan(shape, seqs)
    tiles = [k for c, n in seqs if n > 1 for k in _key_tiles(c, n)]
    split = p["prefill_split"]
    parts = [-(-k // split) for k in tiles]
    assert p["prefill_parts"] == sum(parts)
    assert p["prefill_merges"] == sum(1 for q in parts if q > 1)
    assert (p["prefill_merges"] > 0) == splits, p
    if splits:
        assert 8 <= split < max(tiles)
    else:
        assert split >= max(tiles) and p["prefill_parts"] == len(tiles)


def test_attention_plan_argument_checks():
    spec, b, _ = _fake_batch([(3, 1)])
    d = B._desc(B.layer_cfg(spec.shape), b, with_stream=False)
    v = [ctypes.c_int32(0) for _ in range(6)]
    assert B.lib().hl_attention_plan(ctypes.byref(d), *[ctypes.byref(x) for x in v[:5]],
                                     None) == B.HL_ERR_NULL
    assert B.lib().hl_attention_plan(None, *[ctypes.byref(x) for x in v]) == B.HL_ERR_NULL
    p = _plan(workloads.SHAPES["tiny"], [])
    assert p["prefill_parts"] == 0 and p["decode_units"] == 0


def test_attention_option_checks_and_choice():
    spec, b, _ = _fake_batch([(300, 200), (40, 1), (500, 1)])
    cfg = B.layer_cfg(spec.shape)
    n = ctypes.c_size_t(0)
    for bad in (-1, 3):
        b.attention = bad
        d = B._desc(cfg, b, with_stream=False)
        assert B.lib().hl_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == B.HL_ERR_DESC
    # forced modes: fused only when the batch has both paths
    for mode, want in ((B.HL_ATTN_AUTO, 0), (B.HL_ATTN_FUSED, 1), (B.HL_ATTN_SEPARATE, 0)):
        b.attention = mode
        assert B.attention_plan(cfg, b)["fused"] == want, mode
    spec2, b2, _ = _fake_batch([(300, 200)])
    b2.attention = B.HL_ATTN_FUSED
    assert B.attention_plan(B.layer_cfg(spec2.shape), b2)["fused"] == 0


def test_attention_run_argument_checks():
    """hl_attention_run: paths outside 1..3, a misaligned low query half, a NULL output and a
    small workspace are refused on the host; hl_attention_build_lists validates like the step."""
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    cfg = B.layer_cfg(spec.shape)
    s = spec.shape
    need = B.workspace_bytes(cfg, b)
    ws = torch.zeros(need + 512, dtype=torch.uint8)
    off = (-ws.data_ptr()) % 256
    d = B._desc(cfg, b, None, None, None, with_stream=False)
    d.workspace = ws.data_ptr() + off
    d.workspace_bytes = need
    q = torch.zeros(spec.num_tokens * s.n_q_heads * s.head_dim + 64, dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    kp = torch.zeros(pool * s.n_kv_heads * 16 * s.head_dim, dtype=torch.bfloat16)
    kv = B.KvPages(kp.data_ptr(), kp.data_ptr(), pool)
    bt = B.BlockTable(b.table.data_ptr(), b.h_table.ctypes.data_as(B._c_i32p), b.max_blocks)
    run = lambda qlo, out, paths: B.lib().hl_attention_run(
        ctypes.byref(d), q.data_ptr(), qlo, ctypes.byref(kv), ctypes.byref(bt), out, paths)
    for bad in (0, 4, -1):
        assert run(None, o.data_ptr(), bad) == B.HL_ERR_ARG
    assert run(q.data_ptr() + 2, o.data_ptr(), 3) == B.HL_ERR_ALIGN
    assert run(None, None, 2) == B.HL_ERR_NULL
    d.workspace_bytes = need - 256
    assert run(None, o.data_ptr(), 3) == B.HL_ERR_WORKSPACE
    assert B.lib().hl_attention_build_lists(ctypes.byref(d), ctypes.byref(kv),
                                            ctypes.byref(bt)) == B.HL_ERR_WORKSPACE
    b.h_table[1, 0] = pool
    d.workspace_bytes = need
    assert B.lib().hl_attention_build_lists(ctypes.byref(d), ctypes.byref(kv),
                                            ctypes.byref(bt)) == B.HL_ERR_BLOCK


def test_noalloc_step_refuses_batches_beyond_its_array():
    """hybrid_layer_step_noalloc checks the batch's workspace against its fixed array first: a
    batch that needs more gets HL_ERR_WORKSPACE with nothing launched and no device touched."""
    spec = workloads.make_spec(3)
    table, _ = workloads.block_table(spec)
    b = B.Batch(spec.q_start, spec.num_cached, table, "cpu")
    cfg = B.layer_cfg(spec.shape)
    assert B.workspace_bytes(cfg, b) > (192 << 20)
    d = B._desc(cfg, b, with_stream=False)
    assert B.lib().hybrid_layer_step_noalloc(ctypes.byref(d), None, None, None,
                                             None) == B.HL_ERR_WORKSPACE
    assert B.lib().hybrid_layer_step_noalloc(None, None, None, None, None) == B.HL_ERR_NULL


def test_attention_run_traced_argument_checks():
    """The traced run refuses a missing, misaligned or short trace buffer on the host."""
    spec, b, pool = _fake_batch([(20, 4), (7, 1)])
    cfg = B.layer_cfg(spec.shape)
    s = spec.shape
    need = B.workspace_bytes(cfg, b)
    ws = torch.zeros(need + 512, dtype=torch.uint8)
    off = (-ws.data_ptr()) % 256
    d = B._desc(cfg, b, None, None, None, with_stream=False)
    d.workspace = ws.data_ptr() + off
    d.workspace_bytes = need
    q = torch.zeros(spec.num_tokens * s.n_q_heads * s.head_dim + 64, dtype=torch.bfloat16)
    kp = torch.zeros(pool * s.n_kv_heads * 16 * s.head_dim, dtype=torch.bfloat16)
    kv = B.KvPages(kp.data_ptr(), kp.data_ptr(), pool)
    bt = B.BlockTable(b.table.data_ptr(), b.h_table.ctypes.data_as(B._c_i32p), b.max_blocks)
    plan = B.attention_plan(cfg, b)
    items = plan["prefill_parts"] * s.n_q_heads + plan["decode_units"] * s.n_kv_heads
    tr = torch.zeros(3 * items + 8, dtype=torch.int64)
    run = lambda t, n: B.lib().hl_attention_run_traced(
        ctypes.byref(d), q.data_ptr(), None, ctypes.byref(kv), ctypes.byref(bt), q.data_ptr(), 3,
        t, n)
    assert run(None, 3 * items) == B.HL_ERR_NULL
    assert run(tr.data_ptr() + 8, 3 * items) == B.HL_ERR_ALIGN
    assert run(tr.data_ptr(), 3 * items - 1) == B.HL_ERR_ARG
    assert B.lib().hl_trace_clock_khz(None) == B.HL_ERR_NULL


def test_step_events_descriptor():
    """The step's phase marks reach the descriptor as HL_STEP_EVENTS raw handles, NULL where the
    caller passes None; a wrong count or a never-recorded event is refused before any call."""
    class Ev:  # stands in for torch.cuda.Event: only the raw handle is read
        def __init__(self, h):
            self.cuda_event = h
    spec, b, _ = _fake_batch([(20, 4), (7, 1)])
    cfg = B.layer_cfg(spec.shape)
    assert B._desc(cfg, b, with_stream=False).events is None
    evs = [Ev(0x1000 + 16 * i) if i in (1, 2, 6) else None for i in range(B.HL_STEP_EVENTS)]
    d = B._desc(cfg, b, with_stream=False, events=evs)
    arr = ctypes.cast(d.events, ctypes.POINTER(ctypes.c_void_p))
    got = [arr[i] for i in range(B.HL_STEP_EVENTS)]
    assert got == [None, 0x1010, 0x1020, None, None, None, 0x1060]
    with pytest.raises(ValueError):
        B._desc(cfg, b, with_stream=False, events=evs[:-1])
    with pytest.raises(ValueError):
        B._desc(cfg, b, with_stream=False, events=[Ev(0)] + evs[1:])
    # the C struct ends with the events pointer, after the attention mode
    assert B.BatchDesc._fields_[-1][0] == "events"
    assert B.BatchDesc.events.offset >= B.BatchDesc.attention.offset + 4
