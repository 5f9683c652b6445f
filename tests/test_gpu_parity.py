"""GPU parity: every phase and the whole hybrid layer step against the fp64 oracle, through the
C ABI. Tolerance (from the step's bf16 storage / fp32 accumulation): max|gpu - ref| <=
1e-2 * max|ref| per output tensor, attention checked separately on prompt-chunk rows and decode
rows. KV placement is bit-exact: the set of written (block, head, slot) addresses equals the
oracle's, and every other byte of both pools is unchanged.
"""
import math

import numpy as np
import pytest
import torch

import oracle.layer as OL
import workloads
from hybrid_prefill_decode_amd import binding as B
from hybrid_prefill_decode_amd import kvcache as KC
from tests._gpu import (DeviceCase, assert_close, bits, changed_slots, k_rows, make_pools,
                        rel_err, say, SENTINEL)
from tests._util import f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()
    yield
    torch.cuda.synchronize()


def _randn(shape, seed, std=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(*shape, generator=g, device=DEV) * std).to(torch.bfloat16)


# ------------------------------------------------------------------------------- phases

@pytest.mark.parametrize("m,n,k", [(1, 128, 64), (68, 512, 256), (130, 384, 320), (257, 256, 128),
                                   (1040, 1024, 512)])
@pytest.mark.parametrize("epi", [B.HL_EPI_NONE, B.HL_EPI_RESIDUAL, B.HL_EPI_SWIGLU])
@pytest.mark.parametrize("scaled", [False, True])
def test_gemm_vs_oracle(m, n, k, epi, scaled):
    say(f"gemm m={m} n={n} k={k} epi={epi} row_scale={scaled}")
    a = _randn((m, k), 1 + m)
    w = _randn((n, k), 2 + n, 0.05)
    res = _randn((m, n // 2 if epi == B.HL_EPI_SWIGLU else n), 3 + k)
    rs = (0.5 + torch.rand(m, generator=torch.Generator(device=DEV).manual_seed(m), device=DEV)) \
        if scaled else None
    out_n = n // 2 if epi == B.HL_EPI_SWIGLU else n
    c = torch.full((m, out_n), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.gemm_bf16_nt(a, w, c, res if epi == B.HL_EPI_RESIDUAL else None, epi, row_scale=rs)
    torch.cuda.synchronize()
    A, W = f64(a), f64(w)
    if scaled:
        A = A * f64(rs)[:, None]  # s * (A W^T) == (s A) W^T
    if epi == B.HL_EPI_SWIGLU:
        ref = OL.swiglu(A, W, n // 2)
    else:
        ref = OL.linear(A, W)
        if epi == B.HL_EPI_RESIDUAL:
            ref = ref + f64(res)
    assert_close(f64(c), ref, "gemm")


@pytest.mark.parametrize("m,n,k", [(1040, 1024, 512), (300, 512, 1024), (1, 256, 256)])
@pytest.mark.parametrize("epi", [B.HL_EPI_NONE, B.HL_EPI_RESIDUAL])
def test_gemm_streamk_vs_oracle(m, n, k, epi):
    """With a workspace the plain / residual GEMM may split tiles over workgroups (stream-K):
    fp32 pieces summed by the fix-up kernel. Small K runs make every tile a multi-piece one."""
    say(f"gemm stream-K m={m} n={n} k={k} epi={epi}")
    a = _randn((m, k), 21 + m)
    w = _randn((n, k), 22 + n, 0.05)
    res = _randn((m, n), 23 + k)
    ws = torch.empty(B.gemm_workspace_bytes(m, n, k, epi), dtype=torch.uint8, device=DEV)
    c = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.gemm_bf16_nt(a, w, c, res if epi == B.HL_EPI_RESIDUAL else None, epi, workspace=ws)
    torch.cuda.synchronize()
    ref = OL.linear(f64(a), f64(w))
    if epi == B.HL_EPI_RESIDUAL:
        ref = ref + f64(res)
    assert_close(f64(c), ref, "gemm stream-K")


@pytest.mark.parametrize("tile", B.GEMM_TILES, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("epi,stream_k", [(B.HL_EPI_NONE, 0), (B.HL_EPI_RESIDUAL, 0),
                                          (B.HL_EPI_SWIGLU, 0), (B.HL_EPI_NONE, 1),
                                          (B.HL_EPI_RESIDUAL, 1), (B.HL_EPI_SWIGLU, 2),
                                          (B.HL_EPI_SWIGLU, 3), (B.HL_EPI_NONE, 3),
                                          (B.HL_EPI_RESIDUAL, 2)],
                         ids=["plain", "residual", "swiglu", "plain-sk", "residual-sk",
                              "swiglu-split2", "swiglu-split3", "plain-split3",
                              "residual-split2"])
def test_gemm_every_tile_shape(tile, epi, stream_k):
    """Every compiled tile shape, one tile per workgroup, stream-K and split-K, through the
    explicit-tile entry point. 300 rows leave a ragged last M tile for every BM; the stream-K shape
    (2100 x 8192 x 192: 3 k-steps per tile, runs of 4 or more) mixes tiles split across runs
    (fix-up) with tiles whole inside one run (finished in the main kernel); split-K cuts the 5
    k-steps of K = 320 into unequal ranges (2 + 3, or 1 + 2 + 2). Both use a row scale."""
    bm, bn = tile
    shapes = [(300, 512, 320)] + ([(2100, 8192, 192)] if stream_k == 1 else [])
    for m, n, k in shapes:
        say(f"gemm tile {bm}x{bn} stream_k={stream_k} epi={epi} m={m} n={n} k={k}")
        a = _randn((m, k), 41 + m + bm)
        w = _randn((n, k), 42 + n + bn, 0.05)
        out_n = n // 2 if epi == B.HL_EPI_SWIGLU else n
        res = _randn((m, out_n), 43 + k) if epi == B.HL_EPI_RESIDUAL else None
        rs = (0.5 + torch.rand(m, generator=torch.Generator(device=DEV).manual_seed(m),
                               device=DEV)) if stream_k else None
        ws = torch.empty(B.gemm_workspace_bytes(m, n, k, epi), dtype=torch.uint8, device=DEV) \
            if stream_k else None
        c = torch.full((m, out_n), float("nan"), dtype=torch.bfloat16, device=DEV)
        B.gemm_bf16_nt_tiled(a, w, c, bm, bn, stream_k, res, epi, workspace=ws, row_scale=rs)
        torch.cuda.synchronize()
        A, W = f64(a), f64(w)
        if rs is not None:
            A = A * f64(rs)[:, None]
        if epi == B.HL_EPI_SWIGLU:
            ref = OL.swiglu(A, W, n // 2)
        else:
            ref = OL.linear(A, W)
            if epi == B.HL_EPI_RESIDUAL:
                ref = ref + f64(res)
        assert_close(f64(c), ref, f"gemm {bm}x{bn} sk={stream_k}")


@pytest.mark.parametrize("tile", B.SWIGLU_TILES, ids=lambda t: f"{t[0]}x{t[1]}")
def test_gemm_swiglu_192_wide_tiles(tile):
    """The 192-wide SwiGLU tiles (96 gate and 96 up rows each), one tile per workgroup, through the
    explicit-tile entry point: 300 rows leave a ragged last M tile and K = 320 gives an odd count
    of 5 k-steps (the deeper load pipeline of 128 x 192 starts one step early on zeros); then the
    gate/up projection of a 512-token chunk of the 8B-shaped layer (512 x 24576 x 4096, the shape
    these tiles exist for), checked on 48 sampled rows. Both apply a row scale."""
    bm, bn = tile
    for m, n, k, rows in ((300, 768, 320, None), (512, 24576, 4096, 48)):
        say(f"gemm swiglu tile {bm}x{bn} m={m} n={n} k={k}")
        a = _randn((m, k), 51 + m + bm)
        w = _randn((n, k), 52 + n + bm, 0.02)
        rs = 0.5 + torch.rand(m, generator=torch.Generator(device=DEV).manual_seed(m), device=DEV)
        c = torch.full((m, n // 2), float("nan"), dtype=torch.bfloat16, device=DEV)
        B.gemm_bf16_nt_tiled(a, w, c, bm, bn, 0, None, B.HL_EPI_SWIGLU, row_scale=rs)
        torch.cuda.synchronize()
        idx = np.arange(m) if rows is None else np.unique(np.concatenate([
            [0, bm - 1, bm, m - 1], np.random.default_rng(m).permutation(m)[:rows - 4]]))
        A = f64(a)[idx] * f64(rs)[idx][:, None]
        ref = OL.swiglu(A, f64(w), n // 2)
        assert_close(f64(c)[idx], ref, f"swiglu gemm {bm}x{bn} m={m}")


@pytest.mark.parametrize("tile", B.GEMM_TILES, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("epi,splits", [(B.HL_EPI_NONE, 2), (B.HL_EPI_RESIDUAL, 3),
                                        (B.HL_EPI_SWIGLU, 2), (B.HL_EPI_SWIGLU, 3)],
                         ids=["plain-2", "residual-3", "swiglu-2", "swiglu-3"])
def test_gemm_tail_split(tile, epi, splits):
    """Tail split: one full round of 256 whole tiles, then the 8..16 tiles left over cut into 2 or
    3 K ranges (the 5 k-steps of K = 320 as 2 + 3 or 1 + 2 + 2) in the same launch, finished by the
    split-K fix-up from the right tile on. 300 rows leave a ragged last M tile; a row scale is
    applied."""
    bm, bn = tile
    m, k = 300, 320
    mtiles = -(-m // bm)
    n = bn * -(-264 // mtiles)
    tiles = mtiles * (n // bn)
    assert 256 < tiles <= 256 + 16
    say(f"gemm tail split {bm}x{bn} s={splits} epi={epi} m={m} n={n} k={k} tiles={tiles}")
    a = _randn((m, k), 81 + bm)
    w = _randn((n, k), 82 + bn, 0.05)
    out_n = n // 2 if epi == B.HL_EPI_SWIGLU else n
    res = _randn((m, out_n), 83) if epi == B.HL_EPI_RESIDUAL else None
    rs = 0.5 + torch.rand(m, generator=torch.Generator(device=DEV).manual_seed(9), device=DEV)
    ws = torch.empty(B.gemm_workspace_bytes(m, n, k, epi), dtype=torch.uint8, device=DEV)
    c = torch.full((m, out_n), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.gemm_bf16_nt_tiled(a, w, c, bm, bn, -splits, res, epi, workspace=ws, row_scale=rs)
    torch.cuda.synchronize()
    A, W = f64(a) * f64(rs)[:, None], f64(w)
    if epi == B.HL_EPI_SWIGLU:
        ref = OL.swiglu(A, W, n // 2)
    else:
        ref = OL.linear(A, W)
        if epi == B.HL_EPI_RESIDUAL:
            ref = ref + f64(res)
    assert_close(f64(c), ref, f"gemm tail split {bm}x{bn} s={splits}")


@pytest.mark.parametrize("tile", [(128, 128), (160, 256), (256, 256)], ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("epi", [B.HL_EPI_NONE, B.HL_EPI_RESIDUAL, B.HL_EPI_SWIGLU])
def test_gemm_tall_one_tile(tile, epi):
    """Many M tiles (34, the last ragged) in the one-tile schedule: every tile id maps to one
    output tile, dealt across the XCDs."""
    bm, bn = tile
    m, n, k = 33 * bm + 7, 3 * bn, 128
    say(f"gemm tall {bm}x{bn} epi={epi} m={m} n={n} k={k}")
    a = _randn((m, k), 61 + bm)
    w = _randn((n, k), 62 + bn, 0.05)
    out_n = n // 2 if epi == B.HL_EPI_SWIGLU else n
    res = _randn((m, out_n), 63) if epi == B.HL_EPI_RESIDUAL else None
    c = torch.full((m, out_n), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.gemm_bf16_nt_tiled(a, w, c, bm, bn, 0, res, epi)
    torch.cuda.synchronize()
    A, W = f64(a), f64(w)
    if epi == B.HL_EPI_SWIGLU:
        ref = OL.swiglu(A, W, n // 2)
    else:
        ref = OL.linear(A, W)
        if epi == B.HL_EPI_RESIDUAL:
            ref = ref + f64(res)
    assert_close(f64(c), ref, f"gemm tall {bm}x{bn}")


@pytest.mark.parametrize("tile", [(128, 128), (160, 128), (224, 128), (256, 128)],
                         ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("k", [64, 192, 256])
@pytest.mark.parametrize("epi", [B.HL_EPI_NONE, B.HL_EPI_RESIDUAL])
def test_gemm_load_depth_k_steps(tile, k, epi):
    """The 128-wide tiles run their k-steps in pairs with two staging sets in flight; an odd count
    (1 or 3 here) starts one step early on a tile of zeros, an even one (4) does not."""
    bm, bn = tile
    m, n = 2 * bm + 5, 2 * bn
    say(f"gemm load depth {bm}x{bn} epi={epi} m={m} n={n} k={k}")
    a = _randn((m, k), 71 + k)
    w = _randn((n, k), 72 + bm, 0.05)
    res = _randn((m, n), 73) if epi == B.HL_EPI_RESIDUAL else None
    c = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.gemm_bf16_nt_tiled(a, w, c, bm, bn, 0, res, epi)
    torch.cuda.synchronize()
    ref = OL.linear(f64(a), f64(w))
    if epi == B.HL_EPI_RESIDUAL:
        ref = ref + f64(res)
    assert_close(f64(c), ref, f"gemm load depth {bm}x{bn} k={k}")


@pytest.mark.parametrize("m", [1, 7, 16, 33, 64])
@pytest.mark.parametrize("n,k", [(384, 320), (1024, 4096)])
@pytest.mark.parametrize("epi", [B.HL_EPI_NONE, B.HL_EPI_RESIDUAL, B.HL_EPI_SWIGLU])
def test_gemm_few_tokens_vs_oracle(m, n, k, epi):
    """Up to 64 token rows with a workspace: the split-K weight-streaming path (fp32 partials per
    K chunk, summed in chunk order by the epilogue pass), with a row scale."""
    assert B.gemm_tile_choice(m, n, k, epi, True)[2] == 2
    say(f"gemm few tokens m={m} n={n} k={k} epi={epi}")
    a = _randn((m, k), 51 + m)
    w = _randn((n, k), 52 + n, 0.05)
    out_n = n // 2 if epi == B.HL_EPI_SWIGLU else n
    res = _randn((m, out_n), 53 + k) if epi == B.HL_EPI_RESIDUAL else None
    rs = 0.5 + torch.rand(m, generator=torch.Generator(device=DEV).manual_seed(m), device=DEV)
    ws = torch.empty(B.gemm_workspace_bytes(m, n, k, epi), dtype=torch.uint8, device=DEV)
    c = torch.full((m, out_n), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.gemm_bf16_nt(a, w, c, res, epi, workspace=ws, row_scale=rs)
    torch.cuda.synchronize()
    A, W = f64(a) * f64(rs)[:, None], f64(w)
    if epi == B.HL_EPI_SWIGLU:
        ref = OL.swiglu(A, W, n // 2)
    else:
        ref = OL.linear(A, W)
        if epi == B.HL_EPI_RESIDUAL:
            ref = ref + f64(res)
    assert_close(f64(c), ref, "gemm few tokens")


def _edge_sample(size, tile, count, seed):
    """Indices that include both edges of every tile plus the ragged end, and random fill."""
    idx = {0, size - 1}
    for t in range(0, size, tile):
        idx.update({t, min(t + tile - 1, size - 1)})
    rng = np.random.default_rng(seed)
    idx.update(rng.integers(0, size, count).tolist())
    return torch.tensor(sorted(idx), dtype=torch.long)


# The O and down projections of the layer shapes with the layer's workspace: these are the shapes
# whose schedules differ (128 x 256 or 256 x 256 stream-K, XCD-contiguous or phase-aligned runs).
# The oracle computes a sampled block of outputs: rows at every M tile edge plus random rows,
# columns at every N tile edge plus random columns.
@pytest.mark.parametrize("m,n,k", [(1040, 4096, 4096), (1040, 4096, 12288), (2144, 5120, 17408),
                                   (4160, 4096, 12288), (1024, 8192, 28672)])
def test_gemm_layer_shapes_sampled(m, n, k):
    say(f"gemm layer shape m={m} n={n} k={k} residual, workspace")
    a = _randn((m, k), 31 + m)
    w = _randn((n, k), 32 + n, 0.02)
    res = _randn((m, n), 33 + k)
    ws = torch.empty(B.gemm_workspace_bytes(m, n, k, B.HL_EPI_RESIDUAL), dtype=torch.uint8,
                     device=DEV)
    c = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.gemm_bf16_nt(a, w, c, res, B.HL_EPI_RESIDUAL, workspace=ws)
    torch.cuda.synchronize()
    rows, cols = _edge_sample(m, 128, 48, m), _edge_sample(n, 256, 48, n)
    A, W = f64(a[rows.to(DEV)]), f64(w[cols.to(DEV)])
    ref = OL.linear(A, W) + f64(res[rows.to(DEV)][:, cols.to(DEV)])
    got = f64(c[rows.to(DEV)][:, cols.to(DEV)])
    assert_close(got, ref, "gemm layer shape (sampled)")
    assert not torch.isnan(c).any().item(), "unwritten outputs"


@pytest.mark.parametrize("rows,cols", [(1, 256), (68, 256), (5, 8192), (3, 20480)])
def test_rmsnorm_vs_oracle(rows, cols):
    say(f"rmsnorm rows={rows} cols={cols}")
    x = _randn((rows, cols), 10 + cols)
    g = (1.0 + _randn((cols,), 11, 0.1).float()).to(torch.bfloat16)
    y = torch.empty_like(x)
    B.rmsnorm(x, g, y, 1e-6)
    torch.cuda.synchronize()
    assert_close(f64(y), OL.rmsnorm(f64(x), f64(g), 1e-6), "rmsnorm")


@pytest.mark.parametrize("rows,cols", [(1, 256), (68, 4096), (3, 20480)])
def test_rms_scale_vs_oracle(rows, cols):
    say(f"rms_scale rows={rows} cols={cols}")
    x = _randn((rows, cols), 20 + cols)
    g = (1.0 + _randn((cols,), 21, 0.1).float()).to(torch.bfloat16)
    xg = torch.empty_like(x)
    r = torch.empty(rows, dtype=torch.float32, device=DEV)
    B.rms_scale(x, g, xg, r, 1e-6)
    torch.cuda.synchronize()
    assert_close(f64(xg) * f64(r)[:, None], OL.rmsnorm(f64(x), f64(g), 1e-6), "r * xg")
    # with unit gain the scaled row is the input itself, bit for bit
    one = torch.ones(cols, dtype=torch.bfloat16, device=DEV)
    B.rms_scale(x, one, xg, r, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(bits(xg), bits(x))


QKV_CASES = {
    "cfg1": (workloads.SHAPES["tiny"], None),
    "d128": (workloads.LayerShape(1024, 8, 2, 128, 512), [(0, 130), (70000, 1), (33, 1), (15, 17)]),
    # ~6000 rows: 256 x 256 tiles take fewer rounds than 128 x 256 ones, so the RoPE epilogue
    # stages each tile in two 128-row passes
    "wide_d128": (workloads.LayerShape(1024, 8, 2, 128, 512),
                  [(0, 2900), (777, 3000), (5000, 1), (33, 1), (15, 130)]),
    "wide_d64": (workloads.LayerShape(1024, 16, 4, 64, 512),
                 [(3, 3100), (0, 2800), (4095, 1), (16, 1), (250, 100)]),
    # at most 64 tokens: the split-K weight-streaming path and its RoPE / KV-append epilogue pass
    "few_d128": (workloads.LayerShape(1024, 8, 2, 128, 512), [(0, 9), (70000, 1), (33, 1), (15, 17)]),
    "few_d64": (workloads.LayerShape(1024, 16, 4, 64, 512), [(0, 1), (4095, 1), (16, 30), (255, 1)]),
}
# One case per RoPE-epilogue tile shape: the token count decides the tile the QKV projection gets
# (checked against the library's own choice below), so each count below lands on another shape.
_QKV_TILE_ROWS = {(160, 128): 2716, (224, 128): 3382, (256, 128): 4714, (160, 256): 5380,
                  (192, 256): 6749, (224, 256): 8081, (256, 256): 9413, (128, 256): 10782}


def _qkv_rows_case(total):
    return [(0, total - 200), (777, 130), (5000, 1), (33, 1), (15, 66), (4096, 1), (64, 1)]


for _t, _rows in _QKV_TILE_ROWS.items():
    QKV_CASES[f"tile{_t[0]}x{_t[1]}_d128"] = (workloads.LayerShape(1024, 8, 2, 128, 512),
                                             _qkv_rows_case(_rows))
for _t in [(160, 128), (224, 256), (256, 128)]:
    QKV_CASES[f"tile{_t[0]}x{_t[1]}_d64"] = (workloads.LayerShape(1024, 16, 4, 64, 512),
                                            _qkv_rows_case(_QKV_TILE_ROWS[_t]))
# a few hundred rows: too few tiles for the compute units, so the projection runs split-K (K cut
# into equal ranges whose fp32 pieces the fix-up sums before the RoPE / append epilogue)
_QKV_SPLIT = {"split160x128_d128": ((4096, 8, 2, 128), 150),
              "split128x128_d64": ((4096, 16, 4, 64), 100),
              "split224x128_d128": ((4096, 24, 8, 128), 200),
              "split160x128_d64": ((4096, 16, 4, 64), 300)}
for _name, (_dims, _rows) in _QKV_SPLIT.items():
    QKV_CASES[_name] = (workloads.LayerShape(*_dims, 512),
                        [(0, _rows - 69), (777, 40), (5000, 1), (33, 1), (15, 26), (4096, 1)])
# 10884 rows at hidden 4096: 49 x 6 = 294 tiles of 224 x 256, one full round of 256 whole tiles and
# 38 tiles cut into 4 K ranges, whose fix-up rotates and appends from tile 256 on
QKV_CASES["tail224x256_d128"] = (workloads.LayerShape(4096, 8, 2, 128, 512), _qkv_rows_case(10884))


@pytest.mark.parametrize("case", sorted(QKV_CASES))
def test_qkv_rope_append_vs_oracle(case):
    shape, seqs = QKV_CASES[case]
    spec = workloads.make_spec(1) if seqs is None else workloads.custom_spec(shape, seqs, 3)
    say(f"qkv+rope+append {case}: {spec.seqs}")
    s = spec.shape
    if case.startswith(("tile", "split", "tail")):
        want = tuple(int(v) for v in case[4 + case.startswith("split"):].split("_")[0].split("x"))
        qkv_cols = (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim
        got = B.gemm_tile_choice(spec.num_tokens, qkv_cols, s.hidden, B.HL_EPI_NONE, True,
                                 s.head_dim)
        assert got[:2] == want and (got[2] == 3) == case.startswith("split"), (case, got)
        assert (got[2] == 4) == case.startswith("tail"), (case, got)
    table, pool = workloads.block_table(spec)
    cfg = B.layer_cfg(s)
    b = B.Batch(spec.q_start, spec.num_cached, table, DEV)
    x = workloads.hidden_states(spec, DEV)
    w = workloads.weights(spec, DEV, gain_jitter=0.1)
    kp, vp = KC.alloc_pools(pool, s.n_kv_heads, s.head_dim, DEV)
    kp0, vp0 = kp.clone(), vp.clone()
    q_rot = torch.empty(spec.num_tokens, s.n_q_heads * s.head_dim, dtype=torch.bfloat16, device=DEV)
    ws = B.alloc_workspace(cfg, b, DEV)
    B.qkv_rope_append(cfg, b, x, w, q_rot, kp, vp, ws)
    torch.cuda.synchronize()
    hq, hkv, d = s.n_q_heads, s.n_kv_heads, s.head_dim
    h1 = OL.rmsnorm(f64(x), f64(w["attn_norm"]), s.rms_eps)
    qkv = OL.linear(h1, f64(w["w_qkv"]))
    expect = set()
    for si, (c, n) in enumerate(spec.seqs):
        r0 = int(spec.q_start[si])
        pos = c + np.arange(n)
        rows = qkv[r0:r0 + n]
        qr = OL.rope(rows[:, :hq * d].reshape(n, hq, d), pos, s.rope_theta)
        kr = OL.rope(rows[:, hq * d:(hq + hkv) * d].reshape(n, hkv, d), pos, s.rope_theta)
        vv = rows[:, (hq + hkv) * d:].reshape(n, hkv, d)
        assert_close(f64(q_rot[r0:r0 + n]).reshape(n, hq, d), qr, f"q_rot seq {si}")
        blk, slot = OL.kv_slot_addresses(table[si], pos, 16)
        tb, ts = torch.from_numpy(blk).to(DEV), torch.from_numpy(slot).to(DEV)
        assert_close(f64(k_rows(kp, tb, ts)), kr, f"K rows seq {si}")
        assert_close(f64(vp[tb, :, :, ts]), vv, f"V rows seq {si}")
        expect |= {(int(bb), h, int(ss)) for bb, ss in zip(blk, slot) for h in range(hkv)}
    assert changed_slots(kp0, kp, vp0, vp) == expect


def _attention_inputs(spec, seed):
    """Pools holding seeded K/V for every position 0..c+n-1 (the state after the append) and a
    seeded q_rot, so attention is checked on its own."""
    s = spec.shape
    table, pool = workloads.block_table(spec)
    full = workloads.custom_spec(s, [(c + n, n) for c, n in spec.seqs], spec.seed)
    kp, vp = make_pools(full, table, pool, DEV)
    q = _randn((spec.num_tokens, s.n_q_heads * s.head_dim), seed)
    return table, pool, full, kp, vp, q


def _oracle_attention(spec, full, q):
    s = spec.shape
    ref = np.zeros((spec.num_tokens, s.n_q_heads * s.head_dim))
    Q = f64(q).reshape(spec.num_tokens, s.n_q_heads, s.head_dim)
    for si, (c, n) in enumerate(spec.seqs):
        k, v = workloads.cached_kv(full, si, DEV)
        r0 = int(spec.q_start[si])
        pos = c + np.arange(n)
        o = OL.causal_attention(Q[r0:r0 + n], f64(k), f64(v), pos, 1.0 / math.sqrt(s.head_dim))
        ref[r0:r0 + n] = o.reshape(n, -1)
    return ref


ATTN_CASES = {
    "cfg1": (workloads.SHAPES["tiny"], None),
    "ragged": (workloads.SHAPES["tiny"], [(0, 2), (3, 129), (45, 1), (0, 1), (15, 1), (16, 1),
                                          (31, 33), (1000, 1), (511, 1)]),
    "g16_d128": (workloads.LayerShape(2048, 16, 1, 128, 512), [(100, 77), (600, 1), (17, 1)]),
    # 16 query heads per KV head at d = 64 with multi-unit decodes (the merge's wide-group build)
    "g16_d64": (workloads.LayerShape(2048, 32, 2, 64, 512), [(300, 40), (900, 1), (255, 1)]),
    "g5_d128": (workloads.LayerShape(1280, 10, 2, 128, 512), [(40, 300), (2047, 1), (2048, 1)]),
    # fused launch with far more decode units than prefill items, and the other way round
    "many_decodes": (workloads.SHAPES["tiny"], [(7, 200)] + [(17 * i % 1500, 1) for i in range(300)]),
    "many_prefill": (workloads.LayerShape(1280, 10, 2, 128, 512),
                     [(64 * i, 257 + 31 * i) for i in range(6)] + [(900, 1), (3, 1)]),
    # prefill tiles cut into key-range parts and merged: a short chunk after a long prefix, a
    # d = 128 chunk with a ragged last tile, a causal chunk alone (its last tiles are the longest,
    # split where they exceed 8 key tiles; 1500 rows leave a ragged last tile)
    "split_long_prefix": (workloads.SHAPES["tiny"], [(3000, 100), (2500, 1), (40, 1)]),
    "split_d128": (workloads.LayerShape(1024, 8, 2, 128, 512), [(5000, 200), (70, 1)]),
    "split_causal": (workloads.LayerShape(1024, 8, 2, 128, 512), [(0, 1500)]),
    # more sequences than one round of the list build takes (1024 at a time in the attention entry
    # points): 1100 short decodes, then a prompt chunk in the second round
    "rounds_1100": (workloads.SHAPES["tiny"],
                    [((7 * i) % 300 + (2000 if i % 10 == 0 else 0), 1) for i in range(1100)] + [(50, 130)]),
    # decode-heavy at d = 128: fused, each worker runs several decode units in a row and prefetches
    # the next one (contexts 0 mod 16, 15 mod 16 and in between)
    "decode_heavy_d128": (workloads.LayerShape(1024, 8, 2, 128, 512),
                          [(37, 70)] + [(2000 + 97 * i + (i % 3) * 7, 1) for i in range(200)]),
}


@pytest.mark.parametrize("attention", [B.HL_ATTN_AUTO, B.HL_ATTN_FUSED],
                         ids=["auto", "fused"])
@pytest.mark.parametrize("case", sorted(ATTN_CASES))
def test_attention_paths_vs_oracle(case, attention):
    shape, seqs = ATTN_CASES[case]
    spec = workloads.make_spec(1) if seqs is None else workloads.custom_spec(shape, seqs, 77)
    say(f"attention {case}: seqs={spec.seqs[:6]}")
    table, pool, full, kp, vp, q = _attention_inputs(spec, 5)
    cfg = B.layer_cfg(spec.shape)
    b = B.Batch(spec.q_start, spec.num_cached, table, DEV, attention=attention)
    if attention == B.HL_ATTN_FUSED and spec.num_tokens > len(spec.seqs) and \
            any(n == 1 for _, n in spec.seqs):
        assert B.attention_plan(cfg, b)["fused"] >= 1
    if case.startswith("split"):
        plan = B.attention_plan(cfg, b)
        say(f"  plan {plan}")
        assert plan["prefill_merges"] > 0, plan
    ws = B.alloc_workspace(cfg, b, DEV)
    out = torch.full_like(q, float("nan"))
    B.attention(cfg, b, q, kp, vp, out, ws)
    torch.cuda.synchronize()
    ref = _oracle_attention(spec, full, q)
    got = f64(out)
    pre = np.concatenate([np.arange(spec.q_start[i], spec.q_start[i + 1])
                          for i, (c, n) in enumerate(spec.seqs) if n > 1] or [np.zeros(0, int)])
    dec = np.array([spec.q_start[i] for i, (c, n) in enumerate(spec.seqs) if n == 1], dtype=int)
    if pre.size:
        assert_close(got[pre], ref[pre], "prefill attention rows")
    if dec.size:
        assert_close(got[dec], ref[dec], "decode attention rows")
    # each path alone writes only its own rows, bit-identical to the fused launch of both
    out2 = torch.full_like(q, float("nan"))
    B.decode_attention(cfg, b, q, kp, vp, out2, ws)
    torch.cuda.synchronize()
    g2 = f64(out2)
    if pre.size:
        assert np.isnan(g2[pre]).all()
    if dec.size:
        assert np.array_equal(g2[dec], got[dec])
    out3 = torch.full_like(q, float("nan"))
    B.prefill_attention(cfg, b, q, kp, vp, out3, ws)
    torch.cuda.synchronize()
    g3 = f64(out3)
    if dec.size:
        assert np.isnan(g3[dec]).all()
    if pre.size:
        assert np.array_equal(g3[pre], got[pre])


@pytest.mark.parametrize("attention", [B.HL_ATTN_AUTO, B.HL_ATTN_FUSED, B.HL_ATTN_SEPARATE],
                         ids=["auto", "fused", "separate"])
@pytest.mark.parametrize("case", sorted(ATTN_CASES))
def test_attention_two_part_query_vs_oracle(case, attention):
    """The decode path the layer step runs: the query in two bf16 halves (q_hi = bf16(q),
    q_lo = bf16(q - q_hi)), work lists built by their own call, then the kernels (fused or
    separate). Decode rows are checked against the oracle on q_hi + q_lo (exact in fp64), prompt
    rows on q_hi alone; each path run alone gives the same rows bit for bit."""
    shape, seqs = ATTN_CASES[case]
    spec = workloads.custom_spec(shape, seqs, 77) if seqs is not None else workloads.make_spec(1)
    say(f"attention two-part query {case} mode={attention}: seqs={spec.seqs[:6]}")
    table, pool, full, kp, vp, _ = _attention_inputs(spec, 5)
    s = spec.shape
    g = torch.Generator(device=DEV)
    g.manual_seed(606)
    q32 = torch.randn(spec.num_tokens, s.n_q_heads * s.head_dim, generator=g, device=DEV)
    q_hi = q32.to(torch.bfloat16)
    q_lo = (q32 - q_hi.float()).to(torch.bfloat16)
    cfg = B.layer_cfg(s)
    b = B.Batch(spec.q_start, spec.num_cached, table, DEV, attention=attention)
    ws = B.alloc_workspace(cfg, b, DEV)
    out = torch.full_like(q_hi, float("nan"))
    B.attention_build_lists(cfg, b, kp, vp, ws)
    B.attention_run(cfg, b, q_hi, kp, vp, out, ws, q_lo=q_lo, paths=B.ATTN_BOTH)
    torch.cuda.synchronize()
    pre = np.concatenate([np.arange(spec.q_start[i], spec.q_start[i + 1])
                          for i, (c, n) in enumerate(spec.seqs) if n > 1] or [np.zeros(0, int)])
    dec = np.array([spec.q_start[i] for i, (c, n) in enumerate(spec.seqs) if n == 1], dtype=int)
    got = f64(out)
    if pre.size:
        ref_pre = _oracle_attention(spec, full, q_hi)
        assert_close(got[pre], ref_pre[pre], "prefill rows (q_hi)")
    if dec.size:
        q_two = torch.from_numpy(f64(q_hi) + f64(q_lo))
        ref_dec = _oracle_attention(spec, full, q_two)
        assert_close(got[dec], ref_dec[dec], "decode rows (q_hi + q_lo)")
    for paths, rows, other in ((B.ATTN_DECODE, dec, pre), (B.ATTN_PREFILL, pre, dec)):
        o2 = torch.full_like(q_hi, float("nan"))
        B.attention_build_lists(cfg, b, kp, vp, ws)
        B.attention_run(cfg, b, q_hi, kp, vp, o2, ws, q_lo=q_lo, paths=paths)
        torch.cuda.synchronize()
        g2 = f64(o2)
        if rows.size:
            assert np.array_equal(g2[rows], got[rows]), f"paths={paths} rows differ"
        if other.size:
            assert np.isnan(g2[other]).all(), f"paths={paths} wrote other rows"


@pytest.mark.parametrize("attention", [B.HL_ATTN_FUSED, B.HL_ATTN_SEPARATE],
                         ids=["fused", "separate"])
@pytest.mark.parametrize("case", ["ragged", "many_decodes", "split_long_prefix", "g5_d128"])
def test_attention_traced_run(case, attention):
    """hl_attention_run_traced: rows bit-identical to hl_attention_run, and one record per work
    item (start <= end on the constant-rate clock, a valid workgroup), prefill items first."""
    shape, seqs = ATTN_CASES[case]
    spec = workloads.custom_spec(shape, seqs, 77)
    say(f"attention traced {case} mode={attention}")
    table, pool, full, kp, vp, q = _attention_inputs(spec, 5)
    s = spec.shape
    cfg = B.layer_cfg(s)
    b = B.Batch(spec.q_start, spec.num_cached, table, DEV, attention=attention)
    plan = B.attention_plan(cfg, b)
    items = plan["prefill_parts"] * s.n_q_heads + plan["decode_units"] * s.n_kv_heads
    ws = B.alloc_workspace(cfg, b, DEV)
    ref = torch.full_like(q, float("nan"))
    B.attention_build_lists(cfg, b, kp, vp, ws)
    B.attention_run(cfg, b, q, kp, vp, ref, ws)
    out = torch.full_like(q, float("nan"))
    trace = torch.zeros(3 * items + 6, dtype=torch.int64, device=DEV)
    B.attention_build_lists(cfg, b, kp, vp, ws)
    B.attention_run_traced(cfg, b, q, kp, vp, out, ws, trace)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref))
    rec = trace.cpu().numpy()
    assert (rec[3 * items:] == 0).all(), "records past the items"
    rec = rec[:3 * items].reshape(items, 3)
    assert (rec[:, 0] > 0).all() and (rec[:, 1] >= rec[:, 0]).all(), "an item without a record"
    assert (rec[:, 2] >= 0).all() and (rec[:, 2] < max(items, 2 * 256 * 8)).all()
    khz = B.trace_clock_khz()
    span_us = (rec[:, 1].max() - rec[:, 0].min()) * 1000.0 / khz
    say(f"  {items} items over {span_us:.1f} us (clock {khz} kHz)")
    assert 0 < span_us < 1e6


def test_rope_kv_append_vs_oracle():
    spec = workloads.custom_spec(workloads.SHAPES["tiny"], [(64, 64), (32, 1), (57, 1), (0, 3),
                                                            (4095, 1), (100000, 1)], 5, pool_slack=1.0)
    say(f"rope+append seqs={spec.seqs}")
    s = spec.shape
    table, pool = workloads.block_table(spec)
    cfg = B.layer_cfg(s)
    b = B.Batch(spec.q_start, spec.num_cached, table, DEV)
    kp, vp = KC.alloc_pools(pool, s.n_kv_heads, s.head_dim, DEV)
    kp0, vp0 = kp.clone(), vp.clone()
    qkv = _randn((spec.num_tokens, s.qkv_cols), 9)
    q_rot = torch.empty(spec.num_tokens, s.n_q_heads * s.head_dim, dtype=torch.bfloat16, device=DEV)
    B.rope_kv_append(cfg, b, qkv, q_rot, kp, vp)
    torch.cuda.synchronize()
    Q = f64(qkv)
    hq, hkv, d = s.n_q_heads, s.n_kv_heads, s.head_dim
    expect_slots = set()
    for si, (c, n) in enumerate(spec.seqs):
        r0 = int(spec.q_start[si])
        pos = c + np.arange(n)
        rows = Q[r0:r0 + n]
        qr = OL.rope(rows[:, :hq * d].reshape(n, hq, d), pos, s.rope_theta)
        kr = OL.rope(rows[:, hq * d:(hq + hkv) * d].reshape(n, hkv, d), pos, s.rope_theta)
        vv = rows[:, (hq + hkv) * d:].reshape(n, hkv, d)
        assert_close(f64(q_rot[r0:r0 + n]).reshape(n, hq, d), qr, f"q_rot seq {si}")
        blk, slot = OL.kv_slot_addresses(table[si], pos, 16)
        gk = f64(k_rows(kp, torch.from_numpy(blk).to(DEV), torch.from_numpy(slot).to(DEV)))
        gv = f64(vp[torch.from_numpy(blk).to(DEV), :, :, torch.from_numpy(slot).to(DEV)])
        assert_close(gk, kr, f"k rows seq {si}")
        # V is copied, not recomputed: bit-exact with the input bf16
        assert np.array_equal(gv, vv), f"v rows seq {si}"
        for bb, ss in zip(blk.tolist(), slot.tolist()):
            for h in range(hkv):
                expect_slots.add((bb, h, ss))
    got_slots = changed_slots(kp0, kp, vp0, vp)
    assert got_slots == expect_slots
    # nothing else moved: the untouched bytes are still the sentinel
    mask_k = torch.ones(pool, hkv, 16, dtype=torch.bool, device=DEV)
    for (bb, h, ss) in expect_slots:
        mask_k[bb, h, ss] = False
    assert bool((bits(KC.k_token_major(kp))[mask_k] == SENTINEL).all())
    assert bool((bits(vp).permute(0, 1, 3, 2)[mask_k] == SENTINEL).all())


# ------------------------------------------------------------------------------- whole step

def _check_full_step(case, label):
    spec = case.spec
    s = spec.shape
    kp0, vp0 = case.kp.clone(), case.vp.clone()
    case.step()
    torch.cuda.synchronize()
    x, w, cached = case.oracle_host()
    ref = OL.layer_step(s, x, w, spec.seqs, [cached[i] for i in range(spec.num_seqs)], case.table)
    got = f64(case.out)
    assert_close(got, ref["out"], f"{label} out")
    assert_close(f64(case.taps["h2"]), ref["h2"], f"{label} h2")
    assert_close(f64(case.taps["q_rot"]).reshape(ref["q_rot"].shape), ref["q_rot"], f"{label} q_rot")
    att = f64(case.taps["attn_out"])
    pre = np.concatenate([np.arange(spec.q_start[i], spec.q_start[i + 1])
                          for i, (c, n) in enumerate(spec.seqs) if n > 1] or [np.zeros(0, int)])
    dec = np.array([spec.q_start[i] for i, (c, n) in enumerate(spec.seqs) if n == 1], dtype=int)
    if pre.size:
        assert_close(att[pre], ref["attn_out"][pre], f"{label} attn prefill rows")
    if dec.size:
        assert_close(att[dec], ref["attn_out"][dec], f"{label} attn decode rows")
    # placement: exactly the oracle's (block, head, slot) set changed, with the oracle's values
    a = ref["kv_addr"]
    expect = {(int(bb), h, int(ss)) for bb, ss in zip(a[:, 2], a[:, 3]) for h in range(s.n_kv_heads)}
    assert changed_slots(kp0, case.kp, vp0, case.vp) == expect
    bt = torch.from_numpy(a[:, 2]).to(DEV)
    sl = torch.from_numpy(a[:, 3]).to(DEV)
    assert_close(f64(k_rows(case.kp, bt, sl)), ref["k_new"], f"{label} new K rows")
    assert_close(f64(case.vp[bt, :, :, sl]), ref["v_new"], f"{label} new V rows")
    return ref


def test_step_tiny_workload_full():
    say("step cfg1 full")
    case = DeviceCase(workloads.make_spec(1), DEV)
    _check_full_step(case, "cfg1")


def test_step_tiny_with_norm_gains():
    say("step cfg1 gains")
    case = DeviceCase(workloads.make_spec(1), DEV, gain_jitter=0.2)
    _check_full_step(case, "cfg1-gains")


def test_step_ragged_small_layer():
    shape = workloads.LayerShape(512, 8, 2, 128, 1024)
    spec = workloads.custom_spec(shape, [(0, 200), (37, 129), (0, 1), (1234, 1), (16, 1), (5, 2)], 31)
    say(f"step ragged {spec.seqs}")
    _check_full_step(DeviceCase(spec, DEV), "ragged")


def test_step_many_sequences_work_lists():
    """300 sequences, every other one a prompt chunk of 129..378 rows after a short prefix: the
    step's work lists take several rounds of sequences, and the first round holds more query
    tiles and prefill entries than the building workgroup has threads."""
    seqs = [((i * 37) % 600, 129 + (i * 53) % 250) if i % 2 == 0 else ((i * 97) % 3000, 1)
            for i in range(300)]
    spec = workloads.custom_spec(workloads.SHAPES["tiny"], seqs, 5)
    assert sum((n + 127) // 128 for _, n in seqs[:256] if n > 1) > 256
    say(f"step many sequences: T={spec.num_tokens} seqs={spec.num_seqs}")
    _check_full_step(DeviceCase(spec, DEV), "many-seqs")


def test_step_deterministic_and_block_permutation_invariant():
    say("step determinism / permutation")
    spec = workloads.make_spec(1)
    c1 = DeviceCase(spec, DEV)
    c1.step()
    out1 = c1.out.clone()
    k1, v1 = c1.kp.clone(), c1.vp.clone()
    c1.step()  # appends are idempotent: the second run sees the same cache
    torch.cuda.synchronize()
    assert torch.equal(bits(out1), bits(c1.out))
    assert torch.equal(bits(k1), bits(c1.kp)) and torch.equal(bits(v1), bits(c1.vp))
    c2 = DeviceCase(spec, DEV, permute_seed=4242)
    assert not np.array_equal(c2.table, c1.table)
    c2.step()
    torch.cuda.synchronize()
    assert torch.equal(bits(out1), bits(c2.out))


def test_step_phase_events():
    """The step's phase marks (hl_batch_desc::events): every mark is recorded, in phase order,
    the phases add up to the whole step, a list with NULL entries records only its events, and
    the results are bit-identical to a step without marks."""
    say("step phase events")
    spec = workloads.make_spec(2)
    case = DeviceCase(spec, DEV)
    case.step(taps=False)
    torch.cuda.synchronize()
    out0 = case.out.clone()
    st = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(B.HL_STEP_EVENTS)]
    for e in evs:
        e.record(st)  # torch creates the handle at the first record
    torch.cuda.synchronize()
    case.step(taps=False, events=evs)
    torch.cuda.synchronize()
    assert torch.equal(bits(out0), bits(case.out))
    phases = [evs[i].elapsed_time(evs[i + 1]) for i in range(B.HL_STEP_EVENTS - 1)]
    whole = evs[0].elapsed_time(evs[-1])
    say(f"phases ms {[round(p, 4) for p in phases]} whole {whole:.4f}")
    assert all(p >= 0 for p in phases) and whole > 0
    assert abs(sum(phases) - whole) <= 1e-3 * whole + 1e-3
    # attention and the gate/up projection are the step's two largest phases at this size
    assert phases[1] > 0 and phases[4] > 0
    # only the attention bracket: the other events keep their earlier timestamps
    old = evs[0].elapsed_time(evs[3])
    fresh = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in fresh:
        e.record(st)
    torch.cuda.synchronize()
    case.step(taps=False, events=[None, fresh[0], fresh[1], None, None, None, None])
    torch.cuda.synchronize()
    assert fresh[0].elapsed_time(fresh[1]) > 0
    assert evs[0].elapsed_time(evs[3]) == old
    assert torch.equal(bits(out0), bits(case.out))
    with pytest.raises(ValueError):
        case.step(taps=False, events=evs[:3])


# ------------------------------------------------------------------------------- full sizes

def _decode_sample(spec, want, seed):
    """Decode sequences to finish through the oracle: all of them when there are at most `want`,
    otherwise the longest, the shortest, up to four whose new token opens a fresh page (c mod 16
    == 0) and four that fill a page's last slot (c mod 16 == 15), and seeded random ones."""
    dec = [i for i, (c, n) in enumerate(spec.seqs) if n == 1]
    if len(dec) <= want:
        return dec
    ctx = {i: spec.seqs[i][0] for i in dec}
    picks = {max(dec, key=ctx.get), min(dec, key=ctx.get)}
    for r in (0, 15):
        picks.update([i for i in dec if ctx[i] % 16 == r][:4])
    rng = np.random.default_rng(seed)
    rest = [i for i in dec if i not in picks]
    picks.update(int(i) for i in rng.choice(rest, size=want - len(picks), replace=False))
    return sorted(picks)


def _full_size_check(case, label, n_dec=64, pre_rows=(0, 1, 63, 64, 127, 128, 129)):
    """Full-size step on the GPU against the oracle:
      * placement, bit-exact: the set of (block, head, slot) whose bytes changed in either pool
        equals the oracle's addresses of the batch's new tokens (so every other byte of both
        pools is unchanged);
      * q_rot and the new K and V rows of every token (the oracle's norm, QKV projection and
        rotation over the whole token matrix), K/V read back from the slots they were written to;
      * out, attention output and h2 on sampled rows: every decode when there are at most n_dec,
        else n_dec of them (longest, shortest, page-edge contexts, seeded random), and spread rows
        of each prompt chunk, each request finished by the oracle on its own."""
    spec = case.spec
    s = spec.shape
    T = spec.num_tokens
    hq, hkv, d = s.n_q_heads, s.n_kv_heads, s.head_dim
    kp0, vp0 = case.kp.clone(), case.vp.clone()
    case.step()
    torch.cuda.synchronize()
    say(f"  step done; checking placement over {case.kp.shape[0]} blocks")
    pos_all, blk_all, slot_all = [], [], []
    for si, (c, n) in enumerate(spec.seqs):
        pos = c + np.arange(n)
        blk, slot = OL.kv_slot_addresses(case.table[si], pos, 16)
        pos_all.append(pos)
        blk_all.append(blk)
        slot_all.append(slot)
    pos_all, blk_all, slot_all = map(np.concatenate, (pos_all, blk_all, slot_all))
    expect = {(int(b), h, int(sl)) for b, sl in zip(blk_all, slot_all) for h in range(hkv)}
    got = changed_slots(kp0, case.kp, vp0, case.vp)
    assert got == expect, (f"{label}: {len(got - expect)} unexpected slots changed, "
                           f"{len(expect - got)} expected slots untouched")
    say(f"  placement bit-exact: {len(expect)} (block, head, slot) triples")
    del kp0, vp0
    torch.cuda.empty_cache()

    x, w, _ = case.oracle_host([])
    h1 = OL.rmsnorm(x, w["attn_norm"], s.rms_eps)
    qkv = OL.linear(h1, w["w_qkv"])
    q_ref = OL.rope(qkv[:, :hq * d].reshape(T, hq, d), pos_all, s.rope_theta)
    k_ref = OL.rope(qkv[:, hq * d:(hq + hkv) * d].reshape(T, hkv, d), pos_all, s.rope_theta)
    v_ref = qkv[:, (hq + hkv) * d:].reshape(T, hkv, d)
    assert_close(f64(case.taps["q_rot"]).reshape(T, hq, d), q_ref, f"{label} q_rot (all rows)")
    tb = torch.from_numpy(blk_all).to(DEV)
    ts = torch.from_numpy(slot_all).to(DEV)
    assert_close(f64(k_rows(case.kp, tb, ts)), k_ref, f"{label} new K rows (all tokens)")
    assert_close(f64(case.vp[tb, :, :, ts]), v_ref, f"{label} new V rows (all tokens)")
    del qkv, q_ref, k_ref, v_ref

    dec_ids = _decode_sample(spec, n_dec, spec.seed)
    pre_ids = [i for i, (c, n) in enumerate(spec.seqs) if n > 1]
    if dec_ids:
        ctx = sorted(spec.seqs[i][0] for i in dec_ids)
        all_ctx = [c for c, n in spec.seqs if n == 1]
        say(f"  {len(dec_ids)} decodes sampled, contexts {ctx[0]}..{ctx[-1]}")
        assert ctx[0] == min(all_ctx) and ctx[-1] == max(all_ctx)
        for r in (0, 15):
            if any(c % 16 == r for c in all_ctx):
                assert any(c % 16 == r for c in ctx), f"no sampled decode with c mod 16 == {r}"
    out, att, h2 = f64(case.out), f64(case.taps["attn_out"]), f64(case.taps["h2"])
    for si in pre_ids:
        c, n = spec.seqs[si]
        rows = sorted(set(r for r in pre_rows if r < n) | {n - 1, n // 2})
        r0 = int(spec.q_start[si])
        ref = OL.sequence_step(s, x[r0:r0 + n], w, c, *case.cached_host(si), rows=rows)
        g_rows = r0 + np.array(ref["rows"])
        assert_close(out[g_rows], ref["out"], f"{label} prefill seq {si} out rows {rows}")
        assert_close(att[g_rows], ref["attn_out"], f"{label} prefill seq {si} attn rows")
        assert_close(h2[g_rows], ref["h2"], f"{label} prefill seq {si} h2 rows")
    if dec_ids:
        refs = {"out": [], "attn_out": [], "h2": []}
        rows = []
        for si in dec_ids:
            c, _ = spec.seqs[si]
            r0 = int(spec.q_start[si])
            ref = OL.sequence_step(s, x[r0:r0 + 1], w, c, *case.cached_host(si))
            for k in refs:
                refs[k].append(ref[k][0])
            rows.append(r0)
        rows = np.array(rows)
        assert_close(out[rows], np.stack(refs["out"]), f"{label} decode out ({len(rows)} rows)")
        assert_close(att[rows], np.stack(refs["attn_out"]),
                     f"{label} decode attn ({len(rows)} rows)")
        assert_close(h2[rows], np.stack(refs["h2"]), f"{label} decode h2 ({len(rows)} rows)")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfgid,variant", [(2, "mixed"), (3, "mixed"), (4, "mixed"),
                                           (4, "prefill_only"), (4, "decode_only"), (5, "mixed")])
def test_step_full_size(cfgid, variant):
    spec = workloads.make_spec(cfgid, variant)
    say(f"step full size {spec.name}: T={spec.num_tokens} seqs={spec.num_seqs}")
    case = DeviceCase(spec, DEV)
    _full_size_check(case, spec.name)
    del case
    torch.cuda.empty_cache()
