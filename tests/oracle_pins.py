"""Checks that pin the fp64 oracle to facts other than its own code.

Each check is a plain function so that tests/test_oracle_mutants.py can re-run the whole set
against deliberately broken copies of the oracle and confirm that every planted mistake is
caught. Sources of truth used here:
  * brute force (pure-Python loops with math.exp) on tiny inputs;
  * library routines: torch fp64 scaled_dot_product_attention with an explicit k_pos <= q_pos
    mask (the rule of "7.8 Disaggregated Prefill/Decode & Chunked Prefill", "Attention on Partial
    KV Caches"), repeat_interleave for GQA (its GQA exercise), torch rms_norm / silu / linear;
  * closed forms (single visible key, equal keys, equal values, hand-worked 2-token case,
    hand-worked rotary and RMSNorm values);
  * invariants the pages state: linear rows are independent and each request attends only to its
    own KV ("ConfluxServe" summary, "Why can linear layers be batched but attention cannot?"),
    chunked prefill equals one-shot prefill (chapter 7.8, "Choosing the Chunk Size C"), a finished
    prompt continues as a decode ("Chunked prefill ... explained", "How it works, step by step").
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle.kv_transfer as OKV
import oracle.model as OM
import oracle.scheduler as OS
import oracle.layer as OL
import workloads

TOL = 1e-12


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------- attention

def check_attention_bruteforce():
    rng = np.random.default_rng(7)
    hq, hkv, d, L = 4, 2, 3, 6
    n = 3
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    q_pos = np.array([3, 4, 5])
    scale = 0.7
    got = OL.causal_attention(q, k, v, q_pos, scale)
    g = hq // hkv
    for i in range(n):
        for h in range(hq):
            kv = h // g
            sc = []
            for j in range(q_pos[i] + 1):
                sc.append(sum(q[i, h, t] * k[j, kv, t] for t in range(d)) * scale)
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = sum(e)
            for t in range(d):
                ref = sum(e[j] * v[j, kv, t] for j in range(len(e))) / z
                assert abs(got[i, h, t] - ref) < 1e-12, (i, h, t)


def check_attention_sdpa_library():
    rng = np.random.default_rng(11)
    for c, n in ((0, 5), (7, 4), (9, 1)):
        hq, hkv, d = 6, 2, 8
        L = c + n
        q = rng.standard_normal((n, hq, d))
        k = rng.standard_normal((L, hkv, d))
        v = rng.standard_normal((L, hkv, d))
        pos = c + np.arange(n)
        got = OL.causal_attention(q, k, v, pos, 1.0 / math.sqrt(d))
        tq = torch.from_numpy(q).permute(1, 0, 2)
        tk = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
        tv = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
        if c == 0:
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
        else:
            mask = torch.arange(L)[None, :] <= torch.from_numpy(pos)[:, None]
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
        assert _rel(got, ref.permute(1, 0, 2).numpy()) < TOL, (c, n)


def check_attention_closed_forms():
    rng = np.random.default_rng(3)
    d = 4
    # a query at position 0 sees only key 0: the output is V row 0
    k = rng.standard_normal((5, 1, d))
    v = rng.standard_normal((5, 1, d))
    q = rng.standard_normal((1, 1, d))
    o = OL.causal_attention(q, k, v, np.array([0]), 0.5)
    assert _rel(o[0, 0], v[0, 0]) < TOL
    # all keys equal: uniform weights over the visible rows -> mean of V[0..p]
    k_eq = np.repeat(rng.standard_normal((1, 1, d)), 5, axis=0)
    o = OL.causal_attention(q, k_eq, v, np.array([3]), 0.5)
    assert _rel(o[0, 0], v[:4, 0].mean(axis=0)) < TOL
    # all values equal u: output is u whatever the weights
    u = rng.standard_normal(d)
    v_eq = np.tile(u, (5, 1, 1))
    o = OL.causal_attention(rng.standard_normal((2, 1, d)), k, v_eq, np.array([2, 4]), 0.9)
    assert _rel(o[:, 0], np.stack([u, u])) < TOL
    # hand-worked: q1 = (0, 1), k0 = (1, 0), k1 = (0, 2), scale 1/sqrt(2):
    # scores (0, sqrt 2) -> weight of key 1 is 1 / (1 + e^-sqrt2)
    q2 = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    k2 = np.array([[[1.0, 0.0]], [[0.0, 2.0]]])
    v2 = np.array([[[1.0, 2.0]], [[3.0, -1.0]]])
    o = OL.causal_attention(q2, k2, v2, np.array([0, 1]), 1.0 / math.sqrt(2.0))
    w1 = 1.0 / (1.0 + math.exp(-math.sqrt(2.0)))
    exp_row1 = [(1 - w1) * 1.0 + w1 * 3.0, (1 - w1) * 2.0 + w1 * -1.0]
    assert _rel(o[0, 0], [1.0, 2.0]) < TOL
    assert _rel(o[1, 0], exp_row1) < TOL


def check_gqa_group_mapping():
    # query head h must read KV head h // group: give each KV head a constant, distinct V
    hq, hkv, d, L = 8, 2, 4, 3
    k = np.zeros((L, hkv, d))
    v = np.zeros((L, hkv, d))
    v[:, 0, :] = 1.0
    v[:, 1, :] = 2.0
    q = np.random.default_rng(0).standard_normal((1, hq, d))
    o = OL.causal_attention(q, k, v, np.array([2]), 1.0)
    expect = np.array([1.0] * 4 + [2.0] * 4)
    assert np.allclose(o[0, :, 0], expect, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- RoPE

def check_rope_hand_values():
    v = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    got = OL.rope(v, np.array([1]), 10000.0)[0, 0]
    # d = 4: pair (0, 2) turns by 1 rad, pair (1, 3) by 10000^(-1/2) = 0.01 rad
    c1, s1 = math.cos(1.0), math.sin(1.0)
    c2, s2 = math.cos(0.01), math.sin(0.01)
    ref = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    assert _rel(got, ref) < TOL
    # position 0 is the identity
    x = np.random.default_rng(1).standard_normal((2, 3, 8))
    assert _rel(OL.rope(x, np.array([0, 0]), 10000.0), x) < TOL


def check_rope_complex_form_and_invariance():
    rng = np.random.default_rng(5)
    d = 16
    x = rng.standard_normal((4, 2, d))
    pos = np.array([0, 3, 100, 4097])
    got = OL.rope(x, pos, 500000.0)
    # the same rotation written as complex multiplication z * e^(i p w_j), z = x_j + i x_{j+d/2}
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    w = 500000.0 ** (-np.arange(d // 2) * 2.0 / d)
    zr = z * np.exp(1j * pos[:, None, None] * w[None, None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    assert _rel(got, ref) < TOL
    # norms of every pair are kept
    assert _rel(np.abs(got[..., : d // 2] + 1j * got[..., d // 2:]), np.abs(z)) < TOL
    # scores depend only on the position difference
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    base = float(np.sum(OL.rope(q, np.array([17]), 1e4) * OL.rope(k, np.array([5]), 1e4)))
    shifted = float(np.sum(OL.rope(q, np.array([17 + 300]), 1e4) * OL.rope(k, np.array([5 + 300]), 1e4)))
    assert abs(base - shifted) < 1e-10 * max(1.0, abs(base))


# --------------------------------------------------------------------------- norms, MLP

def check_rmsnorm():
    got = OL.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 1.0)
    ref = [3.0 / math.sqrt(12.5 + 1.0), 2.0 * 4.0 / math.sqrt(12.5 + 1.0)]
    assert _rel(got[0], ref) < TOL
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 64))
    g = 1.0 + 0.1 * rng.standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    assert _rel(OL.rmsnorm(x, g, 1e-6), ref) < TOL


def check_silu_swiglu():
    assert OL.silu(np.array([0.0]))[0] == 0.0
    assert abs(OL.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    z = np.linspace(-6, 6, 25)
    assert _rel(OL.silu(z), F.silu(torch.from_numpy(z)).numpy()) < TOL
    # W_gate_up = [gate rows; up rows]: gate reads feature 0, up reads feature 1
    w = np.array([[1.0, 0.0], [0.0, 1.0]])
    h = np.array([[0.5, -3.0]])
    assert abs(OL.swiglu(h, w, 1)[0, 0] - (0.5 / (1 + math.exp(-0.5))) * -3.0) < 1e-15


def check_slot_addresses():
    row = np.array([9, 4, 7, 1])
    pos = np.arange(0, 64)
    blk, slot = OL.kv_slot_addresses(row, pos, 16)
    for p in pos:
        assert blk[p] == row[p // 16] and slot[p] == p % 16
    assert len(set(zip(blk.tolist(), slot.tolist()))) == 64


# --------------------------------------------------------------------------- whole layer

def _torch_layer(shape, x, w, c, cached_k, cached_v):
    """Independent fp64 formulation of one request through the layer, from torch library
    routines (rms_norm, linear, scaled_dot_product_attention with an explicit mask, silu) and
    complex-number RoPE."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    n = x.shape[0]
    hq, hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    X = t(x)
    h1 = F.rms_norm(X, (shape.hidden,), t(w["attn_norm"]), eps=shape.rms_eps)
    qkv = F.linear(h1, t(w["w_qkv"]))
    q = qkv[:, : hq * d].reshape(n, hq, d)
    k = qkv[:, hq * d: (hq + hkv) * d].reshape(n, hkv, d)
    v = qkv[:, (hq + hkv) * d:].reshape(n, hkv, d)
    pos = torch.arange(c, c + n, dtype=torch.float64)
    freq = shape.rope_theta ** (-torch.arange(d // 2, dtype=torch.float64) * 2.0 / d)
    rot = torch.polar(torch.ones(n, d // 2, dtype=torch.float64), pos[:, None] * freq[None, :])

    def rope_c(a):
        z = torch.complex(a[..., : d // 2], a[..., d // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    qr, kr = rope_c(q), rope_c(k)
    K = torch.cat([t(cached_k).reshape(c, hkv, d), kr]).repeat_interleave(hq // hkv, dim=1)
    V = torch.cat([t(cached_v).reshape(c, hkv, d), v]).repeat_interleave(hq // hkv, dim=1)
    mask = torch.arange(c + n)[None, :] <= (c + torch.arange(n))[:, None]
    o = F.scaled_dot_product_attention(qr.permute(1, 0, 2), K.permute(1, 0, 2),
                                       V.permute(1, 0, 2), attn_mask=mask)
    o = o.permute(1, 0, 2).reshape(n, hq * d)
    h2 = X + F.linear(o, t(w["w_o"]))
    h3 = F.rms_norm(h2, (shape.hidden,), t(w["mlp_norm"]), eps=shape.rms_eps)
    gu = F.linear(h3, t(w["w_gate_up"]))
    m = F.silu(gu[:, : shape.d_ff]) * gu[:, shape.d_ff:]
    out = h2 + F.linear(m, t(w["w_down"]))
    return {"out": out.numpy(), "attn_out": o.numpy(), "h2": h2.numpy(), "k_new": kr.numpy(),
            "v_new": v.numpy(), "q_rot": qr.numpy()}


def _tiny_inputs(gain_jitter=0.02):
    from tests._util import oracle_inputs
    spec = workloads.make_spec(1)
    return spec, oracle_inputs(spec, "cpu", gain_jitter=gain_jitter)


def check_layer_vs_torch_library():
    spec, d = _tiny_inputs()
    shape = spec.shape
    cached = [d["cached"][s] for s in range(spec.num_seqs)]
    res = OL.layer_step(shape, d["x"], d["w"], spec.seqs, cached, d["block_table"])
    row = 0
    for s, (c, n) in enumerate(spec.seqs):
        ref = _torch_layer(shape, d["x"][row:row + n], d["w"], c, *cached[s])
        for key in ("out", "attn_out", "h2", "q_rot"):
            assert _rel(res[key][row:row + n], ref[key]) < 1e-11, (s, key)
        row += n
    assert _rel(res["k_new"], np.concatenate([_torch_layer(shape, d["x"][a:a + n], d["w"], c, *cached[s])["k_new"]
                                             for s, (c, n), a in zip(range(spec.num_seqs), spec.seqs, spec.q_start[:-1])])) < 1e-11


def check_batch_equals_alone():
    spec, d = _tiny_inputs()
    shape = spec.shape
    cached = [d["cached"][s] for s in range(spec.num_seqs)]
    full = OL.layer_step(shape, d["x"], d["w"], spec.seqs, cached, d["block_table"])
    row = 0
    for s, (c, n) in enumerate(spec.seqs):
        alone = OL.layer_step(shape, d["x"][row:row + n], d["w"], [(c, n)], [cached[s]],
                              d["block_table"][s:s + 1])
        assert _rel(alone["out"], full["out"][row:row + n]) < TOL
        assert _rel(alone["attn_out"], full["attn_out"][row:row + n]) < TOL
        row += n


def check_chunked_equals_one_shot():
    spec, d = _tiny_inputs()
    shape = spec.shape
    x = d["x"][:64]
    w = d["w"]
    hkv, hd = shape.n_kv_heads, shape.head_dim
    empty = np.zeros((0, hkv, hd))
    one = OL.sequence_step(shape, x, w, 0, empty, empty)
    # three chunks of 24, 1, 39 tokens; each appends to the cache the previous ones built
    k_c, v_c, outs = empty, empty, []
    start = 0
    for n in (24, 1, 39):
        r = OL.sequence_step(shape, x[start:start + n], w, start, k_c, v_c)
        k_c = np.concatenate([k_c, r["k_new"]])
        v_c = np.concatenate([v_c, r["v_new"]])
        outs.append(r["out"])
        start += n
    assert _rel(np.concatenate(outs), one["out"]) < 1e-11
    assert _rel(k_c, one["k_new"]) < 1e-11


def check_decode_equals_last_prefill_row():
    spec, d = _tiny_inputs()
    shape = spec.shape
    x = d["x"][:41]
    w = d["w"]
    hkv, hd = shape.n_kv_heads, shape.head_dim
    empty = np.zeros((0, hkv, hd))
    full = OL.sequence_step(shape, x, w, 0, empty, empty)
    prefix = OL.sequence_step(shape, x[:40], w, 0, empty, empty)
    dec = OL.sequence_step(shape, x[40:41], w, 40, prefix["k_new"], prefix["v_new"])
    assert _rel(dec["out"][0], full["out"][40]) < 1e-11
    assert _rel(dec["q_rot"][0], full["q_rot"][40]) < 1e-11


def check_sampled_rows_match_full():
    spec, d = _tiny_inputs()
    shape = spec.shape
    x = d["x"][:64]
    ck, cv = d["cached"][0]
    full = OL.sequence_step(shape, x, d["w"], 64, ck, cv)
    part = OL.sequence_step(shape, x, d["w"], 64, ck, cv, rows=[5, 0, 33])
    assert list(part["rows"]) == [0, 5, 33]
    assert _rel(part["out"], full["out"][[0, 5, 33]]) < TOL


def check_block_permutation_addresses():
    spec, d = _tiny_inputs()
    shape = spec.shape
    cached = [d["cached"][s] for s in range(spec.num_seqs)]
    t1, _ = workloads.block_table(spec)
    t2, _ = workloads.block_table(spec, permute_seed=99)
    r1 = OL.layer_step(shape, d["x"], d["w"], spec.seqs, cached, t1)
    r2 = OL.layer_step(shape, d["x"], d["w"], spec.seqs, cached, t2)
    assert np.array_equal(r1["out"], r2["out"])
    for r, tab in ((r1, t1), (r2, t2)):
        a = r["kv_addr"]
        # each new token lands in its own sequence's row at block p // 16, slot p % 16
        assert np.array_equal(a[:, 2], tab[a[:, 0], a[:, 1] // 16])
        assert np.array_equal(a[:, 3], a[:, 1] % 16)
        q0 = spec.q_start
        assert np.array_equal(a[:, 1], np.concatenate([c + np.arange(n) for c, n in spec.seqs]))
        assert len(set(map(tuple, a[:, 2:].tolist()))) == a.shape[0]


def check_cfg1_kv_slots_literal():
    """Where the tiny workload's new K/V rows land, worked by hand from the reading that a decode
    "at context c" appends position c and a chunk (c, n) writes positions c .. c+n-1, position p
    going to slot p mod 16 of logical page p // 16 of its own table row ("Chunked prefill ...
    explained", "How it works, step by step"; paged blocks of "7.8 ...", "Attention on Partial KV
    Caches"). The block table is written out by hand with scrambled ids, and the expected
    (sequence, position, block, slot) rows below are literals: decode at 32 -> slot 0 of a fresh
    page 2; 57 -> slot 9 of page 3; 96 -> slot 0 of page 6; 128 -> slot 0 of page 8; the chunk
    (64, 64) fills logical pages 4..7 completely."""
    spec = workloads.make_spec(1)
    assert spec.seqs == [(64, 64), (32, 1), (57, 1), (96, 1), (128, 1)]
    table = np.full((5, 9), -1, dtype=np.int32)
    table[0, :8] = [17, 3, 29, 8, 41, 12, 36, 5]
    table[1, :3] = [22, 40, 9]
    table[2, :4] = [1, 33, 27, 14]
    table[3, :7] = [31, 6, 19, 44, 2, 25, 38]
    table[4, :9] = [10, 34, 7, 21, 45, 0, 28, 16, 30]
    want = [(0, 64 + j, 41, j) for j in range(16)] + [(0, 80 + j, 12, j) for j in range(16)] + \
           [(0, 96 + j, 36, j) for j in range(16)] + [(0, 112 + j, 5, j) for j in range(16)] + \
           [(1, 32, 9, 0), (2, 57, 14, 9), (3, 96, 38, 0), (4, 128, 30, 0)]
    rng = np.random.default_rng(3)
    sh = spec.shape
    w = {"attn_norm": np.ones(sh.hidden), "mlp_norm": np.ones(sh.hidden),
         "w_qkv": 0.02 * rng.standard_normal((sh.qkv_cols, sh.hidden)),
         "w_o": 0.02 * rng.standard_normal((sh.hidden, sh.n_q_heads * sh.head_dim)),
         "w_gate_up": 0.02 * rng.standard_normal((2 * sh.d_ff, sh.hidden)),
         "w_down": 0.02 * rng.standard_normal((sh.hidden, sh.d_ff))}
    x = rng.standard_normal((spec.num_tokens, sh.hidden))
    cached = [(rng.standard_normal((c, sh.n_kv_heads, sh.head_dim)),
               rng.standard_normal((c, sh.n_kv_heads, sh.head_dim))) for c, _ in spec.seqs]
    r = OL.layer_step(sh, x, w, spec.seqs, cached, table)
    got = [tuple(int(v) for v in row) for row in r["kv_addr"]]
    assert got == want, got
    # the addressed rows are the new tokens' K/V in batch row order: the decode at context 57
    # (batch row 65) carries the rotated K of that token alone
    alone = OL.sequence_step(sh, x[65:66], w, 57, *cached[2])
    assert _rel(r["k_new"][65], alone["k_new"][0]) < TOL


# --------------------------------------------------------------------------- KV transfer

def _code(b, h, s, d):
    """An exact fp64 label of pool element (block, head, slot, dim)."""
    return ((np.asarray(b) * 64.0 + h) * 16.0 + s) * 256.0 + d


def _coded_pools(nblk, hkv, dim):
    b, h, s, d = np.meshgrid(np.arange(nblk), np.arange(hkv), np.arange(16), np.arange(dim),
                             indexing="ij")
    k = _code(b, h, s, d)                       # K[b][h][s][d]
    v = np.transpose(_code(b, h, s, d), (0, 1, 3, 2)).copy()  # V[b][h][d][s] holds code(b,h,s,d)
    return k, v


def check_kv_export_closed_form():
    """Every exported element is the label of the slot the table names for its position."""
    rng = np.random.default_rng(3)
    nblk, hkv, dim, L = 23, 3, 8, 4
    k, v = _coded_pools(nblk, hkv, dim)
    table = rng.permutation(nblk)[:9]
    for start, count, layer in [(0, 16, 0), (5, 100, 2), (37, 1, 3), (31, 2, 1), (0, 0, 0)]:
        out = np.full((L, 2, count, hkv, dim), np.nan)
        OKV.export_layer(k, v, table, start, count, layer, out)
        p = start + np.arange(count)
        want = _code(table[p // 16][:, None, None], np.arange(hkv)[None, :, None],
                     (p % 16)[:, None, None], np.arange(dim)[None, None, :])
        assert np.array_equal(out[layer, 0], want) and np.array_equal(out[layer, 1], want)
        others = [l for l in range(L) if l != layer]
        assert np.isnan(out[others]).all(), "export wrote outside its layer"


def check_kv_import_closed_form():
    """Import writes exactly the slots of the span, each from the element of its position, and
    leaves every other slot alone."""
    rng = np.random.default_rng(4)
    nblk, hkv, dim, L = 17, 2, 8, 3
    table = rng.permutation(nblk)[:7]
    start, count, layer = 9, 90, 1
    p = start + np.arange(count)
    src = np.full((L, 2, count, hkv, dim), np.nan)
    src[layer, 0] = (p[:, None, None] * 10.0 + np.arange(hkv)[None, :, None]) * 100.0 + np.arange(dim)
    src[layer, 1] = -src[layer, 0]
    k = np.full((nblk, hkv, 16, dim), 7.5)
    v = np.full((nblk, hkv, dim, 16), 7.5)
    OKV.import_layer(src, table, start, count, layer, k, v)
    inv = {int(b): j for j, b in enumerate(table)}
    for b in range(nblk):
        for s in range(16):
            pos = inv[b] * 16 + s if b in inv else -1
            kk, vv = k[b, :, s, :], v[b, :, :, s]
            if start <= pos < start + count:
                want = (pos * 10.0 + np.arange(hkv)[:, None]) * 100.0 + np.arange(dim)[None, :]
                assert np.array_equal(kk, want) and np.array_equal(vv, -want), (b, s)
            else:
                assert (kk == 7.5).all() and (vv == 7.5).all(), (b, s)


def check_kv_round_trip_across_tables():
    """Exporting, importing into another pool under another table and exporting again gives the
    same transfer tensor (what a decode instance receives is what the prefill instance held)."""
    rng = np.random.default_rng(5)
    hkv, dim, L = 2, 16, 2
    k1, v1 = rng.standard_normal((12, hkv, 16, dim)), rng.standard_normal((12, hkv, dim, 16))
    t1, t2 = rng.permutation(12)[:8], rng.permutation(30)[:8]
    start, count = 3, 120
    a = np.zeros((L, 2, count, hkv, dim))
    OKV.export_layer(k1, v1, t1, start, count, 1, a)
    k2, v2 = np.zeros((30, hkv, 16, dim)), np.zeros((30, hkv, dim, 16))
    OKV.import_layer(a, t2, start, count, 1, k2, v2)
    b = np.zeros_like(a)
    OKV.export_layer(k2, v2, t2, start, count, 1, b)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------- model step

def _tiny_model(layers, zero_residual_branches):
    shape = workloads.SHAPES["tiny"]
    spec = workloads.custom_spec(shape, [(5, 9), (0, 1), (17, 1), (0, 4)], 11)
    table, _ = workloads.block_table(spec)
    t = workloads.model_tensors(spec, 64)
    Ws, caches = [], []
    for l in range(layers):
        ls = workloads.layer_spec(spec, l)
        w = {k: v.double().numpy() for k, v in workloads.weights(ls).items()}
        if zero_residual_branches:
            w["w_o"][:] = 0.0
            w["w_down"][:] = 0.0
        Ws.append(w)
        caches.append([tuple(a.double().numpy() for a in workloads.cached_kv(ls, si))
                       for si in range(spec.num_seqs)])
    return shape, spec, table, t, Ws, caches


def check_model_head_library_and_identity_stack():
    """With the attention and MLP outputs projected to zero, every layer is the identity on the
    residual stream, so a stack of any depth gives the logits of the embedded tokens themselves;
    those are checked against torch's rms_norm and linear on the last row of each sequence."""
    for layers in (0, 2):
        shape, spec, table, t, Ws, caches = _tiny_model(layers, True)
        emb, head = t["embed"].double().numpy(), t["lm_head"].double().numpy()
        gain = t["final_norm"].double().numpy()
        r = OM.model_step(shape, t["tokens"], emb, Ws, gain, head, spec.seqs, caches, table)
        last = np.cumsum([n for _, n in spec.seqs]) - 1
        xt = torch.from_numpy(emb[t["tokens"][last]])
        want = F.linear(F.rms_norm(xt, (shape.hidden,), torch.from_numpy(gain), shape.rms_eps),
                        torch.from_numpy(head)).numpy()
        assert _rel(r["logits"], want) < TOL
        assert np.array_equal(r["hidden"], emb[t["tokens"]])


def check_model_stack_is_layer_by_layer():
    """A two-layer stack equals the first layer's output fed to the second (rows of each request
    see only that request), and its logits rows follow the sequences' last rows."""
    shape, spec, table, t, Ws, caches = _tiny_model(2, False)
    emb, head = t["embed"].double().numpy(), t["lm_head"].double().numpy()
    gain = t["final_norm"].double().numpy()
    r = OM.model_step(shape, t["tokens"], emb, Ws, gain, head, spec.seqs, caches, table)
    x = emb[t["tokens"]]
    row = 0
    for s, (c, n) in enumerate(spec.seqs):
        h = x[row:row + n]
        for l in range(2):
            h = OL.sequence_step(shape, h, Ws[l], c, *caches[l][s])["out"]
        assert _rel(r["hidden"][row:row + n], h) < TOL
        want = F.linear(F.rms_norm(torch.from_numpy(h[-1:]), (shape.hidden,),
                                   torch.from_numpy(gain), shape.rms_eps), torch.from_numpy(head))
        assert _rel(r["logits"][s:s + 1], want.numpy()) < TOL
        row += n


def check_greedy_hand_values():
    assert list(OM.greedy(np.array([[1.0, 3.0, 3.0, 2.0], [-5.0, -7.0, -5.0, -6.0]]))) == [1, 0]
    assert list(OM.last_rows([(0, 3), (9, 1), (2, 5)])) == [2, 3, 8]


# --------------------------------------------------------------------------- scheduler

def _golden_lines(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    return [l.split(":", 1)[1].strip() for l in open(path) if l[0].isdigit()]


def _run_trace(sched, reqs, names, iters):
    for rid, p, o in reqs:
        sched.submit(rid, p, o)
    got = []
    for it in range(iters):
        b = sched.next()
        got.append(" ".join(f"{names[e['rid']]}:{e['num_cached']}+{e['q_len']}"
                            f"{'*' if e['emits'] else ''}" for e in b))
        sched.complete([100 + it] * len(b))
    return got


def check_scheduler_hand_trace():
    """The hand-worked trace in tests/golden/scheduler_trace.txt (budget 8, 2 slots)."""
    want = _golden_lines("scheduler_trace.txt")
    s = OS.Scheduler(budget=8, max_seqs=2, num_blocks=40)
    got = _run_trace(s, [(0, 10, 3), (1, 5, 1), (2, 3, 2)], {0: "A", 1: "B", 2: "C"}, len(want))
    assert got == want, got
    assert len(s.free) == 40


def check_scheduler_adaptive_two_prompt_trace():
    """The hand-worked trace in tests/golden/scheduler_adaptive_trace.txt: the adaptive prompt
    share at decode loads 0, 1 and 2, and an iteration in which one prompt finishes and the next
    starts inside the same share."""
    want = _golden_lines("scheduler_adaptive_trace.txt")
    s = OS.Scheduler(adaptive=True, max_seqs=4, num_blocks=40, min_chunk=4, base_chunk=8,
                     max_chunk=12, pressure_threshold=4)
    got = _run_trace(s, [(0, 3, 4), (1, 20, 2), (2, 20, 2)], {0: "C", 1: "A", 2: "B"}, len(want))
    assert got == want, got
    assert len(s.free) == 40


def check_scheduler_blocks_and_adaptive_budget():
    """Blocks for the whole lifetime are taken at admission (lowest ids first) and come back at
    the end; the adaptive prompt share is max_chunk with no decodes, min_chunk at the threshold,
    and the linear rule rounded down in between (chapter 7.8's dynamic chunk sizing), with the
    decode tokens on top."""
    s = OS.Scheduler(budget=4, max_seqs=4, num_blocks=10)
    s.submit(7, 20, 13)            # 32 tokens over its lifetime: 2 blocks
    s.submit(8, 3, 1)              # 3 tokens: 1 block
    b = s.next()
    assert [e["blocks"] for e in b] == [[0, 1]] and len(s.free) == 8
    # a request that could never fit the pool is refused at submission
    try:
        s.submit(9, 170, 2)        # 171 tokens: 11 blocks > 10
        raise AssertionError("oversized request accepted")
    except ValueError:
        pass
    # a decoding sequence holds its slot: with one slot, B waits until A has finished
    one = OS.Scheduler(budget=8, max_seqs=1, num_blocks=10)
    one.submit(0, 2, 3)
    one.submit(1, 2, 1)
    seen = []
    for it in range(5):
        b = one.next()
        seen.append([e["rid"] for e in b])
        one.complete([5] * len(b))
    assert seen == [[0], [0], [0], [1], []], seen
    # decode tokens count against the budget: the prompt in progress gets what they leave
    tb = OS.Scheduler(budget=4, max_seqs=4, num_blocks=10)
    tb.submit(0, 2, 3)
    tb.submit(1, 10, 1)
    b0 = tb.next()
    assert [(e["rid"], e["q_len"]) for e in b0] == [(0, 2), (1, 2)]
    tb.complete([9, 9])
    b1 = tb.next()
    assert [(e["rid"], e["num_cached"], e["q_len"]) for e in b1] == [(0, 2, 1), (1, 2, 3)]
    a = OS.Scheduler(adaptive=True, max_seqs=64, num_blocks=10, min_chunk=128, base_chunk=512,
                     max_chunk=4096, pressure_threshold=16)
    assert a.prompt_share() == 4096
    a.running = [OS.Request(i, 1, 2) for i in range(16)]
    assert a.prompt_share() == 128
    a.running = a.running[:4]
    assert a.prompt_share() == 416                 # 512 - 4/16 * (512 - 128)
    a.running = a.running[:3]
    assert a.prompt_share() == 440                 # 512 - 72
    a.min_chunk, a.threshold = 100, 7
    assert a.prompt_share() == 335                 # 512 - 3/7 * 412 = 335.43, rounded down
    a.running = a.running[:1]
    assert a.prompt_share() == 453                 # 512 - 412/7 = 453.14, rounded down


ALL_CHECKS = [
    check_attention_bruteforce, check_attention_sdpa_library, check_attention_closed_forms,
    check_gqa_group_mapping, check_rope_hand_values, check_rope_complex_form_and_invariance,
    check_rmsnorm, check_silu_swiglu, check_slot_addresses, check_layer_vs_torch_library,
    check_batch_equals_alone, check_chunked_equals_one_shot,
    check_decode_equals_last_prefill_row, check_sampled_rows_match_full,
    check_block_permutation_addresses, check_kv_export_closed_form, check_kv_import_closed_form,
    check_kv_round_trip_across_tables, check_model_head_library_and_identity_stack,
    check_model_stack_is_layer_by_layer, check_greedy_hand_values, check_scheduler_hand_trace,
    check_scheduler_adaptive_two_prompt_trace, check_scheduler_blocks_and_adaptive_budget,
    check_cfg1_kv_slots_literal,
]
