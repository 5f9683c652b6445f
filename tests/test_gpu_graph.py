"""The layer step captured in a HIP graph and replayed, on a batch that takes the schedules a
small hybrid batch gets: split-K for the QKV projection (the fix-up applies RoPE and the KV
append), a prompt chunk after a long prefix whose key range is split into merged parts, and split
decode attention with its merge; once with two attention launches and once fused. Every replay,
with eager work and synchronisations between replays, must give the eager step's output bit for
bit (the K/V appends are idempotent, so a replay repeats the same batch). The launches record no
memset and no host-side state, so capture is valid for any batch."""
import pytest
import torch

import workloads
from hybrid_prefill_decode_amd import binding as B
from tests._gpu import make_pools, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("attention", [B.HL_ATTN_SEPARATE, B.HL_ATTN_FUSED],
                         ids=["separate", "fused"])
def test_layer_step_graph_replays(attention):
    shape = workloads.LayerShape(4096, 8, 2, 128, 512)
    spec = workloads.custom_spec(shape, [(3000, 100)] + [(700 + 97 * i, 1) for i in range(20)], 41)
    table, pool = workloads.block_table(spec)
    cfg = B.layer_cfg(shape)
    batch = B.Batch(spec.q_start, spec.num_cached, table, DEV, attention=attention)
    plan = B.attention_plan(cfg, batch)
    choice = B.gemm_tile_choice(spec.num_tokens, shape.qkv_cols, shape.hidden, B.HL_EPI_NONE,
                                True, shape.head_dim)
    say(f"graph replay ({attention}): T={spec.num_tokens}, plan {plan}, QKV choice {choice}")
    assert choice[2] == 3 and plan["prefill_merges"] > 0 and plan["decode_units"] > 0
    assert (plan["fused"] >= 1) == (attention == B.HL_ATTN_FUSED)
    x = workloads.hidden_states(spec, DEV)
    w = workloads.weights(spec, DEV)
    kp, vp = make_pools(spec, table, pool, DEV)
    out = torch.empty(spec.num_tokens, shape.hidden, dtype=torch.bfloat16, device=DEV)
    ws = B.alloc_workspace(cfg, batch, DEV)
    B.hybrid_layer_step(cfg, batch, x, w, kp, vp, out, ws)  # eager first: one-time set-up
    torch.cuda.synchronize()
    want = out.clone()
    want_k, want_v = kp.clone(), vp.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.hybrid_layer_step(cfg, batch, x, w, kp, vp, out, ws, stream=s)
    junk = torch.zeros(1 << 20, device=DEV)
    for rep in range(4):
        out.fill_(0)
        ws.fill_(0)  # nothing may rely on workspace contents left by an earlier call
        junk.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
        assert torch.equal(kp.view(torch.int16), want_k.view(torch.int16)), rep
        assert torch.equal(vp.view(torch.int16), want_v.view(torch.int16)), rep
    say("graph replays bit-identical to the eager step")
