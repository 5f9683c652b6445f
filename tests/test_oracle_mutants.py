"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

Every mutant is a textual edit of one oracle function, re-executed in the oracle module's
namespace and patched in for the duration of the check run. A mutant that no pin notices would
mean that part of the oracle is unpinned.
"""
import inspect
import textwrap

import pytest

import oracle.kv_transfer as OKV
import oracle.model as OM
import oracle.scheduler as OS
import oracle.layer as OL
from tests import oracle_pins

MUTANTS = [
    ("rmsnorm", "np.sqrt(ms + eps)", "np.sqrt(ms)"),
    ("rmsnorm", "np.mean(x * x", "np.sum(x * x"),
    ("rmsnorm", "np.sqrt(ms + eps) * gain", "np.sqrt(ms + eps)"),
    ("rope", "a * cos - b * sin", "a * cos + b * sin"),
    ("rope", "-2.0 * j / d", "-1.0 * j / d"),
    ("rope", "a = v[..., :half]", "a = v[..., 0::2]"),
    ("causal_attention", "np.arange(L)[None, :] <= q_pos[:, None]",
     "np.arange(L)[None, :] <= q_pos[:, None] + 1"),
    ("causal_attention", "h // group", "h % hkv"),
    ("causal_attention", ") * scale", ")"),
    ("silu", "np.exp(-z)", "np.exp(z)"),
    ("swiglu", "w_gate_up[:d_ff])", "w_gate_up[d_ff:])"),
    ("sequence_step", "pos_all = num_cached + np.arange(last)", "pos_all = np.arange(last)"),
    ("sequence_step", "h2 = x_seq[sel] + linear(attn", "h2 = linear(attn"),
    ("sequence_step", "v_new = linear(h1, v_w).reshape(last, hkv, d)",
     "v_new = rope(linear(h1, v_w).reshape(last, hkv, d), pos_all, shape.rope_theta)"),
    ("sequence_step", "h3 = rmsnorm(h2, w[\"mlp_norm\"], shape.rms_eps)", "h3 = h2"),
    ("sequence_step", "out = h2 + linear(", "out = linear("),
    ("sequence_step", "q_rot = rope(q, pos, shape.rope_theta)", "q_rot = q"),
    ("kv_slot_addresses", "positions % block_size", "positions % (block_size + 1)"),
    ("kv_slot_addresses", "positions % block_size", "(positions + 1) % block_size"),
    ("kv_slot_addresses", "block_table_row[positions // block_size]",
     "block_table_row[(positions + 1) // block_size]"),
    ("layer_step", "pos = c + np.arange(n)", "pos = np.arange(n)"),
]
# planted mistakes in the KV-transfer reference
KV_MUTANTS = [
    ("export_layer", "out[layer, 1, i] = vpool[b, :, :, s]", "out[layer, 1, i] = vpool[b, :, s, :]"),
    ("export_layer", "p = start + i", "p = i"),
    ("export_layer", "out[layer, 0, i] = kpool[b, :, s, :]", "out[0, 0, i] = kpool[b, :, s, :]"),
    ("export_layer", "b, s = int(table_row[p // BLOCK]), p % BLOCK", "b, s = p // BLOCK, p % BLOCK"),
    ("import_layer", "vpool[b, :, :, s] = src[layer, 1, i]", "vpool[b, :, :, s] = src[layer, 0, i]"),
    ("import_layer", "p = start + i", "p = start + i + 1"),
    ("import_layer", "b, s = int(table_row[p // BLOCK]), p % BLOCK", "b, s = int(table_row[p // BLOCK]), (p + 1) % BLOCK"),
]
# planted mistakes in the model-step reference
MODEL_MUTANTS = [
    ("last_rows", "np.cumsum([n for _, n in seqs]) - 1", "np.cumsum([n for _, n in seqs]) - 2"),
    ("lm_logits", "OL.linear(OL.rmsnorm(h, final_norm, eps), lm_head)", "OL.linear(h, lm_head)"),
    ("greedy", "np.argmax(logits, axis=-1)", "np.argmax(logits[:, ::-1], axis=-1)"),
    ("model_step", "x = OL.layer_step(shape, x, w, seqs, caches[l], block_table)[\"out\"]",
     "x = OL.layer_step(shape, x, w, seqs, caches[0], block_table)[\"out\"]"),
    ("model_step", "for l, w in enumerate(layers):", "for l, w in enumerate(layers[:1]):"),
]


def _mutant(fn_name, old, new, mod=OL):
    src = textwrap.dedent(inspect.getsource(getattr(mod, fn_name)))
    fn = getattr(mod, fn_name)
    if fn.__doc__:  # edit code, never the docstring
        src = src.replace(fn.__doc__, "", 1)
    assert old in src, f"mutation site not found in {fn_name}: {old!r}"
    ns = dict(vars(mod))
    exec(compile(src.replace(old, new, 1), f"<mutant {fn_name}>", "exec"), ns)
    return ns[fn_name]


@pytest.mark.parametrize("fn_name,old,new", MUTANTS, ids=[f"{m[0]}:{m[1][:24]}" for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, fn_name, old, new):
    monkeypatch.setattr(OL, fn_name, _mutant(fn_name, old, new))
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception:  # an assertion, or NaN/shape fallout of the mistake
            caught.append(check.__name__)
    assert caught, f"no pin caught the mutant {fn_name}: {old!r} -> {new!r}"


@pytest.mark.parametrize("fn_name,old,new", KV_MUTANTS,
                         ids=[f"{m[0]}:{m[1][:24]}" for m in KV_MUTANTS])
def test_pins_catch_planted_kv_transfer_mistake(monkeypatch, fn_name, old, new):
    monkeypatch.setattr(OKV, fn_name, _mutant(fn_name, old, new, OKV))
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception:
            caught.append(check.__name__)
    assert caught, f"no pin caught the mutant {fn_name}: {old!r} -> {new!r}"


@pytest.mark.parametrize("fn_name,old,new", MODEL_MUTANTS,
                         ids=[f"{m[0]}:{m[1][:24]}" for m in MODEL_MUTANTS])
def test_pins_catch_planted_model_mistake(monkeypatch, fn_name, old, new):
    monkeypatch.setattr(OM, fn_name, _mutant(fn_name, old, new, OM))
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception:
            caught.append(check.__name__)
    assert caught, f"no pin caught the mutant {fn_name}: {old!r} -> {new!r}"


# planted mistakes in the scheduler reference (methods of OS.Scheduler)
SCHED_MUTANTS = [
    ("next", "take = min(share, r.prompt_len - r.prefilled)", "take = min(share, r.prompt_len)"),
    ("_admit", "if busy >= self.max_seqs or need > len(self.free):",
     "if len(self.prefilling) >= self.max_seqs or need > len(self.free):"),
    ("_admit", "r.blocks, self.free = self.free[:need], self.free[need:]",
     "r.blocks, self.free = self.free[-need:], self.free[:-need]"),
    ("next", '"emits": 1 if dec or r.prefilled + n == r.prompt_len else 0',
     '"emits": 1 if dec else 0'),
    ("next", "share -= take", "share -= take - 1"),
    ("complete", "r.generated, r.last_token = 1, tok", "r.generated, r.last_token = 0, tok"),
    ("prompt_share", "return self.budget - d", "return self.budget"),
    ("submit", "if lifetime_blocks(r) > self.num_blocks:", "if False:"),
]
# planted mistakes in the adaptive prompt-share rule (a module function of the scheduler oracle)
SHARE_MUTANTS = [
    ("adaptive_chunk", "drop = -(-d * (base - lo) // threshold)", "drop = d * (base - lo) // threshold"),
    ("adaptive_chunk", "return hi", "return base"),
    ("adaptive_chunk", "return base - drop", "return lo + drop"),
]


def _method_mutant(name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(OS.Scheduler, name)))
    assert old in src, f"mutation site not found in Scheduler.{name}: {old!r}"
    ns = dict(vars(OS))
    exec(compile(src.replace(old, new, 1), f"<mutant Scheduler.{name}>", "exec"), ns)
    return ns[name]


@pytest.mark.parametrize("name,old,new", SCHED_MUTANTS, ids=[f"{m[0]}:{m[1][:24]}" for m in SCHED_MUTANTS])
def test_pins_catch_planted_scheduler_mistake(monkeypatch, name, old, new):
    monkeypatch.setattr(OS.Scheduler, name, _method_mutant(name, old, new))
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception:
            caught.append(check.__name__)
    assert caught, f"no pin caught the mutant Scheduler.{name}: {old!r} -> {new!r}"


@pytest.mark.parametrize("fn_name,old,new", SHARE_MUTANTS,
                         ids=[f"{m[0]}:{m[1][:24]}" for m in SHARE_MUTANTS])
def test_pins_catch_planted_share_mistake(monkeypatch, fn_name, old, new):
    monkeypatch.setattr(OS, fn_name, _mutant(fn_name, old, new, OS))
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception:
            caught.append(check.__name__)
    assert caught, f"no pin caught the mutant {fn_name}: {old!r} -> {new!r}"


@pytest.mark.parametrize("fn_name,old,new", [m for m in MUTANTS if m[0] == "kv_slot_addresses"],
                         ids=lambda v: str(v)[:24])
def test_literal_slot_pin_catches_shifted_mapping(monkeypatch, fn_name, old, new):
    """A shifted slot mapping fails the hand-worked literal slots, a pin whose expected values
    do not come from the oracle's own slot function."""
    monkeypatch.setattr(OL, fn_name, _mutant(fn_name, old, new))
    with pytest.raises(Exception):
        oracle_pins.check_cfg1_kv_slots_literal()
