"""ctypes binding of libhybrid_layer.so: the C ABI of include/hybrid_layer.h with the same names.

Argument marshalling only. Torch tensors supply device memory and the stream; every step of the
layer runs in the library's HIP kernels. There is no fallback: if the shared library is missing
or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhybrid_layer.so")

HL_OK = 0
HL_ERR_NULL, HL_ERR_SHAPE, HL_ERR_DESC, HL_ERR_BLOCK = -1, -2, -3, -4
HL_ERR_ALIGN, HL_ERR_WORKSPACE, HL_ERR_HIP, HL_ERR_ARG = -5, -6, -7, -8
HL_EPI_NONE, HL_EPI_RESIDUAL, HL_EPI_SWIGLU = 0, 1, 2
HL_ATTN_AUTO, HL_ATTN_FUSED, HL_ATTN_SEPARATE = 0, 1, 2
BLOCK_SIZE = 16

_c_i32p = ctypes.POINTER(ctypes.c_int32)


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("softmax_scale", ctypes.c_float)]


class BatchDesc(ctypes.Structure):
    _fields_ = [("cfg", ctypes.POINTER(LayerCfg)), ("num_seqs", ctypes.c_int32),
                ("num_tokens", ctypes.c_int32), ("q_start", ctypes.c_void_p),
                ("num_cached", ctypes.c_void_p), ("h_q_start", _c_i32p),
                ("h_num_cached", _c_i32p), ("x", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stream", ctypes.c_void_p), ("tap_q_rot", ctypes.c_void_p),
                ("tap_attn_out", ctypes.c_void_p), ("tap_h2", ctypes.c_void_p),
                ("attention", ctypes.c_int32), ("events", ctypes.c_void_p)]


HL_STEP_EVENTS = 7  # phase marks of hybrid_layer_step (hl_batch_desc::events)
HL_VERSION = 2      # the hl_batch_desc layout above (with `events`)


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")]


class KvPages(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("num_blocks", ctypes.c_int64)]


class BlockTable(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("h_table", _c_i32p),
                ("max_blocks_per_seq", ctypes.c_int32)]


class KvSpan(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_layers", ctypes.c_int32), ("layer", ctypes.c_int32),
                ("start", ctypes.c_int32), ("count", ctypes.c_int32),
                ("table", ctypes.c_void_p), ("h_table", _c_i32p), ("table_len", ctypes.c_int32),
                ("stream", ctypes.c_void_p)]


class Model(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("embed", ctypes.c_void_p), ("layers", ctypes.c_void_p), ("kv", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p)]


class SchedParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("budget", "max_seqs", "num_blocks",
                                             "max_blocks_per_seq", "adaptive", "min_chunk",
                                             "base_chunk", "max_chunk", "pressure_threshold")]


class SchedBatch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("q_start", _c_i32p), ("num_cached", _c_i32p), ("request_ids", _c_i32p),
                ("table", _c_i32p), ("decode_tokens", _c_i32p), ("emits", _c_i32p),
                ("max_blocks_per_seq", ctypes.c_int32)]


class HLError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


_lib = None

# every function the header declares, with its ctypes signature
_SIGS = {
    "hl_version": ([], ctypes.c_int),
    "hl_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "hl_workspace_bytes": ([ctypes.POINTER(BatchDesc), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "hl_attention_plan": ([ctypes.POINTER(BatchDesc)] + [_c_i32p] * 6, ctypes.c_int),
    "hybrid_layer_step": ([ctypes.POINTER(BatchDesc), ctypes.POINTER(Weights),
                           ctypes.POINTER(KvPages), ctypes.POINTER(BlockTable), ctypes.c_void_p],
                          ctypes.c_int),
    "hl_rmsnorm": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                    ctypes.c_int32, ctypes.c_float, ctypes.c_void_p], ctypes.c_int),
    "hl_gemm_bf16_nt": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p],
                        ctypes.c_int),
    "hl_gemm_bf16_nt_tiled": ([ctypes.c_void_p] * 5 + [ctypes.c_int32] * 7 +
                              [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "hl_rms_scale": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p], ctypes.c_int),
    "hl_qkv_rope_append": ([ctypes.POINTER(BatchDesc), ctypes.POINTER(Weights), ctypes.c_void_p,
                            ctypes.POINTER(KvPages), ctypes.POINTER(BlockTable)], ctypes.c_int),
    "hl_gemm_workspace_bytes": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "hl_model_workspace_bytes": ([ctypes.POINTER(Model), ctypes.POINTER(BatchDesc),
                                  ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "hl_model_step": ([ctypes.POINTER(Model), ctypes.POINTER(BatchDesc), ctypes.c_void_p, _c_i32p,
                       ctypes.POINTER(BlockTable), ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p], ctypes.c_int),
    "hl_sched_create": ([ctypes.POINTER(SchedParams)], ctypes.c_void_p),
    "hl_sched_destroy": ([ctypes.c_void_p], None),
    "hl_sched_submit": ([ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                         _c_i32p], ctypes.c_int),
    "hl_sched_next": ([ctypes.c_void_p, ctypes.POINTER(SchedBatch)], ctypes.c_int),
    "hl_sched_complete": ([ctypes.c_void_p, _c_i32p, _c_i32p, _c_i32p], ctypes.c_int),
    "hl_sched_counts": ([ctypes.c_void_p, _c_i32p, _c_i32p, _c_i32p, _c_i32p], ctypes.c_int),
    "hl_kv_export": ([ctypes.POINTER(KvSpan), ctypes.POINTER(KvPages), ctypes.c_void_p],
                     ctypes.c_int),
    "hl_kv_import": ([ctypes.POINTER(KvSpan), ctypes.c_void_p, ctypes.POINTER(KvPages)],
                     ctypes.c_int),
    "hl_gemm_tile_choice": ([ctypes.c_int32] * 6 + [ctypes.POINTER(ctypes.c_int32)] * 4,
                            ctypes.c_int),
    "hl_rope_kv_append": ([ctypes.POINTER(BatchDesc), ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.POINTER(KvPages), ctypes.POINTER(BlockTable)], ctypes.c_int),
    "hl_attention": ([ctypes.POINTER(BatchDesc), ctypes.c_void_p, ctypes.POINTER(KvPages),
                      ctypes.POINTER(BlockTable), ctypes.c_void_p], ctypes.c_int),
    "hl_prefill_attention": ([ctypes.POINTER(BatchDesc), ctypes.c_void_p, ctypes.POINTER(KvPages),
                              ctypes.POINTER(BlockTable), ctypes.c_void_p], ctypes.c_int),
    "hl_decode_attention": ([ctypes.POINTER(BatchDesc), ctypes.c_void_p, ctypes.POINTER(KvPages),
                             ctypes.POINTER(BlockTable), ctypes.c_void_p], ctypes.c_int),
    "hybrid_layer_step_noalloc": ([ctypes.POINTER(BatchDesc), ctypes.POINTER(Weights),
                                   ctypes.POINTER(KvPages), ctypes.POINTER(BlockTable),
                                   ctypes.c_void_p], ctypes.c_int),
    "hl_attention_build_lists": ([ctypes.POINTER(BatchDesc), ctypes.POINTER(KvPages),
                                  ctypes.POINTER(BlockTable)], ctypes.c_int),
    "hl_attention_run": ([ctypes.POINTER(BatchDesc), ctypes.c_void_p, ctypes.c_void_p,
                          ctypes.POINTER(KvPages), ctypes.POINTER(BlockTable), ctypes.c_void_p,
                          ctypes.c_int32], ctypes.c_int),
    "hl_attention_run_traced": ([ctypes.POINTER(BatchDesc), ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.POINTER(KvPages), ctypes.POINTER(BlockTable),
                                 ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_size_t], ctypes.c_int),
    "hl_trace_clock_khz": ([_c_i32p], ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               f"`python -m hybrid_prefill_decode_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(handle, name)
            f.argtypes = args
            f.restype = res
        # the descriptor structs above must match the library's layout
        if handle.hl_version() != HL_VERSION:
            raise RuntimeError(f"{LIB_PATH} is version {handle.hl_version()}, the binding expects "
                               f"{HL_VERSION}: rebuild it")
        _lib = handle
    return _lib


def strerror(code: int) -> str:
    return lib().hl_strerror(code).decode()


def _check(rc: int, where: str) -> None:
    if rc != HL_OK:
        raise HLError(rc, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def layer_cfg(shape, softmax_scale: float = 0.0) -> LayerCfg:
    """LayerCfg from any object with hidden / n_q_heads / n_kv_heads / head_dim / d_ff
    (and optionally rms_eps / rope_theta)."""
    return LayerCfg(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff,
                    getattr(shape, "block_size", BLOCK_SIZE), getattr(shape, "rms_eps", 1e-6),
                    getattr(shape, "rope_theta", 10000.0), softmax_scale)


class Batch:
    """Batch descriptor arrays: host mirrors (numpy int32) plus device copies (torch)."""

    def __init__(self, q_start, num_cached, table, device="cuda", attention: int = 0):
        """attention: HL_ATTN_AUTO (0), HL_ATTN_FUSED (1) or HL_ATTN_SEPARATE (2)."""
        import torch
        self.attention = attention
        self.h_q_start = np.ascontiguousarray(q_start, dtype=np.int32)
        self.h_num_cached = np.ascontiguousarray(num_cached, dtype=np.int32)
        self.h_table = np.ascontiguousarray(table, dtype=np.int32)
        self.num_seqs = int(self.h_num_cached.shape[0])
        self.num_tokens = int(self.h_q_start[-1]) if self.num_seqs else 0
        self.max_blocks = int(self.h_table.shape[1]) if self.h_table.ndim == 2 else 1
        self.q_start = torch.from_numpy(self.h_q_start).to(device)
        self.num_cached = torch.from_numpy(self.h_num_cached).to(device)
        self.table = torch.from_numpy(self.h_table).to(device)


def _event_array(events):
    """HL_STEP_EVENTS raw hipEvent_t handles from torch.cuda.Event objects (None entries stay
    NULL). torch creates an event's handle at its first record, so each must have been recorded
    once."""
    if len(events) != HL_STEP_EVENTS:
        raise ValueError(f"events: {HL_STEP_EVENTS} entries expected, got {len(events)}")
    arr = (ctypes.c_void_p * HL_STEP_EVENTS)()
    for i, ev in enumerate(events):
        if ev is None:
            continue
        if not ev.cuda_event:
            raise ValueError("events: record each event once before passing it (torch creates "
                             "the underlying hipEvent_t lazily)")
        arr[i] = ev.cuda_event
    return arr


def _desc(cfg: LayerCfg, b: Batch, x=None, workspace=None, stream=None, taps=None,
          with_stream: bool = True, events=None):
    taps = taps or {}
    d = BatchDesc()
    d.cfg = ctypes.pointer(cfg)
    d.num_seqs = b.num_seqs
    d.num_tokens = b.num_tokens
    d.q_start = _ptr(b.q_start)
    d.num_cached = _ptr(b.num_cached)
    d.h_q_start = b.h_q_start.ctypes.data_as(_c_i32p)
    d.h_num_cached = b.h_num_cached.ctypes.data_as(_c_i32p)
    d.x = _ptr(x)
    d.workspace = _ptr(workspace)
    d.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d.stream = _stream_ptr(stream) if with_stream else None
    d.tap_q_rot = _ptr(taps.get("q_rot"))
    d.tap_attn_out = _ptr(taps.get("attn_out"))
    d.tap_h2 = _ptr(taps.get("h2"))
    d.attention = getattr(b, "attention", 0)
    if events is not None:
        d._event_array = _event_array(events)  # kept alive with the descriptor
        d.events = ctypes.cast(d._event_array, ctypes.c_void_p)
    return d


def _pages(k_pool, v_pool) -> KvPages:
    return KvPages(_ptr(k_pool), _ptr(v_pool), int(k_pool.shape[0]))


def _span(table_row, h_table_row, n_kv_heads: int, head_dim: int, num_layers: int, layer: int,
          start: int, count: int, stream) -> KvSpan:
    h = np.ascontiguousarray(h_table_row, dtype=np.int32)
    return KvSpan(n_kv_heads, head_dim, num_layers, layer, start, count, _ptr(table_row),
                  h.ctypes.data_as(_c_i32p), int(h.shape[0]), _stream_ptr(stream)), h


def kv_export(k_pool, v_pool, table_row, h_table_row, start: int, count: int, layer: int,
              dst, stream=None) -> None:
    """dst [L, 2, count, Hkv, d] (device bf16) <- the span's K/V of this layer's pools; only
    dst[layer] is written. table_row: the request's block-table row (device int32), with its host
    mirror h_table_row."""
    L, two, T, hkv, d = dst.shape
    assert two == 2 and T == count
    sp, keep = _span(table_row, h_table_row, hkv, d, L, layer, start, count, stream)
    kv = _pages(k_pool, v_pool)
    _check(lib().hl_kv_export(ctypes.byref(sp), ctypes.byref(kv), _ptr(dst)), "hl_kv_export")


def kv_import(src, table_row, h_table_row, start: int, count: int, layer: int, k_pool, v_pool,
              stream=None) -> None:
    """The span's slots of this layer's pools <- src[layer] ([L, 2, count, Hkv, d] device bf16)."""
    L, two, T, hkv, d = src.shape
    assert two == 2 and T == count
    sp, keep = _span(table_row, h_table_row, hkv, d, L, layer, start, count, stream)
    kv = _pages(k_pool, v_pool)
    _check(lib().hl_kv_import(ctypes.byref(sp), _ptr(src), ctypes.byref(kv)), "hl_kv_import")


class ModelHandle:
    """Host-side description of a layer stack (keeps the ctypes arrays alive)."""

    def __init__(self, layers, kv_pools, embed, final_norm, lm_head):
        n = len(layers)
        self.weights = (Weights * n)(*[_weights(w) for w in layers])
        self.pages = (KvPages * n)(*[_pages(k, v) for k, v in kv_pools])
        self.c = Model(n, int(embed.shape[0]), _ptr(embed), ctypes.cast(self.weights, ctypes.c_void_p),
                       ctypes.cast(self.pages, ctypes.c_void_p), _ptr(final_norm), _ptr(lm_head))


def model_workspace_bytes(cfg: LayerCfg, b: Batch, model: ModelHandle) -> int:
    d = _desc(cfg, b, None, None, None)
    v = ctypes.c_size_t(0)
    _check(lib().hl_model_workspace_bytes(ctypes.byref(model.c), ctypes.byref(d), ctypes.byref(v)),
           "hl_model_workspace_bytes")
    return int(v.value)


def alloc_model_workspace(cfg: LayerCfg, b: Batch, model: ModelHandle, device="cuda"):
    import torch
    n = max(model_workspace_bytes(cfg, b, model), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def model_step(cfg: LayerCfg, b: Batch, model: ModelHandle, tokens, h_tokens, logits,
               next_tokens, workspace, hidden_out=None, stream=None) -> None:
    """tokens: device int32 [T] with host mirror h_tokens (numpy int32); logits: device bf16
    [num_seqs, vocab]; next_tokens: device int32 [num_seqs]."""
    d = _desc(cfg, b, None, workspace, stream)
    ht = np.ascontiguousarray(h_tokens, dtype=np.int32)
    t = _table(b)
    _check(lib().hl_model_step(ctypes.byref(model.c), ctypes.byref(d), _ptr(tokens),
                               ht.ctypes.data_as(_c_i32p), ctypes.byref(t), _ptr(hidden_out),
                               _ptr(logits), _ptr(next_tokens)), "hl_model_step")


class Scheduler:
    """The native token-budget scheduler (hl_sched_*): host-side batch formation."""

    def __init__(self, budget=0, max_seqs=1, num_blocks=1, max_blocks_per_seq=1, adaptive=False,
                 min_chunk=128, base_chunk=512, max_chunk=4096, pressure_threshold=16):
        p = SchedParams(budget, max_seqs, num_blocks, max_blocks_per_seq, int(bool(adaptive)),
                        min_chunk, base_chunk, max_chunk, pressure_threshold)
        self.h = lib().hl_sched_create(ctypes.byref(p))
        if not self.h:
            raise HLError(HL_ERR_ARG, "hl_sched_create")
        self.max_blocks = max_blocks_per_seq

    def __del__(self):
        if getattr(self, "h", None):
            lib().hl_sched_destroy(self.h)
            self.h = None

    def submit(self, rid: int, prompt_len: int, max_new: int) -> int:
        h = ctypes.c_int32(0)
        _check(lib().hl_sched_submit(self.h, rid, prompt_len, max_new, ctypes.byref(h)),
               "hl_sched_submit")
        return h.value

    def next(self):
        """dict of numpy arrays: q_start, num_cached, request_ids, table [S, max_blocks],
        decode_tokens, emits (copies)."""
        b = SchedBatch()
        _check(lib().hl_sched_next(self.h, ctypes.byref(b)), "hl_sched_next")
        S = b.num_seqs

        def arr(p, n):
            return np.ctypeslib.as_array(p, shape=(n,)).copy() if n else np.zeros(0, np.int32)
        return {"num_tokens": b.num_tokens, "q_start": arr(b.q_start, S + 1) if S else
                np.zeros(1, np.int32), "num_cached": arr(b.num_cached, S),
                "request_ids": arr(b.request_ids, S),
                "table": arr(b.table, S * b.max_blocks_per_seq).reshape(S, b.max_blocks_per_seq),
                "decode_tokens": arr(b.decode_tokens, S), "emits": arr(b.emits, S)}

    def complete(self, next_tokens):
        nt = np.ascontiguousarray(next_tokens, dtype=np.int32)
        fin = np.zeros(max(len(nt), 1), dtype=np.int32)
        nf = ctypes.c_int32(0)
        _check(lib().hl_sched_complete(self.h, nt.ctypes.data_as(_c_i32p),
                                       fin.ctypes.data_as(_c_i32p), ctypes.byref(nf)),
               "hl_sched_complete")
        return fin[:nf.value].tolist()

    def counts(self):
        v = [ctypes.c_int32(0) for _ in range(4)]
        _check(lib().hl_sched_counts(self.h, *[ctypes.byref(x) for x in v]), "hl_sched_counts")
        return tuple(x.value for x in v)  # waiting, prefilling, decoding, free blocks


def _table(b: Batch) -> BlockTable:
    return BlockTable(_ptr(b.table), b.h_table.ctypes.data_as(_c_i32p), b.max_blocks)


def workspace_bytes(cfg: LayerCfg, b: Batch) -> int:
    d = _desc(cfg, b, with_stream=False)
    n = ctypes.c_size_t(0)
    _check(lib().hl_workspace_bytes(ctypes.byref(d), ctypes.byref(n)), "hl_workspace_bytes")
    return int(n.value)


def attention_plan(cfg: LayerCfg, b: Batch) -> Dict[str, int]:
    """hl_attention_plan: how the batch's attention work is laid out (host-only)."""
    d = _desc(cfg, b, with_stream=False)
    v = [ctypes.c_int32(0) for _ in range(6)]
    _check(lib().hl_attention_plan(ctypes.byref(d), *[ctypes.byref(x) for x in v]),
           "hl_attention_plan")
    keys = ("fused", "split_pages", "decode_units", "prefill_parts", "prefill_split",
            "prefill_merges")
    return {k: x.value for k, x in zip(keys, v)}


def alloc_workspace(cfg: LayerCfg, b: Batch, device="cuda"):
    import torch
    n = max(workspace_bytes(cfg, b), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def hybrid_layer_step(cfg: LayerCfg, b: Batch, x, w: Dict[str, object], k_pool, v_pool, out,
                      workspace, stream=None, taps=None, events=None) -> None:
    """events: optional list of HL_STEP_EVENTS torch.cuda.Event (or None) recorded at the step's
    phase boundaries (hl_batch_desc::events)."""
    d = _desc(cfg, b, x, workspace, stream, taps, events=events)
    wt = _weights(w)
    kv = _pages(k_pool, v_pool)
    bt = _table(b)
    _check(lib().hybrid_layer_step(ctypes.byref(d), ctypes.byref(wt), ctypes.byref(kv),
                                   ctypes.byref(bt), _ptr(out)), "hybrid_layer_step")


def rmsnorm(x, gain, y, eps: float, stream=None) -> None:
    rows, cols = x.shape
    _check(lib().hl_rmsnorm(_ptr(x), _ptr(gain), _ptr(y), rows, cols, eps, _stream_ptr(stream)),
           "hl_rmsnorm")


def gemm_bf16_nt(a, w, c, residual=None, epilogue: int = HL_EPI_NONE, workspace=None,
                 stream=None, row_scale=None) -> None:
    m, k = a.shape
    n = w.shape[0]
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hl_gemm_bf16_nt(_ptr(a), _ptr(w), _ptr(c), _ptr(residual), _ptr(row_scale), m,
                                 n, k, epilogue, _ptr(workspace), wsb, _stream_ptr(stream)),
           "hl_gemm_bf16_nt")


def gemm_bf16_nt_tiled(a, w, c, tile_m: int, tile_n: int, stream_k: int = 0, residual=None,
                       epilogue: int = HL_EPI_NONE, workspace=None, stream=None,
                       row_scale=None) -> None:
    """stream_k: 0 one tile per workgroup, 1 stream-K (plain / residual), s >= 2 split-K into s
    K ranges, -s one tile per workgroup with the tiles past the last full round split into s K
    ranges."""
    m, k = a.shape
    n = w.shape[0]
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hl_gemm_bf16_nt_tiled(_ptr(a), _ptr(w), _ptr(c), _ptr(residual), _ptr(row_scale),
                                       m, n, k, epilogue, tile_m, tile_n, int(stream_k),
                                       _ptr(workspace), wsb, _stream_ptr(stream)),
           "hl_gemm_bf16_nt_tiled")


GEMM_TILES = ((256, 256), (224, 256), (192, 256), (160, 256), (128, 256), (256, 128), (224, 128),
              (160, 128), (128, 128))
# SwiGLU epilogue only, one tile per workgroup (stream_k 0)
SWIGLU_TILES = ((256, 192), (128, 192))


def gemm_workspace_bytes(m: int, n: int, k: int, epilogue: int = HL_EPI_NONE) -> int:
    v = ctypes.c_size_t(0)
    _check(lib().hl_gemm_workspace_bytes(m, n, k, epilogue, ctypes.byref(v)),
           "hl_gemm_workspace_bytes")
    return int(v.value)


def gemm_tile_choice(m: int, n: int, k: int, epilogue: int = HL_EPI_NONE,
                     with_workspace: bool = True, qkv_head_dim: int = 0):
    """(tile_m, tile_n, schedule, splits) that hl_gemm_bf16_nt (or, with qkv_head_dim, the step's
    QKV projection) uses for this shape; schedule 0 = one tile per workgroup, 1 = stream-K, 2 =
    the weight-streaming path of up to 64 token rows, 3 = split-K into `splits` K ranges, 4 = one
    tile per workgroup with the tiles past the last full round split into `splits` K ranges.
    Host-only."""
    tm, tn, sk, sp = (ctypes.c_int32(0) for _ in range(4))
    _check(lib().hl_gemm_tile_choice(m, n, k, epilogue, int(bool(with_workspace)), qkv_head_dim,
                                     ctypes.byref(tm), ctypes.byref(tn), ctypes.byref(sk),
                                     ctypes.byref(sp)),
           "hl_gemm_tile_choice")
    return tm.value, tn.value, int(sk.value), int(sp.value)


def rms_scale(x, gain, xg, row_scale, eps: float, stream=None) -> None:
    rows, cols = x.shape
    _check(lib().hl_rms_scale(_ptr(x), _ptr(gain), _ptr(xg), _ptr(row_scale), rows, cols, eps,
                              _stream_ptr(stream)), "hl_rms_scale")


def _weights(w) -> Weights:
    return Weights(*(_ptr(w.get(k)) for k in ("attn_norm", "w_qkv", "w_o", "mlp_norm",
                                                "w_gate_up", "w_down")))


def qkv_rope_append(cfg: LayerCfg, b: Batch, x, w, q_rot, k_pool, v_pool, workspace,
                    stream=None) -> None:
    d = _desc(cfg, b, x, workspace, stream)
    wt = _weights(w)
    kv = _pages(k_pool, v_pool)
    bt = _table(b)
    _check(lib().hl_qkv_rope_append(ctypes.byref(d), ctypes.byref(wt), _ptr(q_rot),
                                    ctypes.byref(kv), ctypes.byref(bt)), "hl_qkv_rope_append")


def rope_kv_append(cfg: LayerCfg, b: Batch, qkv, q_rot, k_pool, v_pool, stream=None) -> None:
    d = _desc(cfg, b, stream=stream)
    kv = _pages(k_pool, v_pool)
    bt = _table(b)
    _check(lib().hl_rope_kv_append(ctypes.byref(d), _ptr(qkv), _ptr(q_rot), ctypes.byref(kv),
                                   ctypes.byref(bt)), "hl_rope_kv_append")


def _attn(fn_name, cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, stream):
    d = _desc(cfg, b, None, workspace, stream)
    kv = _pages(k_pool, v_pool)
    bt = _table(b)
    _check(getattr(lib(), fn_name)(ctypes.byref(d), _ptr(q_rot), ctypes.byref(kv),
                                   ctypes.byref(bt), _ptr(attn_out)), fn_name)


def attention(cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, stream=None) -> None:
    _attn("hl_attention", cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, stream)


def prefill_attention(cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, stream=None) -> None:
    _attn("hl_prefill_attention", cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, stream)


def decode_attention(cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, stream=None) -> None:
    _attn("hl_decode_attention", cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, stream)


ATTN_PREFILL, ATTN_DECODE, ATTN_BOTH = 1, 2, 3


def attention_build_lists(cfg, b, k_pool, v_pool, workspace, stream=None) -> None:
    """hl_attention_build_lists: the batch's attention work lists into the workspace."""
    d = _desc(cfg, b, None, workspace, stream)
    kv = _pages(k_pool, v_pool)
    bt = _table(b)
    _check(lib().hl_attention_build_lists(ctypes.byref(d), ctypes.byref(kv), ctypes.byref(bt)),
           "hl_attention_build_lists")


def attention_run(cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, q_lo=None,
                  paths: int = ATTN_BOTH, stream=None) -> None:
    """hl_attention_run on lists built by attention_build_lists (paths: 1 prompt-chunk rows,
    2 decode rows, 3 both; q_lo: optional low half of a two-part query)."""
    d = _desc(cfg, b, None, workspace, stream)
    kv = _pages(k_pool, v_pool)
    bt = _table(b)
    _check(lib().hl_attention_run(ctypes.byref(d), _ptr(q_rot), _ptr(q_lo), ctypes.byref(kv),
                                  ctypes.byref(bt), _ptr(attn_out), int(paths)),
           "hl_attention_run")


def attention_run_traced(cfg, b, q_rot, k_pool, v_pool, attn_out, workspace, trace, q_lo=None,
                         paths: int = ATTN_BOTH, stream=None) -> None:
    """hl_attention_run_traced: trace is a device int64 tensor of 3 * items entries ((start, end,
    workgroup) per work item, prefill items first; see the header)."""
    d = _desc(cfg, b, None, workspace, stream)
    kv = _pages(k_pool, v_pool)
    bt = _table(b)
    _check(lib().hl_attention_run_traced(ctypes.byref(d), _ptr(q_rot), _ptr(q_lo), ctypes.byref(kv),
                                         ctypes.byref(bt), _ptr(attn_out), int(paths), _ptr(trace),
                                         trace.numel()),
           "hl_attention_run_traced")


def trace_clock_khz() -> int:
    v = ctypes.c_int32(0)
    _check(lib().hl_trace_clock_khz(ctypes.byref(v)), "hl_trace_clock_khz")
    return int(v.value)
