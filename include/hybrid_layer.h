/*
 * hybrid_layer.h - C ABI of one transformer-layer forward step over a hybrid batch on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation. A hybrid batch stacks the new tokens of prompt chunks and of decoding requests
 * into one token matrix. The linear layers (QKV, output projection, SwiGLU MLP) multiply that
 * whole matrix by the same weights, so the weights are read once for both phases; attention then
 * splits, because each request attends only to its own keys and values ("ConfluxServe:
 * Reconciling Resource Utilization and Parallelism Efficiency across Prefill and Decode in LLM
 * Serving", sections "The big picture: what happens inside one Transformer layer" and "Why can
 * linear layers be batched but attention cannot?"). Every request brings a start position (tokens
 * already in the KV cache) and a count of new tokens; prompt chunks write their keys and values
 * into the paged cache and attend causally to everything cached for their request, decodes
 * append one token ("Chunked prefill (stall-free batching), explained", "How it works, step by
 * step"). A query at absolute position p sees keys 0..p; query head h reads KV head
 * h / (n_q_heads / n_kv_heads) ("7.8 Disaggregated Prefill/Decode & Chunked Prefill", "Attention
 * on Partial KV Caches" and its GQA exercise).
 *
 * Layer definition (pre-norm, no biases):
 *   h1  = RMSNorm(x) * attn_norm                      RMSNorm(z) = z / sqrt(mean(z^2) + eps)
 *   qkv = h1 W_qkv^T            -> q [T, Hq, d], k, v [T, Hkv, d]
 *   q, k rotated at position num_cached[s] + i: pair (j, j + d/2) turns by p * theta^(-2j/d)
 *   k, v appended to the paged cache; o = causal softmax(q K^T * scale) V per request
 *   h2  = x + o W_o^T
 *   out = h2 + (silu(h3 W_gate^T) * (h3 W_up^T)) W_down^T,   h3 = RMSNorm(h2) * mlp_norm
 * A sequence with q_len == 1 takes the decode path (split-KV attention); q_len > 1 takes the
 * prefill path (tiled causal attention). Both produce the same mathematics.
 *
 * Numbers: bf16 storage (raw bits, round-to-nearest-even), fp32 accumulation and fp32 softmax.
 *
 * Memory. Every pointer marked "device" is HIP device memory of the current device, 16-byte
 * aligned. "host" pointers are ordinary host memory, read only during the call. The caller
 * allocates and frees everything (weights, cache pools, tables, x, out, workspace, stream); the
 * library allocates nothing and keeps no state between calls.
 *
 * Execution. Calls are asynchronous: they validate on the host, enqueue kernels on `stream` and
 * return. Results are valid once the stream has completed. No call synchronises the device.
 * Calls with distinct workspaces may run concurrently on different streams.
 *
 * Errors. Every entry point returns HL_OK (0) or a negative HL_ERR_* code. Validation reads only
 * the host mirrors and happens before anything is enqueued: on a validation error nothing is
 * launched and nothing is written.
 */
#ifndef HYBRID_LAYER_H
#define HYBRID_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HL_VERSION 2 /* 2: hl_batch_desc gained `events` (its layout changed) */
#define HL_BLOCK_SIZE 16 /* tokens per KV page */

enum {
  HL_OK = 0,
  HL_ERR_NULL = -1,      /* a required pointer is NULL */
  HL_ERR_SHAPE = -2,     /* unsupported layer dimensions (see hl_layer_cfg) */
  HL_ERR_DESC = -3,      /* bad batch descriptor: q_len < 1, q_start not starting at 0 or not
                            increasing, q_start[S] != num_tokens, num_cached < 0, or
                            num_tokens * max(hidden, d_ff, Hq * head_dim) >= 2^31 */
  HL_ERR_BLOCK = -4,     /* a sequence needs more than max_blocks_per_seq pages, or a used
                            block id lies outside [0, num_blocks) */
  HL_ERR_ALIGN = -5,     /* a device pointer is not 16-byte aligned */
  HL_ERR_WORKSPACE = -6, /* workspace NULL or smaller than hl_workspace_bytes() */
  HL_ERR_HIP = -7,       /* a kernel launch failed */
  HL_ERR_ARG = -8        /* other invalid argument (sizes, epilogue id) */
};

typedef uint16_t hl_bf16; /* raw bfloat16 bits */

/* Layer dimensions. Supported: head_dim in {64, 128}; n_q_heads % n_kv_heads == 0 and
 * n_q_heads / n_kv_heads <= 16; hidden % 128 == 0; d_ff % 64 == 0; n_q_heads * head_dim % 64 == 0;
 * (n_q_heads + 2 n_kv_heads) * head_dim % 256 == 0; every weight matrix and every
 * max(hidden, d_ff, n_q_heads * head_dim)-wide row block below 2^31 elements; block_size ==
 * HL_BLOCK_SIZE; rms_eps >= 0, rope_theta > 0, softmax_scale >= 0. softmax_scale == 0 means
 * 1 / sqrt(head_dim). Anything else is HL_ERR_SHAPE. */
typedef struct {
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t d_ff;
  int32_t block_size;
  float rms_eps;
  float rope_theta;
  float softmax_scale;
} hl_layer_cfg;

/* One hybrid batch. Sequence s owns token rows q_start[s] .. q_start[s+1]-1 of x and out; those
 * rows are its new tokens at positions num_cached[s] .. num_cached[s] + q_len - 1. Rows may come
 * in any sequence order (the benchmarks put prompt chunks first, then decodes).
 * q_start / num_cached are given twice: on the device (read by kernels) and as host mirrors
 * (validation and launch planning, so the call never waits for the device); both must hold the
 * same values. The tap pointers, when non-NULL, receive copies of intermediate tensors:
 * tap_q_rot [T, Hq*d] (rotated queries), tap_attn_out [T, Hq*d] (attention output before W_o),
 * tap_h2 [T, hidden] (residual stream after attention). `attention` picks how prefill and decode
 * attention are launched when the batch has both: HL_ATTN_AUTO (0, a zero-initialised
 * descriptor) lets the library choose (hl_attention_plan reports the choice), HL_ATTN_FUSED one
 * launch for both paths, HL_ATTN_SEPARATE two launches; the results are bit-identical either way.
 * The workspace size depends on it: pass the same descriptor to hl_workspace_bytes.
 * `events`, when non-NULL, points to HL_STEP_EVENTS hipEvent_t handles (any entry may be NULL)
 * that hybrid_layer_step (and hybrid_layer_step_noalloc) records on its stream at the boundaries
 * of its phases, so a caller can time each phase inside real steps (hipEventElapsedTime between
 * consecutive marks): [0] before the first norm pass (token info, work lists), [1] after the QKV
 * projection with its RoPE / KV-append epilogue, [2] after attention (its merges included),
 * [3] after the O projection, [4] after the MLP norm pass, [5] after the gate/up projection,
 * [6] after the down projection. A failed record is HL_ERR_HIP; the other entry points ignore
 * the field. */
enum { HL_ATTN_AUTO = 0, HL_ATTN_FUSED = 1, HL_ATTN_SEPARATE = 2 };
#define HL_STEP_EVENTS 7
typedef struct {
  const hl_layer_cfg* cfg;
  int32_t num_seqs;
  int32_t num_tokens;
  const int32_t* q_start;      /* device [num_seqs + 1] */
  const int32_t* num_cached;   /* device [num_seqs] */
  const int32_t* h_q_start;    /* host   [num_seqs + 1] */
  const int32_t* h_num_cached; /* host   [num_seqs] */
  const hl_bf16* x;            /* device [num_tokens, hidden] */
  void* workspace;             /* device, hl_workspace_bytes() bytes, 256-byte aligned */
  size_t workspace_bytes;
  void* stream;                /* hipStream_t; NULL = the null stream */
  hl_bf16* tap_q_rot;          /* device, optional */
  hl_bf16* tap_attn_out;       /* device, optional */
  hl_bf16* tap_h2;             /* device, optional */
  int32_t attention;           /* HL_ATTN_AUTO / HL_ATTN_FUSED / HL_ATTN_SEPARATE */
  void* const* events;         /* optional: HL_STEP_EVENTS hipEvent_t handles (phase marks) */
} hl_batch_desc;

/* Weights, all device, row-major [out_features, in_features] (each row one output feature). */
typedef struct {
  const hl_bf16* attn_norm; /* [hidden] */
  const hl_bf16* w_qkv;     /* [(Hq + 2 Hkv) d, hidden]: q rows, then k rows, then v rows */
  const hl_bf16* w_o;       /* [hidden, Hq d] */
  const hl_bf16* mlp_norm;  /* [hidden] */
  const hl_bf16* w_gate_up; /* [2 d_ff, hidden]: the d_ff gate rows, then the d_ff up rows */
  const hl_bf16* w_down;    /* [hidden, d_ff] */
} hl_weights;

/* Paged KV cache of this layer. Each (block, kv head) page is one contiguous 4 KB run (for
 * d = 128), as the head-before-token layout of "Gescheiden Prefill en Decode" (section on
 * sharded KV cache transfers) keeps a head's page contiguous:
 *   k: [num_blocks][n_kv_heads][head_dim / 8][16 tokens][8]   (chunk-major page: elements
 *      8c .. 8c+7 of token t at ((c * 16) + t) * 8 within the page)
 *   v: [num_blocks][n_kv_heads][head_dim][16 tokens]          (dim-major page: V columns)
 * Keys are stored after the rotary embedding. The step writes only the slots of its new tokens;
 * every other byte is left as it was. Pages written by one step must not be shared between
 * sequences. */
typedef struct {
  hl_bf16* k;
  hl_bf16* v;
  int64_t num_blocks;
} hl_kv_pages;

/* Block table: row s maps logical page j of sequence s (positions 16j .. 16j+15) to a physical
 * block id. Device copy for the kernels, host mirror for validation; entries beyond
 * ceil((num_cached + q_len) / 16) of a row are never read. */
typedef struct {
  const int32_t* table;   /* device [num_seqs, max_blocks_per_seq] */
  const int32_t* h_table; /* host   [num_seqs, max_blocks_per_seq] */
  int32_t max_blocks_per_seq;
} hl_block_table;

/* ---- the step ------------------------------------------------------------------------------ */

/* One forward pass of the layer over the hybrid batch: writes out [num_tokens, hidden] (device)
 * and appends the batch's new K/V rows into kv. `out` must not alias x, the cache or the
 * workspace. Returns HL_OK or an HL_ERR_* code (nothing launched on a validation error). */
int hybrid_layer_step(const hl_batch_desc* batch, const hl_weights* weights, hl_kv_pages* kv,
                      const hl_block_table* block_table, hl_bf16* out);

/* The layer step for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Identical to hybrid_layer_step (same
 * kernels, same results bit for bit), except that batch->workspace and batch->workspace_bytes
 * are ignored: the workspace is a fixed array of HL_NOALLOC_SCRATCH_MIB MiB inside the library,
 * one per device, held until the process ends. The call allocates nothing (no hipMalloc, no
 * library allocation); its first call on a device looks that device's array up. Batches whose
 * hl_workspace_bytes() exceeds the array return HL_ERR_WORKSPACE with nothing launched. All calls
 * on one device share its array, so calls that overlap on one device (other streams, other
 * threads) race and must be serialised by the caller; a call reads nothing a previous call left.
 * Errors as hybrid_layer_step, and HL_ERR_HIP if the array cannot be looked up. */
#define HL_NOALLOC_SCRATCH_MIB 192
int hybrid_layer_step_noalloc(const hl_batch_desc* batch, const hl_weights* weights,
                              hl_kv_pages* kv, const hl_block_table* block_table, hl_bf16* out);

/* Workspace the step (and the phase entries) need for this batch, from the host mirrors only.
 * Writes the byte count to *bytes. */
int hl_workspace_bytes(const hl_batch_desc* batch, size_t* bytes);

/* How the attention of this batch is laid out (host-only, from the host mirrors; no GPU needed),
 * for tuning and tests. Work splits follow from the batch alone ("Chunked prefill (stall-free
 * batching), explained", "How it works, step by step": a chunk attends to its cached prefix plus
 * itself; decode attention is split over the KV length). Outputs:
 *   fused          0 for two launches; 1 if prefill and decode attention run in one launch, 2 if
 *                  they do and its decode units also prefetch their successors (decode-heavy);
 *   split_pages    KV pages per decode work unit;
 *   decode_units   decode work units (each covers all KV heads);
 *   prefill_parts  prefill work entries: 128-query-row tiles, or parts of a tile's key range;
 *   prefill_split  key tiles (64 keys) per part, or 2^30 when no tile is split;
 *   prefill_merges tiles whose parts are merged by the merge pass.
 * Errors: HL_ERR_NULL, and those of hl_workspace_bytes. */
int hl_attention_plan(const hl_batch_desc* batch, int32_t* fused, int32_t* split_pages,
                      int32_t* decode_units, int32_t* prefill_parts, int32_t* prefill_split,
                      int32_t* prefill_merges);

/* Static text for an HL_* code; never NULL. */
const char* hl_strerror(int code);

/* HL_VERSION of the library. */
int hl_version(void);

/* ---- a model step: embedding, the layer stack, LM head, greedy token --------------------- */

/* A decoder stack of num_layers layers of one hl_layer_cfg shape. Every layer has its own
 * weights and its own KV pools; all pools have the same num_blocks and share one block table
 * (a sequence's logical page j is block table[s][j] in every layer). */
typedef struct {
  int32_t num_layers;
  int32_t vocab;              /* multiple of 128 */
  const hl_bf16* embed;       /* device [vocab, hidden] */
  const hl_weights* layers;   /* host array [num_layers] */
  hl_kv_pages* kv;            /* host array [num_layers] */
  const hl_bf16* final_norm;  /* device [hidden] */
  const hl_bf16* lm_head;     /* device [vocab, hidden] */
} hl_model;

/* Workspace of hl_model_step for this batch (the layer step's own, plus the residual stream and
 * the per-sequence last rows), from the host mirrors only. */
int hl_model_workspace_bytes(const hl_model* model, const hl_batch_desc* batch, size_t* bytes);

/* One iteration over the hybrid batch, every layer in turn: x = embed[tokens]; for each layer,
 * x = hybrid_layer_step(x) (each appending the batch's K/V rows to its own pools); then for the
 * last new token of each sequence s, logits[s] = RMSNorm(x[row], final_norm) lm_head^T (bf16,
 * [num_seqs, vocab]) and next_tokens[s] = the first index of its largest logit (greedy). A request
 * whose last prompt chunk completes takes its first token from this same pass ("Chunked prefill
 * (stall-free batching), explained", "How it works, step by step"); chapter 7.8's prefill listing
 * takes the logits of the last position only and their argmax. For a chunk that does not end
 * its prompt, next_tokens[s] is computed but has no meaning. tokens: device [num_tokens] with host
 * mirror h_tokens (ids checked against vocab); batch->x is ignored; batch->workspace must hold
 * hl_model_workspace_bytes() bytes. hidden_out (optional, device [num_tokens, hidden]) receives x
 * after the last layer (before the final norm). No host synchronisation and no allocation: the
 * call can be captured in a HIP graph (replays repeat the same batch). Errors as
 * hybrid_layer_step; HL_ERR_ARG for num_layers < 1, vocab % 128, an id outside [0, vocab) or
 * pools of different sizes. */
int hl_model_step(const hl_model* model, const hl_batch_desc* batch, const int32_t* tokens,
                  const int32_t* h_tokens, const hl_block_table* block_table, hl_bf16* hidden_out,
                  hl_bf16* logits, int32_t* next_tokens);

/* ---- token-budget scheduler (host) ------------------------------------------------------- */

/* The iteration-level scheduler of chunked prefill that produces the hybrid batches: each
 * iteration fills a token budget with one token per running decode, then the next chunk of the
 * prompt being prefilled, then waiting requests in arrival order while budget, sequence slots and
 * KV blocks remain ("Chunked prefill (stall-free batching), explained", "How it works, step by
 * step"). With adaptive != 0 the prefill share follows chapter 7.8's dynamic chunk sizing
 * ("Priority and Preemption Policies"): max_chunk while no request decodes, min_chunk once
 * pressure_threshold or more do, and with d decoding in between the line from base_chunk down to
 * min_chunk rounded down, base_chunk - ceil(d (base_chunk - min_chunk) / pressure_threshold).
 * That share is the iteration's whole prompt-token count, however many prompts it is spread
 * over; the decode tokens come on top of it. A request is admitted only when
 * blocks for its whole lifetime (prompt + outputs, 16 tokens per block) are free; they are taken
 * from one free list of num_blocks ids (the pages of every layer's pool) and returned when it
 * finishes, so nothing is ever preempted. Host memory only; not thread-safe. */
typedef struct {
  int32_t budget;               /* tokens per iteration (fixed policy) */
  int32_t max_seqs;             /* sequences prefilling or decoding at once */
  int32_t num_blocks;           /* KV blocks in the pool */
  int32_t max_blocks_per_seq;   /* block-table row length */
  int32_t adaptive;             /* 0: fixed budget; 1: dynamic chunk sizing */
  int32_t min_chunk, base_chunk, max_chunk, pressure_threshold;  /* adaptive policy */
} hl_sched_params;

/* One iteration's batch, in the layout of hl_batch_desc / hl_block_table (host arrays owned by
 * the scheduler, valid until the next hl_sched_next). Sequences are in priority order: decodes,
 * then prompt chunks. decode_tokens[s] is the token a decode feeds (its last output), -1 for a
 * prompt chunk (the caller supplies prompt tokens num_cached[s] .. num_cached[s] + q_len - 1);
 * emits[s] = 1 if sequence s takes a new token from this iteration (decodes, and prompts whose
 * last chunk this is). */
typedef struct {
  int32_t num_seqs, num_tokens;
  const int32_t* q_start;        /* [num_seqs + 1] */
  const int32_t* num_cached;     /* [num_seqs] */
  const int32_t* request_ids;    /* [num_seqs] */
  const int32_t* table;          /* [num_seqs, max_blocks_per_seq] */
  const int32_t* decode_tokens;  /* [num_seqs] */
  const int32_t* emits;          /* [num_seqs] */
  int32_t max_blocks_per_seq;
} hl_sched_batch;

typedef struct hl_sched hl_sched;

/* NULL for invalid parameters (or no memory). */
hl_sched* hl_sched_create(const hl_sched_params* params);
void hl_sched_destroy(hl_sched* sched);
/* Queue a request (arrival order = call order). HL_ERR_ARG for lengths < 1, HL_ERR_BLOCK if its
 * lifetime needs more than max_blocks_per_seq blocks or more than the pool's num_blocks (such a
 * request could never be admitted, and admission in arrival order would then hold back every
 * later one). *handle: its index. */
int hl_sched_submit(hl_sched* sched, int32_t request_id, int32_t prompt_len,
                    int32_t max_new_tokens, int32_t* handle);
/* The next iteration's batch (possibly empty: num_seqs == 0). */
int hl_sched_next(hl_sched* sched, hl_sched_batch* batch);
/* After the iteration ran: next_tokens[s] (host, one per sequence of the last batch; read where
 * emits[s] is 1) advance every sequence; finished requests (their outputs complete) free their
 * blocks and are listed in finished_ids (optional, room for num_seqs) / *num_finished. */
int hl_sched_complete(hl_sched* sched, const int32_t* next_tokens, int32_t* finished_ids,
                      int32_t* num_finished);
/* Queue sizes and free blocks (any pointer may be NULL). */
int hl_sched_counts(const hl_sched* sched, int32_t* waiting, int32_t* prefilling,
                    int32_t* decoding, int32_t* free_blocks);

/* ---- KV transfer between instances ------------------------------------------------------ */

/* One request's token span [start, start + count) of one layer, for the KV hand-off between a
 * prefill instance and a decode instance. The transfer tensor of a request is
 * [num_layers][2][count][n_kv_heads][head_dim] bf16 (layer, K then V, token, KV head, dim), the
 * shape "7.8 Disaggregated Prefill/Decode & Chunked Prefill" gives for the KV cache a prefill
 * worker transmits ("Lifecycle of a Request", step 3); it moves one layer slice at a time, each as
 * soon as that layer has written its rows ("Layer-Wise Pipelining"). `table` is the request's
 * block-table row (device) with its host mirror `h_table` (validation only), `table_len` entries.
 * head_dim in {64, 128}; 0 <= layer < num_layers; start >= 0, count >= 0, start + count <=
 * 16 * table_len. */
typedef struct {
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t num_layers;
  int32_t layer;
  int32_t start;
  int32_t count;
  const int32_t* table;   /* device [table_len] */
  const int32_t* h_table; /* host   [table_len] */
  int32_t table_len;
  void* stream;           /* hipStream_t; NULL = the null stream */
} hl_kv_span;

/* Export: dst[layer][0][i] = K of position start + i, dst[layer][1][i] = V of it, for every KV
 * head (dst is the whole [num_layers][2][count][n_kv_heads][head_dim] buffer, device; only the
 * layer's slice is written). Bit-exact copy; the pool is only read. Errors: HL_ERR_NULL,
 * HL_ERR_ARG (span fields), HL_ERR_BLOCK (a page of the span outside [0, num_blocks)),
 * HL_ERR_ALIGN (pointers not 16-byte aligned), HL_ERR_HIP. Asynchronous on span->stream. */
int hl_kv_export(const hl_kv_span* span, const hl_kv_pages* kv, hl_bf16* dst);

/* Import: the inverse scatter of src's layer slice into the slots of positions start .. start +
 * count - 1 under this span's table (which may differ from the exporter's). Every other byte of
 * both pools keeps its value. Errors as hl_kv_export. */
int hl_kv_import(const hl_kv_span* span, const hl_bf16* src, hl_kv_pages* kv);

/* ---- the phases the step is composed of (same conventions; used by tests and benchmarks) --- */

/* y[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * gain, rows x cols, all device bf16.
 * cols % 8 == 0. No page defines the normalisation inside the layer: the pages name the linears
 * and attention of the step, and RMSNorm is the norm of the layer shapes the step is measured on
 * (a pre-norm block, the Qwen3 / Llama-70B shapes). This is its standard definition. Errors:
 * HL_ERR_NULL, HL_ERR_ARG (rows < 0, cols not a positive multiple of 8, eps < 0), HL_ERR_ALIGN,
 * HL_ERR_HIP. */
int hl_rmsnorm(const hl_bf16* x, const hl_bf16* gain, hl_bf16* y, int32_t rows, int32_t cols,
               float eps, void* stream);

/* RMSNorm split into its two factors, for a following linear layer: xg[r, :] = x[r, :] * gain
 * (bf16) and row_scale[r] = 1 / sqrt(mean(x[r, :]^2) + eps) (fp32 [rows]), so that
 * RMSNorm(x) W^T = row_scale * (xg W^T) with no rounding of the normalised row. cols % 8 == 0.
 * As for hl_rmsnorm, no page defines the norm; it is the standard RMSNorm of the measured layer
 * shapes, factored so that the token-batched linear that follows applies it. Errors as
 * hl_rmsnorm. */
int hl_rms_scale(const hl_bf16* x, const hl_bf16* gain, hl_bf16* xg, float* row_scale,
                 int32_t rows, int32_t cols, float eps, void* stream);

/* Token-batched linear layer C = s * (A W^T) with A [m, k] and W [n, k] (both k-contiguous), bf16
 * in, fp32 accumulation, bf16 out; s = row_scale[row] (fp32 [m]) or 1 when row_scale is NULL.
 * The rows of A are the tokens of every request of the batch, prompt chunks and decodes alike:
 * a linear layer treats each token row on its own, so one multiply serves the whole hybrid batch
 * and reads the weights once ("ConfluxServe" summary, "Why can linear layers be batched but
 * attention cannot?"; "Chunked prefill (stall-free batching), explained", "The bottleneck:
 * prefill-decode interference", on decode rows riding along in the prompt's multiply).
 * epilogue:
 *   HL_EPI_NONE     c [m, n] = s * A W^T
 *   HL_EPI_RESIDUAL c [m, n] = residual [m, n] + s * A W^T
 *   HL_EPI_SWIGLU   W holds 2f rows (f = n / 2 gate rows, then f up rows);
 *                   c [m, f] = silu(s * A W_gate^T) * (s * A W_up^T)
 * Requirements: k % 64 == 0, n % 128 == 0, m >= 0, m * k and n * k at most 2^31 - 1 (operands
 * are addressed with 32-bit byte offsets; HL_ERR_ARG otherwise). `workspace` (device, may be
 * NULL): when it holds hl_gemm_workspace_bytes() bytes, up to 64 token rows take a split-K
 * weight-streaming path (fp32 partials in the workspace, summed in a fixed order by the epilogue
 * pass), and larger shapes may run a stream-K schedule (partial tiles summed by a fix-up pass);
 * without it every shape runs one tile per workgroup. Results agree to fp32 summation order. */
enum { HL_EPI_NONE = 0, HL_EPI_RESIDUAL = 1, HL_EPI_SWIGLU = 2 };
int hl_gemm_bf16_nt(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, const hl_bf16* residual,
                    const float* row_scale, int32_t m, int32_t n, int32_t k, int32_t epilogue,
                    void* workspace, size_t workspace_bytes, void* stream);
int hl_gemm_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t epilogue, size_t* bytes);

/* hl_gemm_bf16_nt with the tile shape and schedule given by the caller instead of chosen (for
 * tuning and tests). tile_m x tile_n must be one of 256x256, 224x256, 192x256, 160x256, 128x256,
 * 256x128, 224x128, 160x128, 128x128 with n % tile_n == 0, or, for HL_EPI_SWIGLU with stream_k 0
 * only, 256x192 or 128x192 (96 gate and 96 up rows per tile). stream_k: 0 one tile per workgroup;
 * 1 a stream-K schedule (HL_EPI_NONE / HL_EPI_RESIDUAL); s >= 2 split-K into s equal K ranges
 * (any epilogue; s <= k / 64, and the s fp32 pieces per tile must fit the workspace); -s with
 * 2 <= s <= 8 one tile per workgroup for the full rounds of tiles over the compute units and the
 * tiles left over split into s K ranges (any epilogue; same limits; with no tile left over it is
 * schedule 0). Any schedule but 0 needs `workspace` of hl_gemm_workspace_bytes(). Results agree with
 * hl_gemm_bf16_nt to fp32 summation order. Errors as hl_gemm_bf16_nt, and HL_ERR_ARG for an
 * unsupported tile or schedule. */
int hl_gemm_bf16_nt_tiled(const hl_bf16* a, const hl_bf16* w, hl_bf16* c,
                          const hl_bf16* residual, const float* row_scale, int32_t m, int32_t n,
                          int32_t k, int32_t epilogue, int32_t tile_m, int32_t tile_n,
                          int32_t stream_k, void* workspace, size_t workspace_bytes, void* stream);

/* The tile shape (*tile_m x *tile_n outputs per workgroup) and schedule (*stream_k: 1 for a
 * stream-K run with a fix-up pass, 0 for one tile per workgroup, 2 for the weight-streaming path of
 * up to 64 token rows, whose workgroups each cover 64 columns of all rows over a K range, 3 for
 * split-K into *splits equal K ranges summed by a fix-up pass that applies the epilogue, 4 for one
 * tile per workgroup with the tiles past the last full round over the compute units split into
 * *splits K ranges; *splits is 0 otherwise) that hl_gemm_bf16_nt uses for
 * these arguments (with_workspace != 0: a stream-K workspace is passed). qkv_head_dim 64 or 128
 * asks instead for the QKV projection of the layer step (RoPE + KV-append epilogue: whole heads
 * per tile); 0 otherwise. Host-only: no device work, no GPU needed. The choice minimises a cost
 * model of the launch (rounds of tiles over the compute units, the stream-K run length, or the
 * split-K rounds, plus the fix-up traffic); the token count of a hybrid batch is arbitrary, so
 * fixed tiles would hit the tile-quantisation cliff that the chunked-prefill page describes.
 * Errors: HL_ERR_NULL, HL_ERR_ARG (the same size rules as hl_gemm_bf16_nt). */
int hl_gemm_tile_choice(int32_t m, int32_t n, int32_t k, int32_t epilogue, int32_t with_workspace,
                        int32_t qkv_head_dim, int32_t* tile_m, int32_t* tile_n, int32_t* stream_k,
                        int32_t* splits);

/* First half of the layer up to attention, as the step runs it: RMSNorm of batch->x (gain
 * w->attn_norm), the QKV projection (w->w_qkv) and, in the same kernel's epilogue, the rotary
 * embedding of q and k and the append of the new K/V rows into their pages. Writes q_rot
 * [num_tokens, Hq d] (device). Uses the batch workspace. */
int hl_qkv_rope_append(const hl_batch_desc* batch, const hl_weights* weights, hl_bf16* q_rot,
                       hl_kv_pages* kv, const hl_block_table* block_table);

/* Rotary embedding of q and k and KV append, on its own. qkv [num_tokens, (Hq + 2 Hkv) d]
 * (device, the QKV projection output); writes q_rot [num_tokens, Hq d] and the new K (rotated)
 * and V rows into their pages: position p of sequence s goes to block table[s][p / 16], slot
 * p % 16. Every new token is written at its absolute position: a prompt chunk of n tokens after
 * num_cached cached ones writes positions num_cached .. num_cached + n - 1 and a decode appends
 * one ("Chunked prefill (stall-free batching), explained", "How it works, step by step", the
 * forward pass over (start_pos, n) per request; "7.8 Disaggregated Prefill/Decode & Chunked
 * Prefill", "Attention on Partial KV Caches", a chunk's keys and values written into the cache
 * before its attention). Rotation: pair (j, j + d/2) turns by p * theta^(-2j/d), applied to q and
 * k, never v. Only the slots of the batch's new tokens change; every other byte of both pools is
 * left as it was. Errors: HL_ERR_NULL, HL_ERR_ALIGN, those of the batch descriptor
 * (HL_ERR_SHAPE, HL_ERR_DESC) and of the table (HL_ERR_BLOCK), HL_ERR_HIP. */
int hl_rope_kv_append(const hl_batch_desc* batch, const hl_bf16* qkv, hl_bf16* q_rot,
                      hl_kv_pages* kv, const hl_block_table* block_table);

/* Attention of every sequence of the batch over its cached keys plus its new ones (the new K/V
 * must already be in the cache, as hl_rope_kv_append leaves them). q_rot [T, Hq d] device;
 * writes attn_out [T, Hq d]. Uses the batch workspace. hl_prefill_attention computes only rows of
 * sequences with q_len > 1, hl_decode_attention only rows of sequences with q_len == 1 (other
 * rows are left untouched). hl_attention computes both: when the batch holds both kinds it runs
 * them either as two launches or in ONE fused launch whose persistent workers share every compute
 * unit between the compute-bound prefill items and the bandwidth-bound decode units (the two
 * attention paths of a hybrid step are independent and overlap: "ConfluxServe" summary, "Why can
 * linear layers be batched but attention cannot?"; a fused prefill-decode kernel is what the
 * overlap needs, "Chunked prefill (stall-free batching), explained", "Simulated numbers: choosing
 * the budget"). batch->attention picks one, or lets the library choose from the batch (fused for
 * a long prefill with many work items, or very large decode work; hl_attention_plan reports it).
 * A prompt tile whose key range is long while the batch has few prefill work items is split into
 * key-range parts merged by a second pass. Rows are bit-identical whichever launch form runs, and
 * to those of the two separate entry points. hybrid_layer_step uses the same path. */
int hl_attention(const hl_batch_desc* batch, const hl_bf16* q_rot, const hl_kv_pages* kv,
                 const hl_block_table* block_table, hl_bf16* attn_out);
int hl_prefill_attention(const hl_batch_desc* batch, const hl_bf16* q_rot,
                         const hl_kv_pages* kv, const hl_block_table* block_table,
                         hl_bf16* attn_out);
int hl_decode_attention(const hl_batch_desc* batch, const hl_bf16* q_rot,
                        const hl_kv_pages* kv, const hl_block_table* block_table,
                        hl_bf16* attn_out);

/* The attention phase in two calls, as the layer step itself runs it: the work lists are built
 * first (the step builds them in its first normalisation pass), then the kernels run on them.
 * hl_attention_build_lists writes the batch's work lists (decode units, prefill tiles or
 * key-range parts, merges) and zeroes the fused launch's work-queue counters in the batch
 * workspace (one small kernel on batch->stream). hl_attention_run then runs attention on those
 * lists: paths 1 = prompt-chunk rows only, 2 = decode rows only, 3 = both (fused in one launch or
 * as two launches, as hl_attention chooses for the batch). q_lo (device [T, Hq d], optional) is
 * the low half of a two-part query, bf16(q - bf16(q)) with q_rot = bf16(q): decode rows then score
 * with q_rot + q_lo, as the layer step does; prompt-chunk rows ignore it; NULL means a one-part
 * query. The batch (its descriptor values and its workspace) must be the one the lists were
 * built for; a fused launch consumes the work-queue counters, so every run of paths 3 whose batch
 * fuses needs a build of its own before it (the separate kernels only read the lists). Rows agree
 * with hl_attention bit for bit when q_lo is NULL. The split is what makes each launch timeable on
 * its own; the mathematics is that of hl_attention ("ConfluxServe" summary, "Why can linear
 * layers be batched but attention cannot?"). Errors: those of hl_attention, HL_ERR_ARG for paths
 * outside 1..3. */
int hl_attention_build_lists(const hl_batch_desc* batch, const hl_kv_pages* kv,
                             const hl_block_table* block_table);
int hl_attention_run(const hl_batch_desc* batch, const hl_bf16* q_rot, const hl_bf16* q_lo,
                     const hl_kv_pages* kv, const hl_block_table* block_table, hl_bf16* attn_out,
                     int32_t paths);

/* hl_attention_run that also records every work item it runs, for measuring how the two paths
 * share the GPU when they run in one launch (the overlap the ConfluxServe summary asks of them,
 * "Why can linear layers be batched but attention cannot?": decode keeping most of its standalone
 * bandwidth while prefill runs). trace (device, trace_entries uint64 values, 16-byte aligned)
 * receives three values per item: start and end time on the device's constant-rate clock
 * (hl_trace_clock_khz), and the workgroup that ran it. Items are numbered prefill items first
 * (entry * n_q_heads + query head, entries as hl_attention_plan's prefill_parts), then decode work
 * (unit * n_kv_heads + kv head, units as its decode_units, numbered in sequence order: each decode
 * sequence's pages in order, split_pages per unit, whatever order they ran in); a path that does
 * not run leaves its
 * records untouched. Results equal hl_attention_run's bit for bit. Errors: those of
 * hl_attention_run; HL_ERR_NULL for a NULL trace, HL_ERR_ALIGN, HL_ERR_ARG if trace_entries is
 * less than 3 * (prefill_parts * n_q_heads + decode_units * n_kv_heads). */
int hl_attention_run_traced(const hl_batch_desc* batch, const hl_bf16* q_rot, const hl_bf16* q_lo,
                            const hl_kv_pages* kv, const hl_block_table* block_table,
                            hl_bf16* attn_out, int32_t paths, uint64_t* trace,
                            size_t trace_entries);

/* Ticks per millisecond of the clock hl_attention_run_traced records (the current device's
 * constant-rate wall clock). Errors: HL_ERR_NULL, HL_ERR_HIP. */
int hl_trace_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* HYBRID_LAYER_H */
