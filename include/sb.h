/*
 * sb.h -- C ABI of the selective-batching library (libsb.so, MI355X / gfx950).
 *
 * One selective-batched Transformer iteration over a ragged batch, plus the
 * host-side K/V manager and iteration-level scheduler that feed it.
 *
 * Sources (web pages on Orca-style continuous batching):
 *   [W]  "连续批处理完全拆解：Orca 的迭代级调度与选择性批处理" -- Algorithm 1,
 *        sections 观察 (selective batching), Figure 5 (Split / Merge, K/V
 *        manager), 迭代级 FCFS, 两个约束 (max_bs, K/V slots).
 *   [L2] "CS349D Lecture 2 · 批处理与调度" -- sections 4.1-4.3, 5.1 (memory
 *        manager try_admit / free), exercise 4.
 *   [OB] "Orca: The beginning of Morden LLM serving" -- section Scheduling
 *        Algorithm (select_batch).
 *
 * Conventions for every entry point:
 *   - Return value: SB_OK (0) or a negative sb_status.  No exception crosses
 *     the ABI.  sb_last_error() returns a thread-local message for the last
 *     failure on the calling thread.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are GPU
 *     memory owned by the caller (the library never allocates device memory
 *     and never frees caller memory).  Opaque handles (sb_kv, sb_sched) are
 *     owned by the library and released with their destroy call.
 *   - Device work is enqueued asynchronously on the HIP stream passed as
 *     `stream` (a hipStream_t; NULL = the default stream); the call returns
 *     after the launches.  A launch failure returns SB_ERR_DEVICE.
 *   - Matrices are row-major.  Weights are [out_features, in_features]
 *     (K-contiguous).  Activations are [tokens, features].
 */
#ifndef SB_H
#define SB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
typedef enum {
    SB_OK = 0,
    SB_ERR_INVALID = -1,    /* bad argument (null handle, non-positive size, unsupported shape) */
    SB_ERR_NO_SLOTS = -2,   /* reservation would exceed n_slots                                  */
    SB_ERR_NOT_FOUND = -3,  /* unknown request id, or already freed                              */
    SB_ERR_TOO_LARGE = -4,  /* max_tokens > n_slots: the request could never be admitted         */
    SB_ERR_DEVICE = -5,     /* HIP launch / runtime error                                        */
    SB_ERR_WORKSPACE = -6,  /* caller-provided buffer too small                                  */
    SB_ERR_STATE = -7,      /* call not valid in the request's current state                     */
    SB_ERR_CAPACITY = -8    /* output array capacity too small                                   */
} sb_status;

const char* sb_last_error(void);

/* ------------------------------------------------------------------ types  */
enum { SB_F32 = 0, SB_BF16 = 1 };          /* storage dtype of weights, K/V and GEMM operands */
enum { SB_ARCH_GPT = 0, SB_ARCH_LLAMA = 1 };

/* Model shape.  GPT-style: LayerNorm (gain, shift), biases, exact-erf GeLU,
 * learned absolute positions.  Llama-style: RMSNorm (gain), no biases,
 * SwiGLU, rotary embedding (rotate-half, base rope_theta) on q and k.
 * Query head h reads K/V head h / (n_heads / n_kv_heads). */
typedef struct {
    int32_t arch, dtype;
    int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, max_pos;
    float eps, rope_theta;
} sb_model_dims;

/* One layer's weights (device, model dtype).  Shapes:
 *   ln1_g, ln1_b, ln2_g, ln2_b : [hidden]            (ln*_b NULL for Llama)
 *   w_qkv : [(n_heads + 2 n_kv_heads) head_dim, hidden] -- Q rows, K rows, V rows
 *   b_qkv : [(n_heads + 2 n_kv_heads) head_dim]       (NULL for Llama)
 *   w_o   : [hidden, n_heads head_dim]; b_o : [hidden] (NULL for Llama)
 *   w1    : [ffn, hidden] (GPT) or [2 ffn, hidden] gate rows then up rows (Llama)
 *   b1    : [ffn] (NULL for Llama); w2 : [hidden, ffn]; b2 : [hidden] (NULL for Llama) */
typedef struct {
    const void *ln1_g, *ln1_b, *w_qkv, *b_qkv, *w_o, *b_o, *ln2_g, *ln2_b, *w1, *b1, *w2, *b2;
} sb_layer_weights;

/* Embedding / head weights (device, model dtype):
 *   tok_emb [vocab, hidden]; pos_emb [max_pos, hidden] (GPT, else NULL);
 *   lnf_g, lnf_b [hidden] (lnf_b NULL for Llama); w_lm [vocab, hidden] (not tied). */
typedef struct {
    const void *tok_emb, *pos_emb, *lnf_g, *lnf_b, *w_lm;
} sb_model_weights;

/* ------------------------------------------------------------------ K/V manager
 * The Attention K/V manager of [W] Figure 5: keeps each request's keys and
 * values until the scheduler frees the request.  Admission follows the
 * reservation rule of [W] 两个约束 / Algorithm 1 and [L2] 4.3: a request
 * reserves max_tokens slots (one slot = one token's K and V in every layer)
 * when first scheduled; the reservation fails iff n_rsrv + max_tokens > n_slots.
 * Each reservation is one contiguous slot range starting at a multiple of 8;
 * when no hole fits, live ranges are compacted (device copies on the stream
 * given to sb_kv_set_stream).  The counter alone decides admission.
 *
 * Arena layouts (caller-allocated device memory, dtype of the model):
 *   K: [n_layers][n_kv_heads][arena_slots][head_dim]
 *   V: [n_layers][n_kv_heads][arena_slots / 8][head_dim][8]  (8-slot blocks,
 *      dim-major inside a block, so 8 consecutive slots of one dim are 16
 *      contiguous bytes in bf16)                                              */
typedef struct sb_kv sb_kv;

/* Physical slots the arenas need for n_slots reservable slots and at most
 * max_live simultaneously live requests (8-slot alignment of every range). */
int64_t sb_kv_arena_slots(int64_t n_slots, int32_t max_live);
/* Bytes of EACH of the K and V arenas. */
size_t sb_kv_arena_bytes(int64_t arena_slots, int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                         int32_t dtype);
/* k_arena / v_arena may both be NULL: bookkeeping only (no device copies). */
int sb_kv_create(int64_t n_slots, int64_t arena_slots, int32_t n_layers, int32_t n_kv_heads,
                 int32_t head_dim, int32_t dtype, void* k_arena, void* v_arena, sb_kv** out);
int sb_kv_set_stream(sb_kv* kv, void* stream);
/* Reserve max_tokens slots for req_id; *slot_base receives the first slot.
 * SB_ERR_NO_SLOTS if the counter would exceed n_slots (nothing changes),
 * SB_ERR_STATE if req_id already holds a reservation. */
int sb_kv_reserve(sb_kv* kv, int64_t req_id, int32_t max_tokens, int64_t* slot_base);
/* Release req_id's reservation.  SB_ERR_NOT_FOUND if it holds none. */
int sb_kv_free(sb_kv* kv, int64_t req_id);
int sb_kv_lookup(const sb_kv* kv, int64_t req_id, int64_t* slot_base, int32_t* max_tokens);
int sb_kv_stats(const sb_kv* kv, int64_t* n_rsrv, int64_t* n_slots, int64_t* n_live, int64_t* n_compactions);
/* Device pointers of layer `layer`'s K and V planes (for the kernels). */
int sb_kv_layer_ptrs(const sb_kv* kv, int32_t layer, void** k, void** v);
/* Scatter n rows of K and V ([n][n_kv_heads][head_dim], device, model dtype)
 * of layer `layer` to the slots slots[0..n) (device int32).  A slot outside
 * [0, arena_slots) is skipped (its row is neither written nor read). */
int sb_kv_write(const sb_kv* kv, int32_t layer, int32_t n, const int32_t* slots, const void* k,
                const void* v, void* stream);
/* Gather the rows of slots[0..n) back into [n][n_kv_heads][head_dim] (device). */
int sb_kv_read(const sb_kv* kv, int32_t layer, int32_t n, const int32_t* slots, void* k, void* v,
               void* stream);
void sb_kv_destroy(sb_kv* kv);

/* ------------------------------------------------------------------ scheduler
 * Iteration-level FCFS of [W] Algorithm 1 (Select) with one worker, as in
 * [L2] 4.3 and [OB] select_batch.  Requests enter INITIATION; Select scans
 * the pool in arrival order (ties: submission order), stops at max_bs, and
 * stops (never skips) at the first INITIATION request whose reservation
 * fails.  After the iteration every batch member becomes INCREMENT; a member
 * that has generated out_len tokens is finished and its slots are freed.   */
typedef struct sb_sched sb_sched;

int sb_sched_create(int32_t max_bs, sb_kv* kv, sb_sched** out);       /* SB_ERR_INVALID if max_bs <= 0 */
/* Submit a request.  prompt_tokens: host [prompt_len] (may be NULL: zeros).
 * SB_ERR_TOO_LARGE if max_tokens > n_slots; SB_ERR_INVALID if
 * prompt_len + out_len - 1 > max_tokens or a length is < 1; SB_ERR_STATE on a duplicate id. */
int sb_sched_add(sb_sched* s, int64_t req_id, double arrival, int32_t prompt_len,
                 const int32_t* prompt_tokens, int32_t out_len, int32_t max_tokens);
/* Submit a request that already generated `generated` (>= 1) tokens, the last
 * being last_token, whose K/V history (prompt_len + generated - 1 slots) the
 * caller fills.  It reserves its slots now (SB_ERR_NO_SLOTS if they do not fit). */
int sb_sched_add_running(sb_sched* s, int64_t req_id, double arrival, int32_t prompt_len,
                         const int32_t* prompt_tokens, int32_t out_len, int32_t max_tokens,
                         int32_t generated, int32_t last_token);
/* Chunked prefill ("从静态批处理到连续批处理", section Chunked Prefill; "CS349D
 * Lecture 2", exercise 9): from the next Select on, an iteration feeds at most
 * token_budget tokens.  Decoding requests go first (one token each, arrival
 * order); then requests still in their prompt, in arrival order, each feed
 * min(chunk, prompt tokens left, budget left) prompt tokens -- the first time
 * a request is scheduled it reserves max_tokens as in Algorithm 1 and a
 * failed reservation stops the scan.  Only the chunk that ends a prompt yields
 * a token: sb_sched_complete ignores the other members' new_tokens entries.
 * Both 0 (the default) turns it off: whole prompts, Algorithm 1 exactly.
 * SB_ERR_INVALID unless both are positive or both 0. */
int sb_sched_set_chunking(sb_sched* s, int32_t token_budget, int32_t chunk);
/* Request-level (static) batching, the baseline iteration-level scheduling is
 * compared against ("CS349D Lecture 2", section 4.1, static grid): with on != 0,
 * Select forms a new batch (as Algorithm 1: arrival order, max_bs, reservation)
 * only once the previous batch has entirely finished, and until then returns
 * that batch's unfinished members; nobody joins mid-batch.  Finished members
 * leave the computed batch (no padding work on ragged kernels) but their seats
 * are not refilled.  SB_ERR_INVALID while chunking is on. */
int sb_sched_set_request_level(sb_sched* s, int32_t on);
/* Select the next batch (host arrays of capacity cap).  For member i:
 * n_new[i] = tokens fed this iteration (the prompt or a chunk of it, or 1),
 * ctx[i] = tokens already cached, slot_base[i] = first slot of its reservation
 * as the K/V manager holds it once the whole batch is admitted (a reservation
 * made during this Select may compact the arena and move members admitted
 * before it: their histories are copied on the manager's stream, and only
 * these bases are valid for this iteration and after).
 * *n_out == 0 is legal (empty pool). */
int sb_select_batch(sb_sched* s, int32_t cap, int64_t* ids, int32_t* n_new, int32_t* ctx,
                    int64_t* slot_base, int32_t* n_out);
/* Token ids fed this iteration by the n selected requests, flattened in batch
 * order: the prompt (or this iteration's chunk of it), else the last generated token. */
int sb_batch_tokens(const sb_sched* s, int32_t n, const int64_t* ids, int32_t cap, int32_t* tokens,
                    int32_t* n_tokens);
/* The iteration returned one token per member (new_tokens, host).  Finished
 * requests are freed and their ids written to finished_ids (capacity n). */
int sb_sched_complete(sb_sched* s, int32_t n, const int64_t* ids, const int32_t* new_tokens,
                      int32_t* n_finished, int64_t* finished_ids);

/* Deferred completion, so the next iteration can be selected and launched
 * while this one still runs on the GPU.  Completion depends only on counts
 * (a request finishes when it has generated out_len tokens, [W] Algorithm 1
 * lines on Complete), never on token values: this call does everything
 * sb_sched_complete does -- advances every member, finishes and frees the
 * ones that are done -- but leaves each member's new token value pending
 * under *ticket.  Until sb_sched_set_tokens(ticket) supplies the values,
 * sb_batch_tokens refuses (SB_ERR_STATE) a batch that needs one of them and
 * sb_batch_token_refs refers to them instead. */
int sb_sched_complete_deferred(sb_sched* s, int32_t n, const int64_t* ids, int32_t* n_finished,
                               int64_t* finished_ids, int64_t* ticket);
/* Values of a deferred completion's tokens (host [n], batch order of that
 * iteration, n = its batch size).  SB_ERR_NOT_FOUND for an unknown or already
 * settled ticket, SB_ERR_INVALID if n differs. */
int sb_sched_set_tokens(sb_sched* s, int64_t ticket, int32_t n, const int32_t* tokens);
/* As sb_batch_tokens, but a member whose last token is still pending gets the
 * reference -(1 + j) instead of a token id, j being its row in the batch of the
 * iteration that generated it (its row of that iteration's device id buffer,
 * resolved by sb_embed_chained).  *ref_ticket receives that iteration's
 * ticket, or -1 if no reference was needed; SB_ERR_STATE if the pending
 * tokens come from more than one iteration. */
int sb_batch_token_refs(const sb_sched* s, int32_t n, const int64_t* ids, int32_t cap, int32_t* tokens,
                        int32_t* n_tokens, int64_t* ref_ticket);
/* Generated tokens of a live or finished request (host, capacity cap). */
int sb_sched_output(const sb_sched* s, int64_t req_id, int32_t cap, int32_t* tokens, int32_t* n);
int sb_sched_stats(const sb_sched* s, int32_t* pool_size, int64_t* n_rsrv, int64_t* n_finished);

/* Reservation policies ("CS349D Lecture 2", section 6.1, KV 预留): how many
 * slots (max_tokens) a request reserves when first scheduled.  MAX: prompt +
 * the longest output allowed (max_out), all a real system can know; POW2: the
 * prompt + the output length rounded up to a power of two (a length
 * prediction over-reserving at most 2x); ORACLE: prompt + out_len - 1, exactly
 * the tokens that ever get K/V.  SB_ERR_INVALID unless
 * 1 <= out_len <= max_out <= 2^30 and prompt_len >= 1. */
enum { SB_RESERVE_MAX = 0, SB_RESERVE_POW2 = 1, SB_RESERVE_ORACLE = 2 };
int sb_reservation_tokens(int32_t policy, int32_t prompt_len, int32_t out_len, int32_t max_out, int32_t* max_tokens);
/* K/V slots reserved (n_rsrv) and slots holding K/V (section 6.1's 'reserved'
 * vs 'actually stored'): every token written so far by a pool request, the
 * current iteration's tokens included for the members of a selected batch
 * (call it between sb_select_batch and the Complete). */
int sb_kv_usage(const sb_sched* s, int64_t* reserved, int64_t* stored);
void sb_sched_destroy(sb_sched* s);

/* ------------------------------------------------------------------ ragged batch
 * Split / Merge as offsets ([W] Figure 5, [L2] 4.2): request i owns rows
 * cu_seqlens[i] .. cu_seqlens[i+1]-1 of every [T, *] activation; its j-th
 * new token has position ctx_i + j and K/V slot slot_base_i + ctx_i + j.
 * sb_ragged_build lays this metadata plus the attention work list out in
 * host_staging, copies it to dev_meta (one async H2D on `stream`) and fills
 * *out with device pointers into dev_meta.  host_staging must stay untouched
 * until the copy is done (pinned memory recommended).                        */
typedef struct {
    int32_t n_req, n_tokens;       /* B and T = sum of n_new                         */
    int32_t n_items, n_partials;   /* attention work items; unit partial tiles       */
    int32_t n_groups, max_new;     /* unit-combine groups; max n_new in the batch    */
    const int32_t* cu_seqlens;     /* device [B+1]                                   */
    const int32_t* ctx_lens;       /* device [B]                                     */
    const int32_t* last_row;       /* device [B]  cu_seqlens[i+1]-1                  */
    const int32_t* tok_pos;        /* device [T]  position of each row               */
    const int32_t* tok_slot;       /* device [T]  K/V slot of each row               */
    const int32_t* tok_ids;        /* device [T]  token id of each row (or NULL)     */
    const int32_t* items;          /* device [n_items][12] attention work list (items
                                      with n_rows 0 are empty: dispatch-order padding)  */
    const int32_t* groups;         /* device [n_groups][8] unit-combine list         */
} sb_ragged;

size_t sb_ragged_bytes(const sb_model_dims* dims, int32_t max_req, int32_t max_tokens, int64_t max_keys_total);
/* Upper bound of sb_ragged.n_partials over batches of at most max_req requests
 * holding at most max_keys_total keys (cached + new) in total: sizes the
 * attention part of the workspace (sb_layer_workspace_bytes' max_partials). */
int64_t sb_attn_max_partials(const sb_model_dims* dims, int32_t max_req, int64_t max_keys_total);
/* n_new, ctx: host [n_req]; slot_base: host [n_req]; token_ids: host [sum n_new] or NULL.
 * A token id is in [0, vocab) or a reference -(1 + j), j < 2^20, to row j of the
 * previous iteration's device ids (sb_batch_token_refs); SB_ERR_INVALID otherwise. */
int sb_ragged_build(const sb_model_dims* dims, int32_t n_req, const int32_t* n_new, const int32_t* ctx,
                    const int64_t* slot_base, const int32_t* token_ids, void* host_staging,
                    void* dev_meta, size_t bytes, void* stream, sb_ragged* out);

/* ------------------------------------------------------------------ device steps
 * Residual stream x is fp32 [T, hidden] (device) for both dtypes; GEMM
 * operands, K/V and weights are in the model dtype.                          */

/* Workspace bytes of sb_layer_step / sb_lm_argmax for up to max_tokens rows,
 * max_req requests and max_partials split-attention partial tiles. */
size_t sb_layer_workspace_bytes(const sb_model_dims* dims, int32_t max_tokens, int32_t max_req,
                                int32_t max_partials);

/* Token embedding (+ learned position for GPT) of every row: x[t] = E[id_t] (+ P[pos_t]).
 * The rows are the flattened [sum L_i, H] input of [W] Figure 5 (request i's
 * new tokens at rows cu_seqlens[i] ..); each is the token the request feeds
 * this iteration: prompt tokens in the initiation phase, else the token the
 * previous iteration generated ([W] 为什么这对生成式模型是灾难: an iteration's
 * input is the previous iteration's output; Figure 3).  The pages do not fix
 * the position scheme: GPT-style models use learned absolute positions
 * ctx_i + j, Llama-style models none here (RoPE is applied inside the layer).
 * rg->tok_ids must be set; ids outside [0, vocab) are refused by
 * sb_ragged_build.  x: device fp32 [T, hidden], written entirely. */
int sb_embed(const sb_model_dims* dims, const sb_model_weights* w, const sb_ragged* rg, float* x,
             void* stream);
/* sb_embed for chained iterations ([W] 控制面与数据面分离: keep the host's
 * control path free of per-iteration GPU waits -- here the host schedules
 * the next iteration without waiting for the device's tokens; "CS349D
 * Lecture 2" section 7, CPU-side scheduling as the bottleneck):
 * resolves token references -(1 + j) to prev_ids[j] (device int32
 * [prev_n]: the previous iteration's sb_lm_argmax output, read in stream order,
 * so it is never copied through the host).  A reference with j >= prev_n, or
 * any id outside [0, vocab), embeds a clamped id: it cannot read outside the
 * tables; the host-side checks of sb_ragged_build keep literal ids in range. */
int sb_embed_chained(const sb_model_dims* dims, const sb_model_weights* w, const sb_ragged* rg,
                     const int32_t* prev_ids, int32_t prev_n, float* x, void* stream);

/* One decoder layer over the ragged batch ([W] Figure 5 data flow), in place on x:
 *   h = norm1(x); qkv = h W_qkv^T (+b); [RoPE q,k]; append k,v to the K/V
 *   manager at tok_slot; o = per-request causal attention over each request's
 *   slots [slot_base, slot_base + ctx + n_new); x += o W_o^T (+b);
 *   h = norm2(x); x += FFN(h)  (GeLU or SwiGLU)                              */
int sb_layer_step(const sb_model_dims* dims, const sb_layer_weights* w, const sb_ragged* rg,
                  const sb_kv* kv, int32_t layer, float* x, void* workspace, size_t ws_bytes,
                  void* stream);

/* Final norm of each request's last row, LM head, greedy argmax (lowest index
 * on ties).  Each iteration yields one token per request from the last of its
 * rows ([W] Figure 3: every iteration of an autoregressive model emits one
 * token, the initiation iteration its first one; "CS349D Lecture 2" 4.2:
 * greedy decoding, batched ids equal one-by-one ids).  Row r = last_row[r]
 * of x (device fp32 [T, hidden]); logits: device fp32 [B, vocab] (may be
 * NULL: then held in the workspace); out_ids: device int32 [B], request order.
 * SB_ERR_WORKSPACE if ws_bytes < sb_layer_workspace_bytes for this batch. */
int sb_lm_argmax(const sb_model_dims* dims, const sb_model_weights* w, const sb_ragged* rg,
                 const float* x, float* logits, int32_t* out_ids, void* workspace, size_t ws_bytes,
                 void* stream);

/* One iteration's whole device side in one call -- the engine's "run one
 * iteration for the batch" of [W] Algorithm 1 (the scheduler hands the engine
 * a batch, the engine runs exactly one iteration and returns one token per
 * request) over the Figure-5 data flow of every layer.  One host call instead
 * of 2 + n_layers: sb_embed_chained (prev_ids may be NULL), sb_layer_step for
 * layers 0 .. n_layers-1 with layers[l] (host array of n_layers structs),
 * then sb_lm_argmax.  Arguments, ownership and errors as for those calls; the
 * first failing step's status is returned and nothing after it is enqueued.
 * It only enqueues kernels on `stream` (no allocation, copy, memset or host
 * wait), and which kernels it launches depends only on the host fields of
 * `rg`, on `n_layers` and on the pointers passed: a caller may capture it in a
 * HIP graph and replay that graph for later iterations with the same fields
 * and buffers, whatever the buffers then hold.  Kernel timing (sb_timing_enable)
 * records events around launches: keep it off while capturing. */
int sb_forward(const sb_model_dims* dims, const sb_model_weights* w, const sb_layer_weights* layers, int32_t n_layers,
               const sb_ragged* rg, const sb_kv* kv, const int32_t* prev_ids, int32_t prev_n, float* x,
               float* logits, int32_t* out_ids, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ timing
 * Per-kernel-class HIP event timing of launches made by the library (for
 * benchmarks): an event pair is recorded on the launch stream around every
 * launch of an enabled class, which itself costs time, so enable only the
 * classes to be measured.                                                    */
enum { SB_K_GEMM_QKV = 0, SB_K_GEMM_O, SB_K_GEMM_FFN1, SB_K_GEMM_FFN2, SB_K_GEMM_LM, SB_K_ATTN,
       SB_K_ATTN_COMBINE, SB_K_NORM, SB_K_ROPE_APPEND, SB_K_EMBED, SB_K_ARGMAX, SB_K_COUNT };
#define SB_TIMING_ALL (-1)
/* mask: bit k enables class k (SB_TIMING_ALL: every class, 0: off). */
int sb_timing_enable(int32_t mask);
/* Sum of elapsed ms and number of launches of class k since the last reset;
 * synchronizes on the recorded events. */
int sb_timing_read(int32_t k, double* total_ms, int64_t* count);
int sb_timing_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* SB_H */
