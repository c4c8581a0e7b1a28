/*
 * sb_ops.h -- op-level entry points of libsb: the individual kernels that
 * sb_layer_step / sb_lm_argmax chain together, exported so each step of the
 * iteration can be checked on its own.  Same conventions as sb.h (status
 * codes, caller-owned device memory, asynchronous on `stream`).
 */
#ifndef SB_OPS_H
#define SB_OPS_H

#include "sb.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of the token-wise linear layer (selective batching runs Linear
 * on the flattened [T, K] rows: "连续批处理完全拆解", section 观察). */
enum { SB_EPI_STORE = 0,   /* C = A W^T (+ bias)                                   */
       SB_EPI_GELU = 1,    /* C = GeLU(A W^T + bias), exact erf form               */
       SB_EPI_RESID = 2,   /* x += A W^T (+ bias); C is the fp32 residual stream x */
       SB_EPI_SWIGLU = 3   /* C = SiLU(A Wg^T) * (A Wu^T); W = [Wg (F rows); Wu (F rows)] */
};

/* C[M, N] = epilogue(A[M, K] W[N, K]^T).  A, W, bias (may be NULL) in dtype;
 * C in dtype unless out_f32 (or SB_EPI_RESID: fp32).  For SB_EPI_SWIGLU N is
 * the output width F and W has 2F rows; pass F also in `F`.
 * bf16 needs K % 64 == 0, fp32 K % 16 == 0; strides in elements. */
int sb_op_gemm(int32_t dtype, int32_t epilogue, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
               const void* W, int64_t ldw, const void* bias, void* C, int64_t ldc, int32_t out_f32, int32_t F,
               void* stream);

/* LayerNorm (kind 0: (x - mean) / sqrt(var + eps) * g + b) or RMSNorm (kind 1:
 * x / sqrt(mean(x^2) + eps) * g) of fp32 rows x[row_map ? row_map[r] : r]
 * into out[r] (dtype).  b may be NULL.  hidden <= 12288, multiple of 4. */
int sb_op_norm(int32_t dtype, int32_t kind, int32_t rows, int32_t hidden, const float* x, const int32_t* row_map,
               const void* g, const void* b, float eps, void* out, void* stream);

/* RoPE of q in place inside qkv (Llama-style dims only) and append of k
 * (rotated likewise) and v to layer `layer` of the K/V manager at
 * rg->tok_slot; qkv's k and v parts are left as they are.  qkv must be
 * 16-byte aligned (SB_ERR_INVALID otherwise). */
int sb_op_rope_append(const sb_model_dims* dims, const sb_ragged* rg, const sb_kv* kv, int32_t layer, void* qkv,
                      void* stream);

/* Per-request causal attention of the whole ragged batch in one launch
 * (+ split combine): q read from qkv [T, (nq + 2 nkv) d], K/V from the
 * manager, output o [T, nq d].  workspace: >= n_partials * 16 * (d + 2) * 4 bytes. */
int sb_op_attention(const sb_model_dims* dims, const sb_ragged* rg, const sb_kv* kv, int32_t layer, const void* qkv,
                    void* o, void* workspace, size_t ws_bytes, void* stream);

/* sb_op_attention without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The split-attention unit partials go to
 * a static device array of SB_ATTN_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends (its address is taken
 * on the first call on each device).  The call allocates nothing and frees
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (two streams, or two threads) race and give undefined results.
 * Each partial a call reads is written earlier in the same call, so nothing
 * carries over from the previous call.  SB_ERR_WORKSPACE if the batch needs
 * more than the array holds (n_partials * 16 * (head_dim + 2) * 4 bytes);
 * other arguments and errors as sb_op_attention. */
#define SB_ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int sb_op_attention_noalloc(const sb_model_dims* dims, const sb_ragged* rg, const sb_kv* kv, int32_t layer,
                            const void* qkv, void* o, void* stream);

/* out[r] = index of the largest of logits[r, 0..V) (lowest index on ties). */
int sb_op_argmax(int32_t rows, int32_t V, const float* logits, int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SB_OPS_H */
