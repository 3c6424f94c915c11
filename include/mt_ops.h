/*
 * mt_ops.h — per-operation entry points of libmt, the pieces the stateless
 * decoder-layer template (mt.h) is built from.  They exist so each kernel
 * can be checked on its own against the CPU oracle and timed on its own;
 * mt_layer_fwd / mt_layer_recompute_bwd / mt_stream_step call the same
 * kernels.  Conventions (status codes, ownership, layouts, validation before
 * enqueue, streams as void*) are those of mt.h.  All buffers are device
 * memory; bf16 is stored as uint16_t bit patterns.
 */
#ifndef MT_OPS_H
#define MT_OPS_H

#include <stddef.h>
#include <stdint.h>

#include "mt.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { MT_GEMM_NT = 0, MT_GEMM_NN = 1, MT_GEMM_TN = 2 };
enum {
  MT_EPI_BF16 = 0,       /* C bf16 = acc */
  MT_EPI_F32 = 1,        /* C fp32 = acc */
  MT_EPI_ACC_F32 = 2,    /* C fp32 += acc */
  MT_EPI_RESID_BF16 = 3, /* C bf16 = R + acc (residual branch) */
  MT_EPI_SWIGLU = 4,     /* NT, B = [W_gate; W_up] [2F, K], N = 2F: C [M, F] = silu(gate)*up */
  MT_EPI_SWIGLU_SAVE = 5,/* as SWIGLU and C2 [M, 2F] = [gate | up] */
  MT_EPI_SWIGLU_BWD = 6  /* acc = dm [M, F]; G = [gate | up]; C2 [M, 2F] = [dgate | dup] */
};

/* Dense product on bf16 MFMA with fp32 accumulation (the projections of
 * the decoder layer, MegaTrain listing page Table 2 shapes).
 *   NT: C[M,N] = A[M,K] B[N,K]^T;  NN: C = A[M,K] B[K,N];  TN: C = A[K,M]^T B[K,N].
 * Row strides lda/ldb/ldc/ldr/ldc2/ldg are in elements.  K and the
 * contiguous dimension of every operand must be multiples of 8; M and N
 * (the strided ones) may be anything.  A and B must be 16-byte aligned.
 * workspace (device, 16-byte aligned; may be null): when the 256 x 256
 * tiles leave a last round at most half full, its tiles are split along K
 * and their fp32 partial sums go here (up to MT_GEMM_SPLIT_BYTES); with a
 * smaller or no workspace the product runs unsplit.  Both are
 * deterministic; they differ only in fp32 summation order.  Calls sharing a
 * workspace must not overlap. */
#define MT_GEMM_SPLIT_BYTES ((size_t)64 << 20)
mt_status mt_op_gemm(int32_t layout, int32_t epilogue, int32_t M, int32_t N, int32_t K,
                     const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                     int64_t ldc, const void* R, int64_t ldr, void* C2, int64_t ldc2,
                     const void* G, int64_t ldg, int32_t F, void* workspace,
                     size_t workspace_bytes, void* stream);

/* The same product in the fp32 debug precision (MT_PREC_FP32_DEBUG of
 * mt.h): every operand, R, G and C2 is fp32, and so is C for MT_EPI_BF16
 * and MT_EPI_RESID_BF16 ("storage" outputs); plain fp32 FMA with fp32
 * accumulation.  No alignment or multiple-of-8 constraints. */
mt_status mt_op_gemm_f32(int32_t layout, int32_t epilogue, int32_t M, int32_t N, int32_t K,
                         const float* A, int64_t lda, const float* B, int64_t ldb, void* C,
                         int64_t ldc, const float* R, int64_t ldr, float* C2, int64_t ldc2,
                         const float* G, int64_t ldg, int32_t F, void* stream);

/* RMSNorm over rows: y = x / sqrt(mean(x^2)+eps) * g; rstd [rows] fp32
 * (nullable).  x, y bf16 [rows, cols]; g bf16 [cols]; cols % 8 == 0. */
mt_status mt_op_rmsnorm_fwd(const void* x, const void* g, void* y, float* rstd, int32_t rows,
                            int32_t cols, float eps, void* stream);

/* RMSNorm backward: dx = resid + rstd*(dy*g - xh*mean(dy*g*xh)), xh = x*rstd;
 * dg = sum over rows of dy*xh (bf16 [cols], fixed summation order).
 * resid nullable.  workspace: >= mt_op_rmsnorm_bwd_workspace(rows, cols) bytes. */
size_t mt_op_rmsnorm_bwd_workspace(int32_t rows, int32_t cols);
mt_status mt_op_rmsnorm_bwd(const void* dy, const void* x, const void* g, const float* rstd,
                            const void* resid, void* dx, void* dg, int32_t rows, int32_t cols,
                            void* workspace, size_t workspace_bytes, void* stream);

/* RoPE (rotate-half) applied in place to the q and k heads of
 * qkv [batch*seq, (Hq+2Hkv)*head_dim]; inverse = 1 rotates back (backward).
 * tables: device fp32 cos/sin [seq, head_dim/2] from mt_op_rope_table. */
mt_status mt_op_rope_table(float* cos_t, float* sin_t, int32_t seq, int32_t head_dim,
                           double theta, void* stream);
mt_status mt_op_rope(void* qkv, int32_t batch, int32_t seq, int32_t n_heads,
                     int32_t n_kv_heads, int32_t head_dim, const float* cos_t,
                     const float* sin_t, int32_t inverse, void* stream);

/* Causal GQA attention: q, k, v are column blocks of qkv (see above);
 * o bf16 [batch*seq, Hq*head_dim]; lse fp32 [batch, Hq, seq]. */
mt_status mt_op_attn_fwd(const void* qkv, void* o, float* lse, int32_t batch, int32_t seq,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, void* stream);

/* Attention backward: given o, lse and dout = dL/do, writes dq, dk, dv into
 * the matching column blocks of dqkv (bf16).  delta: fp32 workspace
 * [batch, Hq, seq]. */
mt_status mt_op_attn_bwd(const void* qkv, const void* o, const float* lse, const void* dout,
                         float* delta, void* dqkv, int32_t batch, int32_t seq, int32_t n_heads,
                         int32_t n_kv_heads, int32_t head_dim, void* stream);

/* mt_op_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results (the same kernels), with the delta rows
 * in a static device array of the library instead of a caller workspace.
 * It allocates nothing; the array (MT_ATTN_NOALLOC_MAX_ROWS floats, 64 MiB)
 * exists once per GPU the library runs on and is held until the process
 * ends; its address is looked up on the first call on each device.
 * batch * n_heads * seq above MT_ATTN_NOALLOC_MAX_ROWS returns MT_E_SHAPE
 * (7B heads: up to 524288 tokens).  Every call on one GPU uses that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be ordered by the caller.  Nothing needs clearing between calls
 * (each call writes every delta row it reads). */
#define MT_ATTN_NOALLOC_MAX_ROWS ((size_t)16 << 20)
mt_status mt_op_attn_bwd_noalloc(const void* qkv, const void* o, const float* lse,
                                 const void* dout, void* dqkv, int32_t batch, int32_t seq,
                                 int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                 void* stream);

/* Attention forward and backward in the fp32 debug precision: the same
 * contract with fp32 qkv, o, dout and dqkv (exact softmax per row, fp32
 * FMA; written for exactness, not speed). */
mt_status mt_op_attn_fwd_f32(const float* qkv, float* o, float* lse, int32_t batch, int32_t seq,
                             int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, void* stream);
mt_status mt_op_attn_bwd_f32(const float* qkv, const float* o, const float* lse,
                             const float* dout, float* delta, float* dqkv, int32_t batch,
                             int32_t seq, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                             void* stream);

/* Cross-entropy rows on fp32 logits [rows, vocab]: target[r] < 0 = no
 * target.  dlogits bf16 = (softmax - onehot) * inv_n; loss_part fp32 [rows]. */
mt_status mt_op_ce_rows(const float* logits, const int32_t* target, void* dlogits,
                        float* loss_part, int32_t rows, int32_t vocab, float inv_n,
                        void* stream);

/* Finiteness of a gradient buffer (the engine's per-unit check, run on the
 * GPU so the host never re-reads the gradient): flags[NONFINITE_BLOCKS =
 * 2048] int32 receive 1 where that workgroup's strided share of the buffer
 * holds an Inf or NaN, else 0.  g: device, bytes % 16 == 0, bf16 (f32 = 0)
 * or fp32 (f32 = 1) values. */
mt_status mt_op_nonfinite_flags(const void* g, size_t bytes, int32_t f32, int32_t* flags,
                                void* stream);

/* The stream schedule of mt_stream_step for n_layers, checkpoint interval,
 * prefetch depth, kept internals (mt_run_cfg.keep_internals) and resident
 * layers (mt_run_cfg.resident_layers), as plain integers so its hazards can
 * be checked without a GPU.  out receives, per compute op, (kind, layer,
 * load) with kind 0 forward, 1 head, 2 segment re-forward, 3
 * (recompute+)backward, 4 forward keeping internals (the last segment, with
 * keep_internals); then, per weight load, (unit, slot, first_use, last_use,
 * wait_use, gate_use): the load may start once compute ops wait_use and
 * gate_use have finished (-1: no wait); slot -2 is the head's own slot,
 * slot -3 - c resident slot c (layer 1 + c, or c when every layer is
 * resident; one load serving every op of that layer, skipped when the
 * previous step left the layer there).  counts = {n_ops, n_loads, n_slots}.
 * MT_E_SHAPE if the schedule would deadlock, MT_E_OOM_HOST if cap
 * (entries) is too small. */
mt_status mt_debug_plan(int32_t n_layers, int32_t ckpt_interval, int32_t prefetch_depth,
                        int32_t keep_internals, int32_t resident_layers, int32_t* out, size_t cap,
                        int32_t* counts);

#ifdef __cplusplus
}
#endif

#endif /* MT_OPS_H */
