// C-ABI wrappers of the per-operation kernels (mt_ops.h) and the error
// plumbing every exported call shares.
#include <stdarg.h>
#include <stdio.h>

#include "kernels.h"
#include "mt_ops.h"
#include "status.h"

namespace mt {

static thread_local char g_last_error[1024] = "";

mt_status set_error(mt_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

}  // namespace mt

using namespace mt;

extern "C" {

const char* mt_last_error(void) { return g_last_error; }

mt_status mt_op_gemm(int32_t layout, int32_t epilogue, int32_t M, int32_t N, int32_t K,
                     const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                     int64_t ldc, const void* R, int64_t ldr, void* C2, int64_t ldc2,
                     const void* G, int64_t ldg, int32_t F, void* workspace,
                     size_t workspace_bytes, void* stream) {
  MT_CHECK(!workspace || ((uintptr_t)workspace & 15u) == 0, MT_E_INVALID,
           "mt_op_gemm: workspace must be 16-byte aligned");
  GemmArgs a;
  a.layout = layout; a.epi = epilogue; a.M = M; a.N = N; a.K = K;
  a.A = static_cast<const uint16_t*>(A); a.lda = lda;
  a.B = static_cast<const uint16_t*>(B); a.ldb = ldb;
  a.C = C; a.ldc = ldc;
  a.R = static_cast<const uint16_t*>(R); a.ldr = ldr;
  a.C2 = static_cast<uint16_t*>(C2); a.ldc2 = ldc2;
  a.G = static_cast<const uint16_t*>(G); a.ldg = ldg;
  a.F = F;
  a.ws = static_cast<float*>(workspace);
  a.ws_elems = workspace ? (long)(workspace_bytes / sizeof(float)) : 0;
  if (const char* msg = gemm_check(a)) return set_error(MT_E_SHAPE, "mt_op_gemm: %s", msg);
  MT_HIP(gemm_launch(a, static_cast<hipStream_t>(stream)));
  return MT_OK;
}

mt_status mt_op_gemm_f32(int32_t layout, int32_t epilogue, int32_t M, int32_t N, int32_t K,
                         const float* A, int64_t lda, const float* B, int64_t ldb, void* C,
                         int64_t ldc, const float* R, int64_t ldr, float* C2, int64_t ldc2,
                         const float* G, int64_t ldg, int32_t F, void* stream) {
  GemmArgsF32 a;
  a.layout = layout; a.epi = epilogue; a.M = M; a.N = N; a.K = K;
  a.A = A; a.lda = lda;
  a.B = B; a.ldb = ldb;
  a.C = C; a.ldc = ldc;
  a.R = R; a.ldr = ldr;
  a.C2 = C2; a.ldc2 = ldc2;
  a.G = G; a.ldg = ldg;
  a.F = F;
  if (const char* msg = gemm_check(a)) return set_error(MT_E_SHAPE, "mt_op_gemm_f32: %s", msg);
  MT_HIP(gemm_launch(a, static_cast<hipStream_t>(stream)));
  return MT_OK;
}

mt_status mt_op_rmsnorm_fwd(const void* x, const void* g, void* y, float* rstd, int32_t rows,
                            int32_t cols, float eps, void* stream) {
  MT_CHECK(x && g && y, MT_E_INVALID, "mt_op_rmsnorm_fwd: null pointer");
  MT_CHECK(rows >= 0 && cols > 0 && cols % 8 == 0, MT_E_SHAPE,
           "mt_op_rmsnorm_fwd: cols must be a positive multiple of 8");
  MT_HIP(rmsnorm_fwd(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(g),
                     static_cast<uint16_t*>(y), rstd, rows, cols, eps,
                     static_cast<hipStream_t>(stream)));
  return MT_OK;
}

size_t mt_op_rmsnorm_bwd_workspace(int32_t rows, int32_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)rmsnorm_bwd_blocks(rows) * (size_t)cols * sizeof(float);
}

mt_status mt_op_rmsnorm_bwd(const void* dy, const void* x, const void* g, const float* rstd,
                            const void* resid, void* dx, void* dg, int32_t rows, int32_t cols,
                            void* workspace, size_t workspace_bytes, void* stream) {
  MT_CHECK(dy && x && g && rstd && dx && dg, MT_E_INVALID, "mt_op_rmsnorm_bwd: null pointer");
  MT_CHECK(rows >= 0 && cols > 0 && cols % 8 == 0 && cols <= RMSNORM_MAX_COLS, MT_E_SHAPE,
           "mt_op_rmsnorm_bwd: cols must be a positive multiple of 8, at most %d",
           RMSNORM_MAX_COLS);
  MT_CHECK(workspace_bytes >= mt_op_rmsnorm_bwd_workspace(rows, cols) && (rows == 0 || workspace),
           MT_E_OOM_DEVICE, "mt_op_rmsnorm_bwd: workspace too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (rows == 0) return MT_OK;
  float* part = static_cast<float*>(workspace);
  MT_HIP(rmsnorm_bwd(static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(g), rstd, static_cast<const uint16_t*>(resid),
                     static_cast<uint16_t*>(dx), part, rows, cols, s));
  MT_HIP(reduce_rows(part, rmsnorm_bwd_blocks(rows), cols, static_cast<uint16_t*>(dg), s));
  return MT_OK;
}

mt_status mt_op_rope_table(float* cos_t, float* sin_t, int32_t seq, int32_t head_dim,
                           double theta, void* stream) {
  MT_CHECK(cos_t && sin_t, MT_E_INVALID, "mt_op_rope_table: null pointer");
  MT_CHECK(seq >= 0 && head_dim > 0 && head_dim % 2 == 0 && theta > 0, MT_E_SHAPE,
           "mt_op_rope_table: bad shape");
  MT_HIP(rope_table(cos_t, sin_t, seq, head_dim, theta, static_cast<hipStream_t>(stream)));
  return MT_OK;
}

mt_status mt_op_rope(void* qkv, int32_t batch, int32_t seq, int32_t n_heads, int32_t n_kv_heads,
                     int32_t head_dim, const float* cos_t, const float* sin_t, int32_t inverse,
                     void* stream) {
  MT_CHECK(qkv && cos_t && sin_t, MT_E_INVALID, "mt_op_rope: null pointer");
  MT_CHECK(batch >= 0 && seq >= 0 && n_heads > 0 && n_kv_heads > 0 && head_dim % 2 == 0,
           MT_E_SHAPE, "mt_op_rope: bad shape");
  const long ldq = (long)(n_heads + 2 * n_kv_heads) * head_dim;
  MT_HIP(rope_apply(static_cast<uint16_t*>(qkv), ldq, batch, seq, n_heads, n_kv_heads, head_dim,
                    cos_t, sin_t, inverse, static_cast<hipStream_t>(stream)));
  return MT_OK;
}

static const char* attn_shape_check(int32_t batch, int32_t seq, int32_t n_heads,
                                    int32_t n_kv_heads, int32_t head_dim) {
  if (batch < 0 || seq < 0) return "negative batch or seq";
  if (n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads) return "n_heads % n_kv_heads != 0";
  if (head_dim != 64 && head_dim != 128) return "head_dim must be 64 or 128";
  return nullptr;
}

mt_status mt_op_attn_fwd(const void* qkv, void* o, float* lse, int32_t batch, int32_t seq,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, void* stream) {
  MT_CHECK(qkv && o && lse, MT_E_INVALID, "mt_op_attn_fwd: null pointer");
  if (const char* m = attn_shape_check(batch, seq, n_heads, n_kv_heads, head_dim))
    return set_error(MT_E_SHAPE, "mt_op_attn_fwd: %s", m);
  MT_HIP(attn_fwd(static_cast<const uint16_t*>(qkv), static_cast<uint16_t*>(o), lse, batch, seq,
                  n_heads, n_kv_heads, head_dim, static_cast<hipStream_t>(stream)));
  return MT_OK;
}

mt_status mt_op_attn_bwd(const void* qkv, const void* o, const float* lse, const void* dout,
                         float* delta, void* dqkv, int32_t batch, int32_t seq, int32_t n_heads,
                         int32_t n_kv_heads, int32_t head_dim, void* stream) {
  MT_CHECK(qkv && o && lse && dout && delta && dqkv, MT_E_INVALID, "mt_op_attn_bwd: null pointer");
  if (const char* m = attn_shape_check(batch, seq, n_heads, n_kv_heads, head_dim))
    return set_error(MT_E_SHAPE, "mt_op_attn_bwd: %s", m);
  MT_HIP(attn_bwd(static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(o), lse,
                  static_cast<const uint16_t*>(dout), delta, static_cast<uint16_t*>(dqkv), batch,
                  seq, n_heads, n_kv_heads, head_dim, static_cast<hipStream_t>(stream)));
  return MT_OK;
}

static_assert(MT_ATTN_NOALLOC_MAX_ROWS == ATTN_STATIC_SCRATCH_FLOATS,
              "the header's limit is the static array's size");

mt_status mt_op_attn_bwd_noalloc(const void* qkv, const void* o, const float* lse,
                                 const void* dout, void* dqkv, int32_t batch, int32_t seq,
                                 int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                 void* stream) {
  MT_CHECK(qkv && o && lse && dout && dqkv, MT_E_INVALID, "mt_op_attn_bwd_noalloc: null pointer");
  if (const char* m = attn_shape_check(batch, seq, n_heads, n_kv_heads, head_dim))
    return set_error(MT_E_SHAPE, "mt_op_attn_bwd_noalloc: %s", m);
  const size_t need = (size_t)batch * n_heads * seq;
  MT_CHECK(need <= MT_ATTN_NOALLOC_MAX_ROWS, MT_E_SHAPE,
           "mt_op_attn_bwd_noalloc: batch * n_heads * seq = %zu exceeds the static scratch of "
           "%zu rows (use mt_op_attn_bwd with a workspace)",
           need, (size_t)MT_ATTN_NOALLOC_MAX_ROWS);
  MT_HIP(attn_bwd_static(static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(o), lse,
                         static_cast<const uint16_t*>(dout), static_cast<uint16_t*>(dqkv), batch,
                         seq, n_heads, n_kv_heads, head_dim, static_cast<hipStream_t>(stream)));
  return MT_OK;
}

mt_status mt_op_attn_fwd_f32(const float* qkv, float* o, float* lse, int32_t batch, int32_t seq,
                             int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, void* stream) {
  MT_CHECK(qkv && o && lse, MT_E_INVALID, "mt_op_attn_fwd_f32: null pointer");
  if (const char* m = attn_shape_check(batch, seq, n_heads, n_kv_heads, head_dim))
    return set_error(MT_E_SHAPE, "mt_op_attn_fwd_f32: %s", m);
  MT_HIP(attn_fwd(qkv, o, lse, batch, seq, n_heads, n_kv_heads, head_dim,
                  static_cast<hipStream_t>(stream)));
  return MT_OK;
}

mt_status mt_op_attn_bwd_f32(const float* qkv, const float* o, const float* lse,
                             const float* dout, float* delta, float* dqkv, int32_t batch,
                             int32_t seq, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                             void* stream) {
  MT_CHECK(qkv && o && lse && dout && delta && dqkv, MT_E_INVALID,
           "mt_op_attn_bwd_f32: null pointer");
  if (const char* m = attn_shape_check(batch, seq, n_heads, n_kv_heads, head_dim))
    return set_error(MT_E_SHAPE, "mt_op_attn_bwd_f32: %s", m);
  MT_HIP(attn_bwd(qkv, o, lse, dout, delta, dqkv, batch, seq, n_heads, n_kv_heads, head_dim,
                  static_cast<hipStream_t>(stream)));
  return MT_OK;
}

mt_status mt_op_ce_rows(const float* logits, const int32_t* target, void* dlogits,
                        float* loss_part, int32_t rows, int32_t vocab, float inv_n,
                        void* stream) {
  MT_CHECK(logits && target && dlogits && loss_part, MT_E_INVALID, "mt_op_ce_rows: null pointer");
  MT_CHECK(rows >= 0 && vocab > 0 && vocab % 4 == 0, MT_E_SHAPE,
           "mt_op_ce_rows: vocab must be a positive multiple of 4");
  MT_HIP(ce_rows(logits, target, static_cast<uint16_t*>(dlogits), loss_part, rows, vocab, inv_n,
                 static_cast<hipStream_t>(stream)));
  return MT_OK;
}

mt_status mt_op_nonfinite_flags(const void* g, size_t bytes, int32_t f32, int32_t* flags,
                                void* stream) {
  MT_CHECK(g && flags, MT_E_INVALID, "mt_op_nonfinite_flags: null pointer");
  MT_CHECK(bytes % 16 == 0 && (f32 == 0 || f32 == 1), MT_E_INVALID,
           "mt_op_nonfinite_flags: bytes must be a multiple of 16, f32 0 or 1");
  MT_HIP(nonfinite_flags(g, bytes, f32, flags, static_cast<hipStream_t>(stream)));
  return MT_OK;
}

}  // extern "C"
