// Internal launch API of libmt's HIP kernels (host side).  Every launcher
// enqueues on the given stream and returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace mt {

// ---------------------------------------------------------------- GEMM
// C[M, N] = op(A) * op(B) with fp32 accumulation.  Operands are stored as
// E: bf16 bit patterns (uint16_t; bf16 MFMA kernels) or fp32 (float; the
// fp32 debug precision, plain fp32 FMA).  "Storage" below means E.
//  NT: A [M, K] (row stride lda), B [N, K] (ldb)      C = A B^T
//  NN: A [M, K],                  B [K, N]            C = A B
//  TN: A [K, M],                  B [K, N]            C = A^T B
enum GemmLayout { GEMM_NT = 0, GEMM_NN = 1, GEMM_TN = 2 };

enum GemmEpi {
  EPI_BF16 = 0,        // C (storage) = acc
  EPI_F32 = 1,         // C (fp32) = acc
  EPI_ACC_F32 = 2,     // C (fp32) += acc
  EPI_RESID_BF16 = 3,  // C (storage) = R (storage) + acc
  EPI_SWIGLU = 4,      // NT only; B = [W_gate; W_up] (2F rows); N = 2F:
                       //   C (storage) [M, F] = silu(gate) * up
  EPI_SWIGLU_SAVE = 5, // as EPI_SWIGLU, and C2 (storage) [M, 2F] = [gate | up]
  EPI_SWIGLU_BWD = 6   // acc = dm [M, F]; G = [gate | up] (storage, ldg);
                       //   C2 (storage) [M, 2F] = [dgate | dup]
};

template <class E>
struct GemmArgsT {
  int layout = GEMM_NT, epi = EPI_BF16;
  int M = 0, N = 0, K = 0;
  const E* A = nullptr; long lda = 0;
  const E* B = nullptr; long ldb = 0;
  void* C = nullptr; long ldc = 0;
  const E* R = nullptr; long ldr = 0;
  E* C2 = nullptr; long ldc2 = 0;
  const E* G = nullptr; long ldg = 0;
  int F = 0;  // FFN width for the SwiGLU epilogues
  int vec = 0;  // set by the launcher: strides and alignment allow 16-byte epilogue accesses
  // fp32 workspace for splitting the tiles of a partly filled last round
  // along K (null: no split; the 256 x 256 tile needs up to 64 MiB)
  float* ws = nullptr;
  long ws_elems = 0;
  int split_full = 0, split_s = 1;  // set by the launcher
};
using GemmArgs = GemmArgsT<uint16_t>;
using GemmArgsF32 = GemmArgsT<float>;

// Returns a message for unsupported arguments, or nullptr if OK.
const char* gemm_check(const GemmArgs& a);
hipError_t gemm_launch(const GemmArgs& a, hipStream_t s);
// Name of the kernel instantiation a launch with these arguments runs (as
// profilers report it, without namespace and parameter list).
std::string gemm_kernel_name(const GemmArgs& a);
const char* gemm_check(const GemmArgsF32& a);
hipError_t gemm_launch(const GemmArgsF32& a, hipStream_t s);

// ------------------------------------------------------------ elementwise
// Each storage-typed launcher below has a bf16 (uint16_t) and an fp32
// (float) overload running the same kernel template; math is fp32.
//
// RMSNorm over rows of x [rows, cols]: y = x * rstd * g, rstd [rows] fp32
// (may be null).
hipError_t rmsnorm_fwd(const uint16_t* x, const uint16_t* g, uint16_t* y, float* rstd,
                       int rows, int cols, float eps, hipStream_t s);
hipError_t rmsnorm_fwd(const float* x, const float* g, float* y, float* rstd, int rows,
                       int cols, float eps, hipStream_t s);
// dx = resid + rstd*(e - xh*mean(e*xh)), e = dy*g, xh = x*rstd (resid may
// be null).  Writes per-block partial gain gradients dg_part [nblk, cols]
// fp32; nblk = rmsnorm_bwd_blocks(rows).
int rmsnorm_bwd_blocks(int rows);
// Widest row the RMSNorm backward takes (the hidden size limit).
constexpr int RMSNORM_MAX_COLS = 16384;
hipError_t rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* g,
                       const float* rstd, const uint16_t* resid, uint16_t* dx,
                       float* dg_part, int rows, int cols, hipStream_t s);
hipError_t rmsnorm_bwd(const float* dy, const float* x, const float* g, const float* rstd,
                       const float* resid, float* dx, float* dg_part, int rows, int cols,
                       hipStream_t s);
// out[c] = sum_b part[b, c] in fixed block order, stored as the out type.
hipError_t reduce_rows(const float* part, int nblk, int cols, uint16_t* out, hipStream_t s);
hipError_t reduce_rows(const float* part, int nblk, int cols, float* out, hipStream_t s);

// cos/sin tables [seq, head_dim/2] fp32, angle = t * theta^(-2j/d) in fp64.
hipError_t rope_table(float* cos_t, float* sin_t, int seq, int head_dim, double theta,
                      hipStream_t s);
// Rotate the q and k column blocks of qkv [B*T, ldq] in place (inverse=1
// rotates by the negative angle: the backward).
hipError_t rope_apply(uint16_t* qkv, long ldq, int batch, int seq, int n_heads,
                      int n_kv_heads, int head_dim, const float* cos_t, const float* sin_t,
                      int inverse, hipStream_t s);
hipError_t rope_apply(float* qkv, long ldq, int batch, int seq, int n_heads, int n_kv_heads,
                      int head_dim, const float* cos_t, const float* sin_t, int inverse,
                      hipStream_t s);

// out[i] = in[i] stored as the out type (bf16: RNE).
// Finiteness of a gradient buffer: NONFINITE_BLOCKS workgroups each scan a
// strided share of `bytes` bytes of bf16 (f32 = 0) or fp32 values and write
// flags[block] = 1 if any is Inf or NaN, else 0 (bytes % 16 == 0).
constexpr int NONFINITE_BLOCKS = 2048;
// With ssq, each workgroup also writes the sum of squares of its share
// (fp32, a fixed order within the workgroup): the gradient norm's pieces.
hipError_t nonfinite_flags(const void* g, size_t bytes, int f32, int32_t* flags, hipStream_t s,
                           float* ssq = nullptr);
hipError_t cast_f32(const float* in, uint16_t* out, size_t n, hipStream_t s);
hipError_t cast_f32(const float* in, float* out, size_t n, hipStream_t s);
hipError_t fill_f32(float* p, float v, size_t n, hipStream_t s);
hipError_t copy_rows_bf16(const uint16_t* src, long lds, uint16_t* dst, long ldd, int rows,
                          int cols, hipStream_t s);

// ------------------------------------------------------------- attention
// Causal GQA attention over q/k/v held in qkv [B*T, (Hq+2Hkv)*d] (bf16).
// o [B*T, Hq*d] bf16; lse [B, Hq, T] fp32.
hipError_t attn_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int batch, int seq,
                    int n_heads, int n_kv_heads, int head_dim, hipStream_t s);
// Backward: delta [B, Hq, T] fp32 workspace; dqkv [B*T, (Hq+2Hkv)*d] bf16 out.
// Three kernels in order: delta = rowsum(dO * O), then dK/dV per key block,
// then dQ per query block; `stages` (a mask of ATTN_BWD_*) launches a
// subset, so a caller can time each kernel on its own (in that order).
enum { ATTN_BWD_DELTA = 1, ATTN_BWD_DKDV = 2, ATTN_BWD_DQ = 4, ATTN_BWD_ALL = 7 };
hipError_t attn_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse,
                    const uint16_t* dout, float* delta, uint16_t* dqkv, int batch, int seq,
                    int n_heads, int n_kv_heads, int head_dim, hipStream_t s,
                    int stages = ATTN_BWD_ALL);
// attn_bwd with its delta rows in a static device array of the library
// (ATTN_STATIC_SCRATCH_FLOATS floats per GPU) instead of a caller
// workspace; allocates nothing.  batch * n_heads * seq must not exceed
// that size (hipErrorInvalidValue).  Calls on one GPU share the array.
constexpr size_t ATTN_STATIC_SCRATCH_FLOATS = (size_t)16 << 20;
hipError_t attn_bwd_static(const uint16_t* qkv, const uint16_t* o, const float* lse,
                           const uint16_t* dout, uint16_t* dqkv, int batch, int seq, int n_heads,
                           int n_kv_heads, int head_dim, hipStream_t s);
// Name of the kernel behind attn_fwd (which 0) and the three backward
// stages (1 delta, 2 dK/dV, 3 dQ) for a head dimension, as profilers print it.
const char* attn_kernel_name(int head_dim, int which);
// fp32 storage (debug precision): same contract, one wave per query row
// (forward, dq) or key row (dk, dv) with fp32 FMA and exact exp/log.
hipError_t attn_fwd(const float* qkv, float* o, float* lse, int batch, int seq, int n_heads,
                    int n_kv_heads, int head_dim, hipStream_t s);
hipError_t attn_bwd(const float* qkv, const float* o, const float* lse, const float* dout,
                    float* delta, float* dqkv, int batch, int seq, int n_heads, int n_kv_heads,
                    int head_dim, hipStream_t s);

// ------------------------------------------------------------------ head
// Row-wise softmax cross-entropy on fp32 logits [rows, V] for next-token
// targets: target[r] < 0 means no target (zero gradient, no loss).
// dlogits (storage) = (softmax - onehot) * inv_n; loss_part[r] = lse - picked.
hipError_t ce_rows(const float* logits, const int32_t* target, uint16_t* dlogits,
                   float* loss_part, int rows, int vocab, float inv_n, hipStream_t s);
hipError_t ce_rows(const float* logits, const int32_t* target, float* dlogits, float* loss_part,
                   int rows, int vocab, float inv_n, hipStream_t s);
// loss = sum(loss_part[0..n)) * inv_n in fixed order -> out[0] (fp32).
hipError_t sum_loss(const float* part, int n, float inv_n, float* out, hipStream_t s);

}  // namespace mt
