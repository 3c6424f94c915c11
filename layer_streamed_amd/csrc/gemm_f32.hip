// fp32-storage GEMM for the debug precision: the same three layouts and
// seven epilogues as the bf16 MFMA kernels, computed with plain fp32 FMA so
// the whole layer can be checked against an fp32 CPU evaluation to ~1e-5.
// It is written for exactness and simplicity, not speed: 64 x 64 output
// tiles, 16-deep K slices staged through LDS (k-major), 256 threads with a
// 4 x 4 register block each (rows ty + 16i, columns tx + 16j).
//
// The SwiGLU forward epilogues compute a tile of the F gate/up columns with
// two accumulators (gate column f and up column F + f of B), so both halves
// of a pair land in the same thread.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

constexpr int FT = 64;   // tile edge
constexpr int FK = 16;   // K slice

__device__ __forceinline__ float sigmoid_exact(float z) { return 1.f / (1.f + expf(-z)); }

// Element (m, k) of op(A) and (k, n) of op(B); zero outside the matrix.
template <int LAYOUT>
__device__ __forceinline__ float a_at(const float* A, long lda, int m, int k, int M, int K) {
  if (m >= M || k >= K) return 0.f;
  return LAYOUT == GEMM_TN ? A[(long)k * lda + m] : A[(long)m * lda + k];
}
template <int LAYOUT>
__device__ __forceinline__ float b_at(const float* B, long ldb, int k, int n, int N, int K) {
  if (n >= N || k >= K) return 0.f;
  return LAYOUT == GEMM_NT ? B[(long)n * ldb + k] : B[(long)k * ldb + n];
}

template <int LAYOUT, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmArgsF32 a) {
  constexpr bool DUAL = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE;
  __shared__ float As[FK][FT + 1];
  __shared__ float Bs[FK][FT + 1];
  __shared__ float Us[DUAL ? FK : 1][FT + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  const int M = a.M, K = a.K;
  const int NC = DUAL ? a.F : a.N;  // columns of the output tile space
  float acc[4][4] = {}, accu[DUAL ? 4 : 1][DUAL ? 4 : 1] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
    // 64 x 16 elements per operand tile, 4 per thread.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = tid + 256 * r;
      const int kk = e % FK, mm = e / FK;  // k fastest: coalesced for k-contiguous operands
      const int kk2 = e / FT, mm2 = e % FT;  // m/n fastest: coalesced for the others
      if (LAYOUT == GEMM_TN) As[kk2][mm2] = a_at<LAYOUT>(a.A, a.lda, m0 + mm2, k0 + kk2, M, K);
      else As[kk][mm] = a_at<LAYOUT>(a.A, a.lda, m0 + mm, k0 + kk, M, K);
      if (LAYOUT == GEMM_NT) {
        Bs[kk][mm] = b_at<LAYOUT>(a.B, a.ldb, k0 + kk, n0 + mm, NC, K);
        if constexpr (DUAL)
          Us[kk][mm] = (n0 + mm < NC && k0 + kk < K) ? a.B[(long)(a.F + n0 + mm) * a.ldb + k0 + kk]
                                                     : 0.f;
      } else {
        Bs[kk2][mm2] = b_at<LAYOUT>(a.B, a.ldb, k0 + kk2, n0 + mm2, NC, K);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
      if constexpr (DUAL) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Us[k][tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) accu[i][j] = fmaf(av[i], bv[j], accu[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty + 16 * i, col = n0 + tx + 16 * j;
      if (row >= M || col >= NC) continue;
      const float v = acc[i][j];
      float* C = reinterpret_cast<float*>(a.C);
      const long c = (long)row * a.ldc + col;
      if constexpr (EPI == EPI_BF16 || EPI == EPI_F32) {
        C[c] = v;
      } else if constexpr (EPI == EPI_ACC_F32) {
        C[c] += v;
      } else if constexpr (EPI == EPI_RESID_BF16) {
        C[c] = a.R[(long)row * a.ldr + col] + v;
      } else if constexpr (DUAL) {
        const float u = accu[i][j];
        C[c] = v * sigmoid_exact(v) * u;
        if constexpr (EPI == EPI_SWIGLU_SAVE) {
          a.C2[(long)row * a.ldc2 + col] = v;
          a.C2[(long)row * a.ldc2 + a.F + col] = u;
        }
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        const float gt = a.G[(long)row * a.ldg + col], u = a.G[(long)row * a.ldg + a.F + col];
        const float sg = sigmoid_exact(gt);
        a.C2[(long)row * a.ldc2 + col] = v * u * sg * (1.f + gt * (1.f - sg));
        a.C2[(long)row * a.ldc2 + a.F + col] = v * gt * sg;
      }
    }
}

template <int LAYOUT, int EPI>
hipError_t launch_f32(const GemmArgsF32& a, hipStream_t s) {
  constexpr bool DUAL = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE;
  const int nc = DUAL ? a.F : a.N;
  const dim3 grid((nc + FT - 1) / FT, (a.M + FT - 1) / FT);
  hipLaunchKernelGGL((gemm_f32_kernel<LAYOUT, EPI>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int LAYOUT>
hipError_t launch_f32_epi(const GemmArgsF32& a, hipStream_t s) {
  switch (a.epi) {
    case EPI_BF16: return launch_f32<LAYOUT, EPI_BF16>(a, s);
    case EPI_F32: return launch_f32<LAYOUT, EPI_F32>(a, s);
    case EPI_ACC_F32: return launch_f32<LAYOUT, EPI_ACC_F32>(a, s);
    case EPI_RESID_BF16: return launch_f32<LAYOUT, EPI_RESID_BF16>(a, s);
    case EPI_SWIGLU_BWD: return launch_f32<LAYOUT, EPI_SWIGLU_BWD>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

const char* gemm_check(const GemmArgsF32& a) {
  if (a.M < 0 || a.N < 0 || a.K < 0) return "negative GEMM size";
  if (!a.A || !a.B || !a.C) return "null GEMM operand";
  if (a.layout < GEMM_NT || a.layout > GEMM_TN) return "bad GEMM layout";
  if (a.epi < EPI_BF16 || a.epi > EPI_SWIGLU_BWD) return "bad GEMM epilogue";
  if (a.layout == GEMM_TN ? a.lda < a.M : a.lda < a.K) return "GEMM lda too small";
  if (a.layout == GEMM_NT ? a.ldb < a.K : a.ldb < a.N) return "GEMM ldb too small";
  if (a.ldc < ((a.epi == EPI_SWIGLU || a.epi == EPI_SWIGLU_SAVE) ? a.F : a.N)) return "GEMM ldc too small";
  if (a.epi == EPI_RESID_BF16 && (!a.R || a.ldr < a.N)) return "residual epilogue needs R, ldr >= N";
  if (a.epi == EPI_SWIGLU || a.epi == EPI_SWIGLU_SAVE) {
    if (a.layout != GEMM_NT) return "SwiGLU forward epilogue needs the NT layout";
    if (a.F < 1 || a.N != 2 * a.F) return "SwiGLU epilogue needs N == 2F";
    if (a.epi == EPI_SWIGLU_SAVE && (!a.C2 || a.ldc2 < 2 * a.F)) return "SwiGLU save needs C2, ldc2 >= 2F";
  }
  if (a.epi == EPI_SWIGLU_BWD &&
      (!a.G || !a.C2 || a.N != a.F || a.ldg < 2 * a.F || a.ldc2 < 2 * a.F))
    return "SwiGLU bwd epilogue needs G, C2, N == F, ldg and ldc2 >= 2F";
  return nullptr;
}

hipError_t gemm_launch(const GemmArgsF32& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.epi == EPI_SWIGLU) return launch_f32<GEMM_NT, EPI_SWIGLU>(a, s);
  if (a.epi == EPI_SWIGLU_SAVE) return launch_f32<GEMM_NT, EPI_SWIGLU_SAVE>(a, s);
  switch (a.layout) {
    case GEMM_NT: return launch_f32_epi<GEMM_NT>(a, s);
    case GEMM_NN: return launch_f32_epi<GEMM_NN>(a, s);
    case GEMM_TN: return launch_f32_epi<GEMM_TN>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mt
