// bf16 MFMA GEMM for gfx950 with fused epilogues.
//
// One kernel template serves the three operand layouts the decoder layer
// needs (forward NT, activation-gradient NN, weight-gradient TN).  Both
// operands are staged through LDS in a K-contiguous layout ([rows][BK+8]
// bf16, the 8-element pad spreads rows over LDS banks), so the MFMA
// fragment reads are single 16-byte ds_read_b128 per lane for every layout.
// An operand whose memory order is K-major ([K, rows], rows contiguous) is
// loaded as 8(k) x 4(rows) blocks of 8-byte global loads and transposed in
// registers before the LDS store.  The K loop is double buffered in LDS with
// one barrier per 64-wide K step; the next step's global loads are issued
// before the current step's MFMAs.
//
// Workgroup-to-tile order: the flat workgroup id is first re-ranked so each
// of the 8 XCDs (which the dispatcher feeds round-robin) owns a contiguous
// range of tiles, then walked in groups of 8 tile-rows so that neighbouring
// workgroups on one XCD share A rows and B columns in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;

// K-contiguous operand: ROWS x BK tile of X[row][k] (row stride ld).
// Row pointers are formed once per tile (rows past the edge are clamped to
// a valid row and their data zeroed), so the K loop only adds k0.  CHECK
// selects the guarded form for edge tiles and the K tail; interior tiles
// take plain loads with no per-lane branches.
template <int ROWS, int NTHR>
struct LoadKC {
  static constexpr int CPR = BK / 8;  // 16-byte chunks per row
  static constexpr int PER = ROWS * CPR / NTHR;
  static_assert(PER >= 1 && ROWS * CPR % NTHR == 0, "tile/thread mismatch");
  u32x4_t r[PER];
  const uint16_t* ptr[PER];
  bool rok[PER];

  template <class Map>
  __device__ __forceinline__ void init(const uint16_t* __restrict__ X, long ld, int r0, int nrows,
                                       int tid, Map map) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * NTHR;
      const int row = c / CPR, kc = c % CPR;
      const int gr = r0 + row;
      rok[p] = gr < nrows;
      ptr[p] = X + (long)map(rok[p] ? gr : nrows - 1) * ld + kc * 8;
    }
  }
  template <bool CHECK>
  __device__ __forceinline__ void load(int k0, int K, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      if constexpr (CHECK) {
        const int gk = k0 + ((tid + p * NTHR) % CPR) * 8;
        const bool ok = rok[p] && gk < K;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ptr[p] + (gk < K ? k0 : 0));
        r[p] = ok ? v : u32x4_t{0, 0, 0, 0};
      } else {
        r[p] = *reinterpret_cast<const u32x4_t*>(ptr[p] + k0);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * NTHR;
      const int row = c / CPR, kc = c % CPR;
      *reinterpret_cast<u32x4_t*>(s + row * LDK + kc * 8) = r[p];
    }
  }
};

// K-major operand: X[k][row] (row contiguous, stride ld between k), loaded
// as 8(k) x 4(rows) blocks and transposed to the K-contiguous LDS layout.
template <int ROWS, int NTHR>
struct LoadT {
  static constexpr int RB = ROWS / 4;  // 4-row groups
  static constexpr int PER = (BK / 8) * RB / NTHR;
  static_assert(PER >= 1 && (BK / 8) * RB % NTHR == 0, "tile/thread mismatch");
  u32x2_t r[PER][8];
  const uint16_t* ptr[PER];
  bool rok[PER];
  long ld_;

  __device__ __forceinline__ void init(const uint16_t* __restrict__ X, long ld, int r0, int nrows,
                                       int tid) {
    ld_ = ld;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + p * NTHR;
      const int kb = b / RB, rb = b % RB;
      const int gr = r0 + rb * 4;
      rok[p] = gr < nrows;
      ptr[p] = X + (long)(kb * 8) * ld + (rok[p] ? gr : 0);
    }
  }
  template <bool CHECK>
  __device__ __forceinline__ void load(int k0, int K, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int kb = (tid + p * NTHR) / RB;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if constexpr (CHECK) {
          const int gk = k0 + kb * 8 + kk;
          const bool ok = rok[p] && gk < K;
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(ptr[p] + (gk < K ? (long)(k0 + kk) * ld_ : 0));
          r[p][kk] = ok ? v : u32x2_t{0, 0};
        } else {
          r[p][kk] = *reinterpret_cast<const u32x2_t*>(ptr[p] + (long)(k0 + kk) * ld_);
        }
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + p * NTHR;
      const int kb = b / RB, rb = b % RB;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        uint32_t h[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const uint32_t w = (mi < 2) ? r[p][kk].x : r[p][kk].y;
          h[kk] = (mi & 1) ? (w >> 16) : (w & 0xFFFFu);
        }
        u32x4_t o;
        o.x = h[0] | (h[1] << 16);
        o.y = h[2] | (h[3] << 16);
        o.z = h[4] | (h[5] << 16);
        o.w = h[6] | (h[7] << 16);
        *reinterpret_cast<u32x4_t*>(s + (rb * 4 + mi) * LDK + kb * 8) = o;
      }
    }
  }
};

struct IdMap {
  __device__ __forceinline__ int operator()(int r) const { return r; }
};
// Virtual column n of the gate/up product -> row of [W_gate; W_up]:
// 64-wide pair blocks hold 32 gate rows then the 32 up rows of the same f.
struct SwiMap {
  int F;
  __device__ __forceinline__ int operator()(int n) const {
    const int p = n >> 6, w = n & 63;
    return w < 32 ? p * 32 + w : F + p * 32 + (w - 32);
  }
};

__device__ __forceinline__ float silu_f(float z) { return z / (1.f + __expf(-z)); }

// Epilogue shared by the GEMM kernels: acc holds the wave's TM x TN blocks of
// 32 x 32 (lane l: column l % 32, rows 8j + 4(l/32) + i in element 4j + i).
template <int WM, int WN, int TM, int TN, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& a, f32x16_t (&acc)[TM][TN], int m0, int n0,
                                         int wm, int wn, int lane) {
  const int M = a.M, N = a.N;
  const int rbase = m0 + wm * TM * 32 + 4 * (lane >> 5);
  const int cbase = n0 + wn * TN * 32 + (lane & 31);
  if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) {
    static_assert(TN % 2 == 0, "SwiGLU pairs need an even TN");
    uint16_t* Cm = reinterpret_cast<uint16_t*>(a.C);
    const int fbase = (n0 + wn * TN * 32) / 2 + (lane & 31);
    const int F = a.F;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < TN / 2; ++q)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
          const int f = fbase + 32 * q;
          if (row < M && f < F) {
            const float gv = acc[i][2 * q][e], uv = acc[i][2 * q + 1][e];
            Cm[(long)row * a.ldc + f] = f2bf(silu_f(gv) * uv);
            if constexpr (EPI == EPI_SWIGLU_SAVE) {
              a.C2[(long)row * a.ldc2 + f] = f2bf(gv);
              a.C2[(long)row * a.ldc2 + F + f] = f2bf(uv);
            }
          }
        }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
          const int col = cbase + j * 32;
          if (row >= M || col >= N) continue;
          const float v = acc[i][j][e];
          if constexpr (EPI == EPI_BF16) {
            reinterpret_cast<uint16_t*>(a.C)[(long)row * a.ldc + col] = f2bf(v);
          } else if constexpr (EPI == EPI_F32) {
            reinterpret_cast<float*>(a.C)[(long)row * a.ldc + col] = v;
          } else if constexpr (EPI == EPI_ACC_F32) {
            reinterpret_cast<float*>(a.C)[(long)row * a.ldc + col] += v;
          }
        }
  }
  if constexpr (EPI == EPI_RESID_BF16 || EPI == EPI_SWIGLU_BWD) {
    // Per 32 x 32 block: issue every load of the block first, then compute
    // and store, so the loads overlap instead of each waiting its latency.
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = cbase + j * 32;
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // half a block at a time bounds the live registers
          float x0[8], x1[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int e = 8 * h + q;
            const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
            const bool ok = row < M && col < N;
            if constexpr (EPI == EPI_RESID_BF16) {
              x0[q] = ok ? bf2f(a.R[(long)row * a.ldr + col]) : 0.f;
            } else {
              x0[q] = ok ? bf2f(a.G[(long)row * a.ldg + col]) : 0.f;
              x1[q] = ok ? bf2f(a.G[(long)row * a.ldg + a.F + col]) : 0.f;
            }
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int e = 8 * h + q;
            const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
            if (row >= M || col >= N) continue;
            const float v = acc[i][j][e];
            if constexpr (EPI == EPI_RESID_BF16) {
              reinterpret_cast<uint16_t*>(a.C)[(long)row * a.ldc + col] = f2bf(x0[q] + v);
            } else {
              const float gt = x0[q], u = x1[q];
              const float sg = 1.f / (1.f + __expf(-gt));
              a.C2[(long)row * a.ldc2 + col] = f2bf(v * u * sg * (1.f + gt * (1.f - sg)));
              a.C2[(long)row * a.ldc2 + a.F + col] = f2bf(v * gt * sg);
            }
          }
        }
      }
  }
}

template <int WM, int WN, int TM, int TN, int LAYOUT, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(const GemmArgs a) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, NTHR = WM * WN * 64;
  constexpr int STAGE = (BM + BN) * LDK;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int M = a.M, N = a.N, K = a.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int pid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = pid / per_group;
  const int first_m = g * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int tile_m = first_m + (pid % per_group) % gm;
  const int tile_n = (pid % per_group) / gm;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  using LA = typename std::conditional<LAYOUT == GEMM_TN, LoadT<BM, NTHR>, LoadKC<BM, NTHR>>::type;
  using LB = typename std::conditional<LAYOUT == GEMM_NT, LoadKC<BN, NTHR>, LoadT<BN, NTHR>>::type;
  LA la;
  LB lb;
  if constexpr (LAYOUT == GEMM_TN) la.init(a.A, a.lda, m0, M, tid);
  else la.init(a.A, a.lda, m0, M, tid, IdMap{});
  if constexpr (LAYOUT == GEMM_NT) {
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE)
      lb.init(a.B, a.ldb, n0, N, tid, SwiMap{a.F});
    else
      lb.init(a.B, a.ldb, n0, N, tid, IdMap{});
  } else {
    lb.init(a.B, a.ldb, n0, N, tid);
  }
  // interior tiles need no row guards; K tiles need guards only at the tail
  const bool edge = (m0 + BM > M) || (n0 + BN > N);
  const int nk = (K + BK - 1) / BK;
  const int nk_full = edge ? 0 : K / BK;
  auto issue = [&](int kt) {
    if (kt < nk_full) {
      la.template load<false>(kt * BK, K, tid);
      lb.template load<false>(kt * BK, K, tid);
    } else {
      la.template load<true>(kt * BK, K, tid);
      lb.template load<true>(kt * BK, K, tid);
    }
  };
  auto commit = [&](int buf) {
    uint16_t* s = smem + buf * STAGE;
    la.store(s, tid);
    lb.store(s + BM * LDK, tid);
  };

  issue(0);
  commit(0);
  __syncthreads();
  const int arow = wm * TM * 32 + (lane & 31);
  const int brow = wn * TN * 32 + (lane & 31);
  const int koff = (lane >> 5) * 8;
  auto compute = [&](int buf) {
    const uint16_t* sA = smem + buf * STAGE;
    const uint16_t* sB = sA + BM * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const u32x4_t*>(sA + (arow + i * 32) * LDK + ks * 16 + koff);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4_t*>(sB + (brow + j * 32) * LDK + ks * 16 + koff);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  };
  // steady state: next tile's loads in flight while this tile computes
  int kt = 0;
  for (; kt + 1 < nk; ++kt) {
    issue(kt + 1);
    compute(kt & 1);
    commit((kt + 1) & 1);
    __syncthreads();
  }
  if (nk > 0) compute(kt & 1);

  epilogue<WM, WN, TM, TN, EPI>(a, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// NT product with direct global -> LDS loads (gfx950 global_load_lds_dwordx4).
// Both operands are K-contiguous, so each lane's 16-byte chunk can land in
// LDS without passing through registers: lane t of a wave instruction writes
// LDS base + 16 t.  A ring of DL_STAGES stages of DL_BK columns keeps three
// stages of loads in flight while one is computed, so the load latency is
// covered by LDS capacity instead of registers.  Within a row the 4 chunks
// are stored in the order c ^ ((row >> 2) & 3), which makes the fragment
// reads (32 lanes, 32 consecutive rows, one chunk) bank-conflict free.
// Requires K % DL_BK == 0; rows past M or N are clamped to a valid row (they
// only feed output elements the epilogue drops).
constexpr int DL_BK = 32;
constexpr int DL_STAGES = 4;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int WM, int WN, int TM, int TN, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_dl_kernel(const GemmArgs a) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32, NW = WM * WN;
  constexpr int CH = DL_BK / 8;  // 16-byte chunks per row
  constexpr int A_CH = BM * CH, B_CH = BN * CH;
  constexpr int A_PER = A_CH / 64 / NW, B_PER = B_CH / 64 / NW;  // instructions per wave
  static_assert(A_PER * 64 * NW == A_CH && B_PER * 64 * NW == B_CH, "tile/wave mismatch");
  constexpr int LPW = A_PER + B_PER;
  constexpr int STAGE = (A_CH + B_CH) * 16;  // bytes
  extern __shared__ __attribute__((aligned(16))) char dl_smem[];

  const int M = a.M, N = a.N, K = a.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int pid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = pid / per_group;
  const int first_m = g * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int tile_m = first_m + (pid % per_group) % gm;
  const int tile_n = (pid % per_group) / gm;
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const uint16_t* ga[A_PER];
  const uint16_t* gb[B_PER];
#pragma unroll
  for (int p = 0; p < A_PER; ++p) {
    const int pos = (wave * A_PER + p) * 64 + lane;
    const int row = pos / CH, slot = pos % CH;
    const int c = slot ^ ((row >> 2) & (CH - 1));
    const int gr = min(m0 + row, M - 1);
    ga[p] = a.A + (long)gr * a.lda + c * 8;
  }
#pragma unroll
  for (int p = 0; p < B_PER; ++p) {
    const int pos = (wave * B_PER + p) * 64 + lane;
    const int row = pos / CH, slot = pos % CH;
    const int c = slot ^ ((row >> 2) & (CH - 1));
    int gr = min(n0 + row, N - 1);
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) gr = SwiMap{a.F}(gr);
    gb[p] = a.B + (long)gr * a.ldb + c * 8;
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = K / DL_BK;
  auto issue = [&](int kt) {
    if (kt >= nk) return;
    const int k0 = kt * DL_BK;
    char* base = dl_smem + (kt % DL_STAGES) * STAGE;
#pragma unroll
    for (int p = 0; p < A_PER; ++p)
      __builtin_amdgcn_global_load_lds(
          (const void*)(ga[p] + k0),
          (__attribute__((address_space(3))) void*)(base + (wave * A_PER + p) * 1024), 16, 0, 0);
#pragma unroll
    for (int p = 0; p < B_PER; ++p)
      __builtin_amdgcn_global_load_lds(
          (const void*)(gb[p] + k0),
          (__attribute__((address_space(3))) void*)(base + A_CH * 16 + (wave * B_PER + p) * 1024), 16,
          0, 0);
  };

  const int arow = wm * TM * 32 + (lane & 31);
  const int brow = wn * TN * 32 + (lane & 31);
  const int hh = lane >> 5;
  auto compute = [&](int kt) {
    const u32x4_t* sA = reinterpret_cast<const u32x4_t*>(dl_smem + (kt % DL_STAGES) * STAGE);
    const u32x4_t* sB = sA + A_CH;
#pragma unroll
    for (int ks = 0; ks < DL_BK / 16; ++ks) {
      const int c = ks * 2 + hh;
      u32x4_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = arow + i * 32;
        af[i] = sA[r * CH + (c ^ ((r >> 2) & (CH - 1)))];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = brow + j * 32;
        bfr[j] = sB[r * CH + (c ^ ((r >> 2) & (CH - 1)))];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  };

#pragma unroll
  for (int st = 0; st < DL_STAGES - 1; ++st) issue(st);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads for stage kt are done once at most `ahead` later
    // stages are still in flight; the barrier then covers every wave's loads
    // and every wave's reads of the stage about to be refilled
    const int ahead = min(DL_STAGES - 2, nk - 1 - kt);
    if (ahead >= 2) wait_vmcnt<2 * LPW>();
    else if (ahead == 1) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    issue(kt + DL_STAGES - 1);
    compute(kt);
  }
  epilogue<WM, WN, TM, TN, EPI>(a, acc, m0, n0, wm, wn, lane);
}

template <int WM, int WN, int TM, int TN, int EPI>
hipError_t launch_dl(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const size_t lds = (size_t)DL_STAGES * (BM + BN) * (DL_BK / 8) * 16;
  auto kern = gemm_nt_dl_kernel<WM, WN, TM, TN, EPI>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(WM * WN * 64), lds, s, a);
  return hipGetLastError();
}

template <int WM, int WN, int TM, int TN, int LAYOUT, int EPI>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const size_t lds = 2 * (BM + BN) * LDK * sizeof(uint16_t);
  auto kern = gemm_kernel<WM, WN, TM, TN, LAYOUT, EPI>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(WM * WN * 64), lds, s, a);
  return hipGetLastError();
}

// Tile choice: 256 x 256 (eight waves of 128 x 64, two per SIMD so one
// wave's memory stalls hide behind the other's MFMAs) cuts LDS reads per
// MFMA flop and L2 re-reads against 128 x 128; it is used when the grid
// still fills the 256 CUs several times over.
inline bool use_big_tile(const GemmArgs& a) {
  const long t = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
  return t >= 4 * 256;
}

template <int LAYOUT, int EPI>
hipError_t launch_layout(const GemmArgs& a, hipStream_t s) {
  if constexpr (LAYOUT == GEMM_NT && EPI != EPI_SWIGLU_BWD) {
    if (use_big_tile(a) && a.K % DL_BK == 0) return launch_dl<2, 4, 4, 2, EPI>(a, s);
  }
  // the SwiGLU-backward epilogue needs more registers than the big tile
  // leaves (it would spill its accumulators), so it keeps the 128 x 128 tile
  if constexpr (EPI != EPI_SWIGLU_BWD) {
    if (use_big_tile(a)) return launch_cfg<2, 4, 4, 2, LAYOUT, EPI>(a, s);
  }
  return launch_cfg<2, 2, 2, 2, LAYOUT, EPI>(a, s);
}

template <int LAYOUT>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s) {
  switch (a.epi) {
    case EPI_BF16: return launch_layout<LAYOUT, EPI_BF16>(a, s);
    case EPI_F32: return launch_layout<LAYOUT, EPI_F32>(a, s);
    case EPI_ACC_F32: return launch_layout<LAYOUT, EPI_ACC_F32>(a, s);
    case EPI_RESID_BF16: return launch_layout<LAYOUT, EPI_RESID_BF16>(a, s);
    case EPI_SWIGLU_BWD: return launch_layout<LAYOUT, EPI_SWIGLU_BWD>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

const char* gemm_check(const GemmArgs& a) {
  if (a.M < 0 || a.N < 0 || a.K < 0) return "negative GEMM size";
  if (!a.A || !a.B || !a.C) return "null GEMM operand";
  if (a.layout != GEMM_TN && a.K % 8) return "NT/NN GEMM K must be a multiple of 8";
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  if (!al16(a.A) || !al16(a.B)) return "GEMM operands must be 16-byte aligned";
  if (a.lda % 8 || a.ldb % 8) return "GEMM leading dimensions must be multiples of 8";
  if (a.layout == GEMM_TN && a.M % 8) return "TN GEMM needs M % 8 == 0";
  if (a.layout != GEMM_NT && a.N % 8) return "NN/TN GEMM needs N % 8 == 0";
  if (a.layout < GEMM_NT || a.layout > GEMM_TN) return "bad GEMM layout";
  if (a.layout == GEMM_TN ? a.lda < a.M : a.lda < a.K) return "GEMM lda too small";
  if (a.layout == GEMM_NT ? a.ldb < a.K : a.ldb < a.N) return "GEMM ldb too small";
  if (a.ldc < ((a.epi == EPI_SWIGLU || a.epi == EPI_SWIGLU_SAVE) ? a.F : a.N)) return "GEMM ldc too small";
  if (a.epi == EPI_RESID_BF16 && a.ldr < a.N) return "GEMM ldr too small";
  if ((a.epi == EPI_SWIGLU_SAVE || a.epi == EPI_SWIGLU_BWD) && a.ldc2 < 2 * a.F) return "GEMM ldc2 too small";
  if (a.epi == EPI_SWIGLU_BWD && a.ldg < 2 * a.F) return "GEMM ldg too small";
  if (a.epi == EPI_SWIGLU || a.epi == EPI_SWIGLU_SAVE) {
    if (a.layout != GEMM_NT) return "SwiGLU forward epilogue needs the NT layout";
    if (a.F % 32 || a.N != 2 * a.F) return "SwiGLU epilogue needs N == 2F, F % 32 == 0";
    if (a.epi == EPI_SWIGLU_SAVE && !a.C2) return "SwiGLU save needs C2";
  }
  if (a.epi == EPI_SWIGLU_BWD && (!a.G || !a.C2 || a.N != a.F)) return "SwiGLU bwd epilogue needs G, C2, N == F";
  if (a.epi == EPI_RESID_BF16 && !a.R) return "residual epilogue needs R";
  if (a.epi < EPI_BF16 || a.epi > EPI_SWIGLU_BWD) return "bad GEMM epilogue";
  return nullptr;
}

hipError_t gemm_launch(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.epi == EPI_SWIGLU) return launch_layout<GEMM_NT, EPI_SWIGLU>(a, s);
  if (a.epi == EPI_SWIGLU_SAVE) return launch_layout<GEMM_NT, EPI_SWIGLU_SAVE>(a, s);
  switch (a.layout) {
    case GEMM_NT: return launch_epi<GEMM_NT>(a, s);
    case GEMM_NN: return launch_epi<GEMM_NN>(a, s);
    case GEMM_TN: return launch_epi<GEMM_TN>(a, s);
  }
  return hipErrorInvalidValue;
}

const char* gemm_kernel_name(const GemmArgs& a) {
  (void)a;
  return "gemm_kernel";
}

}  // namespace mt
