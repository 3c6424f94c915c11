// Causal grouped-query flash attention for gfx950 (forward and backward).
//
// Layout: q, k, v are column blocks of qkv [B*T, (Hq+2Hkv)*d] (bf16);
// query head h reads key/value head h*Hkv/Hq.  Softmax in fp32, scores
// scaled by 1/sqrt(d) and masked causally; the forward saves the row
// log-sum-exp so the backward can rebuild P without storing it.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, see common.h).  The forward
// computes S^T = K Q^T with keys as rows, so in the result every lane holds
// one query (lane % 32) and 16 of its 32 keys; the other 16 are in lane+32.
// The online softmax therefore needs one cross-half exchange per tile, and
// its per-row state (max, sum, rescale factor) is a per-lane scalar.  The
// output is accumulated as O^T = V^T P^T: the P^T operand comes straight
// from the lane's own score registers, because the k-slots an MFMA operand
// lane supplies may be any fixed permutation of k as long as both operands
// agree.  V (and, in the backward, Q, dO, K) is therefore stored in LDS
// transposed, with rows of each 16-row group placed in that permuted order,
// so each lane reads its 8 slots with one 16-byte LDS load.
//
// Backward (deterministic, no atomics): delta = rowsum(dO * O); a dK/dV
// kernel owns 128 keys per workgroup and loops over every query head of the
// GQA group and every query tile at or after its keys; a dQ kernel owns 128
// queries and loops over key tiles up to the diagonal.  For head_dim 128
// the forward and both backward kernels take their streamed tiles (keys and
// values, or queries and dO for dK/dV) straight into LDS and read the
// transposed operands with LDS transpose reads (attn_fwd_pp_kernel,
// attn_dkdv_dl_kernel, attn_dq_dl_kernel); the register-staged forms serve
// head_dim 64.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mt {

// Scratch of the allocation-free attention backward (attn_bwd_static): the
// delta rows, B*Hq*T floats, in a static device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  Host code never uses the array's name as an address: the
// per-device address comes from hipGetSymbolAddress (static_scratch).
static __device__ __align__(256) float scratch[ATTN_STATIC_SCRATCH_FLOATS];

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NEG = -1e30f;

struct AttnArgs {
  const uint16_t* qkv;
  uint16_t* o;
  float* lse;
  const uint16_t* dout;
  const float* delta;
  uint16_t* dqkv;
  int B, T, Hq, Hkv;
  long ldq, ldo;
  float scale;       // 1/sqrt(d)
  float scale_log2;  // scale * log2(e)
};

// Work of a query-block workgroup: query block qb, batch b, query head h.
// Blocks run longest causal rows first.  The heads of one GQA group at one
// query block read the same K/V tiles, and the hardware hands workgroup
// ids to the 8 XCDs (each with its own L2) in turn, so ids are mapped to
// place every such set of heads on one XCD, where the first head's tile
// reads fill the L2 for the others: in whole rounds of 8 sets, XCD x
// (id % 8) takes sets x, x + 8, ... and their heads in order; the sets of a
// last partial round keep the plain order.  A bijection of [0, nqb B Hq).
struct QWork {
  int qb, b, h;
};
__device__ __forceinline__ QWork q_work(int id, int nqb, int B, int Hq, int Hkv) {
  const int grp = Hq / Hkv, sets = nqb * B * Hkv;
  const int whole = (sets >> 3) * 8 * grp;
  int set, hg;
  if (id < whole) {
    const int s = id >> 3;
    set = (s / grp) * 8 + (id & 7);
    hg = s % grp;
  } else {
    set = (sets >> 3) * 8 + (id - whole) / grp;
    hg = (id - whole) % grp;
  }
  const int per = B * Hkv, rest = set % per;
  return {nqb - 1 - set / per, rest / Hkv, (rest % Hkv) * grp + hg};
}

// Row r(s) of the 8-row set (group G of 16 rows, half hs) whose slot order
// matches the MFMA accumulator: slots 0-3 -> rows 4hs..4hs+3, slots 4-7 ->
// rows 8+4hs..8+4hs+3 of the group.
__device__ __forceinline__ int perm_row(int G, int hs, int s) {
  return 16 * G + (s < 4 ? 4 * hs + s : 8 + 4 * hs + (s - 4));
}

// Transpose 8 rows x 4 columns (u32x2 per row) into column di's 8 slots.
__device__ __forceinline__ u32x4_t col_of(const u32x2_t* r, int di) {
  uint32_t h[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint32_t w = (di < 2) ? r[s].x : r[s].y;
    h[s] = (di & 1) ? (w >> 16) : (w & 0xFFFFu);
  }
  u32x4_t o;
  o.x = h[0] | (h[1] << 16);
  o.y = h[2] | (h[3] << 16);
  o.z = h[4] | (h[5] << 16);
  o.w = h[6] | (h[7] << 16);
  return o;
}

// 2^x as the bare v_exp_f32: results below 2^-126 (probabilities of keys
// more than 87 nats below the row maximum) come out as 0 instead of fp32
// denormals, which drops the library exp2f's range-scaling around it (a
// compare, an add, a select and a ldexp per element).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// The values of lanes l and l ^ 32, in an order that depends on the half
// (gfx950 v_permlane32_swap with v in both operands: one instruction instead
// of an LDS permute and its lane arithmetic), for symmetric combinations:
// max(p.x, p.y) or p.x + p.y is the same in both lanes of a pair.
__device__ inline f32x2_t lane_pair32(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return f32x2_t{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}

__device__ __forceinline__ u32x4_t pack_p(const f32x16_t& acc, int jj) {
  u32x4_t v;
  v.x = pack_bf(acc[8 * jj + 0], acc[8 * jj + 1]);
  v.y = pack_bf(acc[8 * jj + 2], acc[8 * jj + 3]);
  v.z = pack_bf(acc[8 * jj + 4], acc[8 * jj + 5]);
  v.w = pack_bf(acc[8 * jj + 6], acc[8 * jj + 7]);
  return v;
}

__device__ __forceinline__ void zero16(f32x16_t& a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = 0.f;
}

// A 64-row x D tile loaded as permuted 8x4 blocks: block b (< 16*D/8... )
// covers rows perm_row(G, hs, 0..7) and columns 4*dq..4*dq+3.
template <int D>
struct PermTile {
  static constexpr int NB = 8 * (D / 4);  // blocks per 64-row tile
  u32x2_t r[8];
  __device__ __forceinline__ void load(const uint16_t* base, long ld, int row0, int nrows,
                                       int tid) {
    if (tid < NB) {
      const int kgrp = tid / (D / 4), dq = tid % (D / 4);
      const int G = kgrp >> 1, hs = kgrp & 1;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int gr = row0 + perm_row(G, hs, s);
        r[s] = gr < nrows ? *reinterpret_cast<const u32x2_t*>(base + (long)gr * ld + dq * 4)
                          : u32x2_t{0, 0};
      }
    }
  }
  // natural layout [64][ld_nat]
  __device__ __forceinline__ void store_nat(uint16_t* s_nat, int ld_nat, int tid) const {
    if (tid < NB) {
      const int kgrp = tid / (D / 4), dq = tid % (D / 4);
      const int G = kgrp >> 1, hs = kgrp & 1;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        *reinterpret_cast<u32x2_t*>(s_nat + perm_row(G, hs, s) * ld_nat + dq * 4) = r[s];
    }
  }
  // transposed, permuted layout [D][ld_t]
  __device__ __forceinline__ void store_t(uint16_t* s_t, int ld_t, int tid) const {
    if (tid < NB) {
      const int kgrp = tid / (D / 4), dq = tid % (D / 4);
      const int G = kgrp >> 1, hs = kgrp & 1;
#pragma unroll
      for (int di = 0; di < 4; ++di)
        *reinterpret_cast<u32x4_t*>(s_t + (dq * 4 + di) * ld_t + G * 16 + hs * 8) = col_of(r, di);
    }
  }
};

// A 64-row x D tile loaded as 16-byte chunks for a natural LDS layout.
template <int D>
struct NatTile {
  static constexpr int PER = 64 * (D / 8) / 256;
  u32x4_t r[PER];
  __device__ __forceinline__ void load(const uint16_t* base, long ld, int row0, int nrows,
                                       int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * 256;
      const int row = c / (D / 8), dc = c % (D / 8);
      const int gr = row0 + row;
      r[p] = gr < nrows ? *reinterpret_cast<const u32x4_t*>(base + (long)gr * ld + dc * 8)
                        : u32x4_t{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int lds, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * 256;
      const int row = c / (D / 8), dc = c % (D / 8);
      *reinterpret_cast<u32x4_t*>(s + row * lds + dc * 8) = r[p];
    }
  }
};

// ------------------------------------------------------------------ forward
// Two workgroups per CU (two waves per SIMD): the kernel fits 248 registers
// without spilling, and one wave's softmax (VALU) then overlaps the other's
// MFMAs: 1.6x (T = 1024) to 1.9x (T = 32K) over one wave per SIMD.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int BQ = 128, BKV = 64, KLD = D + 8, VLD = BKV + 8;
  constexpr int STAGE = BKV * KLD + D * VLD;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int T = a.T;
  const int nqb = (T + BQ - 1) / BQ;
  const QWork wk = q_work(blockIdx.x, nqb, a.B, a.Hq, a.Hkv);
  const int qb = wk.qb, b = wk.b, h = wk.h;
  const int g = (h * a.Hkv) / a.Hq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int q0 = qb * BQ;
  const int qrow = q0 + 32 * w + n;
  const long ldq = a.ldq;
  const uint16_t* base = a.qkv + (long)b * T * ldq;
  const uint16_t* kbase = base + (long)(a.Hq + g) * D;
  const uint16_t* vbase = base + (long)(a.Hq + a.Hkv + g) * D;

  u32x4_t qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = qrow < T ? *reinterpret_cast<const u32x4_t*>(base + (long)qrow * ldq + h * D + ks * 16 + hh * 8)
                      : u32x4_t{0, 0, 0, 0};

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) zero16(oacc[dt]);
  float m = NEG, l = 0.f;

  const int kv_end = min(q0 + BQ, T);
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const int wave_qmax = q0 + 32 * w + 31;

  NatTile<D> kt_ld;
  PermTile<D> vt_ld;
  kt_ld.load(kbase, ldq, 0, T, tid);
  vt_ld.load(vbase, ldq, 0, T, tid);
  kt_ld.store(smem, KLD, tid);
  vt_ld.store_t(smem + BKV * KLD, VLD, tid);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * BKV;
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      kt_ld.load(kbase, ldq, kv0 + BKV, T, tid);
      vt_ld.load(vbase, ldq, kv0 + BKV, T, tid);
    }
    if (kv0 <= wave_qmax) {
      const uint16_t* sk = smem + buf * STAGE;
      const uint16_t* sv = sk + BKV * KLD;
      f32x16_t sacc[2];
      zero16(sacc[0]);
      zero16(sacc[1]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4_t A = *reinterpret_cast<const u32x4_t*>(sk + (32 * kt + n) * KLD + ks * 16 + hh * 8);
          sacc[kt] = mfma32(A, qf[ks], sacc[kt]);
        }
      float mx = NEG;
      auto scores = [&](auto masked) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kv0 + 32 * kt + 8 * (e >> 2) + 4 * hh + (e & 3);
            float s = sacc[kt][e] * a.scale_log2;
            if (decltype(masked)::value && (key > qrow || key >= T)) s = NEG;
            sacc[kt][e] = s;
            mx = fmaxf(mx, s);
          }
      };
      // a tile whose keys all precede the wave's first query and lie in the
      // sequence masks nothing (a wave-uniform test)
      if (kv0 + BKV - 1 <= q0 + 32 * w && kv0 + BKV <= T)
        scores(std::false_type{});
      else
        scores(std::true_type{});
      {
        const f32x2_t mp = lane_pair32(mx);
        mx = fmaxf(mp.x, mp.y);
      }
      const float mnew = fmaxf(m, mx);
      const float alpha = exp2_hw(m - mnew);
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_hw(sacc[kt][e] - mnew);
          sacc[kt][e] = p;
          rs += p;
        }
      {
        const f32x2_t rp = lane_pair32(rs);
        rs = rp.x + rp.y;
      }
      l = l * alpha + rs;
      m = mnew;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
      u32x4_t pf[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) pf[kt][jj] = pack_p(sacc[kt], jj);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const u32x4_t A = *reinterpret_cast<const u32x4_t*>(sv + (32 * dt + n) * VLD + (2 * kt + jj) * 16 + hh * 8);
            oacc[dt] = mfma32(A, pf[kt][jj], oacc[dt]);
          }
    }
    if (t + 1 < ntiles) {
      uint16_t* sk = smem + (buf ^ 1) * STAGE;
      kt_ld.store(sk, KLD, tid);
      vt_ld.store_t(sk + BKV * KLD, VLD, tid);
    }
    __syncthreads();
  }

  if (qrow < T) {
    const float linv = 1.f / l;
    uint16_t* orow = a.o + ((long)b * T + qrow) * a.ldo + h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hh;
        u32x2_t v;
        v.x = pack_bf(oacc[dt][4 * j] * linv, oacc[dt][4 * j + 1] * linv);
        v.y = pack_bf(oacc[dt][4 * j + 2] * linv, oacc[dt][4 * j + 3] * linv);
        *reinterpret_cast<u32x2_t*>(orow + d) = v;
      }
    if (hh == 0) a.lse[((long)b * a.Hq + h) * T + qrow] = (m + log2f(l)) * LN2;
  }
}

// ------------------------------------------------------------ backward prep
// delta[b, h, t] = sum_d O[b, t, h, d] dO[b, t, h, d].  A group of D / 8
// lanes per row (16 bytes each: one contiguous row of O and of dO), the
// groups on consecutive t of one (b, h), so the outputs are contiguous;
// the group's partial sums are combined by lane exchange.
template <int D>
__global__ __launch_bounds__(256) void attn_delta_kernel(const AttnArgs a) {
  constexpr int LPR = D / 8;
  static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "lanes per row");
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long o = gid / LPR;  // flat output index (b Hq + h) T + t
  const int part = (int)(gid % LPR);
  const bool ok = o < (long)a.B * a.Hq * a.T;
  float s = 0.f;
  if (ok) {
    const int t = (int)(o % a.T);
    const long bh = o / a.T;
    const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    const long tok = (long)b * a.T + t;
    const u32x4_t ov = *reinterpret_cast<const u32x4_t*>(a.o + tok * a.ldo + h * D + part * 8);
    const u32x4_t dv = *reinterpret_cast<const u32x4_t*>(a.dout + tok * a.ldo + h * D + part * 8);
    s = lo_bf(ov.x) * lo_bf(dv.x) + hi_bf(ov.x) * hi_bf(dv.x) + lo_bf(ov.y) * lo_bf(dv.y) +
        hi_bf(ov.y) * hi_bf(dv.y) + lo_bf(ov.z) * lo_bf(dv.z) + hi_bf(ov.z) * hi_bf(dv.z) +
        lo_bf(ov.w) * lo_bf(dv.w) + hi_bf(ov.w) * hi_bf(dv.w);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (ok && part == 0) const_cast<float*>(a.delta)[o] = s;
}

// ------------------------------------------------------------- dK and dV
template <int D>
__global__ __launch_bounds__(256) void attn_dkdv_kernel(const AttnArgs a) {
  constexpr int BK = 128, BQ = 64, KLD = D + 8, VLD = BQ + 8;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sQ = smem;
  uint16_t* sdO = sQ + BQ * KLD;
  uint16_t* sQt = sdO + BQ * KLD;
  uint16_t* sdOt = sQt + D * VLD;
  float* sL = reinterpret_cast<float*>(sdOt + D * VLD);
  float* sDl = sL + BQ;

  const int T = a.T;
  const int nkb = (T + BK - 1) / BK;
  const int per = a.Hkv * a.B;
  // key block 0 sees every query tile, the last one only its own: launch
  // the longest first so the short ones fill the tail (the blocks are
  // independent, so the order changes no result)
  const int kb = (int)blockIdx.x / per;
  const int rest = blockIdx.x % per;
  const int g = rest % a.Hkv, b = rest / a.Hkv;
  const int rep = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int k0 = kb * BK;
  const int key = k0 + 32 * w + n;
  const long ldq = a.ldq;
  const uint16_t* base = a.qkv + (long)b * T * ldq;
  const uint16_t* dbase = a.dout + (long)b * T * a.ldo;

  u32x4_t kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bool ok = key < T;
    kf[ks] = ok ? *reinterpret_cast<const u32x4_t*>(base + (long)key * ldq + (a.Hq + g) * D + ks * 16 + hh * 8)
                : u32x4_t{0, 0, 0, 0};
    vf[ks] = ok ? *reinterpret_cast<const u32x4_t*>(base + (long)key * ldq + (a.Hq + a.Hkv + g) * D + ks * 16 + hh * 8)
                : u32x4_t{0, 0, 0, 0};
  }
  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    zero16(dk[dt]);
    zero16(dv[dt]);
  }

  const int ntq = (T - k0 + BQ - 1) / BQ;  // query tiles from k0 to T
  const int nit = rep * ntq;
  PermTile<D> q_ld, d_ld;
  float lse_r = 0.f, del_r = 0.f;
  auto fetch = [&](int it) {
    const int hq = g * rep + it / ntq;
    const int qt0 = k0 + (it % ntq) * BQ;
    q_ld.load(base + hq * D, ldq, qt0, T, tid);
    d_ld.load(dbase + hq * D, a.ldo, qt0, T, tid);
    if (tid < BQ) {
      const int q = qt0 + tid;
      const long li = ((long)b * a.Hq + hq) * T + q;
      lse_r = q < T ? a.lse[li] * LOG2E : -NEG;  // +1e30 makes P = 0 for padding rows
      del_r = q < T ? a.delta[li] : 0.f;
    }
  };
  auto commit = [&]() {
    q_ld.store_nat(sQ, KLD, tid);
    q_ld.store_t(sQt, VLD, tid);
    d_ld.store_nat(sdO, KLD, tid);
    d_ld.store_t(sdOt, VLD, tid);
    if (tid < BQ) {
      sL[tid] = lse_r;
      sDl[tid] = del_r;
    }
  };

  if (nit > 0) {
    fetch(0);
    commit();
  }
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int qt0 = k0 + (it % ntq) * BQ;
    if (it + 1 < nit) fetch(it + 1);
    if (qt0 + BQ - 1 >= k0 + 32 * w) {  // some query of the tile sees this wave's keys
      f32x16_t sacc[2], dpacc[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        zero16(sacc[qt]);
        zero16(dpacc[qt]);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4_t Aq = *reinterpret_cast<const u32x4_t*>(sQ + (32 * qt + n) * KLD + ks * 16 + hh * 8);
          sacc[qt] = mfma32(Aq, kf[ks], sacc[qt]);
          const u32x4_t Ad = *reinterpret_cast<const u32x4_t*>(sdO + (32 * qt + n) * KLD + ks * 16 + hh * 8);
          dpacc[qt] = mfma32(Ad, vf[ks], dpacc[qt]);
        }
      }
      // P and dS, rows = queries (qt0 + 32qt + 8j + 4hh + i), column = key
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qi = 32 * qt + 8 * (e >> 2) + 4 * hh + (e & 3);
          const int q = qt0 + qi;
          float p = exp2_hw(sacc[qt][e] * a.scale_log2 - sL[qi]);
          if (key > q) p = 0.f;
          sacc[qt][e] = p;
          dpacc[qt][e] = p * (dpacc[qt][e] - sDl[qi]);
        }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const u32x4_t Pb = pack_p(sacc[qt], jj);
          const u32x4_t Sb = pack_p(dpacc[qt], jj);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const int off = (32 * dt + n) * VLD + (2 * qt + jj) * 16 + hh * 8;
            dv[dt] = mfma32(*reinterpret_cast<const u32x4_t*>(sdOt + off), Pb, dv[dt]);
            dk[dt] = mfma32(*reinterpret_cast<const u32x4_t*>(sQt + off), Sb, dk[dt]);
          }
        }
    }
    __syncthreads();
    if (it + 1 < nit) commit();
    __syncthreads();
  }

  if (key < T) {
    uint16_t* drow = a.dqkv + ((long)b * T + key) * ldq;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hh;
        u32x2_t vk, vv;
        vk.x = pack_bf(dk[dt][4 * j] * a.scale, dk[dt][4 * j + 1] * a.scale);
        vk.y = pack_bf(dk[dt][4 * j + 2] * a.scale, dk[dt][4 * j + 3] * a.scale);
        vv.x = pack_bf(dv[dt][4 * j], dv[dt][4 * j + 1]);
        vv.y = pack_bf(dv[dt][4 * j + 2], dv[dt][4 * j + 3]);
        *reinterpret_cast<u32x2_t*>(drow + (a.Hq + g) * D + d) = vk;
        *reinterpret_cast<u32x2_t*>(drow + (a.Hq + a.Hkv + g) * D + d) = vv;
      }
  }
}

// dK/dV for head_dim 128 with the Q and dO tiles loaded straight into LDS
// (gfx950 global_load_lds_dwordx4, double-buffered, one barrier per tile)
// in their natural [query][d] layout, 16 chunks of 8 per row stored in the
// order c ^ qtile_swz(row).  The MFMA operands are those of attn_dkdv_kernel
// (same values, same order, so the same bits): Q and dO rows for S and dP
// are one ds_read_b128 per lane; the transposed, permuted dO^T and Q^T for
// dV and dK are two ds_read_b64_tr_b16 per lane (the 16-lane pattern of the
// GEMM's K-major fragments: lane 4j + s addresses query row base + j,
// columns 4s .. 4s+3, and lane i receives column i at rows base .. base+3).
// The copies go out through lds_dma16 (untracked by the compiler, ordered
// by the kernel's own vmcnt wait and barrier), so the compiler's waits for
// the LDS reads never drain the next tile's copies.
//
// The chunk orders keep every tile read on distinct banks.  gfx950's LDS
// has 64 banks (256 bytes per cycle).  A ds_read_b128 is served in four
// passes of 16 lanes: lanes 0-7 with 24-31, 8-15 with 16-23, 32-39 with
// 56-63 and 40-47 with 48-55; a ds_read_b64_tr_b16 in two passes of 32
// consecutive lanes (both measured with the LDS bank-conflict counter on
// access patterns that tell the possible groupings apart).
//  - Forward and dQ tiles (tile_swz): a row read gives lane l row l % 32
//    and one chunk per half-wave, so a pass covers rows 0-7 and 24-31 (or
//    8-15 and 16-23) at one chunk: tile_swz takes 16 different values on
//    any 16 rows aligned at 16.  A transpose read covers 4 consecutive rows
//    x the chunk quad 4 dt .. 4 dt + 3, whose positions are quad
//    dt ^ (row & 3): four quads.
//  - dK/dV tiles (qtile_swz): a row read gives lane 16 g + i row i and
//    chunk c + g, so a pass covers rows 0-7 at chunk c and rows 8-15 at
//    c + 1 (or the reverse): with 2 (row & 7) the two sets of positions are
//    the even and the odd chunks.  A transpose read covers 8 consecutive
//    rows x the chunk pair 2 db, 2 db + 1, whose positions are pair
//    db ^ (row & 7): eight pairs.
// Both orders depend on row bits 0-3 only, so reads at rows +16 and +32 are
// immediate offsets; in tile_swz rows r and r ^ 8 differ in bit 0 of their
// order only, which the forward and dQ pairs of transpose reads (rows r ..
// r+3 and r+8 .. r+11) absorb in a per-lane address offset.
__host__ __device__ constexpr int tile_swz(int row) {
  return ((row & 3) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}
__host__ __device__ constexpr int qtile_swz(int row) { return 2 * (row & 7); }
constexpr bool tile_swz_ok() {
  for (int r = 0; r < 64; ++r) {
    if (tile_swz(r) != tile_swz(r & 15) || tile_swz(r ^ 8) != (tile_swz(r) ^ 1)) return false;
    int seen = 0;
    for (int j = 0; j < 16; ++j) seen |= 1 << tile_swz((r & ~15) + j);
    if (seen != 0xFFFF) return false;
  }
  return true;
}
static_assert(tile_swz_ok(), "tile chunk order");

template <bool QT = false>
__device__ __forceinline__ u32x4_t lds_row16(const char* tile, int row, int chunk) {
  const int sw = QT ? qtile_swz(row) : tile_swz(row);
  return *reinterpret_cast<const u32x4_t*>(tile + row * 256 + ((chunk ^ sw) << 4));
}

// Two transpose reads at p + o0 and p + o1 (constant offsets, which fold
// into the instructions' immediate field) as one MFMA A fragment: rows
// r .. r+3 (o0) and r+8 .. r+11 (o1) of the lane's column, in slots 0-3
// and 4-7.
__device__ __forceinline__ u32x4_t lds_tr_pair(const char* p, const int o0, const int o1) {
  const u32x2_t v0 = lds_tr16(p + o0), v1 = lds_tr16(p + o1);
  return u32x4_t{v0.x, v0.y, v1.x, v1.y};
}

// The same pair from two addresses at one offset: rows r .. r+3 at p and
// r+8 .. r+11 at p8 (whose chunk order differs).
__device__ __forceinline__ u32x4_t lds_tr_pair2(const char* p, const char* p8, const int o) {
  const u32x2_t v0 = lds_tr16(p + o), v1 = lds_tr16(p8 + o);
  return u32x4_t{v0.x, v0.y, v1.x, v1.y};
}

// dK and dV for head_dim 128 on v_mfma_f32_16x16x32_bf16: a workgroup of 8
// waves owns 128 keys, 16 per wave, so a wave's live state (its keys' K and
// V fragments, the dK/dV accumulators, one tile's scores) fits in half the
// register file and two waves share each SIMD.  Per tile of 64 queries
// (streamed into LDS as in the forward, double-buffered, one barrier per
// tile) a wave forms S = Q K^T and dP = dO V^T as 16-query x 16-key blocks
// (lane l: key l & 15, queries 4 (l >> 4) .. + 3 of the block), so each lane
// holds 4 consecutive queries of every block.  For dV^T = dO^T P and
// dK^T = Q^T dS, a 32-query k-step takes its B operand straight from those
// registers: lane group g supplies queries 16 qb + 4g .. + 3 of the step's
// two blocks qb as its 8 k-slots, and the A operand (dO^T, Q^T) is read in
// the same permuted order with two LDS transpose reads (4 query rows each,
// at the two blocks' rows 4g ..).  The summation order over queries is
// therefore fixed: tiles in order, within a tile k-steps in order, slots in
// that permutation.
template <int D>
__global__ __launch_bounds__(512) void attn_dkdv_dl_kernel(const AttnArgs a) {
  static_assert(D == 128, "rows of 16 chunks");
  constexpr int BQ = 64, CH = D / 8, TILE = BQ * D * 2, STAGE = 2 * TILE;
  constexpr int NW = 8;                       // waves per workgroup
  constexpr int PER = BQ * CH / (64 * NW);    // 16-byte loads per wave per operand
  constexpr int NDB = D / 16;                 // 16-column blocks of d
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  float* sLb = reinterpret_cast<float*>(dsm + 2 * STAGE);  // [2][BQ]
  float* sDb = sLb + 2 * BQ;                               // [2][BQ]

  const int T = a.T;
  const int per = a.Hkv * a.B;
  const int kb = (int)blockIdx.x / per;  // most query tiles first
  const int rest = blockIdx.x % per;
  const int g = rest % a.Hkv, b = rest / a.Hkv;
  const int rep = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;  // lane in its 16-lane group, group
  const int k0 = kb * 128;
  const int kw = k0 + 16 * w;  // this wave's first key
  const int key = kw + li;
  const long ldq = a.ldq;
  const uint16_t* base = a.qkv + (long)b * T * ldq;
  const uint16_t* dbase = a.dout + (long)b * T * a.ldo;

  // B operand of S and dP: key li, d-slots 32 ks + 8 lg .. + 7
  u32x4_t kf[D / 32], vf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const bool ok = key < T;
    kf[ks] = ok ? *reinterpret_cast<const u32x4_t*>(base + (long)key * ldq + (a.Hq + g) * D + ks * 32 + lg * 8)
                : u32x4_t{0, 0, 0, 0};
    vf[ks] = ok ? *reinterpret_cast<const u32x4_t*>(base + (long)key * ldq + (a.Hq + a.Hkv + g) * D + ks * 32 + lg * 8)
                : u32x4_t{0, 0, 0, 0};
  }
  // dK^T, dV^T blocks [16 d x 16 keys]: lane: key li, d = 16 db + 4 lg + i
  f32x4_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dv[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int ntq = (T - k0 + BQ - 1) / BQ;  // query tiles from k0 to T
  const int nit = rep * ntq;
  float lse_r = 0.f, del_r = 0.f;
  int lse_q = 0;
  // Loop-invariant address parts, as in the forward: the wave index as a
  // scalar, per copy slot the source row and chunk offsets, per Q / dO
  // fragment the LDS byte offset within a stage (the tile loop is unrolled
  // by two, the stage a constant in each half).
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int crow[PER], qoff[PER], doff[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int slot = (wu * PER + p) * 64 + lane;
    const int row = slot / CH, pos = slot % CH;
    const int c8 = (pos ^ qtile_swz(row)) << 3;
    crow[p] = row;
    qoff[p] = row * (int)ldq + c8;
    doff[p] = row * (int)a.ldo + c8;
  }
  int qro[D / 32];
#pragma unroll
  for (int kn = 0; kn < D / 32; ++kn) qro[kn] = li * 256 + (((4 * kn + lg) ^ qtile_swz(li)) << 4);
  // tile `it` -> stage BUF: Q and dO rows clamped to T - 1 past the end
  // (their P is 0 through lse = +1e30, so they add exact zeros)
  auto issue = [&](int it, auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    const int hq = g * rep + it / ntq;
    const int qt0 = k0 + (it % ntq) * BQ;
    char* sq = dsm + buf * STAGE;
    if (qt0 + BQ <= T) {
      const uint16_t* q0p = base + (long)qt0 * ldq + hq * D;
      const uint16_t* d0p = dbase + (long)qt0 * a.ldo + hq * D;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        lds_dma16(q0p + qoff[p], sq + (wu * PER + p) * 1024);
        lds_dma16(d0p + doff[p], sq + TILE + (wu * PER + p) * 1024);
      }
    } else {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const long gq = min(qt0 + crow[p], T - 1);
        const int c8 = qoff[p] - crow[p] * (int)ldq;
        lds_dma16(base + gq * ldq + hq * D + c8, sq + (wu * PER + p) * 1024);
        lds_dma16(dbase + gq * a.ldo + hq * D + c8, sq + TILE + (wu * PER + p) * 1024);
      }
    }
    // statistics of the tile's rows, raw: nothing reads them before the
    // stage's copies are waited for (a use right after the load would wait
    // for those copies too); rows past the end read row T - 1
    if (tid < BQ) {
      const long lix = ((long)b * a.Hq + hq) * T + min(qt0 + tid, T - 1);
      lse_r = a.lse[lix];
      del_r = a.delta[lix];
      lse_q = qt0 + tid;
    }
  };
  // the stage's statistics into LDS: lse in log2 units, +1e30 for padding
  // rows (P = 0), delta 0 there
  auto stats = [&](int buf) {
    if (tid < BQ) {
      const bool in = lse_q < T;
      sLb[buf * BQ + tid] = in ? lse_r * LOG2E : -NEG;
      sDb[buf * BQ + tid] = in ? del_r : 0.f;
    }
  };

  // Transpose-read addresses of the A operand of dV^T / dK^T for column
  // block db: the lane addresses query row 4 lg + (li >> 2) (plus the
  // step's block offset, an immediate) and columns 16 db + 4 (li & 3);
  // the row's low bits, hence its swizzle, are the same for every step.
  uint32_t trb[NDB];
  {
    const int row = 4 * lg + (li >> 2);
    const int sw = qtile_swz(row);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      trb[db] = row * 256 + (((2 * db + ((li >> 1) & 1)) ^ sw) << 4) + (li & 1) * 8;
  }

  issue(0, std::integral_constant<int, 0>{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // the key's K and V fragments are complete here (as in the forward)
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    asm volatile("" : "+v"(kf[ks]));
    asm volatile("" : "+v"(vf[ks]));
  }
  stats(0);
  __syncthreads();
  auto tile = [&](int it, auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    // the other stage was last read in the previous iteration (the barrier
    // at its end retired those reads): the next tile streams into it under
    // this whole iteration
    if (it + 1 < nit) issue(it + 1, std::integral_constant<int, buf ^ 1>{});
    const int qt0 = k0 + (it % ntq) * BQ;
    const char* sq = dsm + buf * STAGE;
    const char* sdo = sq + TILE;
    const float* sL = sLb + buf * BQ;
    const float* sDl = sDb + buf * BQ;
    // some query of the tile sees this wave's first key
    const bool active = qt0 + BQ - 1 >= kw;
    if (active) {
      // S and dP, blocks qb of 16 queries: A = Q / dO rows 16 qb + li at
      // d-slots 32 ks + 8 lg (one row read each), B = K / V fragments.  The
      // row reads of step s+1 go out before the MFMAs of step s.
      f32x4_t sacc[BQ / 16], dpacc[BQ / 16];
      constexpr int NS1 = (BQ / 16) * (D / 32);
      u32x4_t Aq[2], Ad[2];
      Aq[0] = *reinterpret_cast<const u32x4_t*>(sq + qro[0]);
      Ad[0] = *reinterpret_cast<const u32x4_t*>(sdo + qro[0]);
#pragma unroll
      for (int s = 0; s < NS1; ++s) {
        const int qb = s / (D / 32), ks = s % (D / 32), c = s & 1;
        if (ks == 0) {
          sacc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          dpacc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (s + 1 < NS1) {
          const int qn = (s + 1) / (D / 32), kn = (s + 1) % (D / 32);
          Aq[c ^ 1] = *reinterpret_cast<const u32x4_t*>(sq + qn * 16 * 256 + qro[kn]);
          Ad[c ^ 1] = *reinterpret_cast<const u32x4_t*>(sdo + qn * 16 * 256 + qro[kn]);
        }
        asm volatile("" : "+v"(Aq[c]));
        asm volatile("" : "+v"(Ad[c]));
        sacc[qb] = mfma16x32(Aq[c], kf[ks], sacc[qb]);
        dpacc[qb] = mfma16x32(Ad[c], vf[ks], dpacc[qb]);
      }
      // P and dS: lane holds key li and queries 16 qb + 4 lg + i; the
      // causal mask only where some query of the tile precedes one of this
      // wave's keys (a wave-uniform test)
      auto p_ds = [&](auto masked) {
#pragma unroll
        for (int qb = 0; qb < BQ / 16; ++qb) {
          const f32x4_t L4 = *reinterpret_cast<const f32x4_t*>(sL + 16 * qb + 4 * lg);
          const f32x4_t D4 = *reinterpret_cast<const f32x4_t*>(sDl + 16 * qb + 4 * lg);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p = exp2_hw(sacc[qb][i] * a.scale_log2 - L4[i]);
            if (decltype(masked)::value && key > qt0 + 16 * qb + 4 * lg + i) p = 0.f;
            sacc[qb][i] = p;
            dpacc[qb][i] = p * (dpacc[qb][i] - D4[i]);
          }
        }
      };
      if (qt0 < kw + 15)
        p_ds(std::true_type{});
      else
        p_ds(std::false_type{});
      // dV^T and dK^T over steps (qc, db), qc the 32-query k-step: B is
      // P / dS of blocks 2 qc and 2 qc + 1 packed in that slot order; A the
      // dO^T / Q^T fragment of column block db at those rows (two transpose
      // reads each).  The reads of step s+1 go out before the MFMAs of s.
      constexpr int NS3 = (BQ / 32) * NDB;
      const char* sqa = sq;
      u32x4_t At[2], Aq2[2];
      auto reads = [&](int s, int slot) {
        const int qc = s / NDB, db = s % NDB;
        const int ro = 32 * qc * 256;
        const char* ad = sqa + trb[db];
        At[slot] = lds_tr_pair(ad, TILE + ro, TILE + ro + 16 * 256);
        Aq2[slot] = lds_tr_pair(ad, ro, ro + 16 * 256);
      };
      u32x4_t Pb = {0, 0, 0, 0}, Sb = {0, 0, 0, 0};
      reads(0, 0);
#pragma unroll
      for (int s = 0; s < NS3; ++s) {
        const int qc = s / NDB, db = s % NDB, c = s & 1;
        if (db == 0) {
          Pb = u32x4_t{pack_bf(sacc[2 * qc][0], sacc[2 * qc][1]),
                       pack_bf(sacc[2 * qc][2], sacc[2 * qc][3]),
                       pack_bf(sacc[2 * qc + 1][0], sacc[2 * qc + 1][1]),
                       pack_bf(sacc[2 * qc + 1][2], sacc[2 * qc + 1][3])};
          Sb = u32x4_t{pack_bf(dpacc[2 * qc][0], dpacc[2 * qc][1]),
                       pack_bf(dpacc[2 * qc][2], dpacc[2 * qc][3]),
                       pack_bf(dpacc[2 * qc + 1][0], dpacc[2 * qc + 1][1]),
                       pack_bf(dpacc[2 * qc + 1][2], dpacc[2 * qc + 1][3])};
        }
        if (s + 1 < NS3) {
          reads(s + 1, c ^ 1);
        }
        asm volatile("" : "+v"(At[c]));
        asm volatile("" : "+v"(Aq2[c]));
        dv[db] = mfma16x32(At[c], Pb, dv[db]);
        dk[db] = mfma16x32(Aq2[c], Sb, dk[db]);
      }
    }
    if (it + 1 < nit) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      stats(buf ^ 1);
    }
    __syncthreads();
  };
  {
    int it = 0;
    for (; it + 1 < nit; it += 2) {
      tile(it, std::integral_constant<int, 0>{});
      tile(it + 1, std::integral_constant<int, 1>{});
    }
    if (it < nit) tile(it, std::integral_constant<int, 0>{});
  }

  if (key < T) {
    uint16_t* drow = a.dqkv + ((long)b * T + key) * ldq;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 16 * db + 4 * lg;
      u32x2_t vk, vv;
      vk.x = pack_bf(dk[db][0] * a.scale, dk[db][1] * a.scale);
      vk.y = pack_bf(dk[db][2] * a.scale, dk[db][3] * a.scale);
      vv.x = pack_bf(dv[db][0], dv[db][1]);
      vv.y = pack_bf(dv[db][2], dv[db][3]);
      *reinterpret_cast<u32x2_t*>(drow + (a.Hq + g) * D + d) = vk;
      *reinterpret_cast<u32x2_t*>(drow + (a.Hq + a.Hkv + g) * D + d) = vv;
    }
  }
}

// dQ for head_dim 128 in the dK/dV kernel's form: the K and V tiles of 64
// keys go straight into LDS (global_load_lds, double-buffered, one barrier
// per tile) in their natural [key][d] layout with the same chunk swizzle; K
// and V rows for S^T and dP^T are one ds_read_b128 per lane, and the
// transposed K^T fragments for dQ two ds_read_b64_tr_b16 at immediate
// offsets.  Products, operand k-slot order and summation order per query are
// those of attn_dq_kernel, without its register-staged tile copies.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_dq_dl_kernel(const AttnArgs a) {
  static_assert(D == 128, "rows of 16 chunks");
  constexpr int BQ = 128, BKV = 64, CH = D / 8, TILE = BKV * D * 2, STAGE = 2 * TILE;
  constexpr int PER = BKV * CH / 256;  // 16-byte load instructions per lane per operand
  extern __shared__ __attribute__((aligned(16))) char dsm[];

  const int T = a.T;
  const int nqb = (T + BQ - 1) / BQ;
  const QWork wk = q_work(blockIdx.x, nqb, a.B, a.Hq, a.Hkv);
  const int qb = wk.qb, b = wk.b, h = wk.h;
  const int g = (h * a.Hkv) / a.Hq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int q0 = qb * BQ;
  const int qrow = q0 + 32 * w + n;
  const long ldq = a.ldq;
  const uint16_t* base = a.qkv + (long)b * T * ldq;
  const uint16_t* kbase = base + (long)(a.Hq + g) * D;
  const uint16_t* vbase = base + (long)(a.Hq + a.Hkv + g) * D;

  u32x4_t qf[D / 16], df[D / 16];
  const bool ok = qrow < T;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = ok ? *reinterpret_cast<const u32x4_t*>(base + (long)qrow * ldq + h * D + ks * 16 + hh * 8)
                : u32x4_t{0, 0, 0, 0};
    df[ks] = ok ? *reinterpret_cast<const u32x4_t*>(a.dout + ((long)b * T + qrow) * a.ldo + h * D + ks * 16 + hh * 8)
                : u32x4_t{0, 0, 0, 0};
  }
  const long li = ((long)b * a.Hq + h) * T + qrow;
  const float lse2_l = ok ? a.lse[li] * LOG2E : -NEG;
  const float del_l = ok ? a.delta[li] : 0.f;

  f32x16_t dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) zero16(dq[dt]);

  const int kv_end = min(q0 + BQ, T);
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const int wave_qmax = q0 + 32 * w + 31;
  // tile t -> stage buf: K and V rows clamped to T - 1 past the end (those
  // keys are masked)
  auto issue = [&](int t, int buf) {
    const int kv0 = t * BKV;
    char* sk = dsm + buf * STAGE;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int slot = (w * PER + p) * 64 + lane;
      const int row = slot / CH, pos = slot % CH;
      const int c = pos ^ tile_swz(row);
      const long gk = min(kv0 + row, T - 1);
      lds_dma16(kbase + gk * ldq + c * 8, sk + (w * PER + p) * 1024);
      lds_dma16(vbase + gk * ldq + c * 8, sk + TILE + (w * PER + p) * 1024);
    }
  };
  // K^T read addresses and the row + 8 partner offset, as in the forward
  uint32_t trb[D / 32];
  int d8;
  {
    const int i = lane & 15, r = 4 * hh + (i >> 2);
    const int sw = tile_swz(r);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      trb[dt] = r * 256 + (((4 * dt + 2 * ((lane >> 4) & 1) + ((i >> 1) & 1)) ^ sw) << 4) + (i & 1) * 8;
    const int c0 = 2 * ((lane >> 4) & 1) + ((i >> 1) & 1);
    d8 = 8 * 256 + (((c0 ^ tile_swz(r + 8)) - (c0 ^ sw)) << 4);
  }

  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // as in the forward: the row's fragments and statistics are complete here
  float lse2 = lse2_l, del = del_l;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    asm volatile("" : "+v"(qf[ks]));
    asm volatile("" : "+v"(df[ks]));
  }
  asm volatile("" : "+v"(lse2), "+v"(del));
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) issue(t + 1, buf ^ 1);
    const int kv0 = t * BKV;
    const char* sk = dsm + buf * STAGE;
    const char* sv = sk + TILE;
    if (kv0 <= wave_qmax) {
      f32x16_t sacc[2], dpacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        zero16(sacc[kt]);
        zero16(dpacc[kt]);
        u32x4_t Ak[2], Av[2];
        Ak[0] = lds_row16(sk, 32 * kt + n, hh);
        Av[0] = lds_row16(sv, 32 * kt + n, hh);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int c = ks & 1;
          if (ks + 1 < D / 16) {
            Ak[c ^ 1] = lds_row16(sk, 32 * kt + n, 2 * (ks + 1) + hh);
            Av[c ^ 1] = lds_row16(sv, 32 * kt + n, 2 * (ks + 1) + hh);
          }
          asm volatile("" : "+v"(Ak[c]));
          asm volatile("" : "+v"(Av[c]));
          sacc[kt] = mfma32(Ak[c], qf[ks], sacc[kt]);
          dpacc[kt] = mfma32(Av[c], df[ks], dpacc[kt]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][e] = exp2_hw(sacc[kt][e] * a.scale_log2 - lse2);
      // the causal mask only where some key of the tile follows one of the
      // wave's queries or lies past the end (a wave-uniform test)
      if (!(kv0 + BKV - 1 <= q0 + 32 * w && kv0 + BKV <= T)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int kk = kv0 + 32 * kt + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (kk > qrow || kk >= T) sacc[kt][e] = 0.f;
          }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) dpacc[kt][e] = sacc[kt][e] * (dpacc[kt][e] - del);
      // dQ over steps i = (kt, jj, dt); the two transpose reads of step
      // i+1 go out before the MFMA of step i
      constexpr int NI = 2 * 2 * (D / 32);
      const char* ska = sk;
      u32x4_t Kt[2];
      u32x4_t Sb = {0, 0, 0, 0};
      auto reads = [&](int i, int slot) {
        const int kt = i / (2 * (D / 32)), jj = (i / (D / 32)) & 1, dt = i % (D / 32);
        const int ro = (32 * kt + 16 * jj) * 256;
        const char* ad = ska + trb[dt];
        Kt[slot] = lds_tr_pair2(ad, ad + d8, ro);
      };
      reads(0, 0);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int kt = i / (2 * (D / 32)), jj = (i / (D / 32)) & 1, dt = i % (D / 32);
        const int c = i & 1;
        if (dt == 0) Sb = pack_p(dpacc[kt], jj);
        if (i + 1 < NI) {
          reads(i + 1, c ^ 1);
        }
        asm volatile("" : "+v"(Kt[c]));
        dq[dt] = mfma32(Kt[c], Sb, dq[dt]);
      }
    }
    if (t + 1 < ntiles) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  if (ok) {
    uint16_t* drow = a.dqkv + ((long)b * T + qrow) * ldq + h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hh;
        u32x2_t v;
        v.x = pack_bf(dq[dt][4 * j] * a.scale, dq[dt][4 * j + 1] * a.scale);
        v.y = pack_bf(dq[dt][4 * j + 2] * a.scale, dq[dt][4 * j + 3] * a.scale);
        *reinterpret_cast<u32x2_t*>(drow + d) = v;
      }
  }
}

// --------------------------------------------------------------------- dQ
// Two waves per SIMD as in the forward (a few registers spill, still 4-12%
// faster than one wave); the dK/dV kernel stays at one (its accumulators
// and resident K/V fragments would spill heavily).
template <int D>
__global__ __launch_bounds__(256, 2) void attn_dq_kernel(const AttnArgs a) {
  constexpr int BQ = 128, BKV = 64, KLD = D + 8, VLD = BKV + 8;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sK = smem;
  uint16_t* sV = sK + BKV * KLD;
  uint16_t* sKt = sV + BKV * KLD;

  const int T = a.T;
  const int nqb = (T + BQ - 1) / BQ;
  const QWork wk = q_work(blockIdx.x, nqb, a.B, a.Hq, a.Hkv);
  const int qb = wk.qb, b = wk.b, h = wk.h;
  const int g = (h * a.Hkv) / a.Hq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int q0 = qb * BQ;
  const int qrow = q0 + 32 * w + n;
  const long ldq = a.ldq;
  const uint16_t* base = a.qkv + (long)b * T * ldq;
  const uint16_t* kbase = base + (long)(a.Hq + g) * D;
  const uint16_t* vbase = base + (long)(a.Hq + a.Hkv + g) * D;

  u32x4_t qf[D / 16], df[D / 16];
  const bool ok = qrow < T;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = ok ? *reinterpret_cast<const u32x4_t*>(base + (long)qrow * ldq + h * D + ks * 16 + hh * 8)
                : u32x4_t{0, 0, 0, 0};
    df[ks] = ok ? *reinterpret_cast<const u32x4_t*>(a.dout + ((long)b * T + qrow) * a.ldo + h * D + ks * 16 + hh * 8)
                : u32x4_t{0, 0, 0, 0};
  }
  const long li = ((long)b * a.Hq + h) * T + qrow;
  const float lse2 = ok ? a.lse[li] * LOG2E : -NEG;
  const float del = ok ? a.delta[li] : 0.f;

  f32x16_t dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) zero16(dq[dt]);

  const int kv_end = min(q0 + BQ, T);
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const int wave_qmax = q0 + 32 * w + 31;
  PermTile<D> k_ld;
  NatTile<D> v_ld;
  auto fetch = [&](int kv0) {
    k_ld.load(kbase, ldq, kv0, T, tid);
    v_ld.load(vbase, ldq, kv0, T, tid);
  };
  auto commit = [&]() {
    k_ld.store_nat(sK, KLD, tid);
    k_ld.store_t(sKt, VLD, tid);
    v_ld.store(sV, KLD, tid);
  };
  fetch(0);
  commit();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * BKV;
    if (t + 1 < ntiles) fetch(kv0 + BKV);
    if (kv0 <= wave_qmax) {
      f32x16_t sacc[2], dpacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        zero16(sacc[kt]);
        zero16(dpacc[kt]);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4_t Ak = *reinterpret_cast<const u32x4_t*>(sK + (32 * kt + n) * KLD + ks * 16 + hh * 8);
          sacc[kt] = mfma32(Ak, qf[ks], sacc[kt]);
          const u32x4_t Av = *reinterpret_cast<const u32x4_t*>(sV + (32 * kt + n) * KLD + ks * 16 + hh * 8);
          dpacc[kt] = mfma32(Av, df[ks], dpacc[kt]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = kv0 + 32 * kt + 8 * (e >> 2) + 4 * hh + (e & 3);
          float p = exp2_hw(sacc[kt][e] * a.scale_log2 - lse2);
          if (kk > qrow || kk >= T) p = 0.f;
          dpacc[kt][e] = p * (dpacc[kt][e] - del);
        }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const u32x4_t Sb = pack_p(dpacc[kt], jj);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const u32x4_t A = *reinterpret_cast<const u32x4_t*>(sKt + (32 * dt + n) * VLD + (2 * kt + jj) * 16 + hh * 8);
            dq[dt] = mfma32(A, Sb, dq[dt]);
          }
        }
    }
    __syncthreads();
    if (t + 1 < ntiles) commit();
    __syncthreads();
  }

  if (ok) {
    uint16_t* drow = a.dqkv + ((long)b * T + qrow) * ldq + h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hh;
        u32x2_t v;
        v.x = pack_bf(dq[dt][4 * j] * a.scale, dq[dt][4 * j + 1] * a.scale);
        v.y = pack_bf(dq[dt][4 * j + 2] * a.scale, dq[dt][4 * j + 3] * a.scale);
        *reinterpret_cast<u32x2_t*>(drow + d) = v;
      }
  }
}

// The forward for head_dim 128 as two wave groups in ping-pong.  A
// workgroup of 8 waves takes 256 queries, 32 per wave: group 0 (waves 0-3)
// the first 128, group 1 (waves 4-7) the rest; waves w and w + 4 share a
// SIMD.  Each wave alternates two phases per 64-key tile t, separated by
// workgroup barriers: an MFMA phase (O^T += V^T P^T of tile t - 1, then
// S^T of tile t) and a vector phase (the softmax of tile t).  Group 1 runs
// the same code one phase behind group 0 (one extra barrier at its start,
// one at group 0's end), so on every SIMD one wave's exponentials and
// packing run under the other wave's matrix products, instead of the two
// waves drifting into the same phase.  The K and V tiles go straight into
// LDS (global_load_lds) through a ring of 4 stages, issued by group 0 three
// tiles ahead: tile t + 1 is complete at the barrier that ends group 0's
// vector phase of tile t, and only after that barrier is the stage of tile
// t - 1 (whose V group 1 read in the phase just ended) refilled.  Per query
// the operations and their order are those of attn_fwd_kernel.
template <int D>
__global__ __launch_bounds__(512, 1) void attn_fwd_pp_kernel(const AttnArgs a) {
  static_assert(D == 128, "rows of 16 chunks");
  constexpr int BQ = 256, BKV = 64, CH = D / 8, TILE = BKV * D * 2, STAGE = 2 * TILE, NS = 4;
  constexpr int PER = BKV * CH / 256;  // 16-byte copies per group-0 lane per operand
  static_assert(2 * PER == 8, "the vmcnt immediates below count 8 copies per tile");
  extern __shared__ __attribute__((aligned(16))) char dsm[];

  const int T = a.T;
  const int nqb = (T + BQ - 1) / BQ;
  const QWork wk = q_work(blockIdx.x, nqb, a.B, a.Hq, a.Hkv);
  const int qb = wk.qb, b = wk.b, h = wk.h;
  const int g = (h * a.Hkv) / a.Hq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int grp = wu >> 2;
  const int q0 = qb * BQ;
  const int wq0 = q0 + 32 * wu;  // the wave's first query (a scalar)
  const int qrow = wq0 + n;
  const int wave_qmax = wq0 + 31;
  const long ldq = a.ldq;
  const uint16_t* base = a.qkv + (long)b * T * ldq;
  const uint16_t* kbase = base + (long)(a.Hq + g) * D;
  const uint16_t* vbase = base + (long)(a.Hq + a.Hkv + g) * D;

  u32x4_t qf[D / 16];
  f32x16_t oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) zero16(oacc[dt]);
  float m = NEG, l = 0.f;

  const int kv_end = min(q0 + BQ, T);
  const int ntiles = (kv_end + BKV - 1) / BKV;
  // copy slots of group 0's lanes: source row and chunk (K and V tiles
  // share the layout)
  int crow[PER], ccol[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int slot = (wu * PER + p) * 64 + lane;
    const int row = slot / CH, pos = slot % CH;
    crow[p] = row;
    ccol[p] = row * (int)ldq + ((pos ^ tile_swz(row)) << 3);
  }
  // tile t -> stage t % NS: K and V rows clamped to T - 1 past the end
  // (those keys are masked)
  auto issue = [&](int t) {
    const int kv0 = t * BKV;
    char* sk = dsm + (t % NS) * STAGE;
    if (kv0 + BKV <= T) {
      const uint16_t* kt0 = kbase + (long)kv0 * ldq;
      const uint16_t* vt0 = vbase + (long)kv0 * ldq;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        lds_dma16(kt0 + ccol[p], sk + (wu * PER + p) * 1024);
        lds_dma16(vt0 + ccol[p], sk + TILE + (wu * PER + p) * 1024);
      }
    } else {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const long gk = min(kv0 + crow[p], T - 1);
        const int c8 = ccol[p] - crow[p] * (int)ldq;
        lds_dma16(kbase + gk * ldq + c8, sk + (wu * PER + p) * 1024);
        lds_dma16(vbase + gk * ldq + c8, sk + TILE + (wu * PER + p) * 1024);
      }
    }
  };
  // K row fragments: key row n of each 32-key block at chunk 2 ks + hh
  int kro[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kro[ks] = n * 256 + (((2 * ks + hh) ^ tile_swz(n)) << 4);
  // V^T read addresses, as the dK/dV kernel's Q^T reads, and the offset
  // from a read at row r to its partner at row r + 8: 8 rows, and the
  // chunk's position with bit 0 flipped (the same for every dt: bit 0 of
  // the chunk is (i >> 1) & 1)
  uint32_t trb[D / 32];
  int d8;
  {
    const int i = lane & 15, r = 4 * hh + (i >> 2);
    const int sw = tile_swz(r);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      trb[dt] = r * 256 + (((4 * dt + 2 * ((lane >> 4) & 1) + ((i >> 1) & 1)) ^ sw) << 4) + (i & 1) * 8;
    const int c0 = 2 * ((lane >> 4) & 1) + ((i >> 1) & 1);
    d8 = 8 * 256 + (((c0 ^ tile_swz(r + 8)) - (c0 ^ sw)) << 4);
  }
  uint32_t trb8[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) trb8[dt] = trb[dt] + d8;

  f32x16_t sacc[2];
  u32x4_t pf[2][2];
  // S^T of tile t for both 32-key blocks: the two products alternate, and
  // the K row reads run two k-steps ahead of their MFMAs
  auto s_phase = [&](int t) {
    const char* sk = dsm + (t % NS) * STAGE;
    zero16(sacc[0]);
    zero16(sacc[1]);
    u32x4_t Ak[3][2];
    auto kread = [&](int ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        Ak[ks % 3][kt] = *reinterpret_cast<const u32x4_t*>(sk + kt * 32 * 256 + kro[ks]);
    };
    kread(0);
    kread(1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if (ks + 2 < D / 16) kread(ks + 2);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        asm volatile("" : "+v"(Ak[ks % 3][kt]));
        sacc[kt] = mfma32(Ak[ks % 3][kt], qf[ks], sacc[kt]);
      }
    }
  };
  // online softmax of tile t's scores (left unscaled in S: the positive
  // scale commutes with the max), the running max and sum, the rescale of
  // O when some query's max moved, and P packed to bf16
  auto softmax = [&](int t) {
    const int kv0 = t * BKV;
    float mx = NEG;
    auto scores = [&](auto masked) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv0 + 32 * kt + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (decltype(masked)::value && (key > qrow || key >= T)) sacc[kt][e] = NEG;
          mx = fmaxf(mx, sacc[kt][e]);
        }
    };
    // a tile whose keys all precede the wave's first query and lie in the
    // sequence masks nothing (a wave-uniform test)
    if (kv0 + BKV - 1 <= wq0 && kv0 + BKV <= T)
      scores(std::false_type{});
    else
      scores(std::true_type{});
    {
      const f32x2_t mp = lane_pair32(mx);
      mx = fmaxf(mp.x, mp.y);
    }
    const float mnew = fmaxf(m, mx * a.scale_log2);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2_hw(fmaf(sacc[kt][e], a.scale_log2, -mnew));
        sacc[kt][e] = p;
        rs += p;
      }
    {
      const f32x2_t rp = lane_pair32(rs);
      rs = rp.x + rp.y;
    }
    // where no query's running max moved, the factor is exactly 1 (2^0)
    if (__ballot(mnew != m)) {
      const float alpha = exp2_hw(m - mnew);
      l = l * alpha + rs;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
    } else {
      l = l + rs;
    }
    m = mnew;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) pf[kt][jj] = pack_p(sacc[kt], jj);
  };
  // O^T += V^T P^T(t) over steps i = (kt, jj, dt), consecutive MFMAs into
  // different accumulators; transpose reads two steps ahead
  auto pv_phase = [&](int t) {
    const char* sva = dsm + (t % NS) * STAGE + TILE;
    constexpr int NI = (D / 32) * 2 * 2;
    u32x4_t Vt[3];
    auto reads = [&](int i) {
      const int dt = i % (D / 32), kt = i / (D / 16), jj = (i / (D / 32)) & 1;
      const int ro = (32 * kt + 16 * jj) * 256;
      Vt[i % 3] = lds_tr_pair2(sva + trb[dt], sva + trb8[dt], ro);
    };
    reads(0);
    reads(1);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int dt = i % (D / 32), kt = i / (D / 16), jj = (i / (D / 32)) & 1;
      if (i + 2 < NI) reads(i + 2);
      asm volatile("" : "+v"(Vt[i % 3]));
      oacc[dt] = mfma32(Vt[i % 3], pf[kt][jj], oacc[dt]);
    }
  };

#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = qrow < T ? *reinterpret_cast<const u32x4_t*>(base + (long)qrow * ldq + h * D + ks * 16 + hh * 8)
                      : u32x4_t{0, 0, 0, 0};
  if (grp == 0) {
    issue(0);
    if (1 < ntiles) issue(1);
  }
  // tiles 0 and 1 and the Q fragments complete; tying the fragments to
  // this point keeps the compiler, which does not track the copies, from
  // waiting for them (and so for every copy in flight) later on
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(qf[ks]));
  if (grp == 0 && 2 < ntiles) issue(2);
  __syncthreads();
  // Every wave runs every iteration and its two barriers, and both groups
  // pass 2 ntiles + 4 barriers in all; a wave whose queries all precede a
  // tile skips that tile's work.
  if (grp == 1) __syncthreads();
  for (int t = 0; t <= ntiles; ++t) {
    const bool prev = t >= 1 && (t - 1) * BKV <= wave_qmax;
    const bool cur = t < ntiles && t * BKV <= wave_qmax;
    // the MFMA phase at a raised wave priority, so that the wave's MFMAs
    // and LDS reads issue ahead of its SIMD partner's softmax
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(2);
    __builtin_amdgcn_sched_barrier(0);
    if (prev) pv_phase(t - 1);
    if (cur) s_phase(t);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    if (cur) softmax(t);
    if (grp == 0) {
      // tile t + 1 complete before group 0's next MFMA phase reads it (tile
      // t + 2 may stay in flight)
      if (t + 2 < ntiles)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (t + 1 < ntiles)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (grp == 0 && t + 3 < ntiles) issue(t + 3);
  }
  if (grp == 0) __syncthreads();

  if (qrow < T) {
    const float linv = 1.f / l;
    uint16_t* orow = a.o + ((long)b * T + qrow) * a.ldo + h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hh;
        u32x2_t v;
        v.x = pack_bf(oacc[dt][4 * j] * linv, oacc[dt][4 * j + 1] * linv);
        v.y = pack_bf(oacc[dt][4 * j + 2] * linv, oacc[dt][4 * j + 3] * linv);
        *reinterpret_cast<u32x2_t*>(orow + d) = v;
      }
    if (hh == 0) a.lse[((long)b * a.Hq + h) * T + qrow] = (m + log2f(l)) * LN2;
  }
}

template <class K>
hipError_t set_lds(K kern, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int D>
hipError_t fwd_d(const AttnArgs& a, hipStream_t s) {
  constexpr size_t lds = 2 * (64 * (D + 8) + D * (64 + 8)) * sizeof(uint16_t);
  constexpr size_t lds_pp = 4 * 2 * 64 * D * sizeof(uint16_t);
  static bool attr = false;
  if (!attr) {
    hipError_t e = set_lds(attn_fwd_kernel<D>, lds);
    if (e != hipSuccess) return e;
    if constexpr (D == 128) {
      e = set_lds(attn_fwd_pp_kernel<D>, lds_pp);
      if (e != hipSuccess) return e;
    }
    attr = true;
  }
  if constexpr (D == 128)
    hipLaunchKernelGGL(attn_fwd_pp_kernel<D>, dim3((a.T + 255) / 256 * a.Hq * a.B), dim3(512), lds_pp, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3((a.T + 127) / 128 * a.Hq * a.B), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const AttnArgs& a, int stages, hipStream_t s) {
  constexpr size_t lds_kv = (2 * 64 * (D + 8) + 2 * D * (64 + 8)) * sizeof(uint16_t) + 2 * 64 * sizeof(float);
  constexpr size_t lds_q = (2 * 64 * (D + 8) + D * (64 + 8)) * sizeof(uint16_t);
  constexpr size_t lds_dl = 2 * 2 * 64 * D * sizeof(uint16_t) + 4 * 64 * sizeof(float);
  constexpr size_t lds_dq_dl = 2 * 2 * 64 * D * sizeof(uint16_t);
  static bool attr = false;
  if (!attr) {
    hipError_t e = set_lds(attn_dkdv_kernel<D>, lds_kv);
    if (e != hipSuccess) return e;
    e = set_lds(attn_dq_kernel<D>, lds_q);
    if (e != hipSuccess) return e;
    if constexpr (D == 128) {
      e = set_lds(attn_dkdv_dl_kernel<D>, lds_dl);
      if (e != hipSuccess) return e;
      e = set_lds(attn_dq_dl_kernel<D>, lds_dq_dl);
      if (e != hipSuccess) return e;
    }
    attr = true;
  }
  if (stages & ATTN_BWD_DELTA) {
    const long threads = (long)a.B * a.T * a.Hq * (D / 8);
    hipLaunchKernelGGL(attn_delta_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & ATTN_BWD_DKDV) {
    const int nkb = (a.T + 127) / 128;
    if constexpr (D == 128)
      hipLaunchKernelGGL(attn_dkdv_dl_kernel<D>, dim3(nkb * a.Hkv * a.B), dim3(512), lds_dl, s, a);
    else
      hipLaunchKernelGGL(attn_dkdv_kernel<D>, dim3(nkb * a.Hkv * a.B), dim3(256), lds_kv, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & ATTN_BWD_DQ) {
    const int nqb = (a.T + 127) / 128;
    if constexpr (D == 128)
      hipLaunchKernelGGL(attn_dq_dl_kernel<D>, dim3(nqb * a.Hq * a.B), dim3(256), lds_dq_dl, s, a);
    else
      hipLaunchKernelGGL(attn_dq_kernel<D>, dim3(nqb * a.Hq * a.B), dim3(256), lds_q, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

AttnArgs make_args(const uint16_t* qkv, int batch, int seq, int n_heads, int n_kv_heads,
                   int head_dim) {
  AttnArgs a{};
  a.qkv = qkv;
  a.B = batch;
  a.T = seq;
  a.Hq = n_heads;
  a.Hkv = n_kv_heads;
  a.ldq = (long)(n_heads + 2 * n_kv_heads) * head_dim;
  a.ldo = (long)n_heads * head_dim;
  a.scale = 1.f / sqrtf((float)head_dim);
  a.scale_log2 = a.scale * LOG2E;
  return a;
}

}  // namespace

hipError_t attn_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int batch, int seq, int n_heads,
                    int n_kv_heads, int head_dim, hipStream_t s) {
  if (batch == 0 || seq == 0) return hipSuccess;
  AttnArgs a = make_args(qkv, batch, seq, n_heads, n_kv_heads, head_dim);
  a.o = o;
  a.lse = lse;
  if (head_dim == 128) return fwd_d<128>(a, s);
  if (head_dim == 64) return fwd_d<64>(a, s);
  return hipErrorInvalidValue;
}

hipError_t attn_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse,
                    const uint16_t* dout, float* delta, uint16_t* dqkv, int batch, int seq,
                    int n_heads, int n_kv_heads, int head_dim, hipStream_t s, int stages) {
  if (batch == 0 || seq == 0) return hipSuccess;
  AttnArgs a = make_args(qkv, batch, seq, n_heads, n_kv_heads, head_dim);
  a.o = const_cast<uint16_t*>(o);
  a.lse = const_cast<float*>(lse);
  a.dout = dout;
  a.delta = delta;
  a.dqkv = dqkv;
  if (head_dim == 128) return bwd_d<128>(a, stages, s);
  if (head_dim == 64) return bwd_d<64>(a, stages, s);
  return hipErrorInvalidValue;
}

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
float* scratch_dev[MAX_DEVICES] = {};  // scratch's address on each device
}  // namespace

// The address of `scratch` on the current device, resolved once per device
// with that device current.
static hipError_t static_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

hipError_t attn_bwd_static(const uint16_t* qkv, const uint16_t* o, const float* lse,
                           const uint16_t* dout, uint16_t* dqkv, int batch, int seq, int n_heads,
                           int n_kv_heads, int head_dim, hipStream_t s) {
  if ((size_t)batch * n_heads * seq > ATTN_STATIC_SCRATCH_FLOATS) return hipErrorInvalidValue;
  float* delta = nullptr;
  const hipError_t e = static_scratch(&delta);
  if (e != hipSuccess) return e;
  return attn_bwd(qkv, o, lse, dout, delta, dqkv, batch, seq, n_heads, n_kv_heads, head_dim, s);
}

const char* attn_kernel_name(int head_dim, int which) {
  static const char* n128[4] = {"attn_fwd_pp_kernel<128>", "attn_delta_kernel<128>",
                                "attn_dkdv_dl_kernel<128>", "attn_dq_dl_kernel<128>"};
  static const char* n64[4] = {"attn_fwd_kernel<64>", "attn_delta_kernel<64>",
                               "attn_dkdv_kernel<64>", "attn_dq_kernel<64>"};
  if (which < 0 || which > 3) return "";
  return head_dim == 128 ? n128[which] : n64[which];
}

}  // namespace mt
