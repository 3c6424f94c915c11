// Row-wise and elementwise kernels of the decoder layer (gfx950):
// RMSNorm forward/backward with deterministic gain-gradient partials, RoPE
// tables and rotation, the LM-head cross-entropy rows, casts and fills.
// All are HBM-bound; one wave64 owns one row so every reduction is a
// register loop plus one wave butterfly, with 16-byte vector accesses.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

constexpr int RN_WAVES = 4;  // rows per workgroup in the forward

__device__ __forceinline__ void unpack8(u32x4_t v, float* f) {
  f[0] = lo_bf(v.x); f[1] = hi_bf(v.x); f[2] = lo_bf(v.y); f[3] = hi_bf(v.y);
  f[4] = lo_bf(v.z); f[5] = hi_bf(v.z); f[6] = lo_bf(v.w); f[7] = hi_bf(v.w);
}
__device__ __forceinline__ u32x4_t pack8(const float* f) {
  u32x4_t v;
  v.x = pack_bf(f[0], f[1]); v.y = pack_bf(f[2], f[3]);
  v.z = pack_bf(f[4], f[5]); v.w = pack_bf(f[6], f[7]);
  return v;
}

// Storage of activations, weights and gradients: bf16 bit patterns (the
// training path) or fp32 (the debug precision).  Math is fp32 either way.
template <class E>
struct St;
template <>
struct St<uint16_t> {
  static __device__ __forceinline__ void load8(const uint16_t* p, float* f) {
    unpack8(*reinterpret_cast<const u32x4_t*>(p), f);
  }
  static __device__ __forceinline__ void store8(uint16_t* p, const float* f) {
    *reinterpret_cast<u32x4_t*>(p) = pack8(f);
  }
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f2bf(v); }
};
template <>
struct St<float> {
  static __device__ __forceinline__ void load8(const float* p, float* f) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
    const f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  static __device__ __forceinline__ void store8(float* p, const float* f) {
    reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{f[0], f[1], f[2], f[3]};
    reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{f[4], f[5], f[6], f[7]};
  }
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};

// y = x * rsqrt(mean(x^2) + eps) * g.  One wave per row; cols % 8 == 0.
template <class E>
__global__ __launch_bounds__(RN_WAVES * 64) void rmsnorm_fwd_kernel(
    const E* __restrict__ x, const E* __restrict__ g, E* __restrict__ y,
    float* __restrict__ rstd_out, int rows, int cols, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * RN_WAVES + (threadIdx.x >> 6);
  if (row >= rows) return;
  const E* xr = x + (long)row * cols;
  const int nch = cols / 8;
  float ss = 0.f;
  for (int c = lane; c < nch; c += 64) {
    float f[8];
    St<E>::load8(xr + c * 8, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += f[i] * f[i];
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)cols + eps);
  if (lane == 0 && rstd_out) rstd_out[row] = r;
  E* yr = y + (long)row * cols;
  for (int c = lane; c < nch; c += 64) {
    float f[8], gg[8];
    St<E>::load8(xr + c * 8, f);
    St<E>::load8(g + c * 8, gg);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] * r * gg[i];
    St<E>::store8(yr + c * 8, f);
  }
}

// Backward.  Each workgroup (4 waves) owns RB_ROWS consecutive rows; every
// wave walks its rows and keeps per-column dg sums for its chunk columns in
// registers; the 4 waves are combined in LDS in fixed order and written as
// one partial row of dg_part.  MAXC = max chunk iterations per lane.  16
// rows per workgroup give the memory-bound kernel several waves per SIMD
// (1024 workgroups for 16384 rows).
constexpr int RB_ROWS = 16;

template <class E, int MAXC>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(
    const E* __restrict__ dy, const E* __restrict__ x, const E* __restrict__ g,
    const float* __restrict__ rstd, const E* __restrict__ resid, E* __restrict__ dx,
    float* __restrict__ dg_part,
    int rows, int cols) {
  extern __shared__ float red[];  // [4][cols]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = cols / 8;
  float acc[MAXC][8];
#pragma unroll
  for (int k = 0; k < MAXC; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[k][i] = 0.f;
  const int r0 = blockIdx.x * RB_ROWS;
  const float inv_cols = 1.f / (float)cols;
  for (int rr = wave; rr < RB_ROWS; rr += 4) {
    const int row = r0 + rr;
    if (row >= rows) break;
    const long off = (long)row * cols;
    const float r = rstd[row];
    float dot = 0.f;
    // bf16 rows stay in registers (the raw 16-byte chunks) between the two
    // passes, so dy and x are read once; fp32 rows are read again
    constexpr bool KEEP = std::is_same<E, uint16_t>::value;
    u32x4_t kd[KEEP ? MAXC : 1], kx[KEEP ? MAXC : 1];
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
      const int c = lane + 64 * k;
      if (c < nch) {
        float fd[8], fx[8], fg[8];
        if constexpr (KEEP) {
          kd[k] = *reinterpret_cast<const u32x4_t*>(dy + off + c * 8);
          kx[k] = *reinterpret_cast<const u32x4_t*>(x + off + c * 8);
          unpack8(kd[k], fd);
          unpack8(kx[k], fx);
        } else {
          St<E>::load8(dy + off + c * 8, fd);
          St<E>::load8(x + off + c * 8, fx);
        }
        St<E>::load8(g + c * 8, fg);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xh = fx[i] * r;
          dot += fd[i] * fg[i] * xh;
          acc[k][i] += fd[i] * xh;
        }
      }
    }
    dot = wave_sum(dot) * inv_cols;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
      const int c = lane + 64 * k;
      if (c < nch) {
        float fd[8], fx[8], fg[8], fr[8];
        if constexpr (KEEP) {
          unpack8(kd[k], fd);
          unpack8(kx[k], fx);
        } else {
          St<E>::load8(dy + off + c * 8, fd);
          St<E>::load8(x + off + c * 8, fx);
        }
        St<E>::load8(g + c * 8, fg);
        if (resid) St<E>::load8(resid + off + c * 8, fr);
        else {
#pragma unroll
          for (int i = 0; i < 8; ++i) fr[i] = 0.f;
        }
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xh = fx[i] * r;
          o[i] = fr[i] + r * (fd[i] * fg[i] - xh * dot);
        }
        St<E>::store8(dx + off + c * 8, o);
      }
    }
  }
  // combine the four waves' column sums in fixed order
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int c = lane + 64 * k;
    if (c < nch)
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave * cols + c * 8 + i] = acc[k][i];
  }
  __syncthreads();
  for (int col = threadIdx.x; col < cols; col += 256) {
    const float s = ((red[col] + red[cols + col]) + red[2 * cols + col]) + red[3 * cols + col];
    dg_part[(long)blockIdx.x * cols + col] = s;
  }
}

// The same backward for rows wider than the register-held form allows (the
// pages' widest layers, hidden up to 16384): first each wave walks its rows
// computing the row's dot product and dx (two passes over the row), then
// the workgroup walks the columns in slabs of WIDE_SLAB, summing dy * xh
// over its rows per wave in row order (the rows are re-read, mostly from
// L2) and combining the 4 waves in the same fixed order as above.
constexpr int WIDE_SLAB = 4096;

template <class E>
__global__ __launch_bounds__(256) void rmsnorm_bwd_wide_kernel(
    const E* __restrict__ dy, const E* __restrict__ x, const E* __restrict__ g,
    const float* __restrict__ rstd, const E* __restrict__ resid, E* __restrict__ dx,
    float* __restrict__ dg_part, int rows, int cols) {
  extern __shared__ float red[];  // [4][WIDE_SLAB]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = cols / 8;
  const int r0 = blockIdx.x * RB_ROWS;
  const float inv_cols = 1.f / (float)cols;
  for (int rr = wave; rr < RB_ROWS; rr += 4) {
    const int row = r0 + rr;
    if (row >= rows) break;
    const long off = (long)row * cols;
    const float r = rstd[row];
    float dot = 0.f;
    for (int c = lane; c < nch; c += 64) {
      float fd[8], fx[8], fg[8];
      St<E>::load8(dy + off + c * 8, fd);
      St<E>::load8(x + off + c * 8, fx);
      St<E>::load8(g + c * 8, fg);
#pragma unroll
      for (int i = 0; i < 8; ++i) dot += fd[i] * fg[i] * (fx[i] * r);
    }
    dot = wave_sum(dot) * inv_cols;
    for (int c = lane; c < nch; c += 64) {
      float fd[8], fx[8], fg[8], fr[8];
      St<E>::load8(dy + off + c * 8, fd);
      St<E>::load8(x + off + c * 8, fx);
      St<E>::load8(g + c * 8, fg);
      if (resid) St<E>::load8(resid + off + c * 8, fr);
      else {
#pragma unroll
        for (int i = 0; i < 8; ++i) fr[i] = 0.f;
      }
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fr[i] + r * (fd[i] * fg[i] - (fx[i] * r) * dot);
      St<E>::store8(dx + off + c * 8, o);
    }
  }
  constexpr int SCH = WIDE_SLAB / 8, PER = SCH / 64;  // chunks per slab, per lane
  for (int s0 = 0; s0 < nch; s0 += SCH) {
    float acc[PER][8];
#pragma unroll
    for (int k = 0; k < PER; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[k][i] = 0.f;
    for (int rr = wave; rr < RB_ROWS; rr += 4) {
      const int row = r0 + rr;
      if (row >= rows) break;
      const long off = (long)row * cols;
      const float r = rstd[row];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int c = s0 + lane + 64 * k;
        if (c < nch) {
          float fd[8], fx[8];
          St<E>::load8(dy + off + c * 8, fd);
          St<E>::load8(x + off + c * 8, fx);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[k][i] += fd[i] * (fx[i] * r);
        }
      }
    }
    __syncthreads();  // the previous slab's combine has read red
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int c = lane + 64 * k;
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave * WIDE_SLAB + c * 8 + i] = acc[k][i];
    }
    __syncthreads();
    const int ncol = min(WIDE_SLAB, cols - s0 * 8);
    for (int col = threadIdx.x; col < ncol; col += 256) {
      const float s = ((red[col] + red[WIDE_SLAB + col]) + red[2 * WIDE_SLAB + col]) +
                      red[3 * WIDE_SLAB + col];
      dg_part[(long)blockIdx.x * cols + s0 * 8 + col] = s;
    }
  }
}

// out[col] = sum over the nblk partial rows.  A workgroup covers 64
// columns with 4 row groups (rows b = 4 i + q); each thread keeps 8 running
// sums (over i mod 8) so its loads stay independent; the sums are combined
// in a fixed order (the result does not depend on timing).
template <class E>
__global__ __launch_bounds__(256) void reduce_rows_kernel(const float* __restrict__ part, int nblk,
                                                          int cols, E* __restrict__ out) {
  __shared__ float red[4][64];
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + c;
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  if (col < cols) {
    int i = 0;
    for (; 4 * (i + 7) + q < nblk; i += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += part[(long)(4 * (i + u) + q) * cols + col];
#pragma unroll
    for (int u = 0; u < 7; ++u)
      if (4 * (i + u) + q < nblk) acc[u] += part[(long)(4 * (i + u) + q) * cols + col];
  }
  red[q][c] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (q == 0 && col < cols) St<E>::store(out + col, ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c]);
}

__global__ void rope_table_kernel(float* cos_t, float* sin_t, int seq, int half, int head_dim,
                                  double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= seq * half) return;
  const int t = idx / half, j = idx % half;
  const double inv = pow(theta, -2.0 * (double)j / (double)head_dim);
  const double ang = (double)t * inv;
  cos_t[idx] = (float)cos(ang);
  sin_t[idx] = (float)sin(ang);
}

// One thread per (token, head, 8 consecutive pairs j): rotates
// (x_j, x_{j+d/2}) with 16-byte accesses (half % 8 == 0).
template <class E>
__global__ void rope_kernel(E* __restrict__ qkv, long ldq, int tokens, int seq, int nh,
                            int half, const float* __restrict__ cos_t,
                            const float* __restrict__ sin_t, float sgn) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int h8 = half / 8;
  const long total = (long)tokens * nh * h8;
  if (idx >= total) return;
  const int j = 8 * (int)(idx % h8);
  const long th = idx / h8;
  const int h = (int)(th % nh);
  const int tok = (int)(th / nh);
  const int t = tok % seq;
  E* p = qkv + (long)tok * ldq + (long)h * 2 * half;
  float x1[8], x2[8], c[8], sn[8];
  St<E>::load8(p + j, x1);
  St<E>::load8(p + j + half, x2);
  St<float>::load8(cos_t + t * half + j, c);
  St<float>::load8(sin_t + t * half + j, sn);
  float o1[8], o2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float si = sgn * sn[i];
    o1[i] = x1[i] * c[i] - x2[i] * si;
    o2[i] = x2[i] * c[i] + x1[i] * si;
  }
  St<E>::store8(p + j, o1);
  St<E>::store8(p + j + half, o2);
}

// Cross-entropy over one row of fp32 logits per workgroup (256 threads):
// pass 1 online max/sum, pass 2 writes (softmax - onehot) * inv_n.
template <class E>
__global__ __launch_bounds__(256) void ce_rows_kernel(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ target,
                                                      E* __restrict__ dlogits,
                                                      float* __restrict__ loss_part, int vocab,
                                                      float inv_n) {
  __shared__ float sm[2][4];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* lr = logits + (long)row * vocab;
  E* dr = dlogits + (long)row * vocab;
  const int tgt = target[row];
  if (tgt < 0 || tgt >= vocab) {
    for (int c = tid * 4; c < vocab; c += 1024)
#pragma unroll
      for (int i = 0; i < 4; ++i) St<E>::store(dr + c + i, 0.f);
    if (tid == 0) loss_part[row] = 0.f;
    return;
  }
  float m = -INFINITY, s = 0.f;
  for (int c = tid * 4; c < vocab; c += 1024) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(lr + c);
    const float mv = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    const float nm = fmaxf(m, mv);
    s = s * __expf(m - nm) + __expf(v.x - nm) + __expf(v.y - nm) + __expf(v.z - nm) +
        __expf(v.w - nm);
    m = nm;
  }
  // combine (m, s) across the wave, then across waves
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(m, o, 64), os = __shfl_xor(s, o, 64);
    const float nm = fmaxf(m, om);
    s = (m == -INFINITY ? 0.f : s * __expf(m - nm)) + (om == -INFINITY ? 0.f : os * __expf(om - nm));
    m = nm;
  }
  if (lane == 0) { sm[0][wave] = m; sm[1][wave] = s; }
  __syncthreads();
  float M = fmaxf(fmaxf(sm[0][0], sm[0][1]), fmaxf(sm[0][2], sm[0][3]));
  float S = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) S += sm[1][w] * __expf(sm[0][w] - M);
  const float inv_s = 1.f / S;
  for (int c = tid * 4; c < vocab; c += 1024) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(lr + c);
    float p[4] = {__expf(v.x - M) * inv_s, __expf(v.y - M) * inv_s, __expf(v.z - M) * inv_s,
                  __expf(v.w - M) * inv_s};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c + i == tgt) p[i] -= 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) St<E>::store(dr + c + i, p[i] * inv_n);
  }
  if (tid == 0) loss_part[row] = (M + logf(S)) - lr[tgt];
}

// Fixed-order sum of n values by one workgroup: each thread sums a strided
// slice in index order, then a fixed tree over the 256 partials.
__global__ __launch_bounds__(256) void sum_kernel(const float* __restrict__ part, int n,
                                                  float scale, float* __restrict__ out) {
  __shared__ float sh[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) s += part[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = sh[0] * scale;
}

template <class E>
__global__ void cast_kernel(const float* __restrict__ in, E* __restrict__ out, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) St<E>::store(out + i, in[i]);
}

__global__ void fill_kernel(float* __restrict__ p, float v, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void copy_rows_kernel(const uint16_t* __restrict__ src, long lds,
                                 uint16_t* __restrict__ dst, long ldd, int rows, int cols8) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)rows * cols8) return;
  const int r = (int)(idx / cols8), c = (int)(idx % cols8);
  *reinterpret_cast<u32x4_t*>(dst + r * ldd + c * 8) =
      *reinterpret_cast<const u32x4_t*>(src + r * lds + c * 8);
}

// One flag per workgroup: any Inf/NaN in its strided share of the buffer
// (bf16: exponent bits all ones; fp32 likewise), OR-reduced over the
// workgroup through LDS.
__global__ __launch_bounds__(256) void nonfinite_kernel(const u32x4_t* __restrict__ g, size_t n16,
                                                        int f32, int32_t* __restrict__ flags,
                                                        float* __restrict__ ssq) {
  __shared__ int any;
  __shared__ float part[4];
  if (threadIdx.x == 0) any = 0;
  __syncthreads();
  uint32_t bad = 0;
  float sq = 0.f;  // this lane's sum of squares (the gradient-norm share)
  const uint32_t em = f32 ? 0x7F800000u : 0x7F807F80u;  // exponent masks per dword
  auto check = [&](const u32x4_t v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t x = v[k] & em;
      if (f32) {
        bad |= (x == 0x7F800000u);
        const float f = __uint_as_float(v[k]);
        sq += f * f;
      } else {
        bad |= ((x & 0xFFFFu) == 0x7F80u) | ((x >> 16) == 0x7F80u);
        const float lo = __uint_as_float(v[k] << 16), hi = __uint_as_float(v[k] & 0xFFFF0000u);
        sq += lo * lo;
        sq += hi * hi;
      }
    }
  };
  // four independent 16-byte loads in flight per lane per trip
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = g[i], b = g[i + stride], c = g[i + 2 * stride], d = g[i + 3 * stride];
    check(a);
    check(b);
    check(c);
    check(d);
  }
  for (; i < n16; i += stride) check(g[i]);
  if (bad) any = 1;  // benign race: every writer stores 1
  if (ssq) {
    // the workgroup's sum of squares in a fixed order: lanes, then waves
    sq = wave_sum(sq);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    flags[blockIdx.x] = any;
    if (ssq) ssq[blockIdx.x] = ((part[0] + part[1]) + part[2]) + part[3];
  }
}

}  // namespace

namespace {
template <class E>
hipError_t rmsnorm_fwd_t(const E* x, const E* g, E* y, float* rstd, int rows, int cols, float eps,
                         hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_fwd_kernel<E>, dim3((rows + RN_WAVES - 1) / RN_WAVES),
                     dim3(RN_WAVES * 64), 0, s, x, g, y, rstd, rows, cols, eps);
  return hipGetLastError();
}

template <class E>
hipError_t rmsnorm_bwd_t(const E* dy, const E* x, const E* g, const float* rstd, const E* resid,
                         E* dx, float* dg_part, int rows, int cols, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nch = cols / 8;
  const int iters = (nch + 63) / 64;
  const dim3 grid(rmsnorm_bwd_blocks(rows)), block(256);
  const size_t lds = 4 * (size_t)cols * sizeof(float);
#define MT_RB(C)                                                                           \
  if (iters <= C) {                                                                        \
    static bool attr = false;                                                              \
    if (!attr) {                                                                           \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(rmsnorm_bwd_kernel<E, C>), \
                                         hipFuncAttributeMaxDynamicSharedMemorySize,       \
                                         4 * 8192 * (int)sizeof(float));                   \
      if (e != hipSuccess) return e;                                                       \
      attr = true;                                                                         \
    }                                                                                      \
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<E, C>), grid, block, lds, s, dy, x, g, rstd, resid, dx, \
                       dg_part, rows, cols);                                               \
    return hipGetLastError();                                                              \
  }
  MT_RB(1) MT_RB(2) MT_RB(4) MT_RB(8) MT_RB(16)
#undef MT_RB
  if (cols > RMSNORM_MAX_COLS) return hipErrorInvalidValue;
  static bool attr = false;
  constexpr int lds_w = 4 * WIDE_SLAB * (int)sizeof(float);
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(rmsnorm_bwd_wide_kernel<E>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_w);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(rmsnorm_bwd_wide_kernel<E>, grid, block, lds_w, s, dy, x, g, rstd, resid, dx,
                     dg_part, rows, cols);
  return hipGetLastError();
}

template <class E>
hipError_t reduce_rows_t(const float* part, int nblk, int cols, E* out, hipStream_t s) {
  hipLaunchKernelGGL(reduce_rows_kernel<E>, dim3((cols + 63) / 64), dim3(256), 0, s, part, nblk,
                     cols, out);
  return hipGetLastError();
}

template <class E>
hipError_t rope_apply_t(E* qkv, long ldq, int batch, int seq, int n_heads, int n_kv_heads,
                        int head_dim, const float* cos_t, const float* sin_t, int inverse,
                        hipStream_t s) {
  const int tokens = batch * seq, nh = n_heads + n_kv_heads, half = head_dim / 2;
  if (half % 8) return hipErrorInvalidValue;
  const long total = (long)tokens * nh * (half / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_kernel<E>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, qkv,
                     ldq, tokens, seq, nh, half, cos_t, sin_t, inverse ? -1.f : 1.f);
  return hipGetLastError();
}

template <class E>
hipError_t ce_rows_t(const float* logits, const int32_t* target, E* dlogits, float* loss_part,
                     int rows, int vocab, float inv_n, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_rows_kernel<E>, dim3(rows), dim3(256), 0, s, logits, target, dlogits,
                     loss_part, vocab, inv_n);
  return hipGetLastError();
}

template <class E>
hipError_t cast_t(const float* in, E* out, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(cast_kernel<E>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}
}  // namespace

int rmsnorm_bwd_blocks(int rows) { return (rows + RB_ROWS - 1) / RB_ROWS; }

hipError_t nonfinite_flags(const void* g, size_t bytes, int f32, int32_t* flags, hipStream_t s,
                           float* ssq) {
  if (bytes & 15) return hipErrorInvalidValue;
  hipLaunchKernelGGL(nonfinite_kernel, dim3(NONFINITE_BLOCKS), dim3(256), 0, s,
                     static_cast<const u32x4_t*>(g), bytes / 16, f32, flags, ssq);
  return hipGetLastError();
}

hipError_t rmsnorm_fwd(const uint16_t* x, const uint16_t* g, uint16_t* y, float* rstd, int rows,
                       int cols, float eps, hipStream_t s) {
  return rmsnorm_fwd_t(x, g, y, rstd, rows, cols, eps, s);
}
hipError_t rmsnorm_fwd(const float* x, const float* g, float* y, float* rstd, int rows, int cols,
                       float eps, hipStream_t s) {
  return rmsnorm_fwd_t(x, g, y, rstd, rows, cols, eps, s);
}
hipError_t rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* g,
                       const float* rstd, const uint16_t* resid, uint16_t* dx, float* dg_part,
                       int rows, int cols, hipStream_t s) {
  return rmsnorm_bwd_t(dy, x, g, rstd, resid, dx, dg_part, rows, cols, s);
}
hipError_t rmsnorm_bwd(const float* dy, const float* x, const float* g, const float* rstd,
                       const float* resid, float* dx, float* dg_part, int rows, int cols,
                       hipStream_t s) {
  return rmsnorm_bwd_t(dy, x, g, rstd, resid, dx, dg_part, rows, cols, s);
}
hipError_t reduce_rows(const float* part, int nblk, int cols, uint16_t* out, hipStream_t s) {
  return reduce_rows_t(part, nblk, cols, out, s);
}
hipError_t reduce_rows(const float* part, int nblk, int cols, float* out, hipStream_t s) {
  return reduce_rows_t(part, nblk, cols, out, s);
}
hipError_t rope_apply(uint16_t* qkv, long ldq, int batch, int seq, int n_heads, int n_kv_heads,
                      int head_dim, const float* cos_t, const float* sin_t, int inverse,
                      hipStream_t s) {
  return rope_apply_t(qkv, ldq, batch, seq, n_heads, n_kv_heads, head_dim, cos_t, sin_t, inverse,
                      s);
}
hipError_t rope_apply(float* qkv, long ldq, int batch, int seq, int n_heads, int n_kv_heads,
                      int head_dim, const float* cos_t, const float* sin_t, int inverse,
                      hipStream_t s) {
  return rope_apply_t(qkv, ldq, batch, seq, n_heads, n_kv_heads, head_dim, cos_t, sin_t, inverse,
                      s);
}
hipError_t ce_rows(const float* logits, const int32_t* target, uint16_t* dlogits,
                   float* loss_part, int rows, int vocab, float inv_n, hipStream_t s) {
  return ce_rows_t(logits, target, dlogits, loss_part, rows, vocab, inv_n, s);
}
hipError_t ce_rows(const float* logits, const int32_t* target, float* dlogits, float* loss_part,
                   int rows, int vocab, float inv_n, hipStream_t s) {
  return ce_rows_t(logits, target, dlogits, loss_part, rows, vocab, inv_n, s);
}
hipError_t cast_f32(const float* in, uint16_t* out, size_t n, hipStream_t s) {
  return cast_t(in, out, n, s);
}
hipError_t cast_f32(const float* in, float* out, size_t n, hipStream_t s) {
  return cast_t(in, out, n, s);
}

hipError_t rope_table(float* cos_t, float* sin_t, int seq, int head_dim, double theta,
                      hipStream_t s) {
  const int half = head_dim / 2, n = seq * half;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cos_t, sin_t, seq,
                     half, head_dim, theta);
  return hipGetLastError();
}



hipError_t sum_loss(const float* part, int n, float inv_n, float* out, hipStream_t s) {
  hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(256), 0, s, part, n, inv_n, out);
  return hipGetLastError();
}


hipError_t fill_f32(float* p, float v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t copy_rows_bf16(const uint16_t* src, long lds, uint16_t* dst, long ldd, int rows,
                          int cols, hipStream_t s) {
  const long total = (long)rows * (cols / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src,
                     lds, dst, ldd, rows, cols / 8);
  return hipGetLastError();
}

}  // namespace mt
