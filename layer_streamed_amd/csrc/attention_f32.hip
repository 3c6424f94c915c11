// fp32-storage causal GQA attention for the debug precision.  Same contract
// as the bf16 flash kernels (q/k/v inside qkv [B*T, (Hq + 2 Hkv) d], o
// [B*T, Hq d], lse [B, Hq, T], dqkv in the qkv layout), written for exact
// fp32 arithmetic rather than speed: one wave64 per query row (forward,
// dq) or key row (dk, dv); lane l holds head-dim elements l and l + 64; dot
// products are a register FMA plus one wave butterfly; exp and log are the
// accurate library functions.
//
// Backward (S = q k^T / sqrt(d), P = exp(S - lse), delta = rowsum(dO o)):
//   dP = dO v^T;  dS = P (dP - delta);  dq = dS k / sqrt(d)
//   dk = sum over the GQA group and t >= s of dS q / sqrt(d);  dv = ... P dO
// The dq kernel also writes delta, which the dk/dv kernel then reads, so no
// atomics are needed and the result is deterministic.
#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

constexpr int AW = 4;  // waves (rows) per workgroup

struct Geo {
  int B, T, Hq, Hkv, d, G;  // G = Hq / Hkv
  long ld;                  // qkv row stride
  int Qd, Kvd;
  float scale;
};

template <int NE>
__device__ __forceinline__ void load_row(const float* p, int lane, float (&v)[NE]) {
#pragma unroll
  for (int i = 0; i < NE; ++i) v[i] = p[lane + 64 * i];
}
template <int NE>
__device__ __forceinline__ float dot_row(const float (&a)[NE], const float* p, int lane) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) s = fmaf(a[i], p[lane + 64 * i], s);
  return wave_sum(s);
}

template <int NE>
__global__ __launch_bounds__(AW * 64) void attn_fwd_f32_kernel(const float* __restrict__ qkv,
                                                               float* __restrict__ o,
                                                               float* __restrict__ lse, Geo g) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * AW + (threadIdx.x >> 6);  // (b, h, t) with t fastest
  if (w >= (long)g.B * g.Hq * g.T) return;
  const int t = (int)(w % g.T), h = (int)((w / g.T) % g.Hq), b = (int)(w / ((long)g.T * g.Hq));
  const int kvh = h / g.G;
  const long tok = (long)b * g.T + t;
  float q[NE], acc[NE];
  load_row<NE>(qkv + tok * g.ld + (long)h * g.d, lane, q);
#pragma unroll
  for (int i = 0; i < NE; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float* kbase = qkv + (long)b * g.T * g.ld + g.Qd + (long)kvh * g.d;
  const float* vbase = kbase + g.Kvd;
  for (int s = 0; s <= t; ++s) {
    const float sc = dot_row<NE>(q, kbase + (long)s * g.ld, lane) * g.scale;
    const float nm = fmaxf(m, sc);
    const float corr = expf(m - nm);  // 0 on the first key (m = -inf)
    const float p = expf(sc - nm);
    l = l * corr + p;
    const float* vr = vbase + (long)s * g.ld;
#pragma unroll
    for (int i = 0; i < NE; ++i) acc[i] = fmaf(p, vr[lane + 64 * i], acc[i] * corr);
    m = nm;
  }
  const float inv = 1.f / l;
  float* orow = o + tok * (long)g.Qd + (long)h * g.d;
#pragma unroll
  for (int i = 0; i < NE; ++i) orow[lane + 64 * i] = acc[i] * inv;
  if (lane == 0) lse[((long)b * g.Hq + h) * g.T + t] = m + logf(l);
}

template <int NE>
__global__ __launch_bounds__(AW * 64) void attn_dq_f32_kernel(
    const float* __restrict__ qkv, const float* __restrict__ o, const float* __restrict__ lse,
    const float* __restrict__ dout, float* __restrict__ delta, float* __restrict__ dqkv, Geo g) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * AW + (threadIdx.x >> 6);
  if (w >= (long)g.B * g.Hq * g.T) return;
  const int t = (int)(w % g.T), h = (int)((w / g.T) % g.Hq), b = (int)(w / ((long)g.T * g.Hq));
  const int kvh = h / g.G;
  const long tok = (long)b * g.T + t;
  float q[NE], dO[NE], dq[NE];
  load_row<NE>(qkv + tok * g.ld + (long)h * g.d, lane, q);
  load_row<NE>(dout + tok * (long)g.Qd + (long)h * g.d, lane, dO);
  const float dl = dot_row<NE>(dO, o + tok * (long)g.Qd + (long)h * g.d, lane);
  const long hr = ((long)b * g.Hq + h) * g.T + t;
  if (lane == 0) delta[hr] = dl;
  const float L = lse[hr];
#pragma unroll
  for (int i = 0; i < NE; ++i) dq[i] = 0.f;
  const float* kbase = qkv + (long)b * g.T * g.ld + g.Qd + (long)kvh * g.d;
  const float* vbase = kbase + g.Kvd;
  for (int s = 0; s <= t; ++s) {
    const float* kr = kbase + (long)s * g.ld;
    const float p = expf(dot_row<NE>(q, kr, lane) * g.scale - L);
    const float dp = dot_row<NE>(dO, vbase + (long)s * g.ld, lane);
    const float ds = p * (dp - dl);
#pragma unroll
    for (int i = 0; i < NE; ++i) dq[i] = fmaf(ds, kr[lane + 64 * i], dq[i]);
  }
  float* dqr = dqkv + tok * g.ld + (long)h * g.d;
#pragma unroll
  for (int i = 0; i < NE; ++i) dqr[lane + 64 * i] = dq[i] * g.scale;
}

template <int NE>
__global__ __launch_bounds__(AW * 64) void attn_dkdv_f32_kernel(
    const float* __restrict__ qkv, const float* __restrict__ lse, const float* __restrict__ dout,
    const float* __restrict__ delta, float* __restrict__ dqkv, Geo g) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * AW + (threadIdx.x >> 6);  // (b, kvh, s)
  if (w >= (long)g.B * g.Hkv * g.T) return;
  const int s = (int)(w % g.T), kvh = (int)((w / g.T) % g.Hkv), b = (int)(w / ((long)g.T * g.Hkv));
  const long tok_s = (long)b * g.T + s;
  float k[NE], v[NE], dk[NE], dv[NE];
  load_row<NE>(qkv + tok_s * g.ld + g.Qd + (long)kvh * g.d, lane, k);
  load_row<NE>(qkv + tok_s * g.ld + g.Qd + g.Kvd + (long)kvh * g.d, lane, v);
#pragma unroll
  for (int i = 0; i < NE; ++i) dk[i] = dv[i] = 0.f;
  for (int h = kvh * g.G; h < (kvh + 1) * g.G; ++h) {
    const long hr0 = ((long)b * g.Hq + h) * g.T;
    for (int t = s; t < g.T; ++t) {
      const long tok = (long)b * g.T + t;
      const float* qr = qkv + tok * g.ld + (long)h * g.d;
      const float* dr = dout + tok * (long)g.Qd + (long)h * g.d;
      const float p = expf(dot_row<NE>(k, qr, lane) * g.scale - lse[hr0 + t]);
      const float dp = dot_row<NE>(v, dr, lane);
      const float ds = p * (dp - delta[hr0 + t]);
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        dv[i] = fmaf(p, dr[lane + 64 * i], dv[i]);
        dk[i] = fmaf(ds, qr[lane + 64 * i], dk[i]);
      }
    }
  }
  float* dkr = dqkv + tok_s * g.ld + g.Qd + (long)kvh * g.d;
  float* dvr = dkr + g.Kvd;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    dkr[lane + 64 * i] = dk[i] * g.scale;
    dvr[lane + 64 * i] = dv[i];
  }
}

Geo make_geo(int batch, int seq, int n_heads, int n_kv_heads, int head_dim) {
  Geo g;
  g.B = batch;
  g.T = seq;
  g.Hq = n_heads;
  g.Hkv = n_kv_heads;
  g.d = head_dim;
  g.G = n_heads / n_kv_heads;
  g.Qd = n_heads * head_dim;
  g.Kvd = n_kv_heads * head_dim;
  g.ld = g.Qd + 2L * g.Kvd;
  g.scale = 1.f / sqrtf((float)head_dim);
  return g;
}

bool geo_ok(const Geo& g) {
  return g.B >= 0 && g.T >= 0 && g.Hq > 0 && g.Hkv > 0 && g.Hq % g.Hkv == 0 &&
         (g.d == 64 || g.d == 128);
}

dim3 rows_grid(long rows) { return dim3((unsigned)((rows + AW - 1) / AW)); }

}  // namespace

hipError_t attn_fwd(const float* qkv, float* o, float* lse, int batch, int seq, int n_heads,
                    int n_kv_heads, int head_dim, hipStream_t s) {
  const Geo g = make_geo(batch, seq, n_heads, n_kv_heads, head_dim);
  if (!geo_ok(g)) return hipErrorInvalidValue;
  const long rows = (long)batch * n_heads * seq;
  if (rows == 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<1>, rows_grid(rows), dim3(AW * 64), 0, s, qkv, o, lse, g);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<2>, rows_grid(rows), dim3(AW * 64), 0, s, qkv, o, lse, g);
  return hipGetLastError();
}

hipError_t attn_bwd(const float* qkv, const float* o, const float* lse, const float* dout,
                    float* delta, float* dqkv, int batch, int seq, int n_heads, int n_kv_heads,
                    int head_dim, hipStream_t s) {
  const Geo g = make_geo(batch, seq, n_heads, n_kv_heads, head_dim);
  if (!geo_ok(g)) return hipErrorInvalidValue;
  const long qrows = (long)batch * n_heads * seq, krows = (long)batch * n_kv_heads * seq;
  if (qrows == 0) return hipSuccess;
  if (head_dim == 64) {
    hipLaunchKernelGGL(attn_dq_f32_kernel<1>, rows_grid(qrows), dim3(AW * 64), 0, s, qkv, o, lse,
                       dout, delta, dqkv, g);
    hipLaunchKernelGGL(attn_dkdv_f32_kernel<1>, rows_grid(krows), dim3(AW * 64), 0, s, qkv, lse,
                       dout, delta, dqkv, g);
  } else {
    hipLaunchKernelGGL(attn_dq_f32_kernel<2>, rows_grid(qrows), dim3(AW * 64), 0, s, qkv, o, lse,
                       dout, delta, dqkv, g);
    hipLaunchKernelGGL(attn_dkdv_f32_kernel<2>, rows_grid(krows), dim3(AW * 64), 0, s, qkv, lse,
                       dout, delta, dqkv, g);
  }
  return hipGetLastError();
}

}  // namespace mt
