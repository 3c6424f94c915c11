// Hybrid 8-bit Adam on the host (LazyTrain abstract, on the listing pages:
// 8-bit optimizer states coupled with fast gradient clipping in one
// operator).  The page fixes no format; this is the build's reading:
//  - each moment is kept per tensor in blocks of ADAM8_BLOCK consecutive
//    elements (a tensor's last block may be shorter) as OCP FP8 E4M3 codes
//    (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
//    infinities, largest finite 448) with one fp32 scale per block:
//    scale = absmax / 448, code = E4M3(x * (448 / absmax)) rounded to
//    nearest even (saturating at 448), value = E4M3value(code) * scale;
//  - the first moment m is stored as is, the second moment v as r = sqrt(v);
//  - the update is the fp32 Adam of host.cpp computed from the dequantized
//    old moments and the gradient times the clipping factor, and the new
//    moments are quantized afterwards; the fp32 master stays fp32.
// Compiled with -ffp-contract=off: every fp32 operation is rounded as
// written, so the scalar, AVX2 and AVX-512 paths agree bit for bit with a
// plain fp32 evaluation of the same operations.
#include <immintrin.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "host.h"

namespace mt {

namespace {

// E4M3 values from the format's definition: E > 0: 2^(E-7) (1 + M/8);
// E = 0: 2^-6 M / 8 (E = 15, M = 7, the NaN code, is never produced).
struct E4M3Table {
  float v[256];
  E4M3Table() {
    for (int c = 0; c < 256; ++c) {
      const int E = (c >> 3) & 15, M = c & 7;
      const double mag = E ? ldexp(1.0 + M / 8.0, E - 7) : ldexp(M / 8.0, -6);
      v[c] = (float)((c & 0x80) ? -mag : mag);
    }
  }
};
const E4M3Table kE4M3;

inline uint32_t fbits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

}  // namespace

float e4m3_decode(uint8_t c) { return kE4M3.v[c]; }

// Round to nearest even on the exact value.  At or above 2^-6 (a normal
// E4M3 value) the fp32 mantissa is rounded to 3 bits by adding half an E4M3
// step (minus one, plus the kept lowest bit) and truncating; a carry moves
// into the exponent.  Below 2^-6 the value is a multiple of 2^-9: y * 2^9
// is exact and converts with round-to-nearest-even (code 8 is 2^-6, the
// smallest normal).  Magnitudes above 448 saturate.
uint8_t e4m3_encode(float y) {
  const uint32_t u = fbits(y), a = u & 0x7FFFFFFFu, s = (u >> 24) & 0x80u;
  uint32_t code;
  if (a >= 0x3C800000u) {
    const int32_t t = (int32_t)((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - 960;
    code = (uint32_t)std::min(t, 0x7E);
  } else {
    code = (uint32_t)lrintf(fabsf(y) * 512.f);  // default rounding: nearest even
  }
  return (uint8_t)(code | s);
}

namespace {

// Quantize n <= ADAM8_BLOCK fp32 values into codes with one scale.
inline float quant_block(const float* x, int n, uint8_t* code) {
  float amax = 0.f;
  for (int i = 0; i < n; ++i) amax = std::max(amax, fabsf(x[i]));
  if (amax == 0.f) {
    for (int i = 0; i < n; ++i) code[i] = 0;
    return 0.f;
  }
  const float inv = 448.f / amax;
  for (int i = 0; i < n; ++i) code[i] = e4m3_encode(x[i] * inv);
  return amax / 448.f;
}

// One block, scalar: the reference evaluation of the update.
template <bool BF16_GRAD, int SHADOW>
void adam8_block_scalar(const Adam8Arrays& A, size_t off, int n, size_t b, const AdamHp& h,
                        float clip) {
  float mb[ADAM8_BLOCK], rb[ADAM8_BLOCK];
  const float ms = A.ms[b], rs = A.rs[b];
  for (int i = 0; i < n; ++i) {
    const size_t k = off + i;
    float g;
    if constexpr (BF16_GRAD) g = host_bf2f(A.gb[k]);
    else g = A.gf[k];
    g = g * clip;
    const float m_old = kE4M3.v[A.mq[k]] * ms;
    const float r_old = kE4M3.v[A.rq[k]] * rs;
    const float v_old = r_old * r_old;
    const float m = h.b1 * m_old + h.omb1 * g;
    const float v = h.b2 * v_old + h.omb2 * (g * g);
    const float mh = m / h.bc1;
    const float vh = v / h.bc2;
    const float p = A.p[k] - h.lr * mh / (sqrtf(vh) + h.eps);
    A.p[k] = p;
    if constexpr (SHADOW == 1) A.sb[k] = host_f2bf(p);
    else if constexpr (SHADOW == 2) A.sf[k] = p;
    mb[i] = m;
    rb[i] = sqrtf(v);
  }
  A.ms[b] = quant_block(mb, n, A.mq + off);
  A.rs[b] = quant_block(rb, n, A.rq + off);
}

// ---- vector forms of one full block: the same operations in the same order
// as adam8_block_scalar, so every form gives the scalar one's bits.

// fp32 -> bf16 bits, round to nearest even, NaN -> quiet NaN with the sign
inline __m256i bf16_bits8(__m256 p) {
  const __m256i u = _mm256_castps_si256(p);
  const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(1));
  const __m256i rn =
      _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, _mm256_set1_epi32(0x7FFF)), lsb), 16);
  const __m256i qn = _mm256_or_si256(
      _mm256_and_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(0x8000)),
      _mm256_set1_epi32(0x7FC0));
  const __m256i isnan = _mm256_cmpgt_epi32(_mm256_and_si256(u, _mm256_set1_epi32(0x7FFFFFFF)),
                                           _mm256_set1_epi32(0x7F800000));
  return _mm256_blendv_epi8(rn, qn, isnan);
}

// E4M3 of 8 fp32 lanes (the same decision as e4m3_encode), as 8 x 32-bit.
inline __m256i enc8(__m256 y) {
  const __m256i u = _mm256_castps_si256(y);
  const __m256i a = _mm256_and_si256(u, _mm256_set1_epi32(0x7FFFFFFF));
  const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(a, 20), _mm256_set1_epi32(1));
  __m256i tn = _mm256_sub_epi32(
      _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(a, _mm256_set1_epi32(0x7FFFF)), lsb), 20),
      _mm256_set1_epi32(960));
  tn = _mm256_min_epi32(tn, _mm256_set1_epi32(0x7E));
  const __m256 ay = _mm256_castsi256_ps(a);
  const __m256i ts = _mm256_cvtps_epi32(_mm256_mul_ps(ay, _mm256_set1_ps(512.f)));
  // a >= 0x3C800000 <=> a > 0x3C7FFFFF (a is non-negative as int32)
  const __m256i normal = _mm256_cmpgt_epi32(a, _mm256_set1_epi32(0x3C7FFFFF));
  const __m256i code = _mm256_blendv_epi8(ts, tn, normal);
  return _mm256_or_si256(code, _mm256_and_si256(_mm256_srli_epi32(u, 24), _mm256_set1_epi32(0x80)));
}

// Values of 8 codes (8 bytes) times a scale, decoded arithmetically: a
// normal code is the fp32 pattern sign | (E + 120) << 23 | M << 20; a
// subnormal one (E = 0) is M * 2^-9 (exact), with the sign.
inline __m256 dec8(const uint8_t* c, __m256 scale) {
  const __m256i k = _mm256_cvtepu8_epi32(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(c)));
  const __m256i sign = _mm256_slli_epi32(_mm256_and_si256(k, _mm256_set1_epi32(0x80)), 24);
  const __m256i em = _mm256_and_si256(k, _mm256_set1_epi32(0x7F));
  const __m256i nrm = _mm256_add_epi32(_mm256_slli_epi32(em, 20), _mm256_set1_epi32(120 << 23));
  const __m256 sub = _mm256_mul_ps(_mm256_cvtepi32_ps(em), _mm256_set1_ps(1.f / 512.f));
  const __m256i is_sub = _mm256_cmpgt_epi32(_mm256_set1_epi32(8), em);
  const __m256i mag = _mm256_blendv_epi8(nrm, _mm256_castps_si256(sub), is_sub);
  return _mm256_mul_ps(_mm256_castsi256_ps(_mm256_or_si256(mag, sign)), scale);
}

// 8 x 32-bit values (each < 65536) -> 8 x 16-bit, and (each < 256) -> 8 bytes
inline __m128i narrow16(__m256i c) {
  return _mm_packus_epi32(_mm256_castsi256_si128(c), _mm256_extracti128_si256(c, 1));
}
inline void store8codes(uint8_t* dst, __m256i c) {
  const __m128i w = narrow16(c);
  _mm_storel_epi64(reinterpret_cast<__m128i*>(dst), _mm_packus_epi16(w, w));
}

// Scale of a block from its largest magnitude, and the factor that maps the
// block onto [-448, 448] (0 for an all-zero block: every code is then 0).
inline float block_scale(float amax) { return amax == 0.f ? 0.f : amax / 448.f; }
inline float block_factor(float amax) { return amax == 0.f ? 0.f : 448.f / amax; }

// One full block with 8-wide AVX2.
template <bool BF16_GRAD, int SHADOW>
void adam8_block_avx2(const Adam8Arrays& A, size_t off, size_t b, const AdamHp& h, float clip) {
  alignas(32) float mb[ADAM8_BLOCK], rb[ADAM8_BLOCK];
  const __m256 b1 = _mm256_set1_ps(h.b1), omb1 = _mm256_set1_ps(h.omb1);
  const __m256 b2 = _mm256_set1_ps(h.b2), omb2 = _mm256_set1_ps(h.omb2);
  const __m256 bc1 = _mm256_set1_ps(h.bc1), bc2 = _mm256_set1_ps(h.bc2);
  const __m256 lr = _mm256_set1_ps(h.lr), eps = _mm256_set1_ps(h.eps);
  const __m256 cl = _mm256_set1_ps(clip);
  const __m256 ms = _mm256_set1_ps(A.ms[b]), rs = _mm256_set1_ps(A.rs[b]);
  const __m256 absf = _mm256_castsi256_ps(_mm256_set1_epi32(0x7FFFFFFF));
  __m256 am = _mm256_setzero_ps(), ar = _mm256_setzero_ps();
  for (int j = 0; j < ADAM8_BLOCK; j += 8) {
    const size_t k = off + j;
    __m256 g;
    if constexpr (BF16_GRAD) {
      const __m128i g16 = _mm_loadu_si128(reinterpret_cast<const __m128i*>(A.gb + k));
      g = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(g16), 16));
    } else {
      g = _mm256_loadu_ps(A.gf + k);
    }
    g = _mm256_mul_ps(g, cl);
    const __m256 m_old = dec8(A.mq + k, ms);
    const __m256 r_old = dec8(A.rq + k, rs);
    const __m256 v_old = _mm256_mul_ps(r_old, r_old);
    const __m256 m = _mm256_add_ps(_mm256_mul_ps(b1, m_old), _mm256_mul_ps(omb1, g));
    const __m256 v = _mm256_add_ps(_mm256_mul_ps(b2, v_old), _mm256_mul_ps(omb2, _mm256_mul_ps(g, g)));
    const __m256 mh = _mm256_div_ps(m, bc1);
    const __m256 vh = _mm256_div_ps(v, bc2);
    const __m256 p = _mm256_sub_ps(
        _mm256_loadu_ps(A.p + k),
        _mm256_div_ps(_mm256_mul_ps(lr, mh), _mm256_add_ps(_mm256_sqrt_ps(vh), eps)));
    _mm256_storeu_ps(A.p + k, p);
    if constexpr (SHADOW == 1)
      _mm_storeu_si128(reinterpret_cast<__m128i*>(A.sb + k), narrow16(bf16_bits8(p)));
    else if constexpr (SHADOW == 2)
      _mm256_storeu_ps(A.sf + k, p);
    const __m256 r = _mm256_sqrt_ps(v);
    _mm256_store_ps(mb + j, m);
    _mm256_store_ps(rb + j, r);
    am = _mm256_max_ps(am, _mm256_and_ps(m, absf));
    ar = _mm256_max_ps(ar, r);
  }
  // horizontal maxima (max is exact: the order does not matter)
  alignas(32) float t[8];
  _mm256_store_ps(t, am);
  float amax_m = 0.f;
  for (int i = 0; i < 8; ++i) amax_m = std::max(amax_m, t[i]);
  _mm256_store_ps(t, ar);
  float amax_r = 0.f;
  for (int i = 0; i < 8; ++i) amax_r = std::max(amax_r, t[i]);
  A.ms[b] = block_scale(amax_m);
  A.rs[b] = block_scale(amax_r);
  const __m256 im = _mm256_set1_ps(block_factor(amax_m));
  const __m256 ir = _mm256_set1_ps(block_factor(amax_r));
  for (int j = 0; j < ADAM8_BLOCK; j += 8) {
    const size_t k = off + j;
    store8codes(A.mq + k, enc8(_mm256_mul_ps(_mm256_load_ps(mb + j), im)));
    store8codes(A.rq + k, enc8(_mm256_mul_ps(_mm256_load_ps(rb + j), ir)));
  }
}

// ---- 16-wide AVX-512 (chosen at run time where the CPU has it): the
// block's new moments stay in registers between the update and the
// quantization.
#define MT_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx512dq")))

MT_AVX512 inline __m512i bf16_bits16(__m512 p) {
  const __m512i u = _mm512_castps_si512(p);
  const __m512i lsb = _mm512_and_si512(_mm512_srli_epi32(u, 16), _mm512_set1_epi32(1));
  const __m512i rn =
      _mm512_srli_epi32(_mm512_add_epi32(_mm512_add_epi32(u, _mm512_set1_epi32(0x7FFF)), lsb), 16);
  const __m512i qn = _mm512_or_si512(
      _mm512_and_si512(_mm512_srli_epi32(u, 16), _mm512_set1_epi32(0x8000)),
      _mm512_set1_epi32(0x7FC0));
  const __mmask16 isnan = _mm512_cmpgt_epi32_mask(
      _mm512_and_si512(u, _mm512_set1_epi32(0x7FFFFFFF)), _mm512_set1_epi32(0x7F800000));
  return _mm512_mask_blend_epi32(isnan, rn, qn);
}

MT_AVX512 inline __m512i enc16(__m512 y) {
  const __m512i u = _mm512_castps_si512(y);
  const __m512i a = _mm512_and_si512(u, _mm512_set1_epi32(0x7FFFFFFF));
  const __m512i lsb = _mm512_and_si512(_mm512_srli_epi32(a, 20), _mm512_set1_epi32(1));
  __m512i tn = _mm512_sub_epi32(
      _mm512_srli_epi32(_mm512_add_epi32(_mm512_add_epi32(a, _mm512_set1_epi32(0x7FFFF)), lsb), 20),
      _mm512_set1_epi32(960));
  tn = _mm512_min_epi32(tn, _mm512_set1_epi32(0x7E));
  const __m512i ts = _mm512_cvtps_epi32(_mm512_mul_ps(_mm512_castsi512_ps(a), _mm512_set1_ps(512.f)));
  const __mmask16 normal = _mm512_cmpgt_epi32_mask(a, _mm512_set1_epi32(0x3C7FFFFF));
  const __m512i code = _mm512_mask_blend_epi32(normal, ts, tn);
  return _mm512_or_si512(code, _mm512_and_si512(_mm512_srli_epi32(u, 24), _mm512_set1_epi32(0x80)));
}

MT_AVX512 inline __m512 dec16(const uint8_t* c, __m512 scale) {
  const __m512i k = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(c)));
  const __m512i sign = _mm512_slli_epi32(_mm512_and_si512(k, _mm512_set1_epi32(0x80)), 24);
  const __m512i em = _mm512_and_si512(k, _mm512_set1_epi32(0x7F));
  const __m512i nrm = _mm512_add_epi32(_mm512_slli_epi32(em, 20), _mm512_set1_epi32(120 << 23));
  const __m512 sub = _mm512_mul_ps(_mm512_cvtepi32_ps(em), _mm512_set1_ps(1.f / 512.f));
  const __mmask16 is_sub = _mm512_cmpgt_epi32_mask(_mm512_set1_epi32(8), em);
  const __m512i mag = _mm512_mask_blend_epi32(is_sub, nrm, _mm512_castps_si512(sub));
  return _mm512_mul_ps(_mm512_castsi512_ps(_mm512_or_si512(mag, sign)), scale);
}

template <bool BF16_GRAD, int SHADOW>
MT_AVX512 void adam8_block_avx512(const Adam8Arrays& A, size_t off, size_t b, const AdamHp& h,
                                  float clip) {
  constexpr int NV = ADAM8_BLOCK / 16;
  __m512 mv[NV], rv[NV];
  const __m512 b1 = _mm512_set1_ps(h.b1), omb1 = _mm512_set1_ps(h.omb1);
  const __m512 b2 = _mm512_set1_ps(h.b2), omb2 = _mm512_set1_ps(h.omb2);
  const __m512 bc1 = _mm512_set1_ps(h.bc1), bc2 = _mm512_set1_ps(h.bc2);
  const __m512 lr = _mm512_set1_ps(h.lr), eps = _mm512_set1_ps(h.eps);
  const __m512 cl = _mm512_set1_ps(clip);
  const __m512 ms = _mm512_set1_ps(A.ms[b]), rs = _mm512_set1_ps(A.rs[b]);
  __m512 am = _mm512_setzero_ps(), ar = _mm512_setzero_ps();
#pragma GCC unroll 8
  for (int j = 0; j < NV; ++j) {
    const size_t k = off + 16 * j;
    __m512 g;
    if constexpr (BF16_GRAD) {
      const __m256i g16 = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(A.gb + k));
      g = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(g16), 16));
    } else {
      g = _mm512_loadu_ps(A.gf + k);
    }
    g = _mm512_mul_ps(g, cl);
    const __m512 m_old = dec16(A.mq + k, ms);
    const __m512 r_old = dec16(A.rq + k, rs);
    const __m512 v_old = _mm512_mul_ps(r_old, r_old);
    const __m512 m = _mm512_add_ps(_mm512_mul_ps(b1, m_old), _mm512_mul_ps(omb1, g));
    const __m512 v = _mm512_add_ps(_mm512_mul_ps(b2, v_old), _mm512_mul_ps(omb2, _mm512_mul_ps(g, g)));
    const __m512 mh = _mm512_div_ps(m, bc1);
    const __m512 vh = _mm512_div_ps(v, bc2);
    const __m512 p = _mm512_sub_ps(
        _mm512_loadu_ps(A.p + k),
        _mm512_div_ps(_mm512_mul_ps(lr, mh), _mm512_add_ps(_mm512_sqrt_ps(vh), eps)));
    _mm512_storeu_ps(A.p + k, p);
    if constexpr (SHADOW == 1)
      _mm256_storeu_si256(reinterpret_cast<__m256i*>(A.sb + k), _mm512_cvtepi32_epi16(bf16_bits16(p)));
    else if constexpr (SHADOW == 2)
      _mm512_storeu_ps(A.sf + k, p);
    mv[j] = m;
    rv[j] = _mm512_sqrt_ps(v);
    am = _mm512_max_ps(am, _mm512_abs_ps(m));
    ar = _mm512_max_ps(ar, rv[j]);
  }
  const float amax_m = _mm512_reduce_max_ps(am), amax_r = _mm512_reduce_max_ps(ar);
  A.ms[b] = block_scale(amax_m);
  A.rs[b] = block_scale(amax_r);
  const __m512 im = _mm512_set1_ps(block_factor(amax_m));
  const __m512 ir = _mm512_set1_ps(block_factor(amax_r));
#pragma GCC unroll 8
  for (int j = 0; j < NV; ++j) {
    const size_t k = off + 16 * j;
    _mm_storeu_si128(reinterpret_cast<__m128i*>(A.mq + k),
                     _mm512_cvtepi32_epi8(enc16(_mm512_mul_ps(mv[j], im))));
    _mm_storeu_si128(reinterpret_cast<__m128i*>(A.rq + k),
                     _mm512_cvtepi32_epi8(enc16(_mm512_mul_ps(rv[j], ir))));
  }
}

// ---- dispatch: the widest form this CPU runs (MT_HOST_SIMD=avx2 or
// scalar forces a narrower one), chosen once.
enum Simd { SIMD_SCALAR, SIMD_AVX2, SIMD_AVX512 };

Simd detect_simd() {
  Simd s = SIMD_SCALAR;
  if (__builtin_cpu_supports("avx2")) s = SIMD_AVX2;
  if (s == SIMD_AVX2 && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
      __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512dq"))
    s = SIMD_AVX512;
  if (const char* e = getenv("MT_HOST_SIMD")) {
    if (!strcmp(e, "scalar")) s = SIMD_SCALAR;
    else if (!strcmp(e, "avx2") && s > SIMD_AVX2) s = SIMD_AVX2;
  }
  return s;
}
const Simd kSimd = detect_simd();

template <bool BF16_GRAD, int SHADOW>
inline void adam8_block_t(const Adam8Arrays& A, size_t off, int n, size_t b, const AdamHp& h,
                          float clip) {
  if (n == ADAM8_BLOCK && kSimd == SIMD_AVX512)
    adam8_block_avx512<BF16_GRAD, SHADOW>(A, off, b, h, clip);
  else if (n == ADAM8_BLOCK && kSimd == SIMD_AVX2)
    adam8_block_avx2<BF16_GRAD, SHADOW>(A, off, b, h, clip);
  else
    adam8_block_scalar<BF16_GRAD, SHADOW>(A, off, n, b, h, clip);
}

void adam8_block(const Adam8Arrays& A, size_t off, int n, size_t b, const AdamHp& h, float clip) {
  if (A.gb) {
    if (A.sb) adam8_block_t<true, 1>(A, off, n, b, h, clip);
    else if (A.sf) adam8_block_t<true, 2>(A, off, n, b, h, clip);
    else adam8_block_t<true, 0>(A, off, n, b, h, clip);
  } else {
    if (A.sb) adam8_block_t<false, 1>(A, off, n, b, h, clip);
    else if (A.sf) adam8_block_t<false, 2>(A, off, n, b, h, clip);
    else adam8_block_t<false, 0>(A, off, n, b, h, clip);
  }
}

}  // namespace

size_t adam8_segment_blocks(const Adam8Seg* segs, int nseg) {
  size_t nb = 0;
  for (int i = 0; i < nseg; ++i) nb += adam8_blocks(segs[i].n);
  return nb;
}

void adam8_range(const Adam8Arrays& A, const Adam8Seg* segs, int nseg, size_t blo, size_t bhi,
                 const AdamHp& h, float clip) {
  // walk the segments' blocks [blo, bhi) (blocks numbered across segments)
  size_t first = 0;
  for (int s = 0; s < nseg && blo < bhi; ++s) {
    const size_t nb = adam8_blocks(segs[s].n);
    const size_t lo = std::max(blo, first), hi = std::min(bhi, first + nb);
    for (size_t bi = lo; bi < hi; ++bi) {
      const size_t j = bi - first;
      const size_t off = segs[s].off + j * ADAM8_BLOCK;
      const int n = (int)std::min<size_t>(ADAM8_BLOCK, segs[s].n - j * ADAM8_BLOCK);
      adam8_block(A, off, n, segs[s].sblk + j, h, clip);
    }
    first += nb;
  }
}

void adam8_parallel(const Adam8Arrays& A, const Adam8Seg* segs, int nseg, const AdamHp& h,
                    float clip, ThreadPool* pool) {
  const size_t nb = adam8_segment_blocks(segs, nseg);
  auto body = [&](size_t lo, size_t hi) { adam8_range(A, segs, nseg, lo, hi, h, clip); };
  if (pool) pool->parallel_for(nb, body, 64);
  else body(0, nb);
}

void adam8_dequant(const uint8_t* q, const float* scales, const Adam8Seg& seg, bool square,
                   float* out) {
  for (size_t i = 0; i < seg.n; ++i) {
    const float x = kE4M3.v[q[seg.off + i]] * scales[seg.sblk + i / ADAM8_BLOCK];
    out[i] = square ? x * x : x;
  }
}

}  // namespace mt
