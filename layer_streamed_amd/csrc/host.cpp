// Host runtime: worker pool, CPU Adam (MegaTrain blog summary, section 1:
// the optimizer step runs entirely on the CPU), embedding gather and
// scatter-add.  Compiled with -ffp-contract=off so every fp32 operation is
// rounded as written (no fused multiply-add), which keeps the update
// bit-identical to a plain fp32 evaluation of the same formula.
#include "host.h"

#include <immintrin.h>
#include <math.h>
#include <string.h>

#include <algorithm>

#include "status.h"

namespace mt {

ThreadPool::ThreadPool(int threads) {
  const int n = std::max(1, threads) - 1;
  for (int i = 0; i < n; ++i) workers_.emplace_back([this, i] { loop(i); });
}

ThreadPool::~ThreadPool() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
  }
  cv_.notify_all();
  for (auto& t : workers_) t.join();
}

void ThreadPool::loop(int idx) {
  uint64_t seen = 0;
  for (;;) {
    const std::function<void(size_t, size_t)>* job;
    size_t n;
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
      if (stop_) return;
      seen = gen_;
      job = job_;
      n = n_;
    }
    const size_t parts = workers_.size() + 1;
    const size_t lo = n * (idx + 1) / parts, hi = n * (idx + 2) / parts;
    if (lo < hi) (*job)(lo, hi);
    {
      std::lock_guard<std::mutex> lk(mu_);
      if (--pending_ == 0) done_cv_.notify_all();
    }
  }
}

void ThreadPool::parallel_for(size_t n, const std::function<void(size_t, size_t)>& fn,
                              size_t grain) {
  if (n == 0) return;
  if (workers_.empty() || n < grain) {
    fn(0, n);
    return;
  }
  {
    std::lock_guard<std::mutex> lk(mu_);
    job_ = &fn;
    n_ = n;
    pending_ = (int)workers_.size();
    ++gen_;
  }
  cv_.notify_all();
  const size_t parts = workers_.size() + 1;
  fn(0, n / parts);
  std::unique_lock<std::mutex> lk(mu_);
  done_cv_.wait(lk, [&] { return pending_ == 0; });
}

AdamHp adam_hp(const mt_run_cfg& hp, int64_t step) {
  AdamHp h;
  h.b1 = (float)hp.beta1;
  h.omb1 = (float)(1.0 - hp.beta1);
  h.b2 = (float)hp.beta2;
  h.omb2 = (float)(1.0 - hp.beta2);
  h.bc1 = (float)(1.0 - pow(hp.beta1, (double)step));
  h.bc2 = (float)(1.0 - pow(hp.beta2, (double)step));
  h.lr = (float)hp.lr;
  h.eps = (float)hp.eps;
  return h;
}

namespace {

// Branch-free RNE float32 -> bfloat16 (quiet NaN with the sign kept), written
// so the compiler can vectorize it.
inline uint32_t f2bf_bits(uint32_t u) {
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t q = ((u >> 16) & 0x8000u) | 0x7FC0u;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? q : r;
}

// SHADOW: 0 none, 1 bf16 streamed copy, 2 fp32 streamed copy.
template <bool BF16_GRAD, int SHADOW>
void adam_loop(float* __restrict p, float* __restrict m, float* __restrict v,
               const void* __restrict graw, void* __restrict shadow, size_t lo, size_t hi,
               const AdamHp& h, float clip) {
  const float b1 = h.b1, omb1 = h.omb1, b2 = h.b2, omb2 = h.omb2;
  const float bc1 = h.bc1, bc2 = h.bc2, lr = h.lr, eps = h.eps;
  const uint16_t* __restrict gb = static_cast<const uint16_t*>(graw);
  const float* __restrict gf = static_cast<const float*>(graw);
  for (size_t i = lo; i < hi; ++i) {
    float g;
    if constexpr (BF16_GRAD) {
      const uint32_t gu = (uint32_t)gb[i] << 16;
      __builtin_memcpy(&g, &gu, 4);
    } else {
      g = gf[i];
    }
    g = g * clip;
    const float mi = b1 * m[i] + omb1 * g;
    const float vi = b2 * v[i] + omb2 * (g * g);
    const float mh = mi / bc1;
    const float vh = vi / bc2;
    const float pi = p[i] - lr * mh / (sqrtf(vh) + eps);
    m[i] = mi;
    v[i] = vi;
    p[i] = pi;
    if constexpr (SHADOW == 1) {
      uint32_t pu;
      __builtin_memcpy(&pu, &pi, 4);
      static_cast<uint16_t*>(shadow)[i] = (uint16_t)f2bf_bits(pu);
    } else if constexpr (SHADOW == 2) {
      static_cast<float*>(shadow)[i] = pi;
    }
  }
}

// The hot case (bf16 gradient, bf16 streamed copy) in explicit AVX2: the
// same operations in the same order as adam_loop (no fused multiply-add;
// division and square root are IEEE), so the result is bitwise that of the
// scalar loop.  The bf16 copy is written with streaming stores: it is
// write-only here, and ordinary stores would first read every line of it
// (read-for-ownership), 2 of the ~30 bytes of host traffic per parameter.
void adam_bf16_stream(float* __restrict p, float* __restrict m, float* __restrict v,
                      const uint16_t* __restrict gb, uint16_t* __restrict sh, size_t lo,
                      size_t hi, const AdamHp& h, float clip) {
  // scalar until the copy is 16-byte aligned
  size_t i = lo;
  while (i < hi && ((uintptr_t)(sh + i) & 15)) {
    adam_loop<true, 1>(p, m, v, gb, sh, i, i + 1, h, clip);
    ++i;
  }
  const __m256 b1 = _mm256_set1_ps(h.b1), omb1 = _mm256_set1_ps(h.omb1);
  const __m256 b2 = _mm256_set1_ps(h.b2), omb2 = _mm256_set1_ps(h.omb2);
  const __m256 bc1 = _mm256_set1_ps(h.bc1), bc2 = _mm256_set1_ps(h.bc2);
  const __m256 lr = _mm256_set1_ps(h.lr), eps = _mm256_set1_ps(h.eps);
  const __m256 cl = _mm256_set1_ps(clip);
  const __m256i round = _mm256_set1_epi32(0x7FFF), one = _mm256_set1_epi32(1);
  const __m256i absmask = _mm256_set1_epi32(0x7FFFFFFF), inf = _mm256_set1_epi32(0x7F800000);
  const __m256i sign = _mm256_set1_epi32(0x8000), qnan = _mm256_set1_epi32(0x7FC0);
  for (; i + 8 <= hi; i += 8) {
    const __m128i g16 = _mm_loadu_si128(reinterpret_cast<const __m128i*>(gb + i));
    const __m256 g = _mm256_mul_ps(
        _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(g16), 16)), cl);
    const __m256 mi = _mm256_add_ps(_mm256_mul_ps(b1, _mm256_loadu_ps(m + i)), _mm256_mul_ps(omb1, g));
    const __m256 vi = _mm256_add_ps(_mm256_mul_ps(b2, _mm256_loadu_ps(v + i)),
                                    _mm256_mul_ps(omb2, _mm256_mul_ps(g, g)));
    const __m256 mh = _mm256_div_ps(mi, bc1);
    const __m256 vh = _mm256_div_ps(vi, bc2);
    const __m256 pi = _mm256_sub_ps(
        _mm256_loadu_ps(p + i),
        _mm256_div_ps(_mm256_mul_ps(lr, mh), _mm256_add_ps(_mm256_sqrt_ps(vh), eps)));
    _mm256_storeu_ps(m + i, mi);
    _mm256_storeu_ps(v + i, vi);
    _mm256_storeu_ps(p + i, pi);
    // fp32 -> bf16, round to nearest even, NaN -> quiet NaN with the sign
    const __m256i u = _mm256_castps_si256(pi);
    const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(u, 16), one);
    const __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, round), lsb), 16);
    const __m256i q = _mm256_or_si256(_mm256_and_si256(_mm256_srli_epi32(u, 16), sign), qnan);
    const __m256i isnan = _mm256_cmpgt_epi32(_mm256_and_si256(u, absmask), inf);
    const __m256i b = _mm256_blendv_epi8(r, q, isnan);
    // 8 x 32-bit -> 8 x 16-bit (values fit in 16 bits, packus keeps them)
    const __m256i packed = _mm256_permute4x64_epi64(_mm256_packus_epi32(b, b), 0x08);
    _mm_stream_si128(reinterpret_cast<__m128i*>(sh + i), _mm256_castsi256_si128(packed));
  }
  if (i < hi) adam_loop<true, 1>(p, m, v, gb, sh, i, hi, h, clip);
  _mm_sfence();  // streaming stores visible before the copy is read again
}

}  // namespace

void adam_range(float* p, float* m, float* v, const uint16_t* gb, const float* gf,
                uint16_t* sb, float* sf, size_t lo, size_t hi, const AdamHp& h, float clip) {
  if (gb) {
    if (sb) adam_bf16_stream(p, m, v, gb, sb, lo, hi, h, clip);
    else if (sf) adam_loop<true, 2>(p, m, v, gb, sf, lo, hi, h, clip);
    else adam_loop<true, 0>(p, m, v, gb, nullptr, lo, hi, h, clip);
  } else {
    if (sb) adam_loop<false, 1>(p, m, v, gf, sb, lo, hi, h, clip);
    else if (sf) adam_loop<false, 2>(p, m, v, gf, sf, lo, hi, h, clip);
    else adam_loop<false, 0>(p, m, v, gf, nullptr, lo, hi, h, clip);
  }
}

bool grad_finite(const uint16_t* gb, const float* gf, size_t n, ThreadPool* pool) {
  std::vector<char> bad(pool ? pool->size() + 1 : 1, 0);
  std::mutex mu;
  bool any_bad = false;
  auto body = [&](size_t lo, size_t hi) {
    bool b = false;
    if (gb) {
      for (size_t i = lo; i < hi; ++i) b |= ((gb[i] & 0x7F80u) == 0x7F80u);
    } else {
      for (size_t i = lo; i < hi; ++i) b |= !std::isfinite(gf[i]);
    }
    if (b) {
      std::lock_guard<std::mutex> lk(mu);
      any_bad = true;
    }
  };
  if (pool) pool->parallel_for(n, body);
  else body(0, n);
  return !any_bad;
}

void adam_parallel(float* p, float* m, float* v, const uint16_t* gb, const float* gf,
                   uint16_t* sb, float* sf, size_t n, const AdamHp& h, float clip,
                   ThreadPool* pool) {
  auto body = [&](size_t lo, size_t hi) { adam_range(p, m, v, gb, gf, sb, sf, lo, hi, h, clip); };
  if (pool) pool->parallel_for(n, body);
  else body(0, n);
}

void embed_gather(const void* table, const int32_t* ids, size_t n_tok, size_t row_bytes,
                  void* out, ThreadPool* pool) {
  const char* tb = static_cast<const char*>(table);
  char* ob = static_cast<char*>(out);
  auto body = [&](size_t lo, size_t hi) {
    for (size_t t = lo; t < hi; ++t) memcpy(ob + t * row_bytes, tb + (size_t)ids[t] * row_bytes, row_bytes);
  };
  if (pool) pool->parallel_for(n_tok, body, 64);
  else body(0, n_tok);
}

namespace {
inline float to_f32(uint16_t b) { return host_bf2f(b); }
inline float to_f32(float f) { return f; }

template <class G>
void scatter_add_t(const G* dx0, const int32_t* ids, size_t n_tok, size_t H, float* dE,
                   ThreadPool* pool) {
  // tokens grouped by destination row (stable: token order within a row);
  // each worker owns whole rows and adds their tokens in token order, so
  // the summation order per element is the token order regardless of
  // threads, and every access is a full contiguous row
  std::vector<int32_t> order(n_tok);
  for (size_t t = 0; t < n_tok; ++t) order[t] = (int32_t)t;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return ids[a] < ids[b]; });
  std::vector<size_t> seg;
  for (size_t i = 0; i < n_tok; ++i)
    if (i == 0 || ids[order[i]] != ids[order[i - 1]]) seg.push_back(i);
  seg.push_back(n_tok);
  auto body = [&](size_t s0, size_t s1) {
    for (size_t s = s0; s < s1; ++s) {
      float* row = dE + (size_t)ids[order[seg[s]]] * H;
      for (size_t i = seg[s]; i < seg[s + 1]; ++i) {
        const G* src = dx0 + (size_t)order[i] * H;
        for (size_t c = 0; c < H; ++c) row[c] += to_f32(src[c]);
      }
    }
  };
  const size_t n_seg = seg.size() - 1;
  if (pool) pool->parallel_for(n_seg, body, 16);
  else body(0, n_seg);
}
}  // namespace

void embed_scatter_add(const uint16_t* dx0, const int32_t* ids, size_t n_tok, size_t H,
                       float* dE, ThreadPool* pool) {
  scatter_add_t(dx0, ids, n_tok, H, dE, pool);
}
void embed_scatter_add(const float* dx0, const int32_t* ids, size_t n_tok, size_t H, float* dE,
                       ThreadPool* pool) {
  scatter_add_t(dx0, ids, n_tok, H, dE, pool);
}

}  // namespace mt

using namespace mt;

extern "C" {

void mt_run_cfg_default(mt_run_cfg* r) {
  if (!r) return;
  memset(r, 0, sizeof(*r));
  r->ckpt_interval = 4;
  r->prefetch_depth = 2;
  r->use_slab_pool = 1;
  r->n_slabs = 8;
  r->mlp_chunk_tokens = 0;
  r->head_chunk_tokens = 16384;
  r->precision = MT_PREC_BF16;
  r->host_threads = 16;
  r->check_finite = 1;
  r->serialize = 0;
  r->host_alloc = MT_HOST_PINNED;
  r->keep_grads = 0;
  r->time_kernels = 1;
  r->keep_internals = 1;
  r->defer_updates = 1;
  r->resident_layers = 0;
  r->lr = 1e-4;
  r->beta1 = 0.9;
  r->beta2 = 0.999;
  r->eps = 1e-8;
  r->weight_decay = 0.0;
}

// The worker pool of the standalone optimizer calls (resized on demand).
static ThreadPool* standalone_pool(int threads, std::unique_lock<std::mutex>* lk) {
  static ThreadPool* pool = nullptr;
  static int pool_threads = 0;
  static std::mutex pool_mu;
  *lk = std::unique_lock<std::mutex>(pool_mu);
  const int want = threads > 0 ? threads : 1;
  if (!pool || pool_threads != want) {
    delete pool;
    pool = new ThreadPool(want);
    pool_threads = want;
  }
  return pool;
}

static mt_status check_hp(const mt_run_cfg* hp, int64_t step, const char* fn) {
  MT_CHECK(hp, MT_E_INVALID, "%s: null hyperparameters", fn);
  MT_CHECK(step >= 1, MT_E_INVALID, "%s: step must be >= 1", fn);
  MT_CHECK(hp->weight_decay == 0.0, MT_E_INVALID, "%s: weight decay is not supported", fn);
  MT_CHECK(hp->beta1 >= 0 && hp->beta1 < 1 && hp->beta2 >= 0 && hp->beta2 < 1 && hp->eps >= 0,
           MT_E_INVALID, "%s: betas must be in [0, 1), eps >= 0", fn);
  return MT_OK;
}

mt_status mt_host_adam8(float* param, uint8_t* m_code, float* m_scale, uint8_t* r_code,
                        float* r_scale, const void* grad, int32_t grad_dtype,
                        uint16_t* bf16_shadow, size_t n, int64_t step, float clip,
                        const mt_run_cfg* hp) {
  if (mt_status st = check_hp(hp, step, "mt_host_adam8"); st != MT_OK) return st;
  MT_CHECK(n == 0 || (param && m_code && m_scale && r_code && r_scale && grad), MT_E_INVALID,
           "mt_host_adam8: null array");
  MT_CHECK(grad_dtype == MT_DT_BF16 || grad_dtype == MT_DT_F32, MT_E_INVALID,
           "mt_host_adam8: grad_dtype must be MT_DT_BF16 or MT_DT_F32");
  MT_CHECK(clip > 0.f && clip <= 1.f, MT_E_INVALID, "mt_host_adam8: clip must be in (0, 1]");
  const uint16_t* gb = grad_dtype == MT_DT_BF16 ? static_cast<const uint16_t*>(grad) : nullptr;
  const float* gf = grad_dtype == MT_DT_F32 ? static_cast<const float*>(grad) : nullptr;
  std::unique_lock<std::mutex> lk;
  ThreadPool* pool = standalone_pool(hp->host_threads, &lk);
  if (hp->check_finite && !grad_finite(gb, gf, n, pool))
    return set_error(MT_E_NONFINITE, "mt_host_adam8: gradient has NaN or Inf; nothing updated");
  const Adam8Arrays a{param, m_code, r_code, m_scale, r_scale, gb, gf, bf16_shadow, nullptr};
  const Adam8Seg seg{0, n, 0};
  adam8_parallel(a, &seg, 1, adam_hp(*hp, step), clip, pool);
  return MT_OK;
}

mt_status mt_host_adam(float* param, float* exp_avg, float* exp_avg_sq, const void* grad,
                       int32_t grad_dtype, uint16_t* bf16_shadow, size_t n, int64_t step,
                       const mt_run_cfg* hp) {
  MT_CHECK(hp, MT_E_INVALID, "mt_host_adam: null hyperparameters");
  MT_CHECK(n == 0 || (param && exp_avg && exp_avg_sq && grad), MT_E_INVALID,
           "mt_host_adam: null array");
  MT_CHECK(grad_dtype == MT_DT_BF16 || grad_dtype == MT_DT_F32, MT_E_INVALID,
           "mt_host_adam: grad_dtype must be MT_DT_BF16 or MT_DT_F32");
  MT_CHECK(step >= 1, MT_E_INVALID, "mt_host_adam: step must be >= 1");
  MT_CHECK(hp->weight_decay == 0.0, MT_E_INVALID, "mt_host_adam: weight decay is not supported");
  MT_CHECK(hp->beta1 >= 0 && hp->beta1 < 1 && hp->beta2 >= 0 && hp->beta2 < 1 && hp->eps >= 0,
           MT_E_INVALID, "mt_host_adam: betas must be in [0, 1), eps >= 0");
  const uint16_t* gb = grad_dtype == MT_DT_BF16 ? static_cast<const uint16_t*>(grad) : nullptr;
  const float* gf = grad_dtype == MT_DT_F32 ? static_cast<const float*>(grad) : nullptr;
  std::unique_lock<std::mutex> lk;
  ThreadPool* pool = standalone_pool(hp->host_threads, &lk);
  if (hp->check_finite && !grad_finite(gb, gf, n, pool))
    return set_error(MT_E_NONFINITE, "mt_host_adam: gradient has NaN or Inf; nothing updated");
  adam_parallel(param, exp_avg, exp_avg_sq, gb, gf, bf16_shadow, nullptr, n, adam_hp(*hp, step),
                1.f, pool);
  return MT_OK;
}

}  // extern "C"
