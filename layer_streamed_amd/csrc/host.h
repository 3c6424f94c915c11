// Host-side runtime pieces of libmt: a persistent worker pool, the CPU Adam
// kernel and the embedding gather / scatter-add.  Plain C++ (no HIP).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "mt.h"

namespace mt {

// Fixed set of worker threads; parallel_for splits [0, n) into contiguous
// ranges, one per worker (plus the caller), and returns when all are done.
class ThreadPool {
 public:
  explicit ThreadPool(int threads);
  ~ThreadPool();
  int size() const { return (int)workers_.size() + 1; }
  // grain: below this many items the caller runs fn(0, n) alone
  void parallel_for(size_t n, const std::function<void(size_t, size_t)>& fn, size_t grain = 4096);

 private:
  void loop(int idx);
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(size_t, size_t)>* job_ = nullptr;
  size_t n_ = 0;
  uint64_t gen_ = 0;
  int pending_ = 0;
  bool stop_ = false;
};

struct AdamHp {
  float b1, omb1, b2, omb2, bc1, bc2, lr, eps;
};
AdamHp adam_hp(const mt_run_cfg& hp, int64_t step);

// One Adam update over [lo, hi): grad is bf16 (gb) or fp32 (gf), multiplied
// by `clip` (the global-norm clipping factor, 1 without clipping: an exact
// identity) before the update.  The updated master is also written to the
// streamed copy when one is given: bf16 (sb, round to nearest even) or fp32
// (sf, the debug precision).
void adam_range(float* p, float* m, float* v, const uint16_t* gb, const float* gf,
                uint16_t* sb, float* sf, size_t lo, size_t hi, const AdamHp& h, float clip);
// True if every gradient value in [0, n) is finite.
bool grad_finite(const uint16_t* gb, const float* gf, size_t n, ThreadPool* pool);
void adam_parallel(float* p, float* m, float* v, const uint16_t* gb, const float* gf,
                   uint16_t* sb, float* sf, size_t n, const AdamHp& h, float clip,
                   ThreadPool* pool);

inline uint16_t host_f2bf(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
inline float host_bf2f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

// ---- hybrid 8-bit Adam (host_adam8.cpp)
// Moments per tensor in blocks of ADAM8_BLOCK elements as OCP FP8 E4M3
// codes with one fp32 scale per block; m as is, v as r = sqrt(v).
constexpr int ADAM8_BLOCK = 128;
inline size_t adam8_blocks(size_t n) { return (n + ADAM8_BLOCK - 1) / ADAM8_BLOCK; }
// A tensor inside a unit's flat arrays: elements [off, off + n); its
// blocks' scales start at index sblk of the scale arrays.
struct Adam8Seg {
  size_t off, n, sblk;
};
struct Adam8Arrays {
  float* p;              // fp32 master
  uint8_t *mq, *rq;      // codes of m and of r = sqrt(v)
  float *ms, *rs;        // per-block scales
  const uint16_t* gb;    // gradient: bf16 ...
  const float* gf;       // ... or fp32 (one of the two)
  uint16_t* sb;          // streamed copy written from the new master: bf16,
  float* sf;             // fp32, or neither
};
uint8_t e4m3_encode(float y);  // round to nearest even, saturating at 448
float e4m3_decode(uint8_t c);
size_t adam8_segment_blocks(const Adam8Seg* segs, int nseg);
// Update blocks [blo, bhi) of the segments (numbered across segments in
// order); the gradient is multiplied by `clip` first.
void adam8_range(const Adam8Arrays& a, const Adam8Seg* segs, int nseg, size_t blo, size_t bhi,
                 const AdamHp& h, float clip);
void adam8_parallel(const Adam8Arrays& a, const Adam8Seg* segs, int nseg, const AdamHp& h,
                    float clip, ThreadPool* pool);
// Values of one segment's moment (square = true: r -> v = r * r) into out[n].
void adam8_dequant(const uint8_t* q, const float* scales, const Adam8Seg& seg, bool square,
                   float* out);

// x0[t] = table[ids[t]] (rows of row_bytes bytes: H bf16 or H fp32 values).
void embed_gather(const void* table, const int32_t* ids, size_t n_tok, size_t row_bytes,
                  void* out, ThreadPool* pool);
// dE[ids[t]] += dx0[t] in token order (fp32 accumulate; dE pre-zeroed);
// dx0 rows are H bf16 or H fp32 values.
void embed_scatter_add(const uint16_t* dx0, const int32_t* ids, size_t n_tok, size_t H,
                       float* dE, ThreadPool* pool);
void embed_scatter_add(const float* dx0, const int32_t* ids, size_t n_tok, size_t H, float* dE,
                       ThreadPool* pool);

}  // namespace mt
