// Host store of the model (MegaTrain blog summary, section 1: parameters
// and optimizer states live in host memory; "Performance and Capabilities":
// a flat layout in authoritative host storage keeps host memory linear in
// the parameter count).
//
// Per unit (a layer, the head, the embedding) the fp32 master, m and v are
// three flat arrays with one shared layout; only the bf16 copy of the
// master (what the GPU receives) and the gradient slabs (what it sends back)
// are pinned, since only they are DMA endpoints: 2 B/param pinned plus the
// slab pool, instead of 14 B/param.  In the fp32 debug precision the
// streamed copy, slabs and kept gradients hold fp32 instead.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "model.h"
#include "status.h"

namespace mt {

void* SlabPool::acquire() {
  std::unique_lock<std::mutex> lk(mu_);
  cv_.wait(lk, [&] { return !free_.empty(); });
  void* p = free_.back();
  free_.pop_back();
  return p;
}

void SlabPool::release(void* p) {
  {
    std::lock_guard<std::mutex> lk(mu_);
    free_.push_back(p);
  }
  cv_.notify_one();
}

bool lookup_param(const mt_model* m, const char* name, TensorRef* out) {
  if (!name) return false;
  const Dims& d = m->shape;
  const size_t H = d.H;
  const int L = m->cfg.n_layers;
  std::string s(name);
  if (s == "embed") { *out = {L + 1, 0, (size_t)d.V * H}; return true; }
  if (s == "final_norm") { *out = {L, m->hl.final_norm, H}; return true; }
  if (s == "lm_head") { *out = {L, m->hl.lm_head, (size_t)d.V * H}; return true; }
  if (s.rfind("layers.", 0) != 0) return false;
  const size_t dot = s.find('.', 7);
  if (dot == std::string::npos || dot == 7) return false;
  const std::string num = s.substr(7, dot - 7);
  if (num.find_first_not_of("0123456789") != std::string::npos || num.size() > 6) return false;
  const int l = atoi(num.c_str());
  if (l < 0 || l >= L) return false;
  const std::string t = s.substr(dot + 1);
  const LayerLayout& ll = m->ll;
  if (t == "attn_norm") *out = {l, ll.attn_norm, H};
  else if (t == "w_q") *out = {l, ll.w_q, (size_t)d.Qd * H};
  else if (t == "w_k") *out = {l, ll.w_k, (size_t)d.Kvd * H};
  else if (t == "w_v") *out = {l, ll.w_v, (size_t)d.Kvd * H};
  else if (t == "w_o") *out = {l, ll.w_o, H * d.Qd};
  else if (t == "mlp_norm") *out = {l, ll.mlp_norm, H};
  else if (t == "w_gate") *out = {l, ll.w_gate, (size_t)d.F * H};
  else if (t == "w_up") *out = {l, ll.w_up, (size_t)d.F * H};
  else if (t == "w_down") *out = {l, ll.w_down, H * d.F};
  else return false;
  return true;
}

void unit_adam(mt_model* M, int unit, const uint16_t* gb, const float* gf, const AdamHp& hp,
               float clip) {
  Unit& u = M->units[unit];
  const bool f32 = M->es == 4;
  uint16_t* sb = f32 ? nullptr : static_cast<uint16_t*>(u.shadow);
  float* sf = f32 ? static_cast<float*>(u.shadow) : nullptr;
  if (M->run.opt_8bit) {
    const Adam8Arrays a{u.master, u.mq, u.rq, u.ms, u.rs, gb, gf, sb, sf};
    adam8_parallel(a, u.segs.data(), (int)u.segs.size(), hp, clip, M->pool.get());
  } else {
    adam_parallel(u.master, u.m, u.v, gb, gf, sb, sf, u.n, hp, clip, M->pool.get());
  }
}

void apply_pending_head(mt_model* M) {
  PendingAdam& pa = M->pending;
  if (!pa.head) return;
  const bool f32 = M->es == 4;
  unit_adam(M, M->cfg.n_layers, f32 ? nullptr : static_cast<const uint16_t*>(pa.head_grad),
            f32 ? static_cast<const float*>(pa.head_grad) : nullptr, pa.hp_head, pa.clip_head);
  pa.head = false;
}

namespace {
// Adam over whole embedding rows [r0, r1) of the list (or of every row when
// rows == nullptr), skipping and then marking rows already done.
void embed_rows(mt_model* M, const std::vector<int32_t>* rows) {
  PendingAdam& pa = M->pending;
  Unit& u = M->units[M->cfg.n_layers + 1];
  const size_t H = M->shape.H;
  const bool f32 = M->es == 4;
  const size_t n = rows ? rows->size() : (size_t)M->shape.V;
  M->pool->parallel_for(n, [&](size_t lo, size_t hi) {
    for (size_t i = lo; i < hi; ++i) {
      const size_t r = rows ? (size_t)(*rows)[i] : i;
      if (pa.row_done[r]) continue;
      const size_t a = r * H;
      // an untouched row's gradient is zero: read a cached zero row instead
      // of the row of dE (the same values, so the same result)
      const float* g = pa.touched[r] ? M->dE + a : M->zero_row;
      if (M->run.opt_8bit) {
        // a row is whole 8-bit blocks (hidden % 128 == 0) of the one tensor
        const size_t b = a / ADAM8_BLOCK;
        const Adam8Arrays ar{u.master + a, u.mq + a, u.rq + a, u.ms + b, u.rs + b, nullptr, g,
                             f32 ? nullptr : static_cast<uint16_t*>(u.shadow) + a,
                             f32 ? static_cast<float*>(u.shadow) + a : nullptr};
        const Adam8Seg seg{0, H, 0};
        adam8_range(ar, &seg, 1, 0, adam8_blocks(H), pa.hp_embed, pa.clip_embed);
      } else if (f32)
        adam_range(u.master + a, u.m + a, u.v + a, nullptr, g, nullptr,
                   static_cast<float*>(u.shadow) + a, 0, H, pa.hp_embed, pa.clip_embed);
      else
        adam_range(u.master + a, u.m + a, u.v + a, nullptr, g,
                   static_cast<uint16_t*>(u.shadow) + a, nullptr, 0, H, pa.hp_embed, pa.clip_embed);
      pa.row_done[r] = 1;
    }
  }, 16);
}
}  // namespace

void apply_pending_embed_rows(mt_model* M, const int32_t* ids, size_t n) {
  PendingAdam& pa = M->pending;
  if (!pa.embed) return;
  std::vector<uint8_t> seen(M->shape.V, 0);
  std::vector<int32_t> rows;
  for (size_t t = 0; t < n; ++t)
    if (!seen[ids[t]]) {
      seen[ids[t]] = 1;
      rows.push_back(ids[t]);
    }
  embed_rows(M, &rows);
}

void apply_pending_embed_rest(mt_model* M) {
  PendingAdam& pa = M->pending;
  if (!pa.embed) return;
  embed_rows(M, nullptr);
  pa.embed = false;
}

namespace {
void release_grad(mt_model* M, const PendingAdam::Layer& x) {
  if (x.own_alloc) hipHostFree(x.grad);
  else M->slabs.release(x.grad);
}
}  // namespace

void apply_pending_layers(mt_model* M, const std::function<void(int)>& done) {
  PendingAdam& pa = M->pending;
  std::sort(pa.layers.begin(), pa.layers.end(),
            [](const PendingAdam::Layer& a, const PendingAdam::Layer& b) { return a.unit < b.unit; });
  const bool f32 = M->es == 4;
  for (const PendingAdam::Layer& x : pa.layers) {
    unit_adam(M, x.unit, f32 ? nullptr : static_cast<const uint16_t*>(x.grad),
              f32 ? static_cast<const float*>(x.grad) : nullptr, pa.hp_layers, pa.clip_layers);
    release_grad(M, x);
    if (done) done(x.unit);
  }
  pa.layers.clear();
}

void flush_pending(mt_model* M) {
  apply_pending_head(M);
  apply_pending_layers(M, nullptr);
  apply_pending_embed_rest(M);
}

void drop_pending(mt_model* M) {
  PendingAdam& pa = M->pending;
  pa.head = pa.embed = false;
  for (const PendingAdam::Layer& x : pa.layers) release_grad(M, x);
  pa.layers.clear();
}

}  // namespace mt

using namespace mt;

void* mt_model::host_alloc(size_t bytes, bool pinned) {
  bytes = (bytes + 4095) & ~size_t(4095);
  void* p = nullptr;
  if (pinned) {
    if (hipHostMalloc(&p, bytes, hipHostMallocDefault) != hipSuccess) return nullptr;
    pinned_bytes += (int64_t)bytes;
  } else {
    p = aligned_alloc(4096, bytes);
    if (!p) return nullptr;
    pageable_bytes += (int64_t)bytes;
  }
  blocks.push_back({p, bytes, pinned});
  return p;
}

mt_model::~mt_model() {
  for (auto& x : pending.layers)
    if (x.own_alloc) hipHostFree(x.grad);  // pool slabs go with the blocks below
  for (auto& e : events) hipEventDestroy(e);
  for (auto& b : blocks) {
    if (b.pinned) hipHostFree(b.p);
    else free(b.p);
  }
}

static mt_status check_run(const mt_model_cfg* cfg, const mt_run_cfg* run) {
  MT_CHECK(run->ckpt_interval >= 1, MT_E_INVALID, "ckpt_interval must be >= 1");
  MT_CHECK(run->prefetch_depth >= 1 && run->prefetch_depth <= 3, MT_E_INVALID,
           "prefetch_depth must be 1, 2 or 3");
  MT_CHECK(!run->use_slab_pool || (run->n_slabs >= 1 && run->n_slabs <= 64), MT_E_INVALID,
           "n_slabs must be in [1, 64]");
  MT_CHECK(run->host_threads >= 1 && run->host_threads <= 256, MT_E_INVALID,
           "host_threads must be in [1, 256]");
  MT_CHECK(run->host_alloc == MT_HOST_PINNED || run->host_alloc == MT_HOST_PAGEABLE, MT_E_INVALID,
           "bad host_alloc");
  MT_CHECK(run->weight_decay == 0.0, MT_E_INVALID, "weight decay is not supported");
  MT_CHECK(run->resident_layers >= 0 && run->resident_layers <= cfg->n_layers, MT_E_INVALID,
           "resident_layers must be in [0, n_layers]");
  MT_CHECK(run->lr > 0 && run->beta1 >= 0 && run->beta1 < 1 && run->beta2 >= 0 &&
               run->beta2 < 1 && run->eps >= 0,
           MT_E_INVALID, "bad Adam hyperparameters");
  MT_CHECK(run->opt_8bit == 0 || run->opt_8bit == 1, MT_E_INVALID, "opt_8bit must be 0 or 1");
  MT_CHECK(!run->opt_8bit || cfg->hidden % ADAM8_BLOCK == 0, MT_E_INVALID,
           "opt_8bit needs hidden to be a multiple of %d (embedding rows are whole blocks)",
           ADAM8_BLOCK);
  MT_CHECK(run->clip_norm >= 0, MT_E_INVALID, "clip_norm must be >= 0");
  MT_CHECK(!(run->clip_norm > 0) || !run->use_slab_pool || run->n_slabs >= cfg->n_layers + 1,
           MT_E_INVALID,
           "clip_norm needs every layer's and the head's gradient held at once: n_slabs >= "
           "n_layers + 1 (%d), or no slab pool",
           cfg->n_layers + 1);
  return MT_OK;
}

// The tensors of each unit, in layout order, with their 8-bit blocks'
// first scale index.
static void build_segments(mt_model* m) {
  const Dims& d = m->shape;
  const size_t H = d.H, Q = d.Qd, Kv = d.Kvd, F = d.F, V = d.V;
  const LayerLayout& l = m->ll;
  const int L = m->cfg.n_layers;
  auto fill = [](Unit& u, std::initializer_list<std::pair<size_t, size_t>> t) {
    u.segs.clear();
    size_t b = 0;
    for (const auto& [off, n] : t) {
      u.segs.push_back({off, n, b});
      b += adam8_blocks(n);
    }
  };
  for (int i = 0; i < L; ++i)
    fill(m->units[i], {{l.attn_norm, H}, {l.w_q, Q * H}, {l.w_k, Kv * H}, {l.w_v, Kv * H},
                       {l.w_o, H * Q}, {l.mlp_norm, H}, {l.w_gate, F * H}, {l.w_up, F * H},
                       {l.w_down, H * F}});
  fill(m->units[L], {{m->hl.final_norm, H}, {m->hl.lm_head, V * H}});
  fill(m->units[L + 1], {{0, V * H}});
}

static const Adam8Seg* find_segment(const Unit& u, size_t off) {
  for (const Adam8Seg& s : u.segs)
    if (s.off == off) return &s;
  return nullptr;
}

extern "C" {

mt_status mt_model_create(const mt_model_cfg* cfg, const mt_run_cfg* run, mt_model** out) {
  MT_CHECK(cfg && run && out, MT_E_INVALID, "mt_model_create: null argument");
  *out = nullptr;
  Dims d;
  if (const char* msg = make_dims(cfg, run, 1, 1, &d))
    return set_error(MT_E_SHAPE, "mt_model_create: %s", msg);
  if (mt_status st = check_run(cfg, run); st != MT_OK) return st;

  std::unique_ptr<mt_model> m(new mt_model());
  m->cfg = *cfg;
  m->run = *run;
  m->shape = d;
  m->es = d.es();
  m->ll = layer_layout(d);
  m->hl = head_layout(d);
  const int L = cfg->n_layers;
  m->units.resize(L + 2);
  for (int l = 0; l < L; ++l) m->units[l].n = m->ll.total;
  m->units[L].n = m->hl.total;
  m->units[L + 1].n = align128((size_t)d.V * d.H);
  const bool pinned = run->host_alloc == MT_HOST_PINNED;
  build_segments(m.get());

  // streamed copy of every unit in one pinned region
  const size_t es = m->es;
  size_t shadow_elems = 0;
  for (auto& u : m->units) shadow_elems += u.n;
  char* sh = static_cast<char*>(m->host_alloc(shadow_elems * es, pinned));
  if (!sh) return set_error(MT_E_OOM_HOST, "mt_model_create: %s allocation of %zu bytes failed",
                            pinned ? "pinned" : "host", shadow_elems * es);
  m->pool.reset(new ThreadPool(run->host_threads));
  size_t off = 0;
  for (auto& u : m->units) {
    u.shadow = sh + off * es;
    off += u.n;
    u.master = static_cast<float*>(m->host_alloc(u.n * 4, false));
    if (!u.master)
      return set_error(MT_E_OOM_HOST, "mt_model_create: host allocation of %zu bytes failed", u.n * 4);
    const size_t nb = adam8_segment_blocks(u.segs.data(), (int)u.segs.size());
    if (run->opt_8bit) {
      u.mq = static_cast<uint8_t*>(m->host_alloc(u.n, false));
      u.rq = static_cast<uint8_t*>(m->host_alloc(u.n, false));
      u.ms = static_cast<float*>(m->host_alloc(nb * 4, false));
      u.rs = static_cast<float*>(m->host_alloc(nb * 4, false));
      if (!u.mq || !u.rq || !u.ms || !u.rs)
        return set_error(MT_E_OOM_HOST, "mt_model_create: 8-bit state allocation failed");
    } else {
      u.m = static_cast<float*>(m->host_alloc(u.n * 4, false));
      u.v = static_cast<float*>(m->host_alloc(u.n * 4, false));
      if (!u.m || !u.v)
        return set_error(MT_E_OOM_HOST, "mt_model_create: host allocation of %zu bytes failed",
                         u.n * 4);
    }
    if (run->keep_grads) {
      u.kept = m->host_alloc(u.n * es, false);
      if (!u.kept) return set_error(MT_E_OOM_HOST, "mt_model_create: keep_grads allocation failed");
    }
    // first touch in parallel (places pages, zeroes pads and moments)
    float* ps[3] = {u.master, u.m, u.v};
    uint8_t* qs[2] = {u.mq, u.rq};
    char* shp = static_cast<char*>(u.shadow);
    char* kp = static_cast<char*>(u.kept);
    m->pool->parallel_for(u.n, [&](size_t lo, size_t hi) {
      for (float* p : ps)
        if (p) memset(p + lo, 0, (hi - lo) * 4);
      for (uint8_t* q : qs)
        if (q) memset(q + lo, 0, hi - lo);
      memset(shp + lo * es, 0, (hi - lo) * es);
      if (kp) memset(kp + lo * es, 0, (hi - lo) * es);
    });
    if (u.ms) {
      memset(u.ms, 0, nb * 4);
      memset(u.rs, 0, nb * 4);
    }
  }
  m->dE = static_cast<float*>(m->host_alloc((size_t)d.V * d.H * 4, false));
  m->zero_row = static_cast<float*>(m->host_alloc((size_t)d.H * 4, false));
  if (!m->dE || !m->zero_row)
    return set_error(MT_E_OOM_HOST, "mt_model_create: embedding gradient allocation failed");
  {
    float* dE = m->dE;
    m->pool->parallel_for((size_t)d.V * d.H,
                          [&](size_t lo, size_t hi) { memset(dE + lo, 0, (hi - lo) * 4); });
    memset(m->zero_row, 0, (size_t)d.H * 4);
  }

  // gradient slab pool: each slab fits the largest streamed unit
  m->slab_elems = std::max(m->ll.total, m->hl.total);
  const int n_slabs = run->use_slab_pool ? run->n_slabs : 0;
  for (int i = 0; i < n_slabs; ++i) {
    void* s = m->host_alloc(m->slab_elems * es, pinned);
    if (!s) return set_error(MT_E_OOM_HOST, "mt_model_create: slab allocation failed");
    m->slab_list.push_back(s);
  }
  m->slabs.init(m->slab_list);
  m->slabs.set_total(m->slab_list.size());
  *out = m.release();
  return MT_OK;
}

void mt_model_destroy(mt_model* model) { delete model; }

mt_status mt_model_set_schedule(mt_model* m, const mt_run_cfg* run) {
  MT_CHECK(m && run, MT_E_INVALID, "mt_model_set_schedule: null argument");
  Dims d;
  if (const char* msg = make_dims(&m->cfg, run, 1, 1, &d))
    return set_error(MT_E_SHAPE, "mt_model_set_schedule: %s", msg);
  if (mt_status st = check_run(&m->cfg, run); st != MT_OK) return st;
  const mt_run_cfg& o = m->run;
  MT_CHECK(run->precision == o.precision && run->host_alloc == o.host_alloc &&
               run->keep_grads == o.keep_grads && run->host_threads == o.host_threads &&
               run->opt_8bit == o.opt_8bit,
           MT_E_INVALID,
           "mt_model_set_schedule: precision, host_alloc, keep_grads, host_threads and opt_8bit "
           "are fixed when the model is created");
  MT_CHECK(!run->use_slab_pool || (m->slab_list.size() > 0 && (size_t)run->n_slabs == m->slab_list.size()),
           MT_E_INVALID,
           "mt_model_set_schedule: the slab pool (and its size) is allocated when the model is "
           "created; a model created without it can not switch it on");
  flush_pending(m);  // the pending updates belong to the old schedule's step
  m->resident_valid.clear();  // resident slots are refilled under the new schedule
  m->run = *run;
  return MT_OK;
}

int64_t mt_model_step_count(const mt_model* model) { return model ? model->step : -1; }

mt_status mt_model_kernel_times(const mt_model* model, mt_kernel_time* out, int32_t cap,
                                int32_t* n_out) {
  MT_CHECK(model && n_out && cap >= 0 && (out || cap == 0), MT_E_INVALID,
           "mt_model_kernel_times: null pointer or negative capacity");
  const int32_t n = (int32_t)model->kernel_times.size();
  for (int32_t i = 0; i < n && i < cap; ++i) out[i] = model->kernel_times[i];
  *n_out = n;
  return MT_OK;
}

mt_status mt_model_set_param(mt_model* m, const char* name, const float* src, size_t n) {
  MT_CHECK(m && src, MT_E_INVALID, "mt_model_set_param: null argument");
  TensorRef r;
  MT_CHECK(lookup_param(m, name, &r), MT_E_INVALID, "mt_model_set_param: unknown parameter '%s'",
           name ? name : "(null)");
  MT_CHECK(n == r.n, MT_E_SHAPE, "mt_model_set_param: '%s' has %zu elements, got %zu", name, r.n, n);
  flush_pending(m);  // a pending update must not land on the new value later
  m->resident_valid.assign(m->resident_valid.size(), 0);  // the device copies are stale now
  Unit& u = m->units[r.unit];
  const bool f32 = m->es == 4;
  if (m->run.opt_8bit) {  // fresh moments: zero codes and scales
    const Adam8Seg* s = find_segment(u, r.off);
    MT_CHECK(s && s->n == n, MT_E_STATE, "mt_model_set_param: no 8-bit segment for '%s'", name);
    memset(u.mq + r.off, 0, n);
    memset(u.rq + r.off, 0, n);
    memset(u.ms + s->sblk, 0, adam8_blocks(n) * 4);
    memset(u.rs + s->sblk, 0, adam8_blocks(n) * 4);
  }
  m->pool->parallel_for(n, [&](size_t lo, size_t hi) {
    memcpy(u.master + r.off + lo, src + lo, (hi - lo) * 4);
    if (u.m) memset(u.m + r.off + lo, 0, (hi - lo) * 4);
    if (u.v) memset(u.v + r.off + lo, 0, (hi - lo) * 4);
    if (f32) {
      memcpy(static_cast<float*>(u.shadow) + r.off + lo, src + lo, (hi - lo) * 4);
    } else {
      uint16_t* sh = static_cast<uint16_t*>(u.shadow) + r.off;
      for (size_t i = lo; i < hi; ++i) sh[i] = host_f2bf(src[i]);
    }
  });
  return MT_OK;
}

mt_status mt_model_get_param(const mt_model* m, const char* name, int32_t which, float* dst,
                             size_t n) {
  MT_CHECK(m && dst, MT_E_INVALID, "mt_model_get_param: null argument");
  TensorRef r;
  MT_CHECK(lookup_param(m, name, &r), MT_E_INVALID, "mt_model_get_param: unknown parameter '%s'",
           name ? name : "(null)");
  MT_CHECK(n == r.n, MT_E_SHAPE, "mt_model_get_param: '%s' has %zu elements, got %zu", name, r.n, n);
  // the model is observed: apply any update the last step left pending
  flush_pending(const_cast<mt_model*>(m));
  const Unit& u = m->units[r.unit];
  const bool embed = r.unit == m->cfg.n_layers + 1;
  // element i of a streamed-precision array (bf16 or fp32) as fp32
  auto elem = [&](const void* base, size_t i) {
    return m->es == 4 ? static_cast<const float*>(base)[i]
                      : host_bf2f(static_cast<const uint16_t*>(base)[i]);
  };
  switch (which) {
    case MT_GET_MASTER: memcpy(dst, u.master + r.off, n * 4); break;
    case MT_GET_M:
    case MT_GET_V:
      if (m->run.opt_8bit) {  // the values the 8-bit state holds
        const Adam8Seg* s = find_segment(u, r.off);
        MT_CHECK(s && s->n == n, MT_E_STATE, "mt_model_get_param: no 8-bit segment for '%s'",
                 name);
        if (which == MT_GET_M) adam8_dequant(u.mq, u.ms, *s, false, dst);
        else adam8_dequant(u.rq, u.rs, *s, true, dst);
      } else {
        memcpy(dst, (which == MT_GET_M ? u.m : u.v) + r.off, n * 4);
      }
      break;
    case MT_GET_SHADOW:
      for (size_t i = 0; i < n; ++i) dst[i] = elem(u.shadow, r.off + i);
      break;
    case MT_GET_GRAD:
      MT_CHECK(m->run.keep_grads, MT_E_STATE, "mt_model_get_param: gradients need keep_grads = 1");
      if (embed) memcpy(dst, m->dE + r.off, n * 4);
      else
        for (size_t i = 0; i < n; ++i) dst[i] = elem(u.kept, r.off + i);
      break;
    default: return set_error(MT_E_INVALID, "mt_model_get_param: bad 'which' %d", which);
  }
  return MT_OK;
}

}  // extern "C"
