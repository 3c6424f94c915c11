// The streamed training step (MegaTrain listing page, Abstract and Fig. 3;
// blog summary, sections 1-4): weights stream in per layer on a W stream,
// forward / recompute / backward run on a C stream, and each unit's
// gradient streams out on a G stream into a pinned slab, where a CPU thread
// runs Adam on that unit while the GPU goes on with the next layers.
//
// The schedule is built first as a pure plan (compute ops, weight loads,
// slot assignment and dependencies) that has no HIP in it, so its hazards
// can be checked on the CPU; one executor replays it with HIP events.
//
// Compute order: forward of every layer (keeping the input of layers
// l = 0 mod K), the head (final norm, LM head, loss, its backward), then
// the segments from the last: re-forward the segment's layers from its
// checkpoint to rebuild their inputs, then backward each layer in reverse.
// With kept internals the re-forward runs all K layers of the segment and
// keeps what their backward needs (no second forward per layer), and the
// last segment keeps them in the forward itself (no re-forward at all);
// without, the re-forward runs the first K-1 and each backward recomputes
// its layer's forward.  A weight slot is reused only after the last compute
// op that reads it has finished, and a load may run at most `depth` compute
// ops ahead of its first use (depth 2 = double buffering).  R layers
// (resident_layers: layers 1 .. R, or all of them) each have a slot of their
// own that one load fills for every op of the layer; after the layer's host
// update its new copy is uploaded there, so the next step skips that load.
// They come first in the forward so that their compute, which needs no
// transfer, covers the streamed layers' loads: with resident layers the
// forward loads may run as far ahead as the slots allow.  Layer 0 stays
// streamed because its update ends the step: its upload would add to the
// step's tail.
#include <math.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "kernels.h"
#include "layer.h"
#include "model.h"
#include "status.h"

namespace mt {

// OP_FWDK: forward of a layer of the last segment that keeps its internals
// (that segment's re-forward coincides with the forward itself).
enum OpKind { OP_FWD = 0, OP_HEAD = 1, OP_REFWD = 2, OP_BWD = 3, OP_FWDK = 4 };
struct PlanOp {
  int kind, layer, load;
};
struct PlanLoad {
  int unit, slot, first_use, last_use, wait_use, gate_use;
};
struct Plan {
  std::vector<PlanOp> ops;
  std::vector<PlanLoad> loads;
  int n_slots = 0;
  const char* error = nullptr;
};

static int plan_slots(int K, int depth) { return std::max(2, K + depth); }

int resident_first(int L, int R) { return R < L ? 1 : 0; }

Plan build_plan(int L, int K, int depth, int n_slots, bool keep, int R) {
  Plan p;
  const int rs = resident_first(L, R);  // resident layers rs .. rs + R - 1
  auto resident = [&](int l) { return l >= rs && l < rs + R; };
  p.n_slots = n_slots;
  auto add_load = [&](int unit) {
    p.loads.push_back({unit, -1, -1, -1, -1, -1});
    return (int)p.loads.size() - 1;
  };
  auto add_op = [&](int kind, int layer, int load) {
    const int i = (int)p.ops.size();
    p.ops.push_back({kind, layer, load});
    PlanLoad& ld = p.loads[load];
    if (ld.first_use < 0) ld.first_use = i;
    ld.last_use = i;
  };
  // with kept internals, the last segment's layers keep them already in the
  // forward, and their backward reuses the forward's weight loads
  const int a_last = ((L - 1) / K) * K;
  std::vector<int> fwd_load(L);
  for (int l = 0; l < L; ++l) {
    fwd_load[l] = add_load(l);
    add_op(keep && l >= a_last ? OP_FWDK : OP_FWD, l, fwd_load[l]);
  }
  add_op(OP_HEAD, -1, add_load(L));
  for (int a = a_last; a >= 0; a -= K) {
    const int e = std::min(a + K, L);
    if (keep && a == a_last) {
      for (int l = e - 1; l >= a; --l) add_op(OP_BWD, l, fwd_load[l]);
      continue;
    }
    std::vector<int> ld(e - a);
    for (int l = a; l < e; ++l) ld[l - a] = resident(l) ? fwd_load[l] : add_load(l);
    for (int l = a; l < (keep ? e : e - 1); ++l) add_op(OP_REFWD, l, ld[l - a]);
    for (int l = e - 1; l >= a; --l) add_op(OP_BWD, l, ld[l - a]);
  }
  std::vector<int> free_after(n_slots, -1);
  for (size_t j = 0; j < p.loads.size(); ++j) {
    PlanLoad& ld = p.loads[j];
    // forward loads run up to n_slots ops ahead when resident layers give
    // the link time to get ahead (slot reuse still waits for the readers)
    const int ahead = (R > 0 && ld.first_use < L) ? std::max(depth, n_slots) : depth;
    ld.gate_use = ld.first_use - ahead >= 0 ? ld.first_use - ahead : -1;
    if (ld.unit == L) {  // the head has a slot of its own
      ld.slot = -2;
      ld.wait_use = -1;
      // with resident layers, right behind the last layer's forward load
      if (R > 0 && j > 0) ld.gate_use = std::min(ld.gate_use, p.loads[j - 1].gate_use);
      continue;
    }
    if (resident(ld.unit)) {  // a resident layer's own slot
      ld.slot = -3 - (ld.unit - rs);
      ld.wait_use = -1;
      continue;
    }
    int best = 0;
    for (int s = 1; s < n_slots; ++s)
      if (free_after[s] < free_after[best]) best = s;
    ld.slot = best;
    ld.wait_use = free_after[best];
    if (ld.wait_use >= ld.first_use && !p.error) p.error = "too few weight slots for this schedule";
    free_after[best] = ld.last_use;
  }
  return p;
}

namespace {

constexpr int NG = 6;  // device gradient ring depth

// Device buffers of one step.  Weight slots, gradient buffers and
// activations hold the model's streamed element type (es bytes each).
struct Arena {
  std::vector<char*> res;  // resident layers' slots (first in the arena)
  std::vector<char*> slot;
  char* head_slot = nullptr;
  char* gring[NG] = {};
  char* head_grad = nullptr;
  char* act[2] = {};
  std::vector<char*> ckpt, seg;
  std::vector<char*> keep;  // kept internals, one per layer of a segment
  size_t keep_bytes = 0;
  char* dy = nullptr;
  // [NG + 1][2 * NONFINITE_BLOCKS]: ring slots, then the head; each slot the
  // finiteness flags, then the per-block sums of squares (fp32 bits)
  int32_t* flags = nullptr;
  int32_t* tgt = nullptr;
  float* loss = nullptr;
  void* lws = nullptr;
  size_t lws_bytes = 0;
  void* hws = nullptr;
  size_t hws_bytes = 0;
};

// Whether the step keeps the re-forward's internals for the backward (with
// a chunked MLP, those of the attention half).
bool keep_mode(const mt_model* M, const Dims&) { return M->run.keep_internals != 0; }

Arena carve_arena(const mt_model* M, const Dims& d, char* base, size_t* bytes) {
  Carve c{base};
  Arena a;
  const int L = M->cfg.n_layers, K = M->run.ckpt_interval;
  const size_t es = M->es;
  const size_t lay = M->ll.total * es, head = M->hl.total * es, act = (size_t)d.D * d.H * es;
  // resident slots first: their place must not depend on the step's shape
  for (int i = 0; i < M->run.resident_layers; ++i) a.res.push_back(c.take<char>(lay));
  const int ns = plan_slots(K, M->run.prefetch_depth);
  for (int i = 0; i < ns; ++i) a.slot.push_back(c.take<char>(lay));
  a.head_slot = c.take<char>(head);
  for (int i = 0; i < NG; ++i) a.gring[i] = c.take<char>(lay);
  a.head_grad = c.take<char>(head);
  a.act[0] = c.take<char>(act);
  a.act[1] = c.take<char>(act);
  for (int i = 0; i <= L / K; ++i) a.ckpt.push_back(c.take<char>(act));
  const bool keep = keep_mode(M, d);
  for (int i = 0; i < (keep ? K : K - 1); ++i) a.seg.push_back(c.take<char>(act));
  if (keep) {
    a.keep_bytes = layer_ws_bytes(d, 2);
    for (int i = 0; i < K; ++i) a.keep.push_back(c.take<char>(a.keep_bytes));
  }
  a.dy = c.take<char>(act);
  a.flags = c.take<int32_t>((size_t)(NG + 1) * 2 * NONFINITE_BLOCKS);
  a.tgt = c.take<int32_t>(d.D);
  a.loss = c.take<float>(64);
  a.lws_bytes = layer_ws_bytes(d, 1);
  a.lws = c.take<char>(a.lws_bytes);
  a.hws_bytes = head_ws_bytes(d);
  a.hws = c.take<char>(a.hws_bytes);
  *bytes = c.off + 256;
  return a;
}

mt_layer_view layer_view(const mt_model* M, const char* slab) {
  const LayerLayout& l = M->ll;
  const size_t es = M->es;
  mt_layer_view v;
  v.attn_norm = slab + l.attn_norm * es;
  v.w_qkv = slab + l.w_qkv * es;
  v.w_o = slab + l.w_o * es;
  v.mlp_norm = slab + l.mlp_norm * es;
  v.w_gate_up = slab + l.w_gate_up * es;
  v.w_down = slab + l.w_down * es;
  return v;
}

mt_layer_grad_view grad_view(const mt_model* M, char* slab) {
  const LayerLayout& l = M->ll;
  const size_t es = M->es;
  mt_layer_grad_view v;
  v.attn_norm = slab + l.attn_norm * es;
  v.w_qkv = slab + l.w_qkv * es;
  v.w_o = slab + l.w_o * es;
  v.mlp_norm = slab + l.mlp_norm * es;
  v.w_gate_up = slab + l.w_gate_up * es;
  v.w_down = slab + l.w_down * es;
  return v;
}

// Event pool handed out in order within one step.
struct Events {
  std::vector<hipEvent_t>* pool;
  size_t next = 0;
  mt_status err = MT_OK;
  hipEvent_t get() {
    if (next == pool->size()) {
      hipEvent_t e;
      if (hipEventCreateWithFlags(&e, hipEventBlockingSync) != hipSuccess) {
        err = MT_E_HIP;
        return nullptr;
      }
      pool->push_back(e);
    }
    return (*pool)[next++];
  }
};

float elapsed(hipEvent_t a, hipEvent_t b) {
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return 0.f;
  return ms;
}

struct Offload {
  int unit;          // -1 = dx0
  const char* src;
  size_t elems;
  const int32_t* dflags;  // device finiteness flags of the gradient (or null)
  hipEvent_t after;  // compute event the copy waits for
  int ring;          // gradient ring index or -1
  bool end = false;
};

struct Landed {
  int unit;
  void* host;      // slab, dx0 staging or the head's deferred-gradient buffer
  bool own_alloc;  // allocated for this transfer (no pool)
  hipEvent_t ev;
  bool end = false;
};

template <class T>
struct Queue {
  std::mutex mu;
  std::condition_variable cv;
  std::deque<T> q;
  void push(T v) {
    {
      std::lock_guard<std::mutex> lk(mu);
      q.push_back(v);
    }
    cv.notify_one();
  }
  T pop() {
    std::unique_lock<std::mutex> lk(mu);
    cv.wait(lk, [&] { return !q.empty(); });
    T v = q.front();
    q.pop_front();
    return v;
  }
};

#define MT_STEP_HIP(expr)                                                                     \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) {                                                                   \
      fail = set_error(MT_E_HIP, "mt_stream_step: %s failed: %s", #expr, hipGetErrorString(e_)); \
      goto drain;                                                                             \
    }                                                                                         \
  } while (0)

#define MT_STEP_RUN(expr)        \
  do {                           \
    mt_status s_ = (expr);       \
    if (s_ != MT_OK) {           \
      fail = s_;                 \
      goto drain;                \
    }                            \
  } while (0)

}  // namespace

size_t stream_arena_bytes(const mt_model* M, const Dims& d) {
  size_t b = 0;
  carve_arena(M, d, nullptr, &b);
  return b;
}

}  // namespace mt

using namespace mt;

extern "C" {

size_t mt_stream_arena_bytes(const mt_model* model, int32_t batch, int32_t seq) {
  if (!model) return 0;
  Dims d;
  if (make_dims(&model->cfg, &model->run, batch, seq, &d)) return 0;
  return stream_arena_bytes(model, d);
}

size_t mt_stream_arena_bytes_cfg(const mt_model_cfg* cfg, const mt_run_cfg* run, int32_t batch,
                                 int32_t seq) {
  Dims d0, d;
  if (!cfg || !run || make_dims(cfg, run, 1, 1, &d0) || make_dims(cfg, run, batch, seq, &d))
    return 0;
  if (run->ckpt_interval < 1 || run->prefetch_depth < 1 || run->prefetch_depth > 3 ||
      run->resident_layers < 0 || run->resident_layers > cfg->n_layers)
    return 0;
  // a model with its shape and knobs but no host store: the arena depends
  // on nothing else
  mt_model m;
  m.cfg = *cfg;
  m.run = *run;
  m.shape = d0;
  m.es = d0.es();
  m.ll = layer_layout(d0);
  m.hl = head_layout(d0);
  return stream_arena_bytes(&m, d);
}

// Diagnostic: the plan for L layers, checkpoint interval K, prefetch depth
// and resident layers.  out receives, for each compute op, (kind, layer, load) and then,
// for each load, (unit, slot, first_use, last_use, wait_use, gate_use);
// counts[0..2] = n_ops, n_loads, n_slots.  Returns MT_E_SHAPE if the plan is
// invalid, MT_E_OOM_HOST if out is too small.
mt_status mt_debug_plan(int32_t n_layers, int32_t ckpt_interval, int32_t prefetch_depth,
                        int32_t keep_internals, int32_t resident_layers, int32_t* out, size_t cap,
                        int32_t* counts) {
  MT_CHECK(n_layers >= 1 && ckpt_interval >= 1 && prefetch_depth >= 1 && resident_layers >= 0 &&
               resident_layers <= n_layers && out && counts,
           MT_E_INVALID, "mt_debug_plan: bad arguments");
  Plan p = build_plan(n_layers, ckpt_interval, prefetch_depth,
                      plan_slots(ckpt_interval, prefetch_depth), keep_internals != 0,
                      resident_layers);
  counts[0] = (int32_t)p.ops.size();
  counts[1] = (int32_t)p.loads.size();
  counts[2] = p.n_slots;
  const size_t need = 3 * p.ops.size() + 6 * p.loads.size();
  MT_CHECK(cap >= need, MT_E_OOM_HOST, "mt_debug_plan: need %zu entries", need);
  size_t k = 0;
  for (auto& o : p.ops) {
    out[k++] = o.kind;
    out[k++] = o.layer;
    out[k++] = o.load;
  }
  for (auto& l : p.loads) {
    out[k++] = l.unit;
    out[k++] = l.slot;
    out[k++] = l.first_use;
    out[k++] = l.last_use;
    out[k++] = l.wait_use;
    out[k++] = l.gate_use;
  }
  if (p.error) return set_error(MT_E_SHAPE, "mt_debug_plan: %s", p.error);
  return MT_OK;
}

mt_status mt_stream_step(mt_model* M, const int32_t* tokens, int32_t batch, int32_t seq,
                         void* arena, size_t arena_bytes, void* const streams[3],
                         float* loss_out, mt_step_stats* stats_out) {
  using clock = std::chrono::steady_clock;
  const auto t_begin = clock::now();
  MT_CHECK(M && tokens && arena && streams && loss_out, MT_E_INVALID,
           "mt_stream_step: null argument");
  MT_CHECK(!M->broken, MT_E_STATE, "mt_stream_step: the model was left inconsistent by an earlier failure");
  MT_CHECK(streams[0] && streams[1] && streams[2], MT_E_INVALID, "mt_stream_step: null stream");
  MT_CHECK(M->run.host_alloc == MT_HOST_PINNED, MT_E_INVALID,
           "mt_stream_step: needs a model created with pinned host memory");
  Dims d;
  if (const char* msg = make_dims(&M->cfg, &M->run, batch, seq, &d))
    return set_error(MT_E_SHAPE, "mt_stream_step: %s", msg);
  MT_CHECK(seq >= 2, MT_E_SHAPE, "mt_stream_step: seq must be >= 2 (next-token targets)");
  const int L = M->cfg.n_layers, K = M->run.ckpt_interval, V = d.V;
  for (int i = 0; i < d.D; ++i)
    MT_CHECK(tokens[i] >= 0 && tokens[i] < V, MT_E_INVALID,
             "mt_stream_step: token %d at position %d is outside [0, %d)", tokens[i], i, V);
  size_t need = 0;
  Arena A = carve_arena(M, d, static_cast<char*>(arena), &need);
  MT_CHECK(arena_bytes >= need, MT_E_OOM_DEVICE, "mt_stream_step: arena %zu < %zu bytes",
           arena_bytes, need);
  MT_CHECK(((uintptr_t)arena & 255) == 0, MT_E_INVALID, "mt_stream_step: arena must be 256-byte aligned");
  const bool keep = keep_mode(M, d);
  const int R = M->run.resident_layers, rs = resident_first(L, R);
  Plan plan = build_plan(L, K, M->run.prefetch_depth, plan_slots(K, M->run.prefetch_depth), keep, R);
  MT_CHECK(!plan.error, MT_E_INVALID, "mt_stream_step: %s", plan.error);

  if (!M->sdma) {
    std::unique_ptr<SdmaCopier> c(new SdmaCopier());
    const char* why = "";
    if (!c->init(&why)) return set_error(MT_E_HIP, "mt_stream_step: SDMA setup failed: %s", why);
    M->sdma = std::move(c);
  }
  // pinned per-step staging
  if (M->staging_tokens < (size_t)d.D) {
    const size_t nt = (size_t)d.D;
    M->x0_host = M->host_alloc(nt * d.H * M->es, true);
    M->dx0_host = M->host_alloc(nt * d.H * M->es, true);
    M->tgt_host = static_cast<int32_t*>(M->host_alloc(nt * 4, true));
    M->loss_host = static_cast<float*>(M->host_alloc(64, true));
    if (!M->flags_host)
      M->flags_host = static_cast<int32_t*>(
          M->host_alloc((size_t)(L + 1) * 2 * NONFINITE_BLOCKS * 4, true));
    MT_CHECK(M->flags_host, MT_E_OOM_HOST, "mt_stream_step: pinned flag allocation failed");
    MT_CHECK(M->x0_host && M->dx0_host && M->tgt_host && M->loss_host, MT_E_OOM_HOST,
             "mt_stream_step: pinned staging allocation failed");
    M->staging_tokens = nt;
  }

  const bool ser = M->run.serialize != 0;
  // MT_PROGRESS=1: a line on stderr as each unit's backward completes (long
  // steps, e.g. 256K-token contexts, otherwise print nothing for minutes)
  static const bool progress = [] {
    const char* e = getenv("MT_PROGRESS");
    return e && e[0] == '1';
  }();
  hipStream_t sC = static_cast<hipStream_t>(streams[1]);
  hipStream_t sW = ser ? sC : static_cast<hipStream_t>(streams[0]);
  hipStream_t sG = ser ? sC : static_cast<hipStream_t>(streams[2]);
  const int64_t t_step = M->step + 1;
  const AdamHp hp = adam_hp(M->run, t_step);
  Events ev{&M->events};
  mt_status fail = MT_OK;
  const size_t act = (size_t)d.D * d.H;
  const size_t es = M->es;
  const bool f32 = es == 4;
  // global-norm clipping: each unit's sum of squares comes with its
  // finiteness flags; the flags kernel runs for either
  const bool clipping = M->run.clip_norm > 0;
  const bool stats = M->run.check_finite || clipping;

  if (M->run.defer_updates && !M->pending.head_grad) {
    M->pending.head_grad = M->host_alloc(M->hl.total * M->es, true);
    MT_CHECK(M->pending.head_grad, MT_E_OOM_HOST,
             "mt_stream_step: pinned allocation of the head's gradient buffer failed");
  }
  // the embedding rows this batch touches (its gradient is zero elsewhere),
  // filled once the weight loads are under way
  std::vector<int32_t> rows_now;
  std::vector<uint8_t> touched((size_t)d.V, 0);
  const bool defer = M->run.defer_updates != 0;
  const Unit& emb = M->units[L + 1];
  const float inv_n = 1.f / (float)((size_t)d.B * (d.T - 1));

  // thread state
  Queue<Offload> offq;
  Queue<Landed> landq;
  std::mutex ring_mu;
  std::condition_variable ring_cv;
  std::atomic<bool> abort_all{false};
  std::atomic<int> g_fail{0}, a_fail{0};
  std::atomic<int64_t> units_updated{0};
  double adam_ms = 0.0;
  // clipping: each unit's gradient sum of squares (layers, head, embedding)
  std::vector<double> unit_ss((size_t)L + 2, 0.0);
  double last_clip = 1.0, last_norm = 0.0;
  double d2h_ms = 0, d2h_bytes = 0;
  double ring_wait_ms = 0, slab_wait_ms = 0, op_wait_ms = 0, adam_idle_ms = 0;
  double host_start_ms = 0, gpu_done_ms = 0, grads_landed_ms = 0, updates_done_ms = 0;
  auto ms_since = [](clock::time_point t) {
    return std::chrono::duration<double, std::milli>(clock::now() - t).count();
  };
  hipEvent_t loss_ev = nullptr;
  std::mutex ev_mu;  // guards the event pool across threads
  auto get_ev = [&]() {
    std::lock_guard<std::mutex> lk(ev_mu);
    return ev.get();
  };
  bool nonfinite_loss = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> h2d_ev;
  double h2d_bytes = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> wait_ev_f, wait_ev_b;
  Probe probe;
  hipEvent_t ph_start = nullptr, ph_fwd = nullptr, ph_head = nullptr, ph_end = nullptr;
  std::vector<hipEvent_t> op_done(plan.ops.size(), nullptr), load_done(plan.loads.size(), nullptr);
  // loader thread <-> enqueue (main): ops whose completion events are
  // recorded, loads whose copies are enqueued
  std::mutex load_mu;
  std::condition_variable load_cv;
  size_t ops_enqueued = 0, loads_issued = 0;
  std::atomic<int> w_fail{0};
  double h2d_load_bytes = 0;
  int bwd_count = 0;
  std::thread gthr, athr, wthr;
  // the previous step's head update must land before the head is streamed,
  // and a layer update it left (clipping) before the layer's first load
  std::mutex head_mu;
  std::condition_variable head_cv;
  bool head_done = !M->pending.head;
  std::vector<uint8_t> layer_pending((size_t)L, 0);
  for (const PendingAdam::Layer& x : M->pending.layers) layer_pending[x.unit] = 1;
  std::atomic<int64_t> units_deferred{0};
  std::mutex loss_mu;
  std::condition_variable loss_cv;
  bool loss_ready = false;
  // resident layers: which slots the previous step left current (read by
  // the loader), which this step refilled after the layer's update (written
  // by the optimizer thread)
  std::vector<uint8_t> res_valid, res_uploaded((size_t)R, 0);
  double res_bytes = 0;
  // host-to-device copies outside the loader, timed like its loads: the
  // step's input (main thread) and the resident uploads (optimizer thread)
  std::vector<std::pair<hipEvent_t, hipEvent_t>> x0_ev, res_ev;

  // --------------------------------------------------------- G thread
  // Waits on the host for each backward op, copies its gradient to a pinned
  // slab on an SDMA engine, then frees the ring slot and hands the slab to
  // the optimizer thread.
  long ring_done = 0;  // ring-buffer offloads whose copy has completed
  auto g_main = [&]() {
    for (;;) {
      Offload o = offq.pop();
      if (o.end) {
        landq.push(Landed{0, nullptr, false, nullptr, true});
        return;
      }
      void* host = nullptr;
      bool own = false;
      bool ok = !abort_all.load();
      if (ok) {
        if (o.unit < 0) {
          host = M->dx0_host;
        } else if (o.unit == L && defer) {
          host = M->pending.head_grad;  // free: the previous head update ran first
        } else if (M->run.use_slab_pool) {
          const auto tw = clock::now();
          host = M->slabs.acquire();
          slab_wait_ms += ms_since(tw);
        } else {
          ok = hipHostMalloc(&host, M->slab_elems * es, hipHostMallocDefault) == hipSuccess;
          own = ok;
        }
      }
      if (ok) {
        const auto tw = clock::now();
        ok = hipEventSynchronize(o.after) == hipSuccess;
        op_wait_ms += ms_since(tw);
        if (o.unit == 0 && o.ring >= 0) gpu_done_ms = ms_since(t_begin);
        if (ok && progress && o.unit >= 0)
          fprintf(stderr, "mt_stream_step: %s %d backward done at %.0f ms\n",
                  o.unit == L ? "head" : "layer", o.unit == L ? 0 : o.unit, ms_since(t_begin));
      }
      if (ok) {
        const auto t0 = clock::now();
        ok = M->sdma->copy_d2h(host, o.src, o.elems * es);
        if (ok && o.dflags)
          ok = M->sdma->copy_d2h(M->flags_host + (size_t)o.unit * 2 * NONFINITE_BLOCKS, o.dflags,
                                 2 * NONFINITE_BLOCKS * 4);
        d2h_ms += std::chrono::duration<double, std::milli>(clock::now() - t0).count();
        d2h_bytes += (double)o.elems * es;
        grads_landed_ms = ms_since(t_begin);
      }
      if (o.ring >= 0) {
        std::lock_guard<std::mutex> lk(ring_mu);
        ++ring_done;
        ring_cv.notify_all();
      }
      if (!ok) {
        if (!abort_all.load()) g_fail = M->sdma->ready() ? 1 : 2;
        abort_all = true;
        // after a copy that timed out the engine may still write the slab:
        // it is not handed back (the model is unusable from here on)
        if (host && o.unit >= 0 && !(o.unit == L && defer) && M->sdma->ready()) {
          if (own) hipHostFree(host);
          else M->slabs.release(host);
        }
        continue;
      }
      landq.push(Landed{o.unit, host, own, nullptr, false});
    }
  };

  // ------------------------------------------------------- W thread
  // Issues the weight loads in plan order.  Each load's dependencies (the
  // op that frees its slot, the look-ahead gate, the previous step's head
  // update) are waited for on the host, so no copy is ever submitted with
  // an unresolved wait: a copy waiting inside a copy engine's queue would
  // hold up every later copy the process submits to that engine, the
  // gradient offload's included.
  auto w_main = [&]() {
    auto publish = [&](size_t k) {
      {
        std::lock_guard<std::mutex> lk(load_mu);
        loads_issued = k;
      }
      load_cv.notify_all();
    };
    // wakes the enqueue on every way out (it may wait for a load that an
    // abort leaves unissued)
    struct Wake {
      std::mutex& mu;
      std::condition_variable& cv;
      ~Wake() {
        { std::lock_guard<std::mutex> lk(mu); }
        cv.notify_all();
      }
    } wake{load_mu, load_cv};
    for (size_t k = 0; k < plan.loads.size(); ++k) {
      const PlanLoad& ld = plan.loads[k];
      if (ld.slot <= -3 && res_valid[-3 - ld.slot]) {
        // left on the device by the previous step: nothing to copy
        if (hipEventRecord(load_done[k], sW) != hipSuccess) {
          w_fail = 1;
          abort_all = true;
          return;
        }
        publish(k + 1);
        continue;
      }
      const int need = std::max(ld.wait_use, ld.gate_use);
      {
        std::unique_lock<std::mutex> lk(load_mu);
        load_cv.wait(lk, [&] { return (int)ops_enqueued > need || abort_all.load(); });
      }
      if (abort_all.load()) return;
      bool ok = true;
      if (ld.wait_use >= 0) ok = hipEventSynchronize(op_done[ld.wait_use]) == hipSuccess;
      if (ok && ld.gate_use >= 0 && ld.gate_use != ld.wait_use)
        ok = hipEventSynchronize(op_done[ld.gate_use]) == hipSuccess;
      if (ok && ld.unit == L) {
        std::unique_lock<std::mutex> lk(head_mu);
        head_cv.wait(lk, [&] { return head_done; });
      } else if (ok && ld.unit >= 0 && ld.unit < L) {
        std::unique_lock<std::mutex> lk(head_mu);
        head_cv.wait(lk, [&] { return !layer_pending[ld.unit]; });
      }
      if (ok) {
        const Unit& u = M->units[ld.unit];
        char* dst = ld.slot >= 0 ? A.slot[ld.slot] : ld.slot == -2 ? A.head_slot : A.res[-3 - ld.slot];
        hipEvent_t c0 = get_ev(), c1 = get_ev();
        ok = c0 && c1 && hipEventRecord(c0, sW) == hipSuccess &&
             hipMemcpyAsync(dst, u.shadow, u.n * es, hipMemcpyHostToDevice, sW) == hipSuccess &&
             hipEventRecord(c1, sW) == hipSuccess &&
             hipEventRecord(load_done[k], sW) == hipSuccess;
        if (ok) {
          h2d_ev.push_back({c0, c1});
          h2d_load_bytes += (double)u.n * es;
        }
      }
      if (!ok) {
        w_fail = 1;
        abort_all = true;
        return;
      }
      publish(k + 1);
    }
  };

  // ------------------------------------------------------ Adam thread
  auto a_main = [&]() {
    // the previous step's deferred updates, while the GPU runs the forward
    {
      const auto t0 = clock::now();
      apply_pending_head(M);
      {
        std::lock_guard<std::mutex> lk(head_mu);
        head_done = true;
      }
      head_cv.notify_all();
      // layer 0 first: the forward streams the layers in order
      apply_pending_layers(M, [&](int unit) {
        {
          std::lock_guard<std::mutex> lk(head_mu);
          layer_pending[unit] = 0;
        }
        head_cv.notify_all();
      });
      apply_pending_embed_rest(M);
      adam_ms += std::chrono::duration<double, std::milli>(clock::now() - t0).count();
    }
    // clear the rows the previous step scattered into (dE is zero elsewhere)
    float* dE = M->dE;
    {
      const std::vector<int32_t>& prev = M->dE_rows;
      const size_t H = (size_t)d.H;
      M->pool->parallel_for(prev.size(), [&](size_t lo, size_t hi) {
        for (size_t i = lo; i < hi; ++i) memset(dE + (size_t)prev[i] * H, 0, H * 4);
      }, 64);
      M->dE_rows = rows_now;
    }
    bool checked = false;
    bool skip = false;
    // the first landing waits for the loss: a non-finite loss updates nothing
    auto check_loss = [&]() {
      if (checked) return;
      std::unique_lock<std::mutex> lk(loss_mu);
      loss_cv.wait(lk, [&] { return loss_ready; });
      checked = true;
      if (!loss_ev || hipEventSynchronize(loss_ev) != hipSuccess) {
        a_fail = 1;
        abort_all = true;
      } else if (M->run.check_finite && !std::isfinite(*M->loss_host)) {
        nonfinite_loss = true;
        abort_all = true;
      }
    };
    auto unit_bad = [&](int unit) {
      const int32_t* fl = M->flags_host + (size_t)unit * 2 * NONFINITE_BLOCKS;
      bool bad = false;
      for (int k = 0; k < NONFINITE_BLOCKS && M->run.check_finite; ++k) bad |= fl[k] != 0;
      return bad;
    };
    // dE from dx0 (rows of this batch only); true if a row is not finite
    auto embed_scatter = [&](const Landed& x) {
      if (f32)
        embed_scatter_add(static_cast<const float*>(x.host), tokens, (size_t)d.D, (size_t)d.H,
                          dE, M->pool.get());
      else
        embed_scatter_add(static_cast<const uint16_t*>(x.host), tokens, (size_t)d.D,
                          (size_t)d.H, dE, M->pool.get());
      bool bad = false;
      if (M->run.check_finite) {
        std::atomic<bool> any{false};
        const size_t H = (size_t)d.H;
        M->pool->parallel_for(rows_now.size(), [&](size_t lo, size_t hi) {
          for (size_t i = lo; i < hi && !any.load(std::memory_order_relaxed); ++i)
            if (!grad_finite(nullptr, dE + (size_t)rows_now[i] * H, H, nullptr)) any = true;
        }, 64);
        bad = any.load();
      }
      return bad;
    };
    float clip = 1.f;
    std::vector<Landed> held;  // with clipping: every landing, until the norm is known
    if (clipping) {
      double ss = 0.0;  // the whole gradient's sum of squares, in a fixed order
      bool bad = false;
      for (;;) {
        const auto tw = clock::now();
        Landed x = landq.pop();
        adam_idle_ms += ms_since(tw);
        if (x.end) break;
        check_loss();
        held.push_back(x);
        if (abort_all.load()) continue;
        const auto t0 = clock::now();
        if (x.unit >= 0) {
          bad |= unit_bad(x.unit);
          const float* sq = reinterpret_cast<const float*>(
              M->flags_host + (size_t)x.unit * 2 * NONFINITE_BLOCKS + NONFINITE_BLOCKS);
          double s = 0.0;
          for (int k = 0; k < NONFINITE_BLOCKS; ++k) s += (double)sq[k];
          unit_ss[x.unit] = s;
        } else {
          bad |= embed_scatter(x);
          double s = 0.0;
          const size_t H = (size_t)d.H;
          for (int32_t r : rows_now)
            for (size_t c = 0; c < H; ++c) s += (double)dE[(size_t)r * H + c] * dE[(size_t)r * H + c];
          unit_ss[L + 1] = s;
        }
        adam_ms += std::chrono::duration<double, std::milli>(clock::now() - t0).count();
      }
      if (bad) {
        a_fail = 2;
        abort_all = true;
      }
      for (int u = 0; u <= L + 1; ++u) ss += unit_ss[u];
      clip = (float)std::min(1.0, M->run.clip_norm / (std::sqrt(ss) + 1e-6));
      last_clip = clip;
      last_norm = std::sqrt(ss);
      held.push_back(Landed{0, nullptr, false, nullptr, true});
    }
    size_t next_held = 0;
    for (;;) {
      Landed x;
      if (clipping) {
        x = held[next_held++];
      } else {
        const auto tw = clock::now();
        x = landq.pop();
        adam_idle_ms += ms_since(tw);
      }
      if (x.end) {
        updates_done_ms = ms_since(t_begin);
        return;
      }
      check_loss();
      skip = skip || abort_all.load();
      const auto t0 = clock::now();
      bool left_pending = false;  // the gradient stays with a pending update
      if (!skip) {
        if (x.unit >= 0) {
          Unit& u = M->units[x.unit];
          const uint16_t* gb = f32 ? nullptr : static_cast<const uint16_t*>(x.host);
          const float* gf = f32 ? static_cast<const float*>(x.host) : nullptr;
          const bool bad = unit_bad(x.unit);
          if (bad) {
            a_fail = 2;
            abort_all = true;
            skip = true;
          } else if (defer && x.unit == L) {
            // the head's update waits for the next step (PendingAdam)
            if (u.kept) memcpy(u.kept, x.host, u.n * es);
            M->pending.head = true;  // its gradient stays in pending.head_grad
            M->pending.hp_head = hp;
            M->pending.clip_head = clip;
            ++units_deferred;
          } else if (defer && clipping) {
            // the update runs at the start of the next step (PendingAdam)
            if (u.kept) memcpy(u.kept, x.host, u.n * es);
            M->pending.layers.push_back({x.unit, x.host, x.own_alloc});
            M->pending.hp_layers = hp;
            M->pending.clip_layers = clip;
            left_pending = true;
            ++units_deferred;
          } else {
            unit_adam(M, x.unit, gb, gf, hp, clip);
            if (u.kept) memcpy(u.kept, x.host, u.n * es);
            ++units_updated;
            if (x.unit >= rs && x.unit < rs + R) {
              // a resident layer: its updated copy goes to its slot now, for
              // the next step (every op of this step that reads the slot has
              // finished: its gradient has landed)
              const int c = x.unit - rs;
              hipEvent_t c0 = get_ev(), c1 = get_ev();
              if (c0 && c1 && hipEventRecord(c0, sW) == hipSuccess &&
                  hipMemcpyAsync(A.res[c], u.shadow, u.n * es, hipMemcpyHostToDevice, sW) ==
                      hipSuccess &&
                  hipEventRecord(c1, sW) == hipSuccess) {
                res_uploaded[c] = 1;
                res_bytes += (double)u.n * es;
                res_ev.push_back({c0, c1});
              } else {
                a_fail = 1;
                abort_all = true;
                skip = true;
              }
            }
          }
        } else {
          // only the batch's rows of dE can be nonzero, hence non-finite
          // (with clipping dE was formed, and checked, while collecting)
          const bool bad = clipping ? false : embed_scatter(x);
          if (bad) {
            a_fail = 2;
            abort_all = true;
            skip = true;
          } else {
            // the update of every row (untouched rows with a zero gradient)
            M->pending.embed = true;
            M->pending.hp_embed = hp;
            M->pending.clip_embed = clip;
            M->pending.row_done.assign((size_t)d.V, 0);
            M->pending.touched = touched;
            if (defer) {
              ++units_deferred;  // applied by the next step (PendingAdam)
            } else {
              apply_pending_embed_rest(M);
              ++units_updated;
            }
          }
        }
      }
      adam_ms += std::chrono::duration<double, std::milli>(clock::now() - t0).count();
      if (x.unit >= 0 && !(x.unit == L && defer) && !left_pending) {
        if (x.own_alloc) hipHostFree(x.host);
        else M->slabs.release(x.host);
      }
    }
  };

  // ---------------------------------------------------- enqueue (main)
  loss_ev = get_ev();
  ph_start = get_ev();
  ph_fwd = get_ev();
  ph_head = get_ev();
  ph_end = get_ev();
  hipEvent_t x0_ready = get_ev();
  for (auto& e : op_done) e = get_ev();
  for (auto& e : load_done) e = get_ev();
  if (M->run.time_kernels) {
    // every GEMM and attention launch of the step: per layer forward
    // (2 GEMMs + 1 attention + 2 GEMMs per MLP chunk, run up to twice:
    // forward and segment re-forward) and recompute+backward (a forward's
    // 3 + 1 per chunk, 4 GEMMs + 3 attention + 5 GEMMs per MLP chunk), and
    // 3 per head chunk
    const size_t nmc = (d.D + d.mlp_chunk - 1) / d.mlp_chunk;
    const size_t nhc = (d.D + d.head_chunk - 1) / d.head_chunk;
    const size_t launches =
        (size_t)L * (2 * (3 + 2 * nmc) + (3 + nmc) + 7 + 5 * nmc) + 3 * nhc + 8;
    probe.ev.resize(2 * launches);
    for (auto& e : probe.ev) e = get_ev();
  }
  if (ev.err != MT_OK) return set_error(MT_E_HIP, "mt_stream_step: event creation failed");

  // the resident slots hold current copies only if the previous step left
  // them in this same arena; until this step's uploads land, none does
  if (M->resident_arena != arena || (int)M->resident_valid.size() != R)
    M->resident_valid.assign((size_t)R, 0);
  res_valid = M->resident_valid;
  M->resident_valid.assign((size_t)R, 0);
  M->resident_arena = arena;

  {
    // gradient buffers: pads must read as zero
    MT_STEP_HIP(hipMemsetAsync(A.head_grad, 0, M->hl.total * es, sC));
    for (int i = 0; i < NG; ++i) MT_STEP_HIP(hipMemsetAsync(A.gring[i], 0, M->ll.total * es, sC));
    // the first weight loads go out now, while the host prepares the input
    wthr = std::thread(w_main);
    // the previous step's embedding update, for the rows this batch gathers
    // (the other rows follow on the optimizer thread during the forward;
    // this must precede that thread)
    apply_pending_embed_rows(M, tokens, (size_t)d.D);
    for (int i = 0; i < d.D; ++i)
      if (!touched[tokens[i]]) {
        touched[tokens[i]] = 1;
        rows_now.push_back(tokens[i]);
      }
    // targets and the embedding gather (from the streamed copy)
    for (int b = 0; b < d.B; ++b)
      for (int t = 0; t < d.T; ++t)
        M->tgt_host[(size_t)b * d.T + t] = t + 1 < d.T ? tokens[(size_t)b * d.T + t + 1] : -1;
    embed_gather(emb.shadow, tokens, (size_t)d.D, (size_t)d.H * es, M->x0_host, M->pool.get());
    gthr = std::thread(g_main);
    athr = std::thread(a_main);
    host_start_ms = ms_since(t_begin);
    MT_STEP_HIP(hipEventRecord(ph_start, sC));
    // inputs of the step, on the G stream: idle until the backward, while
    // the W stream is already busy with weights
    x0_ev.push_back({get_ev(), x0_ready});
    MT_STEP_HIP(hipEventRecord(x0_ev[0].first, sG));
    MT_STEP_HIP(hipMemcpyAsync(A.ckpt[0], M->x0_host, act * es, hipMemcpyHostToDevice, sG));
    MT_STEP_HIP(hipMemcpyAsync(A.tgt, M->tgt_host, (size_t)d.D * 4, hipMemcpyHostToDevice, sG));
    MT_STEP_HIP(hipEventRecord(x0_ready, sG));
    h2d_bytes += (double)act * es + (double)d.D * 4;
    MT_STEP_HIP(hipStreamWaitEvent(sC, x0_ready, 0));

    auto xloc = [&](int i) -> char* { return (i % K == 0) ? A.ckpt[i / K] : A.act[i % 2]; };

    for (size_t i = 0; i < plan.ops.size(); ++i) {
      const PlanOp& op = plan.ops[i];
      {
        // every op before this one has its completion event recorded; wait
        // until the loader has enqueued this op's weights
        std::unique_lock<std::mutex> lk(load_mu);
        ops_enqueued = i;
        load_cv.notify_all();
        load_cv.wait(lk, [&] { return loads_issued > (size_t)op.load || abort_all.load(); });
      }
      if (abort_all.load()) {
        if (w_fail.load()) fail = set_error(MT_E_HIP, "mt_stream_step: weight load failed");
        goto drain;  // otherwise the failing thread's status is reported below
      }
      const PlanLoad& ld = plan.loads[op.load];
      const char* w =
          ld.slot >= 0 ? A.slot[ld.slot] : ld.slot == -2 ? A.head_slot : A.res[-3 - ld.slot];
      // wait for this op's weights; the gap is the exposed transfer time
      hipEvent_t w0 = get_ev(), w1 = get_ev();
      MT_STEP_HIP(hipEventRecord(w0, sC));
      MT_STEP_HIP(hipStreamWaitEvent(sC, load_done[op.load], 0));
      MT_STEP_HIP(hipEventRecord(w1, sC));
      (op.kind == OP_BWD ? wait_ev_b : wait_ev_f).push_back({w0, w1});
      if (op.kind == OP_FWDK) {
        // the last segment: inputs land in the segment buffers the backward
        // reads, the last layer's output where the head reads it
        const int l = op.layer, a = (l / K) * K;
        const char* in = l == a ? A.ckpt[a / K] : A.seg[l - a - 1];
        char* out = l == L - 1 ? xloc(L) : A.seg[l - a];
        MT_STEP_RUN(layer_fwd_keep_impl(d, layer_view(M, w), in, out, A.keep[l - a],
                                        A.keep_bytes, sC, M->run.time_kernels ? &probe : nullptr));
        if (l == L - 1) MT_STEP_HIP(hipEventRecord(ph_fwd, sC));
      } else if (op.kind == OP_FWD) {
        const int l = op.layer;
        MT_STEP_RUN(layer_fwd_impl(d, layer_view(M, w), xloc(l), xloc(l + 1), A.lws, A.lws_bytes,
                                   sC, M->run.time_kernels ? &probe : nullptr));
        if (l == L - 1) MT_STEP_HIP(hipEventRecord(ph_fwd, sC));
      } else if (op.kind == OP_HEAD) {
        MT_STEP_RUN(head_impl(d, w + M->hl.final_norm * es, w + M->hl.lm_head * es, xloc(L), A.tgt,
                              inv_n, A.dy, A.head_grad + M->hl.final_norm * es,
                              A.head_grad + M->hl.lm_head * es, A.loss, A.hws, A.hws_bytes, sC,
                              M->run.time_kernels ? &probe : nullptr));
        MT_STEP_HIP(hipMemcpyAsync(M->loss_host, A.loss, 4, hipMemcpyDeviceToHost, sC));
        MT_STEP_HIP(hipEventRecord(loss_ev, sC));
        {
          std::lock_guard<std::mutex> lk(loss_mu);
          loss_ready = true;
        }
        loss_cv.notify_all();
        MT_STEP_HIP(hipEventRecord(ph_head, sC));
        int32_t* hf = A.flags + (size_t)NG * 2 * NONFINITE_BLOCKS;
        if (stats)
          MT_STEP_HIP(nonfinite_flags(A.head_grad, M->hl.total * es, f32, hf, sC,
                                      clipping ? reinterpret_cast<float*>(hf + NONFINITE_BLOCKS)
                                               : nullptr));
        MT_STEP_HIP(hipEventRecord(op_done[i], sC));
        offq.push(Offload{L, A.head_grad, M->hl.total, stats ? hf : nullptr, op_done[i], -1});
        continue;
      } else if (op.kind == OP_REFWD) {
        const int l = op.layer, a = (l / K) * K;
        const char* in = l == a ? A.ckpt[a / K] : A.seg[l - a - 1];
        if (keep)
          MT_STEP_RUN(layer_fwd_keep_impl(d, layer_view(M, w), in, A.seg[l - a], A.keep[l - a],
                                          A.keep_bytes, sC,
                                          M->run.time_kernels ? &probe : nullptr));
        else
          MT_STEP_RUN(layer_fwd_impl(d, layer_view(M, w), in, A.seg[l - a], A.lws, A.lws_bytes, sC,
                                     M->run.time_kernels ? &probe : nullptr));
      } else {  // OP_BWD
        const int l = op.layer, a = (l / K) * K;
        const char* in = l == a ? A.ckpt[a / K] : A.seg[l - a - 1];
        const int r = bwd_count % NG;
        if (bwd_count >= NG) {  // the ring slot's previous gradient must have left
          const auto tw = clock::now();
          std::unique_lock<std::mutex> lk(ring_mu);
          ring_cv.wait(lk, [&] { return ring_done >= bwd_count - NG + 1 || abort_all.load(); });
          ring_wait_ms += ms_since(tw);
          if (abort_all.load()) goto drain;  // the failing thread's status is reported below
        }
        if (keep)
          MT_STEP_RUN(layer_bwd_saved_impl(d, layer_view(M, w), in, A.dy, A.dy,
                                           grad_view(M, A.gring[r]), A.keep[l - a], A.keep_bytes,
                                           A.lws, A.lws_bytes, sC,
                                           M->run.time_kernels ? &probe : nullptr));
        else
          MT_STEP_RUN(layer_bwd_impl(d, layer_view(M, w), in, A.dy, A.dy, grad_view(M, A.gring[r]),
                                     A.lws, A.lws_bytes, sC,
                                     M->run.time_kernels ? &probe : nullptr));
        int32_t* lf = A.flags + (size_t)r * 2 * NONFINITE_BLOCKS;
        if (stats)
          MT_STEP_HIP(nonfinite_flags(A.gring[r], M->ll.total * es, f32, lf, sC,
                                      clipping ? reinterpret_cast<float*>(lf + NONFINITE_BLOCKS)
                                               : nullptr));
        MT_STEP_HIP(hipEventRecord(op_done[i], sC));
        if (l == 0) {
          MT_STEP_HIP(hipEventRecord(ph_end, sC));
          // dx0, the gradient of the embedding output, leaves before layer
          // 0's gradient: its scatter-add then runs while that larger copy
          // is still on the link instead of after the last Adam update
          offq.push(Offload{-1, A.dy, act, nullptr, ph_end, -1});
        }
        Offload o{l, A.gring[r], M->ll.total, stats ? lf : nullptr, op_done[i], r};
        offq.push(o);
        ++bwd_count;
        continue;
      }
      MT_STEP_HIP(hipEventRecord(op_done[i], sC));
    }
    {
      std::lock_guard<std::mutex> lk(load_mu);
      ops_enqueued = plan.ops.size();
    }
    load_cv.notify_all();
  }
drain:
  if (fail != MT_OK || abort_all.load()) {
    abort_all = true;
    {
      std::lock_guard<std::mutex> lk(loss_mu);
      loss_ready = true;
    }
    loss_cv.notify_all();
  }
  {
    std::lock_guard<std::mutex> lk(load_mu);  // the loader sees abort_all or every op
  }
  load_cv.notify_all();
  if (wthr.joinable()) wthr.join();
  offq.push(Offload{0, nullptr, 0, nullptr, nullptr, -1, true});
  if (gthr.joinable()) gthr.join();
  if (athr.joinable()) athr.join();
  const hipError_t e1 = hipStreamSynchronize(sW), e2 = hipStreamSynchronize(sC),
                   e3 = hipStreamSynchronize(sG);
  if (fail == MT_OK && (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess)) {
    fail = set_error(MT_E_HIP, "mt_stream_step: asynchronous HIP error: %s",
                     hipGetErrorString(e1 != hipSuccess ? e1 : e2 != hipSuccess ? e2 : e3));
  }
  if (fail == MT_OK && w_fail.load())
    fail = set_error(MT_E_HIP, "mt_stream_step: weight load failed");
  if (fail == MT_OK && g_fail.load() == 2)
    fail = set_error(MT_E_HIP, "mt_stream_step: a gradient copy to the host did not complete "
                               "within %.0f s", SdmaCopier::COPY_TIMEOUT_S);
  if (fail == MT_OK && (g_fail.load() || a_fail.load() == 1))
    fail = set_error(MT_E_HIP, "mt_stream_step: gradient offload or optimizer thread failed");
  if (fail == MT_OK && nonfinite_loss)
    fail = set_error(MT_E_NONFINITE, "mt_stream_step: loss is not finite; nothing was updated");
  if (fail == MT_OK && a_fail.load() == 2)
    fail = set_error(MT_E_NONFINITE, "mt_stream_step: a gradient is not finite; %lld units were updated",
                     (long long)units_updated.load());
  *loss_out = *M->loss_host;
  if (fail != MT_OK) {
    // an update this step deferred belongs to a step that did not complete
    if (units_deferred.load() > 0) drop_pending(M);
    if (units_updated.load() > 0) M->broken = true;
    return fail;
  }
  M->step = t_step;
  M->resident_valid = res_uploaded;  // the uploads completed with the W stream
  if (stats_out) {
    mt_step_stats& s = *stats_out;
    memset(&s, 0, sizeof(s));
    s.fwd_ms = elapsed(ph_start, ph_fwd);
    s.head_ms = elapsed(ph_fwd, ph_head);
    s.bwd_ms = elapsed(ph_head, ph_end);
    s.adam_ms = adam_ms;
    for (auto& p : h2d_ev) s.h2d_ms += elapsed(p.first, p.second);
    for (auto& p : x0_ev) s.h2d_ms += elapsed(p.first, p.second);
    for (auto& p : res_ev) s.h2d_ms += elapsed(p.first, p.second);
    s.d2h_ms = d2h_ms;
    for (auto& p : wait_ev_f) s.exposed_wait_fwd_ms += elapsed(p.first, p.second);
    for (auto& p : wait_ev_b) s.exposed_wait_bwd_ms += elapsed(p.first, p.second);
    {
      // group the timed launches by kernel (GEMM instantiation or attention
      // kernel); report the one with the largest total time, keep all
      struct Agg { double ms = 0, flops = 0; int64_t n = 0; };
      std::map<std::string, Agg> by;
      for (int i = 0; i + 1 < probe.used; i += 2) {
        const double ms = elapsed(probe.ev[i], probe.ev[i + 1]);
        const std::string& name = probe.name[i / 2];
        Agg& g = by[name];
        g.ms += ms;
        g.flops += probe.flops[i / 2];
        ++g.n;
        if (name.compare(0, 4, "attn") == 0) s.probe_all_attn_ms += ms;
        else s.probe_all_gemm_ms += ms;
        s.probe_all_flops += probe.flops[i / 2];
      }
      M->kernel_times.clear();
      for (auto& kv : by) {
        mt_kernel_time k{};
        snprintf(k.name, sizeof k.name, "%s", kv.first.c_str());
        k.launches = kv.second.n;
        k.ms = kv.second.ms;
        k.flops = kv.second.flops;
        M->kernel_times.push_back(k);
      }
      std::sort(M->kernel_times.begin(), M->kernel_times.end(),
                [](const mt_kernel_time& a, const mt_kernel_time& b) { return a.ms > b.ms; });
      if (!M->kernel_times.empty()) {
        const mt_kernel_time& top = M->kernel_times.front();
        s.probe_kernel_ms = top.ms;
        s.probe_kernel_flops = top.flops;
        s.probe_kernel_launches = top.launches;
        snprintf(s.probe_kernel, sizeof s.probe_kernel, "%s", top.name);
      }
    }
    s.grad_norm = last_norm;
    s.clip_factor = last_clip;
    s.h2d_bytes = h2d_bytes + h2d_load_bytes + res_bytes;
    s.d2h_bytes = d2h_bytes;
    s.pinned_host_bytes = M->pinned_bytes;
    s.pageable_host_bytes = M->pageable_bytes;
    s.device_arena_bytes = (int64_t)need;
    s.units_updated = units_updated.load() + units_deferred.load();
    s.step_ms = std::chrono::duration<double, std::milli>(clock::now() - t_begin).count();
    s.tail_ms = s.step_ms - (s.fwd_ms + s.head_ms + s.bwd_ms);
    s.host_ring_wait_ms = ring_wait_ms;
    s.host_start_ms = host_start_ms;
    s.gpu_done_ms = gpu_done_ms;
    s.grads_landed_ms = grads_landed_ms;
    s.updates_done_ms = updates_done_ms;
    s.host_slab_wait_ms = slab_wait_ms;
    s.host_op_wait_ms = op_wait_ms;
    s.host_adam_idle_ms = adam_idle_ms;
  }
  return MT_OK;
}

}  // extern "C"
