// The host-resident model: the authoritative flat store of fp32 master
// weights and Adam moments, the pinned copy that streams to the GPU (bf16,
// or fp32 in the debug precision), the pinned gradient slab pool, and the
// per-step scratch the engine uses.
#pragma once

#include <hip/hip_runtime_api.h>

#include <condition_variable>
#include <deque>
#include <functional>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "host.h"
#include "layer.h"
#include "mt.h"
#include "sdma.h"

namespace mt {

// Units: 0..L-1 layers, L = head (final norm + LM head), L+1 = embedding.
// Element types of the streamed copy, slabs and kept gradients follow the
// model's precision: bf16 bit patterns (uint16_t) or fp32.
struct Unit {
  size_t n = 0;               // elements (with alignment padding)
  float* master = nullptr;    // fp32, pageable
  float* m = nullptr;         // fp32 Adam moments (without opt_8bit)
  float* v = nullptr;
  uint8_t* mq = nullptr;      // hybrid 8-bit moments (opt_8bit): codes of m and
  uint8_t* rq = nullptr;      // of r = sqrt(v), and their per-block scales
  float* ms = nullptr;
  float* rs = nullptr;
  std::vector<Adam8Seg> segs; // the unit's tensors (8-bit blocks never span two)
  void* shadow = nullptr;     // streamed copy, inside the pinned shadow region
  void* kept = nullptr;       // last step's gradient (keep_grads)
};

struct TensorRef {
  int unit;
  size_t off, n;
};

// Pool of pinned gradient slabs shared by the offload and optimizer threads.
class SlabPool {
 public:
  void init(std::vector<void*> slabs) { free_ = std::move(slabs); }
  void* acquire();
  void release(void* p);
  size_t capacity() const { return total_; }
  void set_total(size_t t) { total_ = t; }

 private:
  std::mutex mu_;
  std::condition_variable cv_;
  std::vector<void*> free_;
  size_t total_ = 0;
};

// Optimizer updates a step leaves for the next one to apply (the LM head
// and the embedding: their weights are needed late in the next forward, or
// for only a few rows at its start, so their host Adam runs while the next
// forward streams the other units instead of after this step's backward).
// With global-norm clipping the layers' updates are left too: none can run
// before the last gradient has landed, so they run while the next forward
// streams, each before its layer's first weight load.  Every reader of the
// model applies them first (flush_pending).
struct PendingAdam {
  bool head = false, embed = false;
  AdamHp hp_head{}, hp_embed{};
  float clip_head = 1.f, clip_embed = 1.f;  // the step's clipping factor
  struct Layer {
    int unit;
    void* grad;      // the landed gradient (a pool slab, or its own pinned buffer)
    bool own_alloc;  // allocated for the transfer (no pool): freed after the update
  };
  std::vector<Layer> layers;
  AdamHp hp_layers{};
  float clip_layers = 1.f;
  // the head's gradient lands in a pinned buffer of its own (never a pool
  // slab: holding a slab across units would stall the offload of the rest
  // of the step when the pool is small)
  void* head_grad = nullptr;
  std::vector<uint8_t> row_done;  // embedding rows already updated
  std::vector<uint8_t> touched;   // embedding rows with a nonzero gradient row in dE
};

struct HostBlock {  // one host allocation
  void* p = nullptr;
  size_t bytes = 0;
  bool pinned = false;
};

}  // namespace mt

struct mt_model {
  mt_model_cfg cfg{};
  mt_run_cfg run{};
  mt::Dims shape{};  // model dims (B = T = 1); per-step dims are rebuilt
  mt::LayerLayout ll{};
  mt::HeadLayout hl{};
  std::vector<mt::Unit> units;
  std::vector<mt::HostBlock> blocks;
  size_t es = 2;  // bytes per streamed element (2: bf16, 4: fp32 debug)
  size_t slab_elems = 0;
  mt::SlabPool slabs;
  std::vector<void*> slab_list;
  std::unique_ptr<mt::ThreadPool> pool;
  float* dE = nullptr;          // fp32 embedding gradient [V, H]; zero outside dE_rows
  std::vector<int32_t> dE_rows; // rows the last step scattered into dE
  float* zero_row = nullptr;    // H zeros: the gradient row of an untouched embedding row
  int32_t* flags_host = nullptr;  // pinned, (n_layers + 1) x NONFINITE_BLOCKS per-unit flags
  // pinned per-step staging, grown on demand
  void* x0_host = nullptr;
  void* dx0_host = nullptr;
  int32_t* tgt_host = nullptr;
  float* loss_host = nullptr;
  size_t staging_tokens = 0;
  std::vector<hipEvent_t> events;  // grown on demand
  std::unique_ptr<mt::SdmaCopier> sdma;  // gradient offload engine (created on first step)
  mt::PendingAdam pending;
  // resident layers (mt_run_cfg.resident_layers): which of the resident
  // slots at the start of resident_arena hold their layer's current
  // streamed copy, left there by the previous step
  std::vector<uint8_t> resident_valid;
  const void* resident_arena = nullptr;
  // the last step's timed kernel launches (time_kernels), grouped by kernel
  std::vector<mt_kernel_time> kernel_times;
  int64_t step = 0;
  bool broken = false;
  int64_t pinned_bytes = 0, pageable_bytes = 0;

  void* host_alloc(size_t bytes, bool pinned);
  ~mt_model();
};

namespace mt {
bool lookup_param(const mt_model* m, const char* name, TensorRef* out);
// Pending head / embedding updates (PendingAdam): apply the head's; apply the
// embedding's for the rows of `ids` only (marking them done) or for every row
// not yet done; apply everything and clear (flush_pending).  Each uses the
// model's thread pool, so callers must not overlap them with other pool work.
void apply_pending_head(mt_model* m);
void apply_pending_embed_rows(mt_model* m, const int32_t* ids, size_t n);
void apply_pending_embed_rest(mt_model* m);
// The pending layer updates in layer order, calling done(unit) after each.
void apply_pending_layers(mt_model* m, const std::function<void(int)>& done);
void flush_pending(mt_model* m);
void drop_pending(mt_model* m);
// Adam (fp32 or hybrid 8-bit moments, per the model) over a whole unit with
// gradient gb (bf16) or gf (fp32), writing the streamed copy.
void unit_adam(mt_model* m, int unit, const uint16_t* gb, const float* gf, const AdamHp& hp,
               float clip);
}
