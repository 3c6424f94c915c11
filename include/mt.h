/*
 * mt.h — C ABI of libmt, the MI355X (gfx950) layer-streamed training step.
 *
 * What it computes: one full-batch training step of a pre-norm GQA decoder
 * whose fp32 parameters and Adam states live in host memory, with the GPU
 * used as a transient compute engine that receives each layer's weights,
 * computes, and sends the layer's gradient back (MegaTrain listing page,
 * Abstract; blog summary, sections 1 and 2).  Weights are bound into a
 * stateless layer template at call time instead of living in a persistent
 * autograd graph (Abstract; blog summary, section 4).  Activations are
 * recomputed from checkpoints kept every K layers (blog summary, section 3).
 * The optimizer step runs on the CPU (blog summary, section 1).
 *
 * Conventions for every call:
 *  - Every call returns mt_status; no C++ exception crosses the ABI.  On a
 *    non-OK return mt_last_error() gives a message (thread-local, valid
 *    until the next failing call on the same thread).
 *  - Arguments are validated before any GPU work is enqueued: a failed
 *    validation enqueues nothing and leaves every buffer and model state as
 *    it was.
 *  - Device pointers are plain HIP device addresses (e.g. a torch tensor's
 *    data_ptr()); streams are hipStream_t values passed as void*.  The
 *    caller owns every pointer it passes and keeps it alive until the work
 *    enqueued on the given stream(s) has finished.
 *  - Activations are token-major row-major: a [D, C] matrix has D = B*T rows
 *    (batch-major, then position) and C contiguous columns.  Weights are
 *    [out, in] row-major, so a linear layer is y = x W^T.
 *  - dtype: bf16 storage (round to nearest even) with fp32 accumulation,
 *    unless a run config selects MT_PREC_FP32_DEBUG, in which case every
 *    buffer the calls below describe as bf16 holds fp32 instead.
 *  - A model handle is not thread-safe; distinct handles are independent.
 */
#ifndef MT_H
#define MT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MT_OK = 0,
  MT_E_INVALID = -1,    /* null pointer, bad enum or knob value */
  MT_E_SHAPE = -2,      /* shape not supported or inconsistent */
  MT_E_OOM_DEVICE = -3, /* caller buffer too small */
  MT_E_OOM_HOST = -4,   /* host (pinned or pageable) allocation failed */
  MT_E_HIP = -5,        /* a HIP runtime call failed */
  MT_E_NONFINITE = -6,  /* loss or gradient not finite (nothing updated) */
  MT_E_STATE = -7       /* model unusable after an earlier failure */
} mt_status;

enum { MT_DT_BF16 = 0, MT_DT_F32 = 1 };
enum { MT_PREC_BF16 = 0, MT_PREC_FP32_DEBUG = 1 };
enum { MT_HOST_PINNED = 0, MT_HOST_PAGEABLE = 1 };

/* Decoder shape (Qwen2.5 shape, MegaTrain listing page, Table 2).
 * Constraints: head_dim in {64, 128}; n_heads % n_kv_heads == 0;
 * hidden, ffn, vocab multiples of 64. */
typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;
  double rope_theta;
} mt_model_cfg;

/* Knobs of one run.  The ablation of the listing page (Table 4) varies the
 * checkpoint interval, double buffering (prefetch_depth 1 vs 2) and the
 * gradient slab pool; chunked MLP execution is Table 7's note on the
 * longest contexts.  Zero means "default" where a default is stated. */
typedef struct {
  int32_t ckpt_interval;     /* K >= 1 (default 4) */
  int32_t prefetch_depth;    /* weight slots ahead of compute: 1, 2 or 3 (default 2) */
  int32_t use_slab_pool;     /* 1: recycle pinned gradient slabs (default); 0: one slab per unit */
  int32_t n_slabs;           /* pool size when use_slab_pool (default 8) */
  int32_t mlp_chunk_tokens;  /* 0: whole token set; else MLP runs over chunks of this many tokens */
  int32_t head_chunk_tokens; /* tokens per LM-head chunk (default 16384) */
  int32_t precision;         /* MT_PREC_BF16 | MT_PREC_FP32_DEBUG */
  int32_t host_threads;      /* CPU threads for Adam and embedding work (default 16) */
  int32_t check_finite;      /* 1: refuse to update on a non-finite loss/gradient */
  int32_t serialize;         /* 1: run W, C and G work on one stream (for invariance tests) */
  int32_t host_alloc;        /* MT_HOST_PINNED (default) | MT_HOST_PAGEABLE (no GPU needed) */
  int32_t keep_grads;        /* 1: keep each step's gradients on the host for mt_model_get_param */
  int32_t time_kernels;      /* 1: time every GEMM and attention launch with HIP events
                                (mt_step_stats, mt_model_kernel_times) */
  int32_t keep_internals;    /* 1 (default): each backward segment's re-forward runs every
                                layer of the segment with mt_layer_fwd_keep and the
                                backward uses mt_layer_bwd_saved (K layers of internals
                                on the device, no second forward per layer; with a
                                chunked MLP the attention half's internals are kept and
                                each chunk's gate/up is recomputed in the backward); 0:
                                the re-forward covers the first K-1 layers and every
                                layer's backward recomputes (mt_layer_recompute_bwd). */
  int32_t defer_updates;     /* 1 (default): the host Adam of the LM head and of the
                                embedding is left to the next step, which applies it
                                while its forward streams the other units (the head is
                                needed only after every layer's forward, the embedding
                                only for the batch's rows at its start); with clip_norm
                                > 0 the layers' updates too (none can start before the
                                last gradient has landed): the next step applies them
                                in layer order, each before that layer's first weight
                                load, holding their gradient slabs until then.  Reading
                                or setting a parameter applies them first, so results
                                are bitwise those of 0 (apply within the step). */
  int32_t resident_layers;   /* C >= 0 (default 0): the weights of C layers (1 .. C, or
                                all when C = n_layers) stay on the device from one step
                                to the next.  Right after such a layer's host Adam
                                update (in the backward, while the host link has time
                                to spare) its new streamed copy is uploaded into one of
                                C slots at the start of the arena, and the next step's
                                forward, re-forward and backward read it there instead
                                of loading it.  The forward, which is link-bound,
                                streams C layers fewer, and its loads run ahead (up to
                                the weight slots) while the resident layers compute.
                                Layer 0 stays streamed: its update ends the step, and
                                its upload would lengthen the step.  Device memory
                                grows by C layers, independent of the depth.  The slots are trusted while steps get the same
                                arena pointer and nothing writes its first
                                C x layer bytes; setting a parameter, a failed step or
                                another arena makes the next step load them again.
                                Results are bitwise those of 0. */
  int32_t opt_8bit;          /* 1: the host store keeps Adam's moments as the hybrid 8-bit
                                states of mt_host_adam8 (E4M3 codes + one fp32 scale per
                                128 elements of a tensor; 2.06 instead of 8 bytes per
                                parameter) and every unit is updated by that operator;
                                needs hidden % 128 == 0; fixed at creation */
  double lr, beta1, beta2, eps, weight_decay; /* Adam (weight_decay must be 0) */
  double clip_norm;          /* > 0: global gradient-norm clipping (LazyTrain's fast
                                clipping): every gradient is multiplied by
                                min(1, clip_norm / (norm + 1e-6)), norm over the whole
                                model.  Each unit's sum of squares is accumulated on the
                                GPU beside its finiteness check (the host never re-reads
                                a gradient) and the factor is applied inside the Adam
                                pass; since it depends on every gradient, each unit's
                                update waits until the last gradient has landed (with
                                defer_updates, the layers' updates then run during the
                                next step's forward), so the slab pool must hold every
                                layer's and the head's gradient (n_slabs >= n_layers +
                                1, or no pool).  0: off */
} mt_run_cfg;

/* Device pointers of one layer's weights: the stateless template's binding.
 * Layouts (bf16): attn_norm [H]; w_qkv [Q+2Kv, H] = rows of W_q, then W_k,
 * then W_v; w_o [H, Q]; mlp_norm [H]; w_gate_up [2F, H] = rows of W_gate
 * then W_up; w_down [H, F].  Q = n_heads*head_dim, Kv = n_kv_heads*head_dim. */
typedef struct {
  const void *attn_norm, *w_qkv, *w_o, *mlp_norm, *w_gate_up, *w_down;
} mt_layer_view;

/* Device pointers receiving one layer's gradients, same layouts as above. */
typedef struct {
  void *attn_norm, *w_qkv, *w_o, *mlp_norm, *w_gate_up, *w_down;
} mt_layer_grad_view;

typedef struct {
  double step_ms;           /* wall time of mt_stream_step */
  double fwd_ms, head_ms, bwd_ms; /* compute-stream phase times (HIP events) */
  double adam_ms;           /* summed host Adam time */
  double tail_ms;           /* from the end of GPU work to return */
  double h2d_bytes, d2h_bytes;
  double h2d_ms, d2h_ms;    /* summed durations of the host-to-device copies (weight
                               loads, resident-layer uploads, the step's input) and of
                               the gradient offload copies */
  double exposed_wait_fwd_ms, exposed_wait_bwd_ms; /* compute idle while waiting on weights */
  double probe_kernel_ms;   /* summed duration of the launches of the kernel (GEMM
                               instantiation or attention kernel) with the largest
                               total time (time_kernels) */
  double probe_kernel_flops;/* algorithmic FLOPs of those launches (GEMM: 2 M N K;
                               attention: 2 head_dim FLOPs per causal score pair per
                               product the kernel needs, see mt_kernel_time) */
  int64_t probe_kernel_launches;
  int64_t pinned_host_bytes, pageable_host_bytes, device_arena_bytes;
  int64_t units_updated;    /* units whose Adam update completed this step */
  /* host-side waits (ms): compute enqueue blocked on a free gradient ring
   * buffer; offload thread blocked on a free slab and on backward ops;
   * optimizer thread idle waiting for a landed gradient */
  double host_ring_wait_ms, host_slab_wait_ms, host_op_wait_ms, host_adam_idle_ms;
  double probe_all_gemm_ms; /* summed duration of every timed GEMM launch of the step */
  char probe_kernel[96];    /* that kernel's name, e.g. "gemm_dl_kernel<2, 2, 4, 4, 2, 0, 64, 2>" */
  /* host-clock times (ms) from the start of mt_stream_step: the step's
   * input (the embedding gather) enqueued, the first weight loads already
   * under way; the host seeing the last backward op complete; the last
   * gradient landed in host memory; the optimizer thread done (the step's
   * tail is what follows gpu_done_ms) */
  double host_start_ms, gpu_done_ms, grads_landed_ms, updates_done_ms;
  double probe_all_attn_ms; /* summed duration of every timed attention launch */
  double probe_all_flops;   /* algorithmic FLOPs of every timed launch of the step */
  double grad_norm;         /* with clip_norm > 0: the step's global gradient norm */
  double clip_factor;       /* ... and the factor every gradient was multiplied by (else 1) */
} mt_step_stats;

/* One kernel's timed launches in the last step (time_kernels = 1): launches
 * grouped by kernel name (a GEMM instantiation as profilers print it, or an
 * attention kernel), with their summed duration from HIP events recorded on
 * the compute stream around each launch and their summed algorithmic FLOPs.
 * GEMM: 2 M N K.  Attention, with P the causal score pairs (T (T + 1) / 2
 * per sequence and query head): forward 4 d P (S = Q K^T, O = P V); dK/dV
 * 8 d P (S, dP = dO V^T, dV = P^T dO, dK = dS^T Q); dQ 6 d P (S, dP,
 * dQ = dS K); delta 0. */
typedef struct {
  char name[96];
  int64_t launches;
  double ms;
  double flops;
} mt_kernel_time;

typedef struct mt_model mt_model;

/* Thread-local text of the last non-OK status returned on this thread. */
const char* mt_last_error(void);

/* ---------------------------------------------------------------------
 * Stateless layer template (blog summary, section 4: weights bound at call
 * time, nothing kept between calls).  Enqueue-only on `stream`: never
 * allocates, never synchronizes.  The caller provides a device workspace of
 * at least mt_layer_workspace_bytes(...) bytes (256-B aligned).
 * ------------------------------------------------------------------- */

/* which: 0 = forward, 1 = recompute + backward, 2 = backward from kept
 * internals (mt_layer_bwd_saved).  Returns 0 for an invalid shape. */
size_t mt_layer_workspace_bytes(const mt_model_cfg* cfg, const mt_run_cfg* run,
                                int32_t batch, int32_t seq, int32_t which);

/* Forward of one decoder layer: x_out = x_in + attn(...) + mlp(...).
 * x_in, x_out: device bf16 [batch*seq, hidden]; x_out may not alias x_in. */
mt_status mt_layer_fwd(const mt_model_cfg* cfg, const mt_run_cfg* run,
                       const mt_layer_view* w, const void* x_in, void* x_out,
                       int32_t batch, int32_t seq, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Recompute the layer's internals from its input x_in (blog summary,
 * section 3), then backward: given dy = dL/dx_out, write dx = dL/dx_in and
 * every weight gradient into dw (bf16, overwritten, not accumulated).
 * x_in, dy, dx: device bf16 [batch*seq, hidden]; dx may alias dy. */
mt_status mt_layer_recompute_bwd(const mt_model_cfg* cfg, const mt_run_cfg* run,
                                 const mt_layer_view* w, const void* x_in,
                                 const void* dy, void* dx,
                                 const mt_layer_grad_view* dw, int32_t batch,
                                 int32_t seq, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The recompute of the backward split off (blog summary, section 3: layer
 * inputs are rebuilt from checkpoints; here a layer forward run while
 * rebuilding them keeps everything its backward needs, so the backward
 * computes no forward of its own).  mt_layer_fwd_keep is mt_layer_fwd that
 * also leaves the layer's internals (normed inputs, rotated q/k and v,
 * attention output and log-sum-exp, mid residual, gate/up pre-activations,
 * SwiGLU output, RMS factors) in `internals`, a caller-owned device buffer
 * of mt_layer_internals_bytes(...) bytes (256-B aligned) that must stay
 * untouched until mt_layer_bwd_saved has consumed it.  mt_layer_bwd_saved
 * is mt_layer_recompute_bwd without the recompute: same inputs, outputs
 * and aliasing rules, plus the internals of a mt_layer_fwd_keep of the same
 * weights and x_in; its workspace is mt_layer_workspace_bytes(..., 2).
 * The results are bitwise equal to mt_layer_recompute_bwd's (same kernels
 * on the same inputs).  With mlp_chunk_tokens > 0 (the chunked MLP exists
 * to avoid holding the full gate/up activations) only the attention half's
 * internals and the normed MLP input are kept, and mt_layer_bwd_saved
 * recomputes each chunk's gate/up from them. */
size_t mt_layer_internals_bytes(const mt_model_cfg* cfg, const mt_run_cfg* run,
                                int32_t batch, int32_t seq);
mt_status mt_layer_fwd_keep(const mt_model_cfg* cfg, const mt_run_cfg* run,
                            const mt_layer_view* w, const void* x_in, void* x_out,
                            int32_t batch, int32_t seq, void* internals,
                            size_t internals_bytes, void* stream);
mt_status mt_layer_bwd_saved(const mt_model_cfg* cfg, const mt_run_cfg* run,
                             const mt_layer_view* w, const void* x_in,
                             const void* dy, void* dx, const mt_layer_grad_view* dw,
                             int32_t batch, int32_t seq, void* internals,
                             size_t internals_bytes, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Host-resident model: the authoritative flat store (blog summary,
 * "Performance and Capabilities": flat tensor layout, authoritative host
 * storage).  One region per unit (each layer, the head = final norm + LM
 * head, the embedding); fp32 master, m and v share one layout, and a bf16
 * copy of the master (pinned) is what streams to the GPU.
 * ------------------------------------------------------------------- */

mt_status mt_model_create(const mt_model_cfg* cfg, const mt_run_cfg* run,
                          mt_model** out);
void mt_model_destroy(mt_model* model);

/* Changes the schedule knobs of a model between steps (the ablation of the
 * listing page's Table 4 runs one model under several schedules):
 * checkpoint interval, prefetch depth, slab pool off (and on again, when
 * the model was created with it), MLP and head
 * chunks, keep_internals, defer_updates, resident_layers, serialize,
 * check_finite, time_kernels and the Adam hyperparameters.  precision,
 * host_alloc, keep_grads, host_threads and the slab pool's size are fixed
 * at creation (MT_E_INVALID if they differ).  Applies any pending update
 * first; resident layers are loaded again by the next step.  The next
 * step's arena size is mt_stream_arena_bytes under the new knobs.  Results
 * do not depend on the schedule (bitwise). */
mt_status mt_model_set_schedule(mt_model* model, const mt_run_cfg* run);

/* Parameter names: "embed", "layers.<l>.{attn_norm,w_q,w_k,w_v,w_o,
 * mlp_norm,w_gate,w_up,w_down}", "final_norm", "lm_head"; shapes [out, in].
 * set: copies n fp32 values into the master, writes the bf16 copy (RNE) and
 * zeroes m and v.  n must equal the tensor's element count. */
mt_status mt_model_set_param(mt_model* model, const char* name,
                             const float* src, size_t n);

enum { MT_GET_MASTER = 0, MT_GET_M = 1, MT_GET_V = 2, MT_GET_GRAD = 3,
       MT_GET_SHADOW = 4 };
/* get: copies a tensor out as fp32 (after applying any update the last
 * step deferred).  MT_GET_GRAD needs keep_grads = 1 and returns the last
 * step's gradient as the optimizer saw it. */
mt_status mt_model_get_param(const mt_model* model, const char* name,
                             int32_t which, float* dst, size_t n);

/* Adam step counter of the model (number of completed steps). */
int64_t mt_model_step_count(const mt_model* model);

/* The last step's per-kernel timings (empty unless the run config set
 * time_kernels).  Writes min(n, cap) entries, sorted by total time, largest
 * first, and the number available to *n_out. */
mt_status mt_model_kernel_times(const mt_model* model, mt_kernel_time* out, int32_t cap,
                                int32_t* n_out);

/* Device arena the streamed step needs for batch x seq tokens. */
size_t mt_stream_arena_bytes(const mt_model* model, int32_t batch, int32_t seq);

/* The same for a model shape and run config without creating the model (no
 * host store): the device bytes a step of that depth would take (listing
 * page, Table 5's depth study: device memory does not grow with depth).
 * Returns 0 for an invalid shape or knob. */
size_t mt_stream_arena_bytes_cfg(const mt_model_cfg* cfg, const mt_run_cfg* run, int32_t batch,
                                 int32_t seq);

/* One training step (blog summary, sections 1-4; listing page, Fig. 3):
 * stream each layer's bf16 weights in on streams[0] (W), run forward,
 * head, segment re-forward, recompute and backward on streams[1] (C), and
 * offload each unit's bf16 gradient on streams[2] (G) into a pinned slab,
 * where a CPU Adam step updates that unit while the GPU continues.
 * tokens: host int32 [batch, seq], ids in [0, vocab).  arena: device, at
 * least mt_stream_arena_bytes bytes.  Blocks until every unit is updated
 * (with defer_updates, every unit but the LM head and the embedding, and
 * with clip_norm > 0 but the layers too, whose updates the next step,
 * mt_model_get_param or mt_model_set_param applies first; the values are
 * the same either way); writes the mean next-token
 * loss to *loss_out and, if stats_out is not null, timings and byte
 * counts.  With check_finite, a non-finite loss returns MT_E_NONFINITE
 * before any update.  A step that fails after validation drops the updates
 * it deferred. */
mt_status mt_stream_step(mt_model* model, const int32_t* tokens, int32_t batch,
                         int32_t seq, void* arena, size_t arena_bytes,
                         void* const streams[3], float* loss_out,
                         mt_step_stats* stats_out);

/* ---------------------------------------------------------------------
 * CPU optimizer (blog summary, section 1: the optimizer step runs entirely
 * on the CPU).  Synchronous, in place, on host memory the caller owns.
 * Adam with bias correction: m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
 * p -= lr * (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps).  grad is bf16 or fp32
 * per grad_dtype; bf16_shadow (nullable) receives RNE(bf16) of the new p.
 * With hp->check_finite, a non-finite gradient returns MT_E_NONFINITE and
 * leaves every array unchanged.  step >= 1.
 * ------------------------------------------------------------------- */
mt_status mt_host_adam(float* param, float* exp_avg, float* exp_avg_sq,
                       const void* grad, int32_t grad_dtype,
                       uint16_t* bf16_shadow, size_t n, int64_t step,
                       const mt_run_cfg* hp);

/* Hybrid 8-bit Adam with gradient clipping (LazyTrain abstract, on the
 * listing pages: 8-bit optimizer states coupled with fast gradient
 * clipping in one operator).  The same update as mt_host_adam, with these
 * readings (the page gives no format): each moment is kept in blocks of
 * 128 consecutive elements (the last block may be shorter) as OCP FP8 E4M3
 * codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest 448)
 * with one fp32 scale per block: scale = absmax / 448, code = E4M3(x /
 * scale) rounded to nearest even, value = E4M3value(code) * scale; the
 * first moment is stored as m, the second as r = sqrt(v).  The update
 * dequantizes m and v = r * r, multiplies the gradient by `clip` (the
 * caller's global-norm clipping factor min(1, max_norm / (norm + 1e-6)),
 * in (0, 1]; 1 = no clipping), applies Adam in fp32 exactly as
 * mt_host_adam, writes param (and bf16_shadow, nullable), then quantizes
 * the new m and r.  Arrays: param [n]; m_code, r_code [n] bytes; m_scale,
 * r_scale [ceil(n / 128)] floats; all zero for a fresh state.  grad as in
 * mt_host_adam.  With hp->check_finite a non-finite gradient returns
 * MT_E_NONFINITE and leaves every array unchanged. */
mt_status mt_host_adam8(float* param, uint8_t* m_code, float* m_scale, uint8_t* r_code,
                        float* r_scale, const void* grad, int32_t grad_dtype,
                        uint16_t* bf16_shadow, size_t n, int64_t step, float clip,
                        const mt_run_cfg* hp);

/* Defaults for every knob (ckpt 4, depth 2, pool of 8, lr 1e-4, betas
 * 0.9/0.999, eps 1e-8, bf16, 16 host threads, pinned host memory). */
void mt_run_cfg_default(mt_run_cfg* out);

#ifdef __cplusplus
}
#endif

#endif /* MT_H */
