// Internal API of the stateless decoder-layer template and the LM head.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "mt.h"

namespace mt {

struct Dims {
  int B, T, D, H, Hq, Hkv, d, Qd, Kvd, NQKV, F, V;
  float eps;
  double theta;
  int mlp_chunk;   // tokens per MLP chunk (== D when not chunked)
  int head_chunk;  // tokens per LM-head chunk
  int prec;        // MT_PREC_BF16 or MT_PREC_FP32_DEBUG
  // bytes per stored element of weights, activations and gradients
  size_t es() const { return prec == MT_PREC_FP32_DEBUG ? 4 : 2; }
};

// Validates the model shape and run knobs; fills dims.  Returns nullptr or
// a message.
const char* make_dims(const mt_model_cfg* cfg, const mt_run_cfg* run, int batch, int seq,
                      Dims* out);

// Optional timing of GEMM launches with event pairs, each tagged with the
// kernel instantiation it ran and its algorithmic FLOPs.
struct Probe {
  std::vector<hipEvent_t> ev;  // pairs
  std::vector<std::string> name;
  std::vector<double> flops;
  int used = 0;  // events used (2 per launch)
};

// Bump allocator over a caller-provided device workspace; with base ==
// nullptr it only measures.
struct Carve {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

// Activations, weights and gradients are stored as bf16 bit patterns or,
// with d.prec == MT_PREC_FP32_DEBUG, as fp32 (d.es() bytes per element).
size_t layer_ws_bytes(const Dims& d, int which);
mt_status layer_fwd_impl(const Dims& d, const mt_layer_view& w, const void* x_in, void* x_out,
                         void* ws, size_t ws_bytes, hipStream_t s, Probe* probe);
mt_status layer_bwd_impl(const Dims& d, const mt_layer_view& w, const void* x_in, const void* dy,
                         void* dx, const mt_layer_grad_view& g, void* ws, size_t ws_bytes,
                         hipStream_t s, Probe* probe);
// Forward that keeps its internals in `internals` (layer_ws_bytes(d, 2)
// bytes; unchunked MLP only), and the backward that uses them instead of
// recomputing (ws: layer_ws_bytes(d, 3) bytes of backward scratch).
mt_status layer_fwd_keep_impl(const Dims& d, const mt_layer_view& w, const void* x_in, void* x_out,
                              void* internals, size_t internals_bytes, hipStream_t s,
                              Probe* probe);
mt_status layer_bwd_saved_impl(const Dims& d, const mt_layer_view& w, const void* x_in,
                               const void* dy, void* dx, const mt_layer_grad_view& g,
                               void* internals, size_t internals_bytes, void* ws,
                               size_t ws_bytes, hipStream_t s, Probe* probe);

// LM head: h = rms(x_L) g_f; logits = h W_out^T per token chunk; next-token
// cross-entropy; dh, dW_out, dg_f; dx_L = rmsnorm backward.  targets: device
// int32 [D] (-1 = none).  loss_dev: device fp32 scalar (mean over targets).
size_t head_ws_bytes(const Dims& d);
mt_status head_impl(const Dims& d, const void* g_f, const void* w_out, const void* x_L,
                    const int32_t* targets, float inv_n, void* dx_L, void* dg_f, void* dw_out,
                    float* loss_dev, void* ws, size_t ws_bytes, hipStream_t s, Probe* probe);

// Element offsets of the tensors inside one layer's flat unit (streamed
// copy, gradient slab and fp32 store share them), each aligned to 128
// elements.
struct LayerLayout {
  size_t attn_norm, w_qkv, w_q, w_k, w_v, w_o, mlp_norm, w_gate_up, w_gate, w_up, w_down, total;
};
LayerLayout layer_layout(const Dims& d);
struct HeadLayout {
  size_t final_norm, lm_head, total;
};
HeadLayout head_layout(const Dims& d);
inline size_t align128(size_t n) { return (n + 127) & ~size_t(127); }

}  // namespace mt
