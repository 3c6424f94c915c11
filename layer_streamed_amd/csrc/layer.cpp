// The stateless decoder-layer template (MegaTrain blog summary, section 4:
// each layer binds its parameters at run time and keeps nothing between
// calls) and the LM head.  Host code only: it enqueues the HIP kernels of
// kernels.h on one stream, carving every intermediate out of a
// caller-provided workspace.
//
// Forward (pre-norm GQA block, Qwen2.5 shape of the listing page's Table 2):
//   a = rms(x) g1;  qkv = a W_qkv^T;  rope(q, k);  o = attn(q, k, v)
//   x_mid = x + o W_o^T;  b = rms(x_mid) g2
//   m = silu(b W_gate^T) * (b W_up^T);  x_out = x_mid + m W_down^T
// The MLP may run over token chunks (listing page, Table 7 note on chunked
// MLP execution); weight gradients then accumulate in fp32 across chunks
// and are rounded to bf16 once.
//
// Recompute + backward (blog summary, section 3): the forward above is run
// again from x to rebuild every internal, then
//   dgu = swiglu'(dy W_down, gate, up);  dW_down = dy^T m;  dW_gu = dgu^T b
//   db = dgu W_gu;  dx_mid = dy + rms2'(db);  dg2
//   do = dx_mid W_o;  dW_o = dx_mid^T o;  dq, dk, dv = attn'(...)
//   rope^-1(dq, dk);  dW_qkv = dqkv^T a;  da = dqkv W_qkv
//   dx = dx_mid + rms1'(da);  dg1
#include "layer.h"

#include <algorithm>
#include <string>
#include <type_traits>

#include "kernels.h"
#include "status.h"

namespace mt {

const char* make_dims(const mt_model_cfg* cfg, const mt_run_cfg* run, int batch, int seq,
                      Dims* out) {
  if (!cfg || !run) return "null config";
  const mt_model_cfg& c = *cfg;
  if (c.n_layers < 1 || c.hidden < 64 || c.n_heads < 1 || c.n_kv_heads < 1 || c.ffn < 64 ||
      c.vocab < 64)
    return "model sizes must be positive (hidden, ffn, vocab >= 64)";
  if (c.hidden % 64 || c.ffn % 64 || c.vocab % 64) return "hidden, ffn and vocab must be multiples of 64";
  if (c.hidden > RMSNORM_MAX_COLS) return "hidden above 16384 is not supported";
  if (c.n_heads % c.n_kv_heads) return "n_heads must be a multiple of n_kv_heads";
  if (c.head_dim != 64 && c.head_dim != 128) return "head_dim must be 64 or 128";
  if (!(c.rms_eps > 0) || !(c.rope_theta > 0)) return "rms_eps and rope_theta must be positive";
  if (batch < 1 || seq < 1) return "batch and seq must be >= 1";
  if ((long)batch * seq > (1L << 30)) return "too many tokens";
  if (run->precision != MT_PREC_BF16 && run->precision != MT_PREC_FP32_DEBUG)
    return "precision must be MT_PREC_BF16 or MT_PREC_FP32_DEBUG";
  if (run->mlp_chunk_tokens < 0 || run->head_chunk_tokens < 0) return "chunk sizes must be >= 0";
  Dims d;
  d.B = batch;
  d.T = seq;
  d.D = batch * seq;
  d.H = c.hidden;
  d.Hq = c.n_heads;
  d.Hkv = c.n_kv_heads;
  d.d = c.head_dim;
  d.Qd = d.Hq * d.d;
  d.Kvd = d.Hkv * d.d;
  d.NQKV = d.Qd + 2 * d.Kvd;
  d.F = c.ffn;
  d.V = c.vocab;
  d.eps = c.rms_eps;
  d.theta = c.rope_theta;
  d.prec = run->precision;
  d.mlp_chunk = run->mlp_chunk_tokens > 0 ? std::min(run->mlp_chunk_tokens, d.D) : d.D;
  d.head_chunk = run->head_chunk_tokens > 0 ? std::min(run->head_chunk_tokens, d.D) : std::min(d.D, 16384);
  *out = d;
  return nullptr;
}

LayerLayout layer_layout(const Dims& d) {
  LayerLayout L;
  size_t o = 0;
  const size_t H = d.H;
  L.attn_norm = o; o += align128(H);
  L.w_qkv = o; L.w_q = o; L.w_k = o + (size_t)d.Qd * H; L.w_v = L.w_k + (size_t)d.Kvd * H;
  o += align128((size_t)d.NQKV * H);
  L.w_o = o; o += align128(H * d.Qd);
  L.mlp_norm = o; o += align128(H);
  L.w_gate_up = o; L.w_gate = o; L.w_up = o + (size_t)d.F * H; o += align128(2 * (size_t)d.F * H);
  L.w_down = o; o += align128(H * d.F);
  L.total = o;
  return L;
}

HeadLayout head_layout(const Dims& d) {
  HeadLayout L;
  L.final_norm = 0;
  L.lm_head = align128(d.H);
  L.total = L.lm_head + align128((size_t)d.V * d.H);
  return L;
}

namespace {

// Workspace of one layer call.  E is the storage type of activations
// (uint16_t: bf16 bit patterns; float: the fp32 debug precision).
// fp32 partial sums of the GEMMs' split tail tiles (up to 256 tiles of
// 256 x 256).  Only bf16 products tiled 256 x 256 split, and that tile needs
// at least 768 tiles, so smaller models carve nothing.
constexpr size_t SPLIT_ELEMS = (size_t)256 * 256 * 256;

template <class E>
size_t split_elems(const Dims& d, bool head) {
  if (!std::is_same_v<E, uint16_t>) return 0;
  const double D = d.D, H = d.H, F = d.F, V = d.V, C = d.mlp_chunk, Ch = d.head_chunk;
  const double largest = head ? std::max(Ch * V, V * H)
                              : std::max({C * 2 * F, 2 * F * H, D * (double)d.NQKV, D * H});
  return largest >= 768.0 * 256 * 256 ? SPLIT_ELEMS : 0;
}

template <class E>
struct LayerWs {
  float* split;  // GEMM split-tail workspace (null for fp32 storage)
  float *cos_t, *sin_t, *rstd1, *rstd2, *lse;
  E *a, *qkv, *o, *x_mid, *b, *gu, *m;
  // backward only
  E *dgu, *db, *dx_mid, *dout, *dqkv, *da;
  float *delta, *dg_part, *acc_d, *acc_gu;
};

template <class E>
void carve_bwd_scratch(const Dims& d, Carve& c, LayerWs<E>* w) {
  const size_t D = d.D, H = d.H, C = d.mlp_chunk;
  w->dgu = c.take<E>(C * 2 * d.F);
  w->db = c.take<E>(D * H);
  w->dx_mid = c.take<E>(D * H);
  w->dout = c.take<E>(D * d.Qd);
  w->dqkv = c.take<E>(D * d.NQKV);
  w->da = c.take<E>(D * H);
  w->delta = c.take<float>((size_t)d.B * d.Hq * d.T);
  w->dg_part = c.take<float>((size_t)rmsnorm_bwd_blocks((int)D) * H);
  if (C < D) {
    w->acc_d = c.take<float>(H * d.F);
    w->acc_gu = c.take<float>(2 * (size_t)d.F * H);
  }
}

template <class E>
// which: 0 forward (internals, gate/up not kept), 1 recompute + backward
// (internals with gate/up, then backward scratch), 2 kept internals of one
// layer (with a whole-token MLP gate/up and the SwiGLU output too; with a
// chunked MLP only the attention half's, and the backward recomputes each
// chunk's gate/up from the kept b), 3 backward scratch only (plus a chunk's
// gate/up and SwiGLU output for that recompute when the MLP is chunked).
LayerWs<E> carve_layer(const Dims& d, char* base, int which, size_t* bytes) {
  Carve c{base};
  LayerWs<E> w{};
  const size_t D = d.D, H = d.H, C = d.mlp_chunk;
  const bool chunked = C < D;
  if (const size_t n = split_elems<E>(d, false)) w.split = c.take<float>(n);
  if (which == 3) {
    carve_bwd_scratch(d, c, &w);
    if (chunked) {
      w.m = c.take<E>(C * d.F);
      w.gu = c.take<E>(C * 2 * d.F);
    }
    *bytes = c.off + 256;
    return w;
  }
  w.cos_t = c.take<float>((size_t)d.T * d.d / 2);
  w.sin_t = c.take<float>((size_t)d.T * d.d / 2);
  w.rstd1 = c.take<float>(D);
  w.rstd2 = c.take<float>(D);
  w.lse = c.take<float>((size_t)d.B * d.Hq * d.T);
  w.a = c.take<E>(D * H);
  w.qkv = c.take<E>(D * d.NQKV);
  w.o = c.take<E>(D * d.Qd);
  w.x_mid = c.take<E>(D * H);
  w.b = c.take<E>(D * H);
  w.m = c.take<E>(C * d.F);
  if (which == 1 || (which == 2 && !chunked)) w.gu = c.take<E>(C * 2 * d.F);
  if (which == 1) carve_bwd_scratch(d, c, &w);
  *bytes = c.off + 256;
  return w;
}

template <class E>
GemmArgsT<E> gemm(int layout, int epi, int M, int N, int K, const E* A, long lda, const E* B,
                  long ldb, void* C, long ldc) {
  GemmArgsT<E> g;
  g.layout = layout;
  g.epi = epi;
  g.M = M;
  g.N = N;
  g.K = K;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  return g;
}

inline std::string kernel_name(const GemmArgsT<uint16_t>& g) { return gemm_kernel_name(g); }
inline std::string kernel_name(const GemmArgsT<float>& g) {
  const int lay = (g.epi == EPI_SWIGLU || g.epi == EPI_SWIGLU_SAVE) ? GEMM_NT : g.layout;
  return "gemm_f32_kernel<" + std::to_string(lay) + ", " + std::to_string(g.epi) + ">";
}

#define MT_RUN(expr)                  \
  do {                                \
    mt_status st_ = (expr);           \
    if (st_ != MT_OK) return st_;     \
  } while (0)

// Runs `launch` (one kernel launch on s) between two of the probe's events
// when a probe with events to spare is given, recording the kernel's name
// and its algorithmic FLOPs.
template <class F>
mt_status timed_launch(Probe* probe, hipStream_t s, const std::string& name, double flops,
                       F&& launch) {
  const bool timed = probe && probe->used + 2 <= (int)probe->ev.size();
  if (timed) MT_HIP(hipEventRecord(probe->ev[probe->used], s));
  MT_HIP(launch());
  if (timed) {
    MT_HIP(hipEventRecord(probe->ev[probe->used + 1], s));
    probe->used += 2;
    probe->name.push_back(name);
    probe->flops.push_back(flops);
  }
  return MT_OK;
}

// `split`: the workspace's split-tail area (SPLIT_ELEMS floats), or null.
template <class E>
mt_status run_gemm(GemmArgsT<E> g, hipStream_t s, Probe* probe, float* split) {
  if (const char* m = gemm_check(g)) return set_error(MT_E_SHAPE, "layer GEMM: %s", m);
  g.ws = split;
  g.ws_elems = split ? (long)SPLIT_ELEMS : 0;
  return timed_launch(probe, s, probe ? kernel_name(g) : std::string(),
                      2.0 * g.M * (double)g.N * g.K, [&] { return gemm_launch(g, s); });
}

// Causal score pairs of the attention (query t sees keys 0..t), over the
// batch and the query heads: the products of the forward and backward each
// take 2 * head_dim FLOPs per pair.
inline double attn_pairs(const Dims& d) {
  return (double)d.B * d.Hq * ((double)d.T * (d.T + 1) / 2);
}

// Attention forward: S = Q K^T and O = P V, 2 products.
template <class E>
mt_status run_attn_fwd(const Dims& d, const E* qkv, E* o, float* lse, hipStream_t s,
                       Probe* probe) {
  if constexpr (std::is_same_v<E, uint16_t>) {
    return timed_launch(probe, s, attn_kernel_name(d.d, 0), 2 * 2.0 * d.d * attn_pairs(d), [&] {
      return attn_fwd(qkv, o, lse, d.B, d.T, d.Hq, d.Hkv, d.d, s);
    });
  } else {
    MT_HIP(attn_fwd(qkv, o, lse, d.B, d.T, d.Hq, d.Hkv, d.d, s));
    return MT_OK;
  }
}

// Attention backward, each kernel timed on its own.  FLOPs per kernel are
// the products it needs for its outputs: dK/dV recomputes S and forms dP,
// dV = P^T dO and dK = dS^T Q (4 products); dQ recomputes S and dP and
// forms dQ = dS K (3).  The backward as a whole needs 5 (S, dP, dV, dK,
// dQ); splitting it so that no two workgroups add into one output (no
// atomics, a fixed summation order) costs the 2 recomputed ones.
template <class E>
mt_status run_attn_bwd(const Dims& d, const E* qkv, const E* o, const float* lse, const E* dout,
                       float* delta, E* dqkv, hipStream_t s, Probe* probe) {
  if constexpr (std::is_same_v<E, uint16_t>) {
    const double pf = 2.0 * d.d * attn_pairs(d);
    auto stage = [&](int st) {
      return [&, st] {
        return attn_bwd(qkv, o, lse, dout, delta, dqkv, d.B, d.T, d.Hq, d.Hkv, d.d, s, st);
      };
    };
    MT_RUN(timed_launch(probe, s, attn_kernel_name(d.d, 1), 0.0, stage(ATTN_BWD_DELTA)));
    MT_RUN(timed_launch(probe, s, attn_kernel_name(d.d, 2), 4 * pf, stage(ATTN_BWD_DKDV)));
    return timed_launch(probe, s, attn_kernel_name(d.d, 3), 3 * pf, stage(ATTN_BWD_DQ));
  } else {
    MT_HIP(attn_bwd(qkv, o, lse, dout, delta, dqkv, d.B, d.T, d.Hq, d.Hkv, d.d, s));
    return MT_OK;
  }
}

// Typed weight pointers of a layer view.
template <class E>
struct LayerW {
  const E *g1, *wqkv, *wo, *g2, *wgu, *wd;
  explicit LayerW(const mt_layer_view& w)
      : g1(static_cast<const E*>(w.attn_norm)), wqkv(static_cast<const E*>(w.w_qkv)),
        wo(static_cast<const E*>(w.w_o)), g2(static_cast<const E*>(w.mlp_norm)),
        wgu(static_cast<const E*>(w.w_gate_up)), wd(static_cast<const E*>(w.w_down)) {}
};

// Attention half of the block, shared by forward and recompute.
template <class E>
mt_status attn_half(const Dims& d, const LayerW<E>& w, const E* x, const LayerWs<E>& ws,
                    hipStream_t s, Probe* probe) {
  MT_HIP(rope_table(ws.cos_t, ws.sin_t, d.T, d.d, d.theta, s));
  MT_HIP(rmsnorm_fwd(x, w.g1, ws.a, ws.rstd1, d.D, d.H, d.eps, s));
  MT_RUN(run_gemm(gemm<E>(GEMM_NT, EPI_BF16, d.D, d.NQKV, d.H, ws.a, d.H, w.wqkv, d.H, ws.qkv,
                          d.NQKV),
                  s, probe, ws.split));
  MT_HIP(rope_apply(ws.qkv, d.NQKV, d.B, d.T, d.Hq, d.Hkv, d.d, ws.cos_t, ws.sin_t, 0, s));
  MT_RUN(run_attn_fwd(d, ws.qkv, ws.o, ws.lse, s, probe));
  GemmArgsT<E> go = gemm<E>(GEMM_NT, EPI_RESID_BF16, d.D, d.H, d.Qd, ws.o, d.Qd, w.wo, d.Qd,
                            ws.x_mid, d.H);
  go.R = x;
  go.ldr = d.H;
  MT_RUN(run_gemm(go, s, probe, ws.split));
  MT_HIP(rmsnorm_fwd(ws.x_mid, w.g2, ws.b, ws.rstd2, d.D, d.H, d.eps, s));
  return MT_OK;
}

// keep = true: the internals (a, qkv, o, lse, x_mid, b, rstd, and with a
// whole-token MLP gate/up and m) stay in the buffer for a later backward
// without recompute of the attention half (nor of the MLP when whole).
template <class E>
mt_status layer_fwd_t(const Dims& d, const mt_layer_view& wv, const E* x_in, E* x_out, void* wsp,
                      size_t ws_bytes, hipStream_t s, Probe* probe, bool keep = false) {
  size_t need = 0;
  LayerWs<E> ws = carve_layer<E>(d, static_cast<char*>(wsp), keep ? 2 : 0, &need);
  MT_CHECK(wsp && ws_bytes >= need, MT_E_OOM_DEVICE, "layer forward: workspace %zu < %zu bytes",
           ws_bytes, need);
  const LayerW<E> w(wv);
  MT_RUN(attn_half(d, w, x_in, ws, s, probe));
  const bool keep_gu = keep && d.mlp_chunk == d.D;  // a chunked MLP keeps no gate/up
  for (int r0 = 0; r0 < d.D; r0 += d.mlp_chunk) {
    const int rows = std::min(d.mlp_chunk, d.D - r0);
    GemmArgsT<E> gu = gemm<E>(GEMM_NT, keep_gu ? EPI_SWIGLU_SAVE : EPI_SWIGLU, rows, 2 * d.F, d.H,
                              ws.b + (size_t)r0 * d.H, d.H, w.wgu, d.H, ws.m, d.F);
    gu.F = d.F;
    if (keep_gu) {
      gu.C2 = ws.gu;
      gu.ldc2 = 2 * d.F;
    }
    MT_RUN(run_gemm(gu, s, probe, ws.split));
    GemmArgsT<E> dn = gemm<E>(GEMM_NT, EPI_RESID_BF16, rows, d.H, d.F, ws.m, d.F, w.wd, d.F,
                              x_out + (size_t)r0 * d.H, d.H);
    dn.R = ws.x_mid + (size_t)r0 * d.H;
    dn.ldr = d.H;
    MT_RUN(run_gemm(dn, s, probe, ws.split));
  }
  return MT_OK;
}

// saved != nullptr: the internals come from layer_fwd_t(keep = true) and
// the attention half is not recomputed (nor the MLP when whole; a chunked
// MLP recomputes each chunk's gate/up from the kept b); wsp then holds the
// backward scratch.
template <class E>
mt_status layer_bwd_t(const Dims& d, const mt_layer_view& wv, const E* x_in, const E* dy, E* dx,
                      const mt_layer_grad_view& g, void* wsp, size_t ws_bytes, hipStream_t s,
                      Probe* probe, void* saved = nullptr, size_t saved_bytes = 0) {
  size_t need = 0;
  LayerWs<E> ws = carve_layer<E>(d, static_cast<char*>(wsp), saved ? 3 : 1, &need);
  MT_CHECK(wsp && ws_bytes >= need, MT_E_OOM_DEVICE,
           "layer recompute/backward: workspace %zu < %zu bytes", ws_bytes, need);
  if (saved) {
    size_t need_s = 0;
    const LayerWs<E> in = carve_layer<E>(d, static_cast<char*>(saved), 2, &need_s);
    MT_CHECK(saved_bytes >= need_s, MT_E_OOM_DEVICE, "layer backward: internals %zu < %zu bytes",
             saved_bytes, need_s);
    ws.cos_t = in.cos_t; ws.sin_t = in.sin_t; ws.rstd1 = in.rstd1; ws.rstd2 = in.rstd2;
    ws.lse = in.lse; ws.a = in.a; ws.qkv = in.qkv; ws.o = in.o; ws.x_mid = in.x_mid;
    ws.b = in.b;
    if (d.mlp_chunk == d.D) {
      ws.m = in.m;
      ws.gu = in.gu;
    }
  }
  const LayerW<E> w(wv);
  // ---- recompute the attention half (rebuilds a, qkv (rotated), o, lse, x_mid, b)
  if (!saved) MT_RUN(attn_half(d, w, x_in, ws, s, probe));
  const bool chunked = d.mlp_chunk < d.D;
  E* gd = static_cast<E*>(g.w_down);
  E* ggu = static_cast<E*>(g.w_gate_up);
  if (chunked) {
    MT_HIP(fill_f32(ws.acc_d, 0.f, (size_t)d.H * d.F, s));
    MT_HIP(fill_f32(ws.acc_gu, 0.f, 2 * (size_t)d.F * d.H, s));
  }
  // ---- MLP: recompute gate/up per chunk, then its backward
  for (int r0 = 0; r0 < d.D; r0 += d.mlp_chunk) {
    const int rows = std::min(d.mlp_chunk, d.D - r0);
    const E* b_c = ws.b + (size_t)r0 * d.H;
    const E* dy_c = dy + (size_t)r0 * d.H;
    GemmArgsT<E> gu = gemm<E>(GEMM_NT, EPI_SWIGLU_SAVE, rows, 2 * d.F, d.H, b_c, d.H, w.wgu, d.H,
                              ws.m, d.F);
    gu.F = d.F;
    gu.C2 = ws.gu;
    gu.ldc2 = 2 * d.F;
    if (!saved || chunked) MT_RUN(run_gemm(gu, s, probe, ws.split));
    // dgate, dup from dm = dy W_down (NN) fused with the SwiGLU derivative
    GemmArgsT<E> dm = gemm<E>(GEMM_NN, EPI_SWIGLU_BWD, rows, d.F, d.H, dy_c, d.H, w.wd, d.F,
                              ws.dgu, 2 * d.F);
    dm.F = d.F;
    dm.G = ws.gu;
    dm.ldg = 2 * d.F;
    dm.C2 = ws.dgu;
    dm.ldc2 = 2 * d.F;
    MT_RUN(run_gemm(dm, s, probe, ws.split));
    // dW_down = dy^T m  (TN: A = dy as [K=rows, M=H], B = m [rows, F])
    MT_RUN(run_gemm(gemm<E>(GEMM_TN, chunked ? EPI_ACC_F32 : EPI_BF16, d.H, d.F, rows, dy_c, d.H,
                            ws.m, d.F,
                            chunked ? static_cast<void*>(ws.acc_d) : static_cast<void*>(gd), d.F),
                    s, probe, ws.split));
    // dW_gu = dgu^T b  (TN: A = dgu [rows, 2F], B = b [rows, H])
    MT_RUN(run_gemm(gemm<E>(GEMM_TN, chunked ? EPI_ACC_F32 : EPI_BF16, 2 * d.F, d.H, rows, ws.dgu,
                            2 * d.F, b_c, d.H,
                            chunked ? static_cast<void*>(ws.acc_gu) : static_cast<void*>(ggu),
                            d.H),
                    s, probe, ws.split));
    // db = dgu W_gu  (NN: B = W_gu [2F, H])
    MT_RUN(run_gemm(gemm<E>(GEMM_NN, EPI_BF16, rows, d.H, 2 * d.F, ws.dgu, 2 * d.F, w.wgu, d.H,
                            ws.db + (size_t)r0 * d.H, d.H),
                    s, probe, ws.split));
  }
  if (chunked) {
    MT_HIP(cast_f32(ws.acc_d, gd, (size_t)d.H * d.F, s));
    MT_HIP(cast_f32(ws.acc_gu, ggu, 2 * (size_t)d.F * d.H, s));
  }
  // ---- second norm (residual dy)
  const int nblk = rmsnorm_bwd_blocks(d.D);
  MT_HIP(rmsnorm_bwd(ws.db, ws.x_mid, w.g2, ws.rstd2, dy, ws.dx_mid, ws.dg_part, d.D, d.H, s));
  MT_HIP(reduce_rows(ws.dg_part, nblk, d.H, static_cast<E*>(g.mlp_norm), s));
  // ---- output projection
  MT_RUN(run_gemm(gemm<E>(GEMM_NN, EPI_BF16, d.D, d.Qd, d.H, ws.dx_mid, d.H, w.wo, d.Qd, ws.dout,
                          d.Qd),
                  s, probe, ws.split));
  MT_RUN(run_gemm(gemm<E>(GEMM_TN, EPI_BF16, d.H, d.Qd, d.D, ws.dx_mid, d.H, ws.o, d.Qd, g.w_o,
                          d.Qd),
                  s, probe, ws.split));
  // ---- attention and RoPE
  MT_RUN(run_attn_bwd(d, ws.qkv, ws.o, ws.lse, ws.dout, ws.delta, ws.dqkv, s, probe));
  MT_HIP(rope_apply(ws.dqkv, d.NQKV, d.B, d.T, d.Hq, d.Hkv, d.d, ws.cos_t, ws.sin_t, 1, s));
  // ---- QKV projection
  MT_RUN(run_gemm(gemm<E>(GEMM_TN, EPI_BF16, d.NQKV, d.H, d.D, ws.dqkv, d.NQKV, ws.a, d.H,
                          g.w_qkv, d.H),
                  s, probe, ws.split));
  MT_RUN(run_gemm(gemm<E>(GEMM_NN, EPI_BF16, d.D, d.H, d.NQKV, ws.dqkv, d.NQKV, w.wqkv, d.H, ws.da,
                          d.H),
                  s, probe, ws.split));
  // ---- first norm (residual dx_mid)
  MT_HIP(rmsnorm_bwd(ws.da, x_in, w.g1, ws.rstd1, ws.dx_mid, dx, ws.dg_part, d.D, d.H, s));
  MT_HIP(reduce_rows(ws.dg_part, nblk, d.H, static_cast<E*>(g.attn_norm), s));
  return MT_OK;
}

}  // namespace

mt_status layer_fwd_keep_impl(const Dims& d, const mt_layer_view& w, const void* x_in, void* x_out,
                              void* internals, size_t internals_bytes, hipStream_t s,
                              Probe* probe) {
  if (d.prec == MT_PREC_FP32_DEBUG)
    return layer_fwd_t(d, w, static_cast<const float*>(x_in), static_cast<float*>(x_out),
                       internals, internals_bytes, s, probe, true);
  return layer_fwd_t(d, w, static_cast<const uint16_t*>(x_in), static_cast<uint16_t*>(x_out),
                     internals, internals_bytes, s, probe, true);
}

mt_status layer_bwd_saved_impl(const Dims& d, const mt_layer_view& w, const void* x_in,
                               const void* dy, void* dx, const mt_layer_grad_view& g,
                               void* internals, size_t internals_bytes, void* ws,
                               size_t ws_bytes, hipStream_t s, Probe* probe) {
  if (d.prec == MT_PREC_FP32_DEBUG)
    return layer_bwd_t(d, w, static_cast<const float*>(x_in), static_cast<const float*>(dy),
                       static_cast<float*>(dx), g, ws, ws_bytes, s, probe, internals,
                       internals_bytes);
  return layer_bwd_t(d, w, static_cast<const uint16_t*>(x_in), static_cast<const uint16_t*>(dy),
                     static_cast<uint16_t*>(dx), g, ws, ws_bytes, s, probe, internals,
                     internals_bytes);
}

size_t layer_ws_bytes(const Dims& d, int which) {
  size_t bytes = 0;
  if (d.prec == MT_PREC_FP32_DEBUG) carve_layer<float>(d, nullptr, which, &bytes);
  else carve_layer<uint16_t>(d, nullptr, which, &bytes);
  return bytes;
}

mt_status layer_fwd_impl(const Dims& d, const mt_layer_view& w, const void* x_in, void* x_out,
                         void* ws, size_t ws_bytes, hipStream_t s, Probe* probe) {
  if (d.prec == MT_PREC_FP32_DEBUG)
    return layer_fwd_t(d, w, static_cast<const float*>(x_in), static_cast<float*>(x_out), ws,
                       ws_bytes, s, probe);
  return layer_fwd_t(d, w, static_cast<const uint16_t*>(x_in), static_cast<uint16_t*>(x_out), ws,
                     ws_bytes, s, probe);
}

mt_status layer_bwd_impl(const Dims& d, const mt_layer_view& w, const void* x_in, const void* dy,
                         void* dx, const mt_layer_grad_view& g, void* ws, size_t ws_bytes,
                         hipStream_t s, Probe* probe) {
  if (d.prec == MT_PREC_FP32_DEBUG)
    return layer_bwd_t(d, w, static_cast<const float*>(x_in), static_cast<const float*>(dy),
                       static_cast<float*>(dx), g, ws, ws_bytes, s, probe);
  return layer_bwd_t(d, w, static_cast<const uint16_t*>(x_in), static_cast<const uint16_t*>(dy),
                     static_cast<uint16_t*>(dx), g, ws, ws_bytes, s, probe);
}

// ------------------------------------------------------------------- head

namespace {
template <class E>
struct HeadWs {
  float* split;  // GEMM split-tail workspace (null for fp32 storage)
  E *h, *dlogits, *dh;
  float *rstd, *logits, *loss_part, *dg_part, *acc_out;
};
template <class E>
HeadWs<E> carve_head(const Dims& d, char* base, size_t* bytes) {
  Carve c{base};
  HeadWs<E> w{};
  const size_t D = d.D, H = d.H, Ch = d.head_chunk;
  if (const size_t n = split_elems<E>(d, true)) w.split = c.take<float>(n);
  w.h = c.take<E>(D * H);
  w.dh = c.take<E>(D * H);
  w.rstd = c.take<float>(D);
  w.loss_part = c.take<float>(D);
  w.logits = c.take<float>(Ch * d.V);
  w.dlogits = c.take<E>(Ch * d.V);
  w.dg_part = c.take<float>((size_t)rmsnorm_bwd_blocks((int)D) * H);
  if ((int)Ch < d.D) w.acc_out = c.take<float>((size_t)d.V * H);
  *bytes = c.off + 256;
  return w;
}

template <class E>
mt_status head_t(const Dims& d, const E* g_f, const E* w_out, const E* x_L,
                 const int32_t* targets, float inv_n, E* dx_L, E* dg_f, E* dw_out, float* loss_dev,
                 void* wsp, size_t ws_bytes, hipStream_t s, Probe* probe) {
  size_t need = 0;
  HeadWs<E> ws = carve_head<E>(d, static_cast<char*>(wsp), &need);
  MT_CHECK(wsp && ws_bytes >= need, MT_E_OOM_DEVICE, "head: workspace %zu < %zu bytes", ws_bytes,
           need);
  const bool chunked = d.head_chunk < d.D;
  MT_HIP(rmsnorm_fwd(x_L, g_f, ws.h, ws.rstd, d.D, d.H, d.eps, s));
  if (chunked) MT_HIP(fill_f32(ws.acc_out, 0.f, (size_t)d.V * d.H, s));
  for (int r0 = 0; r0 < d.D; r0 += d.head_chunk) {
    const int rows = std::min(d.head_chunk, d.D - r0);
    const E* h_c = ws.h + (size_t)r0 * d.H;
    MT_RUN(run_gemm(gemm<E>(GEMM_NT, EPI_F32, rows, d.V, d.H, h_c, d.H, w_out, d.H, ws.logits,
                            d.V),
                    s, probe, ws.split));
    MT_HIP(ce_rows(ws.logits, targets + r0, ws.dlogits, ws.loss_part + r0, rows, d.V, inv_n, s));
    MT_RUN(run_gemm(gemm<E>(GEMM_NN, EPI_BF16, rows, d.H, d.V, ws.dlogits, d.V, w_out, d.H,
                            ws.dh + (size_t)r0 * d.H, d.H),
                    s, probe, ws.split));
    MT_RUN(run_gemm(gemm<E>(GEMM_TN, chunked ? EPI_ACC_F32 : EPI_BF16, d.V, d.H, rows, ws.dlogits,
                            d.V, h_c, d.H,
                            chunked ? static_cast<void*>(ws.acc_out) : static_cast<void*>(dw_out),
                            d.H),
                    s, probe, ws.split));
  }
  if (chunked) MT_HIP(cast_f32(ws.acc_out, dw_out, (size_t)d.V * d.H, s));
  MT_HIP(sum_loss(ws.loss_part, d.D, inv_n, loss_dev, s));
  MT_HIP(rmsnorm_bwd(ws.dh, x_L, g_f, ws.rstd, static_cast<const E*>(nullptr), dx_L, ws.dg_part,
                     d.D, d.H, s));
  MT_HIP(reduce_rows(ws.dg_part, rmsnorm_bwd_blocks(d.D), d.H, dg_f, s));
  return MT_OK;
}
}  // namespace

size_t head_ws_bytes(const Dims& d) {
  size_t b = 0;
  if (d.prec == MT_PREC_FP32_DEBUG) carve_head<float>(d, nullptr, &b);
  else carve_head<uint16_t>(d, nullptr, &b);
  return b;
}

mt_status head_impl(const Dims& d, const void* g_f, const void* w_out, const void* x_L,
                    const int32_t* targets, float inv_n, void* dx_L, void* dg_f, void* dw_out,
                    float* loss_dev, void* ws, size_t ws_bytes, hipStream_t s, Probe* probe) {
  if (d.prec == MT_PREC_FP32_DEBUG)
    return head_t(d, static_cast<const float*>(g_f), static_cast<const float*>(w_out),
                  static_cast<const float*>(x_L), targets, inv_n, static_cast<float*>(dx_L),
                  static_cast<float*>(dg_f), static_cast<float*>(dw_out), loss_dev, ws, ws_bytes, s,
                  probe);
  return head_t(d, static_cast<const uint16_t*>(g_f), static_cast<const uint16_t*>(w_out),
                static_cast<const uint16_t*>(x_L), targets, inv_n, static_cast<uint16_t*>(dx_L),
                static_cast<uint16_t*>(dg_f), static_cast<uint16_t*>(dw_out), loss_dev, ws,
                ws_bytes, s, probe);
}

}  // namespace mt

using namespace mt;

extern "C" {

size_t mt_layer_workspace_bytes(const mt_model_cfg* cfg, const mt_run_cfg* run, int32_t batch,
                                int32_t seq, int32_t which) {
  Dims d;
  if (make_dims(cfg, run, batch, seq, &d) || which < 0 || which > 2) return 0;
  return layer_ws_bytes(d, which == 2 ? 3 : which);
}

size_t mt_layer_internals_bytes(const mt_model_cfg* cfg, const mt_run_cfg* run, int32_t batch,
                                int32_t seq) {
  Dims d;
  if (make_dims(cfg, run, batch, seq, &d)) return 0;
  return layer_ws_bytes(d, 2);
}

static mt_status check_view(const mt_layer_view* w) {
  MT_CHECK(w && w->attn_norm && w->w_qkv && w->w_o && w->mlp_norm && w->w_gate_up && w->w_down,
           MT_E_INVALID, "layer view has a null weight pointer");
  return MT_OK;
}

mt_status mt_layer_fwd(const mt_model_cfg* cfg, const mt_run_cfg* run, const mt_layer_view* w,
                       const void* x_in, void* x_out, int32_t batch, int32_t seq, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Dims d;
  if (const char* m = make_dims(cfg, run, batch, seq, &d))
    return set_error(MT_E_SHAPE, "mt_layer_fwd: %s", m);
  MT_RUN(check_view(w));
  MT_CHECK(x_in && x_out, MT_E_INVALID, "mt_layer_fwd: null activation pointer");
  MT_CHECK(x_in != x_out, MT_E_INVALID, "mt_layer_fwd: x_out may not alias x_in");
  return layer_fwd_impl(d, *w, x_in, x_out, workspace, workspace_bytes,
                        static_cast<hipStream_t>(stream), nullptr);
}

mt_status mt_layer_fwd_keep(const mt_model_cfg* cfg, const mt_run_cfg* run, const mt_layer_view* w,
                            const void* x_in, void* x_out, int32_t batch, int32_t seq,
                            void* internals, size_t internals_bytes, void* stream) {
  Dims d;
  if (const char* m = make_dims(cfg, run, batch, seq, &d))
    return set_error(MT_E_SHAPE, "mt_layer_fwd_keep: %s", m);
  MT_RUN(check_view(w));
  MT_CHECK(x_in && x_out, MT_E_INVALID, "mt_layer_fwd_keep: null activation pointer");
  MT_CHECK(x_in != x_out, MT_E_INVALID, "mt_layer_fwd_keep: x_out may not alias x_in");
  return layer_fwd_keep_impl(d, *w, x_in, x_out, internals, internals_bytes,
                             static_cast<hipStream_t>(stream), nullptr);
}

mt_status mt_layer_bwd_saved(const mt_model_cfg* cfg, const mt_run_cfg* run,
                             const mt_layer_view* w, const void* x_in, const void* dy, void* dx,
                             const mt_layer_grad_view* dw, int32_t batch, int32_t seq,
                             void* internals, size_t internals_bytes, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Dims d;
  if (const char* m = make_dims(cfg, run, batch, seq, &d))
    return set_error(MT_E_SHAPE, "mt_layer_bwd_saved: %s", m);
  MT_RUN(check_view(w));
  MT_CHECK(x_in && dy && dx && internals, MT_E_INVALID, "mt_layer_bwd_saved: null pointer");
  MT_CHECK(dw && dw->attn_norm && dw->w_qkv && dw->w_o && dw->mlp_norm && dw->w_gate_up &&
               dw->w_down,
           MT_E_INVALID, "mt_layer_bwd_saved: null gradient pointer");
  return layer_bwd_saved_impl(d, *w, x_in, dy, dx, *dw, internals, internals_bytes, workspace,
                              workspace_bytes, static_cast<hipStream_t>(stream), nullptr);
}

mt_status mt_layer_recompute_bwd(const mt_model_cfg* cfg, const mt_run_cfg* run,
                                 const mt_layer_view* w, const void* x_in, const void* dy,
                                 void* dx, const mt_layer_grad_view* dw, int32_t batch,
                                 int32_t seq, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  Dims d;
  if (const char* m = make_dims(cfg, run, batch, seq, &d))
    return set_error(MT_E_SHAPE, "mt_layer_recompute_bwd: %s", m);
  MT_RUN(check_view(w));
  MT_CHECK(x_in && dy && dx, MT_E_INVALID, "mt_layer_recompute_bwd: null activation pointer");
  MT_CHECK(dw && dw->attn_norm && dw->w_qkv && dw->w_o && dw->mlp_norm && dw->w_gate_up &&
               dw->w_down,
           MT_E_INVALID, "mt_layer_recompute_bwd: null gradient pointer");
  return layer_bwd_impl(d, *w, x_in, dy, dx, *dw, workspace, workspace_bytes,
                        static_cast<hipStream_t>(stream), nullptr);
}

}  // extern "C"
