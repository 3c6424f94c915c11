"""ctypes binding of libmt (include/mt.h, include/mt_ops.h).

Argument marshalling only: every step of the training path runs inside
libmt.  Device buffers are passed as torch tensors (their data_ptr()),
streams as torch.cuda.Stream (their hipStream_t handle).  A missing or
unloadable library raises at import: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmt.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libmt.so not found at {LIB_PATH}; build it with "
        "`python -m layer_streamed_amd.build` (hipcc for gfx950)")
_lib = C.CDLL(LIB_PATH)

# ----------------------------------------------------------------- constants
MT_OK, MT_E_INVALID, MT_E_SHAPE, MT_E_OOM_DEVICE, MT_E_OOM_HOST = 0, -1, -2, -3, -4
MT_E_HIP, MT_E_NONFINITE, MT_E_STATE = -5, -6, -7
DT_BF16, DT_F32 = 0, 1
PREC_BF16, PREC_FP32_DEBUG = 0, 1
HOST_PINNED, HOST_PAGEABLE = 0, 1
GET_MASTER, GET_M, GET_V, GET_GRAD, GET_SHADOW = 0, 1, 2, 3, 4
GEMM_NT, GEMM_NN, GEMM_TN = 0, 1, 2
EPI_BF16, EPI_F32, EPI_ACC_F32, EPI_RESID_BF16 = 0, 1, 2, 3
EPI_SWIGLU, EPI_SWIGLU_SAVE, EPI_SWIGLU_BWD = 4, 5, 6

_STATUS = {0: "MT_OK", -1: "MT_E_INVALID", -2: "MT_E_SHAPE", -3: "MT_E_OOM_DEVICE",
           -4: "MT_E_OOM_HOST", -5: "MT_E_HIP", -6: "MT_E_NONFINITE", -7: "MT_E_STATE"}


class MTError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


# ------------------------------------------------------------------- structs
class ModelCfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_double)]


class RunCfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "ckpt_interval", "prefetch_depth", "use_slab_pool", "n_slabs", "mlp_chunk_tokens",
        "head_chunk_tokens", "precision", "host_threads", "check_finite", "serialize",
        "host_alloc", "keep_grads", "time_kernels", "keep_internals", "defer_updates",
        "resident_layers", "opt_8bit")] + [
        (n, C.c_double) for n in ("lr", "beta1", "beta2", "eps", "weight_decay", "clip_norm")]


class LayerView(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")]


class StepStats(C.Structure):
    _fields_ = [(n, C.c_double) for n in (
        "step_ms", "fwd_ms", "head_ms", "bwd_ms", "adam_ms", "tail_ms", "h2d_bytes",
        "d2h_bytes", "h2d_ms", "d2h_ms", "exposed_wait_fwd_ms", "exposed_wait_bwd_ms",
        "probe_kernel_ms", "probe_kernel_flops")] + [(n, C.c_int64) for n in (
            "probe_kernel_launches", "pinned_host_bytes", "pageable_host_bytes",
            "device_arena_bytes", "units_updated")] + [(n, C.c_double) for n in (
                "host_ring_wait_ms", "host_slab_wait_ms", "host_op_wait_ms", "host_adam_idle_ms",
                "probe_all_gemm_ms")] + [("probe_kernel", C.c_char * 96)] + [
            (n, C.c_double) for n in ("host_start_ms", "gpu_done_ms", "grads_landed_ms",
                                      "updates_done_ms", "probe_all_attn_ms", "probe_all_flops",
                                      "grad_norm", "clip_factor")]

    def as_dict(self):
        d = {n: getattr(self, n) for n, _ in self._fields_}
        d["probe_kernel"] = self.probe_kernel.decode()
        return d


class KernelTime(C.Structure):
    _fields_ = [("name", C.c_char * 96), ("launches", C.c_int64), ("ms", C.c_double),
                ("flops", C.c_double)]


# ---------------------------------------------------------------- signatures
_P, _I32, _I64, _SZ, _F, _D = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float, C.c_double


def _fn(name, res, *args):
    f = getattr(_lib, name, None)
    if f is None:
        return None
    f.restype = res
    f.argtypes = list(args)
    return f


_lib.mt_last_error.restype = C.c_char_p
_lib.mt_last_error.argtypes = []

_SIGS = {
    "mt_op_gemm": (_I32, _I32, _I32, _I32, _I32, _I32, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                   _P, _I64, _P, _I64, _I32, _P, _SZ, _P),
    "mt_op_gemm_f32": (_I32, _I32, _I32, _I32, _I32, _I32, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                       _P, _I64, _P, _I64, _I32, _P),
    "mt_op_attn_fwd_f32": (_I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P),
    "mt_op_attn_bwd_f32": (_I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P),
    "mt_op_rmsnorm_fwd": (_I32, _P, _P, _P, _P, _I32, _I32, _F, _P),
    "mt_op_rmsnorm_bwd": (_I32, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _SZ, _P),
    "mt_op_rope_table": (_I32, _P, _P, _I32, _I32, _D, _P),
    "mt_op_rope": (_I32, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _P),
    "mt_op_attn_fwd": (_I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P),
    "mt_op_attn_bwd": (_I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P),
    "mt_op_attn_bwd_noalloc": (_I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P),
    "mt_op_ce_rows": (_I32, _P, _P, _P, _P, _I32, _I32, _F, _P),
    "mt_layer_workspace_bytes": (_SZ, _P, _P, _I32, _I32, _I32),
    "mt_layer_fwd": (_I32, _P, _P, _P, _P, _P, _I32, _I32, _P, _SZ, _P),
    "mt_layer_recompute_bwd": (_I32, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _SZ, _P),
    "mt_model_create": (_I32, _P, _P, _P),
    "mt_model_destroy": (None, _P),
    "mt_model_set_schedule": (_I32, _P, _P),
    "mt_model_set_param": (_I32, _P, C.c_char_p, _P, _SZ),
    "mt_model_get_param": (_I32, _P, C.c_char_p, _I32, _P, _SZ),
    "mt_model_step_count": (_I64, _P),
    "mt_model_kernel_times": (_I32, _P, _P, _I32, _P),
    "mt_stream_arena_bytes": (_SZ, _P, _I32, _I32),
    "mt_stream_arena_bytes_cfg": (_SZ, _P, _P, _I32, _I32),
    "mt_stream_step": (_I32, _P, _P, _I32, _I32, _P, _SZ, _P, _P, _P),
    "mt_host_adam": (_I32, _P, _P, _P, _P, _I32, _P, _SZ, _I64, _P),
    "mt_host_adam8": (_I32, _P, _P, _P, _P, _P, _P, _I32, _P, _SZ, _I64, _F, _P),
    "mt_run_cfg_default": (None, _P),
    "mt_op_rmsnorm_bwd_workspace": (_SZ, _I32, _I32),
    "mt_debug_plan": (_I32, _I32, _I32, _I32, _I32, _I32, _P, _SZ, _P),
    "mt_layer_internals_bytes": (_SZ, _P, _P, _I32, _I32),
    "mt_layer_fwd_keep": (_I32, _P, _P, _P, _P, _P, _I32, _I32, _P, _SZ, _P),
    "mt_layer_bwd_saved": (_I32, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _SZ, _P, _SZ, _P),
    "mt_op_nonfinite_flags": (_I32, _P, _SZ, _I32, _P, _P),
}
FN = {}
for _name, (_res, *_args) in _SIGS.items():
    FN[_name] = _fn(_name, _res, *_args)

EXPORTED = sorted(n for n, f in FN.items() if f is not None) + ["mt_last_error"]


def last_error() -> str:
    return (_lib.mt_last_error() or b"").decode()


def check(status: int, what: str = ""):
    if status != MT_OK:
        raise MTError(status, f"{what}: {last_error()}")


def call(name, *args):
    f = FN.get(name)
    if f is None:
        raise MTError(MT_E_INVALID, f"{name} is not exported by {LIB_PATH}")
    return f(*args)


# ------------------------------------------------------------------- helpers
def ptr(t):
    """Device or host address of a torch tensor / numpy array (None -> NULL)."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data  # numpy


def stream_handle(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def run_cfg(**kw) -> RunCfg:
    r = RunCfg()
    call("mt_run_cfg_default", C.byref(r))
    for k, v in kw.items():
        if not hasattr(r, k):
            raise AttributeError(k)
        setattr(r, k, v)
    return r


def model_cfg(shape) -> ModelCfg:
    return ModelCfg(shape.n_layers, shape.hidden, shape.n_heads, shape.n_kv_heads,
                    shape.head_dim, shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta)


# ----------------------------------------------------------------- op calls
GEMM_SPLIT_BYTES = 64 << 20  # MT_GEMM_SPLIT_BYTES


def gemm(layout, epi, M, N, K, A, lda, B, ldb, Cm, ldc, R=None, ldr=0, C2=None, ldc2=0,
         G=None, ldg=0, F=0, workspace=None, stream=None):
    """`workspace`: optional device tensor for the split tail tiles (see
    mt_op_gemm); None runs every tile whole."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(call("mt_op_gemm", layout, epi, M, N, K, ptr(A), lda, ptr(B), ldb, ptr(Cm), ldc,
               ptr(R), ldr, ptr(C2), ldc2, ptr(G), ldg, F, ptr(workspace), ws_bytes,
               stream_handle(stream)), "mt_op_gemm")


def gemm_f32(layout, epi, M, N, K, A, lda, B, ldb, Cm, ldc, R=None, ldr=0, C2=None, ldc2=0,
             G=None, ldg=0, F=0, stream=None):
    """The fp32 debug-precision product: every operand fp32."""
    check(call("mt_op_gemm_f32", layout, epi, M, N, K, ptr(A), lda, ptr(B), ldb, ptr(Cm), ldc,
               ptr(R), ldr, ptr(C2), ldc2, ptr(G), ldg, F, stream_handle(stream)),
          "mt_op_gemm_f32")


def rmsnorm_fwd(x, g, y, rstd, rows, cols, eps, stream=None):
    check(call("mt_op_rmsnorm_fwd", ptr(x), ptr(g), ptr(y), ptr(rstd), rows, cols, eps,
               stream_handle(stream)), "mt_op_rmsnorm_fwd")


def rmsnorm_bwd(dy, x, g, rstd, resid, dx, dg, rows, cols, ws, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    check(call("mt_op_rmsnorm_bwd", ptr(dy), ptr(x), ptr(g), ptr(rstd), ptr(resid), ptr(dx),
               ptr(dg), rows, cols, ptr(ws), nbytes, stream_handle(stream)), "mt_op_rmsnorm_bwd")


def rmsnorm_bwd_workspace(rows, cols) -> int:
    return call("mt_op_rmsnorm_bwd_workspace", rows, cols)


def rope_table(cos_t, sin_t, seq, head_dim, theta, stream=None):
    check(call("mt_op_rope_table", ptr(cos_t), ptr(sin_t), seq, head_dim, theta,
               stream_handle(stream)), "mt_op_rope_table")


def rope(qkv, batch, seq, n_heads, n_kv_heads, head_dim, cos_t, sin_t, inverse=0, stream=None):
    check(call("mt_op_rope", ptr(qkv), batch, seq, n_heads, n_kv_heads, head_dim, ptr(cos_t),
               ptr(sin_t), inverse, stream_handle(stream)), "mt_op_rope")


def attn_fwd(qkv, o, lse, batch, seq, n_heads, n_kv_heads, head_dim, stream=None):
    check(call("mt_op_attn_fwd", ptr(qkv), ptr(o), ptr(lse), batch, seq, n_heads, n_kv_heads,
               head_dim, stream_handle(stream)), "mt_op_attn_fwd")


def attn_bwd(qkv, o, lse, dout, delta, dqkv, batch, seq, n_heads, n_kv_heads, head_dim,
             stream=None):
    check(call("mt_op_attn_bwd", ptr(qkv), ptr(o), ptr(lse), ptr(dout), ptr(delta), ptr(dqkv),
               batch, seq, n_heads, n_kv_heads, head_dim, stream_handle(stream)), "mt_op_attn_bwd")


ATTN_NOALLOC_MAX_ROWS = 16 << 20  # MT_ATTN_NOALLOC_MAX_ROWS


def attn_bwd_noalloc(qkv, o, lse, dout, dqkv, batch, seq, n_heads, n_kv_heads, head_dim,
                     stream=None):
    """Attention backward with the library's static scratch (no workspace)."""
    check(call("mt_op_attn_bwd_noalloc", ptr(qkv), ptr(o), ptr(lse), ptr(dout), ptr(dqkv),
               batch, seq, n_heads, n_kv_heads, head_dim, stream_handle(stream)),
          "mt_op_attn_bwd_noalloc")


def attn_fwd_f32(qkv, o, lse, batch, seq, n_heads, n_kv_heads, head_dim, stream=None):
    check(call("mt_op_attn_fwd_f32", ptr(qkv), ptr(o), ptr(lse), batch, seq, n_heads, n_kv_heads,
               head_dim, stream_handle(stream)), "mt_op_attn_fwd_f32")


def attn_bwd_f32(qkv, o, lse, dout, delta, dqkv, batch, seq, n_heads, n_kv_heads, head_dim,
                 stream=None):
    check(call("mt_op_attn_bwd_f32", ptr(qkv), ptr(o), ptr(lse), ptr(dout), ptr(delta),
               ptr(dqkv), batch, seq, n_heads, n_kv_heads, head_dim, stream_handle(stream)),
          "mt_op_attn_bwd_f32")


def ce_rows(logits, target, dlogits, loss_part, rows, vocab, inv_n, stream=None):
    check(call("mt_op_ce_rows", ptr(logits), ptr(target), ptr(dlogits), ptr(loss_part), rows,
               vocab, inv_n, stream_handle(stream)), "mt_op_ce_rows")


# ------------------------------------------------------------- layer / model
class GradView(C.Structure):
    _fields_ = LayerView._fields_


def layer_workspace_bytes(mcfg, rcfg, batch, seq, which) -> int:
    return call("mt_layer_workspace_bytes", C.byref(mcfg), C.byref(rcfg), batch, seq, which)


def layer_fwd(mcfg, rcfg, view, x_in, x_out, batch, seq, ws, stream=None):
    check(call("mt_layer_fwd", C.byref(mcfg), C.byref(rcfg), C.byref(view), ptr(x_in),
               ptr(x_out), batch, seq, ptr(ws), ws.numel() * ws.element_size(),
               stream_handle(stream)), "mt_layer_fwd")


def layer_recompute_bwd(mcfg, rcfg, view, x_in, dy, dx, gview, batch, seq, ws, stream=None):
    check(call("mt_layer_recompute_bwd", C.byref(mcfg), C.byref(rcfg), C.byref(view), ptr(x_in),
               ptr(dy), ptr(dx), C.byref(gview), batch, seq, ptr(ws),
               ws.numel() * ws.element_size(), stream_handle(stream)), "mt_layer_recompute_bwd")


def layer_internals_bytes(mcfg, rcfg, batch, seq) -> int:
    return call("mt_layer_internals_bytes", C.byref(mcfg), C.byref(rcfg), batch, seq)


def layer_fwd_keep(mcfg, rcfg, view, x_in, x_out, batch, seq, internals, stream=None):
    check(call("mt_layer_fwd_keep", C.byref(mcfg), C.byref(rcfg), C.byref(view), ptr(x_in),
               ptr(x_out), batch, seq, ptr(internals), internals.numel() * internals.element_size(),
               stream_handle(stream)), "mt_layer_fwd_keep")


def layer_bwd_saved(mcfg, rcfg, view, x_in, dy, dx, gview, batch, seq, internals, ws,
                    stream=None):
    check(call("mt_layer_bwd_saved", C.byref(mcfg), C.byref(rcfg), C.byref(view), ptr(x_in),
               ptr(dy), ptr(dx), C.byref(gview), batch, seq, ptr(internals),
               internals.numel() * internals.element_size(), ptr(ws),
               ws.numel() * ws.element_size(), stream_handle(stream)), "mt_layer_bwd_saved")


def arena_bytes_for(shape, batch=None, seq=None, **run_kw) -> int:
    """mt_stream_arena_bytes_cfg: device arena of a step without a model."""
    mcfg = model_cfg(shape)
    kw = dict(ckpt_interval=shape.ckpt_interval, mlp_chunk_tokens=shape.mlp_chunk_tokens)
    kw.update(run_kw)
    r = run_cfg(**kw)
    return call("mt_stream_arena_bytes_cfg", C.byref(mcfg), C.byref(r),
                shape.batch if batch is None else batch, shape.seq if seq is None else seq)


def debug_plan(n_layers, ckpt_interval, prefetch_depth, keep_internals=1, resident_layers=0):
    """The engine's schedule as (status, ops [n,3], loads [n,6], n_slots)."""
    import numpy as np
    cap = 64 * (n_layers + 2) * 4 + 64
    out = np.zeros(cap, np.int32)
    counts = np.zeros(3, np.int32)
    st = call("mt_debug_plan", n_layers, ckpt_interval, prefetch_depth, keep_internals,
              resident_layers, ptr(out), cap, ptr(counts))
    n_ops, n_loads, n_slots = (int(c) for c in counts)
    ops = out[: 3 * n_ops].reshape(n_ops, 3).copy()
    loads = out[3 * n_ops: 3 * n_ops + 6 * n_loads].reshape(n_loads, 6).copy()
    return st, ops, loads, n_slots


class Model:
    """Host-resident model (mt_model) plus the streamed training step."""

    def __init__(self, shape, **run_kw):
        self.shape = shape
        self.mcfg = model_cfg(shape)
        kw = dict(ckpt_interval=shape.ckpt_interval, mlp_chunk_tokens=shape.mlp_chunk_tokens,
                  lr=shape.lr, beta1=shape.beta1, beta2=shape.beta2, eps=shape.adam_eps)
        kw.update(run_kw)
        self.rcfg = run_cfg(**kw)
        h = C.c_void_p()
        check(call("mt_model_create", C.byref(self.mcfg), C.byref(self.rcfg), C.byref(h)),
              "mt_model_create")
        self.h = h

    def close(self):
        if self.h:
            call("mt_model_destroy", self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_schedule(self, **run_kw):
        """Change schedule knobs between steps (mt_model_set_schedule); the
        knobs not named keep their current values."""
        r = RunCfg()
        C.memmove(C.byref(r), C.byref(self.rcfg), C.sizeof(RunCfg))
        for k, v in run_kw.items():
            if not hasattr(r, k):
                raise AttributeError(k)
            setattr(r, k, v)
        check(call("mt_model_set_schedule", self.h, C.byref(r)), "mt_model_set_schedule")
        self.rcfg = r

    def set_param(self, name, arr):
        import numpy as np
        a = np.ascontiguousarray(arr, dtype=np.float32).reshape(-1)
        check(call("mt_model_set_param", self.h, name.encode(), ptr(a), a.size),
              f"mt_model_set_param({name})")

    def set_params(self, weights):
        for n, a in weights.items():
            self.set_param(n, a)

    def get(self, name, which=GET_MASTER, shape=None):
        import numpy as np
        from synth import param_shapes
        shp = shape or param_shapes(self.shape)[name]
        out = np.empty(int(np.prod(shp)), np.float32)
        check(call("mt_model_get_param", self.h, name.encode(), which, ptr(out), out.size),
              f"mt_model_get_param({name})")
        return out.reshape(shp)

    def kernel_times(self):
        """The last step's timed launches per kernel (time_kernels=1), largest
        total time first: [{name, launches, ms, flops}]."""
        n = C.c_int32()
        check(call("mt_model_kernel_times", self.h, None, 0, C.byref(n)), "mt_model_kernel_times")
        arr = (KernelTime * max(n.value, 1))()
        check(call("mt_model_kernel_times", self.h, arr, n.value, C.byref(n)),
              "mt_model_kernel_times")
        return [{"name": k.name.decode(), "launches": int(k.launches), "ms": float(k.ms),
                 "flops": float(k.flops)} for k in arr[: n.value]]

    @property
    def step_count(self):
        return call("mt_model_step_count", self.h)

    def arena_bytes(self, batch, seq):
        return call("mt_stream_arena_bytes", self.h, batch, seq)

    def step(self, tokens, arena, streams):
        """One streamed training step; returns (loss, stats dict)."""
        import numpy as np
        ids = np.ascontiguousarray(tokens, dtype=np.int32)
        B, T = ids.shape
        loss = C.c_float()
        stats = StepStats()
        handles = (C.c_void_p * 3)(*[s.cuda_stream for s in streams])
        check(call("mt_stream_step", self.h, ptr(ids), B, T, ptr(arena),
                   arena.numel() * arena.element_size(), handles, C.byref(loss),
                   C.byref(stats)), "mt_stream_step")
        return float(loss.value), stats.as_dict()
