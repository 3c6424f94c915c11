"""Runs the step's dominant kernel alone, at the 7B shape, for hardware
counter collection (rocprofv3 --pmc), next to a plain device copy of known
size whose counter readings calibrate bytes per counter unit.

The kernel is the gate/up projection with its SwiGLU epilogue:
[16384 x 3584] x [37888 x 3584]^T -> m [16384 x 18944] (bf16), the same
launch mt_stream_step makes for every layer's forward and re-forward.

Usage: python -m layer_streamed_amd.kernel_profile [--reps N]
"""
import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    import torch

    from layer_streamed_amd import mt

    D, H, F = 16384, 3584, 18944
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((D, H), device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn((2 * F, H), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    m = torch.empty((D, F), device="cuda", dtype=torch.bfloat16)
    copy_bytes = 1 << 30
    src = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        mt.gemm(mt.GEMM_NT, mt.EPI_SWIGLU, D, 2 * F, H, x, H, w, H, m, F, F=F)
        dst.copy_(src)
    torch.cuda.synchronize()
    algo = (D * H + 2 * F * H) * 2 + D * F * 2
    print(f"gate/up GEMM: algorithmic bytes per launch {algo} "
          f"(A {D * H * 2}, B {2 * F * H * 2}, C {D * F * 2}); copy kernel bytes "
          f"{copy_bytes} read + {copy_bytes} written per launch", flush=True)


if __name__ == "__main__":
    main()
