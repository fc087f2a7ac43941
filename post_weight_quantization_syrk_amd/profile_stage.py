"""Run one stage of the path in isolation, for profilers (rocprofv3).

  python -m post_weight_quantization_syrk_amd.profile_stage --stage hessian --reps 3

Stages: hessian (H += 2 X^T X, 4096 wide, 262144 bf16 tokens), prepare
(d = 4096), quantize (4096 x 4096, 4-bit g128), pack, copy (a 1 GiB device
copy of known size, to calibrate byte counters).  Inputs are random device
tensors (values do not change the work done, except that the Hessian handed
to prepare is made positive definite).
"""
from __future__ import annotations

import argparse
import sys
import time

import torch

from . import gptq


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--stage", required=True,
                    choices=["hessian", "prepare", "quantize", "pack", "copy"])
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--d", type=int, default=4096)
    ap.add_argument("--d-out", type=int, default=4096)
    ap.add_argument("--tokens", type=int, default=262144)
    a = ap.parse_args(argv)
    dev = "cuda:0"
    torch.manual_seed(0)
    d, n, d_out = a.d, a.tokens, a.d_out
    if a.stage == "copy":
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        run = lambda: dst.copy_(src)
    elif a.stage == "hessian":
        X = torch.randn((n, d), device=dev, dtype=torch.float32).to(torch.bfloat16)
        H = torch.zeros((d, d), device=dev)
        ws = torch.empty(gptq.gptq_hessian_workspace(d, n, gptq.GPTQ_BF16), dtype=torch.uint8,
                         device=dev)
        run = lambda: gptq.gptq_hessian_accumulate(H, X, ws=ws)
    else:
        x = torch.randn((4 * d, d), device=dev)
        H0 = 2.0 * (x.T @ x)
        H = H0.clone()
        U = torch.empty((d, d), device=dev)
        dead = torch.empty(d, dtype=torch.uint8, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        wsp = torch.empty(gptq.gptq_prepare_workspace(d), dtype=torch.uint8, device=dev)

        def prep():
            H.copy_(H0)
            gptq.gptq_prepare_hinv(H, 0.01, U, dead, st, ws=wsp, check=False)

        if a.stage == "prepare":
            run = prep
        else:
            prep()
            W = (0.02 * torch.randn((d_out, d), device=dev)).to(torch.bfloat16)
            wsq = torch.empty(gptq.gptq_quantize_workspace(d_out, d, 128), dtype=torch.uint8,
                              device=dev)
            codes = torch.empty((d_out, d), dtype=torch.uint8, device=dev)
            sc = torch.empty((d_out, d // 128), device=dev)
            ze = torch.empty((d_out, d // 128), device=dev)
            quant = lambda: gptq.gptq_quantize_layer(W, U, dead, bits=4, group_size=128,
                                                     codes=codes, scales=sc, zeros=ze,
                                                     want_loss=False, ws=wsq)
            if a.stage == "quantize":
                run = quant
            else:
                quant()
                run = lambda: gptq.gptq_pack(codes, sc, ze, bits=4, group_size=128, sym=False)
    torch.cuda.synchronize()
    for r in range(a.reps):
        t0 = time.perf_counter()
        run()
        torch.cuda.synchronize()
        print(f"[profile_stage] {a.stage} rep {r}: {(time.perf_counter() - t0) * 1e3:.3f} ms",
              flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
