"""Child program of tests/test_gpu_steady_state.py (run under rocprofv3).

One plan serves forwards at token counts in every block-size bucket of a
128-expert top-8 layer (16- and 32-row streaming blocks, row- and tile-wise
LoRA, 128-row LDS-tiled blocks).  Everything is allocated, and one forward
run, before a first marker call; the forwards at every other token count
follow, then a second marker.  The trace between the two markers must show
kernel launches only: no code-object load, no allocation, no copy, no
synchronisation.  The markers are hipDriverGetVersion calls (the program
makes no other).
"""
import ctypes
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import lora_expert_gemm_amd as L  # noqa: E402
import synth  # noqa: E402

TOKENS = [1, 3, 24, 40, 64, 100, 256, 300, 700, 1024, 2048]


def main():
    w = synth.Workload("steady", T=max(TOKENS), H=2048, I=768, E=128, k=8, NA=32, r=16,
                       dtype="bf16", adapters="uniform_with_none", seed=17)
    d = synth.make_inputs(w)
    t = {n: torch.from_numpy(np.ascontiguousarray(v.view(np.int16) if v.dtype == np.uint16 else v))
         .cuda() for n, v in d.items() if v is not None}
    plan = L.Plan(w.T, w.H, w.I, w.E, w.k, w.NA, w.r, L.BF16)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.T, w.H), dtype=torch.int16, device="cuda")
    buckets = {T: plan.info(T).split()[1] for T in TOKENS}
    print("[child] buckets " + " ".join(f"{T}:{b}" for T, b in buckets.items()), flush=True)
    hip = ctypes.CDLL("libamdhip64.so")
    ver = ctypes.c_int()

    def fwd(T):
        plan.forward(T, t["x"], out, ws, router_logits=t["logits"],
                     adapter_ids=t["adapter_ids"], w_gate_up=t["W_gu"], w_down=t["W_d"],
                     lora_a_gu=t["A_gu"], lora_b_gu=t["B_gu"], lora_a_d=t["A_d"],
                     lora_b_d=t["B_d"])

    fwd(TOKENS[0])
    torch.cuda.synchronize()
    hip.hipDriverGetVersion(ctypes.byref(ver))   # marker: steady state begins
    for T in TOKENS[1:] + TOKENS[::-1]:
        fwd(T)
    hip.hipDriverGetVersion(ctypes.byref(ver))   # marker: steady state ends
    torch.cuda.synchronize()
    print(f"[child] done: {2 * len(TOKENS) - 1} forwards after the first", flush=True)


if __name__ == "__main__":
    main()
