"""moelora_forward_noalloc, the entry point that allocates nothing (its
workspace is the library's static device scratch array), against
moelora_forward with a caller workspace: the same kernels on the same
layout, so the outputs agree bit for bit.  Two calls in a row on the shared
array, the second with fewer tokens, check that what a call leaves behind
does not leak into the next; an oversized call is refused before any
device work."""
import numpy as np
import pytest
import torch

import oracle
import synth
from layer_harness import Run, check_close, dev, lib, oracle_out

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def noalloc(run, T):
    L = lib()
    t = run.t
    out = torch.full_like(run.out, -1)
    L.moelora_forward_noalloc(run.plan.handle, T, t["x"], t["logits"], None, None,
                              t["adapter_ids"], t["W_gu"], t["W_d"], t.get("A_gu"),
                              t.get("B_gu"), t.get("A_d"), t.get("B_d"), out)
    return out


CASES = [
    # T, H, I, E, k, NA, r, then the smaller second call
    ((40, 256, 384, 8, 2, 3, 16), 9),     # row-wise LoRA, streaming blocks
    ((200, 128, 192, 64, 2, 3, 16), 50),  # tile-wise LoRA, split shrinks
    ((16, 2880, 2880, 32, 4, 8, 32), 5),  # the decode workload's shape
]


@pytest.mark.parametrize("shape,T2", CASES)
def test_noalloc_matches_workspace_entry_point(shape, T2):
    T, H, I, E, k, NA, r = shape
    w = synth.Workload("noalloc", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T + H)
    d = synth.make_inputs(w)
    run = Run(w, d)
    assert run.plan.workspace_bytes <= lib().STATIC_SCRATCH_BYTES
    say(f"[noalloc] {w}: plan {run.plan.info(T)}")
    a1 = noalloc(run, T)          # two calls in a row on the shared array,
    a2 = noalloc(run, T2)         # the second with fewer tokens
    torch.cuda.synchronize()
    for n, got in ((T, a1), (T2, a2)):
        run.out.fill_(-1)
        run.forward(T=n)
        torch.cuda.synchronize()
        assert torch.equal(got, run.out), f"n_tokens={n}: noalloc output differs"
        assert (got[n:].cpu().numpy() == -1).all()
    rid, rw = oracle.ref_route(d["logits"], k)
    tok = np.arange(T2, dtype=np.int32)
    got = synth.bf16_bits_to_f32(a2[:T2].cpu().numpy().view(np.uint16))
    d2 = dict(d, x=d["x"][:T2], logits=d["logits"][:T2], adapter_ids=d["adapter_ids"][:T2])
    w2 = synth.Workload("noalloc", T=T2, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                        adapters="uniform_with_none", seed=T + H)
    check_close(got, oracle_out(w2, d2, rid[:T2], rw[:T2], tokens=tok), "bf16", "noalloc")


def test_noalloc_refuses_calls_beyond_the_array():
    """A call whose workspace exceeds the static array returns
    MOELORA_ERR_TOO_LARGE; a smaller call on the same plan runs."""
    L = lib()
    T, H, I, E, k = 200_000, 64, 64, 4, 2
    plan = L.Plan(T, H, I, E, k, 0, 0, L.BF16)
    assert int(dict(kv.split("=") for kv in plan.info(T).split())["workspace"]) > \
        L.STATIC_SCRATCH_BYTES
    rng = np.random.default_rng(5)
    x = dev(synth.f32_to_bf16_bits(rng.standard_normal((T, H), np.float32)))
    logits = dev(rng.standard_normal((T, E), np.float32))
    wgu = dev(synth.f32_to_bf16_bits(rng.standard_normal((E, 2 * I, H), np.float32) / 8))
    wd = dev(synth.f32_to_bf16_bits(rng.standard_normal((E, H, I), np.float32) / 8))
    out = torch.full((T, H), -1, dtype=torch.int16, device="cuda")
    with pytest.raises(L.MoeLoraError) as ei:
        L.moelora_forward_noalloc(plan.handle, T, x, logits, None, None, None, wgu, wd,
                                  None, None, None, None, out)
    assert ei.value.status == L.ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == -1).all()
    n = 2000
    L.moelora_forward_noalloc(plan.handle, n, x, logits, None, None, None, wgu, wd,
                              None, None, None, None, out)
    ref = torch.full_like(out, -1)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    plan.forward(n, x, ref, ws, router_logits=logits, w_gate_up=wgu, w_down=wd)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
