"""Helpers for the GPU tests: upload a seeded workload, run the layer
through the C ABI, run the oracle on the same bytes, and compare."""
import numpy as np
import torch

import oracle
import synth

# Tolerances of the fused layer against the oracle: max|err| <= 2e-2 *
# max|ref| and relative Frobenius error <= 5e-3 for bf16 storage (1e-5 for
# float32 storage).
MAX_REL = 2e-2
FRO_REL = {"bf16": 5e-3, "f32": 1e-5}


def lib():
    import lora_expert_gemm_amd
    return lora_expert_gemm_amd


def dev(a):
    """numpy -> cuda tensor with the same bytes (bf16 bits as int16)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Run:
    """One layer call: plan, device inputs, workspace, output."""

    def __init__(self, w: synth.Workload, d, *, route="logits", lora=True, ids=None,
                 wts=None, max_tokens=None, adapter_ids="given"):
        L = lib()
        self.w, self.d = w, d
        self.dtype = L.BF16_FP8W if w.wdtype == "fp8" else L.BF16 if w.dtype == "bf16" else L.F32
        self.plan = L.Plan(max_tokens or w.T, w.H, w.I, w.E, w.k, w.NA, w.r, self.dtype)
        self.ws = torch.empty(max(self.plan.workspace_bytes, 256), dtype=torch.uint8,
                              device="cuda")
        self.t = {n: dev(v) for n, v in d.items()
                  if v is not None and n != "logits" and not n.endswith("_scale")}
        if w.wdtype == "fp8":  # codes and row scales in one buffer, as the ABI lays them out
            for n in ("W_gu", "W_d"):
                self.t[n] = dev(L.fp8_weight_buffer(d[n], d[n + "_scale"]))
        self.t["logits"] = dev(d["logits"])
        if ids is not None:
            self.t["ids"] = dev(np.ascontiguousarray(ids, np.int32))
            self.t["w"] = dev(np.ascontiguousarray(wts, np.float32))
        self.route = route
        self.lora = lora
        self.use_aid = adapter_ids
        out_dtype = torch.int16 if w.dtype == "bf16" else torch.float32
        self.out = torch.full((w.T, w.H), -1, dtype=out_dtype, device="cuda")

    def forward(self, T=None, stream=None):
        t = self.t
        lo = self.lora
        self.plan.forward(
            self.w.T if T is None else T, t["x"], self.out, self.ws,
            router_logits=t["logits"] if self.route == "logits" else None,
            topk_ids=t.get("ids") if self.route == "ids" else None,
            topk_w=t.get("w") if self.route == "ids" else None,
            adapter_ids=t["adapter_ids"] if self.use_aid == "given" else None,
            w_gate_up=t["W_gu"], w_down=t["W_d"],
            lora_a_gu=t.get("A_gu") if lo else None, lora_b_gu=t.get("B_gu") if lo else None,
            lora_a_d=t.get("A_d") if lo else None, lora_b_d=t.get("B_d") if lo else None,
            stream=stream)
        return self

    def out_f32(self):
        torch.cuda.synchronize()
        o = self.out.cpu().numpy()
        if self.w.dtype == "bf16":
            return synth.bf16_bits_to_f32(o.view(np.uint16))
        return o

    def ws_ints(self, off, n, dtype=np.int32):
        torch.cuda.synchronize()
        b = self.ws[off: off + 4 * n].cpu().numpy()
        return b.view(dtype).copy()

    def routing(self, T=None):
        T = self.w.T if T is None else T
        lay = self.plan.layout(T)
        R = T * self.w.k
        ids = self.ws_ints(lay["off_topk_ids"], R).reshape(T, self.w.k)
        wts = self.ws_ints(lay["off_topk_w"], R, np.float32).reshape(T, self.w.k)
        return ids, wts

    def alignment(self, T=None):
        T = self.w.T if T is None else T
        lay = self.plan.layout(T)
        g = lambda name, n: self.ws_ints(lay[name], n)
        counts = g("off_counts", 4)
        return dict(block_m=lay["block_m"],
                    sorted_rows=g("off_sorted_rows", lay["cap"]),
                    block_expert=g("off_block_expert", lay["nblk"]),
                    seg_start=g("off_seg_start", self.w.E + 1),
                    lora_seg=g("off_lora_seg", 4 * lay["max_seg"]).reshape(-1, 4),
                    tiles=g("off_tiles", 4 * lay["max_tiles"]).reshape(-1, 4),
                    block_tile_start=g("off_block_tile_start", lay["nblk"] + 1),
                    num_padded=int(counts[0]), n_lora_seg=int(counts[1]),
                    n_tiles=int(counts[2]))

    def device_error(self):
        return lib().moelora_read_device_error(self.plan.handle, self.ws, stream=None)


def oracle_out(w, d, ids, wts, tokens=None, lora=True, adapter_ids="given"):
    dt = oracle.BF16_FP8W if w.wdtype == "fp8" else oracle.BF16 if w.dtype == "bf16" \
        else oracle.F32
    use = lora and w.NA > 0 and w.r > 0 and d["A_gu"] is not None
    aid = d["adapter_ids"] if adapter_ids == "given" else None
    return oracle.ref_forward(
        d["x"], ids, wts, aid if use else None, d["W_gu"], d["W_d"],
        d["A_gu"] if use else None, d["B_gu"] if use else None,
        d["A_d"] if use else None, d["B_d"] if use else None,
        inter=w.I, rank=w.r if use else 0, n_adapters=w.NA if use else 0, dtype=dt,
        tokens=None if tokens is None else np.asarray(tokens, np.int32),
        W_gu_scale=d.get("W_gu_scale"), W_d_scale=d.get("W_d_scale"))


def check_close(got, ref, dtype, what=""):
    """The layer's tolerance; returns (max_rel, fro_rel) for logging."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = got - ref
    scale = np.abs(ref).max()
    max_rel = np.abs(err).max() / scale if scale > 0 else np.abs(err).max()
    fro = np.linalg.norm(ref)
    fro_rel = np.linalg.norm(err) / fro if fro > 0 else np.linalg.norm(err)
    assert max_rel <= MAX_REL, f"{what}: max|err|/max|ref| = {max_rel:.3e}"
    assert fro_rel <= FRO_REL[dtype], f"{what}: relative Frobenius error {fro_rel:.3e}"
    return max_rel, fro_rel


def check_alignment(got, ref):
    n = ref["num_padded"]
    assert got["num_padded"] == n
    assert np.array_equal(got["seg_start"], ref["seg_start"])
    assert np.array_equal(got["sorted_rows"], ref["sorted_rows"])
    assert np.array_equal(got["block_expert"], ref["block_expert"])
    assert got["n_lora_seg"] == ref["n_lora_seg"]
    assert np.array_equal(got["lora_seg"], ref["lora_seg"])
    assert got["n_tiles"] == ref["n_tiles"]
    assert np.array_equal(got["tiles"], ref["tiles"])
    assert np.array_equal(got["block_tile_start"], ref["block_tile_start"])
