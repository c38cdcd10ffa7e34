"""Seeded synthetic workloads for the fused MoE-LoRA layer.

This module draws inputs only; it holds none of the layer's arithmetic and
is shared by the tests, the smoke check and the benchmark, so that the GPU
library and the CPU oracle receive identical bytes.

Recipe (numpy PCG64 streams seeded by ``default_rng([seed, tensor, ...])``;
seed = 1000 + workload index for the named workloads):
  tensor 0  router logits [T][E] ~ N(0, 1), plus, for the skewed workload, a
            per-expert bias ~ N(0, bias_var) drawn after the logits;
  tensor 1  adapter ids (scheme per workload, see adapter_ids());
  tensor 2  x [T][H] ~ N(0, 1);
  tensors 3..8  W_gu ~ N(0, 1/H), W_d ~ N(0, 1/I), A_gu ~ N(0, 1/H),
            B_gu ~ N(0, 1/r), A_d ~ N(0, 1/H), B_d ~ N(0, 1/r).
N(0, v) means variance v.  Workloads with E4M3 base weights (wdtype "fp8")
draw W_gu and W_d the same way in float32 and store each weight row as
OCP 8-bit E4M3 codes with one float32 scale: scale = max|row| / 448 (the
format's largest finite value; 1 for an all-zero row), codes = the row
divided by its scale, rounded to the nearest E4M3 value (ties to even, by
torch's float8_e4m3fn conversion).  Weight tensors are drawn per leading index i (an
expert, or an adapter-expert pair) in chunks of 2**22 elements, chunk c from
``default_rng([seed, tensor, i, c])``, so generation can run on several
threads and gives the same bytes on any host.  Normal draws are float32;
bf16 workloads round every draw to bf16 with round-to-nearest-even; the
router logits stay float32.

The shapes stand in for the serving workload of the AWS post "Efficiently
serve dozens of fine-tuned models with vLLM on Amazon SageMaker AI and Amazon
Bedrock" (section "Implementing multi-LoRA inference for MoE models in vLLM":
input length 1600, concurrency 16; Figure 1: hidden 4096, intermediate
11008, rank 32; Figure 3: rank 32 with 8 adapters), which is not reproduced.
"""
import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    H: int            # hidden size
    I: int            # expert intermediate size (gate_up produces 2I)
    E: int            # experts
    k: int            # top-k
    NA: int           # adapters
    r: int            # LoRA rank
    dtype: str        # "f32" or "bf16"
    adapters: str     # adapter-id scheme, see adapter_ids()
    seq_len: int = 0  # tokens per sequence for the "per_sequence" scheme
    bias_var: float = 0.0  # variance of a per-expert router bias (0 = none)
    seed: int = 0
    wdtype: str = ""  # base weights: "" (the layer dtype) or "fp8" (E4M3 + row scales)


WORKLOADS = [
    Workload("tiny_fp32", T=8, H=128, I=256, E=4, k=2, NA=2, r=8,
             dtype="f32", adapters="uniform_with_none", seed=1000),
    Workload("decode_bf16", T=16, H=2880, I=2880, E=32, k=4, NA=8, r=32,
             dtype="bf16", adapters="uniform", seed=1001),
    Workload("illustrative_bf16", T=64, H=4096, I=11008, E=8, k=2, NA=16,
             r=32, dtype="bf16", adapters="uniform_with_none", seed=1002),
    Workload("prefill_bf16", T=6400, H=2880, I=2880, E=32, k=4, NA=4, r=64,
             dtype="bf16", adapters="per_sequence", seq_len=1600, seed=1003),
    Workload("many_expert_bf16", T=256, H=2048, I=768, E=128, k=8, NA=32,
             r=16, dtype="bf16", adapters="zipf_with_none", bias_var=0.5,
             seed=1004),
    # dense (non-MoE) multi-LoRA: one expert, top-1, on the illustrative
    # shape (the post's Figure 1 MLP); not one of the five reference configs
    Workload("dense_bf16", T=64, H=4096, I=11008, E=1, k=1, NA=16, r=32,
             dtype="bf16", adapters="uniform_with_none", seed=1005),
    # E4M3 base weights with row scales (the low-precision weights of the
    # aib.vote news item on SageMaker fused-MoE kernel optimizations, second
    # item) on the decode, illustrative and many-expert shapes
    Workload("decode_fp8w", T=16, H=2880, I=2880, E=32, k=4, NA=8, r=32,
             dtype="bf16", adapters="uniform", seed=1006, wdtype="fp8"),
    Workload("illustrative_fp8w", T=64, H=4096, I=11008, E=8, k=2, NA=16,
             r=32, dtype="bf16", adapters="uniform_with_none", seed=1007, wdtype="fp8"),
    Workload("many_expert_fp8w", T=256, H=2048, I=768, E=128, k=8, NA=32,
             r=16, dtype="bf16", adapters="zipf_with_none", bias_var=0.5,
             seed=1008, wdtype="fp8"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def workload(name_or_index, **overrides):
    w = WORKLOADS[name_or_index] if isinstance(name_or_index, int) \
        else BY_NAME[name_or_index]
    return replace(w, **overrides) if overrides else w


def f32_to_bf16_bits(a):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even
    (NaN kept quiet)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def adapter_ids(w: Workload, rng):
    """Per-token adapter ids (-1 = base model only).

    uniform            uniform over 0..NA-1
    uniform_with_none  uniform over -1..NA-1
    per_sequence       token t belongs to sequence t // seq_len, which uses
                       adapter (t // seq_len) % NA
    zipf_with_none     P(j) proportional to (j+1)**-1.2 over 0..NA-1, then
                       round(0.3 T) tokens chosen by a seeded permutation are
                       set to -1
    none               all -1
    """
    T, NA = w.T, w.NA
    if w.adapters == "uniform":
        return rng.integers(0, NA, size=T).astype(np.int32)
    if w.adapters == "uniform_with_none":
        return rng.integers(-1, NA, size=T).astype(np.int32)
    if w.adapters == "per_sequence":
        return ((np.arange(T) // w.seq_len) % NA).astype(np.int32)
    if w.adapters == "zipf_with_none":
        p = (np.arange(1, NA + 1, dtype=np.float64)) ** -1.2
        ids = rng.choice(NA, size=T, p=p / p.sum()).astype(np.int32)
        off = rng.permutation(T)[: int(round(0.3 * T))]
        ids[off] = -1
        return ids
    if w.adapters == "none":
        return np.full(T, -1, np.int32)
    raise ValueError(w.adapters)


def _normal(rng, shape, var):
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(np.sqrt(var))
    return a


def _fill_bf16(out_u16, f, u):
    """Round the (finite) float32 values in f to bf16 bits into out_u16,
    round to nearest even; u is uint32 scratch of the same size."""
    fb = f.view(np.uint32)
    np.right_shift(fb, 16, out=u)
    np.bitwise_and(u, 1, out=u)
    np.add(u, 0x7FFF, out=u)
    np.add(u, fb, out=u)
    np.right_shift(u, 16, out=u)
    np.copyto(out_u16, u, casting="unsafe")


_CHUNK = 1 << 22
_tls = threading.local()


def _scratch(n):
    f = getattr(_tls, "f", None)
    if f is None or f.size < n:
        _tls.f = np.empty(n, np.float32)
        _tls.u = np.empty(n, np.uint32)
    return _tls.f[:n], _tls.u[:n]


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


def _stacked(seed, tensor, lead, shape, var, store):
    """Draw a [*lead, *shape] tensor; chunk c of leading index i comes from
    its own stream default_rng([seed, tensor, i, c])."""
    n = int(np.prod(lead))
    m = int(np.prod(shape))
    out = np.empty((n, m), np.uint16 if store == "bf16" else np.float32)
    std = np.float32(np.sqrt(var))

    def job(i, c):
        lo, hi = c * _CHUNK, min(m, (c + 1) * _CHUNK)
        rng = np.random.default_rng([seed, tensor, i, c])
        if store == "bf16":
            f, u = _scratch(hi - lo)
            rng.standard_normal(out=f, dtype=np.float32)
            f *= std
            _fill_bf16(out[i, lo:hi], f, u)
        else:
            o = out[i, lo:hi]
            rng.standard_normal(out=o, dtype=np.float32)
            o *= std

    jobs = [(i, c) for i in range(n) for c in range((m + _CHUNK - 1) // _CHUNK)]
    if len(jobs) == 1 or n * m < (1 << 20):
        for j in jobs:
            job(*j)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(lambda j: job(*j), jobs))
    return out.reshape(tuple(lead) + tuple(shape))


def quantize_e4m3_rows(f):
    """float32 [..., rows, K] -> (uint8 E4M3 codes, float32 scales [..., rows]),
    one scale per row (max|row| / 448, 1 for an all-zero row)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f, np.float32))
    amax = t.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (t / scale.unsqueeze(-1)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), scale.numpy().astype(np.float32)


def _stacked_fp8(seed, tensor, lead, shape, var):
    """The float32 draws of _stacked (the same streams), each weight row
    quantised to E4M3 with its scale, one leading index at a time."""
    n = int(np.prod(lead))
    m = int(np.prod(shape))
    codes = np.empty((n,) + tuple(shape), np.uint8)
    scales = np.empty((n, shape[0]), np.float32)
    std = np.float32(np.sqrt(var))
    f = np.empty(m, np.float32)

    def job(i, c):
        lo, hi = c * _CHUNK, min(m, (c + 1) * _CHUNK)
        np.random.default_rng([seed, tensor, i, c]).standard_normal(out=f[lo:hi], dtype=np.float32)
        f[lo:hi] *= std

    nchunk = (m + _CHUNK - 1) // _CHUNK
    with ThreadPoolExecutor(_workers()) as ex:
        for i in range(n):
            list(ex.map(lambda c: job(i, c), range(nchunk)))
            codes[i], scales[i] = quantize_e4m3_rows(f.reshape(shape))
    return codes.reshape(tuple(lead) + tuple(shape)), scales.reshape(tuple(lead) + (shape[0],))


def make_inputs(w: Workload, lora=True):
    """All inputs of one layer call as numpy arrays in storage form
    (float32, or uint16 bf16 bits for bf16 workloads; E4M3 base weights as
    uint8 codes with float32 row scales W_gu_scale [E][2I], W_d_scale [E][H])."""
    T, H, I, E, NA, r = w.T, w.H, w.I, w.E, w.NA, w.r
    rng = np.random.default_rng([w.seed, 0])
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if w.bias_var > 0:
        bias = _normal(rng, (E,), w.bias_var)
        logits = (logits + bias[None, :]).astype(np.float32)
    aid = adapter_ids(w, np.random.default_rng([w.seed, 1]))
    st = w.dtype
    x = _stacked(w.seed, 2, (), (T, H), 1.0, st)
    d = dict(logits=logits, adapter_ids=aid, x=x)
    if w.wdtype == "fp8":
        d["W_gu"], d["W_gu_scale"] = _stacked_fp8(w.seed, 3, (E,), (2 * I, H), 1.0 / H)
        d["W_d"], d["W_d_scale"] = _stacked_fp8(w.seed, 4, (E,), (H, I), 1.0 / I)
    else:
        d["W_gu"] = _stacked(w.seed, 3, (E,), (2 * I, H), 1.0 / H, st)
        d["W_d"] = _stacked(w.seed, 4, (E,), (H, I), 1.0 / I, st)
    if lora and NA > 0 and r > 0:
        d["A_gu"] = _stacked(w.seed, 5, (NA, E), (r, H), 1.0 / H, st)
        d["B_gu"] = _stacked(w.seed, 6, (NA, E), (2 * I, r), 1.0 / r, st)
        d["A_d"] = _stacked(w.seed, 7, (NA, E), (r, I), 1.0 / H, st)
        d["B_d"] = _stacked(w.seed, 8, (NA, E), (H, r), 1.0 / r, st)
    else:
        d["A_gu"] = d["B_gu"] = d["A_d"] = d["B_d"] = None
    return d
