"""Pins of the CPU oracle to facts other than itself.

Each test checks the oracle against one of: a closed-form example worked by
hand (tests/golden/), brute force, a library routine (numpy sort, torch
SiLU / softmax, float64 matmul), or a mathematical identity of the method
(B = 0 gives the base MoE; one adapter equals the merged weight W + AB; the
top-k weights sum to one; identical experts make the routing irrelevant).
The method is the fused MoE-LoRA layer of the AWS ML blog post "Efficiently
serve dozens of fine-tuned models with vLLM on Amazon SageMaker AI and Amazon
Bedrock", section "Implementing multi-LoRA inference for MoE models in vLLM".
"""
import json
import os

import numpy as np
import pytest
import torch

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f32(a):
    return np.asarray(a, np.float32)


def small_workload(T=6, H=16, I=12, E=3, k=2, NA=2, r=4, adapters="uniform_with_none", seed=7):
    w = synth.Workload("pin", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="f32",
                       adapters=adapters, seed=seed)
    return w, synth.make_inputs(w)


def run_oracle(o, d, w, ids, wts, lora=True, **kw):
    return o.ref_forward(d["x"], ids, wts, d["adapter_ids"] if lora else None,
                         d["W_gu"], d["W_d"],
                         d["A_gu"] if lora else None, d["B_gu"] if lora else None,
                         d["A_d"] if lora else None, d["B_d"] if lora else None,
                         inter=w.I, rank=w.r if lora else 0,
                         n_adapters=w.NA if lora else 0, dtype=o.F32, **kw)


# ---------------------------------------------------------------- golden


def test_golden_hand_example(oracle_lib):
    g = _load("hand_two_tokens.json")
    dm = g["dims"]
    out = oracle_lib.ref_forward(
        _f32(g["x"]), np.asarray(g["ids"], np.int32), np.asarray(g["w"]),
        np.asarray(g["adapter_ids"], np.int32), _f32(g["W_gu"]), _f32(g["W_d"]),
        _f32(g["A_gu"]), _f32(g["B_gu"]), _f32(g["A_d"]), _f32(g["B_d"]),
        inter=dm["I"], rank=dm["r"], n_adapters=dm["NA"], dtype=oracle_lib.F32)
    np.testing.assert_allclose(out, np.asarray(g["expected_out"]), rtol=1e-14, atol=1e-15)


def test_golden_route_cases(oracle_lib):
    for c in _load("route_cases.json")["cases"]:
        ids, w = oracle_lib.ref_route(_f32([c["logits"]]), c["k"])
        assert ids[0].tolist() == c["ids"], c["note"]
        np.testing.assert_allclose(w[0], c["w"], rtol=0, atol=c["tol"] + 1e-15)


# ---------------------------------------------------------------- router


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (40, 32, 4), (20, 128, 8), (10, 5, 5)])
def test_route_matches_stable_sort_and_softmax(oracle_lib, T, E, k):
    rng = np.random.default_rng(T * E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[: T // 2] = np.round(logits[: T // 2], 1)  # plenty of exact ties
    ids, w = oracle_lib.ref_route(logits, k)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert (ids == order).all()
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    sel = np.take_along_axis(p, order, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    if k == E:  # top-E of a softmax, renormalised, is the softmax itself
        np.testing.assert_allclose(w, np.take_along_axis(p, ids, axis=1), rtol=1e-13)


# ---------------------------------------------------------------- alignment


def brute_align(ids, aid, E, NA, BM):
    """Alignment by Python's sorted() on the key (expert, adapter rank, row)."""
    T, k = ids.shape
    R = T * k
    arank = [aid[p // k] if aid is not None and 0 <= aid[p // k] < NA else NA for p in range(R)]
    rows = sorted((p for p in range(R) if 0 <= ids.flat[p] < E),
                  key=lambda p: (ids.flat[p], arank[p], p))
    seg, pos, sorted_rows, block_expert, lora_seg, tiles = [0], 0, [], [], [], []
    for e in range(E):
        mine = [p for p in rows if ids.flat[p] == e]
        padded = -(-len(mine) // BM) * BM
        for a in range(NA):
            run = [i for i, p in enumerate(mine) if arank[p] == a]
            if run:
                lora_seg.append((e, a, pos + run[0], len(run)))
        sorted_rows += mine + [R] * (padded - len(mine))
        block_expert += [e] * (padded // BM)
        pos += padded
        seg.append(pos)
    for (e, a, start, n) in lora_seg:
        for b in range(start // BM, (start + n - 1) // BM + 1):
            lo, hi = max(start, b * BM), min(start + n, (b + 1) * BM)
            tiles.append((b, a, lo - b * BM, hi - lo))
    return dict(sorted_rows=sorted_rows, block_expert=block_expert, seg_start=seg,
                lora_seg=lora_seg, tiles=tiles)


@pytest.mark.parametrize("T,k,E,NA,BM", [
    (16, 4, 32, 8, 16), (37, 2, 5, 3, 4), (64, 2, 8, 16, 16), (30, 8, 16, 4, 32),
    (1, 1, 1, 1, 16), (12, 3, 4, 0, 8), (25, 2, 3, 2, 1), (0, 2, 4, 2, 16)])
def test_align_matches_bruteforce(oracle_lib, T, k, E, NA, BM):
    rng = np.random.default_rng(T + 100 * E + BM)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    aid = rng.integers(-1, max(NA, 1), size=T).astype(np.int32)
    if T > 3:
        ids[0, 0] = E  # out-of-range expert id: dropped
        aid[1] = NA + 3  # out-of-range adapter id: treated as none
    got = oracle_lib.ref_align(ids, aid, E, NA, BM)
    ref = brute_align(ids, aid, E, NA, BM)
    R = T * k
    n = got["num_padded"]
    assert got["seg_start"].tolist() == ref["seg_start"]
    assert got["sorted_rows"][:n].tolist() == ref["sorted_rows"]
    assert (got["sorted_rows"][n:] == R).all()
    nb = n // BM
    assert got["block_expert"][:nb].tolist() == ref["block_expert"]
    assert (got["block_expert"][nb:] == -1).all()
    assert got["n_lora_seg"] == len(ref["lora_seg"])
    assert [tuple(s) for s in got["lora_seg"][: got["n_lora_seg"]]] == ref["lora_seg"]
    assert (got["lora_seg"][got["n_lora_seg"]:] == [-1, -1, 0, 0]).all()
    assert got["n_tiles"] == len(ref["tiles"])
    assert [tuple(t) for t in got["tiles"][: got["n_tiles"]]] == ref["tiles"]
    tb = [t[0] for t in ref["tiles"]]
    for b, s in enumerate(got["block_tile_start"]):
        assert s == next((i for i, x in enumerate(tb) if x >= b), len(tb))
    # invariants: each valid row exactly once; padding holds only sentinels
    valid = [p for p in range(R) if 0 <= ids.flat[p] < E]
    assert sorted(p for p in got["sorted_rows"] if p < R) == valid
    assert sum(s[3] for s in ref["lora_seg"]) == sum(
        1 for p in valid if 0 <= aid[p // k] < NA)


# ---------------------------------------------------------------- the layer


def test_dense_ffn_is_textbook(oracle_lib):
    """E = 1, k = 1, no adapter: a SiLU-gated FFN (torch SiLU, float64)."""
    w, d = small_workload(T=5, H=24, I=20, E=1, k=1, NA=0, r=0)
    ids = np.zeros((5, 1), np.int32)
    out = run_oracle(oracle_lib, d, w, ids, np.ones((5, 1)), lora=False)
    x = torch.from_numpy(d["x"]).double()
    Wg, Wu = torch.from_numpy(d["W_gu"][0]).double().split(w.I)
    h = torch.nn.functional.silu(x @ Wg.T) * (x @ Wu.T)
    ref = h @ torch.from_numpy(d["W_d"][0]).double().T
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def dense_numpy(d, ids, wts, I, lora=True):
    """Every expert evaluated for every token (float64 matmuls), weighted by
    the token's routing weight for that expert or 0."""
    X = d["x"].astype(np.float64)
    T = X.shape[0]
    E = d["W_gu"].shape[0]
    route = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            route[t, ids[t, j]] += wts[t, j]
    out = np.zeros((T, d["W_d"].shape[1]))
    aid = d["adapter_ids"]
    NA = d["A_gu"].shape[0] if lora else 0
    for e in range(E):
        G = X @ d["W_gu"][e].astype(np.float64).T
        for a in range(NA):
            m = aid == a
            G[m] += (X[m] @ d["A_gu"][a, e].T.astype(np.float64)) @ d["B_gu"][a, e].T.astype(np.float64)
        Hh = torch.nn.functional.silu(torch.from_numpy(G[:, :I])).numpy() * G[:, I:]
        Y = Hh @ d["W_d"][e].astype(np.float64).T
        for a in range(NA):
            m = aid == a
            Y[m] += (Hh[m] @ d["A_d"][a, e].T.astype(np.float64)) @ d["B_d"][a, e].T.astype(np.float64)
        out += route[:, e:e + 1] * Y
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_grouped_equals_dense(oracle_lib, seed):
    w, d = small_workload(T=9, H=16, I=12, E=4, k=2, NA=3, r=4, seed=seed)
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    out = run_oracle(oracle_lib, d, w, ids, wts)
    np.testing.assert_allclose(out, dense_numpy(d, ids, wts, w.I), rtol=1e-11, atol=1e-12)


def test_b_zero_is_base_moe_bit_exact(oracle_lib):
    w, d = small_workload()
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    d0 = dict(d, B_gu=np.zeros_like(d["B_gu"]), B_d=np.zeros_like(d["B_d"]))
    assert np.array_equal(run_oracle(oracle_lib, d0, w, ids, wts),
                          run_oracle(oracle_lib, d, w, ids, wts, lora=False))


def test_single_adapter_equals_merged_weights(oracle_lib):
    """One adapter on every token equals the base layer with W' = W + AB
    (math layout), i.e. W_gu'[e] = W_gu[e] + B_gu[e] @ A_gu[e] in storage
    layout.  Dyadic values keep every merge exact in float32."""
    w, d = small_workload(T=5, H=8, I=6, E=3, k=2, NA=1, r=2, adapters="uniform")
    rng = np.random.default_rng(3)
    dy = lambda shape: (rng.integers(-4, 5, size=shape) / 8.0).astype(np.float32)
    for name in ("W_gu", "W_d", "A_gu", "B_gu", "A_d", "B_d"):
        d[name] = dy(d[name].shape)
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    lora = run_oracle(oracle_lib, d, w, ids, wts)
    merged = dict(d)
    merged["W_gu"] = (d["W_gu"] + np.einsum("enc,ech->enh", d["B_gu"][0], d["A_gu"][0])).astype(np.float32)
    merged["W_d"] = (d["W_d"] + np.einsum("emc,eci->emi", d["B_d"][0], d["A_d"][0])).astype(np.float32)
    assert np.array_equal(merged["W_gu"].astype(np.float64),
                          d["W_gu"] + np.einsum("enc,ech->enh", d["B_gu"][0].astype(np.float64),
                                                d["A_gu"][0].astype(np.float64)))
    base = run_oracle(oracle_lib, merged, w, ids, wts, lora=False)
    np.testing.assert_allclose(lora, base, rtol=1e-13, atol=1e-14)


def test_identical_experts_make_routing_irrelevant(oracle_lib):
    w, d = small_workload(E=4, k=3)
    for name in ("W_gu", "W_d"):
        d[name] = np.repeat(d[name][:1], w.E, axis=0)
    for name in ("A_gu", "B_gu", "A_d", "B_d"):
        d[name] = np.repeat(d[name][:, :1], w.E, axis=1)
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    out = run_oracle(oracle_lib, d, w, ids, wts)
    one = run_oracle(oracle_lib, d, w, np.zeros((w.T, 1), np.int32), np.ones((w.T, 1)))
    np.testing.assert_allclose(out, one, rtol=1e-13, atol=1e-14)


def test_output_is_affine_in_b_down(oracle_lib):
    w, d = small_workload()
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    o = lambda s: run_oracle(oracle_lib, dict(d, B_d=(s * d["B_d"]).astype(np.float32)), w, ids, wts)
    o0, o1, o2 = o(0.0), o(1.0), o(2.0)
    np.testing.assert_allclose(o2 - o1, o1 - o0, rtol=1e-11, atol=1e-12)


def test_adapter_slot_permutation_bit_exact(oracle_lib):
    w, d = small_workload(NA=3)
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    perm = np.array([2, 0, 1])  # new slot of old adapter a is perm[a]
    dp = dict(d)
    for name in ("A_gu", "B_gu", "A_d", "B_d"):
        dp[name] = np.empty_like(d[name])
        dp[name][perm] = d[name]
    aid = d["adapter_ids"]
    dp["adapter_ids"] = np.where(aid >= 0, perm[np.maximum(aid, 0)], -1).astype(np.int32)
    assert np.array_equal(run_oracle(oracle_lib, d, w, ids, wts),
                          run_oracle(oracle_lib, dp, w, ids, wts))


def test_token_subset_and_no_adapter_rows(oracle_lib):
    w, d = small_workload(T=7)
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    full = run_oracle(oracle_lib, d, w, ids, wts)
    sub = run_oracle(oracle_lib, d, w, ids, wts, tokens=np.array([5, 0, 3], np.int32))
    assert np.array_equal(sub, full[[5, 0, 3]])
    base = run_oracle(oracle_lib, d, w, ids, wts, lora=False)
    none = d["adapter_ids"] < 0
    assert np.array_equal(full[none], base[none])


def test_bf16_inputs_widen_exactly(oracle_lib):
    """bf16 storage is read as the exact float value of its bits."""
    w, d = small_workload(T=4, H=8, I=4, E=2, k=1, NA=1, r=2)
    db = {n: (synth.f32_to_bf16_bits(v) if isinstance(v, np.ndarray) and v.dtype == np.float32
              and n != "logits" else v) for n, v in d.items()}
    df = {n: (synth.bf16_bits_to_f32(v) if n in db and isinstance(v, np.ndarray) and v.dtype == np.uint16
              else v) for n, v in db.items()}
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    a = oracle_lib.ref_forward(db["x"], ids, wts, d["adapter_ids"], db["W_gu"], db["W_d"], db["A_gu"],
                               db["B_gu"], db["A_d"], db["B_d"], inter=w.I, rank=w.r, n_adapters=w.NA,
                               dtype=oracle_lib.BF16)
    b = run_oracle(oracle_lib, df, w, ids, wts)
    assert np.array_equal(a, b)


def test_thread_count_does_not_change_results():
    """Tokens are independent and each is computed by one thread in the
    written order, so one thread and all threads agree bit for bit."""
    import oracle
    w, d = small_workload(T=23, H=24, I=20, E=5, k=3, NA=3, r=4)
    ids, wts = oracle.ref_route(d["logits"], w.k)
    try:
        oracle.set_threads(1)
        one = run_oracle(oracle, d, w, ids, wts)
        assert oracle.set_threads(0) >= 1
        many = run_oracle(oracle, d, w, ids, wts)
    finally:
        oracle.set_threads(0)
    assert np.array_equal(one, many)


# ------------------------------------------------ fp8 (E4M3) base weights


def _torch_e4m3(codes):
    """float64 values of E4M3 codes by torch's float8_e4m3fn (a library
    implementation of the same OCP format)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_fp8_e4m3_codes_match_the_format(oracle_lib):
    """All 256 codes against torch's float8_e4m3fn, and points of the OCP
    E4M3 definition worked out by hand (bias 7, 3 mantissa bits, subnormals
    at exponent 0, S.1111.111 = NaN, no infinities)."""
    ours = np.array([oracle_lib.fp8_e4m3(c) for c in range(256)])
    lib = _torch_e4m3(np.arange(256))
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], lib[~nan])
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2 ** -6,
            0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xBC: -1.5, 0xFE: -448.0}
    for c, v in hand.items():
        assert oracle_lib.fp8_e4m3(c) == v, hex(c)
    assert np.signbit(oracle_lib.fp8_e4m3(0x80)) and oracle_lib.fp8_e4m3(0x80) == 0.0


def fp8_workload(T=7, H=16, I=12, E=3, k=2, NA=2, r=4, seed=9, pow2=False):
    """A small layer with E4M3 base weights (codes over every finite value)
    and one scale per weight row; x and the adapters in bf16."""
    w, d = small_workload(T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, seed=seed)
    rng = np.random.default_rng(seed)
    out = {n: (synth.f32_to_bf16_bits(v) if n in ("x", "A_gu", "B_gu", "A_d", "B_d") else v)
           for n, v in d.items()}
    for n, rows in (("W_gu", 2 * I), ("W_d", H)):
        codes = rng.integers(0, 256, size=d[n].shape).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x3F        # no NaN codes
        scale = (2.0 ** rng.integers(-4, 4, size=(E, rows)) if pow2
                 else rng.uniform(0.01, 0.1, size=(E, rows))).astype(np.float32)
        out[n], out[n + "_scale"] = codes, scale
    return w, out


def run_fp8(o, d, w, ids, wts, **kw):
    return o.ref_forward(d["x"], ids, wts, d["adapter_ids"], d["W_gu"], d["W_d"], d["A_gu"],
                         d["B_gu"], d["A_d"], d["B_d"], inter=w.I, rank=w.r, n_adapters=w.NA,
                         dtype=o.BF16_FP8W, W_gu_scale=d["W_gu_scale"],
                         W_d_scale=d["W_d_scale"], **kw)


def test_fp8_weights_equal_bf16_dequantised_weights(oracle_lib):
    """With power-of-two scales every dequantised weight (a 4-bit significand
    times a power of two) is a bf16 value, so the fp8 layer must equal, bit
    for bit, the bf16 layer on those weights (dequantised here with torch)."""
    w, d = fp8_workload(pow2=True)
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    deq = dict(d)
    for n in ("W_gu", "W_d"):
        v = _torch_e4m3(d[n]) * d[n + "_scale"][..., None].astype(np.float64)
        b = synth.f32_to_bf16_bits(v.astype(np.float32))
        assert np.array_equal(synth.bf16_bits_to_f32(b).astype(np.float64), v)
        deq[n] = b
    bf = oracle_lib.ref_forward(deq["x"], ids, wts, d["adapter_ids"], deq["W_gu"], deq["W_d"],
                                d["A_gu"], d["B_gu"], d["A_d"], d["B_d"], inter=w.I, rank=w.r,
                                n_adapters=w.NA, dtype=oracle_lib.BF16)
    assert np.array_equal(run_fp8(oracle_lib, d, w, ids, wts), bf)


def test_fp8_weights_against_dense_float64(oracle_lib):
    """Arbitrary per-row scales: the fp8 layer against every expert evaluated
    densely in float64 on weights dequantised with torch (scale x value)."""
    w, d = fp8_workload(seed=4)
    ids, wts = oracle_lib.ref_route(d["logits"], w.k)
    dd = {n: (synth.bf16_bits_to_f32(v) if n in ("x", "A_gu", "B_gu", "A_d", "B_d") else v)
          for n, v in d.items()}
    for n in ("W_gu", "W_d"):
        dd[n] = _torch_e4m3(d[n]) * d[n + "_scale"][..., None].astype(np.float64)
    np.testing.assert_allclose(run_fp8(oracle_lib, d, w, ids, wts),
                               dense_numpy(dd, ids, wts, w.I), rtol=1e-11, atol=1e-12)
