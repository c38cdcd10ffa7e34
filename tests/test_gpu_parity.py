"""GPU parity of the fused MoE-LoRA layer against the CPU oracle.

Every call goes through the C ABI (lora_expert_gemm_amd -> libmoelora.so).
Routing ids and the alignment must match the oracle bit for bit; routing
weights to a few float32 ulps; the layer output to the layer's tolerance
(max|err| <= 2e-2 max|ref|, relative Frobenius <= 5e-3 for bf16 and 1e-5
for float32).  The named workloads run at full size: every output row is checked
for being written and finite, and compared with the oracle on every token
(the 6400-token prefill: on tokens covering every block, LoRA run and
expert); the small shapes compare every token and span several blocks,
several 64-column tiles and ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from layer_harness import Run, check_alignment, check_close, oracle_out

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


SMALL = [
    # T, H, I, E, k, NA, r, dtype, adapters
    (37, 136, 200, 6, 3, 5, 16, "bf16", "uniform_with_none"),   # ragged K tail, H % 64 != 0
    (64, 256, 192, 4, 2, 3, 32, "bf16", "uniform_with_none"),   # 64-row blocks
    (200, 512, 320, 8, 2, 4, 64, "bf16", "uniform_with_none"),  # several 64-row blocks
    (9, 96, 80, 3, 2, 2, 8, "f32", "uniform_with_none"),
    (70, 160, 144, 4, 2, 3, 16, "f32", "uniform_with_none"),    # float, 64-row blocks
    (5, 100, 200, 4, 2, 2, 16, "bf16", "uniform_with_none"),    # unaligned rows (K = 100)
    (5, 100, 200, 4, 2, 2, 16, "f32", "uniform_with_none"),
    (16, 128, 128, 8, 4, 1, 8, "bf16", "uniform"),              # one adapter
    (16, 128, 128, 8, 4, 2, 64, "bf16", "none"),                # adapters loaded, none used
    (1, 64, 64, 4, 2, 2, 16, "bf16", "uniform"),                # one token
    (20, 64, 96, 300, 3, 0, 0, "bf16", "none"),                 # E > 256, no adapters
    (120, 64, 96, 300, 3, 2, 16, "bf16", "uniform_with_none"),  # E > 256, large-batch path
    (90, 128, 64, 100, 4, 3, 16, "bf16", "uniform_with_none"),  # 64 < E <= 128
    (300, 256, 320, 4, 2, 3, 16, "bf16", "uniform_with_none"),  # LDS-tiled, partial column tile
    (260, 200, 136, 4, 2, 2, 32, "bf16", "uniform_with_none"),  # LDS-tiled, K % 64 != 0
    (512, 128, 128, 2, 1, 0, 0, "bf16", "none"),                # LDS-tiled, no adapters
    (300, 256, 192, 4, 2, 3, 32, "bf16", "uniform_with_none"),  # 8-wave tiled, LoRA slabs (2r = 64)
    (400, 128, 256, 2, 2, 5, 64, "bf16", "uniform_with_none"),  # 8-wave tiled, several LoRA tiles per block
    (30, 128, 96, 8, 2, 3, 16, "bf16", "uniform_with_none"),    # 32-row blocks, row-wise LoRA
    (200, 128, 96, 64, 2, 3, 16, "bf16", "uniform_with_none"),  # 32-row blocks, tile-wise LoRA
    (60, 256, 128, 8, 2, 4, 16, "bf16", "uniform_with_none"),   # 64-row blocks, row-wise LoRA
    (40, 136, 96, 8, 2, 3, 16, "bf16", "uniform_with_none"),    # 32-row blocks, H % 32 != 0 (down tiles clamped)
    (8, 64, 96, 1024, 32, 7, 256, "bf16", "uniform_with_none"), # maximum E, top-k and rank (row mode)
    (64, 64, 64, 32, 2, 255, 8, "bf16", "uniform_with_none"),   # maximum adapters: 8192 alignment buckets
    (300, 64, 64, 64, 2, 3, 256, "bf16", "uniform_with_none"),  # rank 256 in tile mode (split shrink)
    (100, 64, 64, 64, 2, 8, 16, "bf16", "uniform_with_none"),   # 576 buckets: one-wave alignment plan, 9 per lane
    (100, 64, 64, 64, 2, 9, 16, "bf16", "uniform_with_none"),   # 640 buckets: block-wide alignment plan
    (40, 64, 64, 65, 2, 2, 16, "bf16", "uniform_with_none"),    # 65 experts: block-wide plan in the small kernel
    (24, 256, 384, 1, 1, 3, 16, "bf16", "uniform_with_none"),   # dense: one expert, top-1, row-wise LoRA
    (300, 256, 384, 1, 1, 3, 16, "bf16", "uniform_with_none"),  # dense, LDS-tiled 128-row blocks
    (20, 96, 160, 1, 1, 2, 8, "f32", "uniform_with_none"),      # dense, float
    (150, 96, 80, 16, 2, 3, 16, "f32", "uniform_with_none"),    # float, tile-wise LoRA (shrink kernel)
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r,dt,ad", SMALL)
def test_small_shapes(T, H, I, E, k, NA, r, dt, ad):
    w = synth.Workload("small", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype=dt, adapters=ad,
                       seed=T * 7 + H)
    say(f"[parity] small {w}")
    d = synth.make_inputs(w)
    run = Run(w, d).forward()
    say(f"[parity] plan {run.plan.info(T)}")
    rid, rw = oracle.ref_route(d["logits"], k)
    ids, wts = run.routing()
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(wts, rw, rtol=1e-6, atol=1e-7)
    check_alignment(run.alignment(), oracle.ref_align(rid, d["adapter_ids"], E, NA,
                                                      run.alignment()["block_m"]))
    mr, fr = check_close(run.out_f32(), oracle_out(w, d, rid, rw), dt, "small")
    say(f"[parity] max_rel={mr:.3e} fro_rel={fr:.3e}")


@pytest.mark.parametrize("T", [40, 150])  # small and large alignment paths
def test_caller_ids_one_expert_and_duplicates(T):
    """Caller-supplied routing: every token on expert 0 (many blocks of one
    expert, all other experts empty), plus duplicate ids within a token."""
    w = synth.Workload("ids", T=T, H=128, I=96, E=5, k=2, NA=3, r=16, dtype="bf16",
                       adapters="uniform_with_none", seed=5)
    d = synth.make_inputs(w)
    ids = np.zeros((w.T, w.k), np.int32)
    ids[::3, 1] = 3
    wts = np.full((w.T, w.k), 0.5, np.float32)
    wts[::2] = [0.7, 0.3]
    run = Run(w, d, route="ids", ids=ids, wts=wts).forward()
    check_alignment(run.alignment(), oracle.ref_align(ids, d["adapter_ids"], w.E, w.NA,
                                                      run.alignment()["block_m"]))
    check_close(run.out_f32(), oracle_out(w, d, ids, wts.astype(np.float64)), "bf16", "ids")


def test_long_lora_segment_shrinks_in_chunks():
    """Tile-mode gate_up shrink riding along with the alignment scatter: one
    (expert, adapter) segment of 600 rows (more than the scatter's 512-row
    chunk), every other row spread over the remaining experts."""
    w = synth.Workload("segment", T=600, H=128, I=96, E=64, k=2, NA=1, r=16, dtype="bf16",
                       adapters="uniform", seed=11)
    d = synth.make_inputs(w)
    ids = np.zeros((w.T, w.k), np.int32)
    ids[:, 1] = 1 + np.arange(w.T) % (w.E - 1)
    wts = np.full((w.T, w.k), 0.5, np.float32)
    run = Run(w, d, route="ids", ids=ids, wts=wts).forward()
    info = run.plan.info(w.T)
    say(f"[parity] long segment: plan {info}")
    assert "lora_mode=tile" in info and "shrink_gu=scatter" in info
    check_alignment(run.alignment(), oracle.ref_align(ids, d["adapter_ids"], w.E, w.NA,
                                                      run.alignment()["block_m"]))
    check_close(run.out_f32(), oracle_out(w, d, ids, wts.astype(np.float64)), "bf16", "segment")


def test_all_base_rows_equal_no_lora_bit_exact():
    """Adapter id -1 everywhere with LoRA weights given equals the call with
    no LoRA pointers, bit for bit (the LoRA work adds exactly nothing)."""
    w = synth.Workload("base", T=24, H=256, I=192, E=6, k=2, NA=4, r=32, dtype="bf16",
                       adapters="none", seed=11)
    d = synth.make_inputs(w)
    a = Run(w, d).forward().out_f32()
    b = Run(w, d, lora=False).forward().out_f32()
    c = Run(w, d, adapter_ids="null").forward().out_f32()
    assert np.array_equal(a, b) and np.array_equal(a, c)
    rid, rw = oracle.ref_route(d["logits"], w.k)
    check_close(b, oracle_out(w, d, rid, rw, lora=False), "bf16", "base")


def test_zero_tokens_leaves_output_untouched():
    w = synth.Workload("zero", T=4, H=64, I=64, E=4, k=2, NA=2, r=16, dtype="bf16",
                       adapters="uniform", seed=3)
    run = Run(w, synth.make_inputs(w)).forward(T=0)
    o = run.out.cpu().numpy()
    assert (o == -1).all()


def test_fewer_tokens_than_planned():
    """A plan for 64 tokens serving 24: only the first 24 rows are written."""
    w = synth.Workload("partial", T=64, H=128, I=128, E=8, k=2, NA=4, r=16, dtype="bf16",
                       adapters="uniform_with_none", seed=21)
    d = synth.make_inputs(w)
    run = Run(w, d).forward(T=24)
    out = run.out_f32()
    assert (run.out[24:].cpu().numpy() == -1).all()
    d24 = dict(d, x=d["x"][:24], logits=d["logits"][:24], adapter_ids=d["adapter_ids"][:24])
    w24 = synth.Workload("partial", T=24, H=128, I=128, E=8, k=2, NA=4, r=16, dtype="bf16",
                         adapters="uniform_with_none", seed=21)
    rid, rw = oracle.ref_route(d24["logits"], 2)
    check_close(out[:24], oracle_out(w24, d24, rid, rw), "bf16", "partial")


def test_repeat_calls_are_bitwise_identical():
    w = synth.workload("decode_bf16")
    d = synth.make_inputs(w)
    run = Run(w, d)
    outs, als = [], []
    for _ in range(3):
        run.forward()
        outs.append(run.out_f32())
        als.append(run.alignment())
    for o, a in zip(outs[1:], als[1:]):
        assert np.array_equal(o, outs[0])
        check_alignment(a, als[0])


GRAPH = [
    # T, H, I, E, k, NA, r: 16-row blocks (row-wise LoRA, ring stream), 32-row
    # blocks (tile-wise LoRA with split shrinks), LDS-tiled 128-row blocks
    (16, 256, 192, 16, 4, 4, 32),
    (200, 128, 192, 64, 2, 3, 16),
    (300, 256, 192, 4, 2, 3, 32),
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r", GRAPH)
def test_graph_replay_matches_eager(T, H, I, E, k, NA, r):
    """One layer call captured in a HIP graph (the forward only launches
    kernels on the given stream: no allocation, copy, memset or sync) and
    replayed three times, with other work on the device between replays:
    every replay reproduces the eager output bit for bit."""
    w = synth.Workload("graph", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T + 5 * E)
    d = synth.make_inputs(w)
    run = Run(w, d).forward()
    torch.cuda.synchronize()
    eager = run.out.clone()
    say(f"[parity] graph capture {w}: plan {run.plan.info(T)}")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap):
        run.forward(stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    for i in range(3):
        run.out.fill_(-1)
        run.ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.out, eager), f"replay {i} differs from the eager call"


def test_stage_timing_hook():
    L = __import__("lora_expert_gemm_amd")
    w = synth.Workload("timing", T=16, H=256, I=256, E=8, k=2, NA=2, r=16, dtype="bf16",
                       adapters="uniform", seed=2)
    run = Run(w, synth.make_inputs(w))
    L.moelora_timing_begin(run.plan.handle, 4)
    for _ in range(3):
        run.forward()
    ms, n = L.moelora_timing_end(run.plan.handle)
    assert n == 3 and all(m >= 0 for m in ms) and ms[2] > 0 and ms[4] > 0


# Streaming-block shapes whose contractions are multiples of 64, so the weight
# stream can run through the LDS ring: 16-row blocks (row-wise LoRA), 32-row
# blocks (row-wise, and tile-wise with two-tile down waves) and 64-row blocks.
RING = [
    (8, 256, 192, 8, 2, 3, 16),    # 16-row blocks
    (30, 128, 128, 8, 2, 3, 32),   # 32-row blocks, row-wise LoRA
    (200, 128, 192, 64, 2, 3, 16), # 32-row blocks, tile-wise LoRA
    (100, 192, 128, 4, 2, 2, 16),  # 64-row blocks
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r", RING)
def test_weight_stream_paths_agree(T, H, I, E, k, NA, r, monkeypatch):
    """The LDS-ring weight stream (2, 3 or 4 slots) and the register path
    feed the MFMAs the same contraction indices in the same order, so the
    four outputs are bitwise identical; each is also checked against the
    oracle.  Two slots read each slab right after the wait that lands it, so
    they test the wait counts with no slack."""
    w = synth.Workload("ring", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T * 11 + I)
    d = synth.make_inputs(w)
    rid, rw = oracle.ref_route(d["logits"], k)
    ref = oracle_out(w, d, rid, rw)
    outs = {}
    for slots in ("0", "2", "3", "4"):
        monkeypatch.setenv("MOELORA_SLOTS", slots)
        run = Run(w, d).forward()
        say(f"[parity] ring slots={slots} {w}: plan {run.plan.info(T)}")
        outs[slots] = run.out.cpu().numpy().copy()
        check_close(run.out_f32(), ref, "bf16", f"slots {slots}")
    for slots in ("2", "3", "4"):
        assert np.array_equal(outs["0"], outs[slots]), f"{slots} slots differ from registers"


# Weight rows that are a multiple of 4 KB: the LDS-ring walks start at a
# slab that depends on the workgroup (gate_up rows of 2048 bf16, then down
# rows of 2048 bf16 with 32-row blocks).
ROT = [
    (8, 2048, 256, 4, 2, 2, 16),
    (40, 256, 2048, 8, 2, 3, 16),
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r", ROT)
def test_staggered_walks(T, H, I, E, k, NA, r, monkeypatch):
    """Staggered and aligned slab walks each meet the oracle's tolerance and
    agree with each other to within it (the contraction is summed in another
    order); 3 and 4 ring slots walk the same order, so they agree bit for bit."""
    w = synth.Workload("rot", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T * 13 + H)
    d = synth.make_inputs(w)
    rid, rw = oracle.ref_route(d["logits"], k)
    ref = oracle_out(w, d, rid, rw)
    outs = {}
    for rot in ("1", "0"):
        monkeypatch.setenv("MOELORA_ROTATE", rot)
        for slots in ("3", "4"):
            monkeypatch.setenv("MOELORA_SLOTS", slots)
            run = Run(w, d).forward()
            say(f"[parity] rotate={rot} slots={slots} {w}: plan {run.plan.info(T)}")
            outs[rot, slots] = run.out.cpu().numpy().copy()
            check_close(run.out_f32(), ref, "bf16", f"rotate {rot} slots {slots}")
        assert np.array_equal(outs[rot, "3"], outs[rot, "4"])
    f32 = lambda o: synth.bf16_bits_to_f32(o.view(np.uint16))
    check_close(f32(outs["1", "3"]), f32(outs["0", "3"]), "bf16", "staggered vs aligned")


# Down GEMM with its contraction split over workgroups (partial y per split,
# added in split order by the combine): row-wise LoRA (small batch, expand in
# the combine), tile-wise LoRA (64-row blocks, expand in split 0 only) and a
# dense layer (one expert, top-1).
KSPLIT = [
    (24, 256, 256, 4, 2, 3, 16),    # 32-row blocks, row-wise LoRA
    (160, 128, 256, 8, 2, 3, 16),   # 64-row blocks, tile-wise LoRA
    (40, 128, 512, 1, 1, 3, 16),    # dense
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r", KSPLIT)
def test_down_contraction_splits(T, H, I, E, k, NA, r, monkeypatch):
    """1, 2 and 4 contraction splits of the down GEMM each meet the oracle's
    tolerance and agree with each other to within it (the split sums round
    differently, so not bit for bit)."""
    w = synth.Workload("ksplit", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T * 7 + I)
    d = synth.make_inputs(w)
    rid, rw = oracle.ref_route(d["logits"], k)
    ref = oracle_out(w, d, rid, rw)
    outs = {}
    for ks in ("1", "2", "4"):
        monkeypatch.setenv("MOELORA_KSPLIT_D", ks)
        run = Run(w, d).forward()
        info = run.plan.info(T)
        say(f"[parity] down ksplit={ks} {w}: plan {info}")
        assert f"down_ksplit={ks}" in info
        outs[ks] = run.out_f32()
        check_close(outs[ks], ref, "bf16", f"ksplit {ks}")
    check_close(outs["2"], outs["1"], "bf16", "ksplit 2 vs 1")
    check_close(outs["4"], outs["1"], "bf16", "ksplit 4 vs 1")


# Shrink workgroups of 4, 8 and 16 waves (tile-mode LoRA): one tile's
# contraction is cut into 16 / (row groups x token groups) parts per
# workgroup, which meet in LDS; few waves leave one part per pair.
SHRINK_WAVES = [
    (200, 128, 256, 16, 2, 3, 16),  # 32-row blocks, r = 16
    (160, 128, 256, 8, 2, 3, 16),   # 64-row blocks, r = 16
    (300, 256, 192, 32, 4, 5, 40),  # 64-row blocks, r = 40: three 16-row groups of A
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r", SHRINK_WAVES)
def test_shrink_workgroup_sizes(T, H, I, E, k, NA, r, monkeypatch):
    """4-, 8- and 16-wave shrink workgroups each meet the oracle's tolerance."""
    w = synth.Workload("shrink_waves", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T * 5 + r)
    d = synth.make_inputs(w)
    rid, rw = oracle.ref_route(d["logits"], k)
    ref = oracle_out(w, d, rid, rw)
    for nw in ("4", "8", "16"):
        monkeypatch.setenv("MOELORA_SHRINK_WAVES", nw)
        run = Run(w, d).forward()
        info = run.plan.info(T)
        say(f"[parity] shrink waves={nw} {w}: plan {info}")
        assert "lora_mode=tile" in info and f"shrink_waves={nw}" in info
        check_close(run.out_f32(), ref, "bf16", f"shrink waves {nw}")


# Tokens shared by the four waves of a workgroup through an LDS ring, against
# tokens loaded by each wave: same MFMAs in the same slab order on the same
# token rows, so at equal waves (4) and one contraction split the outputs
# are identical bit for bit.  16-, 32- and 64-row blocks, row-wise and
# tile-wise LoRA, a dense layer, ragged last column tiles (gate_up: I = 200,
# where the down contraction cannot use the ring; down: H = 320).
TOKSHARE = [
    (16, 256, 320, 8, 2, 3, 16),    # 16-row blocks, row-wise LoRA
    (24, 256, 200, 4, 2, 3, 16),    # 32-row blocks, row-wise LoRA, ragged gate_up columns
    (24, 320, 256, 4, 2, 3, 16),    # 32-row blocks, ragged down columns
    (200, 128, 256, 16, 2, 3, 16),  # 32-row blocks, tile-wise LoRA
    (160, 128, 256, 8, 2, 3, 16),   # 64-row blocks, tile-wise LoRA
    (40, 128, 512, 1, 1, 3, 16),    # dense
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r", TOKSHARE)
def test_shared_token_ring(T, H, I, E, k, NA, r, monkeypatch):
    """Shared-token and per-wave-token streaming GEMMs agree bit for bit and
    meet the oracle's tolerance."""
    w = synth.Workload("tokshare", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T * 3 + I)
    d = synth.make_inputs(w)
    rid, rw = oracle.ref_route(d["logits"], k)
    ref = oracle_out(w, d, rid, rw)
    monkeypatch.setenv("MOELORA_WAVES_GU", "4")
    monkeypatch.setenv("MOELORA_WAVES_D", "4")
    monkeypatch.setenv("MOELORA_KSPLIT_D", "1")
    outs = {}
    for sh in ("1", "0"):
        monkeypatch.setenv("MOELORA_TOKSHARE", sh)
        run = Run(w, d).forward()
        info = run.plan.info(T)
        say(f"[parity] tokshare={sh} {w}: plan {info}")
        share_d = sh if I % 64 == 0 else "0"
        assert f"tok_share_gu={sh}" in info and f"tok_share_d={share_d}" in info
        outs[sh] = run.out.cpu().numpy().copy()
        check_close(run.out_f32(), ref, "bf16", f"tokshare {sh}")
    assert np.array_equal(outs["1"], outs["0"])
    # the shared ring with two slots: each slab read right after the wait
    # and barrier that land it
    monkeypatch.setenv("MOELORA_TOKSHARE", "1")
    monkeypatch.setenv("MOELORA_SLOTS", "2")
    run = Run(w, d).forward()
    say(f"[parity] tokshare=1 slots=2 {w}: plan {run.plan.info(T)}")
    assert np.array_equal(run.out.cpu().numpy(), outs["1"])


def coverage_tokens(w, ref_al):
    """Tokens that put at least one routed row in every block of the
    alignment, in every (expert, adapter) LoRA run and at the end of every
    expert's rows (its base-only rows, if any), plus the first and last two."""
    rows, R = ref_al["sorted_rows"], w.T * w.k
    BM = len(rows) // max(1, len(ref_al["block_expert"]))
    pick = {0, 1, w.T - 2, w.T - 1}
    for b in range(len(ref_al["block_expert"])):
        blk = rows[b * BM:(b + 1) * BM]
        if len(blk) and blk[0] < R:
            pick.add(int(blk[0]) // w.k)
    for e, a, start, n in ref_al["lora_seg"][:ref_al["n_lora_seg"]]:
        pick.add(int(rows[start]) // w.k)
    seg = ref_al["seg_start"]
    for e in range(w.E):
        real = [p for p in rows[seg[e]:seg[e + 1]] if p < R]
        if real:
            pick.add(int(real[-1]) // w.k)
    return np.array(sorted(t for t in pick if 0 <= t < w.T), np.int32)


# Workloads whose oracle run over every token stays within seconds on the
# test host's cores; the 6400-token prefill compares the coverage sample.
FULL = {"tiny_fp32", "decode_bf16", "illustrative_bf16", "many_expert_bf16", "dense_bf16",
        "decode_fp8w", "illustrative_fp8w", "many_expert_fp8w"}


@pytest.mark.parametrize("name", [w.name for w in synth.WORKLOADS])
def test_named_workload(name):
    """Full-size workloads: routing ids and the alignment bit for bit, routing
    weights to 1e-6; every output row written and finite; the output against
    the oracle on every token (prefill: tokens covering every 128-row block,
    every (expert, adapter) run and every expert)."""
    w = synth.workload(name)
    say(f"[parity] workload {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} NA={w.NA} r={w.r}")
    d = synth.make_inputs(w)
    run = Run(w, d).forward()
    say(f"[parity] {name}: plan {run.plan.info(w.T)}")
    ids, wts = run.routing()
    rid, rw = oracle.ref_route(d["logits"], w.k)
    assert np.array_equal(ids, rid), "router ids differ from the oracle"
    np.testing.assert_allclose(wts, rw, rtol=1e-6, atol=1e-7)
    ref_al = oracle.ref_align(rid, d["adapter_ids"], w.E, w.NA, run.alignment()["block_m"])
    check_alignment(run.alignment(), ref_al)
    raw = run.out.cpu().numpy()
    unwritten = (raw == -1).all(axis=1)   # out was filled with -1 (a bf16 NaN pattern)
    assert not unwritten.any(), f"rows never written: {np.flatnonzero(unwritten)[:8]}"
    full = run.out_f32()
    assert np.isfinite(full).all(), "non-finite output"
    tok = np.arange(w.T, dtype=np.int32) if name in FULL else coverage_tokens(w, ref_al)
    ref = oracle_out(w, d, rid, rw, tokens=tok)
    mr, fr = check_close(full[tok], ref, w.dtype, name)
    say(f"[parity] {name}: max_rel={mr:.3e} fro_rel={fr:.3e} tokens={len(tok)} of {w.T}")
    assert run.device_error() == 0


# E4M3 base weights with row scales: contractions that are multiples of 128
# and odd multiples of 64 (a 64-wide tail slab), 16-, 32- and 64-row
# streaming blocks, row- and tile-wise LoRA, two-tile down waves, 4 KB
# weight rows (staggered walks), one expert, no adapters.
FP8 = [
    # T, H, I, E, k, NA, r, adapters
    (16, 256, 192, 8, 2, 3, 16, "uniform_with_none"),    # 16-row blocks, row LoRA, H % 128 == 0, I tail
    (37, 192, 320, 6, 3, 5, 16, "uniform_with_none"),    # both tails, 16/32-row
    (30, 128, 128, 8, 2, 3, 32, "uniform_with_none"),    # 32-row blocks, row-wise LoRA
    (200, 128, 192, 64, 2, 3, 16, "uniform_with_none"),  # 32-row blocks, tile-wise LoRA
    (300, 256, 320, 4, 2, 3, 16, "uniform_with_none"),   # 64-row blocks (no LDS-tiled path for E4M3)
    (24, 4096, 256, 4, 2, 2, 16, "uniform_with_none"),   # 4 KB gate_up rows: staggered walks
    (24, 256, 384, 1, 1, 3, 16, "uniform_with_none"),    # dense: one expert, top-1
    (20, 192, 128, 8, 2, 0, 0, "none"),                  # no adapters
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r,ad", FP8)
def test_fp8_weights(T, H, I, E, k, NA, r, ad):
    w = synth.Workload("fp8", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16", adapters=ad,
                       seed=T * 5 + H + I, wdtype="fp8")
    say(f"[parity] fp8 {w}")
    d = synth.make_inputs(w)
    run = Run(w, d).forward()
    say(f"[parity] plan {run.plan.info(T)}")
    assert run.plan.info(T).startswith("dtype=bf16_fp8w")
    rid, rw = oracle.ref_route(d["logits"], k)
    ids, _ = run.routing()
    assert np.array_equal(ids, rid)
    mr, fr = check_close(run.out_f32(), oracle_out(w, d, rid, rw), "bf16", "fp8")
    say(f"[parity] max_rel={mr:.3e} fro_rel={fr:.3e}")


GROUPED = [  # LDS-tiled shapes: (T, H, I, E, k, NA, r)
    (300, 256, 320, 4, 2, 3, 16),   # 4-wave tiled, partial column tile
    (400, 128, 256, 2, 2, 5, 64),   # 8-wave tiled, LoRA slabs
    (1200, 256, 1600, 8, 2, 3, 32), # 8-wave tiled, 7 column tiles in groups of 3 (+1)
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r", GROUPED)
def test_grouped_item_order(T, H, I, E, k, NA, r, monkeypatch):
    """The LDS-tiled GEMMs give the same bits whatever order the workgroups
    take the (block, column tile) items in: none, groups of 2, 3 or 4
    column tiles, or expert-major."""
    w = synth.Workload("grouped", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T + I)
    d = synth.make_inputs(w)
    outs = {}
    for g in ("0", "2", "3", "4", "-1"):
        monkeypatch.setenv("MOELORA_GROUP", g)
        run = Run(w, d).forward()
        assert "tg=8" in run.plan.info(T), run.plan.info(T)
        outs[g] = run.out.cpu().numpy().copy()
    rid, rw = oracle.ref_route(d["logits"], k)
    check_close(Run(w, d).forward().out_f32(), oracle_out(w, d, rid, rw), "bf16", "grouped order")
    for g, o in outs.items():
        assert np.array_equal(o, outs["0"]), f"group {g} differs from the plain order"


FP8_PATHS = [
    (16, 256, 320, 8, 2, 3, 16),    # 16-row blocks, tail in the down contraction
    (24, 192, 256, 4, 2, 3, 16),    # 32-row blocks, tail in gate_up
    (200, 128, 256, 16, 2, 3, 16),  # 32-row blocks, tile-wise LoRA
    (160, 128, 192, 8, 2, 3, 16),   # 64-row blocks
]


@pytest.mark.parametrize("T,H,I,E,k,NA,r", FP8_PATHS)
def test_fp8_stream_forms_agree(T, H, I, E, k, NA, r, monkeypatch):
    """The E4M3 stream with tokens shared through LDS or loaded per wave, and
    with 3 or 4 ring slots, feeds the MFMAs the same operands in the same
    order: bit-identical outputs, each within the oracle's tolerance."""
    w = synth.Workload("fp8paths", T=T, H=H, I=I, E=E, k=k, NA=NA, r=r, dtype="bf16",
                       adapters="uniform_with_none", seed=T * 3 + I, wdtype="fp8")
    d = synth.make_inputs(w)
    rid, rw = oracle.ref_route(d["logits"], k)
    ref = oracle_out(w, d, rid, rw)
    monkeypatch.setenv("MOELORA_WAVES_GU", "4")
    monkeypatch.setenv("MOELORA_WAVES_D", "4")
    outs = {}
    for sh in ("1", "0"):
        for slots in ("3", "4"):
            monkeypatch.setenv("MOELORA_TOKSHARE", sh)
            monkeypatch.setenv("MOELORA_SLOTS", slots)
            run = Run(w, d).forward()
            say(f"[parity] fp8 tokshare={sh} slots={slots} {w}: plan {run.plan.info(T)}")
            outs[sh, slots] = run.out.cpu().numpy().copy()
            check_close(run.out_f32(), ref, "bf16", f"fp8 tokshare {sh} slots {slots}")
    for key, o in outs.items():
        assert np.array_equal(o, outs["1", "3"]), f"{key} differs from shared tokens, 3 slots"
