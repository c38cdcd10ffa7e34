"""Host-side logic of bench.py (no GPU): the algorithmic bytes and FLOPs the
roofline divides by, the kernel-code hash that decides whether committed
counters still apply, the stage-keyed counter lookup, and the one-GPU
contract of the command line."""
import json
import os
import shutil
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_algorithmic_counts_by_hand():
    # T = 3 tokens, k = 2: token 0 -> experts (1, 2) with adapter 0,
    # token 1 -> (2, 0) with adapter 1, token 2 -> (1, 3) without adapter.
    w = synth.Workload("hand", T=3, H=8, I=4, E=4, k=2, NA=2, r=2, dtype="bf16",
                       adapters="uniform_with_none", seed=0)
    ids = np.array([[1, 2], [2, 0], [1, 3]], np.int32)
    aid = np.array([0, 1, -1], np.int32)
    a = bench.algorithmic(w, ids, aid)
    H, I, r, s = 8, 4, 2, 2
    assert a["n_exp"] == 4 and a["R"] == 6
    # pairs (0, 1), (0, 2), (1, 2), (1, 0)
    assert a["n_pair"] == 4 and a["R_lora"] == 4
    assert a["layer_bytes"] == s * (4 * 3 * H * I + 4 * r * (2 * H + 3 * I) + 2 * 3 * H)
    assert a["layer_flop"] == 6 * 6 * H * I + 4 * 2 * r * (2 * H + 3 * I)
    # gate_up: base + expand; down: base + expand; the two shrinks are the rest
    shrinks = 4 * 2 * r * (H + I)
    assert a["gate_up_flop"] + a["down_flop"] + shrinks == a["layer_flop"]
    assert a["gate_up_flop"] == 6 * 4 * H * I + 4 * 4 * I * r
    assert a["gate_up_bytes"] == s * (4 * 2 * I * H + 4 * 2 * I * r + 3 * H + 6 * I) + 4 * 4 * r
    assert a["down_bytes"] == s * (4 * H * I + 4 * H * r + 6 * I) + 4 * 6 * H + 4 * 4 * r
    # row-wise LoRA: the down launch holds the down shrink instead of the expand
    b = bench.algorithmic(w, ids, aid, row_mode=True)
    assert b["down_flop"] == 6 * 2 * H * I + 4 * 2 * I * r
    assert b["down_bytes"] == s * (4 * H * I + 4 * I * r + 6 * I) + 4 * 6 * H + 4 * 4 * r
    assert b["gate_up_bytes"] == a["gate_up_bytes"] and b["layer_flop"] == a["layer_flop"]


def test_algorithmic_ignores_dropped_rows_and_out_of_range_adapters():
    w = synth.Workload("hand", T=2, H=8, I=4, E=4, k=2, NA=1, r=2, dtype="f32",
                       adapters="uniform", seed=0)
    ids = np.array([[0, -1], [0, 9]], np.int32)  # two rows outside [0, E)
    aid = np.array([0, 5], np.int32)              # adapter 5 >= NA: base only
    a = bench.algorithmic(w, ids, aid)
    assert (a["n_exp"], a["R"], a["n_pair"], a["R_lora"]) == (1, 2, 1, 1)


def _copy_csrc(tmp_path):
    src = os.path.join(ROOT, "lora_expert_gemm_amd", "csrc")
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    return dst


def test_kernel_hash_ignores_comments_not_code(tmp_path):
    d = _copy_csrc(tmp_path)
    h0 = bench.kernel_source_hash(str(d))
    assert h0 == bench.kernel_source_hash()
    p = d / "expert_gemm.hip"
    text = p.read_text()
    p.write_text("// a new comment line\n" + text.replace("\n", "\n  ", 3) + "/* block */\n")
    assert bench.kernel_source_hash(str(d)) == h0
    p.write_text(text.replace("kShrinkWaves", "kShrinkWaves + 0", 1))
    assert bench.kernel_source_hash(str(d)) != h0
    # the host ABI file is not kernel code
    q = d / "api.hip"
    q.write_text(q.read_text() + "\nint unused_symbol_for_the_test;\n")
    p.write_text(text)
    assert bench.kernel_source_hash(str(d)) == h0


def test_measured_traffic_only_for_current_kernel_code(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    data = {"kernel_source": bench.kernel_source_hash(),
            "workloads": {"decode_bf16": {"gate_up": {"kernel": "k", "fetch_kib": 1.0,
                                                      "write_kib": 1.0, "bytes": 1234.0}}}}
    (prof / "hbm_traffic.json").write_text(json.dumps(data))
    h = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: h)
    assert bench.measured_traffic("decode_bf16", "gate_up") == 1234.0
    assert bench.measured_traffic("decode_bf16", "down") is None
    assert bench.measured_traffic("prefill_bf16", "gate_up") is None
    data["kernel_source"] = "0" * 16
    (prof / "hbm_traffic.json").write_text(json.dumps(data))
    assert bench.measured_traffic("decode_bf16", "gate_up") is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_roofline_bound_follows_the_ridge_point():
    # bf16 ridge: 2500 TFLOP/s / 8000 GB/s = 312.5 FLOP per byte
    assert bench.hbm_bound({"gate_up_flop": 312.0, "gate_up_bytes": 1.0}, "gate_up", "bf16")
    assert not bench.hbm_bound({"gate_up_flop": 313.0, "gate_up_bytes": 1.0}, "gate_up", "bf16")
    # the five workloads' gate_up by hand: decode-sized steps stream, prefill computes
    w = synth.workload("decode_bf16")
    rows = w.T * w.k
    flop, byts = 2.0 * rows * 2 * w.I * w.H, 2.0 * 26 * 2 * w.I * w.H
    assert bench.hbm_bound({"d_flop": flop, "d_bytes": byts}, "d", "bf16")
    w = synth.workload("prefill_bf16")
    rows = w.T * w.k
    flop, byts = 2.0 * rows * 2 * w.I * w.H, 2.0 * w.E * 2 * w.I * w.H + 2.0 * w.T * w.H
    assert not bench.hbm_bound({"p_flop": flop, "p_bytes": byts}, "p", "bf16")


def test_profile_stage_names():
    from lora_expert_gemm_amd import profiling as P
    ns = "void moelora::(anonymous namespace)::"
    cases = {
        "k_shrink<unsigned short, 2, true, true, false, 8>(moelora::GemmArgs)": "shrink_gate_up",
        "k_shrink<unsigned short, 2, true, true, true, 8>(moelora::GemmArgs)": "shrink_down",
        "k_shrink<float, 1, true, false, true, 16>(moelora::GemmArgs)": "shrink_down",
        "k_tiled_shrink<false, 64, true>(moelora::GemmArgs)": "shrink_gate_up",
        "k_gate_up<unsigned short, 1, 4, true, true, 2, 4, true>(moelora::GemmArgs)": "gate_up",
        "k_down<unsigned short, 2, 4, true, true, 1, true, 3, true>(moelora::GemmArgs)": "down",
    }
    for name, stage in cases.items():
        assert P.stage_of(ns + name) == stage, name
    assert P.stage_of("__amd_rocclr_copyBuffer") is None
