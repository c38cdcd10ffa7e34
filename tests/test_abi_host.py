"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/moelora.h declares, validates shapes, lays out
its workspace as documented, and rejects bad arguments before touching the
device."""
import ctypes
import json
import os

import numpy as np
import pytest

import oracle

lib = pytest.importorskip("lora_expert_gemm_amd")

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_every_declared_symbol_is_exported():
    names = lib.exported_symbols()
    assert "moelora_forward" in names and "moelora_plan" in names
    so = ctypes.CDLL(lib.LIB_PATH)
    for n in names:
        assert hasattr(so, n), f"{n} declared in moelora.h but not exported"


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.moelora_status_string(st) != "unknown status"


DECODE = dict(max_tokens=16, hidden=2880, inter=2880, n_experts=32, top_k=4,
              n_adapters=8, rank=32, dtype=lib.BF16)


@pytest.mark.parametrize("bad,status", [
    (dict(n_experts=0), lib.ERR_UNSUPPORTED),
    (dict(n_experts=2000), lib.ERR_UNSUPPORTED),
    (dict(top_k=33, n_experts=64), lib.ERR_UNSUPPORTED),
    (dict(top_k=5, n_experts=4), lib.ERR_UNSUPPORTED),
    (dict(n_adapters=300), lib.ERR_UNSUPPORTED),
    (dict(n_experts=512, n_adapters=32), lib.ERR_UNSUPPORTED),  # E (NA + 1) > 8448
    (dict(rank=0), lib.ERR_UNSUPPORTED),                      # adapters need a rank
    (dict(rank=257), lib.ERR_UNSUPPORTED),
    (dict(dtype=7), lib.ERR_UNSUPPORTED),
    (dict(hidden=0), lib.ERR_UNSUPPORTED),
    (dict(max_tokens=-1), lib.ERR_UNSUPPORTED),
    (dict(flags=4), lib.ERR_UNSUPPORTED),                     # an undefined flag bit
    (dict(flags=0x80000000), lib.ERR_UNSUPPORTED),
])
def test_plan_rejects_out_of_range_shapes(bad, status):
    with pytest.raises(lib.MoeLoraError) as ei:
        lib.moelora_plan(**dict(DECODE, **bad))
    assert ei.value.status == status


@pytest.mark.parametrize("flags", [
    lib.FLAG_DETERMINISTIC, lib.FLAG_DEBUG_CHECK_IDS,
    lib.FLAG_DETERMINISTIC | lib.FLAG_DEBUG_CHECK_IDS])
def test_plan_accepts_the_defined_flags(flags):
    """Both behaviours are always on, so the flags change neither the kernels
    nor the workspace."""
    p0 = lib.Plan(**DECODE)
    p = lib.Plan(**DECODE, flags=flags)
    assert p.workspace_bytes == p0.workspace_bytes
    for T in (1, 7, 16):
        assert p.info(T) == p0.info(T)


def _info(p, T):
    return dict(kv.split("=") for kv in p.info(T).split())


# Shapes whose max_tokens sits inside a token-count bucket, where the
# workspace of a smaller token count can exceed that of max_tokens (the
# split counts of the shrink and of the down GEMM fall as T grows).
SCAN = [
    dict(max_tokens=100, hidden=4096, inter=11008, n_experts=1, top_k=1, n_adapters=16,
         rank=32, dtype=lib.BF16),
    dict(max_tokens=300, hidden=2048, inter=768, n_experts=128, top_k=8, n_adapters=32,
         rank=16, dtype=lib.BF16),
    dict(max_tokens=77, hidden=2880, inter=2880, n_experts=32, top_k=4, n_adapters=8,
         rank=32, dtype=lib.BF16),
    dict(max_tokens=50, hidden=128, inter=256, n_experts=4, top_k=2, n_adapters=2, rank=8,
         dtype=lib.F32),
]


@pytest.mark.parametrize("desc", SCAN)
def test_plan_workspace_covers_every_token_count(desc):
    p = lib.Plan(**desc)
    need = [int(_info(p, T)["workspace"]) for T in range(desc["max_tokens"] + 1)]
    assert max(need) == p.workspace_bytes


def test_tuning_switches_are_read_at_plan_time(monkeypatch):
    """A forward never reads the environment: a switch set after the plan
    changes nothing, and one set before it holds after it is unset."""
    monkeypatch.delenv("MOELORA_TG", raising=False)
    p = lib.Plan(**DECODE)
    before = [p.info(T) for T in (1, 8, 16)]
    monkeypatch.setenv("MOELORA_TG", "4")
    assert [p.info(T) for T in (1, 8, 16)] == before
    forced = lib.Plan(**DECODE)
    monkeypatch.delenv("MOELORA_TG")
    assert all(_info(forced, T)["block_m"] == "64" for T in (1, 8, 16))


@pytest.mark.parametrize("desc,T,where", [
    (DECODE, 16, "routing"),            # row mode: per-row shrinks in the routing launch
    (dict(max_tokens=256, hidden=2048, inter=768, n_experts=128, top_k=8, n_adapters=32,
          rank=16, dtype=lib.BF16), 256, "scatter"),   # tile mode, large alignment: folded
    (dict(max_tokens=256, hidden=2048, inter=768, n_experts=128, top_k=8, n_adapters=32,
          rank=16, dtype=lib.F32), 256, "kernel"),     # float: its own launch
    (dict(max_tokens=256, hidden=2050, inter=768, n_experts=128, top_k=8, n_adapters=32,
          rank=16, dtype=lib.BF16), 256, "kernel"),    # rows not 16-byte aligned
    (dict(max_tokens=6400, hidden=2880, inter=2880, n_experts=32, top_k=4, n_adapters=4,
          rank=64, dtype=lib.BF16), 6400, "kernel"),   # LDS-tiled 128-row blocks
    (dict(max_tokens=256, hidden=2048, inter=768, n_experts=128, top_k=8, n_adapters=0,
          rank=0, dtype=lib.BF16), 256, "none"),
])
def test_where_the_gate_up_shrink_runs(desc, T, where):
    """The plan reports which launch computes the gate_up shrink."""
    assert _info(lib.Plan(**desc), T)["shrink_gu"] == where


@pytest.mark.parametrize("desc", [
    DECODE,
    dict(max_tokens=6400, hidden=2880, inter=2880, n_experts=32, top_k=4, n_adapters=4,
         rank=64, dtype=lib.BF16),
    dict(max_tokens=256, hidden=2048, inter=768, n_experts=128, top_k=8, n_adapters=32,
         rank=16, dtype=lib.BF16),
    dict(max_tokens=8, hidden=128, inter=256, n_experts=4, top_k=2, n_adapters=2, rank=8,
         dtype=lib.F32),
])
def test_layout_sizes_and_offsets(desc):
    p = lib.Plan(**desc)
    E, k, NA = desc["n_experts"], desc["top_k"], desc["n_adapters"]
    for T in sorted({0, 1, 2, desc["max_tokens"] // 3, desc["max_tokens"]}):
        lay = p.layout(T)
        BM = lay["block_m"]
        assert BM % 16 == 0
        cap, nblk, max_seg, max_tiles = oracle.align_sizes(T * k, E, NA, BM)
        assert (lay["cap"], lay["nblk"], lay["max_seg"], lay["max_tiles"]) == \
            (cap, nblk, max_seg, max_tiles)
        assert lay["off_error"] == 0
        offs = sorted(v for n, v in lay.items() if n.startswith("off_"))
        assert all(o % 256 == 0 for o in offs)
        if T > 0:  # at T = 0 the empty arrays share offsets
            assert len(set(offs)) == len(offs)
        assert max(offs) < p.workspace_bytes
    with pytest.raises(lib.MoeLoraError):
        p.layout(desc["max_tokens"] + 1)


def test_even_k_instance_choice_matches_the_masking_example():
    g = json.load(open(os.path.join(GOLD, "even_k.json")))
    # the example's own arithmetic: two blocks of 64 over K = 100
    assert 2 * g["block_k"] - g["k"] == g["invalid_positions_in_last_block"]
    assert (g["k"] % g["block_k"] == 0) == g["even_k"]
    # the library's bf16 contraction step is 32: K = 100 also leaves 28
    # masked positions in its last step and needs the masked instance
    p = lib.Plan(max_tokens=4, hidden=g["k"], inter=200, n_experts=4, top_k=2,
                 n_adapters=2, rank=16, dtype=lib.BF16)
    info = dict(kv.split("=") for kv in p.info(4).split())
    assert info["even_k_gu"] == "0" and info["vec"] == "0"
    assert int(info["k_tail_gu"]) == g["invalid_positions_in_last_block"]
    p2 = lib.Plan(**DECODE)
    info2 = dict(kv.split("=") for kv in p2.info(16).split())
    assert info2["even_k_gu"] == "1" and info2["even_k_d"] == "1" and info2["k_tail_gu"] == "0"


FAKE = 1 << 20  # a 256-aligned address that is never dereferenced

# The argument checks below hand the library fake device addresses and rely
# on it rejecting the call before any launch.  They only run where no GPU is
# visible, so a regression in the checks can never reach a device.
def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_device = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer checks run only without a GPU")


def _fwd(p, **over):
    args = dict(n_tokens=4, x=FAKE, router_logits=FAKE, topk_ids=None, topk_w=None,
                adapter_ids=FAKE, w_gate_up=FAKE, w_down=FAKE, lora_a_gu=FAKE,
                lora_b_gu=FAKE, lora_a_d=FAKE, lora_b_d=FAKE, out=FAKE, workspace=FAKE,
                workspace_bytes=p.workspace_bytes, stream=0)
    args.update(over)
    lib.moelora_forward(p.handle, **args)


@pytest.mark.parametrize("over", [
    dict(x=None), dict(w_gate_up=None), dict(w_down=None), dict(out=None),
    dict(workspace=None), dict(router_logits=None),                 # nothing to route from
    dict(topk_ids=FAKE),                                            # ids without weights
    dict(topk_ids=FAKE, topk_w=FAKE),                               # ids and logits both
    dict(lora_b_d=None),                                            # partial LoRA set
    dict(x=FAKE + 8),                                               # misaligned
    dict(workspace=FAKE + 16),                                      # workspace misaligned
    dict(n_tokens=17), dict(n_tokens=-1),
])
@no_device
def test_forward_rejects_bad_arguments(over):
    p = lib.Plan(**DECODE)
    with pytest.raises(lib.MoeLoraError) as ei:
        _fwd(p, **over)
    assert ei.value.status == lib.ERR_INVALID_ARG


@no_device
def test_forward_rejects_small_workspace():
    p = lib.Plan(**DECODE)
    need = p.layout(4)
    with pytest.raises(lib.MoeLoraError) as ei:
        _fwd(p, workspace_bytes=256)
    assert ei.value.status == lib.ERR_WORKSPACE
    assert need["cap"] > 0


@no_device
def test_zero_tokens_is_a_noop():
    p = lib.Plan(**DECODE)
    _fwd(p, n_tokens=0)  # returns OK without any device work


def test_binding_loads_torch_first():
    """The package imports PyTorch (when installed) before loading the HIP
    library, so both use one HIP runtime: loaded the other way round,
    PyTorch brings a second runtime and one of them finds no device."""
    import subprocess
    import sys
    code = ("import sys; import lora_expert_gemm_amd as L; "
            "print(int('torch' in sys.modules))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


@pytest.mark.parametrize("K", [64, 192, 2880, 4096])
def test_fp8_weight_buffer_layout(K):
    """The E4M3 weight buffer as the header lays it out: rows of K codes
    padded with zero bytes to a multiple of 128 bytes, then the float32 row
    scales at the next 256-byte boundary."""
    E, rows = 3, 5
    rng = np.random.default_rng(K)
    codes = rng.integers(0, 256, size=(E, rows, K), dtype=np.uint8)
    scales = rng.random((E, rows), dtype=np.float32)
    buf = lib.fp8_weight_buffer(codes, scales)
    pitch = (K + 127) // 128 * 128
    off = (E * rows * pitch + 255) // 256 * 256
    assert buf.dtype == np.uint8 and buf.size == off + 4 * E * rows
    body = buf[:E * rows * pitch].reshape(E, rows, pitch)
    assert np.array_equal(body[..., :K], codes)
    assert not body[..., K:].any()
    assert not buf[E * rows * pitch:off].any()
    assert np.array_equal(buf[off:].view(np.float32).reshape(E, rows), scales)
