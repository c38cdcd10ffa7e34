"""CPU oracle for the fused MoE-LoRA layer (ctypes wrapper of moelora_ref.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does, and the
two share no code.  The arithmetic lives in ``moelora_ref.c`` (plain C,
double precision); this module only marshals numpy arrays.

Functions follow the AWS Machine Learning blog post "Efficiently serve dozens
of fine-tuned models with vLLM on Amazon SageMaker AI and Amazon Bedrock",
section "Implementing multi-LoRA inference for MoE models in vLLM" (router,
gate_up / down experts, y = xW + xAB with shrink z = xA and expand zB); the
readings taken where the post is silent are documented in the C source.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against brute force, closed forms, numpy float64 dense evaluation and the
hand-derived fixtures under ``tests/golden/``.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moelora_ref.c")
_LIB_DIR = os.path.join(_HERE, "_lib")
_LIB = os.path.join(_LIB_DIR, "libmoelora_ref.so")

F32, BF16, BF16_FP8W = 0, 1, 2


_CFLAGS = ["-O2", "-fopenmp", "-std=c11", "-fPIC", "-shared"]


def build(force=True):
    """Compile the oracle with gcc (no fast-math, so every sum stays
    sequential; OpenMP spreads independent tokens over threads)."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    subprocess.check_call(
        ["gcc", *_CFLAGS, "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i = ctypes.c_int
    lib.ref_route.argtypes = [i, i, i, P, P, P]
    lib.ref_route.restype = i
    lib.ref_align_sizes.argtypes = [i, i, i, i, P, P, P, P]
    lib.ref_align_sizes.restype = None
    lib.ref_align.argtypes = [i, i, i, i, i, P, P, P, P, P, P, P, P, P]
    lib.ref_align.restype = i
    lib.ref_forward.argtypes = [i, i, i, i, i, i, i, i,
                                P, P, P, P, P, P, P, P, P, P, P, i, P, P, P]
    lib.ref_forward.restype = i
    lib.ref_fp8_e4m3.argtypes = [i]
    lib.ref_fp8_e4m3.restype = ctypes.c_double
    lib.ref_set_threads.argtypes = [i]
    lib.ref_set_threads.restype = i
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def ref_route(logits, k, _lib_override=None):
    """logits [T][E] float32 -> (ids [T][k] int32, w [T][k] float64)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    rc = (_lib_override or _load()).ref_route(T, E, k, _ptr(logits), _ptr(ids), _ptr(w))
    if rc:
        raise ValueError(f"ref_route failed ({rc})")
    return ids, w


def align_sizes(R, E, NA, BM, _lib_override=None):
    v = [ctypes.c_int64() for _ in range(4)]
    (_lib_override or _load()).ref_align_sizes(R, E, NA, BM, *[ctypes.byref(x) for x in v])
    return tuple(int(x.value) for x in v)  # cap, nblk, max_seg, max_tiles


def ref_align(ids, adapter_ids, E, NA, BM, _lib_override=None):
    """ids [T][k] int32, adapter_ids [T] int32 or None -> dict of arrays."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    aid = _c(adapter_ids, np.int32)
    cap, nblk, max_seg, max_tiles = align_sizes(T * k, E, NA, BM, _lib_override)
    out = dict(
        sorted_rows=np.zeros(cap, np.int32),
        block_expert=np.zeros(nblk, np.int32),
        seg_start=np.zeros(E + 1, np.int32),
        lora_seg=np.zeros((max_seg, 4), np.int32),
        tiles=np.zeros((max_tiles, 4), np.int32),
        block_tile_start=np.zeros(nblk + 1, np.int32),
    )
    counts = np.zeros(3, np.int32)
    rc = (_lib_override or _load()).ref_align(T, k, E, NA, BM, _ptr(ids), _ptr(aid),
                           _ptr(out["sorted_rows"]), _ptr(out["block_expert"]),
                           _ptr(out["seg_start"]), _ptr(out["lora_seg"]),
                           _ptr(out["tiles"]), _ptr(out["block_tile_start"]),
                           _ptr(counts))
    if rc:
        raise ValueError(f"ref_align failed ({rc})")
    out["num_padded"] = int(counts[0])
    out["n_lora_seg"] = int(counts[1])
    out["n_tiles"] = int(counts[2])
    return out


def ref_forward(x, ids, w, adapter_ids, W_gu, W_d, A_gu=None, B_gu=None,
                A_d=None, B_d=None, *, inter, rank=0, n_adapters=0,
                dtype=F32, tokens=None, W_gu_scale=None, W_d_scale=None,
                _lib_override=None):
    """The layer output (float64) for the selected tokens.

    Arrays of the storage dtype are float32 (dtype=F32) or uint16 bf16 bit
    patterns (dtype=BF16).  With dtype=BF16_FP8W, x and the LoRA arrays are
    bf16 patterns and W_gu / W_d are uint8 E4M3 codes with float32 scales
    W_gu_scale [E][2I] and W_d_scale [E][H], one per weight row.
    ``tokens`` selects rows of the output (all when None); the result has
    shape [len(tokens)][H].
    """
    st = np.float32 if dtype == F32 else np.uint16
    wt = np.uint8 if dtype == BF16_FP8W else st
    x = _c(x, st)
    T, H = x.shape
    ids = _c(ids, np.int32)
    k = ids.shape[1]
    E = W_gu.shape[0]
    w = _c(w, np.float64)
    aid = _c(adapter_ids, np.int32)
    arrs = [_c(W_gu, wt), _c(W_d, wt)] + [_c(a, st) for a in (A_gu, B_gu, A_d, B_d)]
    sg, sd = _c(W_gu_scale, np.float32), _c(W_d_scale, np.float32)
    sel = None if tokens is None else _c(tokens, np.int32)
    n_sel = T if sel is None else len(sel)
    out = np.zeros((n_sel, H), np.float64)
    rc = (_lib_override or _load()).ref_forward(T, H, inter, E, k, n_adapters, rank, dtype,
                             _ptr(x), _ptr(ids), _ptr(w), _ptr(aid),
                             *[_ptr(a) for a in arrs], _ptr(sel), n_sel,
                             _ptr(out), _ptr(sg), _ptr(sd))
    if rc:
        raise ValueError(f"ref_forward failed ({rc})")
    return out


def fp8_e4m3(code, _lib_override=None):
    """Value of an OCP E4M3 code (0..255) as the oracle decodes it."""
    return float((_lib_override or _load()).ref_fp8_e4m3(int(code)))


def set_threads(n):
    """Threads the oracle's forward uses (0: all, the OpenMP default);
    returns that count.  Results do not depend on it."""
    return int(_load().ref_set_threads(int(n)))


class Variant:
    """The oracle's API bound to another build of the C source (used by the
    test that plants mistakes in a copy of the oracle to show the pins catch
    them)."""
    F32, BF16, BF16_FP8W = F32, BF16, BF16_FP8W

    def __init__(self, so_path):
        self._l = _bind(so_path)

    def ref_route(self, logits, k):
        return ref_route(logits, k, _lib_override=self._l)

    def ref_align(self, ids, adapter_ids, E, NA, BM):
        return ref_align(ids, adapter_ids, E, NA, BM, _lib_override=self._l)

    def ref_forward(self, *a, **kw):
        return ref_forward(*a, _lib_override=self._l, **kw)

    def fp8_e4m3(self, code):
        return fp8_e4m3(code, _lib_override=self._l)


def build_variant(src_text, so_path):
    """Compile C source text (a modified copy of moelora_ref.c) to so_path."""
    c_path = so_path[:-3] + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *_CFLAGS, "-w", "-o", so_path, c_path, "-lm"])
    return Variant(so_path)


def source():
    with open(_SRC) as f:
        return f.read()
