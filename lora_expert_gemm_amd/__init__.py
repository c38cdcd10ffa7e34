"""Python binding of the MI355X (gfx950) fused MoE-LoRA layer library.

Thin ctypes marshalling over the C ABI of ``include/moelora.h``: every
function here has the name of the C entry point it calls and only converts
arguments (tensors to device pointers, status codes to exceptions).  All of
the layer's work runs in the library's HIP kernels; there is no fallback.
Importing this package fails loudly when ``_lib/libmoelora.so`` has not been
built (``python lora_expert_gemm_amd/build.py``).

Tensor arguments may be torch tensors (their ``data_ptr()`` is passed), raw
integer addresses, or None for a null pointer.
"""
import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libmoelora.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moelora.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python lora_expert_gemm_amd/build.py)")

# One HIP runtime per process.  PyTorch for ROCm ships its own libamdhip64
# (requested by the unversioned name libamdhip64.so); this library requests
# libamdhip64.so.7.  Loaded after PyTorch, it binds to PyTorch's copy (same
# soname); loaded first, it would pull in ROCm's copy and PyTorch would then
# load a second runtime, and whichever initialises second finds no device.
# So PyTorch, when installed, is imported before the library is loaded.
try:
    import torch  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_DEVICE = 0, -1, -2, -3, -4, -5
ERR_TOO_LARGE = -6
STATIC_SCRATCH_BYTES = 64 << 20
F32, BF16, BF16_FP8W = 0, 1, 2
DEVERR_EXPERT_ID, DEVERR_ADAPTER_ID = 1, 2
FLAG_DETERMINISTIC, FLAG_DEBUG_CHECK_IDS = 1, 2
N_STAGES = 6
STAGES = ("route_align", "shrink_gate_up", "gate_up", "shrink_down", "down", "combine")


class moelora_desc(ctypes.Structure):
    _fields_ = [("max_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_adapters", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class moelora_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("block_m", "cap", "nblk", "max_seg", "max_tiles", "reserved")] + \
               [(n, ctypes.c_size_t) for n in
                ("off_topk_ids", "off_topk_w", "off_sorted_rows", "off_block_expert",
                 "off_seg_start", "off_lora_seg", "off_tiles", "off_block_tile_start",
                 "off_counts", "off_error")]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_lib.moelora_plan.argtypes = [ctypes.POINTER(moelora_desc), ctypes.POINTER(_P),
                              ctypes.POINTER(ctypes.c_size_t)]
_lib.moelora_plan.restype = ctypes.c_int
_lib.moelora_plan_destroy.argtypes = [_P]
_lib.moelora_plan_destroy.restype = None
_lib.moelora_forward.argtypes = [_P, _I32] + [_P] * 13 + [ctypes.c_size_t, _P]
_lib.moelora_forward.restype = ctypes.c_int
_lib.moelora_forward_noalloc.argtypes = [_P, _I32] + [_P] * 12 + [_P]
_lib.moelora_forward_noalloc.restype = ctypes.c_int
_lib.moelora_status_string.argtypes = [ctypes.c_int]
_lib.moelora_status_string.restype = ctypes.c_char_p
_lib.moelora_workspace_layout.argtypes = [_P, _I32, ctypes.POINTER(moelora_layout)]
_lib.moelora_workspace_layout.restype = ctypes.c_int
_lib.moelora_read_device_error.argtypes = [_P, _P, ctypes.POINTER(_I32), _P]
_lib.moelora_read_device_error.restype = ctypes.c_int
_lib.moelora_plan_info.argtypes = [_P, _I32, ctypes.c_char_p, ctypes.c_size_t]
_lib.moelora_plan_info.restype = ctypes.c_int
_lib.moelora_timing_begin.argtypes = [_P, _I32]
_lib.moelora_timing_begin.restype = ctypes.c_int
_lib.moelora_timing_end.argtypes = [_P, ctypes.POINTER(ctypes.c_double), _I32,
                                    ctypes.POINTER(_I32)]
_lib.moelora_timing_end.restype = ctypes.c_int


def fp8_weight_buffer(codes, scales):
    """The weight-buffer layout of MOELORA_BF16_FP8W as a numpy uint8 array:
    the E4M3 codes ([E][rows][K] bytes), each row padded with zero bytes to a
    multiple of 128 bytes, zero bytes up to the next 256-byte boundary, then
    the float32 row scales ([E][rows])."""
    import numpy as np
    codes = np.asarray(codes, np.uint8)
    K = codes.shape[-1]
    pitch = (K + 127) // 128 * 128
    c = np.zeros(codes.shape[:-1] + (pitch,), np.uint8)
    c[..., :K] = codes
    c = c.reshape(-1)
    sc = np.ascontiguousarray(scales, np.float32).reshape(-1).view(np.uint8)
    off = (c.size + 255) // 256 * 256
    out = np.zeros(off + sc.size, np.uint8)
    out[:c.size] = c
    out[off:] = sc
    return out


class MoeLoraError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {moelora_status_string(status)} ({status})")


def _check(status, where):
    if status != OK:
        raise MoeLoraError(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def exported_symbols():
    """Names of the functions include/moelora.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(moelora_[a-z_]+)\s*\(", text)))


def moelora_status_string(status):
    return _lib.moelora_status_string(int(status)).decode()


def moelora_plan(max_tokens, hidden, inter, n_experts, top_k, n_adapters, rank,
                 dtype, flags=0):
    """-> (plan handle, workspace bytes)."""
    d = moelora_desc(max_tokens, hidden, inter, n_experts, top_k, n_adapters, rank,
                     dtype, flags)
    plan = _P()
    ws = ctypes.c_size_t()
    _check(_lib.moelora_plan(ctypes.byref(d), ctypes.byref(plan), ctypes.byref(ws)),
           "moelora_plan")
    return plan.value, ws.value


def moelora_plan_destroy(plan):
    _lib.moelora_plan_destroy(plan)


def moelora_forward(plan, n_tokens, x, router_logits, topk_ids, topk_w, adapter_ids,
                    w_gate_up, w_down, lora_a_gu, lora_b_gu, lora_a_d, lora_b_d,
                    out, workspace, workspace_bytes, stream=None):
    _check(_lib.moelora_forward(
        plan, n_tokens, _ptr(x), _ptr(router_logits), _ptr(topk_ids), _ptr(topk_w),
        _ptr(adapter_ids), _ptr(w_gate_up), _ptr(w_down), _ptr(lora_a_gu),
        _ptr(lora_b_gu), _ptr(lora_a_d), _ptr(lora_b_d), _ptr(out), _ptr(workspace),
        workspace_bytes, _stream(stream)), "moelora_forward")


def moelora_forward_noalloc(plan, n_tokens, x, router_logits, topk_ids, topk_w, adapter_ids,
                            w_gate_up, w_down, lora_a_gu, lora_b_gu, lora_a_d, lora_b_d,
                            out, stream=None):
    _check(_lib.moelora_forward_noalloc(
        plan, n_tokens, _ptr(x), _ptr(router_logits), _ptr(topk_ids), _ptr(topk_w),
        _ptr(adapter_ids), _ptr(w_gate_up), _ptr(w_down), _ptr(lora_a_gu),
        _ptr(lora_b_gu), _ptr(lora_a_d), _ptr(lora_b_d), _ptr(out), _stream(stream)),
        "moelora_forward_noalloc")


def moelora_workspace_layout(plan, n_tokens):
    lay = moelora_layout()
    _check(_lib.moelora_workspace_layout(plan, n_tokens, ctypes.byref(lay)),
           "moelora_workspace_layout")
    return {n: getattr(lay, n) for n, _ in moelora_layout._fields_}


def moelora_read_device_error(plan, workspace, stream=None):
    bits = _I32()
    _check(_lib.moelora_read_device_error(plan, _ptr(workspace), ctypes.byref(bits),
                                          _stream(stream)), "moelora_read_device_error")
    return bits.value


def moelora_plan_info(plan, n_tokens):
    buf = ctypes.create_string_buffer(512)
    _check(_lib.moelora_plan_info(plan, n_tokens, buf, len(buf)), "moelora_plan_info")
    return buf.value.decode()


def moelora_timing_begin(plan, max_calls):
    _check(_lib.moelora_timing_begin(plan, max_calls), "moelora_timing_begin")


def moelora_timing_end(plan):
    """-> (summed milliseconds per stage, number of timed forwards)."""
    ms = (ctypes.c_double * N_STAGES)()
    n = _I32()
    _check(_lib.moelora_timing_end(plan, ms, N_STAGES, ctypes.byref(n)), "moelora_timing_end")
    return list(ms), n.value


class Plan:
    """Owning wrapper of a plan handle."""

    _destroy_fn = _lib.moelora_plan_destroy  # ctypes function object (holds the library)

    def __init__(self, max_tokens, hidden, inter, n_experts, top_k, n_adapters, rank,
                 dtype, flags=0):
        self.handle, self.workspace_bytes = moelora_plan(
            max_tokens, hidden, inter, n_experts, top_k, n_adapters, rank, dtype, flags)
        self.desc = dict(max_tokens=max_tokens, hidden=hidden, inter=inter,
                         n_experts=n_experts, top_k=top_k, n_adapters=n_adapters,
                         rank=rank, dtype=dtype)

    def __del__(self):
        # the destroy function is held by the class: module globals may
        # already be gone when a plan is collected at interpreter shutdown
        h = getattr(self, "handle", None)
        if h:
            self._destroy_fn(h)
            self.handle = None

    def layout(self, n_tokens):
        return moelora_workspace_layout(self.handle, n_tokens)

    def info(self, n_tokens):
        return moelora_plan_info(self.handle, n_tokens)

    def forward(self, n_tokens, x, out, workspace, *, router_logits=None, topk_ids=None,
                topk_w=None, adapter_ids=None, w_gate_up, w_down, lora_a_gu=None,
                lora_b_gu=None, lora_a_d=None, lora_b_d=None, stream=None):
        ws_bytes = workspace.numel() * workspace.element_size() \
            if hasattr(workspace, "numel") else self.workspace_bytes
        moelora_forward(self.handle, n_tokens, x, router_logits, topk_ids, topk_w,
                        adapter_ids, w_gate_up, w_down, lora_a_gu, lora_b_gu, lora_a_d,
                        lora_b_d, out, workspace, ws_bytes, stream)
