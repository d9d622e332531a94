"""ctypes declarations of libmk.so (the C ABI in include/mk.h).

Argument marshalling only: every step of the decoder runs in the library's
HIP kernels.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK, MK_EINVAL, MK_ENOMEM, MK_ELAUNCH, MK_EDEVICE, MK_ENOTSUP = 0, -1, -2, -3, -4, -5
MK_F32, MK_BF16 = 0, 1
MK_DECODE, MK_PREFILL = 0, 1
MK_MEGAKERNEL, MK_KERNEL_PER_OP, MK_KERNEL_PER_OP_GRAPH, MK_MULTI_STREAM = 0, 1, 2, 3
MK_PART_META, MK_PART_INSTR, MK_PART_WAITS, MK_PART_TARGETS, MK_PART_DEVICE = range(5)
MK_STATIC_SCRATCH_BYTES = 64 << 20
(MK_T_X, MK_T_QKV, MK_T_OPART, MK_T_ATT, MK_T_HRES, MK_T_ACT, MK_T_COUNTERS, MK_T_HEADS,
 MK_T_ERROR, MK_T_LMPART) = range(10)
(MK_OPT_WORKERS_PER_CU, MK_OPT_SPIN_LIMIT, MK_OPT_NUM_CUS, MK_OPT_TRACE_BUFFER, MK_OPT_TRACE_BYTES,
 MK_OPT_GEMV_PIPE, MK_OPT_DELAY_SEED, MK_OPT_STREAMS, MK_OPT_MEGAKERNELS,
 MK_OPT_PREFILL_LO) = range(10)


class mk_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("qk_norm", C.c_int32), ("has_embed", C.c_int32),
                ("has_lm_head", C.c_int32), ("dtype", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_double)]


class mk_plan(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("mode", "rows", "ctx_max", "tq", "to", "tf", "td", "kb",
                                         "bm", "bn", "n_queues", "fuse_combine", "loop", "attn_pop")]


class mk_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("wqkv", "wo", "wgate", "wup", "wdown", "attn_norm",
                                          "ffn_norm", "q_norm", "k_norm", "embed", "lm_head",
                                          "final_norm")]


class mk_kv(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("rows", C.c_int32)]


class mk_dev_error(C.Structure):
    _fields_ = [(n, C.c_uint32) for n in ("code", "instr", "barrier", "value", "target")]


_lib = None


def lib() -> C.CDLL:
    """The loaded library; raises if it was never built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m tile_synchronized_decoder_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, I32, SZ, VP = C.POINTER, C.c_int32, C.c_size_t, C.c_void_p
    sig = {
        "mk_build_queue": (I32, [P(mk_config), P(mk_plan), P(VP)]),
        "mk_queue_nbytes": (SZ, [VP, I32]),
        "mk_queue_export": (I32, [VP, I32, VP, SZ]),
        "mk_queue_free": (None, [VP]),
        "mk_workspace_nbytes": (I32, [VP, P(SZ)]),
        "mk_workspace_offset": (I32, [VP, I32, I32, P(SZ)]),
        "mk_decode_step": (I32, [VP, VP, P(mk_weights), P(mk_kv), VP, VP, VP, I32, VP, SZ, VP, VP,
                                 I32, VP]),
        "mk_decode_step_static": (I32, [VP, VP, P(mk_weights), P(mk_kv), VP, VP, VP, I32, VP, VP, VP, I32,
                                        VP]),
        "mk_decode_loop": (I32, [VP, VP, P(mk_weights), P(mk_kv), VP, VP, I32, I32, I32, VP, SZ, VP, VP, VP]),
        "mk_lm_head": (I32, [VP, P(mk_weights), VP, SZ, VP, VP, VP]),
        "mk_prefill": (I32, [VP, VP, P(mk_weights), P(mk_kv), VP, I32, I32, VP, SZ, VP, VP, I32, VP]),
        "mk_device_error": (I32, [VP, VP, P(mk_dev_error), VP]),
        "mk_set_option": (I32, [I32, C.c_int64]),
        "mk_get_option": (C.c_int64, [I32]),
        "mk_status_str": (C.c_char_p, [I32]),
        "mk_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


EXPORTED = ["mk_build_queue", "mk_queue_nbytes", "mk_queue_export", "mk_queue_free",
            "mk_workspace_nbytes", "mk_workspace_offset", "mk_decode_step", "mk_decode_step_static", "mk_decode_loop",
            "mk_lm_head", "mk_prefill",
            "mk_device_error", "mk_set_option", "mk_get_option", "mk_status_str", "mk_last_error"]


class MkError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        msg = L.mk_last_error().decode(errors="replace")
        super().__init__(f"{where}: {L.mk_status_str(status).decode()} ({status}): {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != MK_OK:
        raise MkError(status, where)
