"""ctypes declarations of libtreeverify's C ABI (include/tree_verify.h)."""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtreeverify.so")

TV_FP32, TV_BF16 = 0, 1
MAX_CHILDREN = 16

STATUS_NAMES = {
    0: "TV_OK", 1: "TV_ERR_NULL", 2: "TV_ERR_SHAPE", 3: "TV_ERR_DTYPE",
    4: "TV_ERR_WORKSPACE", 5: "TV_ERR_TREE", 6: "TV_ERR_PAGES", 7: "TV_ERR_HIP",
    8: "TV_ERR_LOGITS", 9: "TV_ERR_PATH", 10: "TV_ERR_TIMEOUT",
}
DEV_BITS = {1: "TREE", 2: "PAGES", 4: "LOGITS", 8: "PATH", 16: "TIMEOUT", 32: "SHAPE"}


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_nodes", ctypes.c_int32),
                ("max_depth", ctypes.c_int32), ("max_kv_len", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class SampleDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("max_nodes", ctypes.c_int32), ("max_depth", ctypes.c_int32),
                ("rule", ctypes.c_int32), ("greedy", ctypes.c_int32)]


class SparkDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("depths", ctypes.c_int32), ("max_nodes", ctypes.c_int32),
                ("max_siblings", ctypes.c_int32), ("calib_a", ctypes.c_float),
                ("calib_b", ctypes.c_float)]


TV_RULE_WITHOUT_REPLACEMENT = 0
TV_RULE_WITH_REPLACEMENT = 1
TV_GREEDY_EVERY_NODE = 0
TV_GREEDY_PATH = 1
TV_SAMPLE_STATIC_MAX_BATCH = 1024


EXPORTS = [
    "tv_attn_workspace_size", "tv_sample_workspace_size", "tv_workspace_init",
    "tv_device_status", "tree_verify_attn", "tree_spec_sample", "tree_spec_sample_noalloc",
    "tree_accept_path",
    "tree_kv_commit", "tree_draw_siblings", "tree_expand_step", "tree_rerank",
    "tv_expand_workspace_size", "tv_spark_workspace_size", "tree_spark_build",
    "tv_tree_meta", "tv_validate_tree", "tv_validate_pages", "tv_status_string",
    "tv_last_hip_error", "tv_version",
]

_lib = None


def load():
    """Load libtreeverify.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m tree_verification_verify_amd.build` (hipcc, gfx950)")
    # PyTorch's wheel ships its own HIP runtime under the same sonames as the
    # one the library links (libamdhip64.so.7, libhsa-runtime64.so.1), and a
    # process keeps whichever loads first. Importing torch first makes the
    # library bind to torch's runtime, the one torch's device memory and
    # streams belong to; loaded the other way round, the library's first
    # HIP call can find no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    S = ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "tv_attn_workspace_size": (S, [ctypes.POINTER(AttnDesc)]),
        "tv_sample_workspace_size": (S, [ctypes.POINTER(SampleDesc)]),
        "tv_workspace_init": (st, [P, S, P]),
        "tv_device_status": (st, [P, P, ctypes.POINTER(ctypes.c_uint32)]),
        "tree_verify_attn": (st, [ctypes.POINTER(AttnDesc)] + [P] * 9 + [P, S, P]),
        "tree_spec_sample": (st, [ctypes.POINTER(SampleDesc)] + [P] * 9 + [P, S, P]),
        "tree_spec_sample_noalloc": (st, [ctypes.POINTER(SampleDesc)] + [P] * 9 + [P, P]),
        "tree_accept_path": (st, [I32, I32] + [P] * 10 + [P, P]),
        "tree_kv_commit": (st, [ctypes.POINTER(AttnDesc), I32, ctypes.c_int64] + [P] * 7
                           + [I32, P, P]),
        "tree_draw_siblings": (st, [I32, I32, P, P, P, ctypes.c_uint32, ctypes.c_uint64, P, P, P]),
        "tree_expand_step": (st, [I32, I32, I32, I32, P, P, I32, I32, P, P, P, P, P,
                                  ctypes.c_size_t, P]),
        "tv_expand_workspace_size": (ctypes.c_size_t, [I32, I32, I32]),
        "tree_rerank": (st, [I32, I32, I32, I32, P, P, P, P, P, P, P, P]),
        "tv_tree_meta": (st, [I32, I32] + [P] * 6 + [P, P]),
        "tv_spark_workspace_size": (S, [ctypes.POINTER(SparkDesc)]),
        "tree_spark_build": (st, [ctypes.POINTER(SparkDesc)] + [P] * 6
                             + [ctypes.c_uint32, ctypes.c_uint64] + [P] * 4 + [P, S, P]),
        "tv_validate_tree": (st, [I32, P, P, I32, I32]),
        "tv_validate_pages": (st, [I32, P, P, P, P, I32, I32]),
        "tv_status_string": (ctypes.c_char_p, [st]),
        "tv_last_hip_error": (ctypes.c_char_p, []),
        "tv_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib
