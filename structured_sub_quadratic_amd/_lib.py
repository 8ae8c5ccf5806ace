"""ctypes view of the C ABI in include/monarch_attn.h (marshalling only)."""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmonarch_attn.so")

MA_OK = 0
STATUS_NAMES = {0: "MA_OK", 1: "MA_ERR_INVALID_ARGUMENT", 2: "MA_ERR_UNSUPPORTED",
                3: "MA_ERR_WORKSPACE_TOO_SMALL", 4: "MA_ERR_DEVICE"}
MA_F32, MA_BF16 = 0, 1
LAYOUTS = {"flat": 0, "fh_w": 1, "w_fh": 2, "f_hw": 3, "hw_f": 4, "fw_h": 5, "h_fw": 6}
MA_FLAG_FORCE_STAGED = 1
MA_FLAG_FAST_AGGREGATE = 2
MA_FLAG_FORCE_FUSED = 4
MA_FLAG_PRECISE_AGGREGATE = 8
MA_FLAG_PAD_FRONT = 16
MA_FLAG_REUSE_FORWARD_STATE = 32
MONARCH_ATTN_SCRATCH_BYTES = 64 << 20   # the library-owned workspace of the no-alloc entry point


class MAProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64),
        ("seq_len", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("b1", ctypes.c_int32), ("b2", ctypes.c_int32),
        ("c1", ctypes.c_int32), ("c2", ctypes.c_int32),
        ("steps", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("f", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("kv_heads", ctypes.c_int32),
        ("causal", ctypes.c_int32),
    ]


class MAExports(ctypes.Structure):
    _fields_ = [("L", ctypes.c_void_p), ("R", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("objective", ctypes.c_void_p)]


class MonarchAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


_lib = None


def load():
    """Load the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first with "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python -m structured_sub_quadratic_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(MAProblem)
    vp = ctypes.c_void_p
    lib.monarch_attn_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.monarch_attn_workspace_size.restype = ctypes.c_int
    lib.monarch_attn_forward.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(MAExports), vp,
                                         ctypes.c_size_t, vp]
    lib.monarch_attn_forward.restype = ctypes.c_int
    lib.monarch_attn_forward_noalloc.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(MAExports), vp]
    lib.monarch_attn_forward_noalloc.restype = ctypes.c_int
    lib.monarch_attn_forward_timed.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(MAExports), vp,
                                               ctypes.c_size_t, vp, ctypes.POINTER(vp),
                                               ctypes.c_int32]
    lib.monarch_attn_forward_timed.restype = ctypes.c_int
    lib.monarch_attn_backward_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.monarch_attn_backward_workspace_size.restype = ctypes.c_int
    lib.monarch_attn_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.monarch_attn_backward.restype = ctypes.c_int
    lib.monarch_attn_num_launches.argtypes = [P]
    lib.monarch_attn_num_launches.restype = ctypes.c_int32
    lib.monarch_attn_launch_name.argtypes = [P, ctypes.c_int32]
    lib.monarch_attn_launch_name.restype = ctypes.c_char_p
    lib.monarch_attn_event_create.argtypes = [ctypes.POINTER(vp)]
    lib.monarch_attn_event_create.restype = ctypes.c_int
    lib.monarch_attn_event_destroy.argtypes = [vp]
    lib.monarch_attn_event_destroy.restype = ctypes.c_int
    lib.monarch_attn_event_record.argtypes = [vp, vp]
    lib.monarch_attn_event_record.restype = ctypes.c_int
    lib.monarch_attn_event_elapsed_ms.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_float)]
    lib.monarch_attn_event_elapsed_ms.restype = ctypes.c_int
    lib.monarch_attn_status_string.argtypes = [ctypes.c_int]
    lib.monarch_attn_status_string.restype = ctypes.c_char_p
    lib.monarch_attn_version.argtypes = []
    lib.monarch_attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status, where):
    if status != MA_OK:
        raise MonarchAttnError(status, where)
