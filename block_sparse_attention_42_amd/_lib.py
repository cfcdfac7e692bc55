"""ctypes view of libbsa.so (include/bsa.h).  Loads the in-tree library or fails."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsa.so")

BSA_OK = 0
BSA_ERR_INVALID_ARGUMENT = 1
BSA_ERR_UNSUPPORTED = 2
BSA_ERR_HIP = 3
BSA_DTYPE_BF16 = 0
BSA_DTYPE_F32 = 1
BSA_SELECT_TOPK = 0
BSA_SELECT_SAMPLE = 1
BSA_SPLIT_STATIC_MAX_BYTES = 33554432

EXPORTED = ["bsa_derive", "bsa_pool_blocks", "bsa_pool_qk", "bsa_build_mask", "bsa_forward", "bsa_forward_ex",
            "bsa_forward_split", "bsa_forward_split_workspace_bytes", "bsa_forward_split_static",
            "bsa_cluster_importance", "bsa_select_blocks", "bsa_top_p_workspace_bytes", "bsa_select_top_p",
            "bsa_frame_scores", "bsa_classify_heads", "bsa_structured_lists",
            "bsa_status_string", "bsa_last_error", "bsa_abi_version"]


class bsa_geometry(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("text_len", ctypes.c_int32), ("frames", ctypes.c_int32),
                ("latent_h", ctypes.c_int32), ("latent_w", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("q_block", ctypes.c_int32),
                ("k_block", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("seq_alloc", ctypes.c_int64)]


class bsa_mask_params(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("keep_ratio", ctypes.c_double), ("frame0_dense", ctypes.c_int32),
                ("text_columns", ctypes.c_int32), ("log_cluster", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class bsa_topp_params(ctypes.Structure):
    _fields_ = [("domain", ctypes.c_int32), ("value_aware", ctypes.c_int32),
                ("top_p", ctypes.c_double), ("entropy_eps", ctypes.c_float),
                ("frame0_dense", ctypes.c_int32), ("text_columns", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class bsa_forward_options(ctypes.Structure):
    _fields_ = [("launch_order", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]


class bsa_struct_params(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("dummy_prev", ctypes.c_int32),
                ("block_causal", ctypes.c_int32), ("frame0_dense", ctypes.c_int32),
                ("text_columns", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class bsa_derived(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int64), ("nqb", ctypes.c_int32), ("nkb", ctypes.c_int32),
                ("frame0_first", ctypes.c_int32), ("frame0_last", ctypes.c_int32),
                ("text_last", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("expected", ctypes.c_float), ("reserved", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if libbsa.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m block_sparse_attention_42_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        G = ctypes.POINTER(bsa_geometry)
        M = ctypes.POINTER(bsa_mask_params)
        L.bsa_derive.argtypes = [G, M, ctypes.POINTER(bsa_derived)]
        L.bsa_pool_blocks.argtypes = [P, ctypes.c_int32, G, ctypes.c_int32, P, P]
        L.bsa_pool_qk.argtypes = [P, P, ctypes.c_int32, G, P, P, P]
        L.bsa_build_mask.argtypes = [P, P, G, M, P, P, P, P, P]
        L.bsa_forward.argtypes = [P, P, P, ctypes.c_int32, G, P, P, P, ctypes.c_float, P, P, P]
        L.bsa_forward_ex.argtypes = [P, P, P, ctypes.c_int32, G, P, P, P, ctypes.c_float, P, P,
                                     ctypes.POINTER(bsa_forward_options), P]
        L.bsa_forward_split.argtypes = [P, P, P, ctypes.c_int32, G, P, P, P, ctypes.c_float, P, P,
                                        ctypes.POINTER(bsa_forward_options), ctypes.c_int32, P, ctypes.c_int64, P]
        L.bsa_forward_split_static.argtypes = [P, P, P, ctypes.c_int32, G, P, P, P, ctypes.c_float, P, P,
                                               ctypes.POINTER(bsa_forward_options), ctypes.c_int32, P]
        L.bsa_forward_split_workspace_bytes.argtypes = [G, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
        L.bsa_cluster_importance.argtypes = [P, ctypes.c_int32, P, G, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, P, P]
        L.bsa_select_blocks.argtypes = [P, G, M, P, P, P, P, P]
        L.bsa_top_p_workspace_bytes.argtypes = [G, ctypes.POINTER(ctypes.c_int64)]
        L.bsa_select_top_p.argtypes = [P, P, G, ctypes.POINTER(bsa_topp_params), P, P, ctypes.c_int64,
                                       P, P, P, P]
        L.bsa_frame_scores.argtypes = [P, G, ctypes.c_int32, P, P]
        L.bsa_classify_heads.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
        L.bsa_structured_lists.argtypes = [P, G, ctypes.POINTER(bsa_struct_params), P, P, P, P]
        for f in ("bsa_derive", "bsa_pool_blocks", "bsa_pool_qk", "bsa_build_mask", "bsa_forward", "bsa_forward_ex",
                  "bsa_forward_split", "bsa_forward_split_workspace_bytes", "bsa_forward_split_static",
                  "bsa_abi_version",
                  "bsa_cluster_importance", "bsa_select_blocks", "bsa_top_p_workspace_bytes",
                  "bsa_select_top_p", "bsa_frame_scores", "bsa_classify_heads", "bsa_structured_lists"):
            getattr(L, f).restype = ctypes.c_int32
        L.bsa_status_string.argtypes = [ctypes.c_int32]
        L.bsa_status_string.restype = ctypes.c_char_p
        L.bsa_last_error.argtypes = []
        L.bsa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


class BsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{lib().bsa_status_string(status).decode()}: {message}")
        self.status = status


def check(status):
    if status != BSA_OK:
        raise BsaError(status, lib().bsa_last_error().decode())
