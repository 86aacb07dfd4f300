"""ctypes binding of libpkvspec.so (include/pkv_spec.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory (tensor.data_ptr()) and streams
(torch.cuda.current_stream().cuda_stream).  There is no fallback: if the
shared library is missing, importing this module raises.
"""
import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkvspec.so")

PKV_OK = 0
STATUS_NAMES = {
    0: "PKV_OK", 1: "PKV_ERR_INVALID_ARG", 2: "PKV_ERR_OUT_OF_PAGES", 3: "PKV_ERR_UNKNOWN_SEQ",
    4: "PKV_ERR_SEQ_EXISTS", 5: "PKV_ERR_UNSUPPORTED", 6: "PKV_ERR_DEVICE",
    7: "PKV_ERR_WORKSPACE", 8: "PKV_ERR_NO_SLOT", 9: "PKV_ERR_CAPACITY",
}
F32, BF16, FP8_E4M3, FP8_E4M3_MX64 = 0, 1, 2, 3
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp8mx": FP8_E4M3_MX64}


class PkvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class OutOfPages(PkvError):
    pass


class PoolDesc(C.Structure):
    _fields_ = [
        ("num_pages", C.c_int32), ("page_size", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("kv_dtype", C.c_int), ("max_seqs", C.c_int32),
        ("max_pages_per_seq", C.c_int32), ("k_pages", C.c_void_p), ("v_pages", C.c_void_p),
        ("k_scale", C.c_void_p), ("v_scale", C.c_void_p), ("block_table", C.c_void_p),
        ("seq_lens", C.c_void_p), ("free_order", C.POINTER(C.c_int32)),
    ]


class PoolStats(C.Structure):
    _fields_ = [
        ("free_pages", C.c_int32), ("used_pages", C.c_int32), ("shared_pages", C.c_int32),
        ("num_seqs", C.c_int32), ("cow_copies", C.c_int64), ("used_token_slots", C.c_int64),
    ]


class VerifyArgs(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("n_q", C.c_int32), ("num_q_heads", C.c_int32),
        ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("page_size", C.c_int32),
        ("q_dtype", C.c_int), ("kv_dtype", C.c_int), ("q", C.c_void_p),
        ("k_pages", C.c_void_p), ("v_pages", C.c_void_p), ("k_scale", C.c_void_p),
        ("v_scale", C.c_void_p), ("block_table", C.c_void_p), ("block_table_stride", C.c_int32),
        ("seq_lens", C.c_void_p), ("batch_slots", C.c_void_p), ("anc_mask", C.c_void_p),
        ("sm_scale", C.c_float), ("out", C.c_void_p), ("lse", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("num_splits", C.c_int32),
        ("n_q_seq", C.c_void_p), ("shared_prefix_pages", C.c_int32),
    ]


class AcceptArgs(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("gamma", C.c_int32), ("vocab", C.c_int32),
        ("target_logits", C.c_void_p), ("draft_logits", C.c_void_p),
        ("draft_tokens", C.c_void_p), ("seed", C.c_uint64), ("step", C.c_uint32),
        ("accepted_len", C.c_void_p), ("next_token", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("gammas", C.c_void_p),
        ("step_ptr", C.c_void_p),
    ]


class TreeAcceptArgs(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("n_nodes", C.c_int32), ("max_children", C.c_int32),
        ("vocab", C.c_int32), ("target_logits", C.c_void_p), ("draft_logits", C.c_void_p),
        ("parents", C.c_void_p), ("tokens", C.c_void_p), ("seed", C.c_uint64), ("step", C.c_uint32),
        ("accepted_len", C.c_void_p), ("accepted_nodes", C.c_void_p), ("next_token", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("step_ptr", C.c_void_p),
    ]


EXPORTS = {
    # name: (restype, argtypes)
    "pkv_page_bytes": (C.c_int64, [C.c_int, C.c_int32, C.c_int32]),
    "pkv_pool_create": (C.c_int, [C.POINTER(PoolDesc), C.POINTER(C.c_void_p)]),
    "pkv_pool_destroy": (None, [C.c_void_p]),
    "paged_kv_alloc": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int32,
                                 C.POINTER(C.c_int32), C.c_void_p]),
    # int64_t* seqs and int32_t* n_tokens are passed as addresses
    "paged_kv_append": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_int, C.c_void_p]),
    "paged_kv_rollback": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "paged_kv_release": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p]),
    "paged_kv_commit_path": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p]),
    "paged_kv_block_table": (C.c_int, [C.c_void_p, C.c_int64, C.POINTER(C.c_int32), C.c_int32,
                                       C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                       C.POINTER(C.c_int32)]),
    "paged_kv_stats": (C.c_int, [C.c_void_p, C.POINTER(PoolStats)]),
    "paged_kv_page_refcount": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32)]),
    "spec_tree_ancestor_masks": (C.c_int, [C.c_int32, C.POINTER(C.c_int32),
                                           C.POINTER(C.c_uint64)]),
    "spec_verify_workspace_size": (C.c_int, [C.POINTER(VerifyArgs), C.POINTER(C.c_size_t)]),
    "spec_verify_attention": (C.c_int, [C.POINTER(VerifyArgs), C.c_void_p]),
    "spec_verify_attention_static": (C.c_int, [C.POINTER(VerifyArgs), C.c_void_p]),
    "pkv_page_read_probe": (C.c_int, [C.POINTER(VerifyArgs), C.c_void_p, C.c_int32, C.c_void_p]),
    "spec_verify_attention_append": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                               C.POINTER(VerifyArgs), C.c_void_p]),
    "spec_accept_workspace_size": (C.c_int, [C.POINTER(AcceptArgs), C.POINTER(C.c_size_t)]),
    "spec_accept": (C.c_int, [C.POINTER(AcceptArgs), C.c_void_p]),
    "spec_accept_tree_workspace_size": (C.c_int, [C.POINTER(TreeAcceptArgs), C.POINTER(C.c_size_t)]),
    "spec_accept_tree": (C.c_int, [C.POINTER(TreeAcceptArgs), C.c_void_p]),
    "pkv_status_string": (C.c_char_p, [C.c_int]),
    "pkv_last_error": (C.c_char_p, []),
    "pkv_version": (C.c_char_p, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python paged_kv_speculative_amd/csrc/build.py` (there is no fallback)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def check(status):
    if status != PKV_OK:
        msg = lib.pkv_last_error().decode()
        if status == 2:
            raise OutOfPages(status, msg)
        raise PkvError(status, msg)


def i64_array(values):
    values = [int(v) for v in values]
    return (C.c_int64 * max(1, len(values)))(*values)


def i32_array(values):
    values = [int(v) for v in values]
    return (C.c_int32 * max(1, len(values)))(*values)
