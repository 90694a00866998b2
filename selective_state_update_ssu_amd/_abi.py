"""ctypes mirror of include/ssu.h and include/ssd.h. Field order and types must match the header;
the library checks `struct_size` on every call, so a stale mirror fails loudly."""
import ctypes
import os

from ctypes import c_double, c_int32, c_int64, c_size_t, c_uint32, c_void_p, c_char_p

SSU_F32, SSU_F16, SSU_BF16 = 0, 1, 2
SSU_I32, SSU_I64 = 0, 1
SSU_OK, SSU_ERR_INVALID_ARGUMENT, SSU_ERR_UNSUPPORTED, SSU_ERR_LAUNCH = 0, 1, 2, 3
ABI_VERSION = 1

EXPORTS = ("ssu_one_token", "ssu_packed_varlen", "ssu_ring_update", "ssu_ring_commit",
           "ssu_last_error", "ssu_version", "ssu_ssd_workspace_bytes", "ssu_ssd_prefill",
           "ssu_ssd_prefill_noalloc")


class Operands(ctypes.Structure):
    _fields_ = [
        ("state", c_void_p), ("state_dtype", c_int32),
        ("nslots", c_int64), ("nheads", c_int64), ("headdim", c_int64),
        ("dstate", c_int64), ("ngroups", c_int64),
        ("x", c_void_p), ("B", c_void_p), ("C", c_void_p), ("z", c_void_p),
        ("out", c_void_p), ("io_dtype", c_int32),
        ("dt", c_void_p), ("dt_per_dim", c_int32),
        ("A", c_void_p), ("D", c_void_p), ("dt_bias", c_void_p), ("dt_softplus", c_int32),
        ("pad_slot_id", c_int64), ("disable_state_update", c_int32),
        ("rand_seed", c_void_p), ("philox_rounds", c_int32),
        ("heads_per_block", c_int32), ("loads_per_lane", c_int32), ("tile_order", c_int32),
    ]


class OneTokenArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_uint32), ("op", Operands), ("batch", c_int64),
        ("src_slots", c_void_p), ("src_dtype", c_int32),
        ("dst_slots", c_void_p), ("dst_dtype", c_int32),
    ]


class PackedArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_uint32), ("op", Operands), ("rows", c_int64), ("nseq", c_int64),
        ("cu_seqlens", c_void_p), ("seq_len", c_int64),
        ("num_accepted", c_void_p), ("meta_dtype", c_int32),
        ("src_table", c_void_p), ("src_dtype", c_int32),
        ("src_seq_stride", c_int64), ("src_step_stride", c_int64),
        ("dst_table", c_void_p), ("dst_dtype", c_int32),
        ("dst_seq_stride", c_int64), ("dst_step_stride", c_int64),
        ("steps", c_int64),
    ]


class RingArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_uint32),
        ("ring_start", c_void_p), ("prev_num_accepted", c_void_p), ("prev_query_len", c_void_p),
        ("tracker_dtype", c_int32), ("num_states", c_int64),
        ("slots", c_void_p), ("slot_dtype", c_int32), ("slot_stride", c_int64), ("n", c_int64),
        ("num_accepted", c_void_p), ("query_start_loc", c_void_p), ("meta_dtype", c_int32),
        ("reset", c_int32), ("logical_window", c_int64), ("ring_buffer_len", c_int64),
        ("pad_slot_id", c_int64),
    ]


class SsdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_uint32), ("tokens", c_int64),
        ("nheads", c_int64), ("headdim", c_int64), ("dstate", c_int64), ("ngroups", c_int64),
        ("chunk_size", c_int64), ("nchunks", c_int64), ("batch", c_int64),
        ("x", c_void_p), ("dt", c_void_p), ("A", c_void_p), ("B", c_void_p), ("C", c_void_p),
        ("D", c_void_p), ("z", c_void_p), ("dt_bias", c_void_p),
        ("io_dtype", c_int32), ("dt_dtype", c_int32), ("D_per_dim", c_int32),
        ("dt_softplus", c_int32), ("dt_min", c_double), ("dt_max", c_double),
        ("cu_chunk_seqlens", c_void_p), ("seq_idx", c_void_p), ("last_chunk_indices", c_void_p),
        ("meta_dtype", c_int32), ("state_dtype", c_int32), ("initial_states", c_void_p),
        ("out", c_void_p), ("states", c_void_p), ("return_intermediate_states", c_int32),
        ("reserved", c_int32), ("workspace", c_void_p), ("workspace_bytes", c_size_t),
    ]


def load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: the SSU entry points run only on the HIP library. "
            "Build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(or selective_state_update_ssu_amd/build.py).")
    lib = ctypes.CDLL(path)
    lib.ssu_one_token.restype = c_int32
    lib.ssu_one_token.argtypes = [ctypes.POINTER(OneTokenArgs), c_void_p]
    lib.ssu_packed_varlen.restype = c_int32
    lib.ssu_packed_varlen.argtypes = [ctypes.POINTER(PackedArgs), c_void_p]
    for f in (lib.ssu_ring_update, lib.ssu_ring_commit):
        f.restype = c_int32
        f.argtypes = [ctypes.POINTER(RingArgs), c_void_p]
    lib.ssu_ssd_workspace_bytes.restype = c_size_t
    lib.ssu_ssd_workspace_bytes.argtypes = [c_int64] * 7
    for f in (lib.ssu_ssd_prefill, lib.ssu_ssd_prefill_noalloc):
        f.restype = c_int32
        f.argtypes = [ctypes.POINTER(SsdArgs), c_void_p]
    lib.ssu_last_error.restype = c_char_p
    lib.ssu_last_error.argtypes = []
    lib.ssu_version.restype = c_int32
    lib.ssu_version.argtypes = []
    if lib.ssu_version() != ABI_VERSION:
        raise RuntimeError(f"{path} reports ABI {lib.ssu_version()}, expected {ABI_VERSION}")
    return lib
