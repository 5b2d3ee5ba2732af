"""Thin ctypes binding of libkvq2 (argument marshalling only).

Every step of the path runs in the library: this module turns torch tensors
(device memory and streams) or numpy arrays (calibration, host memory) into
the plain pointers of the C ABI declared in include/kvq2.h, and raises on a
non-zero status.  It loads only the in-tree libkvq2.so and fails loudly if it
is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq2.so")
_lib = None

HEAD_DIM = 128
CHUNK_TOKENS = 16
CHUNK_BYTES = 1152


class KvqError(RuntimeError):
    pass


class KvqDims(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_size", C.c_int32), ("n_sink", C.c_int32), ("n_recent", C.c_int32),
                ("sm_scale", C.c_float), ("quant_group", C.c_int32),
                ("hadamard_block", C.c_int32)]


class KvqLayer(C.Structure):
    _fields_ = [("R_K", C.c_void_p), ("R_V", C.c_void_p), ("clip_K", C.c_float),
                ("clip_V", C.c_float)]


class KvqCache(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("num_pages", C.c_int64), ("sink", C.c_void_p),
                ("recent", C.c_void_p), ("block_table", C.c_void_p), ("bt_stride", C.c_int32)]


class KvqPrefixGroups(C.Structure):
    _fields_ = [("n_groups", C.c_int32), ("n_members", C.c_int32), ("member_start", C.c_void_p),
                ("members", C.c_void_p), ("prefix_len", C.c_void_p)]


class KvqHqmqDims(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_size", C.c_int32), ("n_secondary", C.c_int32), ("sm_scale", C.c_float)]


class KvqHqmqLayer(C.Structure):
    _fields_ = [("codebook_K", C.c_void_p), ("codebook_V", C.c_void_p)]


class KvqHqmqCache(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("num_pages", C.c_int64), ("block_table", C.c_void_p),
                ("bt_stride", C.c_int32)]


HQMQ_EXPORTS = ("kvq_hqmq_codebook", "kvq_hqmq_append_workspace_bytes", "kvq_hqmq_append",
                "kvq_hqmq_decode_workspace_bytes", "kvq_hqmq_decode_attention")
HQMQ_TOKEN_BYTES = 192            # K and V records of one (position, KV head)

EXPORTS = ("kvq_calibrate", "kvq_quantize_append", "kvq_decode_workspace_bytes",
           "kvq_decode_attention", "kvq_decode_multi_workspace_bytes",
           "kvq_decode_multi_attention", "kvq_decode_attention_noalloc", "kvq_decode_step",
           "kvq_decode_prefix_workspace_bytes", "kvq_decode_prefix_attention",
           "kvq_status_string", "kvq_last_error")
PROBE_EXPORTS = ("kvq_probe_stream_read", "kvq_probe_chunk_read")


def lib():
    """The loaded libkvq2 (raises if the in-tree build is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise KvqError(f"libkvq2 is not built ({_LIB_PATH} missing): run "
                           "python -m long_context_decode_kvq_amd.build")
        L = C.CDLL(_LIB_PATH)
        P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.kvq_calibrate.argtypes = [C.POINTER(KvqDims), I32, P, P, P, C.c_double, P, P, P, P]
        L.kvq_calibrate.restype = C.c_int
        L.kvq_quantize_append.argtypes = [C.POINTER(KvqDims), C.POINTER(KvqLayer),
                                          C.POINTER(KvqCache), I32, P, P, I32, I32, P, P, P]
        L.kvq_quantize_append.restype = C.c_int
        L.kvq_decode_workspace_bytes.argtypes = [C.POINTER(KvqDims), I32, I32]
        L.kvq_decode_workspace_bytes.restype = SZ
        L.kvq_decode_attention.argtypes = [C.POINTER(KvqDims), C.POINTER(KvqLayer),
                                           C.POINTER(KvqCache), I32, P, I32, P, P, P, SZ, P]
        L.kvq_decode_attention.restype = C.c_int
        L.kvq_decode_multi_workspace_bytes.argtypes = [C.POINTER(KvqDims), I32, I32, I32]
        L.kvq_decode_multi_workspace_bytes.restype = SZ
        L.kvq_decode_multi_attention.argtypes = [C.POINTER(KvqDims), C.POINTER(KvqLayer),
                                                 C.POINTER(KvqCache), I32, P, I32, I32, P, P, P,
                                                 SZ, P]
        L.kvq_decode_multi_attention.restype = C.c_int
        L.kvq_decode_attention_noalloc.argtypes = [C.POINTER(KvqDims), C.POINTER(KvqLayer),
                                                   C.POINTER(KvqCache), I32, P, I32, P, P, P]
        L.kvq_decode_attention_noalloc.restype = C.c_int
        L.kvq_decode_step.argtypes = [C.POINTER(KvqDims), C.POINTER(KvqLayer),
                                      C.POINTER(KvqCache), I32, P, P, I32, I32, P, P, P, I32,
                                      P, P, P, SZ, P]
        L.kvq_decode_step.restype = C.c_int
        L.kvq_decode_prefix_workspace_bytes.argtypes = [C.POINTER(KvqDims), I32, I32,
                                                        C.POINTER(KvqPrefixGroups)]
        L.kvq_decode_prefix_workspace_bytes.restype = SZ
        L.kvq_decode_prefix_attention.argtypes = [C.POINTER(KvqDims), C.POINTER(KvqLayer),
                                                  C.POINTER(KvqCache), I32, P, I32, P, P,
                                                  C.POINTER(KvqPrefixGroups), P, SZ, P]
        L.kvq_decode_prefix_attention.restype = C.c_int
        L.kvq_status_string.argtypes = [C.c_int]
        L.kvq_status_string.restype = C.c_char_p
        L.kvq_last_error.argtypes = []
        L.kvq_last_error.restype = C.c_char_p
        HD, HL, HC = C.POINTER(KvqHqmqDims), C.POINTER(KvqHqmqLayer), C.POINTER(KvqHqmqCache)
        L.kvq_hqmq_codebook.argtypes = [I32, P, P]
        L.kvq_hqmq_codebook.restype = C.c_int
        L.kvq_hqmq_append_workspace_bytes.argtypes = [HD, I32]
        L.kvq_hqmq_append_workspace_bytes.restype = SZ
        L.kvq_hqmq_append.argtypes = [HD, HL, HC, I32, P, P, I32, I32, P, P, P, SZ, P]
        L.kvq_hqmq_append.restype = C.c_int
        L.kvq_hqmq_decode_workspace_bytes.argtypes = [HD, I32, I32]
        L.kvq_hqmq_decode_workspace_bytes.restype = SZ
        L.kvq_hqmq_decode_attention.argtypes = [HD, HL, HC, I32, P, I32, P, P, P, SZ, P]
        L.kvq_hqmq_decode_attention.restype = C.c_int
        L.kvq_probe_stream_read.argtypes = [P, SZ, P, I32, P]
        L.kvq_probe_stream_read.restype = C.c_int
        L.kvq_probe_chunk_read.argtypes = [P, P, I64, P, I32, P]
        L.kvq_probe_chunk_read.restype = C.c_int
        _lib = L
    return _lib


def status_string(rc: int) -> str:
    return lib().kvq_status_string(rc).decode()


def _check(rc: int, what: str):
    if rc != 0:
        extra = lib().kvq_last_error().decode()
        raise KvqError(f"{what}: {status_string(rc)}" + (f" ({extra})" if extra else ""))


def dims(n_q_heads, n_kv_heads, page_size, n_sink, n_recent, sm_scale=0.0, head_dim=HEAD_DIM,
         quant_group=0, hadamard_block=0):
    return KvqDims(n_q_heads, n_kv_heads, head_dim, page_size, n_sink, n_recent, sm_scale,
                   quant_group, hadamard_block)


def chunk_bytes(quant_group: int = 0) -> int:
    """Bytes of one 16-token chunk of the pool for this quantization group size."""
    return 1024 + 128 * (HEAD_DIM // (quant_group or HEAD_DIM))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ calibration (host)

def calibrate(d: KvqDims, q: np.ndarray, k: np.ndarray, v: np.ndarray,
              clip_quantile: float = 0.999):
    """kvq_calibrate on host bf16 arrays (uint16 bit patterns).

    q [N][Hq][128], k/v [N][Hkv][128] -> (R_K, R_V fp32 [Hkv][128][128], clip_K, clip_V).
    """
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    n = q.shape[0]
    R_K = np.zeros((d.n_kv_heads, HEAD_DIM, HEAD_DIM), np.float32)
    R_V = np.zeros_like(R_K)
    cK, cV = C.c_float(0), C.c_float(0)
    rc = lib().kvq_calibrate(C.byref(d), n, _ptr(q), _ptr(k), _ptr(v), float(clip_quantile),
                             _ptr(R_K), _ptr(R_V), C.addressof(cK), C.addressof(cV))
    _check(rc, "kvq_calibrate")
    return R_K, R_V, float(cK.value), float(cV.value)


# ------------------------------------------------------------------ online path (device)

def layer(R_K, R_V, clip_K: float, clip_V: float) -> KvqLayer:
    """R_K / R_V: device fp32 tensors [Hkv][128][128] (kept alive by the caller)."""
    return KvqLayer(_ptr(R_K), _ptr(R_V), clip_K, clip_V)


def cache(pool, num_pages: int, sink, recent, block_table) -> KvqCache:
    return KvqCache(_ptr(pool), num_pages, _ptr(sink), _ptr(recent), _ptr(block_table),
                    int(block_table.shape[1]))


def quantize_append(d: KvqDims, lay: KvqLayer, cch: KvqCache, batch: int, start_pos, cu_new,
                    total_new: int, max_new: int, k_new, v_new, stream=None):
    rc = lib().kvq_quantize_append(C.byref(d), C.byref(lay), C.byref(cch), batch, _ptr(start_pos),
                                   _ptr(cu_new), total_new, max_new, _ptr(k_new), _ptr(v_new),
                                   _stream_handle(stream))
    _check(rc, "kvq_quantize_append")


def decode_workspace_bytes(d: KvqDims, batch: int, max_seq_len: int) -> int:
    return int(lib().kvq_decode_workspace_bytes(C.byref(d), batch, max_seq_len))


def decode_attention(d: KvqDims, lay: KvqLayer, cch: KvqCache, batch: int, seq_len,
                     max_seq_len: int, q, out, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kvq_decode_attention(C.byref(d), C.byref(lay), C.byref(cch), batch, _ptr(seq_len),
                                    max_seq_len, _ptr(q), _ptr(out), _ptr(workspace), nbytes,
                                    _stream_handle(stream))
    _check(rc, "kvq_decode_attention")


def decode_multi_workspace_bytes(d: KvqDims, batch: int, max_seq_len: int, n_query: int) -> int:
    return int(lib().kvq_decode_multi_workspace_bytes(C.byref(d), batch, max_seq_len, n_query))


def decode_multi_attention(d: KvqDims, lay: KvqLayer, cch: KvqCache, batch: int, seq_len,
                           max_seq_len: int, n_query: int, q, out, workspace, stream=None):
    """kvq_decode_multi_attention: q, out [batch][n_query][Hq][128]."""
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kvq_decode_multi_attention(C.byref(d), C.byref(lay), C.byref(cch), batch,
                                          _ptr(seq_len), max_seq_len, n_query, _ptr(q), _ptr(out),
                                          _ptr(workspace), nbytes, _stream_handle(stream))
    _check(rc, "kvq_decode_multi_attention")


def decode_attention_noalloc(d: KvqDims, lay: KvqLayer, cch: KvqCache, batch: int, seq_len,
                             max_seq_len: int, q, out, stream=None):
    """kvq_decode_attention_noalloc: the decode with the library's own scratch."""
    rc = lib().kvq_decode_attention_noalloc(C.byref(d), C.byref(lay), C.byref(cch), batch,
                                            _ptr(seq_len), max_seq_len, _ptr(q), _ptr(out),
                                            _stream_handle(stream))
    _check(rc, "kvq_decode_attention_noalloc")


def decode_step(d: KvqDims, lay: KvqLayer, cch: KvqCache, batch: int, start_pos, cu_new,
                total_new: int, max_new: int, k_new, v_new, seq_len, max_seq_len: int, q, out,
                workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kvq_decode_step(C.byref(d), C.byref(lay), C.byref(cch), batch, _ptr(start_pos),
                               _ptr(cu_new), total_new, max_new, _ptr(k_new), _ptr(v_new),
                               _ptr(seq_len), max_seq_len, _ptr(q), _ptr(out), _ptr(workspace),
                               nbytes, _stream_handle(stream))
    _check(rc, "kvq_decode_step")


def prefix_groups(n_members: int, member_start=None, members=None, prefix_len=None
                  ) -> KvqPrefixGroups:
    """kvq_prefix_groups over device int32 tensors (member_start has
    n_groups + 1 entries); keep the tensors alive while it is used."""
    n_groups = 0 if member_start is None else int(member_start.numel()) - 1
    return KvqPrefixGroups(n_groups, n_members, _ptr(member_start), _ptr(members),
                           _ptr(prefix_len))


def decode_prefix_workspace_bytes(d: KvqDims, batch: int, max_seq_len: int,
                                  groups: KvqPrefixGroups) -> int:
    return int(lib().kvq_decode_prefix_workspace_bytes(C.byref(d), batch, max_seq_len,
                                                       C.byref(groups)))


def decode_prefix_attention(d: KvqDims, lay: KvqLayer, cch: KvqCache, batch: int, seq_len,
                            max_seq_len: int, q, out, groups: KvqPrefixGroups, workspace,
                            stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kvq_decode_prefix_attention(C.byref(d), C.byref(lay), C.byref(cch), batch,
                                           _ptr(seq_len), max_seq_len, _ptr(q), _ptr(out),
                                           C.byref(groups), _ptr(workspace), nbytes,
                                           _stream_handle(stream))
    _check(rc, "kvq_decode_prefix_attention")


# ------------------------------------------------------------------ HQMQ codec (kvq2_hqmq.h)

def hqmq_dims(n_q_heads, n_kv_heads, page_size, n_secondary, sm_scale=0.0,
              head_dim=HEAD_DIM) -> KvqHqmqDims:
    return KvqHqmqDims(n_q_heads, n_kv_heads, head_dim, page_size, n_secondary, sm_scale)


def hqmq_codebook(secondary: np.ndarray) -> np.ndarray:
    """kvq_hqmq_codebook on host fp32 [S][4] -> fp32 [24 S][4]."""
    sec = np.ascontiguousarray(secondary, np.float32)
    out = np.zeros((24 * sec.shape[0], 4), np.float32)
    _check(lib().kvq_hqmq_codebook(sec.shape[0], _ptr(sec), _ptr(out)), "kvq_hqmq_codebook")
    return out


def hqmq_layer(codebook_K, codebook_V) -> KvqHqmqLayer:
    """Device fp32 tensors [Hkv][24 S][4] (kept alive by the caller)."""
    return KvqHqmqLayer(_ptr(codebook_K), _ptr(codebook_V))


def hqmq_cache(pool, num_pages: int, block_table) -> KvqHqmqCache:
    return KvqHqmqCache(_ptr(pool), num_pages, _ptr(block_table), int(block_table.shape[1]))


def hqmq_append_workspace_bytes(d: KvqHqmqDims, total_new: int) -> int:
    return int(lib().kvq_hqmq_append_workspace_bytes(C.byref(d), total_new))


def hqmq_append(d: KvqHqmqDims, lay: KvqHqmqLayer, cch: KvqHqmqCache, batch: int, start_pos,
                cu_new, total_new: int, max_new: int, k_new, v_new, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kvq_hqmq_append(C.byref(d), C.byref(lay), C.byref(cch), batch, _ptr(start_pos),
                               _ptr(cu_new), total_new, max_new, _ptr(k_new), _ptr(v_new),
                               _ptr(workspace), nbytes, _stream_handle(stream))
    _check(rc, "kvq_hqmq_append")


def hqmq_decode_workspace_bytes(d: KvqHqmqDims, batch: int, max_seq_len: int) -> int:
    return int(lib().kvq_hqmq_decode_workspace_bytes(C.byref(d), batch, max_seq_len))


def hqmq_decode_attention(d: KvqHqmqDims, lay: KvqHqmqLayer, cch: KvqHqmqCache, batch: int,
                          seq_len, max_seq_len: int, q, out, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    rc = lib().kvq_hqmq_decode_attention(C.byref(d), C.byref(lay), C.byref(cch), batch,
                                         _ptr(seq_len), max_seq_len, _ptr(q), _ptr(out),
                                         _ptr(workspace), nbytes, _stream_handle(stream))
    _check(rc, "kvq_hqmq_decode_attention")


class HqmqDeviceCache:
    """Owns the device tensors of one layer's HQMQ cache: pool uint8
    [num_pages][Hkv][P][192], block_table int32 [B][stride], and the append
    workspace (zeroed once, as the library requires)."""

    def __init__(self, d: KvqHqmqDims, num_pages: int, block_table, device="cuda", fill=0):
        import torch
        self.d = d
        self.num_pages = num_pages
        self.pool = torch.full((num_pages, d.n_kv_heads, d.page_size, HQMQ_TOKEN_BYTES), fill,
                               dtype=torch.uint8, device=device)
        self.block_table = torch.as_tensor(np.ascontiguousarray(block_table, np.int32)).to(device)
        self.handle = hqmq_cache(self.pool, num_pages, self.block_table)
        self.append_ws = torch.zeros(hqmq_append_workspace_bytes(d, 0), dtype=torch.uint8,
                                     device=device)


# ------------------------------------------------------------------ read-bandwidth probes

def probe_stream_read(src, sink, work_groups: int, stream=None):
    """kvq_probe_stream_read: one sequential pass over `src` (a device tensor)."""
    nbytes = src.numel() * src.element_size()
    rc = lib().kvq_probe_stream_read(_ptr(src), nbytes, _ptr(sink), work_groups,
                                     _stream_handle(stream))
    _check(rc, "kvq_probe_stream_read")


def probe_chunk_read(pool, chunk_off, sink, work_groups: int, stream=None):
    """kvq_probe_chunk_read: the 1152-byte chunks at byte offsets `chunk_off` (int64 tensor)."""
    rc = lib().kvq_probe_chunk_read(_ptr(pool), _ptr(chunk_off), chunk_off.numel(), _ptr(sink),
                                    work_groups, _stream_handle(stream))
    _check(rc, "kvq_probe_chunk_read")


# ------------------------------------------------------------------ device cache holder

class DeviceCache:
    """Owns the torch device tensors of one layer's paged mixed-precision cache.

    pool uint8 [num_pages][Hkv][P/16][chunk bytes]; sink / recent bf16 bit patterns
    (int16 tensors) [B][Hkv][n][2][128]; block_table int32 [B][stride].
    """

    def __init__(self, d: KvqDims, batch: int, num_pages: int, block_table, device="cuda",
                 fill: int = 0):
        import torch
        self.d = d
        self.batch = batch
        self.num_pages = num_pages
        cpp = d.page_size // CHUNK_TOKENS
        self.pool = torch.full((num_pages, d.n_kv_heads, cpp, chunk_bytes(d.quant_group)), fill,
                               dtype=torch.uint8, device=device)
        fill16 = np.int16(np.uint16(fill * 0x0101).view(np.int16))
        self.sink = torch.full((batch, d.n_kv_heads, max(d.n_sink, 1), 2, HEAD_DIM), int(fill16),
                               dtype=torch.int16, device=device)
        self.recent = torch.full((batch, d.n_kv_heads, d.n_recent, 2, HEAD_DIM), int(fill16),
                                 dtype=torch.int16, device=device)
        self.block_table = torch.as_tensor(np.ascontiguousarray(block_table, np.int32)).to(device)
        self.handle = cache(self.pool, num_pages, self.sink if d.n_sink > 0 else None,
                            self.recent, self.block_table)
