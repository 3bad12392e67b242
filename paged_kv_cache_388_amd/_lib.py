"""ctypes binding of libpagedkv (include/pagedkv.h).

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked on the host, then the C entry point of the same name is called with
raw device pointers and torch's current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library is missing this module raises on first use.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}
_STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EWORKSPACE",
           4: "PKV_EHIP", 5: "PKV_ECHECK"}


class PkvPool(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class PagedKVError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load():
    """Load libpagedkv.so (built by paged_kv_cache_388_amd.build) once."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_388_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i32, c_sz, c_vp, c_f = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    lib.pkv_partition_tokens.argtypes = []
    lib.pkv_partition_tokens.restype = c_i32
    lib.paged_kv_append.argtypes = [c_vp, c_vp, c_vp, c_vp, PkvPool, c_vp, c_i32, c_vp]
    lib.paged_kv_append.restype = c_i32
    lib.paged_attention_workspace_bytes.argtypes = [PkvPool, c_i32, c_i32, c_i32]
    lib.paged_attention_workspace_bytes.restype = c_sz
    lib.paged_attention_decode.argtypes = [c_vp, c_vp, c_vp, c_vp, PkvPool, c_vp, c_i32, c_vp,
                                           c_i32, c_i32, c_f, c_i32, c_vp, c_sz, c_vp]
    lib.paged_attention_decode.restype = c_i32
    lib.paged_attention_decode_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, PkvPool, c_vp, c_i32,
                                                   c_vp, c_i32, c_i32, c_f, c_i32, c_vp]
    lib.paged_attention_decode_noalloc.restype = c_i32
    lib.paged_attention_noalloc_max_bytes.argtypes = []
    lib.paged_attention_noalloc_max_bytes.restype = c_sz
    lib.paged_attention_multi_workspace_bytes.argtypes = [PkvPool, c_i32, c_i32, c_i32, c_i32]
    lib.paged_attention_multi_workspace_bytes.restype = c_sz
    lib.paged_attention_multi.argtypes = [c_vp, c_vp, c_vp, c_vp, PkvPool, c_vp, c_i32, c_vp, c_vp,
                                          c_i32, c_i32, c_i32, c_i32, c_f, c_i32, c_vp, c_sz, c_vp]
    lib.paged_attention_multi.restype = c_i32
    lib.paged_copy_blocks.argtypes = [c_vp, c_vp, PkvPool, c_vp, c_i32, c_vp]
    lib.paged_copy_blocks.restype = c_i32
    lib.paged_swap_out.argtypes = [c_vp, c_vp, PkvPool, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]
    lib.paged_swap_out.restype = c_i32
    lib.paged_swap_in.argtypes = [c_vp, c_i32, c_vp, c_vp, PkvPool, c_vp, c_vp, c_sz, c_vp]
    lib.paged_swap_in.restype = c_i32
    lib.pkv_stream_copy.argtypes = [c_vp, c_vp, c_sz, c_vp]
    lib.pkv_stream_copy.restype = c_i32
    lib.pkv_stream_read.argtypes = [c_vp, c_sz, c_vp, c_vp]
    lib.pkv_stream_read.restype = c_i32
    lib.pkv_stream_reread.argtypes = [c_vp, c_sz, c_i32, c_vp, c_vp]
    lib.pkv_stream_reread.restype = c_i32
    lib.pkv_clock_records.argtypes = []
    lib.pkv_clock_records.restype = c_i32
    lib.pkv_clock_read.argtypes = [c_vp, c_sz]
    lib.pkv_clock_read.restype = c_i32
    lib.pkv_status_string.argtypes = [c_i32]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise PagedKVError(status, load().pkv_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _scratch(nbytes, device, stream):
    """Uninitialised device bytes for a call that runs on ``stream`` (None:
    the current stream).  Allocated while that stream is current, so the
    caching allocator hands the memory to other work only once that stream
    has passed the call's kernels."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    with torch.cuda.stream(s):
        return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, dim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")


def pool_of(k_cache):
    """PkvPool describing a [num_blocks, H_kv, block_size, D] cache tensor."""
    if k_cache.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported cache dtype {k_cache.dtype}")
    nb, hkv, bs, d = k_cache.shape
    return PkvPool(nb, hkv, bs, d, _DTYPE_CODE[k_cache.dtype])


def _pools(k_cache, v_cache):
    _need(k_cache, "k_cache", dim=4)
    _need(v_cache, "v_cache", dtype=k_cache.dtype, dim=4, device=k_cache.device)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    return pool_of(k_cache)


def partition_tokens():
    return int(load().pkv_partition_tokens())


def paged_kv_append(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Write key/value [T, H_kv, D] into the slots named by slot_mapping [T] (int32)."""
    pool = _pools(k_cache, v_cache)
    for t, n in ((key, "key"), (value, "value")):
        _need(t, n, dtype=k_cache.dtype, dim=3, device=k_cache.device)
        if t.shape[1:] != k_cache.shape[1:2] + k_cache.shape[3:]:
            raise ValueError(f"{n} must be [T, H_kv, D] matching the pool")
    _need(slot_mapping, "slot_mapping", dtype=torch.int32, dim=1, device=k_cache.device)
    T = slot_mapping.shape[0]
    if key.shape[0] != T or value.shape[0] != T:
        raise ValueError("key, value and slot_mapping disagree on the token count")
    _check(load().paged_kv_append(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), pool,
                                  _ptr(slot_mapping), T, _stream(stream)))


def paged_attention_workspace_bytes(k_cache, num_seqs, num_q_heads, max_context_len):
    """Workspace bytes paged_attention_decode needs for this pool and batch
    on the current device."""
    return int(load().paged_attention_workspace_bytes(pool_of(k_cache), int(num_seqs),
                                                      int(num_q_heads), int(max_context_len)))


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           max_context_len, workspace=None, stream=None):
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over each sequence's
    paged context.  max_context_len is a host-side upper bound of
    context_lens.  workspace: a uint8 device tensor of at least
    paged_attention_workspace_bytes(k_cache, ...) bytes, or None to allocate one."""
    pool = _pools(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", dtype=k_cache.dtype, dim=3, device=dev)
    _need(out, "out", dtype=k_cache.dtype, dim=3, device=dev)
    if out.shape != q.shape or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q/out must be [B, H_q, D] with the pool's D")
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    B, Hq, D = q.shape
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens disagree with q on num_seqs")
    need = paged_attention_workspace_bytes(k_cache, B, Hq, int(max_context_len))
    if workspace is None:
        workspace = _scratch(need, dev, stream)
    else:
        _need(workspace, "workspace", device=dev)
    _check(load().paged_attention_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), pool, _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), B, Hq, float(scale), int(max_context_len),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def paged_attention_noalloc_max_bytes():
    """Bytes of the per-GPU scratch array paged_attention_decode_noalloc uses."""
    return int(load().paged_attention_noalloc_max_bytes())


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   max_context_len, stream=None):
    """paged_attention_decode with no workspace argument: the library takes
    the workspace from its own per-GPU scratch array and allocates nothing.
    Calls that overlap on one GPU share that array and race."""
    pool = _pools(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", dtype=k_cache.dtype, dim=3, device=dev)
    _need(out, "out", dtype=k_cache.dtype, dim=3, device=dev)
    if out.shape != q.shape or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q/out must be [B, H_q, D] with the pool's D")
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    B, Hq, D = q.shape
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens disagree with q on num_seqs")
    _check(load().paged_attention_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), pool, _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), B, Hq, float(scale), int(max_context_len),
        _stream(stream)))
    return out


def paged_attention_multi_workspace_bytes(k_cache, num_seqs, num_q_heads, max_query_len,
                                          max_context_len):
    """Workspace bytes paged_attention_multi needs on the current device (0 if
    the call would be refused)."""
    return int(load().paged_attention_multi_workspace_bytes(
        pool_of(k_cache), int(num_seqs), int(num_q_heads), int(max_query_len),
        int(max_context_len)))


def paged_attention_multi(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                          scale, max_context_len, max_query_len, workspace=None, stream=None):
    """Several new tokens per sequence: q/out [T, H_q, D] packed by sequence,
    query_start [B + 1] int32 (rows of sequence s are query_start[s] ..
    query_start[s+1] - 1; they are the last tokens of its context_lens[s])."""
    pool = _pools(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", dtype=k_cache.dtype, dim=3, device=dev)
    _need(out, "out", dtype=k_cache.dtype, dim=3, device=dev)
    if out.shape != q.shape or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q/out must be [T, H_q, D] with the pool's D")
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    _need(query_start, "query_start", dtype=torch.int32, dim=1, device=dev)
    B = context_lens.shape[0]
    T, Hq, _ = q.shape
    if block_tables.shape[0] != B or query_start.shape[0] != B + 1:
        raise ValueError("block_tables [B, *], context_lens [B], query_start [B + 1] disagree")
    need = paged_attention_multi_workspace_bytes(k_cache, B, Hq, max_query_len, max_context_len)
    if workspace is None:
        workspace = _scratch(need, dev, stream)
    else:
        _need(workspace, "workspace", device=dev)
    _check(load().paged_attention_multi(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), pool, _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(query_start), B, Hq, T,
        int(max_query_len), float(scale), int(max_context_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def paged_copy_blocks(k_cache, v_cache, block_mapping, stream=None):
    """Copy block src -> dst (every head, K and V) for each row of block_mapping [N, 2]."""
    pool = _pools(k_cache, v_cache)
    _need(block_mapping, "block_mapping", dtype=torch.int32, dim=2, device=k_cache.device)
    if block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [N, 2]")
    _check(load().paged_copy_blocks(_ptr(k_cache), _ptr(v_cache), pool, _ptr(block_mapping),
                                    block_mapping.shape[0], _stream(stream)))


SWAP_STAGING_BYTES = 64 << 20


def _swap_args(k_cache, v_cache, block_ids, staging, stream):
    pool = _pools(k_cache, v_cache)
    _need(block_ids, "block_ids", dtype=torch.int32, dim=1, device=k_cache.device)
    entry = 2 * k_cache[0].numel() * k_cache.element_size()
    n = block_ids.shape[0]
    if staging is None:
        nbytes = min(max(n, 1) * entry, max(entry, SWAP_STAGING_BYTES // entry * entry))
        staging = _scratch(nbytes, k_cache.device, stream)
    else:
        _need(staging, "staging", device=k_cache.device)
    return pool, n, (n, 2) + tuple(k_cache.shape[1:]), staging


def _need_host(t, name, dtype, shape):
    if not isinstance(t, torch.Tensor) or t.is_cuda:
        raise ValueError(f"{name} must be a host tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def paged_swap_out(k_cache, v_cache, block_ids, host_image=None, staging=None, stream=None):
    """Copy the listed blocks to a host image [n, 2, H_kv, bs, D] (entry i:
    block_ids[i]'s K then V).  Allocates a pinned image when none is given.
    Asynchronous: the image is complete once the stream is synchronized."""
    pool, n, shape, staging = _swap_args(k_cache, v_cache, block_ids, staging, stream)
    if host_image is None:
        host_image = torch.empty(shape, dtype=k_cache.dtype, pin_memory=True)
    _need_host(host_image, "host_image", k_cache.dtype, shape)
    _check(load().paged_swap_out(_ptr(k_cache), _ptr(v_cache), pool, _ptr(block_ids), n,
                                 _ptr(host_image), _ptr(staging),
                                 staging.numel() * staging.element_size(), _stream(stream)))
    return host_image


def paged_swap_in(host_image, k_cache, v_cache, block_ids, staging=None, stream=None):
    """Write entry i of a host image into block block_ids[i] of both pools
    (distinct destinations).  The host image must stay untouched until the
    stream has reached the end of the call."""
    pool, n, shape, staging = _swap_args(k_cache, v_cache, block_ids, staging, stream)
    _need_host(host_image, "host_image", k_cache.dtype, shape)
    _check(load().paged_swap_in(_ptr(host_image), n, _ptr(k_cache), _ptr(v_cache), pool,
                                _ptr(block_ids), _ptr(staging),
                                staging.numel() * staging.element_size(), _stream(stream)))


def pkv_stream_copy(dst, src, stream=None):
    """Plain 16-byte-vector device copy of src into dst (same byte size)."""
    _need(dst, "dst")
    _need(src, "src", device=dst.device)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src differ in size")
    _check(load().pkv_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))


STREAM_READ_WORKGROUPS = 2048


def pkv_stream_read(src, sink, stream=None):
    """Read every byte of src once; sink is an int32/uint32 device tensor of
    at least 2048 elements that receives one XOR-fold word per workgroup."""
    _need(src, "src")
    _need(sink, "sink", device=src.device)
    if sink.numel() * sink.element_size() < 4 * STREAM_READ_WORKGROUPS:
        raise ValueError("sink must hold 2048 32-bit words")
    _check(load().pkv_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                  _stream(stream)))


def pkv_stream_reread(src, rounds, sink, stream=None):
    """Read every byte of src ``rounds`` times, each XCD re-reading only its
    own eighth of it (the L2 / Infinity Cache read ceilings); sink as for
    pkv_stream_read."""
    _need(src, "src")
    _need(sink, "sink", device=src.device)
    if sink.numel() * sink.element_size() < 4 * STREAM_READ_WORKGROUPS:
        raise ValueError("sink must hold 2048 32-bit words")
    _check(load().pkv_stream_reread(_ptr(src), src.numel() * src.element_size(), int(rounds),
                                    _ptr(sink), _stream(stream)))


def pkv_clock_read(records=None):
    """The clock records of the last attention call made with
    PAGEDKV_CLOCK=1 on the current device (waits for the device): a uint64
    array [records, 4], zeros where nothing was recorded."""
    import numpy as np
    lib = load()
    n = lib.pkv_clock_records() if records is None else int(records)
    buf = np.zeros((max(n, 0), 4), dtype=np.uint64)
    _check(lib.pkv_clock_read(buf.ctypes.data_as(ctypes.c_void_p), n))
    return buf


# ---------------------------------------------------------------------------
# host block manager (pkv_bm_*)
# ---------------------------------------------------------------------------

class PkvBmStats(ctypes.Structure):
    _fields_ = [("blocks_in_use", ctypes.c_int64), ("tokens_stored", ctypes.c_int64),
                ("slots_reserved", ctypes.c_int64), ("cached_blocks", ctypes.c_int64),
                ("free_blocks", ctypes.c_int64), ("num_sequences", ctypes.c_int64)]


def _bm_lib():
    lib = load()
    if getattr(lib, "_bm_ready", False):
        return lib
    c_i32, c_i64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.pkv_bm_create.argtypes = [c_i32, c_i32, c_i32]
    lib.pkv_bm_create.restype = c_vp
    lib.pkv_bm_destroy.argtypes = [c_vp]
    lib.pkv_bm_destroy.restype = None
    lib.pkv_bm_last_error.argtypes = []
    lib.pkv_bm_last_error.restype = ctypes.c_char_p
    lib.pkv_bm_num_free_blocks.argtypes = [c_vp]
    lib.pkv_bm_num_free_blocks.restype = c_i32
    lib.pkv_bm_add_sequence.argtypes = [c_vp, c_i64, c_vp, c_i32, c_vp, c_vp]
    lib.pkv_bm_add_sequence.restype = c_i32
    lib.pkv_bm_append.argtypes = [c_vp, c_i64, c_vp, c_i32, c_vp, c_vp, c_vp]
    lib.pkv_bm_append.restype = c_i32
    lib.pkv_bm_append_step.argtypes = [c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp]
    lib.pkv_bm_append_step.restype = c_i32
    lib.pkv_bm_swap_out.argtypes = [c_vp, c_i64, c_vp, c_i32, c_vp]
    lib.pkv_bm_swap_out.restype = c_i32
    lib.pkv_bm_swap_in.argtypes = [c_vp, c_i64, c_vp, c_i32, c_vp]
    lib.pkv_bm_swap_in.restype = c_i32
    lib.pkv_bm_fork.argtypes = [c_vp, c_i64, c_i64]
    lib.pkv_bm_fork.restype = c_i32
    lib.pkv_bm_free_sequence.argtypes = [c_vp, c_i64]
    lib.pkv_bm_free_sequence.restype = c_i32
    lib.pkv_bm_sequence_info.argtypes = [c_vp, c_i64, c_vp, c_vp]
    lib.pkv_bm_sequence_info.restype = c_i32
    lib.pkv_bm_build_batch.argtypes = [c_vp, c_vp, c_i32, c_vp, c_i32, c_vp]
    lib.pkv_bm_build_batch.restype = c_i32
    lib.pkv_bm_get_stats.argtypes = [c_vp, ctypes.POINTER(PkvBmStats)]
    lib.pkv_bm_get_stats.restype = c_i32
    lib._bm_ready = True
    return lib


class BlockManager:
    """The library's host block manager (pkv_bm_* in include/pagedkv.h).
    Host-side only: it hands out slots, copy-on-write pairs and block tables
    for the device calls.  Methods raise PagedKVError (status PKV_EWORKSPACE
    when the pool is exhausted, nothing changed)."""

    def __init__(self, num_blocks, block_size, prefix_cache=True):
        import numpy as np
        self._np = np
        self._lib = _bm_lib()
        self._h = self._lib.pkv_bm_create(int(num_blocks), int(block_size), int(bool(prefix_cache)))
        if not self._h:
            raise PagedKVError(1, self._lib.pkv_bm_last_error().decode())
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _ok(self, status):
        if status != 0:
            raise PagedKVError(status, self._lib.pkv_bm_last_error().decode())

    def _i32(self, a):
        return self._np.ascontiguousarray(a, dtype=self._np.int32)

    def num_free(self):
        return int(self._lib.pkv_bm_num_free_blocks(self._h))

    def add_sequence(self, seq_id, tokens):
        """Returns (reused leading tokens, slots [n] int32 with -1 where reused)."""
        t = self._i32(tokens)
        slots = self._np.empty(len(t), dtype=self._np.int32)
        reused = ctypes.c_int32(0)
        self._ok(self._lib.pkv_bm_add_sequence(self._h, int(seq_id), t.ctypes.data, len(t),
                                               ctypes.byref(reused), slots.ctypes.data))
        return int(reused.value), slots

    def append(self, seq_id, tokens):
        """Returns (slots [k] int32, (src, dst) copy-on-write pair or None)."""
        t = self._i32(tokens)
        slots = self._np.empty(len(t), dtype=self._np.int32)
        cow = self._np.zeros(2, dtype=self._np.int32)
        ncow = ctypes.c_int32(0)
        self._ok(self._lib.pkv_bm_append(self._h, int(seq_id), t.ctypes.data, len(t),
                                         slots.ctypes.data, cow.ctypes.data, ctypes.byref(ncow)))
        return slots, ((int(cow[0]), int(cow[1])) if ncow.value else None)

    def append_step(self, seq_ids, tokens):
        """One token per listed sequence.  Returns (slots [B] int32,
        copy-on-write pairs [k, 2] int32 in order)."""
        ids = self._np.ascontiguousarray(seq_ids, dtype=self._np.int64)
        t = self._i32(tokens)
        if len(t) != len(ids):
            raise ValueError("one token per sequence")
        slots = self._np.empty(len(ids), dtype=self._np.int32)
        cows = self._np.empty((len(ids), 2), dtype=self._np.int32)
        ncow = ctypes.c_int32(0)
        self._ok(self._lib.pkv_bm_append_step(self._h, ids.ctypes.data, len(ids), t.ctypes.data,
                                              slots.ctypes.data, cows.ctypes.data,
                                              ctypes.byref(ncow)))
        return slots, cows[:ncow.value]

    def _swap(self, fn, seq_id):
        n, _ = self.sequence_info(seq_id)
        cap = -(-n // self.block_size)
        ids = self._np.empty(max(cap, 1), dtype=self._np.int32)
        got = ctypes.c_int32(0)
        self._ok(fn(self._h, int(seq_id), ids.ctypes.data, cap, ctypes.byref(got)))
        return ids[:got.value]

    def swap_out(self, seq_id):
        """Release the sequence's blocks; returns them (int32, table order),
        the blocks to copy to host memory before anything reuses them."""
        return self._swap(self._lib.pkv_bm_swap_out, seq_id)

    def swap_in(self, seq_id):
        """Fresh blocks for a swapped-out sequence (int32, table order), the
        destinations of its host copy."""
        return self._swap(self._lib.pkv_bm_swap_in, seq_id)

    def fork(self, parent, child):
        self._ok(self._lib.pkv_bm_fork(self._h, int(parent), int(child)))

    def free_sequence(self, seq_id):
        self._ok(self._lib.pkv_bm_free_sequence(self._h, int(seq_id)))

    def sequence_info(self, seq_id):
        n, nb = ctypes.c_int32(0), ctypes.c_int32(0)
        self._ok(self._lib.pkv_bm_sequence_info(self._h, int(seq_id), ctypes.byref(n),
                                                ctypes.byref(nb)))
        return int(n.value), int(nb.value)

    def build_batch(self, seq_ids, max_blocks_per_seq):
        """Returns (block_tables [B, max_blocks] int32, context_lens [B] int32)."""
        ids = self._np.ascontiguousarray(seq_ids, dtype=self._np.int64)
        bt = self._np.empty((len(ids), int(max_blocks_per_seq)), dtype=self._np.int32)
        lens = self._np.empty(len(ids), dtype=self._np.int32)
        self._ok(self._lib.pkv_bm_build_batch(self._h, ids.ctypes.data, len(ids), bt.ctypes.data,
                                              int(max_blocks_per_seq), lens.ctypes.data))
        return bt, lens

    def stats(self):
        st = PkvBmStats()
        self._ok(self._lib.pkv_bm_get_stats(self._h, ctypes.byref(st)))
        d = {k: int(getattr(st, k)) for k, _ in PkvBmStats._fields_}
        d["waste"] = ((d["slots_reserved"] - d["tokens_stored"]) / d["slots_reserved"]
                      if d["slots_reserved"] else 0.0)
        return d
