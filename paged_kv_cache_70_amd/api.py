"""Python binding of ``libpaged_kv.so`` (the C ABI in ``include/paged_kv.h``).

Argument marshalling only: every step of the write and the decode runs in the
library's HIP kernels.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or no GPU is present, calls
raise.

Functions keep the names of the C entry points without the ``pa_`` prefix:

    write_kv(k_cache, v_cache, k, v, slot_mapping)          -> None (in place)
    decode(q, k_cache, v_cache, block_tables, context_lens, scale, ...) -> out
    decode_partials(...), decode_merge(...)                  the two halves of decode
    prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, ...) -> out
    partition_size(...), workspace_bytes(...)                host-side planning queries
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PaError",
    "library_path",
    "load_library",
    "CacheDesc",
    "cache_desc",
    "write_kv",
    "decode",
    "decode_partials",
    "decode_merge",
    "decode_shared_prefix",
    "decode_partials_shared_prefix",
    "decode_append",
    "decode_noalloc",
    "measure_read",
    "measure_mfma",
    "check_write",
    "check_decode",
    "check_prefill",
    "NOALLOC_SCRATCH_BYTES",
    "new_append_workspace",
    "prefill",
    "prefill_workspace",
    "partition_size",
    "workspace_bytes",
    "new_workspace",
    "status_string",
    "abi_version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None
_LIB_PATH: Optional[str] = None

PA_F32, PA_BF16 = 0, 1
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}
PA_LAYOUT_P09, PA_LAYOUT_VLLM = 0, 1
NOALLOC_SCRATCH_BYTES = 32 << 20      # PA_NOALLOC_SCRATCH_BYTES of the header


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
    ]


def library_path() -> str:
    return os.path.join(_HERE, "libpaged_kv.so")


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the in-tree library (built by ``paged_kv_cache_70_amd.build``):
    ``libpaged_kv.so``, or the build at ``path`` (the timeline build).  One
    build per process: asking for another once one is loaded is an error."""
    global _LIB, _LIB_PATH
    if _LIB is not None:
        if path is not None and os.path.abspath(path) != _LIB_PATH:
            raise RuntimeError(f"{_LIB_PATH} is already loaded in this process; cannot load {path}")
        return _LIB
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_70_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    pdesc = ctypes.POINTER(CacheDesc)
    sig = {
        "pa_write_kv": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, pdesc, vp]),
        "pa_decode_partition_size": (i32, [i32, i32, i32, pdesc]),
        "pa_decode_workspace_bytes": (sz, [i32, i32, i32, pdesc, i32]),
        "pa_decode": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, pdesc, i32, vp, sz, vp]),
        "pa_decode_partials": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, pdesc, i32, vp, sz, vp]),
        "pa_decode_merge": (ctypes.c_int, [vp, vp, i32, i32, i32, pdesc, i32, vp, sz, vp]),
        "pa_decode_shared_prefix": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, pdesc, i32,
                                                    vp, sz, vp]),
        "pa_decode_partials_shared_prefix": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32,
                                                             pdesc, i32, vp, sz, vp]),
        "pa_prefill": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, pdesc, vp, sz, vp]),
        "pa_prefill_workspace_bytes": (sz, [i32, i32, i32, i32, pdesc]),
        "pa_decode_append_workspace_bytes": (sz, [i32, i32, i32, pdesc, i32]),
        "pa_decode_append": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, pdesc, i32,
                                            vp, sz, vp]),
        "pa_decode_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, pdesc, i32, vp]),
        "pa_measure_read": (ctypes.c_int, [vp, sz, i32, i32, vp, vp]),
        "pa_measure_mfma": (ctypes.c_int, [i32, i32, vp, vp]),
        "pa_check_write_workspace_bytes": (sz, [pdesc]),
        "pa_check_write": (ctypes.c_int, [vp, i32, pdesc, vp, vp, sz, vp]),
        "pa_check_decode": (ctypes.c_int, [vp, vp, i32, i32, pdesc, vp, vp]),
        "pa_check_prefill": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, pdesc, vp, vp]),
        "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "pa_abi_version": (i32, []),
    }
    if hasattr(lib, "pa_timeline_read"):          # the timeline build
        sig["pa_timeline_read"] = (ctypes.c_int, [vp, sz])
        sig["pa_timeline_reset"] = (ctypes.c_int, [])
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    _LIB_PATH = os.path.abspath(path)
    return lib


def status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def abi_version() -> int:
    return int(load_library().pa_abi_version())


def cache_desc(k_cache: torch.Tensor) -> CacheDesc:
    """Geometry of a K cache: [num_blocks, block_size, num_kv_heads, head_dim]
    (the P09 layout), or 5-D [num_blocks, num_kv_heads, head_dim / x,
    block_size, x] with x = 16 bytes of elements (vLLM's layout)."""
    if k_cache.dtype not in _DTYPES:
        raise TypeError(f"unsupported cache dtype {k_cache.dtype}")
    if k_cache.dim() == 4:
        NB, bs, KVH, D = k_cache.shape
        return CacheDesc(NB, bs, KVH, D, _DTYPES[k_cache.dtype], PA_LAYOUT_P09)
    if k_cache.dim() == 5:
        NB, KVH, G, bs, x = k_cache.shape
        if x * k_cache.element_size() != 16:
            raise ValueError("vLLM-layout K cache: the last dimension must hold 16 bytes")
        return CacheDesc(NB, bs, KVH, G * x, _DTYPES[k_cache.dtype], PA_LAYOUT_VLLM)
    raise ValueError("k_cache must be [NB, bs, KVH, D] or vLLM's [NB, KVH, D/x, bs, x]")


def _check_v(k_cache: torch.Tensor, v_cache: torch.Tensor, desc: CacheDesc) -> None:
    if desc.layout == PA_LAYOUT_VLLM:
        want = (desc.num_blocks, desc.num_kv_heads, desc.head_dim, desc.block_size)
    else:
        want = tuple(k_cache.shape)
    if tuple(v_cache.shape) != want or v_cache.dtype != k_cache.dtype:
        raise ValueError(f"v_cache must be {list(want)} of {k_cache.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if not t.is_contiguous():
        # writing through a temporary copy would silently lose the result
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PaError(fn, status)


def write_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             slot_mapping: torch.Tensor) -> None:
    """In place: cache[slot // bs, slot % bs] = k[i] (and v) for slot >= 0."""
    lib = load_library()
    desc = cache_desc(k_cache)
    _check_v(k_cache, v_cache, desc)
    T = slot_mapping.shape[0] if slot_mapping.dim() == 1 else -1
    if T < 0:
        raise ValueError("slot_mapping must be 1-D")
    row = (desc.num_kv_heads, desc.head_dim)
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (T, *row) or t.dtype != k_cache.dtype:
            raise ValueError(f"{name} must be [{T}, {row[0]}, {row[1]}] of {k_cache.dtype}")
    if T == 0:
        return None
    st = lib.pa_write_kv(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k, "k"), _dev(v, "v"),
                         _dev(slot_mapping, "slot_mapping", torch.int64), T, ctypes.byref(desc),
                         _stream(k_cache))
    _check("pa_write_kv", st)
    return None


def partition_size(num_seqs: int, num_heads: int, max_blocks_per_seq: int, k_cache: torch.Tensor) -> int:
    desc = cache_desc(k_cache)
    p = load_library().pa_decode_partition_size(num_seqs, num_heads, max_blocks_per_seq, ctypes.byref(desc))
    _check("pa_decode_partition_size", p if p < 0 else 0)
    return int(p)


def workspace_bytes(num_seqs: int, num_heads: int, max_blocks_per_seq: int, k_cache: torch.Tensor,
                    partition_size: int = 0) -> int:
    desc = cache_desc(k_cache)
    return int(load_library().pa_decode_workspace_bytes(num_seqs, num_heads, max_blocks_per_seq,
                                                        ctypes.byref(desc), partition_size))


def new_workspace(num_seqs: int, num_heads: int, max_blocks_per_seq: int, k_cache: torch.Tensor,
                  partition_size: int = 0) -> torch.Tensor:
    """A decode workspace of the size pa_decode_workspace_bytes() gives."""
    need = workspace_bytes(num_seqs, num_heads, max_blocks_per_seq, k_cache, partition_size)
    return torch.empty(max(need, 16), dtype=torch.uint8, device=k_cache.device)


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, out, workspace, partition_size):
    desc = cache_desc(k_cache)
    _check_v(k_cache, v_cache, desc)
    if q.dim() != 3 or q.dtype != k_cache.dtype or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [num_seqs, num_heads, head_dim] of the cache dtype")
    B, H, D = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if tuple(context_lens.shape) != (B,):
        raise ValueError("context_lens must be [num_seqs]")
    W = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be like q")
    need = load_library().pa_decode_workspace_bytes(B, H, W, ctypes.byref(desc), partition_size)
    if need == 0 and partition_size and partition_size % desc.block_size:
        raise ValueError("partition_size must be a multiple of block_size")
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    return desc, B, H, W, out, workspace, wbytes


def _decode_call(fn_name, q, k_cache, v_cache, block_tables, context_lens, scale, out, workspace,
                 partition_size, shared_tokens=None):
    lib = load_library()
    desc, B, H, W, out, workspace, wbytes = _decode_args(
        q, k_cache, v_cache, block_tables, context_lens, out, workspace, partition_size)
    fn = getattr(lib, fn_name)
    shared = () if shared_tokens is None else (int(shared_tokens),)
    st = fn(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
            float(scale), B, H, W, *shared, ctypes.byref(desc), int(partition_size), _dev(workspace, "workspace"),
            wbytes, _stream(q))
    _check(fn_name, st)
    return out


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
           context_lens: torch.Tensor, scale: float, *, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, partition_size: int = 0) -> torch.Tensor:
    """Paged decode attention; returns ``out`` [B, H, D] in q's dtype."""
    return _decode_call("pa_decode", q, k_cache, v_cache, block_tables, context_lens, scale, out,
                        workspace, partition_size)


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, scale: float, *, out: torch.Tensor,
                   partition_size: int = 0) -> torch.Tensor:
    """decode() without a workspace: the partial results go to the library's
    static device scratch area (pa_decode_noalloc), so nothing is allocated
    here either: ``out`` must be given."""
    lib = load_library()
    desc = cache_desc(k_cache)
    _check_v(k_cache, v_cache, desc)
    if q.dim() != 3 or q.dtype != k_cache.dtype or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [num_seqs, num_heads, head_dim] of the cache dtype")
    B, H, _ = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(context_lens.shape) != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq] and context_lens [num_seqs]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be like q")
    st = lib.pa_decode_noalloc(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                               _dev(block_tables, "block_tables", torch.int32),
                               _dev(context_lens, "context_lens", torch.int32), float(scale), B, H,
                               block_tables.shape[1], ctypes.byref(desc), int(partition_size), _stream(q))
    _check("pa_decode_noalloc", st)
    return out


def decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale, *, out, workspace,
                    partition_size: int = 0) -> torch.Tensor:
    return _decode_call("pa_decode_partials", q, k_cache, v_cache, block_tables, context_lens, scale,
                        out, workspace, partition_size)


def decode_shared_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, scale: float, shared_tokens: int, *,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         partition_size: int = 0) -> torch.Tensor:
    """decode() for tables that may share their first ``shared_tokens`` tokens'
    blocks with row 0 (a common prompt): the same result, with the shared
    blocks read once per group of sequences instead of once per sequence."""
    return _decode_call("pa_decode_shared_prefix", q, k_cache, v_cache, block_tables, context_lens, scale, out,
                        workspace, partition_size, shared_tokens)


def decode_partials_shared_prefix(q, k_cache, v_cache, block_tables, context_lens, scale, shared_tokens, *,
                                  out, workspace, partition_size: int = 0) -> torch.Tensor:
    return _decode_call("pa_decode_partials_shared_prefix", q, k_cache, v_cache, block_tables, context_lens,
                        scale, out, workspace, partition_size, shared_tokens)


def new_append_workspace(num_seqs: int, num_heads: int, max_blocks_per_seq: int, k_cache: torch.Tensor,
                         partition_size: int = 0) -> torch.Tensor:
    """A workspace of the size pa_decode_append_workspace_bytes() gives."""
    desc = cache_desc(k_cache)
    need = load_library().pa_decode_append_workspace_bytes(num_seqs, num_heads, max_blocks_per_seq,
                                                           ctypes.byref(desc), int(partition_size))
    if need == 0:
        raise ValueError("unsupported decode sizes")
    return torch.empty(need, dtype=torch.uint8, device=k_cache.device)


def decode_append(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                  v_new: torch.Tensor, slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                  cached_lens: torch.Tensor, scale: float, *, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, partition_size: int = 0) -> torch.Tensor:
    """One decode step that appends sequence b's new token (k_new[b], v_new[b]
    at slot_mapping[b], none where the slot is negative): the output of
    write_kv followed by decode with context_lens = cached_lens + 1, and the
    same cache contents, from two kernels."""
    lib = load_library()
    if workspace is None and q.dim() == 3 and block_tables.dim() == 2:
        workspace = new_append_workspace(q.shape[0], q.shape[1], block_tables.shape[1], k_cache, partition_size)
    desc, B, H, W, out, workspace, wbytes = _decode_args(q, k_cache, v_cache, block_tables, cached_lens, out,
                                                         workspace, partition_size)
    row = (desc.num_kv_heads, desc.head_dim)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (B, *row) or t.dtype != k_cache.dtype:
            raise ValueError(f"{name} must be [{B}, {row[0]}, {row[1]}] of {k_cache.dtype}")
    if tuple(slot_mapping.shape) != (B,):
        raise ValueError("slot_mapping must be [num_seqs]")
    st = lib.pa_decode_append(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                              _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                              _dev(slot_mapping, "slot_mapping", torch.int64),
                              _dev(block_tables, "block_tables", torch.int32),
                              _dev(cached_lens, "cached_lens", torch.int32), float(scale), B, H, W,
                              ctypes.byref(desc), int(partition_size), _dev(workspace, "workspace"), wbytes,
                              _stream(q))
    _check("pa_decode_append", st)
    return out


def decode_merge(q_like: torch.Tensor, k_cache: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, *, out: torch.Tensor, workspace: torch.Tensor,
                 partition_size: int = 0) -> torch.Tensor:
    lib = load_library()
    desc = cache_desc(k_cache)
    B, H, _ = q_like.shape
    W = block_tables.shape[1]
    st = lib.pa_decode_merge(_dev(out, "out"), _dev(context_lens, "context_lens", torch.int32), B, H, W,
                             ctypes.byref(desc), int(partition_size), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(out))
    _check("pa_decode_merge", st)
    return out


# Bits of the checked mode's error word (pa_check_flag in the header).
CHECK_SLOT_RANGE, CHECK_SLOT_DUPLICATE, CHECK_TABLE_RANGE, CHECK_CONTEXT_RANGE, CHECK_QUERY_RANGE = 1, 2, 4, 8, 16


def _error_word(err: torch.Tensor) -> int:
    if err.numel() != 1 or err.dtype not in (torch.int32,):
        raise ValueError("error_word must be a one-element int32 device tensor")
    return _dev(err, "error_word")


def check_write(slot_mapping: torch.Tensor, k_cache: torch.Tensor, error_word: torch.Tensor, *,
                workspace: Optional[torch.Tensor] = None) -> None:
    """Checked mode: OR CHECK_SLOT_RANGE / CHECK_SLOT_DUPLICATE into
    ``error_word`` (zeroed by the caller) for a write's slot_mapping."""
    lib = load_library()
    desc = cache_desc(k_cache)
    if slot_mapping.dim() != 1:
        raise ValueError("slot_mapping must be 1-D")
    if workspace is None:
        need = int(lib.pa_check_write_workspace_bytes(ctypes.byref(desc)))
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=slot_mapping.device)
    st = lib.pa_check_write(_dev(slot_mapping, "slot_mapping", torch.int64), slot_mapping.shape[0],
                            ctypes.byref(desc), _error_word(error_word), _dev(workspace, "workspace"),
                            workspace.numel() * workspace.element_size(), _stream(slot_mapping))
    _check("pa_check_write", st)


def check_decode(block_tables: torch.Tensor, context_lens: torch.Tensor, k_cache: torch.Tensor,
                 error_word: torch.Tensor) -> None:
    """Checked mode: OR CHECK_CONTEXT_RANGE / CHECK_TABLE_RANGE into ``error_word``."""
    desc = cache_desc(k_cache)
    if block_tables.dim() != 2 or tuple(context_lens.shape) != (block_tables.shape[0],):
        raise ValueError("block_tables must be [B, W] and context_lens [B]")
    st = load_library().pa_check_decode(_dev(block_tables, "block_tables", torch.int32),
                                        _dev(context_lens, "context_lens", torch.int32), block_tables.shape[0],
                                        block_tables.shape[1], ctypes.byref(desc), _error_word(error_word),
                                        _stream(block_tables))
    _check("pa_check_decode", st)


def check_prefill(block_tables: torch.Tensor, context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                  num_tokens: int, k_cache: torch.Tensor, error_word: torch.Tensor) -> None:
    """Checked mode: check_decode's flags plus CHECK_QUERY_RANGE."""
    desc = cache_desc(k_cache)
    B = block_tables.shape[0]
    if block_tables.dim() != 2 or tuple(context_lens.shape) != (B,) or tuple(query_start_loc.shape) != (B + 1,):
        raise ValueError("block_tables must be [B, W], context_lens [B] and query_start_loc [B + 1]")
    st = load_library().pa_check_prefill(_dev(block_tables, "block_tables", torch.int32),
                                         _dev(context_lens, "context_lens", torch.int32),
                                         _dev(query_start_loc, "query_start_loc", torch.int32), B,
                                         block_tables.shape[1], int(num_tokens), ctypes.byref(desc),
                                         _error_word(error_word), _stream(block_tables))
    _check("pa_check_prefill", st)


def measure_read(buf: torch.Tensor, sink: torch.Tensor, *, workgroups_per_cu: int = 4,
                 nontemporal: bool = True) -> None:
    """Measurement helper: one streaming read of all of ``buf`` (16-byte
    loads) on the current stream; ``sink`` is a device int32/uint32 word."""
    nbytes = buf.numel() * buf.element_size()
    st = load_library().pa_measure_read(_dev(buf, "buf"), nbytes, int(workgroups_per_cu), int(bool(nontemporal)),
                                        _dev(sink, "sink"), _stream(buf))
    _check("pa_measure_read", st)


def measure_mfma(sink: torch.Tensor, iters: int, *, workgroups_per_cu: int = 1) -> int:
    """Measurement helper: independent bf16 matrix products on every wavefront
    (pa_measure_mfma); returns the flops enqueued."""
    lib = load_library()
    st = lib.pa_measure_mfma(int(iters), int(workgroups_per_cu), _dev(sink, "sink"), _stream(sink))
    _check("pa_measure_mfma", st)
    cus = torch.cuda.get_device_properties(sink.device).multi_processor_count
    return cus * workgroups_per_cu * 4 * int(iters) * 4 * 32768     # 4 wavefronts x 4 products of 32x32x16


def prefill_workspace(num_seqs: int, num_heads: int, max_blocks_per_seq: int, num_tokens: int,
                      k_cache: torch.Tensor) -> torch.Tensor:
    """A prefill workspace of the size pa_prefill_workspace_bytes() gives."""
    need = int(load_library().pa_prefill_workspace_bytes(num_seqs, num_heads, max_blocks_per_seq, num_tokens,
                                                         ctypes.byref(cache_desc(k_cache))))
    return torch.empty(max(need, 16), dtype=torch.uint8, device=k_cache.device)


def prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
            context_lens: torch.Tensor, query_start_loc: torch.Tensor, scale: float, *,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged causal attention of a packed batch of new queries; returns ``out``
    [T, H, D] in q's dtype.  Sequence b's queries are rows
    query_start_loc[b] .. query_start_loc[b+1] - 1, its last tokens."""
    lib = load_library()
    desc = cache_desc(k_cache)
    _check_v(k_cache, v_cache, desc)
    if q.dim() != 3 or q.dtype != k_cache.dtype or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [num_tokens, num_heads, head_dim] of the cache dtype")
    T, H, _ = q.shape
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    B, W = block_tables.shape
    if tuple(context_lens.shape) != (B,) or tuple(query_start_loc.shape) != (B + 1,):
        raise ValueError("context_lens must be [num_seqs] and query_start_loc [num_seqs + 1]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be like q")
    if workspace is None:
        workspace = prefill_workspace(B, H, W, T, k_cache)
    st = lib.pa_prefill(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                        _dev(block_tables, "block_tables", torch.int32),
                        _dev(context_lens, "context_lens", torch.int32),
                        _dev(query_start_loc, "query_start_loc", torch.int32), float(scale), B, H, W, T,
                        ctypes.byref(desc), _dev(workspace, "workspace"),
                        workspace.numel() * workspace.element_size(), _stream(q))
    _check("pa_prefill", st)
    return out
