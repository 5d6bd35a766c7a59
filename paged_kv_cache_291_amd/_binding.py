"""ctypes binding of libpagedattn.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(``include/pagedattn.h``).  There is no CPU fallback: if the library is not
built, or a tensor is not on a HIP device, the call raises.  PyTorch is used
for device memory and the current stream only.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = 0, -1, -2, -3, -4
PA_ERR_NO_BLOCKS, PA_ERR_CAPACITY, PA_ERR_SCRATCH = -5, -6, -7
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_FLAG_SHARED_BLOCKS = 1
DTYPE_CODES = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
# fp8 pools: raw e4m3 codes as uint8, or torch's float8_e4m3fn (the same encoding)
FP8_POOL_DTYPES = (torch.uint8, torch.float8_e4m3fn)

EXPORTED = ("pa_status_string", "pa_decode_workspace_size", "paged_attention_decode", "reshape_and_cache",
            "paged_attention_decode_noalloc",
            "paged_attention_decode_fp8", "reshape_and_cache_fp8", "paged_attention_prefill",
            "paged_attention_prefill_fp8", "pa_prefill_workspace_size",
            "copy_blocks", "pa_bm_create", "pa_bm_destroy", "pa_bm_allocate", "pa_bm_append_slots", "pa_bm_fork",
            "pa_bm_append_batch", "pa_bm_free", "pa_bm_num_free_blocks", "pa_bm_free_list", "pa_bm_ref_count", "pa_bm_seq_len",
            "pa_bm_block_tables", "pa_bm_num_copies", "pa_bm_take_copies")

_lib = None


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with paged_kv_cache_291_amd/build.py "
                           "(no CPU fallback exists)")
    lib = ctypes.CDLL(p)
    c_int, c_size, vp, c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [c_int]
    lib.pa_decode_workspace_size.restype = c_size
    lib.pa_decode_workspace_size.argtypes = [c_int] * 5
    lib.paged_attention_decode.restype = c_int
    lib.paged_attention_decode.argtypes = [vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int,
                                           c_int, c_int, c_int, c_float, c_int, c_int, ctypes.c_uint, vp,
                                           c_size, vp]
    lib.paged_attention_decode_noalloc.restype = c_int
    lib.paged_attention_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int,
                                                   c_int, c_int, c_int, c_float, c_int, c_int, ctypes.c_uint, vp]
    lib.reshape_and_cache.restype = c_int
    lib.reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp]
    lib.paged_attention_decode_fp8.restype = c_int
    lib.paged_attention_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int,
                                               c_int, c_int, c_int, c_float, c_float, c_float, c_int, c_int,
                                               ctypes.c_uint, vp, c_size, vp]
    lib.reshape_and_cache_fp8.restype = c_int
    lib.reshape_and_cache_fp8.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, c_float,
                                          c_float, vp]
    lib.paged_attention_prefill.restype = c_int
    lib.paged_attention_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp] + [c_int] * 9 + [
        c_float, c_int, ctypes.c_uint, vp, c_size, vp]
    lib.paged_attention_prefill_fp8.restype = c_int
    lib.paged_attention_prefill_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp] + [c_int] * 9 + [
        c_float, c_float, c_float, c_int, ctypes.c_uint, vp, c_size, vp]
    lib.pa_prefill_workspace_size.restype = c_size
    lib.pa_prefill_workspace_size.argtypes = [c_int] * 6
    lib.copy_blocks.restype = c_int
    lib.copy_blocks.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp]
    pbm = ctypes.POINTER(vp)
    lib.pa_bm_create.restype = c_int
    lib.pa_bm_create.argtypes = [c_int, c_int, c_int, c_int, pbm]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_destroy.argtypes = [vp]
    for name in ("pa_bm_allocate", "pa_bm_append_slots"):
        getattr(lib, name).restype = c_int
        getattr(lib, name).argtypes = [vp, c_int, c_int, vp]
    lib.pa_bm_append_batch.restype = c_int
    lib.pa_bm_append_batch.argtypes = [vp, vp, c_int, vp]
    lib.pa_bm_fork.restype = c_int
    lib.pa_bm_fork.argtypes = [vp, c_int, c_int]
    for name in ("pa_bm_free", "pa_bm_ref_count", "pa_bm_seq_len"):
        getattr(lib, name).restype = c_int
        getattr(lib, name).argtypes = [vp, c_int]
    for name in ("pa_bm_num_free_blocks", "pa_bm_num_copies"):
        getattr(lib, name).restype = c_int
        getattr(lib, name).argtypes = [vp]
    lib.pa_bm_free_list.restype = c_int
    lib.pa_bm_free_list.argtypes = [vp, vp, c_int]
    lib.pa_bm_block_tables.restype = c_int
    lib.pa_bm_block_tables.argtypes = [vp, vp, c_int, vp, vp]
    lib.pa_bm_take_copies.restype = c_int
    lib.pa_bm_take_copies.argtypes = [vp, vp, vp, c_int]
    if path is None:
        _lib = lib
    return lib


def pa_status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def _check(rc: int):
    if rc != PA_OK:
        raise PagedAttnError(rc, pa_status_string(rc))


def pa_decode_workspace_size(num_seqs: int, num_heads: int, head_size: int, max_seq_len: int,
                             partition_size: int) -> int:
    return int(load_library().pa_decode_workspace_size(num_seqs, num_heads, head_size, max_seq_len,
                                                       partition_size))


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def decode_workspace_bytes(query: torch.Tensor, block_tables: torch.Tensor, block_size: int,
                           partition_size: int = 0, max_seq_len: int = 0) -> int:
    """Workspace bytes a call with these arguments needs (0 if none)."""
    S, Hq, D = query.shape
    if partition_size == 0 and query.dtype == torch.float32:
        return 0
    msl = max_seq_len if max_seq_len > 0 else block_tables.shape[1] * block_size
    return pa_decode_workspace_size(S, Hq, D, msl, partition_size)


def paged_attention_decode(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                           scale: float, partition_size: int = 0, max_seq_len: int = 0,
                           workspace: Optional[torch.Tensor] = None, flags: int = 0,
                           stream=None) -> torch.Tensor:
    """Enqueue paged decode attention on ``stream`` (default: torch's current stream).

    Shapes: out/query ``[S, Hq, D]``; caches ``[NB, BS, Hkv, D]``;
    block_tables int32 ``[S, max_blocks]``; seq_lens int32 ``[S]``.
    ``partition_size`` 0 lets the library balance the work, > 0 splits every
    sequence into partitions of that many tokens.  When a workspace is needed
    (see ``decode_workspace_bytes``) pass one (uint8 device tensor, 256-byte
    aligned) or let this wrapper allocate it.  ``flags``:
    ``PA_FLAG_SHARED_BLOCKS`` when blocks are shared between sequences.
    """
    S, Hq, D = query.shape
    NB, BS, Hkv, Dk = k_cache.shape
    if tuple(out.shape) != (S, Hq, D) or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between out/query/k_cache/v_cache")
    if query.dtype not in DTYPE_CODES:
        raise TypeError(f"unsupported dtype {query.dtype}")
    dt = query.dtype
    if block_tables.dim() != 2 or block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and seq_lens [S]")
    ws_ptr, ws_bytes = 0, 0
    need = decode_workspace_bytes(query, block_tables, BS, partition_size, max_seq_len)
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    rc = load_library().paged_attention_decode(
        _dev(out, "out", dt), _dev(query, "query", dt), _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), _dev(block_tables, "block_tables", torch.int32),
        _dev(seq_lens, "seq_lens", torch.int32), S, Hq, Hkv, D, BS, block_tables.shape[1], NB,
        int(max_seq_len), float(scale), DTYPE_CODES[dt], int(partition_size), int(flags), ws_ptr, ws_bytes,
        _stream(stream))
    _check(rc)
    return out


def paged_attention_decode_noalloc(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                                   scale: float, partition_size: int = 0, max_seq_len: int = 0, flags: int = 0,
                                   stream=None) -> torch.Tensor:
    """``paged_attention_decode`` with the library's own device scratch array
    in place of a workspace: nothing is allocated (see
    ``include/pagedattn.h``; calls that overlap in time on one device race)."""
    S, Hq, D = query.shape
    NB, BS, Hkv, Dk = k_cache.shape
    if tuple(out.shape) != (S, Hq, D) or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between out/query/k_cache/v_cache")
    if query.dtype not in DTYPE_CODES:
        raise TypeError(f"unsupported dtype {query.dtype}")
    dt = query.dtype
    if block_tables.dim() != 2 or block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and seq_lens [S]")
    rc = load_library().paged_attention_decode_noalloc(
        _dev(out, "out", dt), _dev(query, "query", dt), _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), _dev(block_tables, "block_tables", torch.int32),
        _dev(seq_lens, "seq_lens", torch.int32), S, Hq, Hkv, D, BS, block_tables.shape[1], NB,
        int(max_seq_len), float(scale), DTYPE_CODES[dt], int(partition_size), int(flags), _stream(stream))
    _check(rc)
    return out


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Enqueue the scatter of ``key``/``value`` ``[T, Hkv, D]`` into their cache slots."""
    T, Hkv, D = key.shape
    NB, BS, Hkv2, D2 = k_cache.shape
    if tuple(value.shape) != (T, Hkv, D) or (Hkv2, D2) != (Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between key/value and the caches")
    if key.dtype not in DTYPE_CODES:
        raise TypeError(f"unsupported dtype {key.dtype}")
    dt = key.dtype
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    rc = load_library().reshape_and_cache(
        _dev(key, "key", dt), _dev(value, "value", dt), _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), _dev(slot_mapping, "slot_mapping", torch.int32), T, Hkv, D, BS,
        NB, DTYPE_CODES[dt], _stream(stream))
    _check(rc)


def _fp8_pool(t: torch.Tensor, name: str) -> int:
    if t.dtype not in FP8_POOL_DTYPES:
        raise TypeError(f"{name} must hold e4m3 codes (uint8 or float8_e4m3fn), got {t.dtype}")
    return _dev(t, name)


def paged_attention_decode_fp8(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                               v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                               scale: float, k_scale: float, v_scale: float, partition_size: int = 0,
                               max_seq_len: int = 0, workspace: Optional[torch.Tensor] = None, flags: int = 0,
                               stream=None) -> torch.Tensor:
    """Decode over fp8 (e4m3) pools: a code c means e4m3(c) * k_scale (K) or
    * v_scale (V).  query/out are bf16 or fp16; everything else is as in
    ``paged_attention_decode``."""
    S, Hq, D = query.shape
    NB, BS, Hkv, Dk = k_cache.shape
    if tuple(out.shape) != (S, Hq, D) or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between out/query/k_cache/v_cache")
    if query.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"query must be fp16 or bf16, got {query.dtype}")
    dt = query.dtype
    if block_tables.dim() != 2 or block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and seq_lens [S]")
    ws_ptr, ws_bytes = 0, 0
    need = decode_workspace_bytes(query, block_tables, BS, partition_size, max_seq_len)
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    rc = load_library().paged_attention_decode_fp8(
        _dev(out, "out", dt), _dev(query, "query", dt), _fp8_pool(k_cache, "k_cache"), _fp8_pool(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), _dev(seq_lens, "seq_lens", torch.int32), S, Hq, Hkv, D,
        BS, block_tables.shape[1], NB, int(max_seq_len), float(scale), float(k_scale), float(v_scale),
        DTYPE_CODES[dt], int(partition_size), int(flags), ws_ptr, ws_bytes, _stream(stream))
    _check(rc)
    return out


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          slot_mapping: torch.Tensor, k_scale: float, v_scale: float, stream=None) -> None:
    """Enqueue the scatter of ``key``/``value`` ``[T, Hkv, D]`` (fp32/fp16/bf16)
    into fp8 pools, quantised as in ``include/pagedattn.h``."""
    T, Hkv, D = key.shape
    NB, BS, Hkv2, D2 = k_cache.shape
    if tuple(value.shape) != (T, Hkv, D) or (Hkv2, D2) != (Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between key/value and the caches")
    if key.dtype not in DTYPE_CODES or value.dtype != key.dtype:
        raise TypeError(f"unsupported dtype {key.dtype}")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    rc = load_library().reshape_and_cache_fp8(
        _dev(key, "key", key.dtype), _dev(value, "value", key.dtype), _fp8_pool(k_cache, "k_cache"),
        _fp8_pool(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping", torch.int32), T, Hkv, D, BS, NB,
        DTYPE_CODES[key.dtype], float(k_scale), float(v_scale), _stream(stream))
    _check(rc)


def pa_prefill_workspace_size(num_seqs: int, num_query_tokens: int, num_heads: int, num_kv_heads: int,
                              head_size: int, max_query_len: int) -> int:
    return int(load_library().pa_prefill_workspace_size(num_seqs, num_query_tokens, num_heads, num_kv_heads,
                                                        head_size, max_query_len))


def paged_attention_prefill(out: torch.Tensor, query: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                            query_start: torch.Tensor, scale: float, max_query_len: int = 0,
                            k_scale: Optional[float] = None, v_scale: Optional[float] = None, flags: int = 0,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Several query rows per sequence (its last tokens), causal over the
    paged cache.  query/out ``[T, Hq, D]`` bf16/fp16, query_start int32
    ``[S + 1]``.  With ``k_scale``/``v_scale`` the pools hold e4m3 codes.
    A workspace is allocated when the call needs one and none is given."""
    T, Hq, D = query.shape
    NB, BS, Hkv, Dk = k_cache.shape
    S = seq_lens.shape[0]
    if tuple(out.shape) != (T, Hq, D) or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between out/query/k_cache/v_cache")
    if query.dtype not in DTYPE_CODES:
        raise TypeError(f"unsupported dtype {query.dtype}")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.shape != (S + 1,):
        raise ValueError("block_tables must be [S, max_blocks] and query_start [S + 1]")
    dt = query.dtype
    fp8 = k_scale is not None or v_scale is not None
    ws_ptr, ws_bytes = 0, 0
    need = pa_prefill_workspace_size(S, T, Hq, Hkv, D, int(max_query_len)) if S > 0 else 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    common = (_dev(out, "out", dt), _dev(query, "query", dt),
              _fp8_pool(k_cache, "k_cache") if fp8 else _dev(k_cache, "k_cache", dt),
              _fp8_pool(v_cache, "v_cache") if fp8 else _dev(v_cache, "v_cache", dt),
              _dev(block_tables, "block_tables", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
              _dev(query_start, "query_start", torch.int32), S, T, Hq, Hkv, D, BS, block_tables.shape[1], NB,
              int(max_query_len), float(scale))
    lib = load_library()
    if fp8:
        rc = lib.paged_attention_prefill_fp8(*common, float(k_scale if k_scale is not None else 1.0),
                                             float(v_scale if v_scale is not None else 1.0), DTYPE_CODES[dt],
                                             int(flags), ws_ptr, ws_bytes, _stream(stream))
    else:
        rc = lib.paged_attention_prefill(*common, DTYPE_CODES[dt], int(flags), ws_ptr, ws_bytes, _stream(stream))
    _check(rc)
    return out


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src: torch.Tensor, dst: torch.Tensor,
                stream=None) -> None:
    """Enqueue block copies ``cache[dst[i]] = cache[src[i]]`` in both pools
    (int32 device tensors of equal length; see ``include/pagedattn.h``)."""
    NB, BS, Hkv, D = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if k_cache.dtype not in DTYPE_CODES and k_cache.dtype not in FP8_POOL_DTYPES:
        raise TypeError(f"unsupported dtype {k_cache.dtype}")
    if src.shape != dst.shape or src.dim() != 1:
        raise ValueError("src and dst must be 1-D of equal length")
    dt = k_cache.dtype
    code = DTYPE_CODES.get(dt, PA_FP8_E4M3)
    rc = load_library().copy_blocks(
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt), _dev(src, "src", torch.int32),
        _dev(dst, "dst", torch.int32), int(src.numel()), Hkv, D, BS, NB, code, _stream(stream))
    _check(rc)


class BlockManager:
    """Host block manager of the paged KV cache (``pa_bm_*`` of the C ABI).

    Sequences are ids in ``[0, max_seqs)``.  Slots, tables and copy lists come
    back as int32 NumPy arrays in host memory; move them to the device for
    ``reshape_and_cache`` / ``paged_attention_decode`` / ``copy_blocks``.
    """

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int):
        import numpy as np
        self._np = np
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_bm_create(num_blocks, block_size, max_seqs, max_blocks_per_seq, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_seqs, self.max_blocks_per_seq = max_seqs, max_blocks_per_seq

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _slots(self, fn, seq, n):
        out = self._np.empty(max(n, 0), dtype=self._np.int32)
        _check(fn(self._h, int(seq), int(n), out.ctypes.data if n > 0 else None))
        return out

    def allocate(self, seq: int, num_tokens: int):
        return self._slots(self._lib.pa_bm_allocate, seq, num_tokens)

    def append_slots(self, seq: int, num_tokens: int = 1):
        return self._slots(self._lib.pa_bm_append_slots, seq, num_tokens)

    def append_batch(self, seqs):
        """One more token for each of ``seqs`` (all or nothing); their slots."""
        np = self._np
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        out = np.empty(seqs.size, dtype=np.int32)
        if seqs.size:
            _check(self._lib.pa_bm_append_batch(self._h, seqs.ctypes.data, int(seqs.size), out.ctypes.data))
        return out

    def fork(self, parent: int, child: int) -> None:
        _check(self._lib.pa_bm_fork(self._h, int(parent), int(child)))

    def free(self, seq: int) -> None:
        _check(self._lib.pa_bm_free(self._h, int(seq)))

    def num_free_blocks(self) -> int:
        return self._lib.pa_bm_num_free_blocks(self._h)

    def free_list(self):
        out = self._np.empty(self.num_blocks, dtype=self._np.int32)
        n = self._lib.pa_bm_free_list(self._h, out.ctypes.data if self.num_blocks else None, self.num_blocks)
        if n < 0:
            _check(n)
        return out[:n]

    def ref_count(self, block: int) -> int:
        r = self._lib.pa_bm_ref_count(self._h, int(block))
        if r < 0:
            _check(r)
        return r

    def seq_len(self, seq: int) -> int:
        r = self._lib.pa_bm_seq_len(self._h, int(seq))
        if r < -1:
            _check(r)
        return r

    def block_tables(self, seqs):
        np = self._np
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        n = int(seqs.size)
        bt = np.empty((n, self.max_blocks_per_seq), dtype=np.int32)
        sl = np.empty(n, dtype=np.int32)
        if n:
            _check(self._lib.pa_bm_block_tables(self._h, seqs.ctypes.data, n,
                                                bt.ctypes.data if bt.size else sl.ctypes.data, sl.ctypes.data))
        return bt, sl

    def take_copies(self):
        np = self._np
        n = self._lib.pa_bm_num_copies(self._h)
        src = np.empty(max(n, 1), dtype=np.int32)
        dst = np.empty(max(n, 1), dtype=np.int32)
        got = self._lib.pa_bm_take_copies(self._h, src.ctypes.data, dst.ctypes.data, n)
        if got < 0:
            _check(got)
        return src[:got], dst[:got]
