"""Thin ctypes binding of libuq.so (C ABI in include/uq_paged.h).

Argument marshalling only: tensors are checked for device, dtype and layout, their
pointers and strides are passed through, and every step runs in the HIP kernels.  There
is no fallback: if the library is missing, or the tensors are not on a GPU, the calls
raise.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libuq.so")

UQ_OK, UQ_ERR_INVALID_ARG, UQ_ERR_UNSUPPORTED, UQ_ERR_LAUNCH = 0, 1, 2, 3
UQ_F32, UQ_BF16 = 0, 1
UQ_KV_FP8_E4M3, UQ_KV_FP4_E2M1_E4M3S, UQ_KV_FP4_E2M1_UE8M0S = 0, 1, 2
UQ_KV_FP8_E4M3_TOKSCALE = 3

EXPORTS = ("uq_paged_decode", "uq_paged_reduce", "uq_paged_decode_mtp", "uq_paged_reduce_mtp",
           "uq_paged_attention", "uq_paged_attention_noalloc", "uq_index_score",
           "uq_decode_workspace_bytes",
           "uq_attention_workspace_bytes", "uq_last_error")

_lock = threading.Lock()
_lib = None


class UqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[uq status {status}] {msg}")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libuq.so (built by ``python -m quantized_paged_attention_amd.build``), or the
    library at ``path``, or at $UQ_LIB when that is set (another build of the same
    sources, e.g. one with host-side sanitizers)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or os.environ.get("UQ_LIB") or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with "
                               "`python -m quantized_paged_attention_amd.build`")
        lib = ctypes.CDLL(p)
        V, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        lib.uq_paged_decode.restype = ctypes.c_int
        lib.uq_paged_decode.argtypes = [V, ctypes.c_int, i64, i64, V, i64, i32, i32, i32,
                                        ctypes.c_int, V, V, V, V, i32, V, i32, i32, i32, i32,
                                        f32, i32, V, V, V, V]
        lib.uq_paged_reduce.restype = ctypes.c_int
        lib.uq_paged_reduce.argtypes = [V, V, V, V, i32, i32, i32, i32, i32, i32, V,
                                        ctypes.c_int, i64, i64, V]
        lib.uq_paged_decode_mtp.restype = ctypes.c_int
        lib.uq_paged_decode_mtp.argtypes = [V, ctypes.c_int, i64, i64, V, i64, i32, i32, i32,
                                            ctypes.c_int, V, V, V, V, i32, V, i32, i32, i32,
                                            i32, i32, f32, i32, V, V, V, V]
        lib.uq_paged_reduce_mtp.restype = ctypes.c_int
        lib.uq_paged_reduce_mtp.argtypes = [V, V, V, V, i32, i32, i32, i32, i32, i32, i32, V,
                                            ctypes.c_int, i64, i64, V]
        lib.uq_index_score.restype = ctypes.c_int
        lib.uq_index_score.argtypes = [V, i64, i64, V, i64, i64, V, i32, V, i32, i32, i32,
                                       i32, i32, i32, V, i64, i64, i32, V]
        lib.uq_paged_attention.restype = ctypes.c_int
        lib.uq_paged_attention.argtypes = [V, ctypes.c_int, i64, i64, V, i64, i32, i32, i32,
                                           ctypes.c_int, V, V, V, V, i32, V, i32, i32, i32,
                                           i32, i32, f32, i32, V, ctypes.c_size_t, V, i64,
                                           i64, V]
        lib.uq_paged_attention_noalloc.restype = ctypes.c_int
        lib.uq_paged_attention_noalloc.argtypes = [V, ctypes.c_int, i64, i64, V, i64, i32, i32,
                                                   i32, ctypes.c_int, V, V, V, V, i32, V, i32,
                                                   i32, i32, i32, i32, f32, i32, V, i64, i64, V]
        lib.uq_attention_workspace_bytes.restype = ctypes.c_size_t
        lib.uq_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32,
                                                     ctypes.c_int]
        lib.uq_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.uq_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.uq_last_error.restype = ctypes.c_char_p
        lib.uq_last_error.argtypes = []
        if path is None:
            _lib = lib
        return lib


def _check(status: int):
    if status != UQ_OK:
        raise UqError(status, load_library().uq_last_error().decode())


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("uq kernels take GPU tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return UQ_F32
    if dt == torch.bfloat16:
        return UQ_BF16
    raise ValueError(f"query/output dtype must be float32 or bfloat16, got {dt}")


def _need(t: torch.Tensor, dtype: torch.dtype, name: str):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def decode_workspace_bytes(num_seqs: int, num_kv_heads: int, qg: int, head_dim: int,
                           num_partitions: int) -> int:
    return int(load_library().uq_decode_workspace_bytes(num_seqs, num_kv_heads, qg, head_dim,
                                                        num_partitions))


def alloc_partials(num_seqs: int, num_kv_heads: int, qg: int, head_dim: int,
                   num_partitions: int, device="cuda"):
    """Caller-owned partial buffers for paged_decode (bf16 o, f32 m, f32 l)."""
    shp = (num_seqs, num_kv_heads, num_partitions, qg)
    return (torch.empty(*shp, head_dim, dtype=torch.bfloat16, device=device),
            torch.empty(shp, dtype=torch.float32, device=device),
            torch.empty(shp, dtype=torch.float32, device=device))


def _decode_head(query, kv_cache, block_table, seq_lens, kv_format, max_seq_len, k_scale,
                 v_scale, rot_signs, query_len):
    """Checks shared by the decode entry points; returns the leading C arguments (query
    through num_seqs) and (B, QL, Hq, D, Hk)."""
    if query.dim() != 3 or query.stride(2) != 1:
        raise ValueError("query must be [B, Hq, D] with a contiguous head dim")
    if kv_cache.dim() != 4 or not kv_cache.is_contiguous():
        raise ValueError("kv_cache must be a contiguous [num_blocks, block_size, Hk, slot]")
    _need(kv_cache, torch.uint8, "kv_cache")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [B, max_blocks] with contiguous rows")
    rows, Hq, D = query.shape
    QL = int(query_len)
    B = seq_lens.shape[0] if seq_lens.dim() == 1 else -1
    if QL < 1 or rows != B * QL:
        raise ValueError("query must hold query_len rows per sequence of seq_lens")
    nb, bs, hk, slot = kv_cache.shape
    for t, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t is not None:
            _need(t, torch.float32, nm)
            if kv_format == UQ_KV_FP8_E4M3_TOKSCALE and (
                    tuple(t.shape) != (nb, hk, bs) or not t.is_contiguous()):
                raise ValueError(f"{nm} must be a contiguous [num_blocks, Hk, block_size] "
                                 "tensor of per-token scales")
    if rot_signs is not None:
        _need(rot_signs, torch.int8, "rot_signs")
    if seq_lens.shape != (B,) or block_table.shape[0] != B:
        raise ValueError("seq_lens / block_table do not match the batch")
    if block_table.shape[1] * bs < max_seq_len:
        # (the C ABI sees only the row stride, which a column slice of a wider table keeps)
        raise ValueError(f"block_table has {block_table.shape[1]} columns of {bs} tokens, "
                         f"fewer than max_seq_len {max_seq_len}")
    head = (_ptr(query), _dtype_code(query.dtype), query.stride(0), query.stride(1),
            _ptr(kv_cache), nb, bs, hk, slot, kv_format, _ptr(k_scale), _ptr(v_scale),
            _ptr(rot_signs), _ptr(block_table), block_table.stride(0), _ptr(seq_lens), B)
    return head, (B, QL, Hq, D, hk)


def paged_decode(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, *, kv_format: int, max_seq_len: int,
                 num_partitions: int, part_out: torch.Tensor, part_max: torch.Tensor,
                 part_sum: torch.Tensor, softmax_scale: float = 0.0,
                 k_scale: torch.Tensor | None = None, v_scale: torch.Tensor | None = None,
                 rot_signs: torch.Tensor | None = None, query_len: int = 1,
                 stream=None) -> None:
    """uq_paged_decode (query_len = 1) or uq_paged_decode_mtp on torch tensors: query
    [B*QL, Hq, D] (strided over rows and Hq, D contiguous; row b*QL + j is query j of
    sequence b); kv_cache [num_blocks, block_size, Hk, slot] uint8; partials
    [B, Hk, P, QL*QG(, D)].  k_scale / v_scale: float32 [1] per-tensor scales, or with
    kv_format UQ_KV_FP8_E4M3_TOKSCALE the per-token scales [num_blocks, Hk, block_size]."""
    lib = load_library()
    _need(part_out, torch.bfloat16, "part_out")
    _need(part_max, torch.float32, "part_max")
    _need(part_sum, torch.float32, "part_sum")
    head, (B, QL, Hq, D, hk) = _decode_head(query, kv_cache, block_table, seq_lens, kv_format,
                                            max_seq_len, k_scale, v_scale, rot_signs,
                                            query_len)
    qr = QL * (Hq // hk if hk else 0)
    if tuple(part_out.shape) != (B, hk, num_partitions, qr, D) or not part_out.is_contiguous():
        raise ValueError("part_out must be a contiguous [B, Hk, P, QL*QG, D] tensor")
    for t, nm in ((part_max, "part_max"), (part_sum, "part_sum")):
        if tuple(t.shape) != (B, hk, num_partitions, qr) or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous [B, Hk, P, QL*QG] tensor")
    tail = (Hq, D, int(max_seq_len), float(softmax_scale), int(num_partitions),
            _ptr(part_out), _ptr(part_max), _ptr(part_sum), _stream(stream))
    if QL == 1:
        _check(lib.uq_paged_decode(*head, *tail))
    else:
        _check(lib.uq_paged_decode_mtp(*head, QL, *tail))


def paged_reduce(part_out: torch.Tensor, part_max: torch.Tensor, part_sum: torch.Tensor,
                 seq_lens: torch.Tensor, out: torch.Tensor, *, max_seq_len: int,
                 query_len: int = 1, stream=None) -> None:
    """uq_paged_reduce (query_len = 1) or uq_paged_reduce_mtp into out [B*QL, Hk*QG, D]
    (float32 or bfloat16, D contiguous) from partials [B, Hk, P, QL*QG(, D)]."""
    lib = load_library()
    _need(part_out, torch.bfloat16, "part_out")
    B, hk, P, qr, D = part_out.shape
    QL = int(query_len)
    if QL < 1 or qr % QL:
        raise ValueError("the partial rows must be query_len x QG")
    qg = qr // QL
    if out.dim() != 3 or out.stride(2) != 1 or tuple(out.shape) != (B * QL, hk * qg, D):
        raise ValueError("out must be [B*QL, Hk*QG, D] with a contiguous head dim")
    head = (_ptr(part_out), _ptr(part_max), _ptr(part_sum), _ptr(seq_lens), B, hk)
    tail = (qg, D, P, int(max_seq_len), _ptr(out), _dtype_code(out.dtype), out.stride(0),
            out.stride(1), _stream(stream))
    if QL == 1:
        _check(lib.uq_paged_reduce(*head, *tail))
    else:
        _check(lib.uq_paged_reduce_mtp(*head, QL, *tail))


def attention_workspace_bytes(num_seqs: int, num_kv_heads: int, query_len: int, qg: int,
                              head_dim: int, num_partitions: int, max_seq_len: int,
                              kv_format: int) -> int:
    return int(load_library().uq_attention_workspace_bytes(
        num_seqs, num_kv_heads, query_len, qg, head_dim, num_partitions, max_seq_len,
        kv_format))


def alloc_workspace(num_seqs: int, num_kv_heads: int, query_len: int, qg: int, head_dim: int,
                    num_partitions: int, max_seq_len: int, kv_format: int,
                    device="cuda") -> torch.Tensor:
    """Zero-filled uq_paged_attention workspace (uint8); reusable across calls."""
    n = attention_workspace_bytes(num_seqs, num_kv_heads, query_len, qg, head_dim,
                                  num_partitions, max_seq_len, kv_format)
    if n <= 0:
        raise ValueError("invalid sizes for the attention workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def paged_attention(query, kv_cache, block_table, seq_lens, *, kv_format, max_seq_len,
                    num_partitions, out=None, workspace=None, softmax_scale=0.0,
                    k_scale=None, v_scale=None, rot_signs=None, query_len=1, stream=None):
    """One decode step through uq_paged_attention (decode and flash-combine in one call);
    returns out [B*QL, Hq, D] in the query dtype.  workspace: from alloc_workspace (one is
    allocated when None)."""
    lib = load_library()
    head, (B, QL, Hq, D, hk) = _decode_head(query, kv_cache, block_table, seq_lens, kv_format,
                                            max_seq_len, k_scale, v_scale, rot_signs,
                                            query_len)
    qg = Hq // hk if hk else 0
    if workspace is None:
        workspace = alloc_workspace(B, hk, QL, qg, D, num_partitions, max_seq_len, kv_format,
                                    query.device)
    _need(workspace, torch.uint8, "workspace")
    if workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-d uint8 tensor")
    if out is None:
        out = torch.empty(B * QL, Hq, D, dtype=query.dtype, device=query.device)
    if out.dtype != query.dtype or out.dim() != 3 or out.stride(2) != 1 or \
            tuple(out.shape) != (B * QL, Hq, D):
        raise ValueError("out must be [B*QL, Hq, D] of the query dtype with a contiguous head dim")
    _check(lib.uq_paged_attention(
        *head, QL, Hq, D, int(max_seq_len), float(softmax_scale), int(num_partitions),
        _ptr(workspace), workspace.numel(), _ptr(out), out.stride(0), out.stride(1),
        _stream(stream)))
    return out


def paged_attention_noalloc(query, kv_cache, block_table, seq_lens, *, kv_format,
                            max_seq_len, num_partitions, out=None, softmax_scale=0.0,
                            k_scale=None, v_scale=None, rot_signs=None, query_len=1,
                            stream=None):
    """One decode step through uq_paged_attention_noalloc: as paged_attention, with the
    workspace in the library's per-GPU scratch (no allocation by the library; calls that
    overlap in time on one GPU race).  out is allocated here when None."""
    lib = load_library()
    head, (B, QL, Hq, D, hk) = _decode_head(query, kv_cache, block_table, seq_lens, kv_format,
                                            max_seq_len, k_scale, v_scale, rot_signs,
                                            query_len)
    if out is None:
        out = torch.empty(B * QL, Hq, D, dtype=query.dtype, device=query.device)
    if out.dtype != query.dtype or out.dim() != 3 or out.stride(2) != 1 or \
            tuple(out.shape) != (B * QL, Hq, D):
        raise ValueError("out must be [B*QL, Hq, D] of the query dtype with a contiguous head dim")
    _check(lib.uq_paged_attention_noalloc(
        *head, QL, Hq, D, int(max_seq_len), float(softmax_scale), int(num_partitions),
        _ptr(out), out.stride(0), out.stride(1), _stream(stream)))
    return out


def paged_decode_reduce(query, kv_cache, block_table, seq_lens, *, kv_format, max_seq_len,
                        num_partitions, out=None, partials=None, softmax_scale=0.0,
                        k_scale=None, v_scale=None, rot_signs=None, query_len=1, stream=None):
    """One decode step as two calls: uq_paged_decode then uq_paged_reduce (their _mtp forms
    for query_len > 1) through caller-visible partials; returns out [B*QL, Hq, D] in the
    query dtype."""
    rows, Hq, D = query.shape
    B = seq_lens.shape[0]
    hk = kv_cache.shape[2]
    if partials is None:
        partials = alloc_partials(B, hk, query_len * (Hq // hk), D, num_partitions,
                                  query.device)
    if out is None:
        out = torch.empty(rows, Hq, D, dtype=query.dtype, device=query.device)
    po, pm, pl = partials
    paged_decode(query, kv_cache, block_table, seq_lens, kv_format=kv_format,
                 max_seq_len=max_seq_len, num_partitions=num_partitions, part_out=po,
                 part_max=pm, part_sum=pl, softmax_scale=softmax_scale, k_scale=k_scale,
                 v_scale=v_scale, rot_signs=rot_signs, query_len=query_len, stream=stream)
    paged_reduce(po, pm, pl, seq_lens, out, max_seq_len=max_seq_len, query_len=query_len,
                 stream=stream)
    return out


def index_score(q: torch.Tensor, k_pages: torch.Tensor, block_table: torch.Tensor,
                seq_lens: torch.Tensor, scores: torch.Tensor, *, query_len: int,
                init_blocks: int = 0, local_blocks: int = 0, stream=None) -> None:
    """uq_index_score: q e4m3 codes [R*QL, H, D] uint8; k_pages [num_pages, page_stride]
    uint8; scores float32 [H, R*QL, S] (page index contiguous)."""
    lib = load_library()
    _need(q, torch.uint8, "q")
    _need(k_pages, torch.uint8, "k_pages")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(scores, torch.float32, "scores")
    if q.dim() != 3 or q.stride(2) != 1:
        raise ValueError("q must be [R*QL, H, D] with contiguous dims")
    if k_pages.dim() != 2 or k_pages.stride(1) != 1:
        raise ValueError("k_pages must be [num_pages, page_stride] with contiguous rows")
    if scores.dim() != 3 or scores.stride(2) != 1:
        raise ValueError("scores must be [H, R*QL, S] with a contiguous page index")
    rows, H, D = q.shape
    R = seq_lens.shape[0]
    if rows != R * query_len or scores.shape[0] != H or scores.shape[1] != rows:
        raise ValueError("q / scores shapes do not match seq_lens and query_len")
    if block_table.dim() != 2 or block_table.stride(1) != 1 or block_table.shape[0] != R:
        raise ValueError("block_table must be [R, max_blocks] with contiguous rows")
    if block_table.shape[1] < scores.shape[2]:
        # every score column needs its table column (the C ABI sees only the row stride,
        # which a column slice of a wider table keeps)
        raise ValueError(f"block_table has {block_table.shape[1]} columns, fewer than the "
                         f"{scores.shape[2]} score columns")
    _check(lib.uq_index_score(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_pages), k_pages.stride(0), k_pages.shape[0],
        _ptr(block_table), block_table.stride(0), _ptr(seq_lens), R, int(query_len), H, D,
        int(init_blocks), int(local_blocks), _ptr(scores), scores.stride(0), scores.stride(1),
        scores.shape[2], _stream(stream)))

