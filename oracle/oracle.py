"""ctypes front end of the fp64 CPU oracle (``uq_oracle.c``).

Test infrastructure only: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  The HIP package never imports it.

Inputs are numpy arrays; every floating-point input is widened exactly to float64
before the call (fp32 and bf16 values are exact in fp64), and every result comes
back as float64.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "uq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FMT_FP8_E4M3 = 0
FMT_FP4_E4M3S = 1
FMT_FP4_UE8M0S = 2
FMT_FP8_E4M3_TOK = 3


def build(force: bool = True) -> str:
    """Compile ``uq_oracle.c`` with gcc (IEEE fp64, OpenMP) into ``liboracle.so``."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out_dir: str) -> str:
    """The same library with AddressSanitizer and UndefinedBehaviorSanitizer (gcc); load it
    through $UQ_ORACLE_LIB with gcc's libasan preloaded."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "liboracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", lib, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = os.environ.get("UQ_ORACLE_LIB")   # a planted-mistake build (mutation tests)
        if not path:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build()
            path = _LIB_PATH
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.uqo_num_threads.restype = ctypes.c_int
        lib.uqo_num_threads.argtypes = []
        lib.uqo_e4m3.restype = f64
        lib.uqo_e4m3.argtypes = [ctypes.c_uint32]
        lib.uqo_e2m1.restype = f64
        lib.uqo_e2m1.argtypes = [ctypes.c_uint32]
        lib.uqo_ue8m0.restype = f64
        lib.uqo_ue8m0.argtypes = [ctypes.c_uint32]
        lib.uqo_slot_content_bytes.restype = i32
        lib.uqo_slot_content_bytes.argtypes = [i32, i32]
        lib.uqo_rotate.restype = None
        lib.uqo_rotate.argtypes = [P, P, i32, P]
        lib.uqo_decode.restype = i32
        lib.uqo_decode.argtypes = [P, i64, i64, P, i64, i32, i32, i32, i32, f64, f64, P,
                                   P, i32, P, i32, i32, i32, f64, P, i32, P, P, P]
        lib.uqo_decode_q.restype = i32
        lib.uqo_decode_q.argtypes = [P, i64, i64, P, i64, i32, i32, i32, i32, f64, f64, P,
                                     P, P, P, i32, P, i32, i32, i32, i32, f64, P, i32, P, P,
                                     P]
        lib.uqo_reduce.restype = None
        lib.uqo_reduce.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P]
        lib.uqo_reduce_q.restype = None
        lib.uqo_reduce_q.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, P]
        lib.uqo_index_score.restype = i32
        lib.uqo_index_score.argtypes = [P, i64, i64, P, i64, i64, P, i32, P, i32, i32, i32,
                                        i32, P, i64, i64]
        _lib = lib
        return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ codecs


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().uqo_num_threads())


def e4m3(code: int) -> float:
    return _load().uqo_e4m3(int(code))


def e2m1(nibble: int) -> float:
    return _load().uqo_e2m1(int(nibble))


def ue8m0(code: int) -> float:
    return _load().uqo_ue8m0(int(code))


def slot_content_bytes(kv_format: int, head_dim: int) -> int:
    return int(_load().uqo_slot_content_bytes(kv_format, head_dim))


def rotate(q: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """q' = (q * signs) H / sqrt(D) for a single vector q of length D."""
    q = _c(q, np.float64)
    s = _c(signs, np.int8)
    out = np.empty_like(q)
    _load().uqo_rotate(_ptr(q), _ptr(s), q.shape[0], _ptr(out))
    return out


# ------------------------------------------------------------------ decode


def decode(q: np.ndarray, cache: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
           *, num_kv_heads: int, kv_format: int, softmax_scale: float,
           k_scale: float = 1.0, v_scale: float = 1.0, rot_signs: np.ndarray | None = None,
           num_partitions: int = 0, query_len: int = 1,
           k_scale_tok: np.ndarray | None = None, v_scale_tok: np.ndarray | None = None):
    """Masked-softmax decode attention in fp64, query_len query rows per sequence.

    q: [B*QL, Hq, D] (any float dtype; widened exactly; row b*QL + j is query j of sequence
    b, which sees tokens t < L_b - QL + 1 + j), cache: [num_blocks, BS, Hk, slot] uint8,
    block_table: [B, max_blocks] int32, seq_lens: [B] int32.
    Returns out [B*QL, Hq, D] float64, and (part_m, part_l, part_o) when num_partitions > 0
    (shapes [B, Hk, P, QL*QG], [B, Hk, P, QL*QG], [B, Hk, P, QL*QG, D]; row j*QG + g).
    With kv_format FMT_FP8_E4M3_TOK, k_scale_tok / v_scale_tok are the float32 per-token
    scales [num_blocks, Hk, BS] (k_scale / v_scale then stay 1).
    """
    q = _c(q, np.float64)
    rows, Hq, D = q.shape
    QL = int(query_len)
    cache = np.ascontiguousarray(cache, dtype=np.uint8)
    nb, bs, hk, slot = cache.shape
    assert hk == num_kv_heads
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    B = sl.shape[0]
    assert QL >= 1 and rows == B * QL and bt.shape[0] == B
    QG = Hq // hk
    P = int(num_partitions)
    out = np.zeros((B * QL, Hq, D), np.float64)
    pm = np.zeros((B, hk, max(P, 1), QL * QG), np.float64)
    pl = np.zeros_like(pm)
    po = np.zeros((B, hk, max(P, 1), QL * QG, D), np.float64)
    rot = None if rot_signs is None else _c(rot_signs, np.int8)
    kt = vt = None
    if kv_format == FMT_FP8_E4M3_TOK:
        kt = _c(k_scale_tok, np.float32)
        vt = _c(v_scale_tok, np.float32)
        assert kt.shape == (nb, hk, bs) and vt.shape == (nb, hk, bs)
    st = _load().uqo_decode_q(_ptr(q), Hq * D, D, _ptr(cache), nb, bs, hk, slot, kv_format,
                              float(k_scale), float(v_scale), _ptr(kt), _ptr(vt), _ptr(rot),
                              _ptr(bt), bt.shape[1],
                              _ptr(sl), B, QL, Hq, D, float(softmax_scale), _ptr(out), P,
                              _ptr(pm), _ptr(pl), _ptr(po))
    if st != 0:
        raise ValueError(f"oracle decode rejected its inputs (status {st})")
    if P > 0:
        return out, (pm, pl, po)
    return out


def reduce(part_o: np.ndarray, part_m: np.ndarray, part_l: np.ndarray,
           seq_lens: np.ndarray, query_len: int = 1) -> np.ndarray:
    """Flash-combine of partials [B, Hk, P, QL*QG(, D)] (row j*QG + g) into
    [B*QL, Hk*QG, D] (fp64)."""
    po = _c(part_o, np.float64)
    pm = _c(part_m, np.float64)
    pl = _c(part_l, np.float64)
    sl = _c(seq_lens, np.int32)
    B, Hk, P, QR, D = po.shape
    QL = int(query_len)
    assert QL >= 1 and QR % QL == 0
    QG = QR // QL
    out = np.zeros((B * QL, Hk * QG, D), np.float64)
    _load().uqo_reduce_q(_ptr(po), _ptr(pm), _ptr(pl), _ptr(sl), B, Hk, QL, QG, D, P,
                         _ptr(out))
    return out


# ------------------------------------------------------------------ index scorer


def index_score(q_codes: np.ndarray, pages: np.ndarray, block_table: np.ndarray,
                seq_lens: np.ndarray, *, query_len: int, scores_init: np.ndarray):
    """nvfp4 index scores in fp64.

    q_codes: e4m3 [num_reqs*QL, H, D] uint8; pages: [num_pages, page_stride] uint8;
    block_table: [num_reqs, >= max pages] int32; seq_lens [num_reqs] int32;
    scores_init: [H, num_reqs*QL, S] array whose untouched cells are returned as given.
    """
    q = np.ascontiguousarray(q_codes, dtype=np.uint8)
    rows, H, D = q.shape
    pages = np.ascontiguousarray(pages, dtype=np.uint8)
    npg, pstride = pages.shape
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    R = sl.shape[0]
    assert rows == R * query_len
    sc = np.array(scores_init, dtype=np.float64, copy=True, order="C")
    Hs, rows_s, S = sc.shape
    assert Hs == H and rows_s == rows
    st = _load().uqo_index_score(_ptr(q), H * D, D, _ptr(pages), pstride, npg, _ptr(bt),
                                 bt.shape[1], _ptr(sl), R, query_len, H, D, _ptr(sc),
                                 rows * S, S)
    if st != 0:
        raise ValueError(f"oracle index_score rejected its inputs (status {st})")
    return sc
