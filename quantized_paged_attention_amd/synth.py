"""Seeded synthetic workloads for quantized paged-attention decode and the nvfp4 scorer.

This module only draws random numbers and lays bytes out; it holds none of the
attention or scoring arithmetic.  Values are placed on the fp8 / fp4 code grids by
library casts (torch's float8_e4m3fn) or by nearest-grid rounding, which is how a
cache would be populated -- the decode path itself only ever decodes codes.

Both the HIP path (through the binding) and the fp64 oracle consume the arrays built
here; neither side computes any input for the other.

Workloads (shapes of the pages' decode and scorer problems):
  tiny_fp8   B=2, Hk=1, QG=8, D=128, L={37,200}, block 16, e4m3 K/V from N(0,1),
             fp32 Q, 1 partition, table permuted over 32 blocks (16 poison)
  fp8_mid    B=16, Hk=8, QG=8, D=128, L=16384, block 16, uniform finite e4m3 codes,
             k_scale 0.05, v_scale 0.02, bf16 Q, 64 partitions of 256 tokens
  fp8_high   B=128, same cache format, L ~ U[4096, 16384], random non-contiguous table
  fp4_d256   B=4, Hk=2, QG in {6,8,16}, D=256, L=75000, block 64, 272-byte slot,
             e2m1 codes with e4m3 scales per 32 dims, rotated-domain K, 512 partitions
  nvfp4_idx  32 requests, QL in {1,2,4,8}, H in {1,2,4}, D=128, L ~ U[1024, 32768],
             128-token pages of 64 code bytes + 8 e4m3 scales per token
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

# 254 finite OCP e4m3 codes (0x7F and 0xFF are the two NaN encodings)
E4M3_FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
POISON_BYTE = 0x7F      # NaN as e4m3; as two e2m1 nibbles it is (6.0, -6.0)
SCORE_POISON_BITS = 0x7FC0DEAD   # quiet NaN with a payload, pre-filled into score outputs

# OCP e2m1 magnitudes by 3-bit magnitude code (specification grid; generator-only use)
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)

FMT_FP8_E4M3 = 0
FMT_FP8_E4M3_TOK = 3
FMT_FP4_E2M1_E4M3S = 1
FMT_FP4_E2M1_UE8M0S = 2

TILE_GROUP = 256


# ------------------------------------------------------------------ grid placement


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returned as float32."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 codes (torch's float8_e4m3fn cast) after clipping to +-448."""
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_values(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).float().numpy()


def e4m3_scale_at_least(x: np.ndarray) -> np.ndarray:
    """Smallest positive e4m3 code whose value is >= x (x > 0, x <= 448)."""
    x = np.asarray(x, np.float32)
    c = e4m3_encode(x).astype(np.int32)
    c = np.maximum(c, 1)
    v = _e4m3_values(c.astype(np.uint8))
    c = np.where(v < x, c + 1, c)
    return np.minimum(c, 0x7E).astype(np.uint8)


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e2m1 nibble (saturating at +-6, ties to the even mantissa)."""
    a = np.minimum(np.abs(x), 6.0).astype(np.float32)
    # midpoints between successive grid magnitudes; ties go to the even code
    mids = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2
    idx = np.searchsorted(mids, a, side="left")            # a <= mid -> lower code
    tie = np.isin(a, mids)
    up_on_tie = (np.searchsorted(mids, a, side="left") % 2 == 1)  # lower code odd -> go up
    idx = np.where(tie & up_on_tie, idx + 1, idx)
    sign = (np.signbit(x) & (idx > 0)).astype(np.uint8)
    return (idx.astype(np.uint8) | (sign << 3)).astype(np.uint8)


def pack_nibbles(n: np.ndarray) -> np.ndarray:
    """[..., 2k] nibbles -> [..., k] bytes, element 2i in the low nibble of byte i."""
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def fp4_quantize(x: np.ndarray, group: int, scale_kind: str):
    """Block-scaled e2m1 codes of x [..., D]: per `group` dims a scale S with
    amax / S <= 6, then nearest e2m1 of x / S.  scale_kind 'e4m3' or 'ue8m0'.
    Returns (packed codes [..., D/2], scale bytes [..., D/group])."""
    shp = x.shape
    D = shp[-1]
    xg = x.reshape(*shp[:-1], D // group, group).astype(np.float32)
    amax = np.abs(xg).max(axis=-1)
    need = np.maximum(amax / 6.0, 2.0 ** -9)
    if scale_kind == "e4m3":
        sc_codes = e4m3_scale_at_least(need)
        sc_vals = _e4m3_values(sc_codes)
    elif scale_kind == "ue8m0":
        e = np.ceil(np.log2(need)).astype(np.int32)
        sc_codes = np.clip(e + 127, 1, 254).astype(np.uint8)
        sc_vals = np.ldexp(np.float32(1.0), sc_codes.astype(np.int32) - 127).astype(np.float32)
    else:
        raise ValueError(scale_kind)
    nib = e2m1_encode(xg / sc_vals[..., None]).reshape(shp)
    return pack_nibbles(nib), sc_codes


# ------------------------------------------------------------------ decode workloads


@dataclasses.dataclass
class DecodeCase:
    name: str
    q: np.ndarray               # [B*QL, Hq, D] float32 (bf16-representable when q_dtype == 'bf16')
    q_dtype: str                # 'f32' or 'bf16'
    cache: np.ndarray           # [num_blocks, block_size, Hk, slot_bytes] uint8
    block_table: np.ndarray     # [B, max_blocks] int32, -1 past each sequence's blocks
    seq_lens: np.ndarray        # [B] int32
    num_kv_heads: int
    kv_format: int
    softmax_scale: float
    k_scale: float
    v_scale: float
    num_partitions: int
    rot_signs: np.ndarray | None = None   # [D] int8 of +-1 (fp4 rotated-K workloads)
    query_len: int = 1          # query rows per sequence (row b*QL + j: query j of b)
    k_scale_tok: np.ndarray | None = None  # [num_blocks, Hk, block_size] float32 (per-token)
    v_scale_tok: np.ndarray | None = None

    @property
    def B(self):
        return self.seq_lens.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def QG(self):
        return self.Hq // self.num_kv_heads

    @property
    def block_size(self):
        return self.cache.shape[1]

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes of one decode: every visible slot's content, once."""
        if self.kv_format == FMT_FP8_E4M3:
            content = 2 * self.D
        elif self.kv_format == FMT_FP8_E4M3_TOK:
            content = 2 * self.D + 8          # codes plus one f32 K and one f32 V scale
        else:
            content = 2 * (self.D // 2 + self.D // 32)
        return int(self.seq_lens.astype(np.int64).sum()) * self.num_kv_heads * content


def _table_and_blocks(rng, seq_lens, block_size, spare_blocks, max_blocks=None):
    """Random permuted physical ids for every sequence's blocks, plus spare blocks that
    no table row references.  Returns (block_table, num_blocks, used mask per block)."""
    nblk = [(int(L) + block_size - 1) // block_size for L in seq_lens]
    used = sum(nblk)
    num_blocks = used + spare_blocks
    perm = rng.permutation(num_blocks).astype(np.int32)
    mb = max(max(nblk) if nblk else 1, 1) if max_blocks is None else max_blocks
    bt = np.full((len(seq_lens), mb), -1, np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt, num_blocks, perm[:used]


def _poison(cache, bt, seq_lens, used_ids):
    """Unreferenced blocks and every slot past a sequence's length in its last block
    are filled with the NaN byte, so any read of them shows up in the result."""
    nb, bs = cache.shape[:2]
    mask = np.ones(nb, bool)
    mask[used_ids] = False
    cache[mask] = POISON_BYTE
    for b, L in enumerate(seq_lens):
        L = int(L)
        if L % bs:
            cache[bt[b, L // bs], L % bs:] = POISON_BYTE


def _tok_scale_poison(sc, bt, seq_lens, used_ids):
    """NaN in the per-token scales of unreferenced blocks and of positions past a
    sequence's length in its last block (they must never be used)."""
    nb, _, bs = sc.shape
    mask = np.ones(nb, bool)
    mask[used_ids] = False
    sc[mask] = np.nan
    for b, L in enumerate(seq_lens):
        L = int(L)
        if L % bs:
            sc[bt[b, L // bs], :, L % bs:] = np.nan


def make_fp8_case(name, seed, *, seq_lens, num_kv_heads, qg, head_dim=128, block_size=16,
                  q_dtype="bf16", values="uniform_codes", k_scale=1.0, v_scale=1.0,
                  num_partitions=None, spare_blocks=None, slot_bytes=None,
                  softmax_scale=None, max_blocks=None, query_len=1, scales="tensor",
                  tok_spread=0.5, v_ramp=0.0) -> DecodeCase:
    """fp8 e4m3 cache in the AoS slot [K codes D | V codes D].

    scales="tensor": one per-tensor K and V scale (k_scale, v_scale).
    scales="token": one float32 K and V scale per (physical block, kv head, position)
    ([num_blocks, Hk, block_size]).  With values="normal" every token's K (V) row is
    x ~ sigma N(0,1), sigma lognormal(0, tok_spread), quantised as a per-token cache is
    filled: scale = max|x| / 448, codes = e4m3(x / scale).  With values="uniform_codes"
    the codes are uniform over the finite e4m3 codes and the scales are k_scale (v_scale)
    times lognormal(0, tok_spread).  v_ramp > 0 multiplies the V scale of logical token t
    of every sequence by 2^(v_ramp t / 256), so later tokens carry ever larger V scales."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, np.int32)
    B, Hk, D = len(seq_lens), num_kv_heads, head_dim
    slot = slot_bytes or 2 * D
    if spare_blocks is None:
        spare_blocks = 0
    bt, nb, used = _table_and_blocks(rng, seq_lens, block_size, spare_blocks, max_blocks)
    shape = (nb, block_size, Hk, slot)
    kst = vst = None
    if scales == "token":
        tshape = (nb, Hk, block_size)
        if values == "uniform_codes":
            cache = E4M3_FINITE_CODES[rng.integers(0, 254, size=shape, dtype=np.uint8)]
            kst = (k_scale * np.exp(tok_spread * rng.standard_normal(tshape))).astype(np.float32)
            vst = (v_scale * np.exp(tok_spread * rng.standard_normal(tshape))).astype(np.float32)
        elif values == "normal":
            cache = np.zeros(shape, np.uint8)
            kst = np.zeros(tshape, np.float32)
            vst = np.zeros(tshape, np.float32)
            for o, sc in ((0, kst), (D, vst)):
                sig = np.exp(tok_spread * rng.standard_normal((nb, block_size, Hk, 1)))
                x = (sig * rng.standard_normal((nb, block_size, Hk, D))).astype(np.float32)
                amax = np.abs(x).max(axis=-1)                     # [nb, bs, Hk]
                s_tok = np.maximum(amax / 448.0, 1e-30).astype(np.float32)
                cache[..., o:o + D] = e4m3_encode(x / s_tok[..., None])
                sc[...] = s_tok.transpose(0, 2, 1)
        else:
            raise ValueError(values)
        if v_ramp:
            for b, L in enumerate(seq_lens):
                t = np.arange(int(L))
                blk = bt[b, t // block_size]
                vst[blk, :, t % block_size] *= np.exp2(v_ramp * t / 256.0).astype(
                    np.float32)[:, None]
        _tok_scale_poison(kst, bt, seq_lens, used)
        _tok_scale_poison(vst, bt, seq_lens, used)
        fmt, k_scale, v_scale = FMT_FP8_E4M3_TOK, 1.0, 1.0
    elif scales == "tensor":
        fmt = FMT_FP8_E4M3
        if values == "uniform_codes":
            cache = E4M3_FINITE_CODES[rng.integers(0, 254, size=shape, dtype=np.uint8)]
        elif values == "normal":
            cache = np.zeros(shape, np.uint8)
            x = rng.standard_normal((nb, block_size, Hk, 2 * D), dtype=np.float32)
            cache[..., :2 * D] = e4m3_encode(x)
        else:
            raise ValueError(values)
    else:
        raise ValueError(scales)
    _poison(cache, bt, seq_lens, used)
    q = rng.standard_normal((B * query_len, Hk * qg, D), dtype=np.float32)
    if q_dtype == "bf16":
        q = bf16_round(q)
    P = num_partitions or max(1, -(-int(seq_lens.max()) // TILE_GROUP))
    return DecodeCase(name, q, q_dtype, cache, bt, seq_lens, Hk, fmt,
                      softmax_scale or 1.0 / math.sqrt(D), k_scale, v_scale, P,
                      query_len=query_len, k_scale_tok=kst, v_scale_tok=vst)


def make_fp4_case(name, seed, *, seq_lens, num_kv_heads, qg, head_dim=256, block_size=64,
                  scale_kind="e4m3", rotate=True, num_partitions=None, spare_blocks=16,
                  slot_bytes=None, softmax_scale=None, q_dtype="bf16",
                  query_len=1) -> DecodeCase:
    """fp4 e2m1 cache with 32-dim group scales in the 272-byte AoS slot
    [Kc D/2 | Ks D/32 | Vc D/2 | Vs D/32].  With `rotate`, K is drawn directly in the
    rotated domain: for iid N(0,1) keys k and an orthogonal R, kR is again iid N(0,1),
    so drawing N(0,1) there is the same distribution as rotating N(0,1) keys."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, np.int32)
    B, Hk, D = len(seq_lens), num_kv_heads, head_dim
    content = 2 * (D // 2 + D // 32)
    slot = slot_bytes or content
    bt, nb, used = _table_and_blocks(rng, seq_lens, block_size, spare_blocks)
    cache = np.zeros((nb, block_size, Hk, slot), np.uint8)
    fmt = FMT_FP4_E2M1_E4M3S if scale_kind == "e4m3" else FMT_FP4_E2M1_UE8M0S
    chunk = max(1, (1 << 22) // (block_size * Hk * D))
    for b0 in range(0, nb, chunk):
        b1 = min(nb, b0 + chunk)
        k = rng.standard_normal((b1 - b0, block_size, Hk, D), dtype=np.float32)
        v = rng.standard_normal((b1 - b0, block_size, Hk, D), dtype=np.float32)
        kc, ks = fp4_quantize(k, 32, scale_kind)
        vc, vs = fp4_quantize(v, 32, scale_kind)
        o = 0
        for part in (kc, ks, vc, vs):
            w = part.shape[-1]
            cache[b0:b1, :, :, o:o + w] = part
            o += w
    _poison(cache, bt, seq_lens, used)
    q = rng.standard_normal((B * query_len, Hk * qg, D), dtype=np.float32)
    if q_dtype == "bf16":
        q = bf16_round(q)
    signs = (rng.integers(0, 2, size=D) * 2 - 1).astype(np.int8) if rotate else None
    P = num_partitions or max(1, -(-int(seq_lens.max()) // TILE_GROUP))
    return DecodeCase(name, q, q_dtype, cache, bt, seq_lens, Hk, fmt,
                      softmax_scale or 1.0 / math.sqrt(D), 1.0, 1.0, P, signs,
                      query_len=query_len)


def tiny_fp8() -> DecodeCase:
    return make_fp8_case("tiny_fp8", 1, seq_lens=[37, 200], num_kv_heads=1, qg=8,
                         q_dtype="f32", values="normal", num_partitions=1, spare_blocks=16)


def fp8_mid() -> DecodeCase:
    return make_fp8_case("fp8_mid", 2, seq_lens=[16384] * 16, num_kv_heads=8, qg=8,
                         k_scale=0.05, v_scale=0.02, num_partitions=64)


def fp8_high_seq_lens(seed=3, B=128):
    return np.random.default_rng(seed + 1000).integers(4096, 16385, size=B).astype(np.int32)


def fp8_high() -> DecodeCase:
    return make_fp8_case("fp8_high", 3, seq_lens=fp8_high_seq_lens(), num_kv_heads=8, qg=8,
                         k_scale=0.05, v_scale=0.02, num_partitions=64, spare_blocks=256,
                         max_blocks=1024)


def fp8_high_tok() -> DecodeCase:
    """The high-batch fp8 shape (same lengths and table) with per-token K and V scales:
    uniform finite e4m3 codes, scales 0.05 (K) and 0.02 (V) times lognormal(0, 0.5)."""
    return make_fp8_case("fp8_high_tok", 3, seq_lens=fp8_high_seq_lens(), num_kv_heads=8,
                         qg=8, k_scale=0.05, v_scale=0.02, num_partitions=64,
                         spare_blocks=256, max_blocks=1024, scales="token")


def fp8_high_mtp(query_len=2, qg=4) -> DecodeCase:
    """The high-batch fp8 shape (same lengths, table and cache recipe) with query_len
    query rows per sequence and qg query heads per kv head."""
    return make_fp8_case(f"fp8_high_mtp{query_len}_qg{qg}", 3, seq_lens=fp8_high_seq_lens(),
                         num_kv_heads=8, qg=qg, k_scale=0.05, v_scale=0.02, num_partitions=64,
                         spare_blocks=256, max_blocks=1024, query_len=query_len)


def fp4_d256_mtp(query_len=2, qg=8, scale_kind="e4m3") -> DecodeCase:
    """The FP4 D=256 shape with query_len query rows per sequence."""
    tag = "" if scale_kind == "e4m3" else "_ue8m0"
    return make_fp4_case(f"fp4_d256_mtp{query_len}_qg{qg}{tag}", 4, seq_lens=[75000] * 4,
                         num_kv_heads=2, qg=qg, head_dim=256, block_size=64,
                         num_partitions=512, softmax_scale=1.0 / 16.0, scale_kind=scale_kind,
                         query_len=query_len)


def fp4_d256(qg=16, scale_kind="e4m3") -> DecodeCase:
    tag = "" if scale_kind == "e4m3" else "_ue8m0"
    return make_fp4_case(f"fp4_d256_qg{qg}{tag}", 4, seq_lens=[75000] * 4, num_kv_heads=2, qg=qg,
                         head_dim=256, block_size=64, num_partitions=512,
                         softmax_scale=1.0 / 16.0, scale_kind=scale_kind)


# ------------------------------------------------------------------ index workloads

INDEX_PAGE = 128


@dataclasses.dataclass
class IndexCase:
    name: str
    q: np.ndarray             # e4m3 codes [num_reqs*QL, H, D] uint8
    pages: np.ndarray         # [num_pages, page_stride] uint8
    block_table: np.ndarray   # [num_reqs, max_pages] int32
    seq_lens: np.ndarray      # [num_reqs] int32
    query_len: int
    heads: int
    max_pages: int            # S, the score row length

    @property
    def num_reqs(self):
        return self.seq_lens.shape[0]

    @property
    def D(self):
        return self.q.shape[2]

    def scores_init(self) -> np.ndarray:
        s = np.empty((self.heads, self.num_reqs * self.query_len, self.max_pages), np.uint32)
        s.fill(SCORE_POISON_BITS)
        return s.view(np.float32)

    def unique_page_bytes(self) -> int:
        """Algorithmic bytes when pages that several requests map to are read once: per
        distinct page, its visible tokens (the most any referencing request sees) x 72."""
        vis = {}
        for r, L in enumerate(self.seq_lens):
            L = int(L)
            for b in range(-(-L // INDEX_PAGE)):
                pid = int(self.block_table[r, b])
                vis[pid] = max(vis.get(pid, 0), min(INDEX_PAGE, L - b * INDEX_PAGE))
        return sum(vis.values()) * (self.D // 2 + self.D // 16)

    def page_bytes(self) -> int:
        """Algorithmic bytes: every visible token's 72 bytes (codes + scales), once."""
        return int(self.seq_lens.astype(np.int64).sum()) * (self.D // 2 + self.D // 16)


def make_index_case(name, seed, *, seq_lens, query_len, heads, head_dim=128, page_stride=None,
                    spare_pages=8, max_pages=None) -> IndexCase:
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, np.int32)
    D = head_dim
    content = INDEX_PAGE * (D // 2 + D // 16)
    stride = page_stride or content
    bt, npg, used = _table_and_blocks(rng, seq_lens, INDEX_PAGE, spare_pages, max_pages)
    pages = np.zeros((npg, stride), np.uint8)
    chunk = 256
    for p0 in range(0, npg, chunk):
        p1 = min(npg, p0 + chunk)
        k = rng.standard_normal((p1 - p0, INDEX_PAGE, D), dtype=np.float32)
        codes, sc = fp4_quantize(k, 16, "e4m3")
        pages[p0:p1, :INDEX_PAGE * D // 2] = codes.reshape(p1 - p0, -1)
        pages[p0:p1, INDEX_PAGE * D // 2:content] = sc.reshape(p1 - p0, -1)
    # unreferenced pages and the tail tokens of each request's last page -> NaN scales
    mask = np.ones(npg, bool)
    mask[used] = False
    pages[mask, :content] = POISON_BYTE
    for r, L in enumerate(seq_lens):
        L = int(L)
        if L % INDEX_PAGE:
            pg = bt[r, L // INDEX_PAGE]
            t0 = L % INDEX_PAGE
            pages[pg, t0 * D // 2:INDEX_PAGE * D // 2] = POISON_BYTE
            pages[pg, INDEX_PAGE * D // 2 + t0 * D // 16:content] = POISON_BYTE
    R = len(seq_lens)
    q = e4m3_encode(rng.standard_normal((R * query_len, heads, D), dtype=np.float32))
    S = max_pages or bt.shape[1]
    return IndexCase(name, q, pages, bt, seq_lens, query_len, heads, S)


def index_shared_prefix(case: IndexCase, prefix_pages: int) -> IndexCase:
    """The same requests, but every request's first prefix_pages table entries point at
    request 0's pages (a shared prompt prefix, as a prefix cache lays out).  Requires
    every request to be longer than the prefix; the pages other requests held there are
    left unreferenced."""
    c = dataclasses.replace(case, block_table=case.block_table.copy())
    assert int(c.seq_lens.min()) > prefix_pages * INDEX_PAGE
    c.block_table[:, :prefix_pages] = c.block_table[0, :prefix_pages]
    c.name = f"{case.name}_shared{prefix_pages}"
    return c


def nvfp4_index_shared(query_len=8, heads=4, prefix_pages=64, seed=6) -> IndexCase:
    """32 requests, L ~ U[prefix + 1024, 32768], sharing their first prefix_pages pages
    (8192 tokens at 64)."""
    lo = prefix_pages * INDEX_PAGE + 1024
    lens = np.random.default_rng(seed + 1000).integers(lo, 32769, size=32).astype(np.int32)
    base = make_index_case(f"nvfp4_index_ql{query_len}_h{heads}", seed, seq_lens=lens,
                           query_len=query_len, heads=heads, page_stride=9216)
    return index_shared_prefix(base, prefix_pages)


def nvfp4_index(query_len=8, heads=4, seed=5) -> IndexCase:
    seq_lens = np.random.default_rng(seed + 1000).integers(1024, 32769, size=32).astype(np.int32)
    return make_index_case(f"nvfp4_idx_ql{query_len}_h{heads}", seed, seq_lens=seq_lens,
                           query_len=query_len, heads=heads, max_pages=256)


INDEX_COMBOS = [(ql, h) for ql in (1, 2, 4, 8) for h in (1, 2, 4) if ql * h <= 32]
