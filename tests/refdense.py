"""Test-side helpers that are independent of the oracle: golden-file reader and a dense
re-gather of a paged cache decoded with library casts (torch float8_e4m3fn) and the
OCP e2m1 specification grid, using the byte offsets recorded in tests/golden/."""

from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# OCP FP4 E2M1 value of each nibble (specification grid, sign in bit 3)
E2M1_SPEC = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                      -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], np.float64)


def golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(None, 1)
            out[k] = float(v) if any(c in v for c in ".e") else int(v)
    return out


def e4m3_lib(codes: np.ndarray) -> np.ndarray:
    """e4m3 values via torch's float8_e4m3fn (an independent library decode)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    lo = packed & 15
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    return E2M1_SPEC[nib]


def dense_kv(case, b: int, h: int):
    """Decoded K [L, D] and V [L, D] of sequence b, kv head h (fp64), gathered through
    the block table with numpy fancy indexing."""
    L = int(case.seq_lens[b])
    bs = case.block_size
    t = np.arange(L)
    blk = case.block_table[b, t // bs]
    slots = case.cache[blk, t % bs, h]          # [L, slot_bytes]
    D = case.D
    if case.kv_format == 0:
        return e4m3_lib(slots[:, :D]), e4m3_lib(slots[:, D:2 * D])
    if case.kv_format == 3:
        # per-token scales indexed [physical block, kv head, position in block]
        ks = case.k_scale_tok[blk, h, t % bs].astype(np.float64)
        vs = case.v_scale_tok[blk, h, t % bs].astype(np.float64)
        return e4m3_lib(slots[:, :D]) * ks[:, None], e4m3_lib(slots[:, D:2 * D]) * vs[:, None]
    lay = golden("p1_fp4_slot_layout.txt")
    assert D == lay["head_dim"]
    grp = lay["scale_group_dims"]
    kc = slots[:, lay["k_codes_offset"]:lay["k_codes_offset"] + D // 2]
    ks = slots[:, lay["k_scales_offset"]:lay["k_scales_offset"] + D // grp]
    vc = slots[:, lay["v_codes_offset"]:lay["v_codes_offset"] + D // 2]
    vs = slots[:, lay["v_scales_offset"]:lay["v_scales_offset"] + D // grp]
    if case.kv_format == 1:
        ksv, vsv = e4m3_lib(ks), e4m3_lib(vs)
    else:
        ksv = np.ldexp(1.0, ks.astype(np.int64) - 127)
        vsv = np.ldexp(1.0, vs.astype(np.int64) - 127)
    k = unpack_e2m1(kc) * np.repeat(ksv, grp, axis=1)
    v = unpack_e2m1(vc) * np.repeat(vsv, grp, axis=1)
    return k, v


def sylvester_rotation(signs: np.ndarray) -> np.ndarray:
    """R = diag(signs) H / sqrt(D) with scipy's Sylvester Hadamard matrix."""
    from scipy.linalg import hadamard
    D = signs.shape[0]
    return (signs.astype(np.float64)[:, None] * hadamard(D).astype(np.float64)) / np.sqrt(D)


def sdpa_reference(case) -> np.ndarray:
    """torch scaled_dot_product_attention (fp64, CPU) over the dense gathered cache.  With
    query_len QL, query row j of sequence b attends under a boolean mask to the tokens
    t <= L_b - QL + j; a row that sees no token is zero."""
    B, Hq, D, Hk, QG = case.B, case.Hq, case.D, case.num_kv_heads, case.QG
    QL = getattr(case, "query_len", 1)
    q = case.q.astype(np.float64)
    if case.rot_signs is not None:
        q = q @ sylvester_rotation(case.rot_signs)
    out = np.zeros((B * QL, Hq, D))
    for b in range(B):
        L = int(case.seq_lens[b])
        if L == 0:
            continue
        for h in range(Hk):
            k, v = dense_kv(case, b, h)
            kt = torch.from_numpy(k)[None].expand(QG, -1, -1)
            vt = torch.from_numpy(v)[None].expand(QG, -1, -1)
            for j in range(QL):
                last = L - QL + j                      # last visible token of row j
                if last < 0:
                    continue
                mask = torch.from_numpy(np.arange(L) <= last)[None, None, :].expand(QG, 1, -1)
                qt = torch.from_numpy(q[b * QL + j, h * QG:(h + 1) * QG])[:, None, :]
                o = torch.nn.functional.scaled_dot_product_attention(
                    qt, kt, vt, attn_mask=mask, scale=case.softmax_scale * case.k_scale)
                out[b * QL + j, h * QG:(h + 1) * QG] = o[:, 0].numpy() * case.v_scale
    return out


def index_reference(case) -> np.ndarray:
    """Per-page masked max of q.k with numpy matmuls over the decoded pages."""
    lay = golden("p2_index_page_layout.txt")
    T, cb, sb, g = (lay["tokens_per_page"], lay["code_bytes_per_token"],
                    lay["scale_bytes_per_token"], lay["scale_group_dims"])
    q = e4m3_lib(case.q)                                     # [R*QL, H, D]
    out = case.scores_init().astype(np.float64)
    QL = case.query_len
    for r in range(case.num_reqs):
        L = int(case.seq_lens[r])
        for b in range((L + T - 1) // T):
            pg = case.pages[case.block_table[r, b]]
            codes = pg[:T * cb].reshape(T, cb)
            sc = pg[lay["scale_region_offset"]:lay["scale_region_offset"] + T * sb].reshape(T, sb)
            k = unpack_e2m1(codes) * np.repeat(e4m3_lib(sc), g, axis=1)   # [T, D]
            for j in range(QL):
                lim = L - QL + j
                n_vis = min(T, lim - b * T + 1)
                for h in range(case.heads):
                    if n_vis <= 0:
                        out[h, r * QL + j, b] = -np.inf
                    else:
                        out[h, r * QL + j, b] = (k[:n_vis] @ q[r * QL + j, h]).max()
    return out
