"""Byte layouts of the quantized cache, written out plainly for the oracle.

Test infrastructure: see the package docstring.

The pages fix no byte layout (the TurboQuant page's bit format in section 3.3
is garbled), so the layout is this library's own contract.  It is stated
here, independently of the HIP code, and pinned by tests on hand-built
examples.  Head dimension d = 128.

Segment packing -- 32 codes u = 8*m + e (block m = 0..3, element e = 0..7)
into 4*bits bytes:

* 8-bit: byte u holds code u (two's complement for q8_0).
* 4-bit: byte j holds code 2j in its low nibble and code 2j+1 in its high
  nibble (so the little-endian dword m holds block m, element e at bits 4e).
* 3-bit: three little-endian dwords D0, D1, D2.  For block m and r = 0..3
  the pair (u_a, u_b) = (8m + r, 8m + r + 4) is stored as: the low two bits
  of u_a at bit 2p and of u_b at bit 16 + 2p of D[m // 2], where
  p = 4 * (m % 2) + r; the high bit of u_a at bit H and of u_b at bit 16 + H
  of D2, where H = 8 * (m // 2) + 2r + (m % 2).  (After one shift per block,
  pair r's low bits sit at 2r and its high bit at 2r + 2, so both planes
  carry the same per-pair factor 4^r.)

Key rows ("K-row" layout): every token has a row of 16*bits bytes made of 4
segments q = 0..3; segment q holds channels c = 32m + 8q + e.

Value tiles ("V-tile" layout): tokens are grouped in tiles of 32.  A tile is
64 "lanes" L = 16q + i of 8*bits bytes each (two segments s = 0, 1).  In lane
L, segment s, block m holds channel 16*(4s + m) + i; element e of that block
is token 4q + e (e < 4) or 16 + 4q + (e - 4) (e >= 4) of the tile.

Capacity: the cache holds Tcap = round_up(max_ctx, 1024) tokens per sequence
(``capacity``), a multiple of the 32-token tile.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

D = 128


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def capacity(max_ctx: int) -> int:
    """Token capacity per (sequence, KV head) of the library's allocation:
    max_ctx rounded up to a multiple of 1024 (a layout choice of the
    library: the row stride between (sequence, head) streams then stays a
    multiple of 1024 tokens)."""
    return round_up(max_ctx, 1024)


def row_bytes(bits: int) -> int:
    return D * bits // 8


def pack_segment(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., 32] (ints, already reduced to ``bits`` bits) -> bytes [..., 4*bits]."""
    c = np.asarray(codes).astype(np.int64) & ((1 << bits) - 1)
    lead = c.shape[:-1]
    if bits == 8:
        return c.astype(np.uint8)
    if bits == 4:
        return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    if bits == 3:
        dw = np.zeros(lead + (3,), dtype=np.int64)
        for m in range(4):
            for r in range(4):
                ua, ub = 8 * m + r, 8 * m + r + 4
                p = 4 * (m % 2) + r
                H = 8 * (m // 2) + 2 * r + (m % 2)
                dw[..., m // 2] |= (c[..., ua] & 3) << (2 * p)
                dw[..., m // 2] |= (c[..., ub] & 3) << (16 + 2 * p)
                dw[..., 2] |= (c[..., ua] >> 2) << H
                dw[..., 2] |= (c[..., ub] >> 2) << (16 + H)
        out = np.zeros(lead + (12,), dtype=np.uint8)
        for w in range(3):
            for b in range(4):
                out[..., 4 * w + b] = (dw[..., w] >> (8 * b)) & 0xFF
        return out
    raise ValueError(bits)


def unpack_segment(data: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_segment: bytes [..., 4*bits] -> unsigned codes [..., 32]."""
    b = np.asarray(data).astype(np.int64)
    lead = b.shape[:-1]
    if bits == 8:
        return b
    if bits == 4:
        out = np.empty(lead + (32,), dtype=np.int64)
        out[..., 0::2] = b & 15
        out[..., 1::2] = b >> 4
        return out
    if bits == 3:
        dw = [b[..., 4 * w] | (b[..., 4 * w + 1] << 8) | (b[..., 4 * w + 2] << 16)
              | (b[..., 4 * w + 3] << 24) for w in range(3)]
        out = np.empty(lead + (32,), dtype=np.int64)
        for m in range(4):
            for r in range(4):
                ua, ub = 8 * m + r, 8 * m + r + 4
                p = 4 * (m % 2) + r
                H = 8 * (m // 2) + 2 * r + (m % 2)
                out[..., ua] = ((dw[m // 2] >> (2 * p)) & 3) | (((dw[2] >> H) & 1) << 2)
                out[..., ub] = ((dw[m // 2] >> (16 + 2 * p)) & 3) | (((dw[2] >> (16 + H)) & 1) << 2)
        return out
    raise ValueError(bits)


def k_row_channel(q: int, u: int) -> int:
    """Channel stored at code u of segment q of a K row."""
    return 32 * (u // 8) + 8 * q + (u % 8)


def v_tile_position(lane: int, s: int, u: int):
    """(token-in-tile, channel) stored at code u of segment s of lane ``lane``."""
    q, i = lane // 16, lane % 16
    m, e = u // 8, u % 8
    tok = 4 * q + e if e < 4 else 16 + 4 * q + (e - 4)
    return tok, 16 * (4 * s + m) + i


def pack_k_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., T, 128] -> bytes [..., T, 16*bits] in the K-row layout."""
    codes = np.asarray(codes)
    segs = []
    for q in range(4):
        idx = [k_row_channel(q, u) for u in range(32)]
        segs.append(pack_segment(codes[..., idx], bits))
    return np.concatenate(segs, axis=-1)


def pack_v_tiles(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., T, 128] with T a multiple of 32 -> bytes [..., T/32, 64*8*bits]."""
    codes = np.asarray(codes)
    T = codes.shape[-2]
    assert T % 32 == 0
    tiles = codes.reshape(codes.shape[:-2] + (T // 32, 32, D))
    lanes = []
    for lane in range(64):
        for s in range(2):
            toks, chans = zip(*[v_tile_position(lane, s, u) for u in range(32)])
            seg_codes = tiles[..., list(toks), list(chans)]     # [..., ntiles, 32]
            lanes.append(pack_segment(seg_codes, bits))
    return np.concatenate(lanes, axis=-1)


def v_pair_position(byte: int, half: int):
    """(token-in-tile, channel) held by nibble ``half`` (0 low, 1 high) of byte
    ``byte`` of a codebook value tile: byte 32*l + tau holds channel l (low
    nibble) and channel l + 64 (high nibble) of token tau, l = 0..63."""
    lane, tau = byte // 32, byte % 32
    return tau, lane + 64 * half


def pack_v_pair_tiles(codes: np.ndarray) -> np.ndarray:
    """4-bit codes [..., T, 128] with T a multiple of 32 -> bytes
    [..., T/32, 2048] in the codebook value-tile layout (v_pair_position)."""
    codes = np.asarray(codes)
    T = codes.shape[-2]
    assert T % 32 == 0
    tiles = codes.reshape(codes.shape[:-2] + (T // 32, 32, D))
    lo = tiles[..., :, :64]                          # [..., ntiles, tau, l]
    hi = tiles[..., :, 64:]
    b = (lo | (hi << 4)).astype(np.uint8)
    return np.swapaxes(b, -1, -2).reshape(codes.shape[:-2] + (T // 32, 2048))


def expected_regions(fmt: Dict, enc: Dict[str, np.ndarray], *, batch: int, n_kv_heads: int,
                     n_ctx: int, max_ctx: int, kv_dtype: str, is_key: bool) -> Dict[str, np.ndarray]:
    """Byte-exact image of one tensor's cache regions after ``n_ctx`` tokens.

    Region arrays (unwritten entries are zero):

    * ``codes`` uint8 [B, H, Tcap * row_bytes]: K-row layout for keys,
      V-tile layout for values, the pair-tile layout for codebook values
      (NONE stores raw fp16/bf16 rows instead);
    * ``params``: per-token asymmetric fp16 [B, H, Tcap, d/G, 2] (scale,
      zero); q8_0 fp16 [B, H, Tcap, d/G]; per-channel fp16
      [B, H, Tcap // G, d, 2];
    * ``tail`` (per-channel): [B, H, G, d] raw bits of the unfinished group
      (uint16), zero beyond it;
    * ``tile_off`` uint16 [B * Tcap / 32, round_up(H + 1, 8)] and
      ``tile_ent`` uint32 [B * Tcap / 32, 32 k]: the outliers of each tile
      of 32 tokens grouped by KV head (``outlier_tiles``);
    * ``row_ptr`` int32 [B * Tcap + 1], ``col`` uint16 and ``val`` fp16
      [B * Tcap * k]: CSR over rows r = b * Tcap + t, with
      row_ptr[b * Tcap + t] = k * (b * Tcap + t) for t = 0..n_ctx; a column
      entry holds h * d + c in bits 0-11 and the dense codebook index of that
      position in bits 12-15.
    """
    B, H = batch, n_kv_heads
    Tcap = capacity(max_ctx)
    q = fmt["quantizer"]
    bits = fmt["bits"]
    G = fmt.get("group_size", 0)
    out: Dict[str, np.ndarray] = {}
    if q == "none":
        raise ValueError("raw format has no quantized regions")
    rb = row_bytes(bits)
    codes = np.zeros((B, H, Tcap, D), dtype=np.int64)
    c = np.asarray(enc["codes"]).astype(np.int64)
    codes[:, :, :c.shape[2], :] = c
    if is_key:
        packed = pack_k_rows(codes, bits)                          # [B, H, Tcap, rb]
    elif q == "codebook":
        packed = pack_v_pair_tiles(codes)                          # [B, H, Tcap/32, 2048]
    else:
        packed = pack_v_tiles(codes, bits)                         # [B, H, Tcap/32, 32*rb]
    # tokens that are not yet quantized must leave their bytes at zero
    if is_key:
        packed[:, :, c.shape[2]:, :] = 0
    out["codes"] = packed.reshape(B, H, Tcap * rb)
    layout = fmt.get("layout", "per_token")
    if q in ("asym_minmax", "asym_absmax_offset", "sym_q8_0") and fmt.get("head_group_size"):
        out["params"] = per_head_params(fmt, enc, B, H, Tcap, n_ctx)
    elif q in ("asym_minmax", "asym_absmax_offset"):
        if layout == "per_token":
            p = np.zeros((B, H, Tcap, D // G, 2), dtype=np.float16)
            p[:, :, :n_ctx, :, 0] = enc["scale"]
            p[:, :, :n_ctx, :, 1] = enc["zero"]
        else:
            p = np.zeros((B, H, Tcap // G, D, 2), dtype=np.float16)
            ng = enc["scale"].shape[2]
            p[:, :, :ng, :, 0] = enc["scale"]
            p[:, :, :ng, :, 1] = enc["zero"]
            out["tail"] = tail_ring(enc["tail_rows"], G, int(fmt.get("window_overlap", 0)),
                                    n_ctx, kv_dtype)
        out["params"] = p
    elif q == "sym_q8_0":
        p = np.zeros((B, H, Tcap, D // G), dtype=np.float16)
        p[:, :, :n_ctx, :] = enc["scale"]
        out["params"] = p
    if q == "codebook" and "cols" in enc:
        k = enc["cols"].shape[-1]
        row_ptr = np.zeros(B * Tcap + 1, dtype=np.int64)
        col = np.zeros(B * Tcap * k, dtype=np.uint16)
        val = np.zeros(B * Tcap * k, dtype=np.float16)
        # bits 12-15 of a column entry repeat the dense index it replaces
        cols = np.asarray(enc["cols"]).astype(np.int64)            # [B, n_ctx, k]
        dense = np.asarray(enc["codes"]).astype(np.int64)          # [B, H, n_ctx, d]
        bb = np.arange(B)[:, None, None]
        tt = np.arange(cols.shape[1])[None, :, None]
        packed_cols = cols | (dense[bb, cols // D, tt, cols % D] << 12)
        for b in range(B):
            r0 = b * Tcap
            row_ptr[r0:r0 + n_ctx + 1] = k * np.arange(r0, r0 + n_ctx + 1)
            col[k * r0:k * (r0 + n_ctx)] = packed_cols[b].reshape(-1)
            val[k * r0:k * (r0 + n_ctx)] = enc["vals"][b].reshape(-1).astype(np.float16)
        out["row_ptr"] = row_ptr.astype(np.int32)
        out["col"] = col
        out["val"] = val
        out["tile_off"], out["tile_ent"] = outlier_tiles(
            cols, np.asarray(enc["vals"]), dense, batch=B, n_kv_heads=H, capacity=Tcap, n_ctx=n_ctx)
    return out


def outlier_tiles(cols: np.ndarray, vals: np.ndarray, dense: np.ndarray, *, batch: int,
                  n_kv_heads: int, capacity: int, n_ctx: int):
    """Per-tile index of the outliers (this library's layout; the pages
    keep outliers in CSR without fixing a byte layout -- KVQuant page,
    section 3.3).  For tile j of sequence b (tokens 32 j .. 32 j + 31) and
    KV head h, the entries of its tokens in token order, each token's in
    column order, one uint32 each: channel c (bits 0-6), token in the tile
    (7-11), dense codebook index replaced (12-15), fp16 value bits (16-31).
    ``tile_off[tile, h]`` is where head h's entries start in the tile's
    block of 32 k entries, ``tile_off[tile, H]`` the tile's count; rows of
    round_up(H + 1, 8) entries, tiles b * capacity / 32 + j.

    ``cols`` [B, n_ctx, k] (columns h * d + c, ascending per token),
    ``vals`` [B, n_ctx, k], ``dense`` [B, H, n_ctx, d] codebook indices."""
    B, H = batch, n_kv_heads
    k = cols.shape[-1]
    ntile = capacity // 32
    o_row = (H + 8) // 8 * 8
    toff = np.zeros((B * ntile, o_row), dtype=np.uint16)
    tent = np.zeros((B * ntile, 32 * k), dtype=np.uint32)
    vbits = np.asarray(vals, dtype=np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
    for b in range(B):
        for j in range((n_ctx + 31) // 32):
            lists = [[] for _ in range(H)]
            for t in range(32 * j, min(32 * j + 32, n_ctx)):
                for e in range(k):
                    col = int(cols[b, t, e])
                    h, c = col // D, col % D
                    code = int(dense[b, h, t, c])
                    lists[h].append(c | ((t - 32 * j) << 7) | (code << 12) | (int(vbits[b, t, e]) << 16))
            row = b * ntile + j
            off = 0
            for h in range(H):
                toff[row, h] = off
                tent[row, off:off + len(lists[h])] = lists[h]
                off += len(lists[h])
            toff[row, H] = off
    return toff, tent


def per_head_params(fmt: Dict, enc: Dict, B: int, H: int, Tcap: int, n_ctx: int) -> np.ndarray:
    """Parameter image of a per-token format with a group size per KV head:
    for each sequence, head 0's [Tcap][d / G_0] records, then head 1's, ...
    (a record: fp16 scale, zero; q8_0: fp16 scale).  Flat fp16 array."""
    q8 = fmt["quantizer"] == "sym_q8_0"
    blocks = []
    for b in range(B):
        for h in range(H):
            ng = D // int(fmt["head_group_size"][h])
            if q8:
                p = np.zeros((Tcap, ng), dtype=np.float16)
                p[:n_ctx] = enc["scale"][h][b]
            else:
                p = np.zeros((Tcap, ng, 2), dtype=np.float16)
                p[:n_ctx, :, 0] = enc["scale"][h][b]
                p[:n_ctx, :, 1] = enc["zero"][h][b]
            blocks.append(p.reshape(-1))
    return np.concatenate(blocks)


def tail_ring(raw: np.ndarray, G: int, overlap: int, n_ctx: int, kv_dtype: str) -> np.ndarray:
    """Byte image [B, H, G + overlap, d] of the unquantized key tail of a
    per-channel key cache after n_ctx tokens: a ring of G + overlap rows in
    which token p sits at row p mod (G + overlap).  It holds the tokens of
    the unfinished group [n_full, n_ctx), n_full = floor(n_ctx / G) * G, and
    the ``overlap`` tokens before n_full that the next group's window reads
    (``raw`` [B, H, n_ctx, d]: every token's float32 value); other rows are
    zero.  Without overlap, row i holds token n_full + i."""
    raw = np.asarray(raw, dtype=np.float32)
    B, H = raw.shape[:2]
    R = G + overlap
    n_full = (n_ctx // G) * G
    out = np.zeros((B, H, R, D), dtype=np.uint16)
    for p in range(max(0, n_full - overlap), n_ctx):
        out[:, :, p % R, :] = to_bits(raw[:, :, p, :], kv_dtype)
    return out


def to_bits(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Raw 16-bit patterns of float32 values that are exact fp16/bf16 numbers."""
    x = np.asarray(x, dtype=np.float32)
    if kv_dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "values are not bf16"
    return (u >> 16).astype(np.uint16)


def from_bits(b: np.ndarray, kv_dtype: str) -> np.ndarray:
    """float32 values of raw fp16/bf16 bit patterns."""
    b = np.asarray(b, dtype=np.uint16)
    if kv_dtype == "f16":
        return b.view(np.float16).astype(np.float32)
    return (b.astype(np.uint32) << 16).view(np.float32)


def sink_region(x: np.ndarray, sink: int, *, kv_dtype: str) -> np.ndarray:
    """Byte image of one tensor's attention-sink region: [B, H, sink, d] raw
    fp16/bf16 bits of tokens [0, min(sink, T)) of ``x`` (float32 [B, T, H, d]
    holding fp16/bf16 values), zero beyond."""
    x = np.asarray(x, dtype=np.float32)
    B, T, H, d = x.shape
    s = min(int(sink), T)
    out = np.zeros((B, H, int(sink), d), dtype=np.uint16)
    out[:, :, :s, :] = to_bits(np.transpose(x[:, :s], (0, 2, 1, 3)), kv_dtype)
    return out
