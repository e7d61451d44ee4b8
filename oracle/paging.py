"""Paged cache: where each token's bytes live when the cache is a pool of
pages shared by the sequences through a block table.

Test infrastructure: see the package docstring.

The Survey page (section 3.4, vLLM's fp8 KV cache, ``--block-size 16``)
runs the quantized cache as fixed-size blocks that a per-sequence block
table maps to physical blocks of a shared pool.  Reading taken here (the
page gives the block size and the block table, not a byte layout):

* a page holds 32 tokens (two of the page's 16-token blocks: the value tile
  of this library is 32 tokens) of every KV head;
* logical page i of sequence b (its tokens [32 i, 32 i + 32)) lives in
  physical page ``table[b][i]``;
* every array with one record per token and head -- key rows, value tiles,
  per-token scales and zeros -- holds token t of (b, h) at row
  ``(table[b][t // 32] * H + h) * 32 + t % 32`` instead of
  ``(b * H + h) * Tcap + t``; a value tile is 32 consecutive rows either way;
* the outlier CSR (one row per token, all heads) holds token t of sequence b
  at row ``table[b][t // 32] * 32 + t % 32``, and row_ptr[r] = k * r at both
  ends of every written row; the per-tile outlier index has one tile per
  page;
* per-channel key parameters, the unquantized key tail and the attention
  sink keep their per-sequence arrays.

``paged_regions`` maps the oracle's contiguous byte images
(``layout.expected_regions``) to the paged ones: a gather of whole 32-token
pages.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

PAGE = 32


def token_row(table: np.ndarray, n_kv_heads: int, b: int, h: int, t: int) -> int:
    """Row of token t of (sequence b, KV head h) in the per-token arrays of a
    paged cache."""
    return (int(table[b][t // PAGE]) * n_kv_heads + h) * PAGE + t % PAGE


def csr_row(table: np.ndarray, b: int, t: int) -> int:
    """Row of token t of sequence b in the outlier CSR of a paged cache."""
    return int(table[b][t // PAGE]) * PAGE + t % PAGE


def _gather_pages(img: np.ndarray, table: np.ndarray, n_pages: int, used: int) -> np.ndarray:
    """[B, H, Tcap / 32, X] -> [n_pages, H, X]: logical page i of sequence b
    to physical page table[b][i], for i < used; other pages zero."""
    B, H = img.shape[:2]
    out = np.zeros((n_pages, H) + img.shape[3:], dtype=img.dtype)
    for b in range(B):
        for i in range(used):
            out[table[b][i]] = img[b, :, i]
    return out


def paged_regions(regions: Dict[str, np.ndarray], table: np.ndarray, *, n_pages: int,
                  n_ctx: int, capacity: int, per_channel: bool, k_out: int = 0,
                  head_ng=None, rec_halves: int = 2) -> Dict[str, np.ndarray]:
    """Byte images of one tensor's regions in a paged cache of ``n_pages``
    pages, from its contiguous images over ``capacity`` tokens per sequence
    (codes [B, H, capacity * row bytes]; per-token params [B, H, capacity,
    ...]; CSR over B * capacity rows) and the page table [B, pages_per_seq].
    Pages that no entry below ceil(n_ctx / 32) names stay zero.  The tail
    and per-channel params (``per_channel``) keep their contiguous images.
    With a group size per KV head (``head_ng``: groups per token of each
    head; ``rec_halves``: fp16 values per record) the contiguous params
    hold, per sequence, head 0's [capacity][head_ng[0]] records, then head
    1's, ...; a page holds, per head in turn, its 32 tokens' records."""
    table = np.asarray(table, dtype=np.int64)
    used = (n_ctx + PAGE - 1) // PAGE
    B = table.shape[0]
    npg = capacity // PAGE
    out: Dict[str, np.ndarray] = {}
    for name, img in regions.items():
        img = np.asarray(img)
        if name == "codes":
            H = img.shape[1]
            pages = img.reshape(B, H, npg, -1)            # 32 rows, or one value tile
            out[name] = _gather_pages(pages, table, n_pages, used).reshape(n_pages, H, -1)
        elif name == "params" and head_ng is not None:
            flat = img.reshape(-1)
            tot = sum(head_ng) * rec_halves
            per_seq = flat.reshape(B, capacity * tot)
            dst = np.zeros((n_pages, PAGE * tot), dtype=img.dtype)
            for b in range(B):
                off = 0
                for h, ng in enumerate(head_ng):
                    w = ng * rec_halves                # values per token of head h
                    head = per_seq[b, capacity * off:capacity * (off + w)].reshape(capacity, w)
                    for i in range(used):
                        dst[table[b][i], PAGE * off:PAGE * (off + w)] = \
                            head[PAGE * i:PAGE * (i + 1)].reshape(-1)
                    off += w
            out[name] = dst
        elif name == "params" and not per_channel:
            H = img.shape[1]
            pages = img.reshape((B, H, npg, PAGE) + img.shape[3:])
            out[name] = _gather_pages(pages, table, n_pages, used)
        elif name == "row_ptr":
            rp = np.zeros(n_pages * PAGE + 1, dtype=np.int64)
            for b in range(B):
                for t in range(n_ctx):
                    r = csr_row(table, b, t)
                    rp[r] = k_out * r
                    rp[r + 1] = k_out * (r + 1)
            out[name] = rp.astype(np.int32)
        elif name in ("tile_off", "tile_ent"):
            # one tile of the per-tile outlier index per page
            src = img.reshape(B, npg, -1)
            dst = np.zeros((n_pages, src.shape[2]), dtype=img.dtype)
            for b in range(B):
                for i in range(used):
                    dst[table[b][i]] = src[b, i]
            out[name] = dst
        elif name in ("col", "val"):
            src = img.reshape(B, capacity, k_out)
            dst = np.zeros((n_pages * PAGE, k_out), dtype=img.dtype)
            for b in range(B):
                for t in range(n_ctx):
                    dst[csr_row(table, b, t)] = src[b, t]
            out[name] = dst.reshape(-1)
        else:
            out[name] = img
    return out
