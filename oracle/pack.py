"""Oracle for mixed-state packing (bounding-box gather), exact integer work.

Test infrastructure only (see the package docstring).

From [BlockServe] (page "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务"):
  * §II-A: request r_i has prompt length p_i, K_i blocks of length L, current block index b_i;
    requests in the active set may sit at different block indices.
  * §II-D Eq.(1): row width p_i + (b_i + 1) L (prompt plus finished and in-progress blocks);
    Cost(A) = |A| * max_i (p_i + (b_i + 1) L).
  * §II-E 逻辑位置对齐: the bounding box is materialised as a dense |A| x max-width tensor with
    left padding, so each prompt is contiguous and immediately followed by its generated region;
    position ids come from a running count over the attention mask, so the first non-pad token
    is at logical position 0.
  * §II-E 向量化混合调度执行: gather pulls each request's active block out for denoising.
Readings: pad columns carry pad_id, valid 0 and position 0; the per-row views (mask, threshold,
p, b) are copied out of the request table next to the box.
"""
from __future__ import annotations

import numpy as np


def row_width(p: int, b: int, L: int) -> int:
    """[BlockServe] §II-D: width of a request's row at block index b."""
    return int(p) + (int(b) + 1) * int(L)


def box_width(row_req, rows, p, b, L) -> int:
    """Eq.(1)'s max over the active set (0 for an empty set)."""
    return max((row_width(p[q], b[q], L) for q in row_req[:rows]), default=0)


def cost(row_req, rows, p, b, L) -> int:
    """[BlockServe] §II-D Eq.(1): Cost(A) = |A| * max_i (p_i + (b_i + 1) L)."""
    return rows * box_width(row_req, rows, p, b, L)


def pack(row_req, rows: int, L: int, W: int, pad_id: int, p, b, threshold, arena_off, arena, blk_mask):
    """Materialise the left-padded box for the active rows.

    Returns dict(box_ids int32 [rows, W], box_valid uint8, box_pos int32, mask uint8 [rows, L],
    threshold float32 [rows], p int32 [rows], b int32 [rows]).
    Row r holding request q: pad_r = W - (p_q + (b_q + 1) L) columns of pad_id, then the arena's
    prompt, committed blocks and current block.  valid = (column >= pad_r); pos = column - pad_r
    on valid columns, 0 on pads.  The active block therefore occupies columns W-L .. W-1.
    """
    box_ids = np.empty((rows, W), np.int32)
    box_valid = np.zeros((rows, W), np.uint8)
    box_pos = np.zeros((rows, W), np.int32)
    m = np.empty((rows, L), np.uint8)
    tau = np.empty(rows, np.float32)
    pr = np.empty(rows, np.int32)
    br = np.empty(rows, np.int32)
    for r in range(rows):
        q = int(row_req[r])
        w = row_width(p[q], b[q], L)
        if w > W:
            raise ValueError(f"request {q} (width {w}) does not fit box width {W}")
        pad = W - w
        off = int(arena_off[q])
        box_ids[r, :pad] = pad_id
        box_ids[r, pad:] = arena[off:off + w]
        box_valid[r, pad:] = 1
        box_pos[r, pad:] = np.arange(w)
        m[r] = blk_mask[q]
        tau[r] = threshold[q]
        pr[r] = p[q]
        br[r] = b[q]
    return dict(box_ids=box_ids, box_valid=box_valid, box_pos=box_pos, mask=m, threshold=tau, p=pr, b=br)
