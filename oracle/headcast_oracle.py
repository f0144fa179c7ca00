"""CPU float64 oracle for HeadCast's head-routed attention step.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow definition that the HIP
library is checked against. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the library never calls it and it calls nothing of
the library. It shares no code with the HIP path: inputs are passed in as arrays.

Source: "HeadCast: Casting Attention Heads for Efficient Autoregressive Video
Generation" (arXiv 2607.20125), cited below as HeadCast with its section/equation,
plus its appendices (Chinese translation page) where the English page has none.

Every attention output here is the textbook definition: dense scores QK^T * scale over
the logical window, -inf outside the head's key set, row softmax, times V, in float64.
Routing and gathering in HeadCast are exact restrictions of the key set (Sec. 4.4),
so the masked dense form is the exact result, not an approximation.

Readings taken where the pages are silent or disagree (each one is restated where used):
  * Dummy path = current block only (Sec. 3.2 "Dummy Pattern"; Sec. 4.2 proxy list).
  * Sink path = first (sink) block + current block; the classifier's Sink proxy is the
    first block alone (Sec. 4.2 proxy list; Eq. 5 checks Sink first).
  * Spatial path and proxy = current block in full + a g x g window in every history
    frame, shifted (never truncated) to stay inside the frame.
  * "History" = every window frame before the current block, including the sink block.
  * Statistics: cos(x,y) = x.y / max(|x||y|, 1e-8); P5 = linear-interpolation 5th
    percentile over the L_q token cosines; MSE over all L_q*d elements (Eq. 3, Eq. 4).

Parity pins for every function live in tests/test_oracle_pins.py; none is unpinned.
"""
from __future__ import annotations

import numpy as np

SINK, DUMMY, SPATIAL, GLOBAL = 0, 1, 2, 3
COS_EPS = 1e-8



def attention_scale(head_dim):
    """Score scale of the attention the paths compute: 1/sqrt(d), scaled dot-product
    attention with no bias (HeadCast Sec. 3.1). Owned here, not taken from the caller's
    layer description, so that the oracle does not share it with the library's caller."""
    return 1.0 / np.sqrt(float(head_dim))


# Path variants the pages also describe (deployed forms; see key_set_mask):
DUMMY_PREVIOUS_BLOCK = 1   # Dummy heads also see the latest finished block
SPATIAL_CELLS = 2          # Spatial heads see their own non-overlapping cell in every frame


# ----------------------------------------------------------------------------- geometry
def window_origin(pos: np.ndarray | int, g: int, extent: int):
    """First row (or column) of the g-wide window around `pos` inside a frame of
    `extent` rows (or columns): centred on the query (the query sits at offset g//2),
    then shifted to lie inside the frame; the window is never truncated unless g
    exceeds the frame, where it covers the whole frame (origin 0)."""
    return np.clip(np.asarray(pos) - g // 2, 0, max(extent - g, 0))


def window_extent(g: int, extent: int) -> int:
    return min(g, extent)


def cell_origin(pos, cell: int):
    """First row (column) of the non-overlapping cell holding `pos`: cells tile the frame
    from row (column) 0; the last one keeps the remainder rows (columns)."""
    return (np.asarray(pos) // cell) * cell


def cell_extent(pos, cell: int, extent: int):
    return np.minimum(cell, extent - cell_origin(pos, cell))


def key_coords(frame_h: int, frame_w: int, n_frames: int):
    """(frame, row, col) of every token of `n_frames` consecutive frames (frame-major,
    row-major inside a frame)."""
    S = frame_h * frame_w
    t = np.arange(n_frames * S)
    return t // S, (t % S) // frame_w, t % frame_w


def key_set_mask(cls: int, geom, n_hist: int, q_tokens: np.ndarray, grid=None,
                 sink_proxy: bool = False, sink_proxy_includes_current: bool = False, variant: int = 0):
    """Boolean mask [len(q_tokens)][(n_hist + C) * S] over the logical window
    [history frames 0..n_hist-1 ; current block], for one head class.

    Key sets (HeadCast Sec. 4.3-4.4 and the proxy list of Sec. 4.2):
      SINK    : the sink block (history frames 0..C-1) + the current block;
                with sink_proxy=True: the sink block alone (the classifier's proxy),
                plus the current block if sink_proxy_includes_current.
      DUMMY   : the current block only; with variant DUMMY_PREVIOUS_BLOCK also the
                latest finished block (the last C history frames; appendix B's cost
                model and Sec. 4.4's fused Sink/Dummy launch).
      SPATIAL : the current block + in each history frame the g x g window around the
                query's (row, col); with variant SPATIAL_CELLS instead the query's own
                non-overlapping g_h x g_w cell in every window frame, current block
                included (Sec. 4.4, Fig. 3).
      GLOBAL  : every window frame.
    """
    C, S = geom.chunk_frames, geom.tokens_per_frame
    fh, fw = geom.frame_h, geom.frame_w
    gh, gw = grid if grid is not None else (geom.grid_h, geom.grid_w)
    kf, kr, kc = key_coords(fh, fw, n_hist + C)
    is_cur = kf >= n_hist
    is_hist = ~is_cur
    nq = len(q_tokens)
    qr = (np.asarray(q_tokens) % S) // fw
    qc = np.asarray(q_tokens) % fw
    if cls == GLOBAL:
        m = np.ones((nq, kf.size), dtype=bool)
    elif cls == DUMMY:
        keys = is_cur.copy()
        if variant & DUMMY_PREVIOUS_BLOCK:
            keys |= is_hist & (kf >= n_hist - C)
        m = np.broadcast_to(keys, (nq, kf.size)).copy()
    elif cls == SINK:
        sink_keys = is_hist & (kf < C)
        keys = sink_keys if (sink_proxy and not sink_proxy_includes_current) else (sink_keys | is_cur)
        m = np.broadcast_to(keys, (nq, kf.size)).copy()
    elif cls == SPATIAL and (variant & SPATIAL_CELLS):
        same_row_cell = (kr[None, :] // gh) == (qr[:, None] // gh)
        same_col_cell = (kc[None, :] // gw) == (qc[:, None] // gw)
        m = same_row_cell & same_col_cell
    elif cls == SPATIAL:
        r0 = window_origin(qr, gh, fh)[:, None]
        c0 = window_origin(qc, gw, fw)[:, None]
        eh, ew = window_extent(gh, fh), window_extent(gw, fw)
        in_win = ((kr[None, :] >= r0) & (kr[None, :] < r0 + eh) &
                  (kc[None, :] >= c0) & (kc[None, :] < c0 + ew))
        m = (is_hist[None, :] & in_win) | is_cur[None, :]
    else:
        raise ValueError(f"bad class {cls}")
    return m


# ----------------------------------------------------------------------------- attention
def masked_attention(q, k, v, mask, scale, return_weights=False):
    """softmax(q k^T * scale, restricted to mask) v in float64 (Eq. 2 with the key
    set given by `mask`). q [nq][d], k, v [nk][d], mask [nq][nk] bool.
    Also returns the log-sum-exp of the kept scores (natural log)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q @ k.T) * scale
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=1, keepdims=True)
    p = e / den
    out = p @ v
    lse = (mx + np.log(den))[:, 0]
    if return_weights:
        return out, lse, p
    return out, lse


def head_window(q, k_hist, v_hist, k_cur, v_cur, h):
    """Float64 views of one head: q [Lq][d], k/v over [history ; current]."""
    k = np.concatenate([k_hist[:, h, :], k_cur[:, h, :]], axis=0).astype(np.float64)
    v = np.concatenate([v_hist[:, h, :], v_cur[:, h, :]], axis=0).astype(np.float64)
    return q[:, h, :].astype(np.float64), k, v


def path_attention(inp, h, cls, rows=None, block=512, grid=None, sink_proxy=False,
                   sink_proxy_includes_current=False, variant=0):
    """Output [len(rows)][d] of head h restricted to the key set of `cls`
    (processed in blocks of query rows to bound memory)."""
    g = inp.geom
    if rows is None:
        rows = np.arange(g.lq)
    rows = np.asarray(rows)
    qh, kh, vh = head_window(inp.q, inp.k_hist, inp.v_hist, inp.k_cur, inp.v_cur, h)
    out = np.empty((rows.size, g.head_dim))
    for b in range(0, rows.size, block):
        r = rows[b:b + block]
        m = key_set_mask(cls, g, inp.n_hist_frames, r, grid, sink_proxy, sink_proxy_includes_current, variant)
        out[b:b + block], _ = masked_attention(qh[r], kh, vh, m, attention_scale(g.head_dim))
    return out


def routed_attention(inp, labels=None, rows=None, heads=None, variant=0):
    """The routed step (HeadCast Sec. 4.4): head h attends over the key set of its
    class; outputs concatenated back along heads. Returns [len(rows)][H][d] float64."""
    g = inp.geom
    labels = inp.labels if labels is None else np.asarray(labels)
    if rows is None:
        rows = np.arange(g.lq)
    heads = range(g.num_heads) if heads is None else heads
    out = np.zeros((len(rows), g.num_heads, g.head_dim))
    for h in heads:
        out[:, h, :] = path_attention(inp, h, int(labels[h]), rows, variant=variant)
    return out


def brute_force_attention(inp, h, cls, t, grid=None, sink_proxy=False, variant=0):
    """One query token t of head h by a scalar loop: walk every window key, keep it if
    the class admits it (membership written out key by key), softmax in float64."""
    g = inp.geom
    C, S, fh, fw = g.chunk_frames, g.tokens_per_frame, g.frame_h, g.frame_w
    gh, gw = grid if grid is not None else (g.grid_h, g.grid_w)
    n_hist = inp.n_hist_frames
    qr, qc = (t % S) // fw, t % fw
    # window rows: the g rows around qr, slid into the frame
    r_lo = min(max(qr - gh // 2, 0), max(fh - gh, 0))
    c_lo = min(max(qc - gw // 2, 0), max(fw - gw, 0))
    qv = inp.q[t, h, :].astype(np.float64)
    scores, values = [], []
    for f in range(n_hist + C):
        current = f >= n_hist
        for r in range(fh):
            for c in range(fw):
                if cls == GLOBAL:
                    keep = True
                elif cls == DUMMY:
                    keep = current or (bool(variant & DUMMY_PREVIOUS_BLOCK) and n_hist - C <= f)
                elif cls == SPATIAL and variant & SPATIAL_CELLS:
                    keep = r // gh == qr // gh and c // gw == qc // gw
                elif cls == SINK:
                    keep = (f < C and not current) or (current and not sink_proxy)
                else:
                    keep = current or (r_lo <= r < r_lo + gh and c_lo <= c < c_lo + gw)
                if not keep:
                    continue
                if current:
                    tok = (f - n_hist) * S + r * fw + c
                    kv, vv = inp.k_cur[tok, h, :], inp.v_cur[tok, h, :]
                else:
                    tok = f * S + r * fw + c
                    kv, vv = inp.k_hist[tok, h, :], inp.v_hist[tok, h, :]
                scores.append(float(np.dot(qv, kv.astype(np.float64))) * attention_scale(g.head_dim))
                values.append(vv.astype(np.float64))
    mx = max(scores)
    w = [np.exp(s - mx) for s in scores]
    tot = sum(w)
    return sum(wi * vi for wi, vi in zip(w, values)) / tot


def merge_partials(parts):
    """Combine attention results over disjoint key sets: parts = [(out, lse)], out
    normalised. Softmax over a union = lse-weighted mix of the parts."""
    lses = np.stack([p[1] for p in parts])
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    tot = w.sum(axis=0)
    return sum(w[i][:, None] * parts[i][0] for i in range(len(parts))) / tot[:, None]


# ----------------------------------------------------------------------------- classifier
def cosine(x, y):
    """Row-wise cosine similarity, denominator floored at 1e-8."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    num = (x * y).sum(axis=-1)
    den = np.sqrt((x * x).sum(axis=-1)) * np.sqrt((y * y).sum(axis=-1))
    return num / np.maximum(den, COS_EPS)


def head_statistics(o_sink, o_dummy, o_spatial, o_ref, gamma, percentile=5.0):
    """Eq. 3 (mean token cosine per proxy) and Eq. 4 (conservative Spatial score:
    the 5th-percentile token cosine minus gamma times the MSE against the reference)."""
    cs = cosine(o_sink, o_ref)
    cd = cosine(o_dummy, o_ref)
    cp = cosine(o_spatial, o_ref)
    mse = float(np.mean((np.asarray(o_spatial, np.float64) - np.asarray(o_ref, np.float64)) ** 2))
    p5 = float(np.percentile(cp, percentile))
    return dict(cos_sink=float(cs.mean()), cos_dummy=float(cd.mean()),
                cos_spatial=float(cp.mean()), p5=p5, mse=mse, score=p5 - gamma * mse)


def decide(cos_sink, cos_dummy, cos_spatial, score, theta_sink=0.95, theta_dummy=0.95,
           theta_spatial=0.95, theta_score=0.755):
    """Eq. 5: mutually exclusive decision, checked in the order Sink, Dummy, Spatial."""
    if cos_sink >= theta_sink:
        return SINK
    if cos_dummy >= theta_dummy:
        return DUMMY
    if cos_spatial >= theta_spatial and score >= theta_score:
        return SPATIAL
    return GLOBAL


DEFAULT_PARAMS = dict(theta_sink=0.95, theta_dummy=0.95, theta_spatial=0.95,
                      theta_score=0.755, gamma=5.0, percentile=5.0,
                      proxy_grid=None, sink_proxy_includes_current=False)


def classify_heads(inp, params=None, rows=None):
    """One-time classification (Sec. 4.2): for every head, O_ref over the full window
    (Eq. 2), the three proxy outputs, their statistics (Eq. 3, 4) and the decision
    (Eq. 5). Returns (labels int32 [H], stats list of dicts)."""
    p = dict(DEFAULT_PARAMS)
    p.update(params or {})
    g = inp.geom
    labels, stats = [], []
    for h in range(g.num_heads):
        o_ref = path_attention(inp, h, GLOBAL, rows)
        o_sink = path_attention(inp, h, SINK, rows, sink_proxy=True,
                                sink_proxy_includes_current=p["sink_proxy_includes_current"])
        o_dummy = path_attention(inp, h, DUMMY, rows)
        o_sp = path_attention(inp, h, SPATIAL, rows, grid=p["proxy_grid"])
        st = head_statistics(o_sink, o_dummy, o_sp, o_ref, p["gamma"], p["percentile"])
        st["label"] = decide(st["cos_sink"], st["cos_dummy"], st["cos_spatial"], st["score"],
                             p["theta_sink"], p["theta_dummy"], p["theta_spatial"], p["theta_score"])
        labels.append(st["label"])
        stats.append(st)
    return np.array(labels, dtype=np.int32), stats


# ----------------------------------------------------------------------------- ring
def rolling_capacity(window_frames: int, chunk_frames: int) -> int:
    """Rolling blocks a Global/Spatial buffer holds besides the frozen sink block."""
    return max(window_frames // chunk_frames - 2, 0)


def buffer_position_of_block(b: int, window_frames: int, chunk_frames: int):
    """Buffer block position holding absolute block b (Sec. 4.3: the sink block is
    frozen, later blocks overwrite in a rolling fashion): block 0 -> position 0; block
    b >= 1 -> position 1 + (b - 1) mod R. None when there is no rolling slot."""
    if window_frames <= chunk_frames:
        return None            # no history at all: the window is the current block
    if b == 0:
        return 0
    R = rolling_capacity(window_frames, chunk_frames)
    if R == 0:
        return None
    return 1 + (b - 1) % R


def slot_table(labels, window_frames, chunk_frames, n_blocks_seen, variant=0):
    """Absolute frame held at every history frame position [H][F - C] (-1 = empty) after
    blocks 0..n_blocks_seen-1 were stored in order. Sink heads hold only the frozen
    first block; Dummy heads hold nothing (with DUMMY_PREVIOUS_BLOCK: the window's most
    recent history block, overwritten by every new one while rolling blocks exist);
    Global/Spatial heads hold the ring."""
    C, F = chunk_frames, window_frames
    H = len(labels)
    table = -np.ones((H, F - C), dtype=np.int32)
    for h in range(H):
        cls = int(labels[h])
        if cls == DUMMY:
            hist = window_history_blocks(n_blocks_seen, F, C)
            if variant & DUMMY_PREVIOUS_BLOCK and hist:
                b = hist[-1]                     # the window's most recent history block
                table[h, :C] = np.arange(b * C, b * C + C)
            continue
        for b in range(n_blocks_seen):
            pos = buffer_position_of_block(b, F, C)
            if pos is None or (cls == SINK and pos != 0):
                continue
            for i in range(C):
                table[h, pos * C + i] = b * C + i
    return table


def window_history_blocks(n_blocks_seen, window_frames, chunk_frames):
    """Absolute blocks forming the window's history, oldest first, when the current
    block is block n_blocks_seen: the sink block plus the most recent rolling blocks
    (sliding window with a fixed sink, Sec. 3.1 and Sec. 5.1)."""
    if window_frames <= chunk_frames or n_blocks_seen == 0:
        return []
    R = rolling_capacity(window_frames, chunk_frames)
    recent = list(range(max(1, n_blocks_seen - R), n_blocks_seen))
    return [0] + recent
