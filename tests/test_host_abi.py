"""Host-side checks of the C ABI that need no GPU: the library loads and exports every
declared symbol, argument validation, buffer sizes, the ring slot table, the routed
work plan, and the classifier's host reductions against the oracle."""
import dataclasses
import os
import re

import numpy as np
import pytest

from head_routed_sparse_amd import headcast as hc
from head_routed_sparse_amd import inputs as hin
from oracle import headcast_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "headcast.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hc_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = hc.lib()
    names = declared_symbols()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(hc.EXPORTED)


def desc_of(name="720p", **kw):
    g = hin.CONFIGS[name]["geom"]
    d = hc.make_desc(g)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, 2), ("num_heads", 0, 2), ("num_heads", 65, 2), ("dtype", 7, 3),
    ("window_frames", 20, 2), ("chunk_frames", 0, 2), ("grid_h", 0, 2), ("frame_w", 0, 2),
    ("softmax_scale", -1.0, 2), ("frame_w", 30000, 2), ("variant", 8, 2)])
def test_desc_validation(field, value, status):
    d = desc_of(**{field: value})
    with pytest.raises(hc.HCError) as ei:
        hc.hc_head_buffers_bytes(d, [0] * max(d.num_heads, 1))
    assert ei.value.status == status


def test_label_and_pointer_validation():
    d = desc_of()
    with pytest.raises(hc.HCError) as ei:
        hc.hc_head_buffers_bytes(d, [0, 1, 2, 4] + [3] * 8)
    assert ei.value.status == 4
    import ctypes
    L = hc.lib()
    h = ctypes.c_void_p()
    lab = np.zeros(12, np.int32)
    # NULL history with frames to copy, misaligned memory, bad n_hist_frames
    st = L.hc_build_head_buffers(ctypes.byref(d), lab.ctypes.data_as(ctypes.c_void_p), None, None, 18,
                                 ctypes.c_void_p(4096), 1 << 40, ctypes.byref(h), None)
    assert st == 1
    st = L.hc_build_head_buffers(ctypes.byref(d), lab.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(16),
                                 ctypes.c_void_p(32), 18, ctypes.c_void_p(4100), 1 << 40, ctypes.byref(h), None)
    assert st == 6
    st = L.hc_build_head_buffers(ctypes.byref(d), lab.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(16),
                                 ctypes.c_void_p(32), 19, ctypes.c_void_p(4096), 1 << 40, ctypes.byref(h), None)
    assert st == 2
    st = L.hc_build_head_buffers(ctypes.byref(d), lab.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(16),
                                 ctypes.c_void_p(32), 18, ctypes.c_void_p(4096), 100, ctypes.byref(h), None)
    assert st == 5
    assert b"needs" in L.hc_last_error()
    # planning handles refuse device work
    pb = hc.hc_plan_head_buffers(d, lab, 7)
    st = L.hc_routed_attention(pb.handle, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                               ctypes.c_void_p(16), ctypes.c_void_p(16), 1 << 40, None)
    assert st == 9
    # classification needs the sink block
    p = hc.hc_default_classify_params()
    st = L.hc_classify_heads(ctypes.byref(d), ctypes.byref(p), *[ctypes.c_void_p(16)] * 3, 0,
                             *[ctypes.c_void_p(16)] * 3, 1 << 40, lab.ctypes.data_as(ctypes.c_void_p), None, None)
    assert st == 9


def test_buffer_bytes_match_the_layout():
    for name in ("480p", "720p", "1080p"):
        cfg = hin.CONFIGS[name]
        g = cfg["geom"]
        d = hc.make_desc(g)
        n = hc.hc_head_buffers_bytes(d, cfg["labels"])
        S, C, F, dd = g.tokens_per_frame, g.chunk_frames, g.window_frames, g.head_dim
        rows = {0: C * S, 1: 0, 2: (F - C) * S, 3: (F - C) * S}
        want = 2 * sum(-(-rows[int(c)] * dd * 2 // 256) * 256 for c in cfg["labels"])
        assert n == want
        mono = 2 * (F - C) * S * g.num_heads * dd * 2
        assert n < mono


def test_default_params_are_the_pages():
    p = hc.hc_default_classify_params()
    assert (p.theta_sink, p.theta_dummy, p.theta_spatial) == (np.float32(0.95),) * 3
    assert p.theta_score == np.float32(0.755) and p.gamma == 5.0 and p.percentile == 5.0


@pytest.mark.parametrize("F,C", [(21, 3), (5, 1), (6, 3), (3, 3), (12, 2)])
def test_slot_table_matches_oracle(F, C):
    g = hin.Geometry(4, 64, 3, 5, C, F, 2, 2, "bf16")
    labels = [0, 1, 2, 3]
    for n in range(0, 16):
        pb = hc.hc_plan_head_buffers(hc.make_desc(g), labels, n)
        assert np.array_equal(hc.hc_debug_slot_table(pb), orc.slot_table(labels, F, C, n)), n
        assert hc.hc_buffers_state(pb) == n


@pytest.mark.parametrize("name", ["tiny", "480p", "720p", "1080p"])
@pytest.mark.parametrize("next_block", [0, 1, 3, 7, 12])
def test_routed_plan_covers_every_key_once(name, next_block):
    cfg = hin.CONFIGS[name]
    g = cfg["geom"]
    labels = cfg["labels"]
    for lab in (labels, np.full(g.num_heads, 3, np.int32)):
        pb = hc.hc_plan_head_buffers(hc.make_desc(g), lab, next_block)
        ents, n_items = hc.hc_debug_routed_plan(pb)
        qtile = int(ents[0, 7])
        assert qtile in (128, 256) and np.all(ents[:, 7] == qtile)
        nqt = -(-g.lq // qtile)
        hist_blocks = orc.window_history_blocks(next_block, g.window_frames, g.chunk_frames)
        assert sorted(ents[:, 0]) == list(range(g.num_heads))
        begin = 0
        for head, hist, cur, nsplit, split_len, slot, item_begin, _q in ents:
            cls = int(lab[head])
            n_hist = {0: min(len(hist_blocks), 1), 1: 0, 2: 0, 3: len(hist_blocks)}[cls]
            assert hist == n_hist * g.chunk_frames * g.tokens_per_frame
            assert cur == g.lq
            assert split_len % 64 == 0 and nsplit >= 1
            assert (nsplit - 1) * split_len < hist + cur <= nsplit * split_len
            assert (slot >= 0) == (cls == 2 or nsplit > 1)
            assert item_begin == begin
            begin += nsplit * nqt
        assert begin == n_items
        # longest items first
        assert list(ents[:, 4]) == sorted(ents[:, 4], reverse=True)


def spatial_tile_chunks(g, tile_r, tile_c):
    """32-key chunks of the window union of every position tile (row-major)."""
    def org(p, gg, ext):
        return min(max(p - gg // 2, 0), max(ext - gg, 0))

    steps = []
    for r0 in range(0, g.frame_h, tile_r):
        r1 = min(r0 + tile_r, g.frame_h) - 1
        ur = org(r1, g.grid_h, g.frame_h) + min(g.grid_h, g.frame_h) - org(r0, g.grid_h, g.frame_h)
        for c0 in range(0, g.frame_w, tile_c):
            c1 = min(c0 + tile_c, g.frame_w) - 1
            uc = org(c1, g.grid_w, g.frame_w) + min(g.grid_w, g.frame_w) - org(c0, g.grid_w, g.frame_w)
            steps.append(-(-ur * uc // 32))
    return steps


def spatial_item_steps(g, tile_r, tile_c, parts, n_hist):
    """Steps of the Spatial items of one head in launch order: frame part by frame part,
    tile by tile; part i walks frames [i n_hist / parts, (i + 1) n_hist / parts)."""
    chunks = spatial_tile_chunks(g, tile_r, tile_c)
    return [c * ((i + 1) * n_hist // parts - i * n_hist // parts) for i in range(parts) for c in chunks]


def item_costs(pb, g, labels):
    """32-key steps of every item of the dense launch: the dense items, then (when the
    Spatial tiles run in it) the tiles of each Spatial head."""
    ents, n_items = hc.hc_debug_routed_plan(pb)
    nqt = -(-g.lq // int(ents[0, 7]))
    cost = []
    for head, hist, cur, nsplit, split_len, slot, begin, _q in ents:
        for s in range(nsplit):
            cost += [-(-min(split_len, hist + cur - s * split_len) // 32)] * nqt
    tr, tc, parts, _, fused = hc.hc_debug_spatial_plan(pb)
    if fused:
        cost += spatial_item_steps(g, tr, tc, parts, g.hist_frames) * int(np.sum(np.asarray(labels) == 2))
    return np.array(cost, np.int64), n_items


def planned_balance(pb, g, labels):
    """Sum of the items' 32-key steps over 512 slots x the longest slot, each XCD's queue
    dealt in order to its 64 slots (32 CUs x 2 workgroups), each item to the slot that
    frees first."""
    import heapq
    cost, _ = item_costs(pb, g, labels)
    queues, _ = hc.hc_debug_dense_queues(pb)
    span = 0
    for q in queues:
        heap = [0] * 64
        for first, count in q:
            for i in range(first, first + count):
                heapq.heapreplace(heap, heap[0] + int(cost[i]))
        span = max(span, max(heap))
    return cost.sum() / (512 * span)


@pytest.mark.parametrize("name,floor", [("480p", 0.85), ("720p", 0.95), ("1080p", 0.99)])
def test_key_splits_per_class_and_planned_balance(name, floor):
    """The split search decides per class of equally long entries: entries of one length
    share one piece count and one piece length (a multiple of the key tile, no empty
    piece), and the dense launch of the full window keeps its slots busy (planned balance
    at least `floor`, routed and all-Global)."""
    cfg = hin.CONFIGS[name]
    g = cfg["geom"]
    for lab in (cfg["labels"], np.full(g.num_heads, 3, np.int32)):
        pb = hc.hc_plan_head_buffers(hc.make_desc(g), lab, g.window_frames // g.chunk_frames - 1)
        ents, _ = hc.hc_debug_routed_plan(pb)
        by_len = {}
        for head, hist, cur, nsplit, split_len, slot, begin, _q in ents:
            total = int(hist + cur)
            assert split_len % 64 == 0 and (nsplit - 1) * split_len < total <= nsplit * split_len
            if lab[head] != 2:   # a Spatial head's current block is never split
                by_len.setdefault(total, set()).add((int(nsplit), int(split_len)))
        assert all(len(v) == 1 for v in by_len.values()), by_len
        assert planned_balance(pb, g, lab) >= floor


@pytest.mark.parametrize("name", ["tiny", "480p", "720p", "1080p"])
@pytest.mark.parametrize("variant", [0, 1, 2, 3])
def test_routed_workspace_fits_every_fill_state(name, variant):
    """The routed workspace a handle asks for covers every later fill state of its
    window (warm-up with a growing history, then steady state)."""
    cfg = hin.CONFIGS[name]
    g = cfg["geom"]
    full = g.window_frames // g.chunk_frames - 1
    for lab in (cfg["labels"], np.full(g.num_heads, 3, np.int32), np.full(g.num_heads, 2, np.int32),
                np.full(g.num_heads, 0, np.int32)):
        d = hc.make_desc(g, variant)
        sizes = {hc.hc_routed_workspace_bytes(hc.hc_plan_head_buffers(d, lab, nb)) for nb in range(full + 4)}
        assert len(sizes) == 1, (name, variant, lab, sizes)


def test_fused_launch_form_limits():
    """The Spatial tiles join the dense launch for bf16, d = 128, sliding windows and at
    most 16 Spatial heads with at least one stored history frame; otherwise they keep
    their own launch (or have no history part at all)."""
    def fused(g, labels, nb, variant=0):
        return hc.hc_debug_spatial_plan(hc.hc_plan_head_buffers(hc.make_desc(g, variant), np.array(labels, np.int32), nb))[4]
    g = hin.Geometry(18, 128, 6, 9, 2, 8, 3, 3, "bf16")
    assert fused(g, [2] * 16 + [3, 0], 3) == 1
    assert fused(g, [2] * 17 + [3], 3) == 0
    assert fused(g, [2] * 16 + [3, 0], 0) == 0          # no history frame stored yet
    assert fused(g, [2] * 16 + [3, 0], 3, variant=4) == 0
    assert fused(g, [2] * 16 + [3, 0], 3, variant=2) == 0   # cells walk the current block too
    assert fused(dataclasses.replace(g, head_dim=64), [2] * 16 + [3, 0], 3) == 0
    assert fused(dataclasses.replace(g, dtype="f32"), [2] * 16 + [3, 0], 3) == 0


@pytest.mark.parametrize("name,variant,want", [("720p", 0, (5, 6, 1, 1)), ("480p", 0, (5, 6, 1, 1)),
                                               ("1080p", 0, (4, 8, 1, 1)), ("720p", 2, (5, 5, 1, 0)),
                                               ("480p", 2, (5, 5, 2, 0)), ("480p", 4, (5, 6, 3, 0)),
                                               ("720p", 4, (5, 6, 1, 0))])
def test_spatial_plan(name, variant, want):
    """Spatial tile, frame parts and launch form at the bench sizes: 24..32 positions
    inside the frame; sliding windows run their tiles in the dense launch (current-block
    and history partial per Spatial head) unless variant 4 asks for their own launch; in
    their own launch, parts only while the tiles leave workgroup slots free, at most one
    per frame; the partial slots (those of the Spatial heads plus the key splits) within
    the workspace."""
    cfg = hin.CONFIGS[name]
    g = cfg["geom"]
    if variant & 2:   # the pages' 10 x 10 cells
        g = dataclasses.replace(g, grid_h=10, grid_w=10)
    lab = cfg["labels"]
    n_sp = int((lab == 2).sum())
    pb = hc.hc_plan_head_buffers(hc.make_desc(g, variant), lab, g.window_frames // g.chunk_frames - 1)
    tr, tc, parts, slots, fused = hc.hc_debug_spatial_plan(pb)
    assert (tr, tc, parts, fused) == want
    assert 24 <= tr * tc <= 32 and tr <= g.frame_h and tc <= g.frame_w
    tiles = -(-g.frame_h // tr) * -(-g.frame_w // tc) * n_sp
    if not fused:
        assert parts == max(1, min(512 // tiles, 4, g.hist_frames + (g.chunk_frames if variant & 2 else 0)))
    ents, _ = hc.hc_debug_routed_plan(pb)
    split_slots = int(sum(e[3] for e in ents if e[3] > 1))
    if fused:
        assert parts == 1
        sp_slots = 2 * n_sp
    elif variant & 2:
        sp_slots = n_sp * parts if parts > 1 else 0
    else:
        sp_slots = n_sp * (1 + parts if parts > 1 else 1)
    assert slots == split_slots + sp_slots
    assert hc.hc_routed_workspace_bytes(pb) >= slots * g.lq * (g.head_dim + 2) * 4
    # no Spatial heads: no Spatial launch
    assert hc.hc_debug_spatial_plan(hc.hc_plan_head_buffers(hc.make_desc(g), np.full(g.num_heads, 3, np.int32),
                                                            1))[:3] == (0, 0, 0)


def test_binding_rejects_host_tensors():
    """The binding passes raw device pointers, so it refuses host tensors before any call."""
    import torch
    g = hin.CONFIGS["tiny"]["geom"]
    d = hc.make_desc(g)
    lab = hin.CONFIGS["tiny"]["labels"]
    x = torch.zeros((g.lq, g.num_heads, g.head_dim), dtype=torch.float32)
    with pytest.raises(hc.HCError) as ei:
        hc.hc_build_head_buffers(d, lab, x, x, g.chunk_frames)
    assert ei.value.status == 7
    pb = hc.hc_plan_head_buffers(d, lab, 1)
    for call in (lambda: hc.hc_routed_attention(pb, x, x, x), lambda: hc.hc_append_chunk(pb, x, x),
                 lambda: hc.hc_classify_heads(d, hc.hc_default_classify_params(), x, x, x, g.chunk_frames, x, x)):
        with pytest.raises(hc.HCError) as ei:
            call()
        assert ei.value.status == 7


def test_reduce_statistics_and_decision_match_oracle():
    rng = np.random.default_rng(0)
    lq, d = 333, 128
    ref = rng.standard_normal((lq, d))
    outs = [ref + s * rng.standard_normal((lq, d)) for s in (0.1, 0.5, 0.2)]
    o_sink, o_dummy, o_sp = outs
    per_tok = np.stack([orc.cosine(o_sink, ref), orc.cosine(o_dummy, ref), orc.cosine(o_sp, ref),
                        ((o_sp - ref) ** 2).sum(axis=1)], axis=1).astype(np.float32)
    # both sides from the same float32 per-token values
    f = per_tok.astype(np.float64)
    for gamma, pct in ((5.0, 5.0), (0.5, 5.0), (1.0, 37.5)):
        got = hc.hc_reduce_statistics(per_tok, d, gamma, pct)
        p5 = np.percentile(f[:, 2], pct)
        mse = f[:, 3].sum() / (lq * d)
        want = [f[:, 0].mean(), f[:, 1].mean(), f[:, 2].mean(), p5, mse, p5 - gamma * mse]
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    # oracle statistics on the float64 outputs agree to float32 rounding
    st = orc.head_statistics(o_sink, o_dummy, o_sp, ref, gamma=5.0)
    got = hc.hc_reduce_statistics(per_tok, d, 5.0)
    assert abs(got[0] - st["cos_sink"]) < 1e-6 and abs(got[5] - st["score"]) < 1e-5
    # Eq. 5 on a grid of values, including the thresholds themselves
    p = hc.hc_default_classify_params()
    vals = [0.0, 0.5, float(np.float32(0.755)), 0.9, float(np.float32(0.95)), 0.99]
    for a in vals:
        for b in vals:
            for c in vals:
                for s in vals:
                    assert hc.hc_decide(a, b, c, s, p) == orc.decide(
                        a, b, c, s, float(np.float32(0.95)), float(np.float32(0.95)),
                        float(np.float32(0.95)), float(np.float32(0.755)))


@pytest.mark.parametrize("F,C", [(21, 3), (5, 1), (6, 3), (3, 3), (12, 2)])
def test_variant_slot_table_matches_oracle(F, C):
    g = hin.Geometry(4, 64, 3, 5, C, F, 2, 2, "bf16")
    labels = [0, 1, 2, 3]
    for n in range(0, 14):
        pb = hc.hc_plan_head_buffers(hc.make_desc(g, hc.HC_VARIANT_DUMMY_PREVIOUS), labels, n)
        assert np.array_equal(hc.hc_debug_slot_table(pb),
                              orc.slot_table(labels, F, C, n, variant=orc.DUMMY_PREVIOUS_BLOCK)), n


def test_variant_plans():
    cfg = hin.CONFIGS["720p"]
    g = cfg["geom"]
    S = g.tokens_per_frame
    for var in (1, 2, 3):
        pb = hc.hc_plan_head_buffers(hc.make_desc(g, var), cfg["labels"], 7)
        ents, _ = hc.hc_debug_routed_plan(pb)
        heads = {int(r[0]): r for r in ents}
        for h, cls in enumerate(cfg["labels"]):
            if cls == 2 and var & 2:
                assert h not in heads                       # whole key set in the cell kernel
                continue
            if cls == 1:
                assert heads[h][1] == (g.chunk_frames * S if var & 1 else 0)
        n = hc.hc_head_buffers_bytes(hc.make_desc(g, var), cfg["labels"])
        base = hc.hc_head_buffers_bytes(hc.make_desc(g, 0), cfg["labels"])
        assert n - base == (2 * 3 * g.chunk_frames * S * g.head_dim * 2 if var & 1 else 0)
    with pytest.raises(hc.HCError):
        hc.hc_head_buffers_bytes(hc.make_desc(g, 8), cfg["labels"])
    # the launch option changes no buffer
    assert hc.hc_head_buffers_bytes(hc.make_desc(g, 4), cfg["labels"]) == \
        hc.hc_head_buffers_bytes(hc.make_desc(g, 0), cfg["labels"])


def test_build_at_block_validates_the_window_length():
    """hc_build_head_buffers_at: the history must be exactly the window's blocks when
    next_block is current (checked on the host, before any device call)."""
    import ctypes
    g = hin.Geometry(4, 64, 3, 5, 2, 10, 2, 2, "bf16")     # R = 3 rolling blocks
    d = hc.make_desc(g)
    L = hc.lib()
    lab = np.array([0, 1, 2, 3], np.int32)
    h = ctypes.c_void_p()
    C, R = g.chunk_frames, g.window_frames // g.chunk_frames - 2
    for nb, n_frames_ok in ((0, 0), (1, C), (3, 3 * C), (10, (1 + R) * C), (11, (1 + R) * C)):
        for n_frames in range(0, g.hist_frames + 1, C):
            st = L.hc_build_head_buffers_at(ctypes.byref(d), lab.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(16),
                                            ctypes.c_void_p(32), n_frames, nb, ctypes.c_void_p(4096), 1 << 40,
                                            ctypes.byref(h), None)
            if n_frames != n_frames_ok:
                assert st == 2, (nb, n_frames, st)
            else:   # valid arguments: only the missing device stops it here
                assert st in (0, 7), (nb, n_frames, st)
    st = L.hc_build_head_buffers_at(ctypes.byref(d), lab.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(16),
                                    ctypes.c_void_p(32), (1 + R) * C, -1, ctypes.c_void_p(4096), 1 << 40,
                                    ctypes.byref(h), None)
    assert st == 2


@pytest.mark.parametrize("F,C", [(21, 3), (10, 2), (6, 3)])
def test_resumed_plan_slot_table_at_block_10(F, C):
    """A handle for a rollout resumed at block 10 reports the slot table of the oracle's
    ring after ten stored blocks."""
    g = hin.Geometry(4, 64, 3, 5, C, F, 2, 2, "bf16")
    labels = [0, 1, 2, 3]
    pb = hc.hc_plan_head_buffers(hc.make_desc(g), labels, 10)
    assert np.array_equal(hc.hc_debug_slot_table(pb), orc.slot_table(labels, F, C, 10))


@pytest.mark.parametrize("name", ["tiny", "480p", "720p", "1080p"])
@pytest.mark.parametrize("global_only", [False, True])
def test_dense_xcd_queues_cover_items_balanced_longest_first(name, global_only):
    """The dense launch's per-XCD queues hold every item exactly once, each queue runs
    longest items first, every XCD gets an equal share (within one item) of every class
    of equally long items, and a key-range group spans few XCDs."""
    cfg = hin.CONFIGS[name]
    g = cfg["geom"]
    labels = np.full(g.num_heads, 3, np.int32) if global_only else cfg["labels"]
    pb = hc.hc_plan_head_buffers(hc.make_desc(g), labels, 7)
    ents, n_items = hc.hc_debug_routed_plan(pb)
    queues, qlen = hc.hc_debug_dense_queues(pb)
    nqt = -(-g.lq // int(ents[0, 7]))
    cost = np.zeros(n_items)
    group = np.zeros(n_items, np.int64)
    for head, hist, cur, nsplit, split_len, slot, item_begin, _q in ents:
        for sp in range(nsplit):
            lo = item_begin + sp * nqt
            cost[lo:lo + nqt] = min(split_len, hist + cur - sp * split_len) / 64 + 9.0
            group[lo:lo + nqt] = lo
    tr, tc, parts, _, fused = hc.hc_debug_spatial_plan(pb)
    if fused:   # then the Spatial items, head by head, one class of the planner's item cost
        n_sp = int(np.sum(labels == 2))
        n_per = -(-g.frame_h // tr) * -(-g.frame_w // tc) * parts
        n_hist = len(orc.window_history_blocks(7, g.window_frames, g.chunk_frames)) * g.chunk_frames
        chunks = max(spatial_tile_chunks(g, tr, tc))
        cost = np.concatenate([cost, np.full(n_sp * n_per, 1.2 * chunks * -(-n_hist // parts) * 32 / 64 + 9.0)])
        group = np.concatenate([group, n_items + (np.arange(n_sp * n_per) // n_per) * n_per])
        n_items += n_sp * n_per
    seen = np.zeros(n_items, np.int64)
    per_class = {}
    spans = {}
    for x, q in enumerate(queues):
        assert len(q) <= 16
        items = [f + i for f, c in q for i in range(c)]
        seen[items] += 1
        assert all(cost[a] >= cost[b] for a, b in zip(items, items[1:]))
        for c in set(cost[items]):
            per_class.setdefault(c, []).append(int(np.sum(cost[items] == c)))
        for i in items:
            spans.setdefault(group[i], set()).add(x)
    assert np.all(seen == 1)
    assert qlen == max(sum(c for _, c in q) for q in queues)
    for c, counts in per_class.items():
        counts += [0] * (8 - len(counts))
        assert max(counts) - min(counts) <= 1, (c, counts)
    # groups of a class with at least 8 groups' worth of items span at most 3 XCDs
    n_groups = {c: len({group[i] for i in range(n_items) if cost[i] == c}) for c in per_class}
    for gid, xs in spans.items():
        if n_groups[cost[gid]] >= 8:
            assert len(xs) <= 3, (gid, xs)


def test_random_layers_plan_invariants():
    """Seeded random layers (head count, head size, frame, block, window, grid, dtype,
    variant and launch option, label mix, fill state of the window): every head planned
    once, every key range cut into pieces that cover it exactly, every item of the dense
    launch (Spatial tiles included when they join it) in exactly one XCD queue, the
    partial slots within the workspace the handle asks for, and the launch form of the
    Spatial path as its rules say."""
    rng = np.random.default_rng(2024)
    for case in range(600):
        d = int(rng.choice([64, 128]))
        C = int(rng.integers(1, 5))
        g = hin.Geometry(int(rng.integers(1, 65)), d, int(rng.integers(1, 48)), int(rng.integers(1, 72)), C,
                         C * int(rng.integers(1, 9)), int(rng.integers(1, 13)), int(rng.integers(1, 13)),
                         str(rng.choice(["bf16", "f32"])))
        variant = int(rng.integers(0, 8))
        labels = rng.integers(0, 4, g.num_heads).astype(np.int32)
        R = max(g.window_frames // C - 2, 0)
        next_block = int(rng.integers(0, 2 * R + 4))
        pb = hc.hc_plan_head_buffers(hc.make_desc(g, variant), labels, next_block)
        what = (case, g, variant, list(labels), next_block)
        ents, n_items = hc.hc_debug_routed_plan(pb)
        heads = [int(e[0]) for e in ents]
        assert len(set(heads)) == len(heads) and set(heads) <= set(range(g.num_heads)), what
        qtile = int(ents[0, 7]) if len(ents) else 128
        nqt = -(-g.lq // qtile)
        begin = 0
        for head, hist, cur, nsplit, split_len, slot, item_begin, _q in ents:
            total = int(hist) + int(cur)
            assert 0 <= hist <= (g.window_frames - C) * g.tokens_per_frame and total >= 1, what
            assert nsplit >= 1 and split_len % 64 == 0, what
            assert (nsplit - 1) * split_len < total <= nsplit * split_len, what
            assert item_begin == begin, what
            begin += int(nsplit) * nqt
        assert begin == n_items, what
        tr, tc, parts, slots, fused = hc.hc_debug_spatial_plan(pb)
        n_sp = int(np.sum(labels == 2))
        has_hist = len(orc.window_history_blocks(next_block, g.window_frames, C)) > 0
        want_fused = (g.dtype == "bf16" and d == 128 and not variant & 6 and 0 < n_sp <= 16 and has_hist)
        assert bool(fused) == want_fused, what
        if n_items:
            queues, _ = hc.hc_debug_dense_queues(pb)
            n_all = n_items + (n_sp * -(-g.frame_h // tr) * -(-g.frame_w // tc) * parts if fused else 0)
            seen = np.zeros(n_all, np.int64)
            for q in queues:
                for f, c in q:
                    seen[f:f + c] += 1
            assert np.all(seen == 1), what
        assert hc.hc_routed_workspace_bytes(pb) >= slots * g.lq * (g.head_dim + 2) * 4, what


def test_random_slot_tables_match_oracle():
    """Seeded random windows, label mixes, Dummy variants and block counts (the ring
    rolling over several times): the handle's slot table equals the oracle's."""
    rng = np.random.default_rng(31)
    for case in range(400):
        C = int(rng.integers(1, 5))
        F = C * int(rng.integers(1, 10))
        g = hin.Geometry(int(rng.integers(1, 17)), int(rng.choice([64, 128])), 3, 4, C, F, 2, 2, "bf16")
        labels = rng.integers(0, 4, g.num_heads).astype(np.int32)
        variant = int(rng.choice([0, 1]))
        n = int(rng.integers(0, 4 * max(F // C, 1) + 3))
        pb = hc.hc_plan_head_buffers(hc.make_desc(g, variant), labels, n)
        want = orc.slot_table(labels, F, C, n, variant=orc.DUMMY_PREVIOUS_BLOCK if variant else 0)
        assert np.array_equal(hc.hc_debug_slot_table(pb), want), (case, F, C, list(labels), variant, n)
