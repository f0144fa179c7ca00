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
    ("softmax_scale", -1.0, 2), ("frame_w", 30000, 2)])
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
        nqt = -(-g.lq // 128)
        hist_blocks = orc.window_history_blocks(next_block, g.window_frames, g.chunk_frames)
        assert sorted(ents[:, 0]) == list(range(g.num_heads))
        begin = 0
        for head, hist, cur, nsplit, split_len, slot, item_begin, _ in ents:
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


@pytest.mark.parametrize("name,variant,want", [("720p", 0, (5, 6, 1)), ("480p", 0, (5, 6, 3)),
                                               ("1080p", 0, (4, 8, 1)), ("720p", 2, (5, 5, 1)),
                                               ("480p", 2, (5, 5, 2))])
def test_spatial_plan(name, variant, want):
    """Spatial tile and frame parts at the bench sizes: 24..32 positions inside the frame,
    parts only while the tiles leave workgroup slots free, at most one per frame, and
    the partial slots (current block + one per part per Spatial head, plus the key
    splits) within the workspace."""
    cfg = hin.CONFIGS[name]
    g = cfg["geom"]
    if variant & 2:   # the pages' 10 x 10 cells
        g = dataclasses.replace(g, grid_h=10, grid_w=10)
    lab = cfg["labels"]
    n_sp = int((lab == 2).sum())
    pb = hc.hc_plan_head_buffers(hc.make_desc(g, variant), lab, g.window_frames // g.chunk_frames - 1)
    tr, tc, parts, slots = hc.hc_debug_spatial_plan(pb)
    assert (tr, tc, parts) == want
    assert 24 <= tr * tc <= 32 and tr <= g.frame_h and tc <= g.frame_w
    tiles = -(-g.frame_h // tr) * -(-g.frame_w // tc) * n_sp
    assert parts == max(1, min(512 // tiles, 4, g.hist_frames + (g.chunk_frames if variant & 2 else 0)))
    ents, _ = hc.hc_debug_routed_plan(pb)
    split_slots = int(sum(e[3] for e in ents if e[3] > 1))
    sp_slots = (n_sp * parts if parts > 1 else 0) if variant & 2 else n_sp * (1 + parts if parts > 1 else 1)
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
        hc.hc_head_buffers_bytes(hc.make_desc(g, 4), cfg["labels"])
