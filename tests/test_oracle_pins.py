"""Pins of the CPU oracle against facts fixed outside it: brute force, closed forms,
library routines, textbook identities and the pages' printed shapes and constants.

A plausible slip in the oracle (a dropped key class, a transposed row/col, an
off-by-one in the window origin, a wrong ring slot, a flipped comparison) fails at
least one of these.
"""
import collections
import json
import os

import numpy as np
import pytest
import torch

from head_routed_sparse_amd import inputs as hin
from oracle import headcast_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
S_, D_, P_, G_ = orc.SINK, orc.DUMMY, orc.SPATIAL, orc.GLOBAL


def small_geom(fh=5, fw=7, C=2, F=6, g=3, d=16, H=4, dtype="f32"):
    return hin.Geometry(H, d, fh, fw, C, F, g, g, dtype)


def small_inputs(geom, seed=11, n_hist=None, labels=(0, 1, 2, 3), planted=False):
    return hin.generate(geom, list(labels)[: geom.num_heads], seed, n_hist, planted)


# ----------------------------------------------------------------------------- P1
@pytest.mark.parametrize("g", [1, 2, 3, 8])
@pytest.mark.parametrize("cls", [S_, D_, P_, G_])
def test_p1_brute_force_matches_masked_dense(cls, g):
    geom = small_geom(g=g)
    inp = small_inputs(geom)
    h = 1
    rows = np.arange(geom.lq)
    dense = orc.path_attention(inp, h, cls, rows)
    for t in rows:
        bf = orc.brute_force_attention(inp, h, cls, int(t))
        assert np.max(np.abs(bf - dense[t])) < 1e-12


def test_p1_brute_force_sink_proxy_and_partial_window():
    geom = small_geom()
    inp = small_inputs(geom, n_hist=2)          # only the sink block is present
    dense = orc.path_attention(inp, 0, S_, sink_proxy=True)
    for t in range(geom.lq):
        assert np.allclose(orc.brute_force_attention(inp, 0, S_, t, sink_proxy=True), dense[t],
                           atol=1e-12, rtol=0)
    for cls in (S_, D_, P_, G_):
        dense = orc.path_attention(inp, 2, cls)
        for t in (0, 9, geom.lq - 1):
            assert np.allclose(orc.brute_force_attention(inp, 2, cls, t), dense[t], atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------- P2
@pytest.mark.parametrize("cls", [S_, D_, P_, G_])
def test_p2_softmax_rows_sum_to_one_and_vanish_outside_key_set(cls):
    geom = small_geom()
    inp = small_inputs(geom)
    rows = np.arange(geom.lq)
    qh, kh, vh = orc.head_window(inp.q, inp.k_hist, inp.v_hist, inp.k_cur, inp.v_cur, 0)
    m = orc.key_set_mask(cls, geom, inp.n_hist_frames, rows)
    _, _, p = orc.masked_attention(qh, kh, vh, m, orc.attention_scale(geom.head_dim), return_weights=True)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12
    assert np.all(p[~m] == 0.0)
    assert np.all(p[m] > 0.0)


# ----------------------------------------------------------------------------- P3, P4
def test_p3_full_frame_grid_makes_spatial_global():
    geom = small_geom(g=7)           # g >= max(5, 7)
    inp = small_inputs(geom)
    rows = np.arange(geom.lq)
    assert np.array_equal(orc.key_set_mask(P_, geom, inp.n_hist_frames, rows),
                          orc.key_set_mask(G_, geom, inp.n_hist_frames, rows))
    assert np.allclose(orc.path_attention(inp, 3, P_), orc.path_attention(inp, 3, G_), atol=1e-14, rtol=0)
    # and a grid smaller than the frame is a strict subset
    geom2 = small_geom(g=3)
    m_sp = orc.key_set_mask(P_, geom2, inp.n_hist_frames, rows)
    assert m_sp.sum() < orc.key_set_mask(G_, geom2, inp.n_hist_frames, rows).sum()


def test_p4_one_block_window_makes_all_paths_equal():
    geom = small_geom(C=2, F=2)
    inp = small_inputs(geom)
    assert inp.n_hist_frames == 0
    outs = [orc.path_attention(inp, 2, c) for c in (S_, D_, P_, G_)]
    for o in outs[1:]:
        assert np.allclose(o, outs[0], atol=1e-14, rtol=0)


# ----------------------------------------------------------------------------- P5
def test_p5_all_global_equals_library_sdpa():
    geom = small_geom(fh=6, fw=4, C=1, F=4, d=32)
    inp = small_inputs(geom)
    ours = orc.routed_attention(inp, labels=[G_] * geom.num_heads)
    for h in range(geom.num_heads):
        q = torch.from_numpy(inp.q[:, h, :].astype(np.float64))[None, None]
        k = torch.from_numpy(np.concatenate([inp.k_hist[:, h], inp.k_cur[:, h]]).astype(np.float64))[None, None]
        v = torch.from_numpy(np.concatenate([inp.v_hist[:, h], inp.v_cur[:, h]]).astype(np.float64))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, 0].numpy()
        assert np.max(np.abs(ref - ours[:, h, :])) < 1e-12


# ----------------------------------------------------------------------------- P6
def nearest_feasible_origin(pos, g, extent):
    """Independent of the oracle: among origins whose window lies in the frame, the one
    closest to placing the query at offset g//2 (whole frame when g >= extent)."""
    if g >= extent:
        return 0
    cands = np.arange(0, extent - g + 1)
    return int(cands[np.argmin(np.abs(cands - (pos - g // 2)))])


def moment_values(geom, n_hist):
    """V columns (1, frame, row, col, row^2, col^2) for every window token."""
    S, fw = geom.tokens_per_frame, geom.frame_w
    n = (n_hist + geom.chunk_frames) * S
    t = np.arange(n)
    f, r, c = t // S, (t % S) // fw, t % fw
    cols = np.stack([np.ones(n), f, r, c, r * r, c * c], axis=1).astype(np.float32)
    v = np.zeros((n, geom.num_heads, geom.head_dim), np.float32)
    v[:, :, :6] = cols[:, None, :]
    return v


def expected_moments(geom, n_hist, cls, t):
    """Mean of (1, frame, row, col, row^2, col^2) over the key set, by counting."""
    C, fh, fw = geom.chunk_frames, geom.frame_h, geom.frame_w
    S = fh * fw
    rows_all = np.arange(fh)
    cols_all = np.arange(fw)

    def block(frames, rr, cc):
        # sums over the cartesian product frames x rr x cc
        nf, nr, nc = len(frames), len(rr), len(cc)
        return np.array([nf * nr * nc, sum(frames) * nr * nc, nf * nc * sum(rr), nf * nr * sum(cc),
                         nf * nc * sum(x * x for x in rr), nf * nr * sum(x * x for x in cc)], float)

    cur = list(range(n_hist, n_hist + C))
    hist = list(range(n_hist))
    tot = block(cur, rows_all, cols_all)
    if cls == G_:
        tot = tot + block(hist, rows_all, cols_all)
    elif cls == S_:
        tot = tot + block(hist[:C], rows_all, cols_all)
    elif cls == P_:
        qr, qc = (t % S) // fw, t % fw
        r0 = nearest_feasible_origin(qr, geom.grid_h, fh)
        c0 = nearest_feasible_origin(qc, geom.grid_w, fw)
        rr = list(range(r0, min(r0 + geom.grid_h, fh)))
        cc = list(range(c0, min(c0 + geom.grid_w, fw)))
        tot = tot + block(hist, rr, cc)
    return tot / tot[0]


@pytest.mark.parametrize("g", [1, 2, 3, 4, 9])
def test_p6_zero_query_gives_key_set_moments(g):
    geom = small_geom(fh=5, fw=7, C=2, F=8, g=g)
    inp = small_inputs(geom)
    inp.q[:] = 0.0
    inp.v_hist[:] = moment_values(geom, inp.n_hist_frames)[: inp.n_hist_frames * geom.tokens_per_frame]
    inp.v_cur[:] = moment_values(geom, inp.n_hist_frames)[inp.n_hist_frames * geom.tokens_per_frame:]
    for h, cls in enumerate((S_, D_, P_, G_)):
        out = orc.path_attention(inp, h, cls)
        for t in range(geom.lq):
            assert np.allclose(out[t, :6], expected_moments(geom, inp.n_hist_frames, cls, t),
                               atol=1e-12, rtol=0), (cls, t)


# ----------------------------------------------------------------------------- P7
def test_p7_lse_merge_of_disjoint_parts_equals_union():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((9, 8))
    k = rng.standard_normal((40, 8)) * 2
    v = rng.standard_normal((40, 8))
    full = np.ones((9, 40), bool)
    a = np.zeros((9, 40), bool)
    a[:, :13] = True
    b = ~a
    o, _ = orc.masked_attention(q, k, v, full, 0.3)
    oa = orc.masked_attention(q, k, v, a, 0.3)
    ob = orc.masked_attention(q, k, v, b, 0.3)
    assert np.max(np.abs(orc.merge_partials([oa, ob]) - o)) < 1e-13


# ----------------------------------------------------------------------------- P8
def simulate_buffer(labels, F, C, n_blocks):
    """Independent ring model: the sink block is kept; rolling blocks fill the first
    empty position, then replace the oldest one (FIFO)."""
    H = len(labels)
    R = max(F // C - 2, 0)
    table = -np.ones((H, F - C), np.int32)
    for h, cls in enumerate(labels):
        if cls == D_ or F == C:
            continue
        pos_of = {}
        order = collections.deque()
        for b in range(n_blocks):
            if b == 0:
                pos_of[0] = 0
                continue
            if cls == S_ or R == 0:
                continue
            used = {pos_of[x] for x in order}
            free = [p for p in range(1, R + 1) if p not in used]
            if free:
                pos = free[0]
            else:
                oldest = order.popleft()
                pos = pos_of.pop(oldest)
            pos_of[b] = pos
            order.append(b)
        for b, pos in pos_of.items():
            for i in range(C):
                table[h, pos * C + i] = b * C + i
    return table


@pytest.mark.parametrize("F,C", [(21, 3), (5, 1), (6, 3), (3, 3), (12, 2)])
def test_p8_ring_slot_table(F, C):
    labels = [S_, D_, P_, G_]
    for n in range(0, 20):
        tab = orc.slot_table(labels, F, C, n)
        assert np.array_equal(tab, simulate_buffer(labels, F, C, n)), n
        # Global/Spatial buffers hold exactly the window's history frames
        want = sorted(b * C + i for b in orc.window_history_blocks(n, F, C) for i in range(C))
        for h in (2, 3):
            assert sorted(x for x in tab[h] if x >= 0) == want


def test_p8_ring_closed_form_values():
    # F=21, C=3: rolling capacity 5; block 6 -> position 1 + 5 % 5 = 1 (overwrites block 1)
    assert orc.rolling_capacity(21, 3) == 5
    assert orc.buffer_position_of_block(0, 21, 3) == 0
    assert orc.buffer_position_of_block(1, 21, 3) == 1
    assert orc.buffer_position_of_block(5, 21, 3) == 5
    assert orc.buffer_position_of_block(6, 21, 3) == 1
    assert orc.buffer_position_of_block(7, 6, 3) is None
    assert orc.window_history_blocks(9, 21, 3) == [0, 4, 5, 6, 7, 8]


# ----------------------------------------------------------------------------- P9
def test_p9_gather_origins():
    for extent in (1, 5, 8, 30, 52):
        for g in (1, 2, 3, 8, 9, 60):
            for pos in range(extent):
                assert int(orc.window_origin(pos, g, extent)) == nearest_feasible_origin(pos, g, extent)
    # hand values: 30-row frame, g = 8 (query at offset 4 of the window)
    assert [int(orc.window_origin(r, 8, 30)) for r in (0, 3, 4, 5, 10, 25, 26, 29)] == [0, 0, 0, 1, 6, 21, 22, 22]
    assert [int(orc.window_origin(r, 3, 8)) for r in (0, 1, 2, 7)] == [0, 0, 1, 5]
    assert int(orc.window_origin(17, 40, 30)) == 0 and orc.window_extent(40, 30) == 30


# ----------------------------------------------------------------------------- P10
def test_p10_decision_rule_priorities_and_ties():
    d = orc.decide
    assert d(0.95, 0.0, 0.0, 0.0) == S_                 # >= at the threshold
    assert d(0.9499999, 0.95, 0.0, 0.0) == D_
    assert d(0.99, 0.99, 0.99, 0.99) == S_              # Sink checked first
    assert d(0.1, 0.99, 0.99, 0.99) == D_               # then Dummy
    assert d(0.1, 0.1, 0.95, 0.755) == P_               # Spatial needs both
    assert d(0.1, 0.1, 0.96, 0.754) == G_
    assert d(0.1, 0.1, 0.94, 0.9) == G_
    assert d(0.5, 0.5, 0.5, 0.5, theta_sink=0.4) == S_
    assert d(0.5, 0.5, 0.5, 0.5, theta_sink=0.6, theta_dummy=0.5) == D_
    assert d(0.5, 0.5, 0.5, 0.5, 0.6, 0.6, 0.5, 0.5) == P_


# ----------------------------------------------------------------------------- P11
def test_p11_statistics_closed_forms():
    c = orc.cosine(np.array([[1.0, 0.0], [3.0, 4.0], [0.0, 0.0], [1.0, 1.0]]),
                   np.array([[1.0, 1.0], [-3.0, -4.0], [1.0, 2.0], [2.0, 2.0]]))
    assert np.allclose(c, [1 / np.sqrt(2), -1.0, 0.0, 1.0], atol=1e-15)
    # P5 with linear interpolation: index 0.05 * (n - 1)
    n = 101
    ref = np.zeros((n, 2))
    ref[:, 0] = 1.0
    ang = np.linspace(0.0, np.pi / 2, n)                # token cosines cos(ang), sorted desc
    sp = np.stack([np.cos(ang), np.sin(ang)], axis=1)
    st = orc.head_statistics(ref, ref, sp, ref, gamma=2.0)
    cos_sorted = np.sort(np.cos(ang))
    assert abs(st["p5"] - cos_sorted[5]) < 1e-15       # 0.05 * 100 = 5 exactly
    mse = np.mean((sp - ref) ** 2)
    assert abs(st["mse"] - mse) < 1e-15
    assert abs(st["score"] - (cos_sorted[5] - 2.0 * mse)) < 1e-15
    assert abs(st["cos_sink"] - 1.0) < 1e-15 and abs(st["cos_spatial"] - np.mean(np.cos(ang))) < 1e-15
    st2 = orc.head_statistics(ref[:5], ref[:5], sp[[0, 25, 50, 75, 100]], ref[:5], gamma=0.0)
    # five values sorted: cos(pi/2), cos(3pi/8), cos(pi/4), cos(pi/8), 1 -> index 0.2
    v = np.cos(np.array([np.pi / 2, 3 * np.pi / 8]))
    assert abs(st2["p5"] - (v[0] + 0.2 * (v[1] - v[0]))) < 1e-15


# ----------------------------------------------------------------------------- P12
def test_p12_planted_heads_recovered_with_margin():
    geom = hin.Geometry(8, 64, 12, 20, 3, 21, 8, 8, "bf16")
    labels = [S_, D_, P_, G_, G_, P_, D_, S_]
    inp = hin.generate(geom, labels, seed=5, planted=True)
    got, stats = orc.classify_heads(inp, dict(gamma=0.5))
    assert list(got) == labels
    th = 0.95
    for lab, st in zip(labels, stats):
        if lab == S_:
            assert st["cos_sink"] >= th + 0.04
        else:
            assert st["cos_sink"] <= th - 0.04
        if lab == D_:
            assert st["cos_dummy"] >= th + 0.04
        elif lab != S_:
            assert st["cos_dummy"] <= th - 0.04
        if lab == P_:
            assert st["cos_spatial"] >= th + 0.04 and st["score"] >= 0.755 + 0.04
        if lab == G_:
            assert st["cos_spatial"] <= th - 0.04 or st["score"] <= 0.755 - 0.04


def test_p12_sink_proxy_reading_matters():
    """With a sink proxy that also sees the current block, a planted Dummy head is
    taken for Sink (the proxy would contain the Dummy key set)."""
    geom = hin.Geometry(2, 64, 12, 20, 3, 21, 8, 8, "bf16")
    inp = hin.generate(geom, [D_, G_], seed=6, planted=True)
    got, _ = orc.classify_heads(inp, dict(gamma=0.5))
    assert list(got) == [D_, G_]
    got2, _ = orc.classify_heads(inp, dict(gamma=0.5, sink_proxy_includes_current=True))
    assert got2[0] == S_


# ----------------------------------------------------------------------------- pages' figures
def test_pages_shapes_and_constants():
    with open(os.path.join(GOLDEN, "pages_shapes.json")) as f:
        gold = json.load(f)
    g480 = hin.CONFIGS["480p"]["geom"]
    assert g480.frame_h * g480.frame_w == gold["tokens_per_frame_480p"]
    assert g480.lq == gold["queries_per_block_480p"]
    assert 9 * g480.tokens_per_frame == gold["window_keys_480p_frame6"]
    assert g480.window_frames * g480.tokens_per_frame == gold["window_keys_480p_frame18"]
    assert g480.chunk_frames == gold["frames_per_block"]
    assert g480.window_frames // g480.chunk_frames == gold["blocks_per_window_30s"]
    p = orc.DEFAULT_PARAMS
    assert (p["theta_sink"], p["theta_dummy"], p["theta_spatial"]) == tuple(gold["theta"])
    assert p["theta_score"] == gold["theta_score"] and p["gamma"] == gold["gamma"]


def test_pages_flop_model_ratio():
    """App. B: with an 8-block window, a Sink head costs 2 of a Global head's 8 block
    units (key count ratio 1/4); a Dummy head attending the current block only costs 1/8."""
    geom = small_geom(fh=3, fw=4, C=2, F=16)
    rows = np.arange(geom.lq)
    n = {c: orc.key_set_mask(c, geom, geom.hist_frames, rows).sum() for c in (S_, D_, G_)}
    assert n[S_] * 4 == n[G_]
    assert n[D_] * 8 == n[G_]


# ----------------------------------------------------------------------------- variants
V_DPREV, V_CELLS = orc.DUMMY_PREVIOUS_BLOCK, orc.SPATIAL_CELLS


@pytest.mark.parametrize("g", [1, 2, 3, 4, 8])
def test_variants_brute_force(g):
    geom = small_geom(fh=5, fw=7, C=2, F=8, g=g)
    inp = small_inputs(geom)
    for cls, var in ((D_, V_DPREV), (P_, V_CELLS), (P_, V_CELLS | V_DPREV)):
        dense = orc.path_attention(inp, 2, cls, variant=var)
        for t in range(geom.lq):
            bf = orc.brute_force_attention(inp, 2, cls, t, variant=var)
            assert np.max(np.abs(bf - dense[t])) < 1e-12, (cls, var, t)


def test_variant_special_cases():
    # one cell covering the frame: Spatial cells = Global
    geom = small_geom(fh=5, fw=7, C=2, F=8, g=7)
    inp = small_inputs(geom)
    assert np.allclose(orc.path_attention(inp, 1, P_, variant=V_CELLS), orc.path_attention(inp, 1, G_),
                       atol=1e-14, rtol=0)
    # window = sink block + current block: the previous block is the sink block
    geom = small_geom(fh=5, fw=7, C=2, F=4)
    inp = small_inputs(geom)
    assert np.allclose(orc.path_attention(inp, 1, D_, variant=V_DPREV), orc.path_attention(inp, 1, S_),
                       atol=1e-14, rtol=0)
    # 1x1 cells: every query sees exactly its own position in each window frame
    geom = small_geom(fh=5, fw=7, C=2, F=8, g=1)
    rows = np.arange(geom.lq)
    m = orc.key_set_mask(P_, geom, geom.hist_frames, rows, variant=V_CELLS)
    assert np.all(m.sum(axis=1) == geom.window_frames)
    kf, kr, kc = orc.key_coords(geom.frame_h, geom.frame_w, geom.window_frames)
    S = geom.tokens_per_frame
    for t in (0, 13, geom.lq - 1):
        assert np.all(kr[m[t]] == (t % S) // geom.frame_w) and np.all(kc[m[t]] == t % geom.frame_w)


def test_variant_cell_geometry_hand_values():
    # 45-row frame, 10-row cells: four full cells and a 5-row remainder cell
    assert [int(orc.cell_origin(r, 10)) for r in (0, 9, 10, 39, 40, 44)] == [0, 0, 10, 30, 40, 40]
    assert [int(orc.cell_extent(r, 10, 45)) for r in (0, 39, 40, 44)] == [10, 10, 5, 5]


@pytest.mark.parametrize("g", [1, 2, 3, 4, 9])
def test_variant_zero_query_moments(g):
    geom = small_geom(fh=5, fw=7, C=2, F=8, g=g)
    inp = small_inputs(geom)
    inp.q[:] = 0.0
    S = geom.tokens_per_frame
    mv = moment_values(geom, inp.n_hist_frames)
    inp.v_hist[:] = mv[: inp.n_hist_frames * S]
    inp.v_cur[:] = mv[inp.n_hist_frames * S:]
    n_hist, C = inp.n_hist_frames, geom.chunk_frames

    def block(frames, rr, cc):
        nf, nr, nc = len(frames), len(rr), len(cc)
        return np.array([nf * nr * nc, sum(frames) * nr * nc, nf * nc * sum(rr), nf * nr * sum(cc),
                         nf * nc * sum(x * x for x in rr), nf * nr * sum(x * x for x in cc)], float)

    out_d = orc.path_attention(inp, 1, D_, variant=V_DPREV)
    out_p = orc.path_attention(inp, 2, P_, variant=V_CELLS)
    frames_d = list(range(n_hist - C, n_hist + C))
    for t in range(geom.lq):
        want = block(frames_d, range(geom.frame_h), range(geom.frame_w))
        assert np.allclose(out_d[t, :6], want / want[0], atol=1e-12, rtol=0)
        qr, qc = (t % S) // geom.frame_w, t % geom.frame_w
        rr = [r for r in range(geom.frame_h) if r // g == qr // g]          # the cell, by scanning rows
        cc = [c for c in range(geom.frame_w) if c // g == qc // g]
        want = block(list(range(n_hist + C)), rr, cc)
        assert np.allclose(out_p[t, :6], want / want[0], atol=1e-12, rtol=0)


@pytest.mark.parametrize("F,C", [(21, 3), (5, 1), (6, 3), (12, 2)])
def test_variant_dummy_buffer_holds_latest_block(F, C):
    for n in range(0, 12):
        tab = orc.slot_table([S_, D_, P_, G_], F, C, n, variant=V_DPREV)
        want = -np.ones(F - C, np.int32)
        if n > 0:
            # the latest finished block while rolling blocks exist, else the sink block
            b = n - 1 if F // C > 2 else 0
            want[:C] = np.arange(b * C, b * C + C)
        assert np.array_equal(tab[1], want)
        assert np.array_equal(tab[[0, 2, 3]], orc.slot_table([S_, P_, G_], F, C, n))


# ----------------------------------------------------------------------------- routing and proxy pins
def test_p1_routed_mixed_labels_follow_each_heads_own_class():
    """Routing (Sec. 4.4): on an unsorted mix of classes, head h's output is the brute
    force attention over the key set of ITS OWN label, row by row."""
    geom = small_geom(fh=5, fw=7, C=2, F=8, g=3, H=6)
    labels = [G_, S_, P_, D_, D_, G_]
    inp = small_inputs(geom, seed=31, labels=labels)
    out = orc.routed_attention(inp)
    for h, cls in enumerate(labels):
        for t in range(geom.lq):
            bf = orc.brute_force_attention(inp, h, cls, t)
            assert np.max(np.abs(out[t, h] - bf)) < 1e-12, (h, cls, t)
    # and a different class gives a different answer for every non-Global head here
    for h, cls in enumerate(labels):
        other = G_ if cls != G_ else D_
        assert np.max(np.abs(out[:, h] - orc.path_attention(inp, h, other))) > 1e-3


def test_p11_classify_with_proxy_grid_uses_that_grid():
    """Classification (Sec. 4.2, Eqs. 3-5) with a Spatial proxy window other than the
    routing grid: the statistics equal those built from brute-force outputs of the
    reference, the three proxies and the 5 x 5 window, and differ from the routing grid's."""
    geom = small_geom(fh=7, fw=9, C=2, F=8, g=3, d=16, H=4)
    labels = [P_, G_, P_, D_]
    inp = small_inputs(geom, seed=32, labels=labels, planted=True)
    proxy = (5, 5)
    got_labels, got = orc.classify_heads(inp, dict(gamma=0.5, proxy_grid=proxy))
    rows = range(geom.lq)
    for h in range(geom.num_heads):
        ref = np.array([orc.brute_force_attention(inp, h, G_, t) for t in rows])
        snk = np.array([orc.brute_force_attention(inp, h, S_, t, sink_proxy=True) for t in rows])
        dum = np.array([orc.brute_force_attention(inp, h, D_, t) for t in rows])
        spa = np.array([orc.brute_force_attention(inp, h, P_, t, grid=proxy) for t in rows])
        spa_routing = np.array([orc.brute_force_attention(inp, h, P_, t) for t in rows])
        want = orc.head_statistics(snk, dum, spa, ref, gamma=0.5)
        for k in ("cos_sink", "cos_dummy", "cos_spatial", "p5", "mse", "score"):
            assert abs(got[h][k] - want[k]) < 1e-12, (h, k)
        assert got_labels[h] == orc.decide(want["cos_sink"], want["cos_dummy"], want["cos_spatial"], want["score"])
        if labels[h] != D_:   # (a planted Dummy head attends to the current block either way)
            other = orc.head_statistics(snk, dum, spa_routing, ref, gamma=0.5)
            assert abs(other["cos_spatial"] - want["cos_spatial"]) > 1e-4, h
