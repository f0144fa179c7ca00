"""GPU parity of the HIP path against the CPU fp64 oracle, through the C ABI.

Bit-exact: buffer contents, slot tables, Spatial window origins, labels.
Floating point (outputs against the oracle on the same bf16-rounded inputs):
max-abs <= 1e-2 and mean-abs <= 1e-3 for bf16; max-abs <= 1e-4 for fp32 inputs.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

from gpu_util import TOL, assert_close, dev, host, sample_rows, to_device
from head_routed_sparse_amd import headcast as hc
from head_routed_sparse_amd import inputs as hin
from oracle import headcast_oracle as orc

pytestmark = pytest.mark.gpu
S_, D_, P_, G_ = 0, 1, 2, 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hc.lib()
    yield
    torch.cuda.synchronize()


def run_routed(inp, labels=None):
    g = inp.geom
    labels = inp.labels if labels is None else labels
    t = to_device(inp)
    d = hc.make_desc(g)
    buf = hc.hc_build_head_buffers(d, labels, t["k_hist"], t["v_hist"], inp.n_hist_frames)
    out = hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"])
    torch.cuda.synchronize()
    return host(out), buf, t


GEOMS = {
    # several query tiles with a ragged tail, several key tiles with a ragged tail
    "10x13_C2_F8_d128": hin.Geometry(4, 128, 10, 13, 2, 8, 3, 3, "bf16"),
    "9x17_C3_F12_d64": hin.Geometry(4, 64, 9, 17, 3, 12, 4, 4, "bf16"),
    "tiny_bf16": hin.Geometry(4, 64, 8, 8, 1, 5, 3, 3, "bf16"),
    "tiny_f32": hin.CONFIGS["tiny"]["geom"],
    "7x20_C1_F6_d128_f32": hin.Geometry(4, 128, 7, 20, 1, 6, 5, 2, "f32"),
}


@pytest.mark.parametrize("gname", list(GEOMS))
@pytest.mark.parametrize("labels", [(S_, D_, P_, G_), (G_, G_, G_, G_), (P_, P_, S_, D_)])
def test_routed_matches_oracle(gname, labels):
    g = GEOMS[gname]
    inp = hin.generate(g, labels, seed=zlib.crc32(gname.encode()) % 1000)
    got, _, _ = run_routed(inp)
    want = orc.routed_attention(inp)
    print(gname, labels, assert_close(got, want, *TOL[g.dtype], what=f"{gname} {labels}"))


@pytest.mark.parametrize("n_hist", [0, 2, 4])
def test_routed_partial_window(n_hist):
    g = hin.Geometry(4, 128, 6, 11, 2, 10, 3, 3, "bf16")
    inp = hin.generate(g, (S_, D_, P_, G_), seed=3, n_hist_frames=n_hist)
    got, _, _ = run_routed(inp)
    want = orc.routed_attention(inp)
    assert_close(got, want, *TOL["bf16"], what=f"n_hist={n_hist}")


@pytest.mark.parametrize("grid", [(1, 1), (2, 2), (8, 8), (12, 40), (3, 6)])
def test_spatial_grids(grid):
    g = hin.Geometry(2, 128, 9, 14, 2, 8, grid[0], grid[1], "bf16")
    inp = hin.generate(g, (P_, P_), seed=4)
    got, _, _ = run_routed(inp)
    assert_close(got, orc.routed_attention(inp), *TOL["bf16"], what=f"grid={grid}")
    if grid[0] >= g.frame_h and grid[1] >= g.frame_w:     # full-frame window == Global
        got_g, _, _ = run_routed(inp, labels=(G_, G_))
        assert_close(got, got_g, 2e-3, 2e-4, what="spatial==global")


@pytest.mark.parametrize("frame", [(3, 40), (40, 3), (2, 2), (1, 50), (7, 7), (5, 6)])
@pytest.mark.parametrize("variant", [0, 2, 4])
def test_spatial_tiles_on_odd_frames(frame, variant):
    """Frames narrower or shorter than any 24..32-position tile, or smaller than 24
    positions (the 4 x 8 fallback tile): the tiles in the dense launch (variant 0), in
    their own launch with several frame parts (variant 4), and for the cell variant,
    cells cut at the frame edge."""
    fh, fw = frame
    g = hin.Geometry(4, 128, fh, fw, 3, 12, 3, 4, "bf16")
    inp = hin.generate(g, (P_, G_, P_, S_), seed=fh * 100 + fw + variant)
    t = to_device(inp)
    buf = hc.hc_build_head_buffers(hc.make_desc(g, variant), inp.labels, t["k_hist"], t["v_hist"],
                                   inp.n_hist_frames)
    tile_r, tile_c, parts, _, fused = hc.hc_debug_spatial_plan(buf)
    assert tile_r * tile_c <= 32 and parts >= 1 and fused == (variant == 0)
    got = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
    want = orc.routed_attention(inp, variant=variant & 3)
    print(frame, variant, (tile_r, tile_c, parts),
          assert_close(got, want, *TOL["bf16"], what=f"{frame} v{variant} tile {tile_r}x{tile_c} parts {parts}"))


@pytest.mark.parametrize("variant,d", [(0, 128), (4, 128), (0, 64)])
def test_spatial_unions_past_the_lds_tables(variant, d):
    """16 x 16 windows: a tile's union spans more than the eight 32-key chunks the LDS
    tables hold, so each chunk's tokens and window bits are worked out when it starts
    (tiles in the dense launch, in their own launch, and d = 64)."""
    g = hin.Geometry(3, d, 24, 30, 2, 8, 16, 16, "bf16")
    inp = hin.generate(g, (P_, G_, P_), seed=500 + variant + d)
    t = to_device(inp)
    buf = hc.hc_build_head_buffers(hc.make_desc(g, variant), inp.labels, t["k_hist"], t["v_hist"],
                                   inp.n_hist_frames)
    tr, tc, parts, _, fused = hc.hc_debug_spatial_plan(buf)
    assert fused == (variant == 0 and d == 128)
    assert -(-min(tr + 15, g.frame_h) * min(tc + 15, g.frame_w) // 32) > 8   # an interior tile's union
    got = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
    print(variant, d, (tr, tc, parts),
          assert_close(got, orc.routed_attention(inp), *TOL["bf16"], what=f"v{variant} d{d} tile {tr}x{tc}"))


@pytest.mark.parametrize("geom", [hin.Geometry(2, 128, 8, 8, 1, 40, 3, 3, "bf16"),
                                  hin.Geometry(1, 128, 8, 8, 1, 64, 3, 3, "bf16"),
                                  hin.Geometry(2, 64, 6, 8, 1, 48, 3, 3, "bf16")])
def test_many_key_splits_merge(geom):
    """Few queries against a long window: each Global head's keys are cut into 9 to 16
    pieces (the merge's widest fast path) and joined again."""
    inp = hin.generate(geom, (G_,) * geom.num_heads, seed=600 + geom.window_frames)
    t = to_device(inp)
    buf = hc.hc_build_head_buffers(hc.make_desc(geom), inp.labels, t["k_hist"], t["v_hist"], inp.n_hist_frames)
    ents, _ = hc.hc_debug_routed_plan(buf)
    assert all(9 <= int(e[3]) <= 16 for e in ents), [int(e[3]) for e in ents]
    got = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
    print([int(e[3]) for e in ents], assert_close(got, orc.routed_attention(inp), *TOL["bf16"], what=str(geom)))


def test_random_layers_match_oracle():
    """Seeded random small layers (head count and size, frame, block, window and its
    fill, grid, dtype, path variants and launch option, label mix) against the oracle on
    every query row."""
    rng = np.random.default_rng(77)
    for case in range(16):
        d = int(rng.choice([64, 128]))
        C = int(rng.integers(1, 4))
        g = hin.Geometry(int(rng.integers(1, 9)), d, int(rng.integers(1, 13)), int(rng.integers(1, 21)), C,
                         C * int(rng.integers(1, 6)), int(rng.integers(1, 9)), int(rng.integers(1, 9)),
                         str(rng.choice(["bf16", "bf16", "f32"])))
        variant = int(rng.integers(0, 8))
        labels = rng.integers(0, 4, g.num_heads).astype(np.int32)
        n_hist = C * int(rng.integers(0, g.hist_frames // C + 1))
        inp = hin.generate(g, labels, seed=900 + case, n_hist_frames=n_hist)
        t = to_device(inp)
        buf = hc.hc_build_head_buffers(hc.make_desc(g, variant), inp.labels, t["k_hist"], t["v_hist"], n_hist)
        got = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
        want = orc.routed_attention(inp, variant=variant & 3)
        print(case, g, variant, list(labels), n_hist,
              assert_close(got, want, *TOL[g.dtype], what=f"case {case}: {g} v{variant} {list(labels)} n_hist {n_hist}"))


@pytest.mark.parametrize("n_sp", [16, 17])
def test_spatial_heads_at_the_fused_launch_limit(n_sp):
    """At most 16 Spatial heads run their tiles in the dense launch: 16 with d = 128 are
    fused, 17 take their own launch; both match the oracle."""
    g = hin.Geometry(n_sp + 2, 128, 6, 9, 2, 8, 3, 3, "bf16")
    labels = (P_,) * n_sp + (G_, S_)
    inp = hin.generate(g, labels, seed=300 + n_sp)
    t = to_device(inp)
    buf = hc.hc_build_head_buffers(hc.make_desc(g), inp.labels, t["k_hist"], t["v_hist"], inp.n_hist_frames)
    fused = hc.hc_debug_spatial_plan(buf)[4]
    assert fused == (n_sp <= 16)
    got = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
    print(n_sp, fused, assert_close(got, orc.routed_attention(inp), *TOL["bf16"], what=f"{n_sp} Spatial heads"))


def test_binding_rejects_bad_tensors():
    """Wrong dtype, too few elements or a strided view: refused before the library runs."""
    g = hin.Geometry(4, 64, 8, 8, 1, 5, 3, 3, "bf16")
    inp = hin.generate(g, (S_, D_, P_, G_), seed=9)
    t = to_device(inp)
    buf = hc.hc_build_head_buffers(hc.make_desc(g), inp.labels, t["k_hist"], t["v_hist"], inp.n_hist_frames)
    q = t["q"]
    for bad, status in ((q.float(), 3), (q[: q.shape[0] // 2], 2), (q.transpose(1, 2), 2)):
        with pytest.raises(hc.HCError) as ei:
            hc.hc_routed_attention(buf, bad, t["k_cur"], t["v_cur"])
        assert ei.value.status == status
    with pytest.raises(hc.HCError) as ei:
        hc.hc_append_chunk(buf, t["k_cur"][:1], t["v_cur"])
    assert ei.value.status == 2
    torch.cuda.synchronize()


def test_one_block_window_all_paths_agree():
    g = hin.Geometry(4, 128, 7, 9, 2, 2, 3, 3, "bf16")
    inp = hin.generate(g, (S_, D_, P_, G_), seed=5)
    got, _, _ = run_routed(inp)
    want = orc.routed_attention(inp)
    assert_close(got, want, *TOL["bf16"])
    for h in range(4):     # with no history every class sees exactly the current block
        assert_close(got[:, h], orc.path_attention(inp, h, G_), *TOL["bf16"])


@pytest.mark.parametrize("jumps", [(0, 20, 45, 110), (110, 0, 70, 30), (5, 5, 5, 200)])
def test_rescale_when_scores_jump(jumps):
    """Scores that rise by tens to hundreds of log2 units part-way through the key
    range (a shared direction added to every query and, with growing weight, to the
    keys of later frames): the GPU's reference max must move mid-stream, rescaling O
    and the running sum, and agree with the oracle's exact softmax."""
    g = hin.Geometry(4, 128, 6, 11, 2, 10, 3, 3, "bf16")
    inp = hin.generate(g, (G_, S_, P_, G_), seed=11)
    S, C, d = g.tokens_per_frame, g.chunk_frames, g.head_dim
    rng = np.random.default_rng(12)
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    c = g.softmax_scale * np.log2(np.e)
    inp.q[:] = hin.round_to_bf16(inp.q + u)
    n_hist = inp.n_hist_frames
    # frame groups: history frames split in three, then the current block
    groups = np.array_split(np.arange(n_hist), 3)
    for gi, frames in enumerate(groups):
        for f in frames:
            inp.k_hist[f * S:(f + 1) * S] += (jumps[gi] / c) * u
    inp.k_cur += (jumps[3] / c) * u
    inp.k_hist[:] = hin.round_to_bf16(inp.k_hist)
    inp.k_cur[:] = hin.round_to_bf16(inp.k_cur)
    got, _, _ = run_routed(inp)
    want = orc.routed_attention(inp)
    print(jumps, assert_close(got, want, *TOL["bf16"], what=f"jumps {jumps}"))


def test_zero_query_key_set_moments():
    """q = 0 gives the mean of V over the key set: V columns (1, frame, row, col, row^2,
    col^2) pin every path's membership on the GPU (values exact in bf16)."""
    g = hin.Geometry(4, 128, 6, 11, 2, 10, 3, 3, "bf16")
    inp = hin.generate(g, (S_, D_, P_, G_), seed=6)
    inp.q[:] = 0
    S = g.tokens_per_frame
    n = (inp.n_hist_frames + g.chunk_frames) * S
    t = np.arange(n)
    f, r, c = t // S, (t % S) // g.frame_w, t % g.frame_w
    cols = np.stack([np.ones(n), f, r, c, r * r, c * c], axis=1).astype(np.float32)
    v = np.zeros((n, g.num_heads, g.head_dim), np.float32)
    v[:, :, :6] = cols[:, None, :]
    inp.v_hist[:] = v[: inp.n_hist_frames * S]
    inp.v_cur[:] = v[inp.n_hist_frames * S:]
    got, _, _ = run_routed(inp)
    want = orc.routed_attention(inp)
    rel = np.abs(got[:, :, :6] - want[:, :, :6]) / np.maximum(np.abs(want[:, :, :6]), 1.0)
    assert rel.max() < 8e-3, rel.max()


def test_gather_origins_bit_exact():
    for fh, fw, gh, gw in [(30, 52, 8, 8), (45, 80, 8, 8), (68, 120, 8, 8), (8, 8, 3, 3), (5, 7, 9, 2), (9, 9, 4, 5)]:
        d = hc.make_desc(hin.Geometry(1, 64, fh, fw, 1, 2, gh, gw, "bf16"))
        got = hc.hc_debug_gather_origins(d, gh, gw).cpu().numpy()
        pos = np.arange(fh * fw)
        want = np.stack([orc.window_origin(pos // fw, gh, fh), orc.window_origin(pos % fw, gw, fw)], axis=1)
        assert np.array_equal(got, want), (fh, fw, gh, gw)


def buffer_rows(buf, head, which):
    """Rows of head's K or V buffer region as float64 [rows][d]."""
    k_off, v_off, rows = hc.hc_debug_head_region(buf, head)
    if rows == 0:
        return np.zeros((0, buf.desc.head_dim))
    off = k_off if which == "k" else v_off
    es = 2 if buf.desc.dtype == hc.HC_BF16 else 4
    raw = buf.memory[off: off + rows * buf.desc.head_dim * es]
    t = raw.view(torch.bfloat16 if es == 2 else torch.float32).reshape(rows, buf.desc.head_dim)
    return host(t)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_build_and_append_bit_exact(dtype):
    g = hin.Geometry(4, 64, 3, 5, 2, 10, 2, 2, dtype)     # R = 3 rolling blocks
    labels = (S_, D_, P_, G_)
    C, S = g.chunk_frames, g.tokens_per_frame
    rng = np.random.default_rng(7)
    n_blocks = 10
    chunks = [hin.round_to_bf16(rng.standard_normal((2, C * S, 4, 64), dtype=np.float32)) for _ in range(n_blocks)]
    n0 = 2                                                  # build from blocks 0, 1
    k_hist = np.concatenate([chunks[b][0] for b in range(n0)])
    v_hist = np.concatenate([chunks[b][1] for b in range(n0)])
    buf = hc.hc_build_head_buffers(hc.make_desc(g), labels, dev(k_hist, dtype), dev(v_hist, dtype), n0 * C)
    for nb in range(n0, n_blocks + 1):
        torch.cuda.synchronize()
        table = orc.slot_table(labels, g.window_frames, C, nb)
        assert np.array_equal(hc.hc_debug_slot_table(buf), table)
        for h in range(4):
            for which, idx in (("k", 0), ("v", 1)):
                rows = buffer_rows(buf, h, which)
                for pos in range(rows.shape[0] // S):
                    fr = table[h, pos]
                    if fr < 0:
                        continue
                    b, i = divmod(int(fr), C)
                    want = chunks[b][idx][i * S:(i + 1) * S, h, :]
                    assert np.array_equal(rows[pos * S:(pos + 1) * S], want), (nb, h, pos)
        if nb < n_blocks:
            hc.hc_append_chunk(buf, dev(chunks[nb][0], dtype), dev(chunks[nb][1], dtype))
    assert hc.hc_buffers_state(buf) == n_blocks


@pytest.mark.parametrize("variant", [0, 1])
def test_rebuild_mid_rollout_at_block_10(variant):
    """A rollout resumed at block 10: buffers rebuilt from the window's history in
    logical order (hc_build_head_buffers_at) equal, slot by slot and bit for bit, those of
    a handle that stored all ten blocks in turn; both then take the same appends and
    give bitwise-equal routed outputs, which match the oracle on the logical window."""
    g = hin.Geometry(4, 64, 3, 5, 2, 10, 2, 2, "bf16")     # R = 3 rolling blocks
    labels = (S_, D_, P_, G_)
    C, S, H, d = g.chunk_frames, g.tokens_per_frame, g.num_heads, g.head_dim
    rng = np.random.default_rng(10)
    blocks = [hin.round_to_bf16(rng.standard_normal((3, C * S, H, d), dtype=np.float32)) for _ in range(13)]
    desc = hc.make_desc(g, variant)
    a = hc.hc_build_head_buffers(desc, labels, None, None, 0)
    for b in range(10):
        hc.hc_append_chunk(a, dev(blocks[b][1], "bf16"), dev(blocks[b][2], "bf16"))
    hist = orc.window_history_blocks(10, g.window_frames, C)
    kh = np.concatenate([blocks[b][1] for b in hist])
    vh = np.concatenate([blocks[b][2] for b in hist])
    r = hc.hc_build_head_buffers_at(desc, labels, dev(kh, "bf16"), dev(vh, "bf16"), len(hist) * C, 10)
    ws_a, ws_r = hc.routed_workspace(a), hc.routed_workspace(r)
    for step in range(10, 13):
        torch.cuda.synchronize()
        table = orc.slot_table(labels, g.window_frames, C, step, variant=variant)
        assert np.array_equal(hc.hc_debug_slot_table(r), table)
        assert np.array_equal(hc.hc_debug_slot_table(a), table)
        assert hc.hc_buffers_state(r) == step
        for h in range(H):
            for which in ("k", "v"):
                assert np.array_equal(buffer_rows(r, h, which), buffer_rows(a, h, which)), (step, h, which)
        q, k, v = (dev(x, "bf16") for x in blocks[step])
        out_a = host(hc.hc_routed_attention(a, q, k, v, workspace=ws_a))
        out_r = host(hc.hc_routed_attention(r, q, k, v, workspace=ws_r))
        assert np.array_equal(out_a, out_r)
        hist = orc.window_history_blocks(step, g.window_frames, C)
        inp = hin.LayerInputs(g, np.array(labels, np.int32), blocks[step][0],
                              np.concatenate([blocks[b][1] for b in hist]),
                              np.concatenate([blocks[b][2] for b in hist]), blocks[step][1], blocks[step][2],
                              len(hist) * C)
        assert_close(out_r, orc.routed_attention(inp, variant=variant), *TOL["bf16"], what=f"step {step}")
        hc.hc_append_chunk(a, k, v)
        hc.hc_append_chunk(r, k, v)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rollout_routed_matches_oracle_window(dtype):
    """Warm-up from an empty cache, then one block per step: after every append the
    routed output equals the oracle on the logical window (sink block + recent blocks)."""
    g = hin.Geometry(4, 128 if dtype == "bf16" else 64, 5, 9, 2, 8, 3, 3, dtype)
    labels = (S_, D_, P_, G_)
    C, S, H, d = g.chunk_frames, g.tokens_per_frame, g.num_heads, g.head_dim
    rng = np.random.default_rng(8)
    blocks = [hin.round_to_bf16(rng.standard_normal((3, C * S, H, d), dtype=np.float32)) for _ in range(7)]
    buf = hc.hc_build_head_buffers(hc.make_desc(g), labels, None, None, 0)
    ws = hc.routed_workspace(buf)
    for step in range(7):
        q, k, v = blocks[step]
        out = host(hc.hc_routed_attention(buf, dev(q, dtype), dev(k, dtype), dev(v, dtype), workspace=ws))
        hist = orc.window_history_blocks(step, g.window_frames, C)
        kh = np.concatenate([blocks[b][1] for b in hist]) if hist else np.zeros((0, H, d), np.float32)
        vh = np.concatenate([blocks[b][2] for b in hist]) if hist else np.zeros((0, H, d), np.float32)
        inp = hin.LayerInputs(g, np.array(labels, np.int32), q, kh, vh, k, v, len(hist) * C)
        assert_close(out, orc.routed_attention(inp), *TOL[dtype], what=f"step {step}")
        hc.hc_append_chunk(buf, dev(k, dtype), dev(v, dtype))


def test_random_rollouts_match_oracle():
    """Seeded random layers driven from an empty cache through the ring rolling over
    (head count and size, frame, block, window, grid, dtype, Dummy variant, launch
    option, label mix): after every append, the slot table equals the oracle's and the
    routed output equals the oracle on the logical window."""
    rng = np.random.default_rng(404)
    for case in range(6):
        d = int(rng.choice([64, 128]))
        C = int(rng.integers(1, 4))
        g = hin.Geometry(int(rng.integers(1, 7)), d, int(rng.integers(2, 9)), int(rng.integers(2, 13)), C,
                         C * int(rng.integers(2, 6)), int(rng.integers(1, 6)), int(rng.integers(1, 6)),
                         str(rng.choice(["bf16", "f32"])))
        variant = int(rng.choice([0, 1, 4, 5]))
        labels = rng.integers(0, 4, g.num_heads).astype(np.int32)
        S, H = g.tokens_per_frame, g.num_heads
        n_steps = g.window_frames // C + 3
        blocks = [hin.round_to_bf16(rng.standard_normal((3, C * S, H, d), dtype=np.float32)) if g.dtype == "bf16"
                  else rng.standard_normal((3, C * S, H, d), dtype=np.float32) for _ in range(n_steps)]
        buf = hc.hc_build_head_buffers(hc.make_desc(g, variant), labels, None, None, 0)
        ws = hc.routed_workspace(buf)
        for step in range(n_steps):
            q, k, v = blocks[step]
            table = orc.slot_table(labels, g.window_frames, C, step,
                                   variant=orc.DUMMY_PREVIOUS_BLOCK if variant & 1 else 0)
            assert np.array_equal(hc.hc_debug_slot_table(buf), table), (case, step)
            out = host(hc.hc_routed_attention(buf, dev(q, g.dtype), dev(k, g.dtype), dev(v, g.dtype), workspace=ws))
            hist = orc.window_history_blocks(step, g.window_frames, C)
            kh = np.concatenate([blocks[b][1] for b in hist]) if hist else np.zeros((0, H, d), np.float32)
            vh = np.concatenate([blocks[b][2] for b in hist]) if hist else np.zeros((0, H, d), np.float32)
            inp = hin.LayerInputs(g, labels, q, kh, vh, k, v, len(hist) * C)
            assert_close(out, orc.routed_attention(inp, variant=variant & 3), *TOL[g.dtype],
                         what=f"case {case} {g} v{variant} {list(labels)} step {step}")
            hc.hc_append_chunk(buf, dev(k, g.dtype), dev(v, g.dtype))
        print(case, g, variant, list(labels), n_steps)


@pytest.mark.parametrize("name", ["480p", "720p", "1080p"])
def test_full_size_sampled_rows(name):
    """The benchmark's workloads at full size; sampled query rows against the oracle, the
    routed call in both launch forms of the Spatial path (in the dense launch, its own
    launch), plus the all-Global call of the same kernel."""
    inp = hin.config_inputs(name)
    g = inp.geom
    t = to_device(inp)
    rows = sample_rows(g, n_random=512, seed=1)
    for labels, variants in ((inp.labels, (0, 4)), (np.full(g.num_heads, G_, np.int32), (0,))):
        want = orc.routed_attention(inp, labels=labels, rows=rows)
        for v in variants:
            buf = hc.hc_build_head_buffers(hc.make_desc(g, v), labels, t["k_hist"], t["v_hist"], inp.n_hist_frames)
            out = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
            print(name, labels, v, hc.hc_debug_spatial_plan(buf),
                  assert_close(out[rows], want, *TOL["bf16"], what=f"{name} v{v}"))
            assert np.isfinite(out).all()
            del buf


def test_deterministic_bitwise():
    inp = hin.config_inputs("480p")
    a, _, _ = run_routed(inp)
    b, _, _ = run_routed(inp)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------- classification
def classify_gpu(inp, **params):
    g = inp.geom
    t = to_device(inp)
    p = hc.hc_default_classify_params(**params)
    return hc.hc_classify_heads(hc.make_desc(g), p, t["q"], t["k_hist"], t["v_hist"], inp.n_hist_frames,
                                t["k_cur"], t["v_cur"])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_classify_planted_matches_oracle(dtype, d):
    g = hin.Geometry(8, d, 12, 20, 3, 21, 8, 8, dtype)
    labels = [S_, D_, P_, G_, G_, P_, D_, S_]
    inp = hin.generate(g, labels, seed=5, planted=True)
    got, stats = classify_gpu(inp, gamma=0.5)
    want, ost = orc.classify_heads(inp, dict(gamma=0.5))
    assert list(want) == labels
    assert list(got) == labels
    for h in range(8):
        o = ost[h]
        ref = [o["cos_sink"], o["cos_dummy"], o["cos_spatial"], o["p5"], o["mse"], o["score"]]
        assert np.allclose(stats[h], ref, atol=2e-3), (h, stats[h], ref)


def test_max_heads_routed_and_classifier_batches():
    """The largest head count the ABI takes (64, every class, one dense entry per head)
    and a classification whose per-head slot entries (12 heads x 8 slots) need more
    than one dense launch."""
    g = hin.Geometry(64, 64, 4, 6, 1, 4, 3, 3, "bf16")
    labels = [S_, D_, P_, G_] * 16
    inp = hin.generate(g, labels, seed=21)
    got, _, _ = run_routed(inp)
    assert_close(got, orc.routed_attention(inp), *TOL["bf16"], what="64 heads")
    g = hin.Geometry(12, 128, 10, 12, 3, 21, 8, 8, "bf16")
    labels = [S_, D_, P_, G_, G_, P_, D_, S_, P_, P_, G_, D_]
    inp = hin.generate(g, labels, seed=22, planted=True)
    got, stats = classify_gpu(inp, gamma=0.5)
    want, ost = orc.classify_heads(inp, dict(gamma=0.5))
    assert list(want) == labels and list(got) == labels
    for h in range(12):
        o = ost[h]
        ref = [o["cos_sink"], o["cos_dummy"], o["cos_spatial"], o["p5"], o["mse"], o["score"]]
        assert np.allclose(stats[h], ref, atol=2e-3), (h, stats[h], ref)


@pytest.mark.parametrize("geom", [hin.Geometry(4, 128, 10, 10, 1, 8, 3, 3, "bf16"),
                                  hin.Geometry(4, 64, 5, 13, 1, 7, 3, 3, "bf16")])
def test_classify_middle_blocks_not_a_tile_multiple(geom):
    """C*S = 100 and 65 keys per block (not multiples of the 64-key tile) with 6 and 5
    middle history frames: the reference must cover every middle key."""
    inp = hin.generate(geom, [S_, D_, P_, G_], seed=23, planted=True)
    got, stats = classify_gpu(inp, gamma=0.5)
    want, ost = orc.classify_heads(inp, dict(gamma=0.5))
    assert list(got) == list(want)
    for h in range(4):
        o = ost[h]
        ref = [o["cos_sink"], o["cos_dummy"], o["cos_spatial"], o["p5"], o["mse"], o["score"]]
        assert np.allclose(stats[h], ref, atol=3e-3), (h, stats[h], ref)


def test_classify_unplanted_statistics_match_oracle():
    g = hin.Geometry(4, 128, 9, 14, 2, 8, 3, 3, "bf16")
    inp = hin.generate(g, [G_] * 4, seed=9)
    got, stats = classify_gpu(inp)
    want, ost = orc.classify_heads(inp)
    assert list(got) == list(want)
    for h in range(4):
        o = ost[h]
        ref = [o["cos_sink"], o["cos_dummy"], o["cos_spatial"], o["p5"], o["mse"], o["score"]]
        assert np.allclose(stats[h], ref, atol=3e-3), (h, stats[h], ref)


def test_classify_random_layers_match_oracle():
    """Seeded random small layers, planted and not (head count and size, frame, block,
    window and its fill, grid, dtype, gamma, proxy grid): the six statistics of every head
    within 3e-3 of the oracle's, and the labels equal wherever every statistic is at
    least 0.01 from its threshold (nearer, fp32 cosines and fp64 ones may fall on either
    side)."""
    rng = np.random.default_rng(55)
    th = dict(orc.DEFAULT_PARAMS)
    for case in range(12):
        d = int(rng.choice([64, 128]))
        C = int(rng.integers(1, 4))
        g = hin.Geometry(int(rng.integers(1, 9)), d, int(rng.integers(2, 13)), int(rng.integers(2, 21)), C,
                         C * int(rng.integers(2, 7)), int(rng.integers(1, 9)), int(rng.integers(1, 9)),
                         str(rng.choice(["bf16", "bf16", "f32"])))
        labels = rng.integers(0, 4, g.num_heads).astype(np.int32)
        n_hist = C * int(rng.integers(1, g.hist_frames // C + 1))
        inp = hin.generate(g, labels, seed=1100 + case, n_hist_frames=n_hist, planted=bool(case % 2))
        params = dict(gamma=float(rng.choice([0.5, 5.0])))
        gpu_params = dict(params)
        if rng.integers(0, 2):
            params["proxy_grid"] = (int(rng.integers(1, 9)), int(rng.integers(1, 9)))
            gpu_params.update(proxy_grid_h=params["proxy_grid"][0], proxy_grid_w=params["proxy_grid"][1])
        got, stats = classify_gpu(inp, **gpu_params)
        want, ost = orc.classify_heads(inp, params)
        what = (case, g, list(labels), n_hist, params)
        for h in range(g.num_heads):
            o = ost[h]
            ref = [o["cos_sink"], o["cos_dummy"], o["cos_spatial"], o["p5"], o["mse"], o["score"]]
            assert np.allclose(stats[h], ref, atol=3e-3), (what, h, stats[h], ref)
            margins = [abs(o["cos_sink"] - th["theta_sink"]), abs(o["cos_dummy"] - th["theta_dummy"]),
                       abs(o["cos_spatial"] - th["theta_spatial"]), abs(o["score"] - th["theta_score"])]
            if min(margins) >= 0.01:
                assert got[h] == want[h], (what, h, got[h], want[h], ref)
        print(case, g, n_hist, params, list(want), list(got))


@pytest.mark.parametrize("proxy", [(5, 5), (2, 7), (1, 1)])
def test_classify_proxy_grid_statistics_match_oracle(proxy):
    """A Spatial proxy window other than the routing grid (the pages' radius-2, 5 x 5
    proxy for the deployed cells; non-square; a single key per frame)."""
    g = hin.Geometry(4, 128, 9, 14, 2, 8, 3, 3, "bf16")
    inp = hin.generate(g, [G_, P_, G_, P_], seed=10 + proxy[0], planted=True)
    got, stats = classify_gpu(inp, gamma=0.5, proxy_grid_h=proxy[0], proxy_grid_w=proxy[1])
    want, ost = orc.classify_heads(inp, dict(gamma=0.5, proxy_grid=proxy))
    for h in range(4):
        o = ost[h]
        ref = [o["cos_sink"], o["cos_dummy"], o["cos_spatial"], o["p5"], o["mse"], o["score"]]
        assert np.allclose(stats[h], ref, atol=3e-3), (proxy, h, stats[h], ref)
    assert list(got) == list(want)


def test_classify_sink_proxy_variant():
    g = hin.Geometry(2, 128, 12, 20, 3, 21, 8, 8, "bf16")
    inp = hin.generate(g, [D_, G_], seed=6, planted=True)
    got, _ = classify_gpu(inp, gamma=0.5, sink_proxy_includes_current=1)
    want, _ = orc.classify_heads(inp, dict(gamma=0.5, sink_proxy_includes_current=True))
    assert list(got) == list(want) == [S_, G_]


# ----------------------------------------------------------------------------- path variants
VARIANT_GEOMS = {
    "10x13_C2_F8_d128_cells3": hin.Geometry(4, 128, 10, 13, 2, 8, 3, 3, "bf16"),
    "9x17_C3_F12_d64_cells4x5": hin.Geometry(4, 64, 9, 17, 3, 12, 4, 5, "bf16"),
    "12x20_C3_F9_d128_cells10": hin.Geometry(4, 128, 12, 20, 3, 9, 10, 10, "bf16"),
    "tiny_f32_cells3": hin.CONFIGS["tiny"]["geom"],
}


@pytest.mark.parametrize("gname", list(VARIANT_GEOMS))
@pytest.mark.parametrize("variant", [1, 2, 3])
def test_variants_match_oracle(gname, variant):
    g = VARIANT_GEOMS[gname]
    inp = hin.generate(g, (S_, D_, P_, G_), seed=zlib.crc32(gname.encode()) % 1000 + variant)
    t = to_device(inp)
    buf = hc.hc_build_head_buffers(hc.make_desc(g, variant), inp.labels, t["k_hist"], t["v_hist"],
                                   inp.n_hist_frames)
    got = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
    want = orc.routed_attention(inp, variant=variant)
    print(gname, variant, assert_close(got, want, *TOL[g.dtype], what=f"{gname} v{variant}"))


def test_variant_cell_origins_bit_exact():
    for fh, fw, ch, cw in [(45, 80, 10, 10), (68, 120, 10, 10), (30, 52, 10, 10), (9, 17, 4, 5), (7, 7, 9, 9)]:
        d = hc.make_desc(hin.Geometry(1, 64, fh, fw, 1, 2, ch, cw, "bf16"), hc.HC_VARIANT_SPATIAL_CELLS)
        got = hc.hc_debug_gather_origins(d, ch, cw).cpu().numpy()
        pos = np.arange(fh * fw)
        want = np.stack([orc.cell_origin(pos // fw, ch), orc.cell_origin(pos % fw, cw)], axis=1)
        assert np.array_equal(got, want), (fh, fw, ch, cw)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_variant_rollout_dummy_buffer(dtype):
    """Warm-up with appends under both variants: the Dummy buffer always holds the
    window's latest history block, bit-exact, and outputs follow the oracle."""
    variant = 3
    g = hin.Geometry(4, 64, 5, 9, 2, 8, 3, 3, dtype)
    labels = (S_, D_, P_, G_)
    C, S, H, d = g.chunk_frames, g.tokens_per_frame, g.num_heads, g.head_dim
    rng = np.random.default_rng(9)
    blocks = [hin.round_to_bf16(rng.standard_normal((3, C * S, H, d), dtype=np.float32)) for _ in range(7)]
    buf = hc.hc_build_head_buffers(hc.make_desc(g, variant), labels, None, None, 0)
    ws = hc.routed_workspace(buf)
    for step in range(7):
        q, k, v = blocks[step]
        out = host(hc.hc_routed_attention(buf, dev(q, dtype), dev(k, dtype), dev(v, dtype), workspace=ws))
        hist = orc.window_history_blocks(step, g.window_frames, C)
        kh = np.concatenate([blocks[b][1] for b in hist]) if hist else np.zeros((0, H, d), np.float32)
        vh = np.concatenate([blocks[b][2] for b in hist]) if hist else np.zeros((0, H, d), np.float32)
        inp = hin.LayerInputs(g, np.array(labels, np.int32), q, kh, vh, k, v, len(hist) * C)
        assert_close(out, orc.routed_attention(inp, variant=variant), *TOL[dtype], what=f"step {step}")
        table = orc.slot_table(labels, g.window_frames, C, step, variant=orc.DUMMY_PREVIOUS_BLOCK)
        assert np.array_equal(hc.hc_debug_slot_table(buf), table)
        if table[1, 0] >= 0:   # (before the first append the region holds no block yet)
            b = int(table[1, 0]) // C
            assert np.array_equal(buffer_rows(buf, 1, "k"), blocks[b][1][:, 1, :].astype(np.float64))
        hc.hc_append_chunk(buf, dev(k, dtype), dev(v, dtype))


@pytest.mark.parametrize("name", ["720p", "1080p"])
def test_variant_full_size_sampled_rows(name):
    """The pages' deployed paths at the benchmark's 720P and 1080P sizes: 10 x 10 cells
    for the Spatial heads and the previous block for the Dummy heads."""
    inp = hin.config_inputs(name)
    g = dataclasses.replace(inp.geom, grid_h=10, grid_w=10)
    inp = dataclasses.replace(inp, geom=g)
    t = to_device(inp)
    buf = hc.hc_build_head_buffers(hc.make_desc(g, 3), inp.labels, t["k_hist"], t["v_hist"], inp.n_hist_frames)
    out = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
    rows = sample_rows(g, n_random=96, seed=2)
    want = orc.routed_attention(inp, rows=rows, variant=3)
    print(assert_close(out[rows], want, *TOL["bf16"], what=f"{name} deployed variants"))
