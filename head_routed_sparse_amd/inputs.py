"""Seeded synthetic inputs for head-routed attention.

This module only draws numbers and shapes them; it holds none of the attention or
classification arithmetic. Both the HIP path's tests/benchmark and the CPU oracle's
tests take their inputs from here.

The pages measure on generated videos from trained models (HeadCast, Sec. 5.1
"Experimental Setup"); neither weights nor prompts are available, so Q/K/V are
synthetic stand-ins with the pages' attention shapes: 30x52-token latent frames at
480P (Fig. 1(c) / Fig. 7 axes), 3-frame blocks, and a 7-block window (1 sink block +
rolling blocks + the current block) (Sec. 5.1 "Implementation Details").

Token order is frame-major, then row-major inside a frame:
token = frame * S + row * frame_w + col, with S = frame_h * frame_w.
Every tensor is laid out [tokens][heads][head_dim].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SINK, DUMMY, SPATIAL, GLOBAL = 0, 1, 2, 3
CLASS_NAMES = ("sink", "dummy", "spatial", "global")


@dataclasses.dataclass(frozen=True)
class Geometry:
    num_heads: int
    head_dim: int
    frame_h: int
    frame_w: int
    chunk_frames: int     # C: frames per AR block (the current block)
    window_frames: int    # F: whole window incl. the sink block and the current block
    grid_h: int           # Spatial path window height (g)
    grid_w: int           # Spatial path window width (g)
    dtype: str = "bf16"   # "bf16" or "f32"

    @property
    def tokens_per_frame(self) -> int:
        return self.frame_h * self.frame_w

    @property
    def hist_frames(self) -> int:
        return self.window_frames - self.chunk_frames

    @property
    def lq(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


def _mix(counts):
    out = []
    for cls, n in enumerate(counts):
        out += [cls] * n
    return np.array(out, dtype=np.int32)


# The five workloads: a tiny CPU-checkable step, three single layers shaped like
# 480P / 720P / 1080P latents, and a 30-layer 720P step with planted head behaviour.
CONFIGS = {
    "tiny": dict(geom=Geometry(4, 64, 8, 8, 1, 5, 3, 3, "f32"),
                 labels=_mix((1, 1, 1, 1)), seed=0, layers=1, planted=False),
    "480p": dict(geom=Geometry(12, 128, 30, 52, 3, 21, 8, 8, "bf16"),
                 labels=_mix((3, 3, 3, 3)), seed=480, layers=1, planted=False),
    "720p": dict(geom=Geometry(12, 128, 45, 80, 3, 21, 8, 8, "bf16"),
                 labels=_mix((2, 3, 4, 3)), seed=720, layers=1, planted=False),
    "1080p": dict(geom=Geometry(12, 128, 68, 120, 3, 21, 8, 8, "bf16"),
                  labels=_mix((2, 3, 4, 3)), seed=1080, layers=1, planted=False),
    "full720p": dict(geom=Geometry(12, 128, 45, 80, 3, 21, 8, 8, "bf16"),
                     labels=None, seed=2607, layers=30, planted=True,
                     class_counts=(54, 90, 126, 90)),
}

# Planted logit boosts s = |u|^2 / sqrt(d): 12 for the shared Sink/Dummy vector,
# 16 for the per-position Spatial vector.
PLANT_BOOST_BLOCK = 12.0
PLANT_BOOST_SPATIAL = 16.0


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _random_direction(rng: np.random.Generator, n: int, d: int, norm: float) -> np.ndarray:
    v = rng.standard_normal((n, d), dtype=np.float32)
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    return (v * np.float32(norm)).astype(np.float32)


@dataclasses.dataclass
class LayerInputs:
    geom: Geometry
    labels: np.ndarray            # int32 [H]
    q: np.ndarray                 # float32 [C*S][H][d]
    k_hist: np.ndarray            # float32 [n_hist*S][H][d], logical frame order
    v_hist: np.ndarray
    k_cur: np.ndarray             # float32 [C*S][H][d]
    v_cur: np.ndarray
    n_hist_frames: int


def plant(geom: Geometry, labels, q, k_hist, k_cur, rng, n_hist_frames):
    """Add the planted per-class structure to Q and K in place.

    Sink head: one vector u is added to every query and to every key of the first
    block. Dummy head: u is added to every query and every current-block key.
    Spatial head: an independent vector b(r, c) per position is added to the queries
    and to the keys of every window frame at that position. Global heads are untouched.
    """
    S, C, d = geom.tokens_per_frame, geom.chunk_frames, geom.head_dim
    n_block = np.sqrt(PLANT_BOOST_BLOCK * np.sqrt(d))
    n_spat = np.sqrt(PLANT_BOOST_SPATIAL * np.sqrt(d))
    for h in range(geom.num_heads):
        cls = int(labels[h])
        if cls == SINK:
            u = _random_direction(rng, 1, d, n_block)[0]
            q[:, h, :] += u
            k_hist[: C * S, h, :] += u
        elif cls == DUMMY:
            u = _random_direction(rng, 1, d, n_block)[0]
            q[:, h, :] += u
            k_cur[:, h, :] += u
        elif cls == SPATIAL:
            b = _random_direction(rng, S, d, n_spat)          # [S][d]
            q[:, h, :] += np.tile(b, (C, 1))
            k_hist[:, h, :] += np.tile(b, (n_hist_frames, 1))
            k_cur[:, h, :] += np.tile(b, (C, 1))


def generate(geom: Geometry, labels, seed: int, n_hist_frames: Optional[int] = None,
             planted: bool = False, rng: Optional[np.random.Generator] = None) -> LayerInputs:
    """Q, K_hist, V_hist, K_cur, V_cur ~ N(0, 1), drawn in that order from PCG64(seed).

    With planted=True the per-class structure of `plant` is added afterwards (its
    vectors drawn from the same generator, after the tensors). bf16 geometries are
    rounded to bfloat16 (RNE) last; the arrays stay float32 holding bf16 values.
    """
    if n_hist_frames is None:
        n_hist_frames = geom.hist_frames
    S, C, H, d = geom.tokens_per_frame, geom.chunk_frames, geom.num_heads, geom.head_dim
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((C * S, H, d), dtype=np.float32)
    k_hist = rng.standard_normal((n_hist_frames * S, H, d), dtype=np.float32)
    v_hist = rng.standard_normal((n_hist_frames * S, H, d), dtype=np.float32)
    k_cur = rng.standard_normal((C * S, H, d), dtype=np.float32)
    v_cur = rng.standard_normal((C * S, H, d), dtype=np.float32)
    labels = np.asarray(labels, dtype=np.int32)
    if planted:
        plant(geom, labels, q, k_hist, k_cur, rng, n_hist_frames)
    if geom.dtype == "bf16":
        q, k_hist, v_hist, k_cur, v_cur = (round_to_bf16(a) for a in (q, k_hist, v_hist, k_cur, v_cur))
    return LayerInputs(geom, labels, q, k_hist, v_hist, k_cur, v_cur, n_hist_frames)


def config_inputs(name: str, n_hist_frames: Optional[int] = None) -> LayerInputs:
    """Inputs of a single-layer configuration by name ("tiny", "480p", "720p", "1080p")."""
    cfg = CONFIGS[name]
    return generate(cfg["geom"], cfg["labels"], cfg["seed"], n_hist_frames, cfg["planted"])


def full_step_labels(name: str = "full720p") -> np.ndarray:
    """Planted labels [layers][H] of a multi-layer configuration: a seeded permutation
    of exactly the configured class counts over all (layer, head) pairs."""
    cfg = CONFIGS[name]
    geom = cfg["geom"]
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    pool = _mix(cfg["class_counts"])
    assert pool.size == cfg["layers"] * geom.num_heads
    return rng.permutation(pool).reshape(cfg["layers"], geom.num_heads).astype(np.int32)


def full_step_layer_inputs(name: str, layer: int, geom: Optional[Geometry] = None) -> LayerInputs:
    """Planted inputs of one layer of a multi-layer configuration, from PCG64([seed, layer+1])."""
    cfg = CONFIGS[name]
    geom = geom or cfg["geom"]
    labels = full_step_labels(name)[layer]
    rng = np.random.Generator(np.random.PCG64([cfg["seed"], layer + 1]))
    return generate(geom, labels, cfg["seed"], None, True, rng=rng)


def generate_torch(geom: Geometry, labels, seed: int, device="cuda", planted: bool = False,
                   n_hist_frames: Optional[int] = None):
    """The recipe of `generate` drawn with torch's generator on `device` (fast at full
    size; different numbers from the numpy path). Returns a dict of tensors in the
    geometry's dtype plus the labels. Used where the truth is the planted labels."""
    import torch
    if n_hist_frames is None:
        n_hist_frames = geom.hist_frames
    S, C, H, d = geom.tokens_per_frame, geom.chunk_frames, geom.num_heads, geom.head_dim
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    kw = dict(generator=g, device=device, dtype=torch.float32)
    q = torch.randn((C * S, H, d), **kw)
    k_hist = torch.randn((n_hist_frames * S, H, d), **kw)
    v_hist = torch.randn((n_hist_frames * S, H, d), **kw)
    k_cur = torch.randn((C * S, H, d), **kw)
    v_cur = torch.randn((C * S, H, d), **kw)
    labels = np.asarray(labels, dtype=np.int32)
    if planted:
        def direction(n, boost):
            v = torch.randn((n, d), **kw)
            return v / v.norm(dim=1, keepdim=True) * float(np.sqrt(boost * np.sqrt(d)))
        for h in range(H):
            cls = int(labels[h])
            if cls in (SINK, DUMMY):
                u = direction(1, PLANT_BOOST_BLOCK)[0]
                q[:, h] += u
                if cls == SINK:
                    k_hist[: C * S, h] += u
                else:
                    k_cur[:, h] += u
            elif cls == SPATIAL:
                b = direction(S, PLANT_BOOST_SPATIAL)
                q[:, h] += b.repeat(C, 1)
                k_hist[:, h] += b.repeat(n_hist_frames, 1)
                k_cur[:, h] += b.repeat(C, 1)
    dt = torch.bfloat16 if geom.dtype == "bf16" else torch.float32
    out = {k: v.to(dt) for k, v in dict(q=q, k_hist=k_hist, v_hist=v_hist, k_cur=k_cur, v_cur=v_cur).items()}
    out["labels"] = labels
    out["n_hist_frames"] = n_hist_frames
    return out


def full_step_layer_torch(name: str, layer: int, device="cuda"):
    """Planted inputs of one layer of a multi-layer configuration, drawn on the device
    from seed (seed * 1000 + layer + 1); labels from `full_step_labels`."""
    cfg = CONFIGS[name]
    return generate_torch(cfg["geom"], full_step_labels(name)[layer], cfg["seed"] * 1000 + layer + 1,
                          device, planted=True)
