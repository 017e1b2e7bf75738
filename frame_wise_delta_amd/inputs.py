"""Seeded synthetic inputs for the VDA linear branch (shared by the tests,
``bench.py`` and ``__graft_entry__.smoke``).

This module draws numbers and stores them; it holds none of the method's
arithmetic.  Both the float64 oracle and the HIP path receive exactly the
values produced here (the oracle decodes the stored 16-bit / 32-bit values to
float64, the HIP path uploads the stored bytes).

Distributions follow the workload description of the Video DeltaNet summary
page ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
Generation", section 前置知识 / VAE latent frames and chunks: latent tensor
(24, 102, 48, 84), 5-frame VAE chunks; section 方法步骤详情 step (2): L2
normalised Q/K, per-token write gate beta, per-frame channelwise decay
alpha).  Real activations need the model weights, which are not available, so
these draws stand in for them:

* q, k : N(0, 1) rows, L2-normalised per token
* v    : N(0, 1)
* beta : sigmoid(N(0, 1)) per token
* alpha: lo + (1 - lo) * U(0, 1) per frame and channel (lo = 0.9, or 0.97 for
         the long-video configuration)
* text tokens (k_T, v_T, beta_T) follow the same laws as video tokens.
* raw projections for the fused prep (``raw_head_inputs``): the same draws
  with q, k not normalised and beta, alpha stored as logits;
* softmax branch (``softmax_inputs``): q, k, v and text k, v with N(0, 1)
  entries, bf16;
* readout epilogue (``epilogue_inputs``): gate logits N(0, 1) per frame,
  token and channel; RMSNorm weight 1 + 0.1 N(0, 1) per channel.

Every tensor of every head comes from its own generator
``numpy.random.default_rng([seed, tensor_id, head])`` so that any head can be
regenerated on its own.  Values are drawn in float64, cast to float32 and, for
16-bit configurations, rounded to bfloat16 with round-to-nearest-even.  They
are never renormalised after rounding.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids for the per-tensor generators
_Q, _K, _V, _BETA, _ALPHA, _KT, _VT, _BT, _GATE, _NORMW, _SQ, _SK, _SV, _SKT, _SVT = range(15)


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload.  ``frames`` counts every latent frame (anchors
    included); ``window`` is the number of chunks on each side of a query
    chunk that the softmax branch covers (-1: no exclusion, the readout uses
    the full forward state of each frame)."""

    name: str
    heads: int
    d: int
    frames: int
    tokens: int
    chunk: int
    anchors: int
    window: int
    text_tokens: int
    in_dtype: str          # "f32" or "bf16"
    out_dtype: str         # "f32", "bf16" or "f16"
    alpha_lo: float
    seed: int

    @property
    def scanned(self) -> int:
        return self.frames - 2 * self.anchors

    @property
    def n_chunks(self) -> int:
        return -(-self.scanned // self.chunk)


CONFIGS = [
    # tiny: 1 head, d=16, 22 frames (0 and 21 anchors, 4 chunks of 5), U=16, fp32
    Config("tiny", 1, 16, 22, 16, 5, 1, 1, 8, "f32", "f32", 0.9, 1000),
    # scan-only stress: 8 heads, d=64, 32 frames, U=256, full forward readout,
    # zero initial state
    Config("scan_only", 8, 64, 32, 256, 5, 0, -1, 0, "bf16", "bf16", 0.9, 1001),
    # H3-shaped single layer: latent (24,102,48,84) patchified 2x2 -> U=1008
    Config("h3", 24, 128, 102, 1008, 5, 1, 1, 512, "bf16", "bf16", 0.9, 1002),
    # long video: 202 frames, alpha in [0.97, 1)
    Config("long", 24, 128, 202, 1008, 5, 1, 1, 512, "bf16", "bf16", 0.97, 1003),
    # high-res long: U=2016, 402 frames
    Config("hires", 24, 128, 402, 2016, 5, 1, 1, 512, "bf16", "bf16", 0.9, 1004),
]

CONFIG_BY_NAME = {c.name: c for c in CONFIGS}


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (for small test cases)."""
    return dataclasses.replace(cfg, **kw)


# ---------------------------------------------------------------- storage --

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + (((b >> 16) & 1) + 0x7FFF)
    return (b >> 16).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float64 draws to the storage format: float32 array or bf16 bits."""
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored data (what both sides compute on)."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    raise ValueError(dtype)


# ------------------------------------------------------------------ draws --

def _rng(cfg: Config, tensor: int, head: int):
    return np.random.default_rng([cfg.seed, tensor, head])


def _unit_rows(g, shape):
    x = g.standard_normal(shape)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


@dataclasses.dataclass
class HeadInputs:
    """Stored inputs of one head.  q, k, v: [T, U, d]; beta: [T, U] float32;
    alpha: [T, d] float32; kt, vt: [N_text, d]; bt: [N_text] float32.
    q/k/v/kt/vt are float32 or bf16 bit patterns (uint16) per ``dtype``."""

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    alpha: np.ndarray
    kt: np.ndarray
    vt: np.ndarray
    bt: np.ndarray

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if name in ("beta", "alpha", "bt"):
            return a.astype(np.float64)
        return to_f64(a, self.dtype)


def head_inputs(cfg: Config, head: int, parts=("q", "k", "v", "beta", "alpha", "text")) -> HeadInputs:
    T, U, d, nt = cfg.frames, cfg.tokens, cfg.d, cfg.text_tokens
    dt = cfg.in_dtype
    empty = np.zeros((0,), np.float32)
    out = dict(dtype=dt, q=empty, k=empty, v=empty, beta=empty, alpha=empty,
               kt=np.zeros((0, d), np.float32), vt=np.zeros((0, d), np.float32),
               bt=np.zeros((0,), np.float32))
    if "q" in parts:
        out["q"] = store(_unit_rows(_rng(cfg, _Q, head), (T, U, d)), dt)
    if "k" in parts:
        out["k"] = store(_unit_rows(_rng(cfg, _K, head), (T, U, d)), dt)
    if "v" in parts:
        out["v"] = store(_rng(cfg, _V, head).standard_normal((T, U, d)), dt)
    if "beta" in parts:
        out["beta"] = _sigmoid(_rng(cfg, _BETA, head).standard_normal((T, U))).astype(np.float32)
    if "alpha" in parts:
        lo = cfg.alpha_lo
        out["alpha"] = (lo + (1.0 - lo) * _rng(cfg, _ALPHA, head).random((T, d))).astype(np.float32)
    if "text" in parts and nt > 0:
        out["kt"] = store(_unit_rows(_rng(cfg, _KT, head), (nt, d)), dt)
        out["vt"] = store(_rng(cfg, _VT, head).standard_normal((nt, d)), dt)
        out["bt"] = _sigmoid(_rng(cfg, _BT, head).standard_normal((nt,))).astype(np.float32)
    return HeadInputs(**out)


@dataclasses.dataclass
class EpilogueInputs:
    """Stored inputs of the readout epilogue of one head: gate logits
    [T, U, d] (float32 or bf16 bits per ``dtype``) and the RMSNorm weight
    [d] float32."""

    dtype: str
    gate: np.ndarray
    weight: np.ndarray

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return a.astype(np.float64) if name == "weight" else to_f64(a, self.dtype)


def epilogue_inputs(cfg: Config, head: int) -> EpilogueInputs:
    """Gate logits N(0, 1) per (frame, token, channel) and RMSNorm weights
    1 + 0.1 N(0, 1) per channel: stand-ins for the gate projection of the
    layer input and a trained norm weight."""
    T, U, d = cfg.frames, cfg.tokens, cfg.d
    gate = store(_rng(cfg, _GATE, head).standard_normal((T, U, d)), cfg.in_dtype)
    weight = (1.0 + 0.1 * _rng(cfg, _NORMW, head).standard_normal(d)).astype(np.float32)
    return EpilogueInputs(dtype=cfg.in_dtype, gate=gate, weight=weight)


@dataclasses.dataclass
class SoftmaxInputs:
    """Inputs of the softmax branch of one head, as bf16 bits: q, k, v
    [T, U, d] and the text keys / values kt, vt [N_text, d]."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    kt: np.ndarray
    vt: np.ndarray

    def f64(self, name: str) -> np.ndarray:
        return to_f64(getattr(self, name), "bf16")


def softmax_inputs(cfg: Config, head: int) -> SoftmaxInputs:
    """q, k, v and the text keys / values of the softmax branch: N(0, 1)
    entries (the scale of projections after a QK RMS normalisation, so that
    q.k / sqrt(d) is about N(0, 1)), stored as bf16."""
    T, U, d, nt = cfg.frames, cfg.tokens, cfg.d, cfg.text_tokens
    n = lambda tid, shape: store(_rng(cfg, tid, head).standard_normal(shape), "bf16")
    return SoftmaxInputs(q=n(_SQ, (T, U, d)), k=n(_SK, (T, U, d)), v=n(_SV, (T, U, d)),
                         kt=n(_SKT, (nt, d)), vt=n(_SVT, (nt, d)))


def raw_head_inputs(cfg: Config, head: int) -> HeadInputs:
    """Raw projections for the fused prep: the same draws as head_inputs
    but q, k and the text keys are not normalised, and beta, alpha and the
    text beta are stored as logits (log(p / (1 - p)) of the usual gates,
    computed in float64 and stored as float32)."""
    T, U, d, nt = cfg.frames, cfg.tokens, cfg.d, cfg.text_tokens
    dt = cfg.in_dtype
    logit = lambda p: np.log(p / (1.0 - p))
    lo = cfg.alpha_lo
    out = dict(
        dtype=dt,
        q=store(_rng(cfg, _Q, head).standard_normal((T, U, d)), dt),
        k=store(_rng(cfg, _K, head).standard_normal((T, U, d)), dt),
        v=store(_rng(cfg, _V, head).standard_normal((T, U, d)), dt),
        beta=_rng(cfg, _BETA, head).standard_normal((T, U)).astype(np.float32),
        alpha=logit(lo + (1.0 - lo) * _rng(cfg, _ALPHA, head).random((T, d))).astype(np.float32),
        kt=np.zeros((0, d), np.float32), vt=np.zeros((0, d), np.float32), bt=np.zeros((0,), np.float32))
    if nt > 0:
        out["kt"] = store(_rng(cfg, _KT, head).standard_normal((nt, d)), dt)
        out["vt"] = store(_rng(cfg, _VT, head).standard_normal((nt, d)), dt)
        out["bt"] = _rng(cfg, _BT, head).standard_normal((nt,)).astype(np.float32)
    return HeadInputs(**out)


def all_raw_heads(cfg: Config, heads=None):
    heads = list(range(cfg.heads)) if heads is None else list(heads)
    return [raw_head_inputs(cfg, h) for h in heads]


def all_heads(cfg: Config, heads=None, workers: int | None = None,
              parts=("q", "k", "v", "beta", "alpha", "text")):
    """Inputs of several heads, drawn in parallel threads."""
    heads = list(range(cfg.heads)) if heads is None else list(heads)
    if workers is None:
        workers = min(len(heads), max(1, min(16, len(os.sched_getaffinity(0)))))
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        return list(ex.map(lambda h: head_inputs(cfg, h, parts), heads))


def stack(heads_in, name: str) -> np.ndarray:
    """Stack one stored tensor over heads -> [H, ...] (contiguous)."""
    return np.ascontiguousarray(np.stack([getattr(h, name) for h in heads_in]))
