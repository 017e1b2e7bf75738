"""Device plumbing around the libvda entry points: upload stored inputs into
torch device tensors, allocate the workspace / state / output buffers, and
enqueue the path

    vda_prepare_frames -> vda_scan_fwd || vda_scan_rev -> vda_readout

on HIP streams.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import inputs as inp
from . import vda


@dataclasses.dataclass
class DeviceInputs:
    q: object
    k: object
    v: object
    beta: object
    alpha: object
    kt: object
    vt: object
    bt: object


@dataclasses.dataclass
class Buffers:
    ws: object
    ws_bytes: int
    states_f: object
    states_r: object
    out: object


def _dev(arr: np.ndarray, device):
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)  # raw bf16 bit patterns
    return torch.from_numpy(a).to(device)


def upload(cfg: inp.Config, heads_in, device="cuda") -> DeviceInputs:
    """Stack per-head stored inputs into [H, ...] device tensors."""
    st = lambda name: _dev(inp.stack(heads_in, name), device)
    text = cfg.text_tokens > 0
    return DeviceInputs(q=st("q"), k=st("k"), v=st("v"), beta=st("beta"), alpha=st("alpha"),
                        kt=st("kt") if text else None, vt=st("vt") if text else None,
                        bt=st("bt") if text else None)


_OUT_TORCH = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def allocate(desc: vda.vda_desc, out_dtype: str, device="cuda") -> Buffers:
    import torch
    wsb = vda.vda_workspace_bytes(desc)
    cnt = vda.vda_state_count(desc)
    H, d = desc.heads, desc.d_k
    ws = torch.empty(wsb, dtype=torch.uint8, device=device)
    sf = torch.empty((H, cnt, d, d), dtype=torch.float32, device=device)
    sr = torch.empty((H, cnt, d, d), dtype=torch.float32, device=device)
    out = torch.empty((H, desc.frames, desc.tokens, d), dtype=getattr(torch, _OUT_TORCH[out_dtype]),
                      device=device)
    return Buffers(ws=ws, ws_bytes=wsb, states_f=sf, states_r=sr, out=out)


class Forward:
    """Enqueues the whole hot path with one vda_forward call (the library
    enqueues every kernel on the caller's stream, in order)."""

    def __init__(self, desc: vda.vda_desc, dev: DeviceInputs, bufs: Buffers):
        import torch
        self.desc, self.dev, self.bufs = desc, dev, bufs
        self.main = torch.cuda.current_stream()

    def enqueue(self):
        d, x, b = self.desc, self.dev, self.bufs
        vda.vda_forward(d, x.q, x.k, x.v, x.beta, x.alpha, x.kt, x.vt, x.bt, b.ws, b.states_f, b.states_r,
                        b.out, ws_bytes=b.ws_bytes, stream=self.main)


class Path:
    """Enqueues the whole hot path step by step, one entry point per step;
    the reverse scan runs on a second stream, concurrently with the forward
    scan."""

    def __init__(self, desc: vda.vda_desc, dev: DeviceInputs, bufs: Buffers, s_init=None):
        import torch
        self.desc, self.dev, self.bufs, self.s_init = desc, dev, bufs, s_init
        self.main = torch.cuda.current_stream()
        self.side = torch.cuda.Stream()
        self.ev_prep = torch.cuda.Event()
        self.ev_rev = torch.cuda.Event()

    def enqueue(self):
        d, x, b = self.desc, self.dev, self.bufs
        vda.vda_prepare_frames(d, x.k, x.v, x.beta, x.kt, x.vt, x.bt, b.ws, b.ws_bytes, stream=self.main)
        if d.flags & vda.VDA_CHUNK_SCAN:
            vda.vda_compose_chunks(d, b.ws, x.alpha, ws_bytes=b.ws_bytes, stream=self.main)
        self.ev_prep.record(self.main)
        self.side.wait_event(self.ev_prep)
        vda.vda_scan_rev(d, b.ws, x.alpha, self.s_init, b.states_r, stream=self.side)
        self.ev_rev.record(self.side)
        vda.vda_scan_fwd(d, b.ws, x.alpha, self.s_init, b.states_f, stream=self.main)
        self.main.wait_event(self.ev_rev)
        vda.vda_readout(d, x.q, x.alpha, b.states_f, b.states_r, b.out, stream=self.main)


def run(cfg: inp.Config, heads_in, device="cuda", s_init=None, fused=False, **desc_over):
    """Upload, run once, synchronise; return (desc, DeviceInputs, Buffers).
    fused=True runs the path through vda_forward (no explicit s_init)."""
    import torch
    desc = vda.desc_for(cfg, **desc_over)
    dev = upload(cfg, heads_in, device)
    bufs = allocate(desc, desc_over.get("out_dtype", cfg.out_dtype), device)
    if fused:
        assert s_init is None
        Forward(desc, dev, bufs).enqueue()
    else:
        Path(desc, dev, bufs, s_init=s_init).enqueue()
    torch.cuda.synchronize()
    return desc, dev, bufs


def out_f64(bufs: Buffers) -> np.ndarray:
    return bufs.out.float().cpu().numpy().astype(np.float64)


def upload_epilogue(cfg: inp.Config, epi_in, device="cuda"):
    """Stack per-head epilogue inputs (``inputs.epilogue_inputs``) into device
    tensors: gate logits [H, T, U, d] in the input dtype, weights [H, d]."""
    gate = _dev(np.stack([e.gate for e in epi_in]), device)
    weight = _dev(np.stack([e.weight for e in epi_in]), device)
    return gate, weight


def readout_gated(desc: vda.vda_desc, dev: DeviceInputs, bufs: Buffers, gate, weight, eps: float,
                  out_dtype: str, device="cuda"):
    """Run vda_readout_gated on the states in ``bufs`` into a new output
    tensor, synchronise and return it."""
    import torch
    out = torch.empty(tuple(bufs.out.shape), dtype=getattr(torch, _OUT_TORCH[out_dtype]), device=device)
    d = vda.vda_desc.from_buffer_copy(desc)
    d.out_dtype = vda.DTYPES[out_dtype]
    vda.vda_readout_gated(d, dev.q, dev.alpha, bufs.states_f, bufs.states_r, gate, weight, eps, out)
    torch.cuda.synchronize()
    return out
