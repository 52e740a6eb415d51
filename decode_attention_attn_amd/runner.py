"""Device plumbing around the libmfa binding: upload stored inputs, allocate
outputs and workspaces with torch, call the C entry points on one stream.

No arithmetic of the method happens here; torch only provides device memory
and the stream.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from . import mfa
from .inputs import BF16, F32, FP8, FP8_BLOCK

SOFTMAX_SCALE = 1.0 / math.sqrt(256.0)

_DT = {F32: mfa.MFA_F32, BF16: mfa.MFA_BF16, FP8: mfa.MFA_FP8_E4M3}


def to_device(arr: np.ndarray, kind: str, device="cuda") -> torch.Tensor:
    """Stored numpy array -> torch tensor holding the same bytes on ``device``."""
    arr = np.ascontiguousarray(arr)
    if kind == F32:
        t = torch.from_numpy(arr.astype(np.float32, copy=False))
    elif kind == BF16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    elif kind == FP8:
        t = torch.from_numpy(arr.astype(np.uint8, copy=False))
    elif kind == "i64":
        t = torch.from_numpy(arr.astype(np.int64, copy=False))
    elif kind == "i32":
        t = torch.from_numpy(arr.astype(np.int32, copy=False))
    else:
        raise ValueError(kind)
    return t.to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor (fp32 or bf16) -> exact float64 numpy copy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def dtype_code(kind: str) -> int:
    return _DT[kind]


def _act_torch(kind):
    return torch.float32 if kind == F32 else torch.bfloat16


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def upload_attn(inp: dict, device="cuda") -> dict:
    """Attention inputs on the device; a paged layout (``inputs.to_pages``)
    uploads the pages and the block table instead of the packed cache."""
    paged = "block_table" in inp
    kk = inp["kind_kv"]
    return dict(
        q=to_device(inp["q"], inp["kind_q"], device),
        k=to_device(inp["k_pages"] if paged else inp["k_cache"], kk, device),
        v=to_device(inp["v_pages"] if paged else inp["v_cache"], kk, device),
        off=to_device(inp["seq_off"], "i64", device),
        len=to_device(inp["seq_len"], "i32", device),
        table=to_device(inp["block_table"], "i32", device) if paged else None,
        max_blocks=int(inp["max_blocks"]) if paged else 0,
        page_rows=int(inp["page_rows"]) if paged else 0,
        kind_q=inp["kind_q"], kind_kv=kk, nt=int(inp.get("n_tokens", 1)),
        k_scale=float(inp["k_scale"]) if inp["k_scale"] is not None else 1.0,
        v_scale=float(inp["v_scale"]) if inp["v_scale"] is not None else 1.0,
        B=len(inp["seq_len"]),
    )


class AttnCall:
    """Preallocated outputs + workspace for repeated mfa_decode_attn calls."""

    def __init__(self, dev: dict, num_workgroups: int = 0, want_lse: bool = True, stream=None):
        self.dev = dev
        self.G = num_workgroups
        B = dev["B"]
        device = dev["q"].device
        nt = dev.get("nt", 1)
        shape = (B, 64, 256) if nt == 1 else (B, nt, 64, 256)
        self.out = torch.empty(shape, dtype=_act_torch(dev["kind_q"]), device=device)
        self.lse = torch.empty(shape[:-1], dtype=torch.float32, device=device) if want_lse else None
        self.ws = _ws(mfa.mfa_decode_attn_mt_workspace_size(B, nt, num_workgroups), device)
        self.stream = stream

    def __call__(self, k=None, v=None):
        d = self.dev
        k = d["k"] if k is None else k
        v = d["v"] if v is None else v
        if d.get("table") is not None and d.get("nt", 1) > 1:
            st = mfa.mfa_decode_attn_paged_mt(d["q"], k, v, d["table"], d["max_blocks"], d["page_rows"], d["len"],
                                              d["nt"], SOFTMAX_SCALE, d["k_scale"], d["v_scale"], self.out, self.lse,
                                              self.ws, d["B"], self.G, _DT[d["kind_q"]], _DT[d["kind_kv"]],
                                              self.stream)
            mfa.check(st, "mfa_decode_attn_paged_mt")
        elif d.get("table") is not None:
            st = mfa.mfa_decode_attn_paged(d["q"], k, v, d["table"], d["max_blocks"], d["page_rows"], d["len"],
                                           SOFTMAX_SCALE, d["k_scale"], d["v_scale"], self.out, self.lse, self.ws,
                                           d["B"], self.G, _DT[d["kind_q"]], _DT[d["kind_kv"]], self.stream)
            mfa.check(st, "mfa_decode_attn_paged")
        elif d.get("nt", 1) > 1:
            st = mfa.mfa_decode_attn_mt(d["q"], k, v, d["off"], d["len"], d["nt"], SOFTMAX_SCALE, d["k_scale"],
                                        d["v_scale"], self.out, self.lse, self.ws, d["B"], self.G,
                                        _DT[d["kind_q"]], _DT[d["kind_kv"]], self.stream)
            mfa.check(st, "mfa_decode_attn_mt")
        else:
            st = mfa.mfa_decode_attn(d["q"], k, v, d["off"], d["len"], SOFTMAX_SCALE, d["k_scale"], d["v_scale"],
                                     self.out, self.lse, self.ws, d["B"], self.G, _DT[d["kind_q"]],
                                     _DT[d["kind_kv"]], self.stream)
            mfa.check(st, "mfa_decode_attn")
        return self.out, self.lse


def decode_attn(inp: dict, num_workgroups: int = 0, device="cuda"):
    """Upload, run once, synchronize; returns (out, lse, device inputs)."""
    dev = upload_attn(inp, device)
    call = AttnCall(dev, num_workgroups)
    out, lse = call()
    torch.cuda.synchronize()
    return out, lse, dev


def upload_layer(inp: dict, device="cuda") -> dict:
    ka, kk, kw = inp["kind_act"], inp["kind_kv"], inp.get("kind_w", inp["kind_act"])
    d = {"x": to_device(inp["x"], ka, device)}
    for n in ("w_dq", "w_uq", "w_k", "w_v", "w_o"):
        if kw == FP8_BLOCK:
            d[n] = to_device(inp[n], FP8, device)
            d[n + "_scale"] = to_device(inp[n + "_scale"], F32, device)
        else:
            d[n] = to_device(inp[n], kw, device)
    d.update(kind_w=kw, k=to_device(inp["k_cache"], kk, device), v=to_device(inp["v_cache"], kk, device),
             off=to_device(inp["seq_off"], "i64", device), len=to_device(inp["seq_len"], "i32", device),
             kind_act=ka, kind_kv=kk, B=len(inp["seq_len"]), eps=float(inp.get("eps", 1e-6)),
             k_scale=float(inp["k_scale"]) if inp.get("k_scale") is not None else 1.0,
             v_scale=float(inp["v_scale"]) if inp.get("v_scale") is not None else 1.0)
    return d


class LayerCall:
    """One decode step of the attention layer: q path, K/V append, attention, out-projection."""

    def __init__(self, dev: dict, num_workgroups: int = 0, stream=None, fused_q_kv: bool = True):
        self.dev = dev
        B = dev["B"]
        device = dev["x"].device
        at = _act_torch(dev["kind_act"])
        dt = _DT[dev["kind_act"]]
        self.dt = dt
        if dev["kind_w"] == FP8_BLOCK and dev["kind_act"] != BF16:
            raise ValueError("block-fp8 weights take bf16 activations")
        self.G = num_workgroups
        self.stream = stream
        self.q = torch.empty((B, 64, 256), dtype=at, device=device)
        self.o = torch.empty((B, 64, 256), dtype=at, device=device)
        self.lse = torch.empty((B, 64), dtype=torch.float32, device=device)
        self.y = torch.empty((B, 7168), dtype=at, device=device)
        self.len_after = torch.empty_like(dev["len"])
        self.ws_q = _ws(mfa.mfa_qproj_workspace_size(B, dt), device)
        self.ws_kv = _ws(mfa.mfa_kv_append_workspace_size(B, dt), device)
        self.ws_a = _ws(mfa.mfa_decode_attn_workspace_size(B, num_workgroups), device)
        self.ws_o = _ws(mfa.mfa_oproj_workspace_size(B, dt), device)
        # bf16 activations: the q path and the K/V append as one call (one
        # product over [W_dq; W_k; W_v], mfa_qproj_kv_append, or
        # mfa_qproj_kv_append_w8 for block-fp8 weights)
        self.fused = fused_q_kv and dev["kind_act"] == BF16 and dev["kind_kv"] in (BF16, FP8)
        self.ws_qkv = _ws(mfa.mfa_qproj_kv_append_workspace_size(B), device) if self.fused else None

    def __call__(self):
        d, dt, s = self.dev, self.dt, self.stream
        B = d["B"]
        if d["kind_w"] == FP8_BLOCK:
            return self._call_w8()
        if self.fused:
            mfa.check(mfa.mfa_qproj_kv_append(d["x"], d["w_dq"], None, d["eps"], d["w_uq"], d["w_k"], d["w_v"], self.q,
                                              d["k"], d["v"], d["off"], d["len"], d["k_scale"], d["v_scale"],
                                              self.ws_qkv, B, _DT[d["kind_kv"]], s, seq_len_out=self.len_after),
                      "mfa_qproj_kv_append")
        else:
            self._q_then_kv()
        # the appended row is attended: the append wrote len + 1 into len_after
        mfa.check(mfa.mfa_decode_attn(self.q, d["k"], d["v"], d["off"], self.len_after, SOFTMAX_SCALE,
                                      d["k_scale"], d["v_scale"], self.o, self.lse, self.ws_a, B, self.G, dt,
                                      _DT[d["kind_kv"]], s),
                  "mfa_decode_attn")
        mfa.check(mfa.mfa_oproj(self.o, d["w_o"], self.y, self.ws_o, B, dt, s), "mfa_oproj")
        return self

    def _q_then_kv(self):
        """The q path and the K/V append as two calls."""
        d, dt, s = self.dev, self.dt, self.stream
        B = d["B"]
        mfa.check(mfa.mfa_qproj(d["x"], d["w_dq"], None, d["eps"], d["w_uq"], self.q, self.ws_q, B, dt, s),
                  "mfa_qproj")
        if d["kind_kv"] == FP8:
            mfa.check(mfa.mfa_kv_append_fp8(d["x"], d["w_k"], d["w_v"], d["k"], d["v"], d["off"], d["len"],
                                            d["k_scale"], d["v_scale"], self.ws_kv, B, dt, s,
                                            seq_len_out=self.len_after), "mfa_kv_append_fp8")
        else:
            mfa.check(mfa.mfa_kv_append(d["x"], d["w_k"], d["w_v"], d["k"], d["v"], d["off"], d["len"], self.ws_kv,
                                        B, dt, _DT[d["kind_kv"]], s, seq_len_out=self.len_after), "mfa_kv_append")

    def _call_w8(self):
        # block-fp8 weights: the same steps through the _w8 entry points
        # (bf16 activations; the cache is bf16 or e4m3)
        d, dt, s = self.dev, self.dt, self.stream
        B = d["B"]
        if self.fused:
            mfa.check(mfa.mfa_qproj_kv_append_w8(d["x"], d["w_dq"], d["w_dq_scale"], None, d["eps"], d["w_uq"],
                                                 d["w_uq_scale"], d["w_k"], d["w_k_scale"], d["w_v"], d["w_v_scale"],
                                                 self.q, d["k"], d["v"], d["off"], d["len"], d["k_scale"],
                                                 d["v_scale"], self.ws_qkv, B, _DT[d["kind_kv"]], s,
                                                 seq_len_out=self.len_after), "mfa_qproj_kv_append_w8")
        else:
            mfa.check(mfa.mfa_qproj_w8(d["x"], d["w_dq"], d["w_dq_scale"], None, d["eps"], d["w_uq"],
                                       d["w_uq_scale"], self.q, self.ws_q, B, s), "mfa_qproj_w8")
            mfa.check(mfa.mfa_kv_append_w8(d["x"], d["w_k"], d["w_k_scale"], d["w_v"], d["w_v_scale"], d["k"],
                                           d["v"], d["off"], d["len"], _DT[d["kind_kv"]], d["k_scale"],
                                           d["v_scale"], self.ws_kv, B, s, seq_len_out=self.len_after),
                      "mfa_kv_append_w8")
        mfa.check(mfa.mfa_decode_attn(self.q, d["k"], d["v"], d["off"], self.len_after, SOFTMAX_SCALE,
                                      d["k_scale"], d["v_scale"], self.o, self.lse, self.ws_a, B, self.G, dt,
                                      _DT[d["kind_kv"]], s),
                  "mfa_decode_attn")
        mfa.check(mfa.mfa_oproj_w8(self.o, d["w_o"], d["w_o_scale"], self.y, self.ws_o, B, s), "mfa_oproj_w8")
        return self
