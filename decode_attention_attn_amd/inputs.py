"""Seeded synthetic inputs for the MFA decode path, in their storage form.

This module is shared by the tests, the benchmark and the smoke check. It draws
random numbers and encodes them into the storage formats the library consumes
(fp32, bf16 bit patterns, OCP e4m3fn bytes plus a per-tensor fp32 scale). It
performs none of the method's arithmetic: no projection, norm, softmax or
attention happens here, so neither the HIP path nor the CPU oracle depends on
code that the other also uses for computing results.

Shapes follow the Step-3 MFA description (Step-3 paper summary on
bud-325.pages.dev, "Key claims" and "Method"; redeep.blog Step3 post,
architecture table): hidden 7168, query rank 2048, 64 query heads of width 256,
one shared K head and one shared V head of width 256.

Draw recipe (the pages fix none of it):
  * one independent stream per tensor, ``numpy.random.default_rng([seed, id])``
    with fixed ids, so adding or removing a tensor never shifts another's draws;
  * standard-normal float32 draws; weights are scaled by fan_in**-0.5 in float32
    (variance 1/fan_in);
  * bf16 storage rounds the float32 draw to nearest-even; fp8 storage quantizes
    with one scale per tensor, scale = amax/448, round-to-nearest-even with
    saturation to +-448;
  * ragged lengths are integers drawn uniformly from a closed interval.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

HIDDEN = 7168
RANK = 2048
N_HEADS = 64
HEAD_DIM = 256
QDIM = N_HEADS * HEAD_DIM  # 16384

# Stream ids, one per tensor.
ID_X, ID_WDQ, ID_WUQ, ID_WK, ID_WV, ID_WO, ID_Q, ID_K, ID_V, ID_LEN, ID_PAGES = range(11)

F32, BF16, FP8 = "f32", "bf16", "fp8_e4m3"
FP8_BLOCK = "fp8_block"  # weights: e4m3 bytes with one fp32 scale per 128 x 128 block

E4M3_MAX = 448.0


# ---------------------------------------------------------------- storage codecs
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns.

    bfloat16 is the upper half of an IEEE-754 binary32 word. Inputs here are
    finite (normal draws), so no NaN special case is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def _e4m3fn_positive_codes() -> np.ndarray:
    """Magnitudes of the e4m3fn codes 0x00..0x7E in code order (strictly increasing).

    Encoding (OCP 8-bit floating point, E4M3): 4 exponent bits with bias 7,
    3 mantissa bits, exponent field 0 is subnormal, 0x7F is NaN, no infinity.
    """
    vals = np.empty(0x7F, dtype=np.float64)
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals[code] = m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10)
    return vals


_E4M3_POS = _e4m3fn_positive_codes()


def encode_e4m3fn(v: np.ndarray) -> np.ndarray:
    """Encode values (already divided by the scale) as e4m3fn bytes.

    Nearest representable value, ties to the even code (even mantissa), values
    beyond +-448 saturate to +-448. Zero and negative zero both give 0x00/0x80.
    """
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")  # first code with value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dhi = _E4M3_POS[hi] - mag
    dlo = mag - _E4M3_POS[lo]
    pick_lo = (dlo < dhi) | ((dlo == dhi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(mag == _E4M3_POS[hi], hi, code).astype(np.uint8)
    sign = (np.signbit(v) & (code != 0)).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def quantize_e4m3fn(x: np.ndarray):
    """Per-tensor e4m3fn quantization: returns (codes uint8, scale float32).

    scale = amax(|x|) / 448 in float32; codes = encode(x / scale).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    scale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    codes = encode_e4m3fn(x.astype(np.float64) / np.float64(scale))
    return codes, scale


def quantize_blocks_e4m3fn(w: np.ndarray, block: int = 128):
    """Block-fp8 storage of a weight [out, in]: one float32 scale per
    block x block tile (its amax / 448, 1 for an all-zero tile) and the e4m3
    bytes of w / scale. Returns (codes uint8 [out, in], scales float32
    [out / block, in / block])."""
    w = np.asarray(w, dtype=np.float32)
    o, i = w.shape
    t = np.abs(w).reshape(o // block, block, i // block, block).max(axis=(1, 3))
    scales = np.where(t > 0, t / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    full = np.repeat(np.repeat(scales.astype(np.float64), block, axis=0), block, axis=1)
    return encode_e4m3fn(w.astype(np.float64) / full), scales


def store(x: np.ndarray, kind: str):
    """float32 draws -> storage array for ``kind`` (fp32 copy or bf16 bits)."""
    if kind == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if kind == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(kind)


# ---------------------------------------------------------------- draws
def normal(seed: int, tid: int, shape, scale: Optional[float] = None) -> np.ndarray:
    g = np.random.default_rng([seed, tid])
    z = g.standard_normal(size=shape, dtype=np.float32)
    if scale is not None:
        z *= np.float32(scale)
    return z


def weight(seed: int, tid: int, out_dim: int, in_dim: int) -> np.ndarray:
    """[out, in] float32 draws with variance 1/in."""
    return normal(seed, tid, (out_dim, in_dim), scale=float(in_dim) ** -0.5)


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    g = np.random.default_rng([seed, ID_LEN])
    return g.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


def packed_offsets(capacity: np.ndarray) -> np.ndarray:
    """Start row of each sequence when sequences are packed back to back."""
    off = np.zeros(len(capacity), dtype=np.int64)
    if len(capacity) > 1:
        off[1:] = np.cumsum(np.asarray(capacity, dtype=np.int64))[:-1]
    return off


# ---------------------------------------------------------------- workloads
@dataclasses.dataclass
class Workload:
    """Sizes of one synthetic workload.

    kind "layer": full decode layer (q path, K/V append, attention, out-proj);
    kind "attn": attention core only (q, K and V given).
    """

    name: str
    kind: str
    batch: int
    ctx: int  # cached rows per sequence before the step (layer) / attended rows (attn)
    act: str  # activation / weight / q storage
    kv: str  # cache storage
    ragged: Optional[tuple] = None  # (lo, hi) closed interval of lengths
    seed: int = 0
    description: str = ""
    weights: str = ""  # "" = stored like the activations; FP8_BLOCK = e4m3 with 128 x 128 block scales


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        "tiny_fp32", "layer", 2, 128, F32, F32,
        description="fp32 decode layer, batch 2, 128 cached rows + 1 appended (129 attended)"),
    "attn_bf16_4k": Workload(
        "attn_bf16_4k", "attn", 32, 4096, BF16, BF16,
        description="bf16 attention core, batch 32, 4096 positions each"),
    "attn_fp8kv_4k": Workload(
        "attn_fp8kv_4k", "attn", 64, 4096, BF16, FP8,
        description="bf16 q with e4m3fn K/V cache (per-tensor scales), batch 64, 4096 positions"),
    "attn_bf16_ragged": Workload(
        "attn_bf16_ragged", "attn", 16, 0, BF16, BF16, ragged=(8192, 65536),
        description="bf16 attention core, batch 16, lengths uniform in [8192, 65536], packed"),
    "layer_bf16_8k": Workload(
        "layer_bf16_8k", "layer", 128, 8192, BF16, BF16,
        description="bf16 decode layer, batch 128, 8192 cached rows + 1 appended (8193 attended)"),
    "layer_fp8_8k": Workload(
        "layer_fp8_8k", "layer", 128, 8192, BF16, FP8, weights=FP8_BLOCK,
        description="the FP8 decode layer: block-fp8 weights (e4m3, 128 x 128 block scales), bf16 activations, "
                    "e4m3fn K/V cache, batch 128, 8192 cached rows + 1 appended"),
    "layer_bf16_fp8kv_8k": Workload(
        "layer_bf16_fp8kv_8k", "layer", 128, 8192, BF16, FP8,
        description="bf16 decode layer over an e4m3fn K/V cache (per-tensor scales, new rows quantized on "
                    "append), batch 128, 8192 cached rows + 1 appended"),
}


def scaled(w: Workload, batch: Optional[int] = None, ctx: Optional[int] = None,
           ragged: Optional[tuple] = None, seed: Optional[int] = None) -> Workload:
    """A copy of ``w`` with smaller sizes (for parity runs the oracle can finish)."""
    return dataclasses.replace(
        w,
        batch=w.batch if batch is None else batch,
        ctx=w.ctx if ctx is None else ctx,
        ragged=w.ragged if ragged is None else ragged,
        seed=w.seed if seed is None else seed,
    )


def _kv_store(x: np.ndarray, kind: str):
    if kind == FP8:
        return quantize_e4m3fn(x)
    return store(x, kind), None


def make_attn(w: Workload, lengths: Optional[np.ndarray] = None) -> dict:
    """Attention-core inputs: q [B,64,256], packed K/V caches, offsets, lengths."""
    assert w.kind == "attn"
    B = w.batch
    if lengths is None:
        if w.ragged is not None:
            lengths = ragged_lengths(w.seed, B, *w.ragged)
        else:
            lengths = np.full(B, w.ctx, dtype=np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    off = packed_offsets(lengths)
    rows = int(lengths.sum())
    q = store(normal(w.seed, ID_Q, (B, N_HEADS, HEAD_DIM)), w.act)
    k, k_scale = _kv_store(normal(w.seed, ID_K, (max(rows, 1), HEAD_DIM)), w.kv)
    v, v_scale = _kv_store(normal(w.seed, ID_V, (max(rows, 1), HEAD_DIM)), w.kv)
    return dict(workload=w, q=q, k_cache=k, v_cache=v, k_scale=k_scale, v_scale=v_scale,
                seq_off=off, seq_len=lengths, kind_q=w.act, kind_kv=w.kv)


def with_tokens(inp: dict, n_tokens: int) -> dict:
    """Attention inputs with ``n_tokens`` query tokens per sequence (q
    [B, n_tokens, 64, 256], drawn from the same stream as ``make_attn``'s q,
    so n_tokens = 1 gives the same numbers); the cache is unchanged."""
    w = inp["workload"]
    B = len(inp["seq_len"])
    q = store(normal(w.seed, ID_Q, (B, n_tokens, N_HEADS, HEAD_DIM)), w.act)
    return dict(inp, q=q, n_tokens=n_tokens)


def to_pages(inp: dict, page_rows: int, seed: int = 0, spare_pages: int = 3) -> dict:
    """Paged copy of attention inputs from ``make_attn``: the same keys and
    values, with each sequence's rows cut into blocks of ``page_rows`` and the
    blocks placed on pages in a seeded random order (plus a few unused pages).
    Rows of a sequence's last page past its length, and the unused pages,
    hold NaN codes (bf16 0x7FC0, fp32 NaN, e4m3 0x7F): a read of them shows.
    Unused table entries point at page 0."""
    lens = np.asarray(inp["seq_len"], dtype=np.int64)
    off = np.asarray(inp["seq_off"], dtype=np.int64)
    nblk = (lens + page_rows - 1) // page_rows
    n_pages = int(nblk.sum()) + spare_pages
    max_blocks = max(int(nblk.max()), 1)
    perm = np.random.default_rng([seed, ID_PAGES]).permutation(n_pages)
    table = np.zeros((len(lens), max_blocks), dtype=np.int32)
    kind = inp["kind_kv"]
    fill = {F32: np.float32(np.nan), BF16: np.uint16(0x7FC0), FP8: np.uint8(0x7F)}[kind]
    kc, vc = inp["k_cache"], inp["v_cache"]
    kp = np.full((n_pages * page_rows,) + kc.shape[1:], fill, dtype=kc.dtype)
    vp = np.full((n_pages * page_rows,) + vc.shape[1:], fill, dtype=vc.dtype)
    nxt = 0
    for b in range(len(lens)):
        for j in range(int(nblk[b])):
            page = int(perm[nxt])
            nxt += 1
            table[b, j] = page
            n = int(min(page_rows, lens[b] - j * page_rows))
            src = int(off[b]) + j * page_rows
            kp[page * page_rows:page * page_rows + n] = kc[src:src + n]
            vp[page * page_rows:page * page_rows + n] = vc[src:src + n]
    return dict(inp, k_pages=kp, v_pages=vp, block_table=table, max_blocks=max_blocks, page_rows=page_rows)


CANARY = 1234.0  # value left in cache rows that the step must not read before writing
CANARY_E4M3 = 0x7F  # the same for an e4m3 cache: the NaN code


def make_layer(w: Workload) -> dict:
    """Full-layer inputs: x, five weight matrices, caches with one free row per sequence."""
    assert w.kind == "layer"
    B, ctx = w.batch, w.ctx
    cap = np.full(B, ctx + 1, dtype=np.int64)
    off = packed_offsets(cap)
    total_rows = int(cap.sum())
    x = store(normal(w.seed, ID_X, (B, HIDDEN)), w.act)
    draws = dict(w_dq=weight(w.seed, ID_WDQ, RANK, HIDDEN), w_uq=weight(w.seed, ID_WUQ, QDIM, RANK),
                 w_k=weight(w.seed, ID_WK, HEAD_DIM, HIDDEN), w_v=weight(w.seed, ID_WV, HEAD_DIM, HIDDEN),
                 w_o=weight(w.seed, ID_WO, HIDDEN, QDIM))
    wts = {}
    for name, d in draws.items():
        if w.weights == FP8_BLOCK:
            wts[name], wts[name + "_scale"] = quantize_blocks_e4m3fn(d)
        else:
            wts[name] = store(d, w.act)
    del draws
    caches, scales = [], []
    for tid in (ID_K, ID_V):
        draws = normal(w.seed, tid, (B * ctx, HEAD_DIM)).reshape(B, ctx, HEAD_DIM)
        if w.kv == FP8:
            # per-tensor scale from the cached draws; the free row holds the
            # NaN code, so reading it before the append would poison the output
            codes, sc = quantize_e4m3fn(draws)
            full = np.full((B, ctx + 1, HEAD_DIM), CANARY_E4M3, dtype=np.uint8)
            full[:, :ctx, :] = codes
            caches.append(full.reshape(total_rows, HEAD_DIM))
            scales.append(sc)
        else:
            full = np.full((B, ctx + 1, HEAD_DIM), CANARY, dtype=np.float32)
            full[:, :ctx, :] = draws
            caches.append(store(full.reshape(total_rows, HEAD_DIM), w.kv))
            scales.append(None)
    return dict(workload=w, x=x, **wts,
                k_cache=caches[0], v_cache=caches[1], k_scale=scales[0], v_scale=scales[1], seq_off=off,
                seq_len=np.full(B, ctx, dtype=np.int32), capacity=cap,
                kind_act=w.act, kind_kv=w.kv, kind_w=w.weights or w.act, eps=1e-6)
