"""Plain float64 CPU definition of one MFA decode step (test infrastructure only).

This module is the parity oracle. It is deliberately slow and literal: every
step is the textbook definition written in numpy float64, one sequence at a
time, with no tiling, no online softmax and no split/merge of the key range.
Only the tests, the smoke check and the benchmark's CPU-baseline leg use it; the
HIP library never imports or calls it and it never calls the library.

Sources (the text of the pages about "Step-3 is Large yet Affordable:
Model-system Co-design for Cost-effective Decoding"):
  * Step-3 paper summary (bud-325.pages.dev), "Key claims" and "Method": the
    query is down-projected from hidden 7168 to rank 2048, normalized, and
    up-projected to 64 heads of width 256; one K head and one V head of width
    256 are shared by all 64 query heads; the cache holds one K and one V row
    per token.
  * redeep.blog Step3 post, "What's New" and the architecture table: the same
    shapes (hidden 7168, 64 query heads, head size 256, query rank 2048).
  * Step-3 paper index page (mlsanity.com), "Abstract": FP8 decoding.

Readings where the pages are silent (each one is a choice this library makes):
  * the normalization is RMSNorm, x * (mean(x^2) + eps)^-1/2 * gamma, eps 1e-6,
    gamma defaulting to ones;
  * softmax scale 1/sqrt(256) = 1/16; no rotary or other positional term;
  * no projection biases; K and V are plain projections of the hidden state;
  * weights are stored [out, in] (y = x W^T); column n of the up-projection is
    head n // 256, channel n % 256, and the attention output is flattened the
    same way before the out-projection;
  * the single new query attends to every cached row of its sequence, the row
    appended in this step included; no mask;
  * log-sum-exp uses the natural log; a sequence with no rows gives output 0
    and lse = -inf;
  * with several new tokens per sequence (multi-token decode), their K/V
    rows are the sequence's last rows and token t sees the rows before its
    own successors (causal among the new tokens), none of the later ones;
  * a paged cache holds sequence b's keys j*R .. j*R + R - 1 (R rows per
    page) on page block_table[b][j]; it is the same sequence of keys, laid
    out in pages (the pages give no layout; paging is a serving choice);
  * block-fp8 weights (the model card's checkpoint format) are e4m3 bytes
    with one float32 scale per 128 x 128 block: W = bytes * scale, exactly;
  * an fp8 cache is OCP E4M3 ("fn") bytes with one float32 scale per tensor
    (the model runs in FP8, attention included: Step-3 summary, "Key
    claims"); a new row is stored as e4m3(x / scale), rounded to nearest with
    ties to even and saturated at +-448.

Parity pins: every function here is checked against closed forms, hand-worked
fixtures, invariants and a pure-Python brute force in tests/test_oracle_cpu.py.
"""

from __future__ import annotations

import math

import numpy as np

SOFTMAX_SCALE = 1.0 / math.sqrt(256.0)


# ------------------------------------------------------------------ storage
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper 16 bits of an IEEE-754 binary32 word.
    """
    w = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """The 256 values of the OCP FP8 E4M3 ("fn") format, indexed by byte.

    Bit 7 is the sign, bits 6..3 the exponent (bias 7), bits 2..0 the mantissa.
    Exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there is
    no infinity.
    """
    t = np.empty(256, dtype=np.float64)
    for b in range(256):
        sign = -1.0 if b & 0x80 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            t[b] = math.nan
        elif e == 0:
            t[b] = sign * math.ldexp(m, -9)
        else:
            t[b] = sign * math.ldexp(1.0 + m / 8.0, e - 7)
    return t


_E4M3 = e4m3fn_table()


E4M3_MAX = 448.0


def encode_e4m3fn(y) -> np.ndarray:
    """float64 values -> OCP FP8 E4M3 ("fn") bytes, round to nearest, ties to even.

    Written from the format definition above: in the normal range
    (|y| >= 2^-6) write |y| = 2^e * f with f in [1, 2); the neighbours are
    2^e * (1 + k/8), so k = round_half_even(8 (f - 1)), k = 8 carrying into
    the next binade. Below 2^-6 the step is 2^-9: k = round_half_even(|y| 2^9)
    is the subnormal code itself (k = 8 lands on 2^-6, code 0x08). Magnitudes
    above 448, the largest finite value, saturate to 448 (the quantizer clamps
    before rounding); NaN gives 0x7F; the sign bit follows signbit(y).
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    codes = np.zeros(y.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    codes[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    nrm = ~sub & ~np.isnan(a)
    if np.any(nrm):
        frac, ex = np.frexp(a[nrm])       # a = frac * 2^ex, frac in [0.5, 1)
        e = ex.astype(np.int64) - 1       # a = 2^e * f, f = 2 frac in [1, 2)
        k = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)
        carry = k == 8
        e[carry] += 1
        k[carry] = 0
        codes[nrm] = ((e + 7) << 3) | k
    codes[np.isnan(a)] = 0x7F
    codes |= np.where(np.signbit(y), 0x80, 0)
    return codes.astype(np.uint8)


def quantize_e4m3fn(x, scale) -> np.ndarray:
    """Per-tensor e4m3 storage of x with a float32 scale: bytes encode_e4m3fn(x / scale)."""
    return encode_e4m3fn(np.asarray(x, dtype=np.float64) / np.float64(np.float32(scale)))


def dequantize_blocks_e4m3fn(codes, scales, block: int = 128) -> np.ndarray:
    """Block-fp8 weight -> float64: W[n][k] = e4m3(codes[n][k]) * scales[n // block][k // block]
    (each product is exact in float64)."""
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)
    return _E4M3[np.asarray(codes, dtype=np.uint8)] * full


def decode_e4m3fn(codes: np.ndarray, scale) -> np.ndarray:
    """fp8 bytes with a per-tensor float32 scale -> float64 (the product is exact)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)] * np.float64(np.float32(scale))


def to_f64(arr: np.ndarray, kind: str, scale=None) -> np.ndarray:
    """Upcast a stored tensor ("f64", "f32", "bf16" bit patterns or "fp8_e4m3" bytes) to float64."""
    if kind == "f64":
        return np.asarray(arr, dtype=np.float64)
    if kind == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if kind == "bf16":
        return decode_bf16(arr)
    if kind == "fp8_e4m3":
        return decode_e4m3fn(arr, scale)
    raise ValueError(f"unknown storage kind {kind!r}")


# ------------------------------------------------------------------ query path
def rms_norm(c: np.ndarray, eps: float = 1e-6, gamma=None) -> np.ndarray:
    """RMSNorm over the last axis: c / sqrt(mean(c^2) + eps) * gamma."""
    c = np.asarray(c, dtype=np.float64)
    ms = np.mean(c * c, axis=-1, keepdims=True)
    out = c / np.sqrt(ms + eps)
    if gamma is not None:
        out = out * np.asarray(gamma, dtype=np.float64)
    return out


def q_path(x, w_dq, w_uq, eps=1e-6, gamma=None, n_heads=64, head_dim=256):
    """Low-rank query: c = x W_dq^T, c_hat = RMSNorm(c), q = c_hat W_uq^T -> [B, H, D].

    (Step-3 summary, "Method": down-projection 7168 -> 2048, normalization,
    up-projection to 64 x 256.) Returns (c, c_hat, q).
    """
    x = np.asarray(x, dtype=np.float64)
    c = x @ np.asarray(w_dq, dtype=np.float64).T
    c_hat = rms_norm(c, eps, gamma)
    q = c_hat @ np.asarray(w_uq, dtype=np.float64).T
    return c, c_hat, q.reshape(x.shape[0], n_heads, head_dim)


def kv_project(x, w_k, w_v):
    """The one shared K row and one shared V row of each new token: x W_k^T, x W_v^T.

    (Step-3 summary, "Key claims"/"Method": a single K head and a single V head
    of width 256 shared by all 64 query heads.)
    """
    x = np.asarray(x, dtype=np.float64)
    return x @ np.asarray(w_k, dtype=np.float64).T, x @ np.asarray(w_v, dtype=np.float64).T


# ------------------------------------------------------------------ attention
def attend_one(q_b, k_b, v_b, scale=SOFTMAX_SCALE):
    """Softmax attention of H query rows over one shared K/V head.

    S = q_b K_b^T * scale; m = row max; P = exp(S - m); l = row sum;
    O = P V_b / l; lse = m + ln l. Two passes over the full row, no tiling.
    With zero rows: O = 0 and lse = -inf.
    """
    q_b = np.asarray(q_b, dtype=np.float64)
    k_b = np.asarray(k_b, dtype=np.float64)
    v_b = np.asarray(v_b, dtype=np.float64)
    H, D = q_b.shape
    if k_b.shape[0] == 0:
        return np.zeros((H, v_b.shape[1])), np.full(H, -np.inf)
    s = (q_b @ k_b.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v_b) / l
    return o, (m + np.log(l))[:, 0]


def decode_attn(q, k_cache, v_cache, seq_off, seq_len, scale=SOFTMAX_SCALE,
                kind_q="f64", kind_kv="f64", k_scale=None, v_scale=None, batch_ids=None):
    """Attention for every sequence b over cache rows [off_b, off_b + len_b).

    Inputs may be stored tensors (kind "f32" / "bf16" / "fp8_e4m3") or float64
    ("f64"); each sequence is upcast separately to bound memory. ``batch_ids``
    restricts the work to a subset of sequences (returned in that order).
    Returns (O [n, H, D], lse [n, H]).
    """
    ids = range(len(seq_len)) if batch_ids is None else batch_ids

    def up(a, kind, sc):
        return np.asarray(a, dtype=np.float64) if kind == "f64" else to_f64(a, kind, sc)

    outs, lses = [], []
    for b in ids:
        o0, n = int(seq_off[b]), int(seq_len[b])
        qb = up(q[b], kind_q, None)
        kb = up(k_cache[o0:o0 + n], kind_kv, k_scale)
        vb = up(v_cache[o0:o0 + n], kind_kv, v_scale)
        o, lse = attend_one(qb, kb, vb, scale)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


def decode_attn_mt(q, k_cache, v_cache, seq_off, seq_len, n_tokens, scale=SOFTMAX_SCALE,
                   kind_q="f64", kind_kv="f64", k_scale=None, v_scale=None, batch_ids=None):
    """Several new query tokens per sequence (q [B, n, H, D]), whose K/V rows are
    the last n of the sequence's len_b rows: token t attends, causally, over
    the first len_b - (n - 1 - t) rows (none if that is <= 0: output 0,
    lse -inf). Returns (O [n_b, n, H, D], lse [n_b, n, H])."""
    ids = range(len(seq_len)) if batch_ids is None else batch_ids

    def up(a, kind, sc):
        return np.asarray(a, dtype=np.float64) if kind == "f64" else to_f64(a, kind, sc)

    outs, lses = [], []
    for b in ids:
        o0, L = int(seq_off[b]), int(seq_len[b])
        kb = up(k_cache[o0:o0 + L], kind_kv, k_scale)
        vb = up(v_cache[o0:o0 + L], kind_kv, v_scale)
        ob, lb = [], []
        for t in range(n_tokens):
            m = max(0, L - (n_tokens - 1 - t))
            o, lse = attend_one(up(q[b][t], kind_q, None), kb[:m], vb[:m], scale)
            ob.append(o)
            lb.append(lse)
        outs.append(np.stack(ob))
        lses.append(np.stack(lb))
    return np.stack(outs), np.stack(lses)


def paged_rows(block_table_row, n, page_rows):
    """Cache rows of a paged sequence's first n keys: key j sits in block
    j // page_rows, i.e. on page block_table_row[j // page_rows], at row
    page * page_rows + j % page_rows."""
    j = np.arange(int(n), dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[j // page_rows]
    return pages * page_rows + j % page_rows


def decode_attn_paged(q, k_pages, v_pages, block_table, seq_len, page_rows, scale=SOFTMAX_SCALE,
                      kind_q="f64", kind_kv="f64", k_scale=None, v_scale=None, batch_ids=None):
    """decode_attn over a paged cache: each sequence's keys are gathered from
    its pages in block order, then attended exactly as a contiguous run."""
    ids = range(len(seq_len)) if batch_ids is None else batch_ids

    def up(a, kind, sc):
        return np.asarray(a, dtype=np.float64) if kind == "f64" else to_f64(a, kind, sc)

    outs, lses = [], []
    for b in ids:
        rows = paged_rows(block_table[b], seq_len[b], page_rows)
        o, lse = attend_one(up(q[b], kind_q, None), up(k_pages[rows], kind_kv, k_scale),
                            up(v_pages[rows], kind_kv, v_scale), scale)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


def decode_attn_paged_mt(q, k_pages, v_pages, block_table, seq_len, page_rows, n_tokens, scale=SOFTMAX_SCALE,
                         kind_q="f64", kind_kv="f64", k_scale=None, v_scale=None, batch_ids=None):
    """decode_attn_mt over a paged cache: each sequence's keys are gathered from
    its pages in block order (paged_rows), then the tokens attend causally
    exactly as over a contiguous run. Returns (O [n_b, n, H, D], lse [n_b, n, H])."""
    ids = list(range(len(seq_len))) if batch_ids is None else list(batch_ids)
    kc, vc, off, lens = [], [], [], []
    base = 0
    for b in ids:
        rows = paged_rows(block_table[b], seq_len[b], page_rows)
        kc.append(np.asarray(k_pages)[rows])
        vc.append(np.asarray(v_pages)[rows])
        off.append(base)
        lens.append(int(seq_len[b]))
        base += len(rows)
    k_run = np.concatenate(kc) if kc else np.asarray(k_pages)[:0]
    v_run = np.concatenate(vc) if vc else np.asarray(v_pages)[:0]
    qs = [q[b] for b in ids]
    return decode_attn_mt(qs, k_run, v_run, np.asarray(off, dtype=np.int64), np.asarray(lens, dtype=np.int64),
                          n_tokens, scale, kind_q=kind_q, kind_kv=kind_kv, k_scale=k_scale, v_scale=v_scale)


# ------------------------------------------------------------------ output
def out_proj(o, w_o):
    """y = O_flat W_o^T with O flattened head-major ([B, H*D])."""
    o = np.asarray(o, dtype=np.float64)
    return o.reshape(o.shape[0], -1) @ np.asarray(w_o, dtype=np.float64).T


# ------------------------------------------------------------------ whole step
def decode_layer(inp: dict, batch_ids=None, scale=SOFTMAX_SCALE):
    """One decode step of the attention layer from stored inputs.

    q path -> K/V projection of the new token -> append at row off_b + len_b ->
    attention over len_b + 1 rows -> out-projection. ``inp`` holds stored
    tensors with their storage kinds (see the keys used below). Returns a dict
    with c, c_hat, q, k_new, v_new, o, lse and y (float64); with ``batch_ids``
    only those sequences are computed.
    """
    ka, kk = inp["kind_act"], inp["kind_kv"]
    ids = list(range(len(inp["seq_len"]))) if batch_ids is None else list(batch_ids)
    x = to_f64(inp["x"], ka)[ids]
    kw = inp.get("kind_w", ka)
    if kw == "fp8_block":
        w = {n: dequantize_blocks_e4m3fn(inp[n], inp[n + "_scale"]) for n in ("w_dq", "w_uq", "w_k", "w_v", "w_o")}
    else:
        w = {n: to_f64(inp[n], kw) for n in ("w_dq", "w_uq", "w_k", "w_v", "w_o")}
    c, c_hat, q = q_path(x, w["w_dq"], w["w_uq"], inp.get("eps", 1e-6), inp.get("gamma"))
    k_new, v_new = kv_project(x, w["w_k"], w["w_v"])
    ks, vs = inp.get("k_scale"), inp.get("v_scale")
    extra = {}
    if kk == "fp8_e4m3":
        # an e4m3 cache stores the appended rows quantized with the cache's
        # per-tensor scales, and attention reads them back from the cache
        k_codes, v_codes = quantize_e4m3fn(k_new, ks), quantize_e4m3fn(v_new, vs)
        k_app, v_app = decode_e4m3fn(k_codes, ks), decode_e4m3fn(v_codes, vs)
        extra = dict(k_new_codes=k_codes, v_new_codes=v_codes)
    else:
        k_app, v_app = k_new, v_new
    outs, lses = [], []
    for i, b in enumerate(ids):
        o0, n = int(inp["seq_off"][b]), int(inp["seq_len"][b])
        kb = np.concatenate([to_f64(inp["k_cache"][o0:o0 + n], kk, ks), k_app[i:i + 1]])
        vb = np.concatenate([to_f64(inp["v_cache"][o0:o0 + n], kk, vs), v_app[i:i + 1]])
        o, lse = attend_one(q[i], kb, vb, scale)
        outs.append(o)
        lses.append(lse)
    o = np.stack(outs)
    y = out_proj(o, w["w_o"])
    return dict(c=c, c_hat=c_hat, q=q, k_new=k_new, v_new=v_new, o=o, lse=np.stack(lses), y=y, **extra)
