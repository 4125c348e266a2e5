"""CPU oracle for paged MLA decode and sparse fp8 MLA decode.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code, table or constant with it.

What it computes is the plain definition, in float64, with no tiling, no
online softmax and no splitting:

* Multi-head latent attention decode is multi-query attention over one shared
  latent row per cached token: each query head scores the 576-wide row
  (512 latent dims + 64 RoPE dims) and takes a softmax-weighted sum of the
  row's first 512 dims, which serve as V ("[flashinfer] FlashInfer, NVFP4를
  활용한 DeepSeek-V4 디코딩 성능 최적화", section "코드 분석", item 2: a
  latent row per token that is both K and V).
* S = Q K^T, P = softmax(S), O = P V ("FlashMLA-ETAP: Efficient Transpose
  Attention Pipeline ...", section "방법론 / 핵심 메커니즘"), with the scores
  multiplied by ``softmax_scale`` before the softmax.
* The log-sum-exp returned beside O is the natural log of the softmax
  denominator of the scaled scores, in fp32 on the device ("[flashinfer] ...",
  README tensor table: ``lse`` float32, natural log).
* Cached rows live in 64-token pages; logical token t of sequence b is row
  ``t % 64`` of page ``block_table[b][t // 64]`` ("Qu'est-ce que FlashMLA ?",
  section "Installation et utilisation de FlashMLA", step 3;
  "DeepSeek, FlashMLA 오픈소스 공개", summary: 64-token paged KV cache).
* With ``causal`` and s_q > 1 the s_q queries are the sequence's last s_q
  tokens, and query s sees positions <= L - s_q + s ("[flashinfer] ...",
  README: causal mask inside the block against the request's last tokens).
  ``cache_seqlens`` counts those query tokens.  With s_q = 1 causal changes
  nothing.
* Sparse decode: query token (b, s) attends exactly the rows listed in
  ``indices[b, s, :]``; entries equal to -1 are ignored ("deepseek-ai/
  FlashMLA" project summary, section "기술적 세부 사항", indices tensor).  Each
  listed entry is one term (duplicates count twice).  Rows are fp8 e4m3
  values times a per-token scale (same section, KV cache format), decoded
  exactly in float64 from the OCP E4M3FN encoding.
* An empty visible set gives O = 0 and LSE = -inf.
* DeepSeek-V4 decode geometry ("[flashinfer] ...", README): the cached row is 512 wide and is
  both K and V (no RoPE part), and each head may have an attention sink: one more logit in its
  softmax denominator that carries no value.  Reading: the sink is in the units of the scaled
  scores (natural log, not multiplied by softmax_scale), and the returned LSE is the log of the
  whole denominator, sink included; with no visible token O = 0 and LSE = the sink.
* FP4 KV for that geometry ("[flashinfer] ...", README: E2M1 values two per byte, 256 bytes
  per 512-wide row, UE4M3 scales for blocks of 16 values, 32 bytes per row; "deepseek-ai/
  FlashMLA" project summary, "기술적 세부 사항": e2m1 caches).  Readings: element 2j of a row
  is the low nibble of byte j and element 2j+1 the high nibble; scale byte b covers elements
  16b..16b+15; a UE4M3 byte is decoded like an E4M3FN byte (its sign bit is never set by a
  valid cache); there is no further per-tensor scale.  Row value = e2m1 * scale, exactly.

The split-KV combine used by the GPU path is, mathematically, the same
definition evaluated on a partition of the visible set; ``lse_combine`` states
that identity (section "코드 분석", item 3 of the flashinfer page: split-KV
combine kernel) so the tests can check it.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

D_QK = 576
D_V = 512
PAGE = 64
REC_BYTES = 640
SCALE_OFF = 576


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 raw bits -> float64 (exact): a bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3FN byte: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are
    no infinities, so exponent 15 with mantissa 0..6 is an ordinary value
    (largest 448).
    """
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e2m1_value(nibble: int) -> float:
    """Value of one FP4 E2M1 nibble (OCP microscaling FP4): 1 sign, 2 exponent bits (bias 1),
    1 mantissa bit.  Exponent field 0 is subnormal (m/2); there is no infinity or NaN, so the
    largest magnitude is 1.5 * 2^2 = 6.
    """
    sign = -1.0 if nibble & 0x8 else 1.0
    e = (nibble >> 1) & 0x3
    m = nibble & 0x1
    if e == 0:
        return sign * m / 2.0
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


E2M1_TABLE = np.array([e2m1_value(n) for n in range(16)], dtype=np.float64)
FP4_ROW_BYTES = 256      # 512 E2M1 codes, two per byte
FP4_SCALE_BYTES = 32     # one UE4M3 scale per 16 values
FP4_BLOCK = 16


def sparse_rows_f64(kv_records: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Dequantise selected 640-byte records: e4m3(code) * per-token fp32 scale, in float64."""
    rec = np.asarray(kv_records, dtype=np.uint8)[rows]
    vals = E4M3_TABLE[rec[:, :D_QK]]
    scale = np.ascontiguousarray(rec[:, SCALE_OFF:SCALE_OFF + 4]).view("<f4").reshape(-1).astype(np.float64)
    return vals * scale[:, None]


# --------------------------------------------------------------------------
# The attention definition
# --------------------------------------------------------------------------
def attend(q: np.ndarray, rows: np.ndarray, sigma: float,
           sink: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(sigma * q rows^T) rows[:, :512] and its natural-log LSE, for every query row.

    q: [H, D] float64, rows: [T, D] float64 (D = 576, or 512 for the latent-only row that is
    both K and V).  Returns O [H, 512], LSE [H].

    ``sink`` [H] (natural-log logits, or None) is the per-head attention sink of the DeepSeek-V4
    decode geometry ("[flashinfer] ...", README: an optional per-head attention sink): one more
    logit in each head's softmax denominator that carries no value, compared with the scaled
    scores as it is.  LSE is the log of that whole denominator.
    """
    H = q.shape[0]
    T = rows.shape[0]
    if T == 0 and sink is None:
        return np.zeros((H, D_V)), np.full(H, -np.inf)
    z = sigma * (rows @ q.T)                  # [T, H] scaled scores
    m = z.max(axis=0) if T > 0 else np.full(H, -np.inf)    # [H]
    if sink is not None:
        m = np.maximum(m, sink)
    e = np.exp(z - m)                         # [T, H]
    denom = e.sum(axis=0)                     # [H]
    if sink is not None:
        denom = denom + np.exp(sink - m)
    o = (e.T @ rows[:, :D_V]) / denom[:, None]
    return o, m + np.log(denom)


def gather_paged_rows(kcache_bits: np.ndarray, block_table_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """Rows of logical tokens 0..n_tokens-1 of one sequence, gathered through its block table."""
    out = np.empty((n_tokens, kcache_bits.shape[-1]), dtype=np.float64)
    for t in range(0, n_tokens, PAGE):
        page = int(block_table_row[t // PAGE])
        n = min(PAGE, n_tokens - t)
        out[t:t + n] = bf16_to_f64(kcache_bits[page, :n, 0, :])
    return out


def visible_count(L: int, s_q: int, s: int, causal: bool) -> int:
    """Number of leading tokens query s of a length-L sequence sees."""
    if not causal:
        return max(0, L)
    return max(0, min(L, L - s_q + s + 1))


def paged_decode(q_bits: np.ndarray, kcache_bits: np.ndarray, block_table: np.ndarray,
                 seqlens: np.ndarray, softmax_scale: float, causal: bool,
                 batches: Optional[Iterable[int]] = None,
                 sinks: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Paged MLA decode.

    q_bits [B, s_q, h_q, D] bf16 bits; kcache_bits [pages, 64, 1, D] bf16 bits (D = 576, or 512
    for the DeepSeek-V4 latent row that is both K and V); block_table [B, max_blocks] int32;
    seqlens [B] int32; softmax_scale is an fp32 value; sinks [h_q] fp32 or None (see
    ``attend``).  Returns O [B, s_q, h_q, 512] and LSE [B, s_q, h_q] in float64.  With
    ``batches`` only those sequences are computed (the rest stay NaN).
    """
    B, s_q, h_q, _ = q_bits.shape
    sigma = float(np.float32(softmax_scale))
    O = np.full((B, s_q, h_q, D_V), np.nan)
    LSE = np.full((B, s_q, h_q), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seqlens[b])
        rows = gather_paged_rows(kcache_bits, block_table[b], L)
        for s in range(s_q):
            n = visible_count(L, s_q, s, causal)
            O[b, s], LSE[b, s] = attend(bf16_to_f64(q_bits[b, s]), rows[:n], sigma,
                                        None if sinks is None else np.asarray(sinks, dtype=np.float32).astype(np.float64))
    return O, LSE


def gather_paged_records(kcache_records: np.ndarray, block_table_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """Dequantised rows of logical tokens 0..n_tokens-1 of one sequence from an fp8 paged cache
    ([pages, 64, 640] records), gathered through its block table."""
    out = np.empty((n_tokens, D_QK), dtype=np.float64)
    for t in range(0, n_tokens, PAGE):
        page = int(block_table_row[t // PAGE])
        n = min(PAGE, n_tokens - t)
        out[t:t + n] = sparse_rows_f64(kcache_records[page], np.arange(n))
    return out


def paged_decode_fp8(q_bits: np.ndarray, kcache_records: np.ndarray, block_table: np.ndarray,
                     seqlens: np.ndarray, softmax_scale: float, causal: bool,
                     batches: Optional[Iterable[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Paged MLA decode over an fp8 cache: 64-token pages of 640-byte records (e4m3 codes of the
    576 dims and the token's fp32 scale), the fp8 KV cache layout of the decode path
    ("deepseek-ai/FlashMLA" project summary, sections "사용 방법" step 3 and "기술적 세부 사항").
    Row value = e4m3(code) * scale, exactly; otherwise the definition of ``paged_decode``.

    kcache_records [pages, 64, 640] uint8.  Returns O [B, s_q, h_q, 512] and LSE [B, s_q, h_q]
    in float64 (sequences outside ``batches`` stay NaN).
    """
    B, s_q, h_q, _ = q_bits.shape
    sigma = float(np.float32(softmax_scale))
    O = np.full((B, s_q, h_q, D_V), np.nan)
    LSE = np.full((B, s_q, h_q), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seqlens[b])
        rows = gather_paged_records(kcache_records, block_table[b], L)
        for s in range(s_q):
            n = visible_count(L, s_q, s, causal)
            O[b, s], LSE[b, s] = attend(bf16_to_f64(q_bits[b, s]), rows[:n], sigma)
    return O, LSE


def fp4_rows_f64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantise FP4 rows: codes [N, 256] uint8 (two E2M1 values per byte, low nibble first),
    scales [N, 32] uint8 (UE4M3, one per block of 16 values).  Returns [N, 512] float64 with
    value = e2m1(code) * scale of its block, exactly.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n = codes.shape[0]
    vals = np.empty((n, 2 * codes.shape[1]), dtype=np.float64)
    vals[:, 0::2] = E2M1_TABLE[codes & 0x0F]
    vals[:, 1::2] = E2M1_TABLE[codes >> 4]
    block_scale = E4M3_TABLE[scales]                               # [N, 32]
    return vals * np.repeat(block_scale, FP4_BLOCK, axis=1)


def gather_paged_fp4(kv_codes: np.ndarray, kv_scales: np.ndarray, block_table_row: np.ndarray,
                     n_tokens: int) -> np.ndarray:
    """Dequantised 512-wide rows of logical tokens 0..n_tokens-1 of one sequence from an FP4
    paged cache (codes [pages, 64, 256], scales [pages, 64, 32]), through its block table."""
    out = np.empty((n_tokens, D_V), dtype=np.float64)
    for t in range(0, n_tokens, PAGE):
        page = int(block_table_row[t // PAGE])
        n = min(PAGE, n_tokens - t)
        out[t:t + n] = fp4_rows_f64(kv_codes[page, :n], kv_scales[page, :n])
    return out


def paged_decode_fp4(q_bits: np.ndarray, kv_codes: np.ndarray, kv_scales: np.ndarray,
                     block_table: np.ndarray, seqlens: np.ndarray, softmax_scale: float,
                     causal: bool, batches: Optional[Iterable[int]] = None,
                     sinks: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """DeepSeek-V4 decode geometry over an FP4 paged cache ("[flashinfer] ...", README tensor
    table: ``kv_cache [num_pages, 64, 256]`` packed E2M1 and ``kv_scale [num_pages, 64, 32]``
    UE4M3): each token's dequantised 512-wide row is both K and V; otherwise the definition of
    ``paged_decode`` (causal rule, optional per-head sinks).  q_bits [B, s_q, h_q, 512] bf16 bits.
    Returns O [B, s_q, h_q, 512] and LSE [B, s_q, h_q] in float64 (sequences outside
    ``batches`` stay NaN).
    """
    B, s_q, h_q, _ = q_bits.shape
    sigma = float(np.float32(softmax_scale))
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float32).astype(np.float64)
    O = np.full((B, s_q, h_q, D_V), np.nan)
    LSE = np.full((B, s_q, h_q), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seqlens[b])
        rows = gather_paged_fp4(kv_codes, kv_scales, block_table[b], L)
        for s in range(s_q):
            n = visible_count(L, s_q, s, causal)
            O[b, s], LSE[b, s] = attend(bf16_to_f64(q_bits[b, s]), rows[:n], sigma, sk)
    return O, LSE


def sparse_decode(q_bits: np.ndarray, kv_records: np.ndarray, indices: np.ndarray,
                  softmax_scale: float,
                  sets: Optional[Iterable[Tuple[int, int]]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Sparse fp8 MLA decode.

    q_bits [B, s_q, h_q, 576] bf16 bits; kv_records [N, 640] uint8;
    indices [B, s_q, topk] int32 with -1 = ignore.  Returns O [B, s_q, h_q, 512]
    and LSE [B, s_q, h_q] in float64.  With ``sets`` only those (b, s) are
    computed (the rest stay NaN).
    """
    B, s_q, h_q, _ = q_bits.shape
    sigma = float(np.float32(softmax_scale))
    O = np.full((B, s_q, h_q, D_V), np.nan)
    LSE = np.full((B, s_q, h_q), np.nan)
    todo = [(b, s) for b in range(B) for s in range(s_q)] if sets is None else list(sets)
    for b, s in todo:
        entries = indices[b, s]
        listed = entries[entries != -1].astype(np.int64)
        rows = sparse_rows_f64(kv_records, listed)
        O[b, s], LSE[b, s] = attend(bf16_to_f64(q_bits[b, s]), rows, sigma)
    return O, LSE


def lse_combine(parts_o: np.ndarray, parts_lse: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Merge attention results over disjoint token subsets into the result over their union.

    parts_o [n, H, 512], parts_lse [n, H] (natural log, -inf for an empty part).
    The union's denominator is the sum of the parts' denominators, so
    LSE = log sum_i exp(LSE_i) and O = sum_i exp(LSE_i - LSE) O_i.  All parts
    empty gives O = 0, LSE = -inf.
    """
    parts_o = np.asarray(parts_o, dtype=np.float64)
    parts_lse = np.asarray(parts_lse, dtype=np.float64)
    mu = parts_lse.max(axis=0)                                   # [H]
    safe_mu = np.where(np.isfinite(mu), mu, 0.0)
    w = np.where(np.isfinite(parts_lse), np.exp(parts_lse - safe_mu), 0.0)   # [n, H]
    tot = w.sum(axis=0)
    o = np.where(tot[:, None] > 0, (w[:, :, None] * parts_o).sum(axis=0) / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    lse = np.where(tot > 0, safe_mu + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return o, lse


# --------------------------------------------------------------------------
# Fused decode: Q-norm, RoPE, attention, conjugate RoPE on the output, FP8 cast
# ("deepseek-ai/FlashMLA" project summary, 개요 bullet 3 and 사용 방법 step 5: one kernel merges
# the query norm, rotary position encoding, the attention, the conjugate rotary encoding on the
# output side and the final cast to FP8 for the FP8 einsum that follows).  The pages name the
# stages only; the readings taken here:
#   * the geometry is the DeepSeek-V4 decode one: a 512-wide latent row per token that is both K
#     and V, whose last 64 dims carry the rotary encoding of the token's position;
#   * Q-norm is an RMS norm over each head's 512 query dims with one weight vector shared by the
#     heads: q * weight / sqrt(mean(q^2) + eps);
#   * RoPE rotates the interleaved pairs (448 + 2i, 449 + 2i), i < 32, by the query token's angle
#     theta_i, given as cos/sin per query token; the conjugate RoPE rotates the same pairs of the
#     attention output by -theta_i of the same token, which turns the cached rows' absolute
#     rotations into rotations relative to the query;
#   * the cast writes OCP E4M3FN codes with one fp32 scale per (token, head) row:
#     scale = max(amax, 2^-126) / 448, code = round-to-nearest-even of x / scale (in fp32);
#   * the attention takes its query as a bf16 operand, as every query the decode calls take: the
#     normed, rotated query is rounded to bf16 (nearest even) before it scores the rows.
# --------------------------------------------------------------------------
ROPE_DIMS = 64
ROPE_START = D_V - ROPE_DIMS
E4M3_MAX = 448.0


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """x [..., D] float64 -> x * weight / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * np.asarray(weight, dtype=np.float64) / np.sqrt(ms + float(eps))


def rope_rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, sign: float = 1.0) -> np.ndarray:
    """Rotate the interleaved pairs (448 + 2i, 449 + 2i) of the last axis of x [..., 512] by the
    angle whose cosine and sine are cos[..., i], sin[..., i] (i < 32; sign = -1: by minus the
    angle, the conjugate rotation).  Other dims are unchanged."""
    x = np.array(x, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = sign * np.asarray(sin, dtype=np.float64)
    a = x[..., ROPE_START::2].copy()
    b = x[..., ROPE_START + 1::2].copy()
    x[..., ROPE_START::2] = a * c - b * s
    x[..., ROPE_START + 1::2] = a * s + b * c
    return x


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes of x (float32 values): round to the nearest finite E4M3 value, ties to
    the even code, the sign bit kept (negative values that round to zero give -0); magnitudes
    beyond 448 saturate to 448 (the cast's inputs lie within it)."""
    x = np.asarray(x, dtype=np.float64)
    pos = E4M3_TABLE[:0x7F]                          # codes 0x00..0x7E: 0 .. 448, increasing
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(pos, mag, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - pos[lo]
    d_hi = pos[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def fp8_cast_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row FP8 cast of x [..., 512]: (codes uint8 [..., 512], scale float32 [...]) with
    scale = fp32(max(amax, 2^-126) / 448) and code = e4m3_encode(fp32(fp32(x) / scale))."""
    xf = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.abs(xf).max(axis=-1)
    scale = (np.maximum(amax, np.float32(2.0 ** -126)) / np.float32(E4M3_MAX)).astype(np.float32)
    y = (xf / scale[..., None]).astype(np.float32)
    return e4m3_encode(y), scale


def round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest bf16 value (ties to even), via fp32: a bf16 is the top half of an
    fp32, so the low 16 bits are rounded away."""
    bits = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16 << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def fused_decode(q_bits: np.ndarray, norm_weight: np.ndarray, norm_eps: float, rope_cs: np.ndarray,
                 rows_of, block_table: np.ndarray, seqlens: np.ndarray, softmax_scale: float,
                 causal: bool, sinks: Optional[np.ndarray] = None, round_query: bool = True):
    """The fused decode on the DeepSeek-V4 geometry.

    q_bits [B, s_q, h_q, 512] bf16 bits: the query before its norm and rotation;
    norm_weight [512] fp32; rope_cs [B, s_q, 64] fp32: cos(theta_i) for i < 32, then sin(theta_i),
    of each query token; rows_of(b, L) -> the float64 [L, 512] rows of sequence b's first L tokens
    (bf16 or FP4 pages, gathered through the block table); sinks [h_q] or None.
    Steps: q' = RoPE(RMSNorm(q)), rounded to bf16 (round_query); O, LSE = attention of q' over
    the visible rows (the paged definition, causal rule and sinks included); O' = conjugate
    RoPE(O); codes, scale = the FP8 cast of O'.  Returns (codes uint8 [B, s_q, h_q, 512], scale fp32 [B, s_q, h_q],
    LSE float64 [B, s_q, h_q], O' float64 [B, s_q, h_q, 512]).
    """
    B, s_q, h_q, _ = q_bits.shape
    sigma = float(np.float32(softmax_scale))
    w = np.asarray(norm_weight, dtype=np.float32).astype(np.float64)
    eps = float(np.float32(norm_eps))
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float32).astype(np.float64)
    cs = np.asarray(rope_cs, dtype=np.float32).astype(np.float64)
    O = np.zeros((B, s_q, h_q, D_V))
    LSE = np.zeros((B, s_q, h_q))
    for b in range(B):
        L = int(seqlens[b])
        rows = rows_of(b, L)
        for s in range(s_q):
            n = visible_count(L, s_q, s, causal)
            cos, sin = cs[b, s, :ROPE_DIMS // 2], cs[b, s, ROPE_DIMS // 2:]
            q = rope_rotate(rms_norm(bf16_to_f64(q_bits[b, s]), w, eps), cos, sin)
            if round_query:
                q = round_bf16(q)
            o, lse = attend(q, rows[:n], sigma, sk)
            O[b, s] = rope_rotate(o, cos, sin, sign=-1.0)
            LSE[b, s] = lse
    codes, scale = fp8_cast_rows(O)
    return codes, scale, LSE, O
