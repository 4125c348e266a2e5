"""Seeded input generators for paged and sparse MLA decode.

Shapes follow the decode contract the pages describe: a query tensor
``[batch, s_q, h_q, 576]`` in bf16, a paged latent cache of 64-token pages
``[num_pages, 64, 1, 576]`` in bf16 addressed by a per-sequence
``block_table`` and ``cache_seqlens`` ("Qu'est-ce que FlashMLA ?", section
"Installation et utilisation de FlashMLA", steps 2-3; "DeepSeek, FlashMLA
오픈소스 공개", summary: BF16, 64-token pages), and for the sparse variant an
fp8-e4m3 cache with one scale per token plus a ``[batch, s_q, topk]`` index
tensor where -1 marks an unused entry ("deepseek-ai/FlashMLA" project
summary, section "기술적 세부 사항").

Everything here is input preparation: random draws, page permutations, index
lists, rounding drawn fp32 values to bf16 and quantising the sparse cache to
fp8.  No attention arithmetic lives here.

Draw order for one input set (one ``numpy.random.Generator(PCG64(seed))``):
sequence lengths, block-table permutation, Q, KV, sparse indices, -1 mask.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Union

import numpy as np

D_QK = 576          # latent (512) + RoPE (64) dims of one cached row
D_V = 512           # value dims: the first 512 dims of the same row
PAGE = 64           # tokens per page
REC_BYTES = 640     # sparse fp8 record: 576 e4m3 codes, fp32 scale, zero pad
SCALE_OFF = 576     # byte offset of the fp32 scale inside a record
BF16_NAN = 0x7FC0

_KV_CHUNK_ROWS = 65536


# --------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# --------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to fp32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) fp32 draws rounded to bf16 bits, drawn in row chunks of the leading dims."""
    shape = tuple(int(s) for s in shape)
    n_rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    width = shape[-1]
    out = np.empty((n_rows, width), dtype=np.uint16)
    for r0 in range(0, n_rows, _KV_CHUNK_ROWS):
        r1 = min(n_rows, r0 + _KV_CHUNK_ROWS)
        out[r0:r1] = bf16_bits_from_f32(rng.standard_normal((r1 - r0, width), dtype=np.float32))
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Paged inputs
# --------------------------------------------------------------------------
@dataclasses.dataclass
class PagedInputs:
    q: np.ndarray               # uint16 bf16 bits [batch, s_q, h_q, 576]
    kcache: np.ndarray          # uint16 bf16 bits [num_pages, 64, 1, 576]
    block_table: np.ndarray     # int32 [batch, max_blocks]
    seqlens: np.ndarray         # int32 [batch]
    s_q: int
    h_q: int
    causal: bool
    softmax_scale: float        # an fp32 value, stored as a Python float
    poison_page: int            # index of the all-NaN page, or -1
    sinks: Optional[np.ndarray] = None   # fp32 [h_q] per-head attention sinks, or None

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.kcache.shape[0])

    @property
    def d_qk(self) -> int:
        return int(self.kcache.shape[-1])


def _fp32(x: float) -> float:
    return float(np.float32(x))


def make_paged(batch: int, s_q: int, h_q: int,
               seqlens: Union[Sequence[int], tuple],
               causal: bool, seed: int, poison: bool = True,
               softmax_scale: Optional[float] = None,
               d_qk: int = D_QK, sinks: bool = False) -> PagedInputs:
    """Draw one paged decode input set.

    ``seqlens`` is either an explicit list of ``batch`` lengths or
    ``("uniform", lo, hi)`` for integer lengths drawn uniformly in [lo, hi].
    The page pool is the exact fit sum(ceil(L/64)); its pages are handed out
    in a random permutation, in order per sequence.  With ``poison`` an extra
    all-NaN page is appended, every unused block-table slot points at it, and
    the rows past each sequence's end inside its last page are set to NaN, so
    any read outside the visible tokens shows up in the result.

    ``d_qk = 512`` draws the DeepSeek-V4 geometry's latent-only rows (both K and V, no RoPE
    part; "[flashinfer] ...", README), with the default scale 512^-0.5.  ``sinks`` draws one
    attention-sink logit per head after everything else, ln(mean L) + U[-2, 2], so that a sink
    and the cached tokens carry comparable weight.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if isinstance(seqlens, tuple) and len(seqlens) == 3 and seqlens[0] == "uniform":
        L = rng.integers(int(seqlens[1]), int(seqlens[2]) + 1, size=batch).astype(np.int32)
    else:
        L = np.asarray(seqlens, dtype=np.int32)
        if L.shape != (batch,):
            raise ValueError("seqlens must have one entry per sequence")
    if (L < 0).any():
        raise ValueError("sequence lengths must be >= 0")
    if d_qk not in (D_QK, D_V):
        raise ValueError("d_qk must be 576 or 512")
    nblk = (L.astype(np.int64) + PAGE - 1) // PAGE
    total = int(nblk.sum())
    max_blocks = max(1, int(nblk.max()) if batch else 1)
    perm = rng.permutation(total).astype(np.int32)
    fill = total if poison else 0
    bt = np.full((batch, max_blocks), fill, dtype=np.int32)
    off = 0
    for b in range(batch):
        n = int(nblk[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    q = _normal_bf16(rng, (batch, s_q, h_q, d_qk))
    kc = _normal_bf16(rng, (total, PAGE, 1, d_qk))
    poison_page = -1
    if poison:
        kc = np.concatenate([kc, np.full((1, PAGE, 1, d_qk), BF16_NAN, dtype=np.uint16)], axis=0)
        poison_page = total
        for b in range(batch):
            if L[b] % PAGE:
                kc[bt[b, L[b] // PAGE], L[b] % PAGE:, 0, :] = BF16_NAN
    scale = _fp32(d_qk ** -0.5 if softmax_scale is None else softmax_scale)
    sk = None
    if sinks:
        sk = (np.log(max(1.0, float(L.mean()) if batch else 1.0)) +
              rng.uniform(-2.0, 2.0, size=h_q)).astype(np.float32)
    return PagedInputs(q=q, kcache=kc, block_table=bt, seqlens=L, s_q=s_q, h_q=h_q,
                       causal=bool(causal), softmax_scale=scale, poison_page=poison_page, sinks=sk)


@dataclasses.dataclass
class PagedFp8Inputs:
    q: np.ndarray               # uint16 bf16 bits [batch, s_q, h_q, 576]
    kcache: np.ndarray          # uint8 [num_pages, 64, 640] fp8 records (codes, scale, pad)
    block_table: np.ndarray     # int32 [batch, max_blocks]
    seqlens: np.ndarray         # int32 [batch]
    s_q: int
    h_q: int
    causal: bool
    softmax_scale: float        # an fp32 value, stored as a Python float
    poison_page: int            # index of the all-NaN page, or -1

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.kcache.shape[0])


def make_paged_fp8(batch: int, s_q: int, h_q: int,
                   seqlens: Union[Sequence[int], tuple],
                   causal: bool, seed: int, poison: bool = True,
                   softmax_scale: Optional[float] = None) -> PagedFp8Inputs:
    """Draw one paged decode input set over an fp8 cache.

    Same draws and page permutation as ``make_paged``; the cached rows are
    drawn in fp32 and quantised per token into 640-byte records (e4m3 codes
    and an fp32 scale, as for the sparse cache), stored in 64-token pages:
    the fp8 KV cache layout of the decode path ("deepseek-ai/FlashMLA"
    project summary, sections "사용 방법" step 3 and "기술적 세부 사항").
    Poisoned records (unused pages, rows past a sequence's end) hold NaN codes
    and a NaN scale.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if isinstance(seqlens, tuple) and len(seqlens) == 3 and seqlens[0] == "uniform":
        L = rng.integers(int(seqlens[1]), int(seqlens[2]) + 1, size=batch).astype(np.int32)
    else:
        L = np.asarray(seqlens, dtype=np.int32)
        if L.shape != (batch,):
            raise ValueError("seqlens must have one entry per sequence")
    if (L < 0).any():
        raise ValueError("sequence lengths must be >= 0")
    nblk = (L.astype(np.int64) + PAGE - 1) // PAGE
    total = int(nblk.sum())
    max_blocks = max(1, int(nblk.max()) if batch else 1)
    perm = rng.permutation(total).astype(np.int32)
    fill = total if poison else 0
    bt = np.full((batch, max_blocks), fill, dtype=np.int32)
    off = 0
    for b in range(batch):
        n = int(nblk[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    q = _normal_bf16(rng, (batch, s_q, h_q, D_QK))
    n_rows = total * PAGE
    kc = np.empty((n_rows, REC_BYTES), dtype=np.uint8)
    for r0 in range(0, n_rows, _KV_CHUNK_ROWS):
        r1 = min(n_rows, r0 + _KV_CHUNK_ROWS)
        kc[r0:r1] = quantize_rows_e4m3(rng.standard_normal((r1 - r0, D_QK), dtype=np.float32))
    kc = kc.reshape(total, PAGE, REC_BYTES)
    poison_page = -1
    if poison:
        bad = np.zeros((PAGE, REC_BYTES), dtype=np.uint8)
        bad[:, :D_QK] = 0x7F
        bad[:, SCALE_OFF:SCALE_OFF + 4] = np.full(PAGE, np.nan, dtype="<f4").view(np.uint8).reshape(PAGE, 4)
        kc = np.concatenate([kc, bad[None]], axis=0)
        poison_page = total
        for b in range(batch):
            if L[b] % PAGE:
                kc[bt[b, L[b] // PAGE], L[b] % PAGE:] = bad[L[b] % PAGE:]
    scale = _fp32(D_QK ** -0.5 if softmax_scale is None else softmax_scale)
    return PagedFp8Inputs(q=q, kcache=kc, block_table=bt, seqlens=L, s_q=s_q, h_q=h_q,
                          causal=bool(causal), softmax_scale=scale, poison_page=poison_page)


# --------------------------------------------------------------------------
# FP4 (E2M1) paged inputs, DeepSeek-V4 geometry
# --------------------------------------------------------------------------
FP4_ROW_BYTES = 256     # 512 E2M1 codes, two per byte (low nibble = even element)
FP4_SCALE_BYTES = 32    # one UE4M3 scale byte per block of 16 values
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def quantize_rows_nvfp4(x: np.ndarray):
    """Block-16 FP4 quantisation of 512-wide rows: (codes [N, 256] uint8, scales [N, 32] uint8).

    Per block of 16 values: scale = amax / 6 cast to E4M3 (torch ``float8_e4m3fn``, nearest-even;
    always non-negative, so it is a UE4M3 byte); each value divided by the cast scale is
    clamped to +-6 and replaced by the nearest E2M1 magnitude (ties to the smaller one) with
    its sign; an all-zero block gets scale 0 and zero codes.  Element 2j goes to the low
    nibble of byte j, element 2j+1 to the high nibble.
    """
    import torch  # local import: only the fp8/fp4 generators need torch's e4m3 cast

    x = np.ascontiguousarray(x, dtype=np.float32)
    n, d = x.shape
    if d % 32:
        raise ValueError("row width must be a multiple of 32")
    blk = x.reshape(n, d // 16, 16)
    amax = np.abs(blk).max(axis=2)
    sc8 = torch.from_numpy((amax / np.float32(6.0)).astype(np.float32)).to(torch.float8_e4m3fn)
    scales = sc8.view(torch.uint8).numpy().copy()
    sval = sc8.to(torch.float32).numpy()
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(sval[:, :, None] > 0, blk / sval[:, :, None], np.float32(0.0))
    y = np.clip(y, np.float32(-6.0), np.float32(6.0))
    mag = np.abs(y)
    idx = np.argmin(np.abs(mag[..., None] - _E2M1_GRID), axis=-1).astype(np.uint8)
    nib = idx | np.where((y < 0) & (idx > 0), np.uint8(8), np.uint8(0)).astype(np.uint8)
    nib = nib.reshape(n, d)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return codes, scales


@dataclasses.dataclass
class PagedFp4Inputs:
    q: np.ndarray               # uint16 bf16 bits [batch, s_q, h_q, 512]
    kv_codes: np.ndarray        # uint8 [num_pages, 64, 256] packed E2M1
    kv_scales: np.ndarray       # uint8 [num_pages, 64, 32] UE4M3 block-16 scales
    block_table: np.ndarray     # int32 [batch, max_blocks]
    seqlens: np.ndarray         # int32 [batch]
    s_q: int
    h_q: int
    causal: bool
    softmax_scale: float        # an fp32 value, stored as a Python float
    poison_page: int            # index of the poisoned page, or -1
    sinks: Optional[np.ndarray] = None   # fp32 [h_q], or None

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.kv_codes.shape[0])


def make_paged_fp4(batch: int, s_q: int, h_q: int,
                   seqlens: Union[Sequence[int], tuple],
                   causal: bool, seed: int, poison: bool = True,
                   softmax_scale: Optional[float] = None, sinks: bool = False) -> PagedFp4Inputs:
    """Draw one DeepSeek-V4-geometry decode input set over an FP4 paged cache.

    Same draws and page permutation as ``make_paged`` with ``d_qk = 512``; the latent rows are
    drawn in fp32 and quantised by ``quantize_rows_nvfp4`` into the FP4 cache tensors of the
    V4 decode call ("[flashinfer] ...", README tensor table: ``kv_cache [num_pages, 64, 256]``,
    ``kv_scale [num_pages, 64, 32]``).  The query stays bf16.  Poisoned rows (unused pages,
    rows past a sequence's end) hold NaN scale bytes (0x7F), so any read of them shows up.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if isinstance(seqlens, tuple) and len(seqlens) == 3 and seqlens[0] == "uniform":
        L = rng.integers(int(seqlens[1]), int(seqlens[2]) + 1, size=batch).astype(np.int32)
    else:
        L = np.asarray(seqlens, dtype=np.int32)
        if L.shape != (batch,):
            raise ValueError("seqlens must have one entry per sequence")
    if (L < 0).any():
        raise ValueError("sequence lengths must be >= 0")
    nblk = (L.astype(np.int64) + PAGE - 1) // PAGE
    total = int(nblk.sum())
    max_blocks = max(1, int(nblk.max()) if batch else 1)
    perm = rng.permutation(total).astype(np.int32)
    fill = total if poison else 0
    bt = np.full((batch, max_blocks), fill, dtype=np.int32)
    off = 0
    for b in range(batch):
        n = int(nblk[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    q = _normal_bf16(rng, (batch, s_q, h_q, D_V))
    n_rows = total * PAGE
    codes = np.empty((n_rows, FP4_ROW_BYTES), dtype=np.uint8)
    scales = np.empty((n_rows, FP4_SCALE_BYTES), dtype=np.uint8)
    for r0 in range(0, n_rows, _KV_CHUNK_ROWS):
        r1 = min(n_rows, r0 + _KV_CHUNK_ROWS)
        codes[r0:r1], scales[r0:r1] = quantize_rows_nvfp4(rng.standard_normal((r1 - r0, D_V), dtype=np.float32))
    codes = codes.reshape(total, PAGE, FP4_ROW_BYTES)
    scales = scales.reshape(total, PAGE, FP4_SCALE_BYTES)
    poison_page = -1
    if poison:
        codes = np.concatenate([codes, np.full((1, PAGE, FP4_ROW_BYTES), 0x77, dtype=np.uint8)], axis=0)
        scales = np.concatenate([scales, np.full((1, PAGE, FP4_SCALE_BYTES), 0x7F, dtype=np.uint8)], axis=0)
        poison_page = total
        for b in range(batch):
            if L[b] % PAGE:
                scales[bt[b, L[b] // PAGE], L[b] % PAGE:] = 0x7F
    scale = _fp32(D_V ** -0.5 if softmax_scale is None else softmax_scale)
    sk = None
    if sinks:
        sk = (np.log(max(1.0, float(L.mean()) if batch else 1.0)) +
              rng.uniform(-2.0, 2.0, size=h_q)).astype(np.float32)
    return PagedFp4Inputs(q=q, kv_codes=codes, kv_scales=scales, block_table=bt, seqlens=L, s_q=s_q,
                          h_q=h_q, causal=bool(causal), softmax_scale=scale, poison_page=poison_page,
                          sinks=sk)


# --------------------------------------------------------------------------
# Fused-decode inputs (Q-norm weight, RoPE angles) on the V4 geometry
# --------------------------------------------------------------------------
@dataclasses.dataclass
class FusedExtras:
    norm_weight: np.ndarray      # fp32 [512]: the query RMS-norm weight, shared by the heads
    norm_eps: float              # an fp32 value
    rope_cs: np.ndarray          # fp32 [batch, s_q, 64]: cos(theta_i) for i < 32, then sin(theta_i)
    positions: np.ndarray        # int64 [batch, s_q]: the query tokens' positions (L - s_q + s)


ROPE_BASE = 10000.0


def rope_angles(positions: np.ndarray, base: float = ROPE_BASE) -> np.ndarray:
    """cos/sin [..., 64] (fp32) of the rotary angles pos * base^(-2i/64), i < 32, for integer
    positions: the per-token angle table a caller hands to the fused decode."""
    pos = np.asarray(positions, dtype=np.float64)[..., None]
    inv_freq = base ** (-np.arange(0, 64, 2, dtype=np.float64) / 64.0)
    ang = pos * inv_freq
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def make_fused_extras(inp, seed: int, eps: float = 1e-6) -> FusedExtras:
    """The fused decode's extra inputs for a V4-geometry input set (bf16 or FP4 pages): a norm
    weight 1 + 0.1 N(0,1) (fp32) and the angles of the query tokens, which are the last s_q
    tokens of each sequence (position L - s_q + s, at least 0)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = (1.0 + 0.1 * rng.standard_normal(D_V)).astype(np.float32)
    L = inp.seqlens.astype(np.int64)
    pos = np.maximum(L[:, None] - inp.s_q + np.arange(inp.s_q)[None, :], 0)
    return FusedExtras(norm_weight=w, norm_eps=_fp32(eps), rope_cs=rope_angles(pos), positions=pos)


# --------------------------------------------------------------------------
# Sparse fp8 inputs
# --------------------------------------------------------------------------
@dataclasses.dataclass
class SparseInputs:
    q: np.ndarray               # uint16 bf16 bits [batch, s_q, h_q, 576]
    kv: np.ndarray              # uint8 [num_tokens, 640] records
    indices: np.ndarray         # int32 [batch, s_q, topk], -1 = unused entry
    h_q: int
    softmax_scale: float

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def s_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[2])

    @property
    def num_tokens(self) -> int:
        return int(self.kv.shape[0])


def quantize_rows_e4m3(x: np.ndarray) -> np.ndarray:
    """Per-row fp8-e4m3 quantisation into 640-byte records.

    scale = max(amax|row|, 2^-126) / 448 in fp32; codes are x / scale rounded
    to nearest-even e4m3 (OCP E4M3FN, the torch ``float8_e4m3fn`` cast) after
    clamping to +-448.  Record bytes: [0, 576) codes, [576, 580) scale as
    little-endian fp32, [580, 640) zero.
    """
    import torch  # local import: only the sparse generator needs torch's fp8 cast

    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[0]
    amax = np.abs(x).max(axis=1)
    scale = (np.maximum(amax, np.float32(2.0 ** -126)) / np.float32(448.0)).astype(np.float32)
    y = np.clip(x / scale[:, None], np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    rec = np.zeros((n, REC_BYTES), dtype=np.uint8)
    rec[:, :D_QK] = codes
    rec[:, SCALE_OFF:SCALE_OFF + 4] = scale.astype("<f4").view(np.uint8).reshape(n, 4)
    return rec


def make_sparse(batch: int, s_q: int, h_q: int, tokens_per_seq: int, topk: int,
                p_invalid: float, seed: int,
                softmax_scale: Optional[float] = None) -> SparseInputs:
    """Draw one sparse fp8 decode input set.

    The KV pool holds ``batch * tokens_per_seq`` tokens; sequence b owns rows
    [b*tokens_per_seq, (b+1)*tokens_per_seq).  Query token s of sequence b
    draws ``topk`` distinct positions from [0, tokens_per_seq - s_q + s]
    (its causal window), in random order, mapped to global rows; then each
    entry independently becomes -1 with probability ``p_invalid``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal_bf16(rng, (batch, s_q, h_q, D_QK))
    n_tok = batch * tokens_per_seq
    kv = np.empty((n_tok, REC_BYTES), dtype=np.uint8)
    for r0 in range(0, n_tok, _KV_CHUNK_ROWS):
        r1 = min(n_tok, r0 + _KV_CHUNK_ROWS)
        kv[r0:r1] = quantize_rows_e4m3(rng.standard_normal((r1 - r0, D_QK), dtype=np.float32))
    idx = np.empty((batch, s_q, topk), dtype=np.int32)
    for b in range(batch):
        for s in range(s_q):
            window = tokens_per_seq - s_q + s + 1
            if topk > window:
                raise ValueError("topk exceeds the causal window")
            idx[b, s] = rng.choice(window, size=topk, replace=False).astype(np.int32) + b * tokens_per_seq
    if p_invalid > 0:
        idx[rng.random((batch, s_q, topk)) < p_invalid] = -1
    scale = _fp32(D_QK ** -0.5 if softmax_scale is None else softmax_scale)
    return SparseInputs(q=q, kv=kv, indices=idx, h_q=h_q, softmax_scale=scale)


# --------------------------------------------------------------------------
# The named workloads
# --------------------------------------------------------------------------
CONFIGS = {
    1: dict(kind="paged", name="tiny paged decode: b=2 s_q=1 h_q=16 L={37,130}",
            batch=2, s_q=1, h_q=16, seqlens=[37, 130], causal=False),
    2: dict(kind="paged", name="memory-bound paged decode: b=128 s_q=1 h_q=16 L=4096",
            batch=128, s_q=1, h_q=16, seqlens=[4096] * 128, causal=False),
    3: dict(kind="paged", name="compute-bound varlen paged decode: b=128 s_q=2 causal h_q=128 L~U[1024,8192]",
            batch=128, s_q=2, h_q=128, seqlens=("uniform", 1024, 8192), causal=True),
    4: dict(kind="paged", name="long-context split-KV paged decode: b=16 s_q=1 h_q=16 L=65536",
            batch=16, s_q=1, h_q=16, seqlens=[65536] * 16, causal=False),
    5: dict(kind="sparse", name="sparse fp8 decode: b=32 s_q=6 h_q=64 topk=2048 pool=32768/seq p(-1)=0.05",
            batch=32, s_q=6, h_q=64, tokens_per_seq=32768, topk=2048, p_invalid=0.05),
    # fp8 KV cache for the dense paged path: the memory-bound shape over 640-byte records
    6: dict(kind="paged_fp8", name="memory-bound paged decode, fp8 KV: b=128 s_q=1 h_q=16 L=4096",
            batch=128, s_q=1, h_q=16, seqlens=[4096] * 128, causal=False),
    # DeepSeek-V4 decode geometry: 512-wide latent rows that are K and V, six causal query
    # tokens per request, 64 heads, per-head attention sinks
    7: dict(kind="paged_v4", name="V4-geometry paged decode: b=64 s_q=6 causal h_q=64 L=4096 d=512 + sinks",
            batch=64, s_q=6, h_q=64, seqlens=[4096] * 64, causal=True),
    # the same geometry over an FP4 cache (E2M1 codes, UE4M3 block-16 scales)
    8: dict(kind="paged_v4_fp4", name="V4-geometry paged decode, FP4 KV: b=64 s_q=6 causal h_q=64 L=4096 d=512 + sinks",
            batch=64, s_q=6, h_q=64, seqlens=[4096] * 64, causal=True),
    # sparse prefill: a 4096-token prompt chunk at the end of a 32768-token context, every query
    # token with its own 2048-entry index list in its causal window
    9: dict(kind="sparse_prefill", name="sparse fp8 prefill: s_q=4096 h_q=128 topk=2048 context=32768",
            batch=1, s_q=4096, h_q=128, tokens_per_seq=32768, topk=2048, p_invalid=0.0),
    # the fused decode (query RMS norm, RoPE, attention, conjugate RoPE on the output, FP8 cast)
    # on the V4 geometry, over bf16 pages
    10: dict(kind="fused_v4", name="fused norm-RoPE-attn-RoPE-FP8 decode: b=64 s_q=6 causal h_q=64 L=4096 d=512 + sinks",
             batch=64, s_q=6, h_q=64, seqlens=[4096] * 64, causal=True),
}


def config_info(k: int) -> dict:
    return dict(CONFIGS[k])


def make_config(k: int, seed: Optional[int] = None, poison: bool = True):
    """Inputs for workload ``k`` (1..10) with seed 1000 + k unless given."""
    c = CONFIGS[k]
    seed = 1000 + k if seed is None else seed
    if c["kind"] == "paged":
        return make_paged(c["batch"], c["s_q"], c["h_q"], c["seqlens"], c["causal"], seed, poison=poison)
    if c["kind"] == "paged_fp8":
        return make_paged_fp8(c["batch"], c["s_q"], c["h_q"], c["seqlens"], c["causal"], seed, poison=poison)
    if c["kind"] == "paged_v4":
        return make_paged(c["batch"], c["s_q"], c["h_q"], c["seqlens"], c["causal"], seed, poison=poison,
                          d_qk=D_V, sinks=True)
    if c["kind"] == "paged_v4_fp4":
        return make_paged_fp4(c["batch"], c["s_q"], c["h_q"], c["seqlens"], c["causal"], seed, poison=poison,
                              sinks=True)
    if c["kind"] == "fused_v4":
        inp = make_paged(c["batch"], c["s_q"], c["h_q"], c["seqlens"], c["causal"], seed, poison=poison,
                         d_qk=D_V, sinks=True)
        inp.fused = make_fused_extras(inp, seed + 500)
        return inp
    return make_sparse(c["batch"], c["s_q"], c["h_q"], c["tokens_per_seq"], c["topk"], c["p_invalid"], seed)
