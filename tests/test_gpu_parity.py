"""GPU parity: libmla.so on the MI355X against the float64 CPU oracle, element by element.

Bar: max|O - O_ref| <= 1e-2 * max|O_ref| + 2e-3 and |LSE - LSE_ref| <= 1e-3 (rows that see
no token: O = 0 and LSE = -inf exactly).  Metadata (integer) is compared bit-exactly with
the host twin.
"""

import sys

import numpy as np
import pytest

from mla_inputs import make_config, make_paged, make_paged_fp4, make_paged_fp8, make_sparse
from mla_inputs.gen import bf16_bits_from_f32, bf16_bits_to_f32, quantize_rows_e4m3
from oracle import (E4M3_TABLE, fused_decode, gather_paged_fp4, gather_paged_rows, paged_decode, paged_decode_fp4,
                    paged_decode_fp8, sparse_decode)
from tests.helpers import check_parity, dev_bf16, dev_i32, dev_u8, record_parity, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_paged_amd as mla

    return mla, torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_paged(env, inp, num_parts=None):
    import torch

    mla, dev = env
    q = dev_bf16(inp.q, dev)
    kc = dev_bf16(inp.kcache, dev)
    bt = dev_i32(inp.block_table, dev)
    sl = dev_i32(inp.seqlens, dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, num_parts)
    out, lse = mla.decode_paged(q, kc, bt, sl, meta, inp.softmax_scale, inp.causal)
    torch.cuda.synchronize()
    return to_host(out, lse)


def run_paged_v4(env, inp, num_parts=None):
    """512-wide latent rows (K and V) with optional sinks: mla_decode_paged_latent512."""
    import torch

    mla, dev = env
    q = dev_bf16(inp.q, dev)
    kc = dev_bf16(inp.kcache.reshape(inp.num_pages, 64, 512), dev)
    bt = dev_i32(inp.block_table, dev)
    sl = dev_i32(inp.seqlens, dev)
    sk = None if inp.sinks is None else torch.from_numpy(inp.sinks).to(dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, num_parts)
    out, lse = mla.decode_paged(q, kc, bt, sl, meta, inp.softmax_scale, inp.causal, sinks=sk)
    torch.cuda.synchronize()
    return to_host(out, lse)


def run_paged_fp4(env, inp, num_parts=None):
    """512-wide FP4 rows (codes + UE4M3 block scales) with optional sinks: mla_decode_paged_fp4."""
    import torch

    mla, dev = env
    q = dev_bf16(inp.q, dev)
    codes = dev_u8(inp.kv_codes, dev)
    scales = dev_u8(inp.kv_scales, dev)
    bt = dev_i32(inp.block_table, dev)
    sl = dev_i32(inp.seqlens, dev)
    sk = None if inp.sinks is None else torch.from_numpy(inp.sinks).to(dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, num_parts)
    out, lse = mla.decode_paged_fp4(q, codes, scales, bt, sl, meta, inp.softmax_scale, inp.causal, sinks=sk)
    torch.cuda.synchronize()
    return to_host(out, lse)


def run_paged_fp8(env, inp, num_parts=None):
    import torch

    mla, dev = env
    q = dev_bf16(inp.q, dev)
    kc = dev_u8(inp.kcache, dev)
    bt = dev_i32(inp.block_table, dev)
    sl = dev_i32(inp.seqlens, dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, num_parts)
    out, lse = mla.decode_paged(q, kc, bt, sl, meta, inp.softmax_scale, inp.causal)
    torch.cuda.synchronize()
    return to_host(out, lse)


def run_sparse(env, inp, splits=0):
    import torch

    mla, dev = env
    out, lse = mla.decode_sparse(dev_bf16(inp.q, dev), dev_u8(inp.kv, dev), dev_i32(inp.indices, dev),
                                 inp.softmax_scale, splits)
    torch.cuda.synchronize()
    return to_host(out, lse)


# ----------------------------------------------------------------- metadata
@pytest.mark.parametrize("L,P", [
    ([37, 130], 256), ([4096] * 128, 256), ([65536] * 16, 256), ([1, 64, 65, 0, 128, 3000], 7),
    ([0, 0, 5], 4), ([100] * 9, 1), (list(range(0, 3000, 37)), 64),
    (list(np.random.default_rng(1).integers(0, 9000, size=3000)), 128),
    # batches of more than one pass over the 256 threads, 65 (one wave and one lane), and more
    # parts than sequences
    (list(np.random.default_rng(2).integers(0, 9000, size=1024)), 256),
    (list(np.random.default_rng(3).integers(0, 9000, size=1025)), 256),
    (list(np.random.default_rng(4).integers(0, 200, size=65)), 100), ([7] * 64, 300),
])
@pytest.mark.parametrize("h_q", [16, 128])
def test_metadata_kernel_matches_host_twin(env, L, P, h_q):
    import torch

    mla, dev = env
    _say("metadata", len(L), P, h_q)
    L = np.asarray(L, dtype=np.int32)
    meta_h, ns_h = mla.get_metadata_host(L, P, h_q=h_q)
    meta_d, ns_d = mla.get_metadata(dev_i32(L, dev), h_q, 1, P)
    torch.cuda.synchronize()
    assert np.array_equal(meta_d.cpu().numpy(), meta_h)
    assert np.array_equal(ns_d.cpu().numpy(), ns_h)


# ----------------------------------------------------------------- paged
def test_tiny_config(env):
    inp = make_config(1)
    o, l = run_paged(env, inp)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, inp.causal)
    check_parity(o, l, o_ref, l_ref, "tiny")


PAGED_CASES = [
    # batch, s_q, h_q, seqlens, causal, num_parts
    (3, 1, 16, [1, 64, 65], False, None),
    (4, 1, 16, [63, 128, 129, 300], False, 1),
    (2, 1, 16, [1000, 777], False, 64),
    (3, 2, 16, [2, 100, 257], True, None),
    (2, 4, 16, [3, 200], True, 5),
    (2, 3, 16, [40, 96], True, 3),
    (2, 2, 128, [130, 700], True, None),
    (2, 2, 128, [1, 2], True, 4),
    (2, 1, 64, [500, 64], False, 3),
    (3, 1, 16, [0, 50, 0], False, None),
    (2, 1, 48, [77, 300], False, None),
    (1, 2, 64, [4000], False, 16),
    (5, 1, 32, [33, 31, 32, 1, 97], False, 2),
    # 128-row workgroups that end mid-group: an idle fourth wave (96 rows), a second group of 2
    # rows (130), a partly filled wave (200)
    (2, 3, 32, [300, 77], True, None),
    (2, 2, 65, [150, 64], True, 3),
    (1, 5, 40, [700], True, 2),
    # 128 rows: empty sequences around a short one, an all-empty causal batch, 24 ragged
    # sequences (0..3000 tokens) split over the default parts
    (3, 1, 128, [0, 50, 0], False, None),
    (2, 2, 64, [0, 0], True, None),
    (1, 6, 16, [322], True, 8),
    (24, 1, 128, [2012, 2415, 67, 2423, 1406, 1545, 1890, 857, 2938, 161, 833, 1150, 1713, 1225, 393, 135, 3, 146, 446, 2997, 572, 1957, 2250, 703], False, None),
    # 11 parts of 2 row groups: 8 parts placed XCD by XCD, the other 3 in order after them
    (2, 2, 128, [1500, 700], True, 11),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[str(i) for i in range(len(PAGED_CASES))])
def test_paged_cases(env, case):
    batch, s_q, h_q, L, causal, P = case
    _say("paged case", case)
    inp = make_paged(batch, s_q, h_q, L, causal, seed=100 + sum(L) + h_q, poison=True)
    o, l = run_paged(env, inp, P)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal)
    check_parity(o, l, o_ref, l_ref, str(case))


def test_forced_splits_and_rerun_determinism(env):
    inp = make_paged(3, 2, 32, [900, 1500, 64], True, seed=5, poison=True)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    for P in (1, 2, 8, 64, 256):
        _say("split", P)
        o, l = run_paged(env, inp, P)
        check_parity(o, l, o_ref, l_ref, "P=%d" % P)
        o2, l2 = run_paged(env, inp, P)
        assert np.array_equal(o, o2) and np.array_equal(l, l2), "rerun differs at P=%d" % P


def test_block_table_permutation_is_bitwise_invariant(env):
    inp = make_paged(2, 1, 16, [300, 200], False, seed=9, poison=False)
    o1, l1 = run_paged(env, inp, 8)
    rng = np.random.default_rng(4)
    perm = rng.permutation(inp.num_pages)
    kc2 = np.empty_like(inp.kcache)
    kc2[perm] = inp.kcache
    inp.kcache = kc2
    inp.block_table = perm[inp.block_table].astype(np.int32)
    o2, l2 = run_paged(env, inp, 8)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ----------------------------------------------------------------- paged, fp8 cache
FP8_PAGED_CASES = [
    # batch, s_q, h_q, seqlens, causal, num_parts
    (3, 1, 16, [1, 64, 65], False, None),
    (4, 1, 16, [63, 128, 129, 300], False, 1),
    (2, 1, 16, [1000, 777], False, 64),
    (3, 2, 8, [2, 100, 257], True, None),
    (2, 4, 4, [3, 200], True, 5),
    (3, 1, 16, [0, 50, 0], False, None),
    (2, 2, 32, [130, 700], True, None),
    (2, 2, 64, [1, 2], True, 4),
    (2, 1, 48, [77, 300], False, None),
    (2, 1, 32, [500, 64], False, 3),
    (1, 2, 64, [4000], False, 16),
    (3, 3, 16, [40, 96, 1], True, 3),
    # one part holding more tokens than a sparse split's index list (many-row gathers)
    (1, 2, 64, [5000], True, 1),
    (2, 1, 32, [3000, 2500], False, 2),
    # 128 rows in two 64-row groups over 11 parts: 8 parts placed XCD by XCD, 3 after them
    (2, 2, 64, [3000, 1700], True, 11),
]


@pytest.mark.parametrize("case", FP8_PAGED_CASES, ids=[str(i) for i in range(len(FP8_PAGED_CASES))])
def test_paged_fp8_cases(env, case):
    batch, s_q, h_q, L, causal, P = case
    _say("paged fp8 case", case)
    inp = make_paged_fp8(batch, s_q, h_q, L, causal, seed=300 + sum(L) + h_q, poison=True)
    o, l = run_paged_fp8(env, inp, P)
    o_ref, l_ref = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal)
    check_parity(o, l, o_ref, l_ref, "fp8 " + str(case))


@pytest.mark.parametrize("h_q,scale", [(16, 2.5), (64, 2.5), (16, 0.0), (64, 0.0), (16, -0.05), (64, -0.05)])
def test_paged_fp8_softmax_scales(env, h_q, scale):
    """Large, zero and negative softmax scales over an fp8 cache (16-row and many-row kernels)."""
    _say("paged fp8 scale", h_q, scale)
    inp = make_paged_fp8(2, 1, h_q, [1800, 900], False, seed=450 + h_q, poison=True, softmax_scale=scale)
    o, l = run_paged_fp8(env, inp)
    o_ref, l_ref = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, False)
    check_parity(o, l, o_ref, l_ref, "fp8 scale %g h_q %d" % (scale, h_q))


def test_paged_fp8_forced_splits(env):
    inp = make_paged_fp8(3, 1, 16, [900, 1500, 64], False, seed=15, poison=True)
    o_ref, l_ref = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, False)
    for P in (1, 2, 8, 64, 256):
        _say("fp8 split", P)
        o, l = run_paged_fp8(env, inp, P)
        check_parity(o, l, o_ref, l_ref, "fp8 P=%d" % P)


def test_full_size_paged_fp8(env):
    """The memory-bound shape over fp8 pages, every output row against the oracle."""
    _say("full-size fp8 paged (memory-bound shape)")
    inp = make_config(6, poison=False)
    o, l = run_paged_fp8(env, inp)
    o_ref, l_ref = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale,
                                    inp.causal)
    _whole(o, l, o_ref, l_ref, "config 6")


# ----------------------------------------------------------------- V4 geometry: 512-wide rows, sinks
V4_CASES = [
    # batch, s_q, h_q, seqlens, causal, sinks, num_parts
    (2, 6, 64, [300, 70], True, True, None),
    (2, 6, 64, [300, 70], True, False, None),
    (3, 1, 16, [1, 64, 65], False, True, None),
    (3, 2, 32, [500, 0, 3], True, True, 3),
    (1, 6, 64, [2000], True, True, 16),
    (1, 6, 128, [700], True, True, None),
    (4, 6, 8, [5, 6, 7, 129], True, True, 2),
    # long parts (more than 2048 tokens in one workgroup's segment)
    (1, 6, 64, [5000], True, True, 1),
    # 128-row workgroups that end mid-group (96, 130 and 200 rows)
    (2, 3, 32, [300, 77], True, True, None),
    (2, 2, 65, [150, 64], True, True, None),
    (1, 5, 40, [700], True, False, 3),
    (2, 2, 32, [3000, 2500], True, False, 2),
    # a split whose tokens the first causal rows cannot see (a -inf partial beside the sink): the
    # last block alone (3 parts), and in the combine's second group of splits (8 parts)
    (1, 6, 64, [130], True, True, 3),
    (1, 6, 64, [322], True, True, 8),
    # 13 parts of 3 row groups: 8 parts placed XCD by XCD, the other 5 in order after them
    (2, 6, 64, [900, 333], True, True, 13),
]


@pytest.mark.parametrize("case", V4_CASES, ids=[str(i) for i in range(len(V4_CASES))])
def test_paged_v4_geometry_cases(env, case):
    batch, s_q, h_q, L, causal, sinks, P = case
    _say("paged v4 case", case)
    inp = make_paged(batch, s_q, h_q, L, causal, seed=600 + sum(L) + h_q, poison=True, d_qk=512, sinks=sinks)
    o, l = run_paged_v4(env, inp, P)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal,
                                sinks=inp.sinks)
    check_parity(o, l, o_ref, l_ref, "v4 " + str(case))


@pytest.mark.parametrize("scale", [0.0, -0.05, 0.5, 2.5])
def test_paged_v4_softmax_scales(env, scale):
    _say("paged v4 scale", scale)
    inp = make_paged(2, 6, 64, [900, 300], True, seed=650, poison=True, softmax_scale=scale, d_qk=512,
                     sinks=True)
    o, l = run_paged_v4(env, inp)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True,
                                sinks=inp.sinks)
    check_parity(o, l, o_ref, l_ref, "v4 scale %g" % scale)


def test_full_size_v4_geometry(env):
    _say("full-size V4 geometry")
    inp = make_config(7, poison=False)
    o, l = run_paged_v4(env, inp)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale,
                                inp.causal, sinks=inp.sinks)
    _whole(o, l, o_ref, l_ref, "config 7")


# ----------------------------------------------------------------- V4 geometry over FP4 pages
@pytest.mark.parametrize("case", V4_CASES, ids=[str(i) for i in range(len(V4_CASES))])
def test_paged_fp4_cases(env, case):
    batch, s_q, h_q, L, causal, sinks, P = case
    _say("paged fp4 case", case)
    inp = make_paged_fp4(batch, s_q, h_q, L, causal, seed=700 + sum(L) + h_q, poison=True, sinks=sinks)
    o, l = run_paged_fp4(env, inp, P)
    o_ref, l_ref = paged_decode_fp4(inp.q, inp.kv_codes, inp.kv_scales, inp.block_table, inp.seqlens,
                                    inp.softmax_scale, causal, sinks=inp.sinks)
    check_parity(o, l, o_ref, l_ref, "fp4 " + str(case))


@pytest.mark.parametrize("scale", [0.0, -0.05, 0.5, 2.5])
def test_paged_fp4_softmax_scales(env, scale):
    _say("paged fp4 scale", scale)
    inp = make_paged_fp4(2, 6, 64, [900, 300], True, seed=750, poison=True, softmax_scale=scale, sinks=True)
    o, l = run_paged_fp4(env, inp)
    o_ref, l_ref = paged_decode_fp4(inp.q, inp.kv_codes, inp.kv_scales, inp.block_table, inp.seqlens,
                                    inp.softmax_scale, True, sinks=inp.sinks)
    check_parity(o, l, o_ref, l_ref, "fp4 scale %g" % scale)


def test_paged_fp4_every_code_and_scale_byte(env):
    """Random codes and scale bytes over the whole UE4M3 range (subnormal scales, zero blocks,
    values up to 6 * 448) with a small softmax scale, so that every conversion path is used."""
    _say("paged fp4 full code range")
    inp = make_paged_fp4(2, 6, 64, [700, 200], True, seed=760, poison=True, softmax_scale=2e-4, sinks=True)
    rng = np.random.default_rng(761)
    used = np.unique(inp.block_table[inp.block_table != inp.poison_page])
    inp.kv_codes[used] = rng.integers(0, 256, size=inp.kv_codes[used].shape).astype(np.uint8)
    inp.kv_scales[used] = rng.integers(0, 0x7F, size=inp.kv_scales[used].shape).astype(np.uint8)
    for b in range(inp.batch):     # keep the poison past each sequence's end
        L = int(inp.seqlens[b])
        if L % 64:
            inp.kv_scales[inp.block_table[b, L // 64], L % 64:] = 0x7F
    o, l = run_paged_fp4(env, inp)
    o_ref, l_ref = paged_decode_fp4(inp.q, inp.kv_codes, inp.kv_scales, inp.block_table, inp.seqlens,
                                    inp.softmax_scale, True, sinks=inp.sinks)
    assert np.isfinite(o_ref).all()
    check_parity(o, l, o_ref, l_ref, "fp4 full code range")


def test_full_size_v4_fp4(env):
    _say("full-size V4 geometry, FP4 pages")
    inp = make_config(8, poison=False)
    o, l = run_paged_fp4(env, inp)
    o_ref, l_ref = paged_decode_fp4(inp.q, inp.kv_codes, inp.kv_scales, inp.block_table, inp.seqlens,
                                    inp.softmax_scale, inp.causal, sinks=inp.sinks)
    _whole(o, l, o_ref, l_ref, "config 8")


# ----------------------------------------------------------------- sparse
SPARSE_CASES = [
    # batch, s_q, h_q, tokens_per_seq, topk, p_invalid, splits
    (2, 2, 16, 256, 100, 0.1, 0),
    (2, 1, 64, 512, 33, 0.0, 0),
    (1, 3, 32, 300, 290, 0.5, 3),
    (2, 2, 128, 4096, 2048, 0.05, 0),
    (1, 1, 16, 64, 1, 0.0, 0),
    (2, 6, 64, 2000, 512, 0.05, 1),
    (1, 2, 48, 700, 600, 0.2, 7),
    # more than 64 heads: forced ragged splits with half the entries unused, 96 and 65 heads (a
    # row group that ends mid-way), 200 heads (row groups share the records), a single record
    (1, 2, 128, 600, 77, 0.5, 3),
    (2, 1, 96, 1000, 300, 0.1, 0),
    (1, 1, 65, 500, 400, 0.0, 0),
    (1, 2, 200, 3000, 1000, 0.05, 2),
    (1, 1, 128, 64, 1, 0.0, 0),
    # top-k beyond one split's 2048 entries (at least three splits)
    (1, 2, 128, 6000, 5000, 0.1, 0),
    (2, 1, 16, 9000, 4500, 0.0, 0),
    # 10 work items (5 query tokens x 2 splits) of two 64-row groups: 8 items placed XCD by XCD,
    # 2 after them
    (1, 5, 128, 3000, 1500, 0.1, 2),
]


@pytest.mark.parametrize("case", SPARSE_CASES, ids=[str(i) for i in range(len(SPARSE_CASES))])
def test_sparse_cases(env, case):
    batch, s_q, h_q, T, topk, p, splits = case
    _say("sparse case", case)
    inp = make_sparse(batch, s_q, h_q, T, topk, p, seed=200 + topk + h_q)
    o, l = run_sparse(env, inp, splits)
    o_ref, l_ref = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale)
    check_parity(o, l, o_ref, l_ref, str(case))


@pytest.mark.parametrize("h_q", [16, 64, 128])
def test_sparse_all_skipped_and_duplicates(env, h_q):
    _say("sparse skip/dup h_q", h_q)
    inp = make_sparse(2, 2, h_q, 300, 64, 0.0, seed=31)
    inp.indices[0, 1, :] = -1                         # a query that reads nothing
    inp.indices[1, 0, 10:20] = inp.indices[1, 0, 0]   # repeated rows count repeatedly
    for splits in (0, 1, 2):
        o, l = run_sparse(env, inp, splits)
        o_ref, l_ref = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale)
        check_parity(o, l, o_ref, l_ref, "skip/dup splits=%d" % splits)
        assert np.all(o[0, 1] == 0) and np.all(np.isneginf(l[0, 1]))


# ----------------------------------------------------------------- wide score ranges
def _ramp(inp, top, seed=7):
    """Scores that move linearly along each sequence, from ~0 to ~`top` nats (top < 0: falling
    from ~|top| to ~0).  Rising scores keep outgrowing the softmax reference the kernels hold;
    falling ones drive later probabilities far below the first chunk's."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(576)
    u /= np.linalg.norm(u)
    sigma_inv = 1.0 / inp.softmax_scale
    qf = u * sigma_inv + 0.02 * sigma_inv * rng.standard_normal(inp.q.shape)
    inp.q = bf16_bits_from_f32(qf.astype(np.float32))
    kc = bf16_bits_to_f32(inp.kcache).astype(np.float64)
    for b, L in enumerate(inp.seqlens):
        for t in range(int(L)):
            f = (t + 1) / L if top > 0 else (L - t) / L
            kc[inp.block_table[b, t // 64], t % 64, 0, :] = abs(top) * f * u + 0.5 * rng.standard_normal(576)
    inp.kcache = bf16_bits_from_f32(kc.astype(np.float32))
    return inp


RAMP_CASES = [
    # batch, s_q, h_q, seqlens, causal, top (nats), num_parts
    (2, 1, 16, [1500, 700], False, 150.0, None),
    (2, 1, 16, [1500, 700], False, -150.0, None),
    (2, 1, 64, [1500, 700], False, 150.0, None),
    (2, 1, 64, [1500, 700], False, -150.0, None),
    (2, 1, 32, [1200, 333], False, 150.0, 8),
    (1, 2, 128, [2000], True, 120.0, None),
    (1, 2, 128, [2000], True, -150.0, 4),
    (2, 2, 64, [900, 1300], True, 150.0, 16),
]


@pytest.mark.parametrize("case", RAMP_CASES, ids=[str(i) for i in range(len(RAMP_CASES))])
def test_paged_wide_score_range(env, case):
    batch, s_q, h_q, L, causal, top, P = case
    _say("paged ramp case", case)
    inp = _ramp(make_paged(batch, s_q, h_q, L, causal, seed=300 + h_q, poison=True), top)
    o, l = run_paged(env, inp, P)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal)
    check_parity(o, l, o_ref, l_ref, "ramp " + str(case))


def _ramp_fp8(inp, top, seed=8):
    """The score ramp of _ramp on an fp8 page cache: rows rebuilt along each sequence and
    quantised per token into records (poisoned records stay as they are)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(576)
    u /= np.linalg.norm(u)
    sigma_inv = 1.0 / inp.softmax_scale
    qf = u * sigma_inv + 0.02 * sigma_inv * rng.standard_normal(inp.q.shape)
    inp.q = bf16_bits_from_f32(qf.astype(np.float32))
    for b, L in enumerate(inp.seqlens):
        rows = np.empty((int(L), 576))
        for t in range(int(L)):
            f = (t + 1) / L if top > 0 else (L - t) / L
            rows[t] = abs(top) * f * u + 0.5 * rng.standard_normal(576)
        rec = quantize_rows_e4m3(rows.astype(np.float32))
        for t in range(int(L)):
            inp.kcache[inp.block_table[b, t // 64], t % 64] = rec[t]
    return inp


FP8_RAMP_CASES = [
    # batch, s_q, h_q, seqlens, causal, top (nats), num_parts
    (2, 1, 16, [1500, 700], False, 150.0, None),
    (2, 1, 16, [1500, 700], False, -150.0, None),
    (2, 1, 64, [1500, 700], False, 150.0, None),
    (2, 2, 32, [1200, 333], True, -150.0, 8),
]


@pytest.mark.parametrize("case", FP8_RAMP_CASES, ids=[str(i) for i in range(len(FP8_RAMP_CASES))])
def test_paged_fp8_wide_score_range(env, case):
    batch, s_q, h_q, L, causal, top, P = case
    _say("paged fp8 ramp case", case)
    inp = _ramp_fp8(make_paged_fp8(batch, s_q, h_q, L, causal, seed=320 + h_q, poison=True), top)
    o, l = run_paged_fp8(env, inp, P)
    o_ref, l_ref = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal)
    check_parity(o, l, o_ref, l_ref, "fp8 ramp " + str(case))


def _ramp_sparse(inp, top, seed=9):
    """Sparse input whose scores move linearly along each query's index list, from ~0 to ~`top`
    nats (falling for top < 0); one query token per sequence, so every record has one position."""
    assert inp.s_q == 1
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(576)
    u /= np.linalg.norm(u)
    sigma_inv = 1.0 / inp.softmax_scale
    qf = u * sigma_inv + 0.02 * sigma_inv * rng.standard_normal(inp.q.shape)
    inp.q = bf16_bits_from_f32(qf.astype(np.float32))
    x = 0.5 * rng.standard_normal((inp.num_tokens, 576))
    for b in range(inp.batch):
        lst = inp.indices[b, 0]
        for e, r in enumerate(lst):
            if r >= 0:
                f = (e + 1) / len(lst) if top > 0 else (len(lst) - e) / len(lst)
                x[r] += abs(top) * f * u
    inp.kv = quantize_rows_e4m3(x.astype(np.float32))
    return inp


SPARSE_RAMP_CASES = [
    # batch, h_q, tokens_per_seq, topk, p_invalid, top (nats), splits
    (2, 64, 3000, 2048, 0.05, 150.0, 0),
    (2, 64, 3000, 2048, 0.05, -150.0, 0),
    (2, 128, 2500, 1500, 0.1, 150.0, 2),
    (2, 32, 2500, 1500, 0.1, 150.0, 0),
    (2, 128, 3000, 2048, 0.05, -150.0, 0),
    (1, 160, 2500, 1000, 0.05, 150.0, 0),
]


@pytest.mark.parametrize("case", SPARSE_RAMP_CASES, ids=[str(i) for i in range(len(SPARSE_RAMP_CASES))])
def test_sparse_wide_score_range(env, case):
    batch, h_q, T, topk, p, top, splits = case
    _say("sparse ramp", case)
    inp = _ramp_sparse(make_sparse(batch, 1, h_q, T, topk, p, seed=800 + h_q), top)
    o, l = run_sparse(env, inp, splits)
    o_ref, l_ref = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale)
    check_parity(o, l, o_ref, l_ref, "sparse ramp " + str(case))


@pytest.mark.parametrize("h_q,scale", [(16, 2.5), (64, 2.5), (16, 0.7), (64, 0.7), (128, 2.5), (128, 0.7)])
def test_large_softmax_scale(env, h_q, scale):
    """Scores with a spread of tens to hundreds of nats on random data, paged and sparse."""
    _say("large scale", h_q, scale)
    inp = make_paged(2, 1, h_q, [1800, 900], False, seed=400 + h_q, poison=True, softmax_scale=scale)
    o, l = run_paged(env, inp)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, False)
    check_parity(o, l, o_ref, l_ref, "paged scale %g h_q %d" % (scale, h_q))
    sp = make_sparse(2, 1, h_q, 2048, 1024, 0.05, seed=500 + h_q, softmax_scale=scale)
    for splits in (0, 1):
        o, l = run_sparse(env, sp, splits)
        o_ref, l_ref = sparse_decode(sp.q, sp.kv, sp.indices, sp.softmax_scale)
        check_parity(o, l, o_ref, l_ref, "sparse scale %g h_q %d splits %d" % (scale, h_q, splits))


@pytest.mark.parametrize("h_q", [16, 64, 128])
@pytest.mark.parametrize("scale", [0.0, -0.05])
def test_non_positive_softmax_scale(env, h_q, scale):
    """softmax_scale = 0 (uniform weights) and a negative scale, paged and sparse."""
    _say("scale", scale, "h_q", h_q)
    inp = make_paged(2, 2, h_q // 2, [300, 97], True, seed=600 + h_q, poison=True, softmax_scale=scale)
    o, l = run_paged(env, inp)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    check_parity(o, l, o_ref, l_ref, "paged scale %g h_q %d" % (scale, h_q))
    sp = make_sparse(2, 1, h_q, 512, 200, 0.1, seed=700 + h_q, softmax_scale=scale)
    o, l = run_sparse(env, sp)
    o_ref, l_ref = sparse_decode(sp.q, sp.kv, sp.indices, sp.softmax_scale)
    check_parity(o, l, o_ref, l_ref, "sparse scale %g h_q %d" % (scale, h_q))


# ----------------------------------------------------------------- full-size workloads
def _whole(o, l, o_ref, l_ref, what):
    """The bar over a whole output tensor, with its error figures printed and logged."""
    err, _ = check_parity(o, l, o_ref, l_ref, what)
    rec = record_parity(what, o, l, o_ref, l_ref)
    _say(what, "max err %.3g (tol %.3g) rmse %.3g lse err %.3g" % (err, rec["tol"], rec["rmse"], rec["max_lse_err"]))


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_full_size_paged_config(env, k):
    """The paged workloads at full size: every sequence, query token and head against the oracle."""
    _say("full-size config", k)
    inp = make_config(k, poison=False)
    o, l = run_paged(env, inp)
    o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale,
                                inp.causal)
    _whole(o, l, o_ref, l_ref, "config %d" % k)


def test_full_size_sparse_config(env):
    """The sparse fp8 workload at full size: all 32 x 6 query tokens and 64 heads."""
    _say("full-size config 5")
    inp = make_config(5)
    o, l = run_sparse(env, inp)
    o_ref, l_ref = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale)
    _whole(o, l, o_ref, l_ref, "config 5")


# ----------------------------------------------------------------- sparse prefill
def run_prefill(env, inp, splits=0):
    """A prompt chunk of s_q query tokens (batch 1 of the generator) through mla_sparse_prefill."""
    import torch

    mla, dev = env
    assert inp.batch == 1
    out, lse = mla.sparse_prefill(dev_bf16(inp.q[0], dev), dev_u8(inp.kv, dev), dev_i32(inp.indices[0], dev),
                                  inp.softmax_scale, splits)
    torch.cuda.synchronize()
    return to_host(out, lse)


PREFILL_CASES = [
    # s_q, h_q, context tokens, topk, p_invalid, splits
    (300, 64, 2048, 512, 0.05, 0),
    (97, 128, 4096, 2048, 0.0, 0),
    (64, 16, 1024, 200, 0.1, 0),
    (40, 32, 1024, 100, 0.0, 0),
    (33, 64, 3000, 1000, 0.02, 3),
    (50, 128, 2048, 700, 0.3, 2),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(i) for i in range(len(PREFILL_CASES))])
def test_sparse_prefill_cases(env, case):
    s_q, h_q, ctx, topk, p_inv, splits = case
    _say("sparse prefill case", case)
    inp = make_sparse(1, s_q, h_q, ctx, topk, p_inv, seed=800 + s_q + h_q)
    o, l = run_prefill(env, inp, splits)
    o_ref, l_ref = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale)
    check_parity(o, l, o_ref[0], l_ref[0], "prefill " + str(case))


def test_sparse_prefill_matches_sparse_decode_bitwise(env):
    """The prefill call over a prompt chunk and the decode call over the same query tokens (as
    one sequence of s_q tokens) run the same kernels: identical bits."""
    import torch

    mla, dev = env
    _say("sparse prefill vs decode")
    inp = make_sparse(1, 50, 64, 2048, 700, 0.05, seed=850)
    o, l = run_prefill(env, inp)
    od, ld = mla.decode_sparse(dev_bf16(inp.q, dev), dev_u8(inp.kv, dev), dev_i32(inp.indices, dev),
                               inp.softmax_scale)
    torch.cuda.synchronize()
    od, ld = to_host(od, ld)
    assert np.array_equal(o, od[0]) and np.array_equal(l, ld[0])


@pytest.fixture(scope="module")
def prefill_full(env):
    """The full sparse prefill workload and the GPU's result, shared by the four quarter tests
    (the float64 oracle takes about a minute for all 4096 query tokens)."""
    inp = make_config(9)
    o, l = run_prefill(env, inp)
    return inp, o, l


@pytest.mark.parametrize("quarter", [0, 1, 2, 3])
def test_full_size_sparse_prefill(env, prefill_full, quarter):
    """Sparse prefill at full size, all 4096 query tokens x 128 heads over four tests."""
    inp, o, l = prefill_full
    n = inp.s_q // 4
    toks = list(range(quarter * n, (quarter + 1) * n))
    _say("full-size config 9, query tokens %d..%d" % (toks[0], toks[-1]))
    o_ref, l_ref = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale, sets=[(0, t) for t in toks])
    _whole(o[toks], l[toks], o_ref[0, toks], l_ref[0, toks], "config 9 quarter %d" % quarter)


# ----------------------------------------------------------------- the largest row count, one head
def _run_kind(env, kind, batch, s_q, h_q, L, causal, seed):
    """One paged call of the given cache kind against its oracle (poisoned pools, sinks on the
    512-wide kinds)."""
    if kind == "bf16":
        inp = make_paged(batch, s_q, h_q, L, causal, seed=seed, poison=True)
        o, l = run_paged(env, inp)
        ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal)
    elif kind == "latent512":
        inp = make_paged(batch, s_q, h_q, L, causal, seed=seed, poison=True, d_qk=512, sinks=True)
        o, l = run_paged_v4(env, inp)
        ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal,
                           sinks=inp.sinks)
    elif kind == "fp8":
        inp = make_paged_fp8(batch, s_q, h_q, L, causal, seed=seed, poison=True)
        o, l = run_paged_fp8(env, inp)
        ref = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal)
    else:
        inp = make_paged_fp4(batch, s_q, h_q, L, causal, seed=seed, poison=True, sinks=True)
        o, l = run_paged_fp4(env, inp)
        ref = paged_decode_fp4(inp.q, inp.kv_codes, inp.kv_scales, inp.block_table, inp.seqlens,
                               inp.softmax_scale, causal, sinks=inp.sinks)
    return o, l, ref


@pytest.mark.parametrize("kind,s_q,h_q", [("bf16", 32, 128), ("latent512", 64, 64), ("fp8", 32, 128),
                                          ("fp4", 64, 64)])
def test_maximum_rows(env, kind, s_q, h_q):
    """s_q * h_q = 4096 query rows per sequence, the largest count the calls accept (32 groups of
    128 rows on the one-wave-per-SIMD kernel, 64 groups of 64 on the row-split kernel for fp8
    pages), causal; the second sequence is shorter than s_q, so its first query tokens see no
    token at all (O = 0, LSE = -inf)."""
    _say("maximum rows", kind, s_q, h_q)
    o, l, (o_ref, l_ref) = _run_kind(env, kind, 2, s_q, h_q, [300, 20], True, seed=1200 + s_q + h_q)
    check_parity(o, l, o_ref, l_ref, "maximum rows %s" % kind)


@pytest.mark.parametrize("kind", ["bf16", "latent512", "fp8", "fp4"])
@pytest.mark.parametrize("s_q", [1, 3])
def test_single_head(env, kind, s_q):
    """One query head (h_q = 1): one or three rows in a 16-row tile or a 64-row group, the rest
    of the tile masked."""
    _say("single head", kind, s_q)
    o, l, (o_ref, l_ref) = _run_kind(env, kind, 2, s_q, 1, [200, 70], s_q > 1, seed=1300 + s_q)
    check_parity(o, l, o_ref, l_ref, "single head %s s_q %d" % (kind, s_q))


@pytest.mark.parametrize("splits", [0, 2])
def test_sparse_single_head(env, splits):
    _say("sparse single head", splits)
    inp = make_sparse(2, 3, 1, 500, 200, 0.1, seed=1400 + splits)
    o, l = run_sparse(env, inp, splits)
    o_ref, l_ref = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale)
    check_parity(o, l, o_ref, l_ref, "sparse single head splits %d" % splits)


# ----------------------------------------------------------------- caches beyond 4 GiB
# The gathers address records with 64-bit offsets.  Each test places the real pages or records
# of a small input past the first 4 GiB of a zero-filled device pool (so a 32-bit offset would
# wrap) and compares with the oracle on the small input.
def _big_pool(torch, dev, shape, dtype, small, first):
    """A zero device pool of `shape` with host array `small` copied in at rows first.. ."""
    pool = torch.zeros(shape, dtype=dtype, device=dev)
    src = torch.from_numpy(np.ascontiguousarray(small))
    if dtype == torch.bfloat16:
        src = src.view(torch.int16).view(torch.bfloat16)
    pool[first:first + small.shape[0]] = src.to(dev)
    return pool


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (32, 2), (64, 1)])
def test_paged_fp8_cache_beyond_4gib(env, h_q, s_q):
    import torch

    mla, dev = env
    _say("fp8 pages beyond 4 GiB", h_q, s_q)
    inp = make_paged_fp8(2, s_q, h_q, [700, 130], s_q > 1, seed=980 + h_q, poison=True)
    first = 105000                                   # 105000 pages x 40 KiB = 4.3 GB
    kc = _big_pool(torch, dev, (first + inp.num_pages + 8, 64, 640), torch.uint8, inp.kcache, first)
    assert kc.numel() > (1 << 32)
    q, bt, sl = dev_bf16(inp.q, dev), dev_i32(inp.block_table + first, dev), dev_i32(inp.seqlens, dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, 5)
    out, lse = mla.decode_paged(q, kc, bt, sl, meta, inp.softmax_scale, inp.causal)
    torch.cuda.synchronize()
    o, l = to_host(out, lse)
    del kc
    torch.cuda.empty_cache()
    o_ref, l_ref = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale,
                                    inp.causal)
    check_parity(o, l, o_ref, l_ref, "fp8 pages beyond 4 GiB h_q %d" % h_q)


@pytest.mark.parametrize("h_q", [16, 64])
def test_paged_fp4_cache_beyond_4gib(env, h_q):
    import torch

    mla, dev = env
    _say("FP4 pages beyond 4 GiB", h_q)
    inp = make_paged_fp4(2, 6, h_q, [700, 130], True, seed=985 + h_q, poison=True, sinks=True)
    first = 262200                                   # 262200 pages x 16 KiB of codes = 4.3 GB
    n = first + inp.num_pages + 8
    codes = _big_pool(torch, dev, (n, 64, 256), torch.uint8, inp.kv_codes, first)
    scales = _big_pool(torch, dev, (n, 64, 32), torch.uint8, inp.kv_scales, first)
    assert codes.numel() > (1 << 32)
    q, bt, sl = dev_bf16(inp.q, dev), dev_i32(inp.block_table + first, dev), dev_i32(inp.seqlens, dev)
    sk = torch.from_numpy(inp.sinks).to(dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, 5)
    out, lse = mla.decode_paged_fp4(q, codes, scales, bt, sl, meta, inp.softmax_scale, True, sinks=sk)
    torch.cuda.synchronize()
    o, l = to_host(out, lse)
    del codes, scales
    torch.cuda.empty_cache()
    o_ref, l_ref = paged_decode_fp4(inp.q, inp.kv_codes, inp.kv_scales, inp.block_table, inp.seqlens,
                                    inp.softmax_scale, True, sinks=inp.sinks)
    check_parity(o, l, o_ref, l_ref, "FP4 pages beyond 4 GiB h_q %d" % h_q)


@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
def test_sparse_pool_beyond_4gib(env, h_q):
    import torch

    mla, dev = env
    _say("sparse pool beyond 4 GiB", h_q)
    inp = make_sparse(2, 2, h_q, 3000, 1500, 0.1, seed=990 + h_q)
    first = 6800000                                  # 6.8 M records x 640 B = 4.35 GB
    kv = _big_pool(torch, dev, (first + inp.num_tokens + 8, 640), torch.uint8, inp.kv, first)
    assert kv.numel() > (1 << 32)
    idx = np.where(inp.indices >= 0, inp.indices + first, -1).astype(np.int32)
    out, lse = mla.decode_sparse(dev_bf16(inp.q, dev), kv, dev_i32(idx, dev), inp.softmax_scale)
    torch.cuda.synchronize()
    o, l = to_host(out, lse)
    del kv
    torch.cuda.empty_cache()
    o_ref, l_ref = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale)
    check_parity(o, l, o_ref, l_ref, "sparse pool beyond 4 GiB h_q %d" % h_q)


# ----------------------------------------------------------------- fused decode (norm, RoPE, attn, RoPE, FP8)
def run_fused(env, inp, num_parts=None):
    """mla_decode_fused over bf16 pages (PagedInputs with 512-wide rows) or FP4 pages."""
    import torch

    mla, dev = env
    fx = inp.fused
    q = dev_bf16(inp.q, dev)
    if hasattr(inp, "kv_codes"):
        kc, ks = dev_u8(inp.kv_codes, dev), dev_u8(inp.kv_scales, dev)
    else:
        kc, ks = dev_bf16(inp.kcache.reshape(inp.num_pages, 64, 512), dev), None
    bt, sl = dev_i32(inp.block_table, dev), dev_i32(inp.seqlens, dev)
    sk = None if inp.sinks is None else torch.from_numpy(inp.sinks).to(dev)
    w = torch.from_numpy(fx.norm_weight).to(dev)
    cs = torch.from_numpy(np.ascontiguousarray(fx.rope_cs)).to(dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, num_parts)
    codes, scale, lse = mla.decode_fused(q, kc, bt, sl, meta, w, fx.norm_eps, cs, inp.softmax_scale, inp.causal,
                                         sinks=sk, kv_scales=ks)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scale.cpu().numpy(), lse.cpu().numpy().astype(np.float64)


def oracle_fused(inp):
    fx = inp.fused
    if hasattr(inp, "kv_codes"):
        rows_of = lambda b, L: gather_paged_fp4(inp.kv_codes, inp.kv_scales, inp.block_table[b], L)  # noqa: E731
    else:
        rows_of = lambda b, L: gather_paged_rows(inp.kcache, inp.block_table[b], L)  # noqa: E731
    return fused_decode(inp.q, fx.norm_weight, fx.norm_eps, fx.rope_cs, rows_of, inp.block_table, inp.seqlens,
                        inp.softmax_scale, inp.causal, sinks=inp.sinks)


def check_fused(got, ref, what, softmax_scale=512 ** -0.5):
    """The FP8 output against the exact (float64) fused result.  LSE: the attention bar, scaled
    with the softmax scale above the default 512^-0.5 (the kernel's fp32 norm and the oracle's
    float64 norm round the query to bf16 the same way except within fp32 error of a rounding
    boundary, where one element moves by one bf16 step; the score moves by softmax_scale times
    that, so the bar grows with the scale).  Scale:
    the row maxima may differ by the O bar, so the scales by that over 448.  Values: the
    dequantised code lies within the O bar plus one E4M3 step (at the reference's magnitude plus
    the bar) of the exact value: the kernel's own fp32 value, within the bar, may round to either
    neighbour."""
    codes, scale, lse = got
    codes_r, scale_r, lse_r, O_r = ref
    assert codes.shape == codes_r.shape and scale.shape == scale_r.shape
    fin = np.isfinite(lse_r)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_r)), "%s: -inf rows differ" % what
    if fin.any():
        lerr = np.abs(lse[fin] - lse_r[fin]).max()
        ltol = 1e-3 * max(1.0, abs(softmax_scale) / 512 ** -0.5)
        assert lerr <= ltol, "%s: max|LSE-LSE_ref| = %.3g > %.3g" % (what, lerr, ltol)
    assert not np.any((codes & 0x7F) == 0x7F), "%s: NaN codes" % what
    tol = 1e-2 * np.abs(O_r).max() + 2e-3
    assert np.all(np.abs(scale.astype(np.float64) - scale_r) <= tol / 448.0 + 1e-7 * scale_r), "%s: scales" % what
    sk = scale.astype(np.float64)[..., None]
    deq = E4M3_TABLE[codes] * sk
    y = (np.abs(O_r) + tol) / sk
    step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3), 2.0 ** -9) * sk
    err = np.abs(deq - O_r)
    bad = err > tol + step
    assert not bad.any(), "%s: %d values beyond the bar (worst excess %.3g)" % (what, bad.sum(), (err - tol - step).max())
    same = float(np.mean(codes == codes_r))
    return float(np.abs(deq - O_r).max()), same


FUSED_CASES = [
    # batch, s_q, h_q, seqlens, causal, sinks, num_parts
    (2, 6, 64, [300, 70], True, True, None),
    (2, 6, 64, [300, 70], True, False, 3),
    (3, 1, 16, [1, 64, 65], False, True, None),
    (3, 2, 32, [500, 0, 3], True, True, 3),
    (1, 6, 64, [2000], True, True, 16),
    (1, 6, 128, [700], True, True, None),
    (4, 6, 8, [5, 6, 7, 129], True, True, 2),
    (2, 3, 32, [300, 77], True, True, None),
    (2, 1, 64, [3000, 2500], False, False, 8),
    (1, 6, 64, [322], True, True, 8),
    # the largest row count (4096 per sequence; the first query tokens of the 20-token sequence
    # see nothing) and a single head
    (2, 64, 64, [300, 20], True, True, None),
    (2, 3, 1, [200, 70], True, True, None),
]


@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("case", FUSED_CASES, ids=[str(i) for i in range(len(FUSED_CASES))])
def test_fused_decode_cases(env, case, fp4):
    from mla_inputs import make_fused_extras

    batch, s_q, h_q, L, causal, sinks, P = case
    _say("fused case", case, "fp4" if fp4 else "bf16")
    if fp4:
        inp = make_paged_fp4(batch, s_q, h_q, L, causal, seed=1100 + sum(L) + h_q, poison=True, sinks=sinks)
    else:
        inp = make_paged(batch, s_q, h_q, L, causal, seed=1000 + sum(L) + h_q, poison=True, d_qk=512, sinks=sinks)
    inp.fused = make_fused_extras(inp, 1200 + h_q)
    got = run_fused(env, inp, P)
    err, same = check_fused(got, oracle_fused(inp), "fused " + str(case))
    _say("fused", case, "max err %.3g, codes equal to the oracle's: %.4f" % (err, same))


@pytest.mark.parametrize("scale", [0.0, -0.05, 2.5])
def test_fused_decode_softmax_scales(env, scale):
    from mla_inputs import make_fused_extras

    _say("fused scale", scale)
    inp = make_paged(2, 6, 64, [900, 300], True, seed=1300, poison=True, softmax_scale=scale, d_qk=512, sinks=True)
    inp.fused = make_fused_extras(inp, 1301)
    check_fused(run_fused(env, inp), oracle_fused(inp), "fused scale %g" % scale, inp.softmax_scale)


def test_full_size_fused_decode(env):
    _say("full-size config 10")
    inp = make_config(10, poison=False)
    got = run_fused(env, inp)
    ref = oracle_fused(inp)
    err, same = check_fused(got, ref, "config 10")
    rec = record_parity("config 10 (dequantised FP8 vs exact)", E4M3_TABLE[got[0]] * got[1].astype(np.float64)[..., None],
                        got[2], ref[3], ref[2])
    _say("config 10 max err %.3g rmse %.3g, codes equal to the oracle's %.4f" % (err, rec["rmse"], same))
