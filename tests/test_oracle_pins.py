"""Pins for the CPU oracle: closed forms, invariants, library special cases.

Each test ties the oracle to something other than itself, so that a dropped
term, a wrong sign, index or base, or a transposed operand in it fails here.
"""

import math
import os

import numpy as np
import pytest
import torch

from mla_inputs import (bf16_bits_from_f32, make_paged, make_paged_fp4, make_paged_fp8, make_sparse,
                        quantize_rows_nvfp4)
from oracle import (E2M1_TABLE, E4M3_TABLE, attend, bf16_to_f64, fp4_rows_f64, lse_combine, paged_decode,
                    paged_decode_fp4, paged_decode_fp8, sparse_decode, sparse_rows_f64, visible_count)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SIGMA = float(np.float32(576 ** -0.5))


def _bf16(x):
    return bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def _one_seq_cache(rows_f32, page_order=None):
    """Pack rows [T, 576] into a paged cache with a given page order; returns (kcache bits, block_table row)."""
    T = rows_f32.shape[0]
    nblk = max(1, -(-T // 64))
    order = np.arange(nblk) if page_order is None else np.asarray(page_order)
    kc = np.zeros((nblk, 64, 1, 576), dtype=np.uint16)
    bits = _bf16(rows_f32)
    for j in range(nblk):
        n = min(64, T - 64 * j)
        if n > 0:
            kc[order[j], :n, 0, :] = bits[64 * j:64 * j + n]
    return kc, order.astype(np.int32)


# ----------------------------------------------------------------- fp8 format
def test_e4m3_table_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(E4M3_TABLE), nan)
    assert np.array_equal(E4M3_TABLE[~nan], ref[~nan])
    assert np.array_equal(np.signbit(E4M3_TABLE[~nan]), np.signbit(ref[~nan]))


def test_e4m3_golden_values_from_ocp_spec():
    n = 0
    with open(os.path.join(GOLDEN, "e4m3_ocp.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code_s, val_s = line.split()
            code, val = int(code_s, 16), float(val_s)
            got = E4M3_TABLE[code]
            if math.isnan(val):
                assert math.isnan(got)
            else:
                assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)
            n += 1
    assert n >= 10


def test_every_finite_e4m3_value_is_a_bf16_value():
    finite = E4M3_TABLE[np.isfinite(E4M3_TABLE)]
    back = bf16_to_f64(_bf16(finite.astype(np.float32)))
    assert np.array_equal(back, finite)


def test_sparse_record_dequant_is_code_times_scale():
    rec = np.zeros((2, 640), dtype=np.uint8)
    rec[0, :576] = 0x38            # 1.0
    rec[0, 576:580] = np.array([0.25], dtype="<f4").view(np.uint8)
    rec[1, :576] = np.arange(576) % 0x7e
    rec[1, 576:580] = np.array([3.0], dtype="<f4").view(np.uint8)
    rows = sparse_rows_f64(rec, np.array([1, 0]))
    assert np.all(rows[1] == 0.25)
    assert np.array_equal(rows[0], E4M3_TABLE[np.arange(576) % 0x7e] * 3.0)


# ----------------------------------------------------------------- closed forms
def test_two_token_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "two_token_closed_form.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split()
            vals[k] = float(v)
    q = np.zeros((1, 576)); q[0, 0] = 1.0
    rows = np.zeros((2, 576)); rows[1, 0] = 1.0; rows[1, 1] = 1.0
    o, lse = attend(q, rows, 1.0)
    assert abs(o[0, 0] - vals["O0"]) < 1e-15 and abs(o[0, 1] - vals["O1"]) < 1e-15
    assert np.all(o[0, 2:] == 0)
    assert abs(lse[0] - vals["LSE"]) < 1e-15


def test_single_cached_token_returns_its_value_row():
    rng = np.random.default_rng(0)
    for sigma in (SIGMA, 1.0, 0.5):
        q = bf16_to_f64(_bf16(rng.standard_normal((16, 576))))
        row = bf16_to_f64(_bf16(rng.standard_normal((1, 576))))
        o, lse = attend(q, row, sigma)
        assert np.array_equal(o, np.broadcast_to(row[0, :512], (16, 512)))
        z = np.array([math.fsum(q[h] * row[0]) * sigma for h in range(16)])
        assert np.allclose(lse, z, rtol=0, atol=1e-12)


def test_single_token_uses_first_512_dims_as_value_and_all_576_for_scores():
    q = np.zeros((1, 576)); q[0, 575] = 2.0          # only a RoPE dim scores
    row = np.zeros((1, 576)); row[0, 575] = 3.0; row[0, 0] = 7.0
    o, lse = attend(q, row, 0.5)
    assert o[0, 0] == 7.0 and np.all(o[0, 1:] == 0)
    assert lse[0] == 3.0                                # 0.5 * 2 * 3


def test_two_tokens_closed_form_random():
    rng = np.random.default_rng(1)
    q = bf16_to_f64(_bf16(rng.standard_normal((8, 576))))
    rows = bf16_to_f64(_bf16(rng.standard_normal((2, 576))))
    o, lse = attend(q, rows, SIGMA)
    for h in range(8):
        z0 = SIGMA * math.fsum(q[h] * rows[0]); z1 = SIGMA * math.fsum(q[h] * rows[1])
        w1 = 1.0 / (1.0 + math.exp(z0 - z1)); w0 = 1.0 / (1.0 + math.exp(z1 - z0))
        assert np.allclose(o[h], w0 * rows[0, :512] + w1 * rows[1, :512], rtol=0, atol=1e-13)
        assert abs(lse[h] - np.logaddexp(z0, z1)) < 1e-12


def test_equal_scores_give_mean_of_values_and_log_count():
    rng = np.random.default_rng(2)
    rows = bf16_to_f64(_bf16(rng.standard_normal((37, 576))))
    o, lse = attend(np.zeros((4, 576)), rows, SIGMA)
    assert np.allclose(o, rows[:, :512].mean(axis=0), rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(37), rtol=0, atol=1e-14)
    # equal non-zero scores: query only in the RoPE dims, every row shares its RoPE dims
    rows[:, 512:] = rows[0, 512:]
    q = np.zeros((3, 576)); q[:, 512:] = bf16_to_f64(_bf16(rng.standard_normal((3, 64))))
    o, lse = attend(q, rows, SIGMA)
    z = SIGMA * (q[:, 512:] @ rows[0, 512:])
    assert np.allclose(o, rows[:, :512].mean(axis=0), rtol=0, atol=1e-13)
    assert np.allclose(lse, z + math.log(37), rtol=0, atol=1e-12)


def test_empty_visible_set():
    o, lse = attend(np.ones((2, 576)), np.zeros((0, 576)), SIGMA)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ----------------------------------------------------------------- library special case
def test_paged_matches_torch_sdpa_and_logsumexp():
    inp = make_paged(3, 2, 16, [1, 77, 200], causal=False, seed=5)
    O, LSE = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, False)
    flat = torch.from_numpy(bf16_to_f64(inp.kcache.reshape(-1, 576)))
    for b in range(3):
        L = int(inp.seqlens[b])
        tok = torch.arange(L)
        rid = torch.from_numpy(inp.block_table[b]).long()[tok // 64] * 64 + tok % 64
        K = flat.index_select(0, rid)                        # [L, 576]
        V = K[:, :512].contiguous()
        for s in range(2):
            q = torch.from_numpy(bf16_to_f64(inp.q[b, s]))   # [16, 576]
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[None], K[None].contiguous(), V[None], scale=inp.softmax_scale)[0]
            assert np.allclose(O[b, s], ref.numpy(), rtol=0, atol=1e-12)
            lse = torch.logsumexp(inp.softmax_scale * torch.mm(q, K.t().contiguous()), dim=1)
            assert np.allclose(LSE[b, s], lse.numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------- invariants
def test_block_table_permutation_is_bitwise_invariant():
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((300, 576)).astype(np.float32)
    kc1, bt1 = _one_seq_cache(rows)
    kc2, bt2 = _one_seq_cache(rows, page_order=rng.permutation(5))
    q = _bf16(rng.standard_normal((1, 1, 16, 576)))
    L = np.array([300], dtype=np.int32)
    o1, l1 = paged_decode(q, kc1, bt1[None], L, SIGMA, False)
    o2, l2 = paged_decode(q, kc2, bt2[None], L, SIGMA, False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_poisoned_tails_and_unused_slots_are_never_read():
    inp = make_paged(4, 3, 16, [1, 63, 64, 130], causal=True, seed=7, poison=True)
    assert inp.poison_page >= 0
    O, LSE = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    # L=1 with s_q=3 causal: query 0 and 1 see nothing, query 2 sees token 0
    assert np.all(O[0, :2] == 0) and np.all(np.isneginf(LSE[0, :2]))
    assert np.all(np.isfinite(O[0, 2])) and np.all(np.isfinite(O[1:]))
    assert np.all(np.isfinite(LSE[1:]))


def test_causal_query_equals_noncausal_on_truncated_sequence():
    inp = make_paged(2, 4, 16, [150, 67], causal=True, seed=11)
    O, LSE = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    for b in range(2):
        L = int(inp.seqlens[b])
        for s in range(4):
            Lt = np.array([L - 4 + s + 1], dtype=np.int32)
            o, l = paged_decode(inp.q[b:b + 1, s:s + 1], inp.kcache, inp.block_table[b:b + 1], Lt,
                                inp.softmax_scale, False)
            assert np.array_equal(O[b, s], o[0, 0]) and np.array_equal(LSE[b, s], l[0, 0])


def test_causal_mask_ignores_poisoned_future_rows():
    inp = make_paged(1, 3, 16, [100], causal=True, seed=12, poison=False)
    O, LSE = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    kc = inp.kcache.copy()
    page = inp.block_table[0, 1]
    kc[page, 98 - 64, 0, :] = 0x7FC0      # token 98: visible only to the last query
    O2, LSE2 = paged_decode(inp.q, kc, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    assert np.array_equal(O[0, 0], O2[0, 0]) and np.array_equal(LSE[0, 0], LSE2[0, 0])
    assert np.all(np.isnan(O2[0, 1])) and np.all(np.isnan(O2[0, 2]))   # tokens 98 is visible to queries 1, 2
    assert visible_count(100, 3, 0, True) == 98


def test_causal_with_one_query_equals_noncausal():
    inp = make_paged(3, 1, 16, [5, 64, 129], causal=True, seed=13)
    a = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    c = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, False)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_split_then_combine_equals_unsplit():
    rng = np.random.default_rng(17)
    q = bf16_to_f64(_bf16(rng.standard_normal((16, 576))))
    rows = bf16_to_f64(_bf16(rng.standard_normal((500, 576))))
    o_full, l_full = attend(q, rows, SIGMA)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 500), size=trial + 1, replace=False))
        bounds = [0, *cuts.tolist(), 500]
        parts = [attend(q, rows[a:b], SIGMA) for a, b in zip(bounds[:-1], bounds[1:])]
        o, l = lse_combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert np.allclose(o, o_full, rtol=0, atol=1e-13)
        assert np.allclose(l, l_full, rtol=0, atol=1e-12)
        assert np.allclose(l, np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0), rtol=0, atol=1e-12)
    # empty parts carry no weight; all empty gives (0, -inf)
    e = attend(q, rows[:0], SIGMA)
    o, l = lse_combine(np.stack([e[0], o_full, e[0]]), np.stack([e[1], l_full, e[1]]))
    assert np.allclose(o, o_full, rtol=0, atol=1e-15) and np.allclose(l, l_full, rtol=0, atol=1e-15)
    o, l = lse_combine(np.stack([e[0], e[0]]), np.stack([e[1], e[1]]))
    assert np.all(o == 0) and np.all(np.isneginf(l))


# ----------------------------------------------------------------- sparse
def _small_sparse(seed=21, topk=40, p_invalid=0.1):
    return make_sparse(2, 3, 16, 96, topk, p_invalid, seed)


def test_sparse_minus_one_entries_are_ignored_bitwise():
    inp = _small_sparse()
    O, LSE = sparse_decode(inp.q, inp.kv, inp.indices, inp.softmax_scale)
    idx = np.full((2, 3, 70), -1, dtype=np.int32)
    rng = np.random.default_rng(0)
    for b in range(2):
        for s in range(3):
            keep = inp.indices[b, s]
            pos = np.sort(rng.choice(70, size=keep.size, replace=False))
            idx[b, s, pos] = keep
    O2, LSE2 = sparse_decode(inp.q, inp.kv, idx, inp.softmax_scale)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2)


def test_sparse_all_minus_one_gives_zero_and_neg_inf():
    inp = _small_sparse()
    idx = inp.indices.copy(); idx[1, 2] = -1
    O, LSE = sparse_decode(inp.q, inp.kv, idx, inp.softmax_scale)
    assert np.all(O[1, 2] == 0) and np.all(np.isneginf(LSE[1, 2]))
    assert np.all(np.isfinite(O[0])) and np.all(np.isfinite(LSE[0]))


def test_sparse_duplicate_entry_counts_twice():
    inp = _small_sparse(topk=2, p_invalid=0.0)
    a, c = int(inp.indices[0, 0, 0]), int(inp.indices[0, 0, 1])
    idx = np.array([[[a, a, c]]], dtype=np.int32)
    O, LSE = sparse_decode(inp.q[:1, :1], inp.kv, idx, inp.softmax_scale)
    rows = sparse_rows_f64(inp.kv, np.array([a, c]))
    q = bf16_to_f64(inp.q[0, 0])
    for h in range(16):
        za = inp.softmax_scale * math.fsum(q[h] * rows[0]); zc = inp.softmax_scale * math.fsum(q[h] * rows[1])
        wa = 2 * math.exp(za); wc = math.exp(zc)
        assert np.allclose(O[0, 0, h], (wa * rows[0, :512] + wc * rows[1, :512]) / (wa + wc), rtol=0, atol=1e-12)
        assert abs(LSE[0, 0, h] - math.log(wa + wc)) < 1e-12


def test_sparse_equals_paged_on_the_same_rows():
    """Sparse decode over all visible positions == paged decode on a cache holding the same values.

    With power-of-two scales every dequantised fp8 value is a bf16 value, so
    both entry points see identical rows.
    """
    rng = np.random.default_rng(23)
    T = 150
    rec = np.zeros((T, 640), dtype=np.uint8)
    codes = rng.integers(0, 256, size=(T, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38          # no NaN codes
    rec[:, :576] = codes
    rec[:, 576:580] = (2.0 ** rng.integers(-4, 3, size=T)).astype("<f4").view(np.uint8).reshape(T, 4)
    vals = sparse_rows_f64(rec, np.arange(T))
    kc, bt = _one_seq_cache(vals.astype(np.float32), page_order=rng.permutation(3))
    assert np.array_equal(bf16_to_f64(_bf16(vals.astype(np.float32))), vals)
    q = _bf16(rng.standard_normal((1, 2, 16, 576)))
    L = np.array([T], dtype=np.int32)
    Op, Lp = paged_decode(q, kc, bt[None], L, SIGMA, causal=True)
    idx = np.full((1, 2, T), -1, dtype=np.int32)
    idx[0, 0, :T - 1] = np.arange(T - 1)
    idx[0, 1, :] = np.arange(T)
    Os, Ls = sparse_decode(q, rec, idx, SIGMA)
    assert np.allclose(Op, Os, rtol=0, atol=1e-13) and np.allclose(Lp, Ls, rtol=0, atol=1e-13)


def _exact_records(rng, n):
    """fp8 records whose dequantised values are bf16 values: no NaN codes, power-of-two scales."""
    rec = np.zeros((n, 640), dtype=np.uint8)
    codes = rng.integers(0, 256, size=(n, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    rec[:, :576] = codes
    rec[:, 576:580] = (2.0 ** rng.integers(-4, 3, size=n)).astype("<f4").view(np.uint8).reshape(n, 4)
    return rec


def test_paged_fp8_equals_bf16_paged_on_the_same_values():
    """An fp8 paged cache and a bf16 paged cache holding the same values, through the same block
    tables (permuted pages, ragged lengths, causal with two queries), give the same result."""
    rng = np.random.default_rng(31)
    L = np.array([150, 70], dtype=np.int32)
    pages = 3 + 2
    rec = _exact_records(rng, pages * 64).reshape(pages, 64, 640)
    vals = sparse_rows_f64(rec.reshape(-1, 640), np.arange(pages * 64))
    kc = _bf16(vals.astype(np.float32)).reshape(pages, 64, 1, 576)
    assert np.array_equal(bf16_to_f64(kc).reshape(-1, 576), vals)
    perm = rng.permutation(pages).astype(np.int32)
    bt = np.array([perm[:3], np.r_[perm[3:], 0]], dtype=np.int32)
    q = _bf16(rng.standard_normal((2, 2, 16, 576)))
    Ob, Lb = paged_decode(q, kc, bt, L, SIGMA, causal=True)
    Of, Lf = paged_decode_fp8(q, rec, bt, L, SIGMA, causal=True)
    assert np.allclose(Ob, Of, rtol=0, atol=1e-13) and np.allclose(Lb, Lf, rtol=0, atol=1e-13)


def test_paged_fp8_equals_sparse_over_the_page_rows():
    """Paged fp8 decode == sparse decode whose index list names the same rows of the flattened
    pool (row = page * 64 + position in the page), in token order."""
    inp = make_paged_fp8(2, 1, 16, [130, 64], False, seed=41, poison=False)
    O, LSE = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, False)
    flat = inp.kcache.reshape(-1, 640)
    topk = int(inp.seqlens.max())
    idx = np.full((2, 1, topk), -1, dtype=np.int32)
    for b in range(2):
        t = np.arange(int(inp.seqlens[b]))
        idx[b, 0, :len(t)] = inp.block_table[b, t // 64] * 64 + t % 64
    Os, Ls = sparse_decode(inp.q, flat, idx, inp.softmax_scale)
    assert np.allclose(O, Os, rtol=0, atol=1e-13) and np.allclose(LSE, Ls, rtol=0, atol=1e-13)


def test_paged_fp8_never_reads_poisoned_records():
    """NaN records in unused block-table slots and past each sequence's end change nothing."""
    inp = make_paged_fp8(3, 2, 16, [100, 64, 5], True, seed=43, poison=True)
    O, LSE = paged_decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    assert np.isfinite(O).all() and np.isfinite(LSE).all()
    clean = make_paged_fp8(3, 2, 16, [100, 64, 5], True, seed=43, poison=False)
    Oc, Lc = paged_decode_fp8(clean.q, clean.kcache, clean.block_table, clean.seqlens, clean.softmax_scale, True)
    assert np.array_equal(O, Oc) and np.array_equal(LSE, Lc)


# ----------------------------------------------------------------- V4 geometry: 512-wide rows, sinks
def test_512_wide_rows_equal_576_with_zero_rope_dims():
    """A 512-wide latent row (K and V) scores like a 576-wide row whose 64 RoPE dims are zero in
    both q and k, and its value is the same 512 dims."""
    inp = make_paged(2, 2, 16, [150, 70], True, seed=51, poison=True, d_qk=512)
    O5, L5 = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    zq = np.zeros(inp.q.shape[:-1] + (64,), dtype=np.uint16)
    zk = np.zeros(inp.kcache.shape[:-1] + (64,), dtype=np.uint16)
    q576 = np.concatenate([inp.q, zq], axis=-1)
    k576 = np.concatenate([inp.kcache, zk], axis=-1)
    k576[inp.poison_page] = 0x7FC0
    O6, L6 = paged_decode(q576, k576, inp.block_table, inp.seqlens, inp.softmax_scale, True)
    assert np.allclose(O5, O6, rtol=0, atol=1e-12) and np.allclose(L5, L6, rtol=0, atol=1e-12)


def test_sink_of_minus_infinity_is_no_sink():
    inp = make_paged(2, 1, 16, [100, 3], False, seed=52, d_qk=512)
    O, LSE = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, False)
    Os, Ls = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, False,
                          sinks=np.full(16, -np.inf, dtype=np.float32))
    assert np.array_equal(O, Os) and np.array_equal(LSE, Ls)


def test_sink_closed_forms():
    """Equal scores z = 0 over n tokens with sink s: O = mean(V) * n / (n + e^s), LSE = ln(n + e^s).
    One token with score z0: O = v / (1 + e^(s - z0)), LSE = logaddexp(z0, s).  No tokens:
    O = 0, LSE = s."""
    rng = np.random.default_rng(53)
    n = 37
    rows = bf16_to_f64(_bf16(rng.standard_normal((n, 512))))
    s = np.array([-3.0, 0.0, 2.5, 9.0])
    o, lse = attend(np.zeros((4, 512)), rows, SIGMA, sink=s)
    for h in range(4):
        assert np.allclose(o[h], rows.mean(axis=0) * n / (n + math.exp(s[h])), rtol=0, atol=1e-13)
        assert abs(lse[h] - math.log(n + math.exp(s[h]))) < 1e-12
    q = bf16_to_f64(_bf16(rng.standard_normal((4, 512))))
    o1, l1 = attend(q, rows[:1], SIGMA, sink=s)
    z0 = SIGMA * rows[0] @ q.T
    for h in range(4):
        assert np.allclose(o1[h], rows[0] / (1 + math.exp(s[h] - z0[h])), rtol=1e-12, atol=1e-14)
        assert abs(l1[h] - np.logaddexp(z0[h], s[h])) < 1e-12
    o0, l0 = attend(q, rows[:0], SIGMA, sink=s)
    assert np.all(o0 == 0) and np.array_equal(l0, s)


def test_sink_is_a_valueless_part_in_the_split_combine():
    """Attention with a sink == lse_combine of the sink-free result and a part with O = 0 and
    LSE = sink (the identity the GPU combine uses for split rows)."""
    rng = np.random.default_rng(54)
    rows = bf16_to_f64(_bf16(rng.standard_normal((200, 512))))
    q = bf16_to_f64(_bf16(rng.standard_normal((8, 512))))
    s = rng.uniform(-2, 6, size=8)
    o, lse = attend(q, rows, SIGMA, sink=s)
    o_t, l_t = attend(q, rows, SIGMA)
    oc, lc = lse_combine(np.stack([o_t, np.zeros_like(o_t)]), np.stack([l_t, s]))
    assert np.allclose(o, oc, rtol=0, atol=1e-13) and np.allclose(lse, lc, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- V4 geometry: FP4 (E2M1) KV
def test_e2m1_golden_values_from_ocp_mx_spec():
    n = 0
    with open(os.path.join(GOLDEN, "e2m1_ocp.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code_s, val_s = line.split()
            code, val = int(code_s, 16), float(val_s)
            got = E2M1_TABLE[code]
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)
            n += 1
    assert n == 16


def test_every_fp4_value_times_every_ue4m3_scale_is_a_bf16_value():
    """E2M1 (2 significant bits) times a non-negative E4M3 scale (4 significant bits, 2^-9..448)
    has at most 6 significant bits and stays in bf16's range: the dequantised FP4 cache is
    exactly a bf16 cache."""
    scales = E4M3_TABLE[:0x7F]                       # every finite non-negative E4M3 byte
    prod = (E2M1_TABLE[:, None] * scales[None, :]).reshape(-1)
    back = bf16_to_f64(_bf16(prod.astype(np.float32)))
    assert np.array_equal(back, prod)


def test_fp4_row_layout_low_nibble_first_and_block16_scales():
    """Byte j of a row holds elements 2j (low nibble) and 2j+1 (high nibble); scale byte b
    multiplies elements 16b..16b+15 (hand-computed values)."""
    codes = np.zeros((1, 256), dtype=np.uint8)
    scales = np.full((1, 32), 0x38, dtype=np.uint8)  # 1.0
    codes[0, 0] = 0x21                               # elements 0, 1: 0.5, 1.0
    codes[0, 7] = 0xA3                               # elements 14, 15: 1.5, -1.0
    codes[0, 8] = 0xF7                               # elements 16, 17: 6, -6
    scales[0, 1] = 0x40                              # block 1 (elements 16..31): 2.0
    scales[0, 31] = 0x01                             # block 31: 2^-9
    codes[0, 255] = 0x70                             # elements 510, 511: 0, 6
    v = fp4_rows_f64(codes, scales)[0]
    want = np.zeros(512)
    want[[0, 1, 14, 15, 16, 17, 510, 511]] = [0.5, 1.0, 1.5, -1.0, 12.0, -12.0, 0.0, 6.0 * 2.0 ** -9]
    assert np.array_equal(v, want)


def test_fp4_generator_round_trip_within_the_format_bound():
    """Independently written quantiser (generator) and decoder (oracle): each value comes back
    within one block scale (half the widest E2M1 gap, 4 -> 6), with its sign, and the row error
    is far below the signal; a swapped nibble or a wrong magnitude table breaks both."""
    rng = np.random.default_rng(61)
    x = rng.standard_normal((300, 512)).astype(np.float32)
    codes, scales = quantize_rows_nvfp4(x)
    assert codes.shape == (300, 256) and scales.shape == (300, 32)
    assert (scales < 0x7F).all()
    xh = fp4_rows_f64(codes, scales)
    s = np.repeat(E4M3_TABLE[scales], 16, axis=1)
    assert (np.abs(xh - x) <= s * (1 + 1e-6)).all()
    assert ((np.sign(xh) == np.sign(x)) | (xh == 0)).all()
    rel = np.linalg.norm(xh - x, axis=1) / np.linalg.norm(x, axis=1)
    assert rel.max() < 0.2 and rel.mean() < 0.12


def test_paged_fp4_equals_bf16_latent512_on_the_same_values():
    """An FP4 paged cache and a bf16 512-wide cache holding the same (dequantised) values,
    through the same block tables (permuted pages, ragged, causal with s_q = 3, sinks), give
    the same result."""
    inp = make_paged_fp4(3, 3, 16, [150, 70, 2], True, seed=62, poison=True, sinks=True)
    P = inp.num_pages
    vals = fp4_rows_f64(inp.kv_codes.reshape(-1, 256), inp.kv_scales.reshape(-1, 32))
    kc = _bf16(vals.astype(np.float32)).reshape(P, 64, 1, 512)
    ok = np.isfinite(vals)
    assert np.array_equal(bf16_to_f64(kc).reshape(-1, 512)[ok], vals[ok])
    Ob, Lb = paged_decode(inp.q, kc, inp.block_table, inp.seqlens, inp.softmax_scale, True, sinks=inp.sinks)
    Of, Lf = paged_decode_fp4(inp.q, inp.kv_codes, inp.kv_scales, inp.block_table, inp.seqlens,
                              inp.softmax_scale, True, sinks=inp.sinks)
    assert np.isfinite(Of).all() and np.isfinite(Lf).all()
    assert np.array_equal(Ob, Of) and np.array_equal(Lb, Lf)


def test_paged_fp4_never_reads_poisoned_rows():
    """NaN-scaled rows in unused block-table slots and past each sequence's end change nothing."""
    args = (3, 2, 16, [100, 64, 5], True)
    inp = make_paged_fp4(*args, seed=63, poison=True)
    clean = make_paged_fp4(*args, seed=63, poison=False)
    O, LSE = paged_decode_fp4(inp.q, inp.kv_codes, inp.kv_scales, inp.block_table, inp.seqlens,
                              inp.softmax_scale, True)
    Oc, Lc = paged_decode_fp4(clean.q, clean.kv_codes, clean.kv_scales, clean.block_table, clean.seqlens,
                              clean.softmax_scale, True)
    assert np.isfinite(O).all() and np.array_equal(O, Oc) and np.array_equal(LSE, Lc)


def test_visible_count():
    assert visible_count(10, 1, 0, False) == 10
    assert visible_count(10, 1, 0, True) == 10
    assert [visible_count(10, 3, s, True) for s in range(3)] == [8, 9, 10]
    assert [visible_count(1, 3, s, True) for s in range(3)] == [0, 0, 1]
    assert visible_count(0, 2, 1, False) == 0


# ----------------------------------------------------------------- fused decode: norm, RoPE, FP8 cast
from mla_inputs import make_fused_extras, rope_angles  # noqa: E402
from oracle import (e4m3_encode, fp8_cast_rows, fused_decode, gather_paged_rows, rms_norm, rope_rotate,  # noqa: E402
                    round_bf16)


def test_round_bf16_matches_torch_and_ties_to_even():
    """Library special case: torch's float32 -> bfloat16 cast (nearest, ties to even); every bf16
    value is its own rounding; 1 + 2^-8 (a tie) goes to 1, 1 + 3 * 2^-8 to 1 + 2^-6."""
    rng = np.random.default_rng(69)
    x = np.concatenate([rng.standard_normal(50000) * 10.0, rng.standard_normal(50000) * 1e-3]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x), ref)
    assert np.array_equal(round_bf16(ref), ref)
    assert list(round_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]))) == [1.0, 1 + 2.0 ** -6]


def test_rms_norm_closed_forms():
    """Unit weight: the output's mean square is ms / (ms + eps); eps = 0 makes it scale-free and
    of unit RMS; the weight multiplies element by element."""
    rng = np.random.default_rng(60)
    x = rng.standard_normal((5, 512)) * rng.uniform(0.1, 10.0, size=(5, 1))
    ms = np.mean(x * x, axis=-1)
    y = rms_norm(x, np.ones(512), 1e-3)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-3), rtol=1e-13)
    y0 = rms_norm(x, np.ones(512), 0.0)
    assert np.allclose(np.sqrt(np.mean(y0 * y0, axis=-1)), 1.0, rtol=1e-14)
    assert np.allclose(rms_norm(7.5 * x, np.ones(512), 0.0), y0, rtol=1e-13)
    w = rng.standard_normal(512)
    assert np.allclose(rms_norm(x, w, 1e-3), y * w, rtol=1e-13, atol=1e-15)


def test_rope_rotation_conventions():
    """Angle 0 is the identity; a quarter turn maps each pair (a, b) of dims (448 + 2i, 449 + 2i)
    to (-b, a) and leaves dims below 448 alone; rotations keep pair norms; the conjugate rotation
    undoes the rotation."""
    rng = np.random.default_rng(61)
    x = rng.standard_normal((3, 512))
    assert np.array_equal(rope_rotate(x, np.ones(32), np.zeros(32)), x)
    y = rope_rotate(x, np.zeros(32), np.ones(32))
    assert np.array_equal(y[:, :448], x[:, :448])
    assert np.array_equal(y[:, 448::2], -x[:, 449::2]) and np.array_equal(y[:, 449::2], x[:, 448::2])
    th = rng.uniform(-math.pi, math.pi, size=(3, 32))
    z = rope_rotate(x, np.cos(th), np.sin(th))
    n0 = x[:, 448::2] ** 2 + x[:, 449::2] ** 2
    assert np.allclose(z[:, 448::2] ** 2 + z[:, 449::2] ** 2, n0, rtol=1e-13)
    assert np.allclose(rope_rotate(z, np.cos(th), np.sin(th), sign=-1.0), x, rtol=0, atol=1e-13)


def test_rope_angle_table():
    """The angle table: position 0 is the identity, pair 0 turns by exactly the position (base^0),
    the last pair by position * base^(-62/64)."""
    cs = rope_angles(np.array([0, 5]))
    assert np.array_equal(cs[0, :32], np.ones(32, dtype=np.float32)) and np.all(cs[0, 32:] == 0)
    assert cs[1, 0] == np.float32(math.cos(5.0)) and cs[1, 32] == np.float32(math.sin(5.0))
    a31 = 5.0 * 10000.0 ** (-62.0 / 64.0)
    assert cs[1, 31] == np.float32(math.cos(a31)) and cs[1, 63] == np.float32(math.sin(a31))


def test_e4m3_encode_matches_torch_and_rounds_ties_to_even():
    """Every finite E4M3 value encodes to its own code (library special case: torch's
    float8_e4m3fn cast); midpoints between neighbours go to the even code; 448 is the largest."""
    finite = np.array([c for c in range(256) if np.isfinite(E4M3_TABLE[c])])
    vals = E4M3_TABLE[finite].astype(np.float32)
    enc = e4m3_encode(vals)
    zero = vals == 0
    assert np.array_equal(enc[~zero], finite[~zero].astype(np.uint8))
    rng = np.random.default_rng(62)
    x = np.clip(np.concatenate([rng.standard_normal(20000) * 60.0, rng.standard_normal(20000) * 0.02]),
                -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)
    # 1.0625 lies between 1.0 (0x38) and 1.125 (0x39): even 0x38; 1.1875 between 0x39 and 0x3A: 0x3A
    assert list(e4m3_encode(np.array([1.0625, 1.1875, -1.0625, 448.0], dtype=np.float32))) == [0x38, 0x3A, 0xB8, 0x7E]


def test_fp8_row_cast_bounds():
    """The row's largest magnitude becomes +-448 exactly; every value is within half an E4M3 step
    of code * scale; an all-zero row gets the smallest scale and zero codes."""
    rng = np.random.default_rng(63)
    x = rng.standard_normal((6, 512)) * rng.uniform(1e-3, 1e3, size=(6, 1))
    x[5] = 0.0
    codes, scale = fp8_cast_rows(x)
    deq = E4M3_TABLE[codes] * scale[:, None].astype(np.float64)
    for r in range(5):
        j = np.argmax(np.abs(x[r]))
        assert codes[r, j] & 0x7F == 0x7E
        y = np.abs(x[r] / scale[r])
        step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3), 2.0 ** -9)
        assert np.all(np.abs(deq[r] - x[r]) <= 0.5 * step * scale[r] * (1 + 1e-6) + 1e-30)
    assert scale[5] == np.float32(np.float32(2.0 ** -126) / np.float32(448.0)) and np.all(codes[5] == 0)


def _fused_paged(inp, fx, sinks=None, round_query=True):
    rows_of = lambda b, L: gather_paged_rows(inp.kcache, inp.block_table[b], L)  # noqa: E731
    return fused_decode(inp.q, fx.norm_weight, fx.norm_eps, fx.rope_cs, rows_of, inp.block_table,
                        inp.seqlens, inp.softmax_scale, inp.causal, sinks=sinks, round_query=round_query)


def test_fused_single_token_is_the_counter_rotated_row():
    """One cached token: the attention output is that row, so the fused output before the cast is
    the row turned back by the query's angle, and the LSE is the score of the normed, rotated
    query (with unit norm weight and angle 0: the plain normed query's score)."""
    inp = make_paged(1, 1, 16, [1], False, seed=64, d_qk=512)
    fx = make_fused_extras(inp, 65)
    codes, scale, lse, O = _fused_paged(inp, fx)
    row = bf16_to_f64(inp.kcache[inp.block_table[0, 0], 0, 0])
    cos, sin = fx.rope_cs[0, 0, :32].astype(np.float64), fx.rope_cs[0, 0, 32:].astype(np.float64)
    assert np.allclose(O[0, 0], rope_rotate(np.tile(row, (16, 1)), cos, sin, sign=-1.0), rtol=0, atol=1e-14)
    fx.norm_weight[:] = 1.0
    fx.rope_cs[..., :32] = 1.0
    fx.rope_cs[..., 32:] = 0.0
    _, _, lse1, _ = _fused_paged(inp, fx, round_query=False)
    q = bf16_to_f64(inp.q[0, 0])
    qn = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + float(np.float32(1e-6)))
    assert np.allclose(lse1[0, 0], SIGMA_512 * qn @ row, rtol=1e-12, atol=1e-13)


SIGMA_512 = float(np.float32(512 ** -0.5))


def test_fused_output_depends_only_on_relative_positions():
    """Cached rows whose last 64 dims are rotated by their token positions and queries rotated by
    their own positions: moving every position by the same offset leaves the fused output (before
    the cast) and the LSE unchanged (up to the fp32 rounding of the angle table), while the
    attention output before the conjugate rotation moves.  A wrong sign or a missing rotation on
    either side breaks this."""
    rng = np.random.default_rng(66)
    T, s_q, h_q = 150, 2, 8
    base_rows = rng.standard_normal((T, 512))
    inp = make_paged(1, s_q, h_q, [T], True, seed=67, d_qk=512)
    fx = make_fused_extras(inp, 68)

    def run(offset):
        cs_k = rope_angles(offset + np.arange(T)).astype(np.float64)
        rot = rope_rotate(base_rows, cs_k[:, :32], cs_k[:, 32:])     # exact rows, no bf16 storage
        fx.rope_cs = rope_angles(offset + T - s_q + np.arange(s_q))[None]
        _, _, lse, O = fused_decode(inp.q, fx.norm_weight, fx.norm_eps, fx.rope_cs, lambda b, L: rot[:L],
                                    inp.block_table, inp.seqlens, inp.softmax_scale, True, round_query=False)
        cs_q = fx.rope_cs.astype(np.float64)[0][:, None, :]
        plain = rope_rotate(O[0], cs_q[..., :32], cs_q[..., 32:])  # the attention output itself
        return O, lse, plain

    O0, l0, p0 = run(0)
    O1, l1, p1 = run(1000)
    assert np.allclose(O0, O1, rtol=0, atol=1e-6) and np.allclose(l0, l1, rtol=0, atol=1e-6)
    assert np.abs(p0 - p1)[..., 448:].max() > 1e-2


def _one_seq_cache_512(rows_f32):
    T = rows_f32.shape[0]
    nblk = max(1, -(-T // 64))
    kc = np.zeros((nblk, 64, 1, 512), dtype=np.uint16)
    bits = _bf16(rows_f32)
    for j in range(nblk):
        n = min(64, T - 64 * j)
        kc[j, :n, 0, :] = bits[64 * j:64 * j + n]
    return kc, np.arange(nblk, dtype=np.int32)
