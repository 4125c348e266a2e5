"""The seeded input generators: determinism, bf16 rounding, fp8 quantisation, layouts."""

import numpy as np
import torch

from mla_inputs import (CONFIGS, bf16_bits_from_f32, bf16_bits_to_f32, make_config,
                        make_paged, make_sparse)
from mla_inputs.gen import quantize_rows_e4m3


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-40, 3.0e38, 1.00390625, 1.0117188], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(x), ref)
    assert np.array_equal(bf16_bits_to_f32(ref), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_paged_generator_is_deterministic_and_well_formed():
    a = make_paged(3, 2, 16, ("uniform", 10, 200), True, seed=9)
    b = make_paged(3, 2, 16, ("uniform", 10, 200), True, seed=9)
    for f in ("q", "kcache", "block_table", "seqlens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    nblk = (a.seqlens + 63) // 64
    used = np.concatenate([a.block_table[i, :nblk[i]] for i in range(3)])
    assert sorted(used.tolist()) == list(range(int(nblk.sum())))       # every pool page once
    for i in range(3):
        assert np.all(a.block_table[i, nblk[i]:] == a.poison_page)
        L = int(a.seqlens[i])
        last = a.block_table[i, (L - 1) // 64]
        if L % 64:
            assert np.all(a.kcache[last, L % 64:] == 0x7FC0)
        assert not np.any(a.kcache[last, :(L - 1) % 64 + 1] == 0x7FC0)
    assert a.softmax_scale == float(np.float32(576 ** -0.5))


def test_tiny_config_shape():
    c = make_config(1)
    assert c.q.shape == (2, 1, 16, 576)
    assert c.block_table.shape == (2, 3)
    assert c.kcache.shape == (5, 64, 1, 576)          # 4 pages + the poison page
    assert list(c.seqlens) == [37, 130]
    assert sorted(np.concatenate([c.block_table[0, :1], c.block_table[1]]).tolist()) == [0, 1, 2, 3]


def test_fp8_quantisation_round_trip():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 576)).astype(np.float32)
    rec = quantize_rows_e4m3(x)
    scale = rec[:, 576:580].copy().view("<f4").reshape(-1)
    vals = torch.from_numpy(rec[:, :576].copy()).view(torch.float8_e4m3fn).float().numpy() * scale[:, None]
    assert np.all(np.abs(vals - x) <= np.abs(x) * 2.0 ** -4 + scale[:, None] * 2.0 ** -9 + 1e-30)
    assert np.all(np.abs(rec[:, :576].astype(np.int32) & 0x7F) != 0x7F)     # no NaN codes
    assert np.all(rec[:, 580:] == 0)
    assert np.allclose(scale, np.abs(x).max(axis=1) / 448, rtol=1e-6)


def test_sparse_generator_indices():
    inp = make_sparse(2, 3, 16, 200, 50, 0.2, seed=3)
    assert inp.indices.shape == (2, 3, 50)
    for b in range(2):
        for s in range(3):
            row = inp.indices[b, s]
            valid = row[row >= 0]
            assert len(set(valid.tolist())) == valid.size                     # distinct
            assert np.all(valid >= b * 200) and np.all(valid <= b * 200 + 200 - 3 + s)
    frac = np.mean(inp.indices == -1)
    assert 0.05 < frac < 0.4
    again = make_sparse(2, 3, 16, 200, 50, 0.2, seed=3)
    assert np.array_equal(inp.indices, again.indices) and np.array_equal(inp.kv, again.kv)


def test_config_table():
    assert set(CONFIGS) == {1, 2, 3, 4, 5, 6, 7, 8, 9, 10}
    assert CONFIGS[10]["kind"] == "fused_v4"
    assert all(CONFIGS[10][k] == CONFIGS[7][k] for k in ("batch", "s_q", "h_q", "seqlens", "causal"))
    assert CONFIGS[9]["kind"] == "sparse_prefill" and CONFIGS[9]["batch"] == 1
    assert CONFIGS[2]["batch"] == 128 and CONFIGS[4]["seqlens"][0] == 65536
    assert CONFIGS[5]["topk"] == 2048
    # the fp8-cache workload is the memory-bound shape over fp8 records
    assert CONFIGS[6]["kind"] == "paged_fp8"
    assert all(CONFIGS[6][k] == CONFIGS[2][k] for k in ("batch", "s_q", "h_q", "seqlens", "causal"))


def test_v4_geometry_generator():
    inp = make_paged(3, 6, 8, [100, 64, 5], True, seed=5, d_qk=512, sinks=True)
    assert inp.q.shape == (3, 6, 8, 512) and inp.kcache.shape[1:] == (64, 1, 512)
    assert abs(inp.softmax_scale - float(np.float32(512 ** -0.5))) == 0
    assert inp.sinks.shape == (8,) and inp.sinks.dtype == np.float32
    mean_l = np.log(np.mean([100, 64, 5]))
    assert np.all(np.abs(inp.sinks - mean_l) <= 2.0 + 1e-6)
    # the draws before the sinks are those of the same call without sinks
    plain = make_paged(3, 6, 8, [100, 64, 5], True, seed=5, d_qk=512)
    assert np.array_equal(plain.kcache, inp.kcache) and plain.sinks is None


def test_paged_fp8_generator():
    from mla_inputs import make_paged_fp8
    inp = make_paged_fp8(3, 2, 16, [100, 64, 5], True, seed=5)
    assert inp.kcache.shape == (2 + 1 + 1 + 1, 64, 640) and inp.kcache.dtype == np.uint8
    assert inp.poison_page == 4
    # pages handed out once, unused slots on the poison page
    used = np.concatenate([inp.block_table[0, :2], inp.block_table[1, :1], inp.block_table[2, :1]])
    assert sorted(used.tolist()) == [0, 1, 2, 3]
    assert inp.block_table[1, 1] == 4 and inp.block_table[2, 1] == 4
    # records past a sequence's end carry NaN codes and a NaN scale
    last = inp.kcache[inp.block_table[0, 1], 100 - 64:]
    assert np.all(last[:, :576] == 0x7F)
    assert np.isnan(last[:, 576:580].copy().view("<f4")).all()
    # in-range records: finite positive scales
    sc = inp.kcache[inp.block_table[1, 0], :, 576:580].copy().view("<f4")
    assert np.all(np.isfinite(sc)) and np.all(sc > 0)


def test_paged_fp4_generator():
    from mla_inputs import make_paged_fp4
    inp = make_paged_fp4(3, 6, 8, [100, 64, 5], True, seed=5, sinks=True)
    assert inp.q.shape == (3, 6, 8, 512)
    assert inp.kv_codes.shape == (5, 64, 256) and inp.kv_scales.shape == (5, 64, 32)
    assert inp.kv_codes.dtype == np.uint8 and inp.kv_scales.dtype == np.uint8
    assert inp.poison_page == 4 and inp.block_table[1, 1] == 4
    assert abs(inp.softmax_scale - float(np.float32(512 ** -0.5))) == 0
    # rows past a sequence's end and the poison page carry NaN scale bytes; used rows valid ones
    assert np.all(inp.kv_scales[inp.block_table[0, 1], 100 - 64:] == 0x7F)
    assert np.all(inp.kv_scales[4] == 0x7F)
    assert np.all(inp.kv_scales[inp.block_table[1, 0]] < 0x7F)
    # the same page permutation and query draws as the bf16 512-wide generator
    plain = make_paged(3, 6, 8, [100, 64, 5], True, seed=5, d_qk=512, sinks=True)
    assert np.array_equal(plain.block_table, inp.block_table) and np.array_equal(plain.q, inp.q)
    assert CONFIGS[8]["kind"] == "paged_v4_fp4"
