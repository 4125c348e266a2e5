"""libmla.so without a GPU: exports, status codes, argument validation, host metadata twin."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mla():
    import head_latent_attention_paged_amd as m

    return m


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(mla):
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(mla.lib, n), n
    assert sorted(names) == sorted(mla.EXPORTS)


def test_status_strings(mla):
    assert mla.status_string(0) == "MLA_OK"
    assert mla.status_string(3) == "MLA_ERR_WORKSPACE"
    assert mla.status_string(99) == "MLA_ERR_UNKNOWN"


def test_num_parts_and_workspace(mla):
    assert mla.num_parts(16, 1, num_cus=256) == 256
    assert mla.num_parts(128, 2, num_cus=256) % 8 == 0
    # more than 64 rows: one round of 128-row workgroups (256 rows -> 2 groups, 384 -> 3), with
    # no rounding to a multiple of 8 parts (384 rows: 85 parts, 255 of the 256 compute units)
    assert mla.num_parts(128, 2, num_cus=256) == 128
    assert mla.num_parts(64, 6, num_cus=256) == 85
    # up to 64 rows the part count stays a multiple of 8
    assert mla.num_parts(32, 2, num_cus=250) % 8 == 0
    assert mla.num_parts(32, 2, num_cus=256) == 512
    assert mla.num_parts(16, 1, num_cus=3) >= 1
    ws = mla.workspace_size(128, 1, 16, 256)
    assert ws >= (128 + 256) * 16 * 513 * 4
    assert mla.workspace_size(0, 1, 16, 8) == 0
    # enough work items (query tokens x 64-row groups) for one round: no split
    assert mla.sparse_splits(32, 6, 64, 2048) == 1
    # few query tokens: as many splits as fit one round of 256 items, at most topk / 32
    assert mla.sparse_splits(2, 1, 64, 2048) == 64
    assert mla.sparse_splits(8, 1, 64, 2048) == 32
    assert mla.workspace_size_sparse(1, 1, 16, 32, 1) == 0          # one split needs no workspace


def _paged_call(mla, fp8=False, **kw):
    args = dict(q=16, kc=16, nb=4, bt=16, maxb=1, sl=16, batch=1, s_q=1, h_q=16, scale=0.04, causal=0,
                meta=16, ns=16, P=8, ws=16, wsb=1 << 30, out=16, lse=16)
    args.update(kw)
    f = mla.lib.mla_decode_paged_fp8 if fp8 else mla.lib.mla_decode_paged
    return f(args["q"], args["kc"], args["nb"], args["bt"], args["maxb"], args["sl"],
                                    args["batch"], args["s_q"], args["h_q"], args["scale"], args["causal"],
                                    args["meta"], args["ns"], args["P"], args["ws"], args["wsb"],
                                    args["out"], args["lse"], None)


def test_paged_validation_before_launch(mla):
    # every case is rejected on the host, so no device is touched
    assert _paged_call(mla, q=None) == mla.MLA_ERR_INVALID_ARG
    assert _paged_call(mla, lse=None) == mla.MLA_ERR_INVALID_ARG
    assert _paged_call(mla, batch=0) == mla.MLA_ERR_INVALID_ARG
    assert _paged_call(mla, h_q=-1) == mla.MLA_ERR_INVALID_ARG
    assert _paged_call(mla, scale=float("nan")) == mla.MLA_ERR_INVALID_ARG
    assert _paged_call(mla, q=24) == mla.MLA_ERR_INVALID_ARG          # misaligned
    assert _paged_call(mla, s_q=64, h_q=128) == mla.MLA_ERR_UNSUPPORTED
    assert _paged_call(mla, wsb=100) == mla.MLA_ERR_WORKSPACE
    assert _paged_call(mla, ws=None) == mla.MLA_ERR_INVALID_ARG


def _noalloc_call(mla, **kw):
    a = dict(q=16, kc=16, nb=4, bt=16, maxb=1, sl=16, batch=1, s_q=1, h_q=16, scale=0.04, causal=0,
             meta=16, ns=16, P=8, out=16, lse=16)
    a.update(kw)
    return mla.lib.mla_decode_paged_noalloc(a["q"], a["kc"], a["nb"], a["bt"], a["maxb"], a["sl"], a["batch"],
                                            a["s_q"], a["h_q"], a["scale"], a["causal"], a["meta"], a["ns"],
                                            a["P"], a["out"], a["lse"], None)


def test_paged_noalloc_validation_before_launch(mla):
    # argument errors of mla_decode_paged, and a workspace beyond the library's array, are
    # rejected before the array is looked up or anything is launched (no device is touched)
    assert _noalloc_call(mla, q=None) == mla.MLA_ERR_INVALID_ARG
    assert _noalloc_call(mla, batch=0) == mla.MLA_ERR_INVALID_ARG
    assert _noalloc_call(mla, scale=float("nan")) == mla.MLA_ERR_INVALID_ARG
    assert _noalloc_call(mla, s_q=64, h_q=128) == mla.MLA_ERR_UNSUPPORTED
    # 16 rows: batch + parts up to 1022 fit in 32 MiB, 1023 do not
    assert mla.workspace_size(766, 1, 16, 256) <= mla.NOALLOC_SCRATCH_BYTES < mla.workspace_size(767, 1, 16, 256)
    assert _noalloc_call(mla, batch=767, P=256) == mla.MLA_ERR_WORKSPACE
    assert _noalloc_call(mla, batch=128, s_q=2, h_q=128, P=128) == mla.MLA_ERR_WORKSPACE


def test_paged_fp8_validation_before_launch(mla):
    # the same host checks as the bf16 call
    assert _paged_call(mla, fp8=True, kc=None) == mla.MLA_ERR_INVALID_ARG
    assert _paged_call(mla, fp8=True, nb=0) == mla.MLA_ERR_INVALID_ARG
    assert _paged_call(mla, fp8=True, scale=float("inf")) == mla.MLA_ERR_INVALID_ARG
    assert _paged_call(mla, fp8=True, wsb=100) == mla.MLA_ERR_WORKSPACE
    assert _paged_call(mla, fp8=True, s_q=64, h_q=128) == mla.MLA_ERR_UNSUPPORTED


def test_paged_latent512_validation_before_launch(mla):
    f = mla.lib.mla_decode_paged_latent512
    ok = dict(q=16, kc=16, nb=4, bt=16, maxb=1, sl=16, batch=1, s_q=6, h_q=64, scale=0.04, causal=1,
              sinks=None, meta=16, ns=16, P=8, ws=16, wsb=1 << 30, out=16, lse=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["kc"], a["nb"], a["bt"], a["maxb"], a["sl"], a["batch"], a["s_q"], a["h_q"],
                 a["scale"], a["causal"], a["sinks"], a["meta"], a["ns"], a["P"], a["ws"], a["wsb"],
                 a["out"], a["lse"], None)

    assert call(q=None) == mla.MLA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == mla.MLA_ERR_INVALID_ARG
    assert call(s_q=64, h_q=128) == mla.MLA_ERR_UNSUPPORTED
    assert call(wsb=100) == mla.MLA_ERR_WORKSPACE
    assert call(kc=24) == mla.MLA_ERR_INVALID_ARG                  # misaligned


def test_paged_fp4_validation_before_launch(mla):
    f = mla.lib.mla_decode_paged_fp4
    ok = dict(q=16, kc=16, ks=16, nb=4, bt=16, maxb=1, sl=16, batch=1, s_q=6, h_q=64, scale=0.04, causal=1,
              sinks=None, meta=16, ns=16, P=8, ws=16, wsb=1 << 30, out=16, lse=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["kc"], a["ks"], a["nb"], a["bt"], a["maxb"], a["sl"], a["batch"], a["s_q"],
                 a["h_q"], a["scale"], a["causal"], a["sinks"], a["meta"], a["ns"], a["P"], a["ws"], a["wsb"],
                 a["out"], a["lse"], None)

    assert call(q=None) == mla.MLA_ERR_INVALID_ARG
    assert call(ks=None) == mla.MLA_ERR_INVALID_ARG
    assert call(ks=20) == mla.MLA_ERR_INVALID_ARG                  # misaligned scales
    assert call(kc=24) == mla.MLA_ERR_INVALID_ARG                  # misaligned codes
    assert call(scale=float("nan")) == mla.MLA_ERR_INVALID_ARG
    assert call(nb=0) == mla.MLA_ERR_INVALID_ARG
    assert call(s_q=64, h_q=128) == mla.MLA_ERR_UNSUPPORTED
    assert call(wsb=100) == mla.MLA_ERR_WORKSPACE


def test_fused_validation_before_launch(mla):
    f = mla.lib.mla_decode_fused
    ok = dict(q=16, kc=16, ks=None, nb=4, bt=16, maxb=1, sl=16, batch=1, s_q=6, h_q=64, scale=0.04, causal=1,
              sinks=None, w=16, eps=1e-6, cs=16, meta=16, ns=16, P=8, ws=16, wsb=1 << 30, out=16, osc=16, lse=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["kc"], a["ks"], a["nb"], a["bt"], a["maxb"], a["sl"], a["batch"], a["s_q"], a["h_q"],
                 a["scale"], a["causal"], a["sinks"], a["w"], a["eps"], a["cs"], a["meta"], a["ns"], a["P"],
                 a["ws"], a["wsb"], a["out"], a["osc"], a["lse"], None)

    assert call(w=None) == mla.MLA_ERR_INVALID_ARG
    assert call(cs=None) == mla.MLA_ERR_INVALID_ARG
    assert call(osc=None) == mla.MLA_ERR_INVALID_ARG
    assert call(w=20) == mla.MLA_ERR_INVALID_ARG                   # misaligned weight
    assert call(cs=24) == mla.MLA_ERR_INVALID_ARG                  # misaligned angle table
    assert call(eps=-1.0) == mla.MLA_ERR_INVALID_ARG
    assert call(eps=float("nan")) == mla.MLA_ERR_INVALID_ARG
    assert call(ks=20) == mla.MLA_ERR_INVALID_ARG                  # misaligned FP4 scales
    assert call(s_q=64, h_q=128) == mla.MLA_ERR_UNSUPPORTED
    assert call(wsb=100) == mla.MLA_ERR_WORKSPACE


def test_sparse_validation_before_launch(mla):
    f = mla.lib.mla_decode_sparse
    ok = dict(q=16, kv=16, nt=10, idx=16, topk=64, batch=1, s_q=1, h_q=16, scale=0.04, splits=0,
              ws=16, wsb=1 << 30, out=16, lse=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["kv"], a["nt"], a["idx"], a["topk"], a["batch"], a["s_q"], a["h_q"], a["scale"],
                 a["splits"], a["ws"], a["wsb"], a["out"], a["lse"], None)

    assert call(idx=None) == mla.MLA_ERR_INVALID_ARG
    assert call(topk=0) == mla.MLA_ERR_INVALID_ARG
    assert call(splits=-1) == mla.MLA_ERR_INVALID_ARG
    assert call(scale=float("inf")) == mla.MLA_ERR_INVALID_ARG
    assert call(kv=8) == mla.MLA_ERR_INVALID_ARG
    assert call(splits=2, wsb=10) == mla.MLA_ERR_WORKSPACE
    assert call(h_q=5000) == mla.MLA_ERR_UNSUPPORTED


def test_sparse_prefill_validation_before_launch(mla):
    f = mla.lib.mla_sparse_prefill
    ok = dict(q=16, kv=16, nt=10, idx=16, topk=64, s_q=100, h_q=64, scale=0.04, splits=0,
              ws=16, wsb=1 << 30, out=16, lse=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["kv"], a["nt"], a["idx"], a["topk"], a["s_q"], a["h_q"], a["scale"],
                 a["splits"], a["ws"], a["wsb"], a["out"], a["lse"], None)

    assert call(idx=None) == mla.MLA_ERR_INVALID_ARG
    assert call(s_q=0) == mla.MLA_ERR_INVALID_ARG
    assert call(topk=0) == mla.MLA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == mla.MLA_ERR_INVALID_ARG
    assert call(out=8) == mla.MLA_ERR_INVALID_ARG
    assert call(splits=4, wsb=10) == mla.MLA_ERR_WORKSPACE
    assert call(h_q=5000) == mla.MLA_ERR_UNSUPPORTED
    assert call(s_q=(1 << 24) + 1) == mla.MLA_ERR_UNSUPPORTED


def test_metadata_validation(mla):
    assert mla.lib.mla_get_metadata(None, 1, 16, 1, 8, 16, 16, None) == mla.MLA_ERR_INVALID_ARG
    assert mla.lib.mla_get_metadata(16, 0, 16, 1, 8, 16, 16, None) == mla.MLA_ERR_INVALID_ARG
    assert mla.lib.mla_get_metadata(16, 20000, 16, 1, 8, 16, 16, None) == mla.MLA_ERR_UNSUPPORTED


def _check_partition(L, P, meta, ns):
    """Every (sequence, block) is covered by exactly one part; split counts and slots agree."""
    L = np.asarray(L)
    nb = (L + 63) // 64
    batch = len(L)
    cover = [np.zeros(n, dtype=np.int32) for n in nb]
    seen_slots = set()
    touched = np.zeros(batch, dtype=np.int32)
    for p in range(P):
        b0, k0, b1, k1, slot0 = meta[p, :5]
        assert (b0, k0) <= (b1, k1)
        for b in range(b0, min(b1, batch - 1) + 1):
            lo = k0 if b == b0 else 0
            hi = k1 if b == b1 else nb[b]
            if lo >= hi:
                continue
            cover[b][lo:hi] += 1
            slot = slot0 if b == b0 else ns[b]
            assert ns[b] <= slot < ns[b + 1]
            assert (b, slot) not in seen_slots
            seen_slots.add((b, slot))
            touched[b] += 1
    for b in range(batch):
        assert np.all(cover[b] == 1), b
    assert np.array_equal(np.diff(ns), touched)
    assert ns[0] == 0 and ns[-1] == touched.sum() <= batch + P


@pytest.mark.parametrize("L,P", [
    ([37, 130], 256), ([4096] * 128, 256), ([65536] * 16, 256), ([1, 64, 65, 0, 128, 3000], 7),
    ([0, 0, 5], 4), ([100] * 9, 1), (list(range(0, 3000, 37)), 64), ([8192, 1024, 5000], 128),
])
@pytest.mark.parametrize("h_q", [16, 128])
def test_host_metadata_partition(mla, L, P, h_q):
    meta, ns = mla.get_metadata_host(np.array(L, dtype=np.int32), P, h_q=h_q)
    _check_partition(L, P, meta, ns)


@pytest.mark.parametrize("h_q,overhead", [(16, 0), (64, 0), (128, 4)])
def test_host_metadata_balance(mla, h_q, overhead):
    """Equal shares of blocks plus a fixed cost per sequence: none up to 64 rows, four blocks above."""
    rng = np.random.default_rng(0)
    L = rng.integers(1024, 8193, size=128)
    P = 128
    meta, ns = mla.get_metadata_host(L.astype(np.int32), P, h_q=h_q)
    nb = (L + 63) // 64
    loads = []
    for p in range(P):
        b0, k0, b1, k1 = meta[p, :4]
        tot = 0
        for b in range(b0, min(b1, 127) + 1):
            lo = k0 if b == b0 else 0
            hi = k1 if b == b1 else nb[b]
            if hi > lo:
                tot += hi - lo + (overhead if lo == 0 else 0)
        loads.append(tot)
    # no part holds more than its equal share of the cost (a sequence's fixed cost may straddle
    # a part edge and is counted here whole, with its first block)
    assert max(loads) <= -(-(nb.sum() + overhead * len(L)) // P) + overhead
    assert sum(loads) == nb.sum() + overhead * len(L)
