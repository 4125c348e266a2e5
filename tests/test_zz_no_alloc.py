"""GPU: mla_decode_paged_noalloc through the C ABI against mla_decode_paged with a caller
workspace, on two calls in a row (the second smaller, so it runs over the partials the first
left in the library's array), and against the float64 oracle."""

import ctypes

import numpy as np
import pytest

from mla_inputs import make_paged
from oracle import paged_decode
from tests.helpers import check_parity, dev_bf16, dev_i32, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_paged_amd as mla

    return mla, torch.device("cuda:0")


def _noalloc(mla, torch, dev, inp, P):
    """One mla_decode_paged_noalloc call made directly through the C ABI."""
    q, kc = dev_bf16(inp.q, dev), dev_bf16(inp.kcache, dev)
    bt, sl = dev_i32(inp.block_table, dev), dev_i32(inp.seqlens, dev)
    meta, ns = mla.get_metadata(sl, inp.h_q, inp.s_q, P)
    out = torch.empty((inp.batch, inp.s_q, inp.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.batch, inp.s_q, inp.h_q), dtype=torch.float32, device=dev)
    st = mla.lib.mla_decode_paged_noalloc(
        q.data_ptr(), kc.data_ptr(), kc.shape[0], bt.data_ptr(), bt.shape[1], sl.data_ptr(),
        inp.batch, inp.s_q, inp.h_q, ctypes.c_float(inp.softmax_scale), 1 if inp.causal else 0,
        meta.data_ptr(), ns.data_ptr(), meta.shape[0], out.data_ptr(), lse.data_ptr(),
        torch.cuda.current_stream(dev).cuda_stream)
    assert st == mla.MLA_OK, mla.status_string(st)
    torch.cuda.synchronize()
    return to_host(out, lse)


def _with_workspace(mla, torch, dev, inp, P):
    q, kc = dev_bf16(inp.q, dev), dev_bf16(inp.kcache, dev)
    bt, sl = dev_i32(inp.block_table, dev), dev_i32(inp.seqlens, dev)
    meta = mla.get_metadata(sl, inp.h_q, inp.s_q, P)
    out, lse = mla.decode_paged(q, kc, bt, sl, meta, inp.softmax_scale, inp.causal)
    torch.cuda.synchronize()
    return to_host(out, lse)


CASES = [
    # batch, s_q, h_q, seqlens, causal, num_parts: a large call, then smaller ones over the
    # partials it left behind (fewer slots, a causal 16-row shape, forced splits)
    (40, 1, 16, list(range(7, 40 * 75, 75)), False, 256),
    (3, 1, 16, [1000, 1, 65], False, 64),
    (2, 2, 8, [700, 130], True, 16),
]


def test_noalloc_matches_workspace_call(env):
    import torch

    mla, dev = env
    for case in CASES:
        batch, s_q, h_q, L, causal, P = case
        print("noalloc case", case, flush=True)
        inp = make_paged(batch, s_q, h_q, L, causal, seed=900 + batch, poison=True)
        assert mla.workspace_size(batch, s_q, h_q, P) <= mla.NOALLOC_SCRATCH_BYTES
        o, l = _noalloc(mla, torch, dev, inp, P)
        o_ws, l_ws = _with_workspace(mla, torch, dev, inp, P)
        # the same kernels over the same partition: identical bits
        assert np.array_equal(o, o_ws) and np.array_equal(l, l_ws), case
        o_ref, l_ref = paged_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.softmax_scale, causal)
        check_parity(o, l, o_ref, l_ref, "noalloc " + str(case))


def test_noalloc_rejects_shapes_beyond_its_array(env):
    import torch

    mla, dev = env
    inp = make_paged(2, 2, 128, [300, 20], True, seed=950, poison=False)
    q, kc = dev_bf16(inp.q, dev), dev_bf16(inp.kcache, dev)
    bt, sl = dev_i32(inp.block_table, dev), dev_i32(inp.seqlens, dev)
    meta, ns = mla.get_metadata(sl, inp.h_q, inp.s_q, 4096)
    assert mla.workspace_size(2, 2, 128, 4096) > mla.NOALLOC_SCRATCH_BYTES
    out = torch.empty((2, 2, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((2, 2, 128), dtype=torch.float32, device=dev)
    st = mla.lib.mla_decode_paged_noalloc(
        q.data_ptr(), kc.data_ptr(), kc.shape[0], bt.data_ptr(), bt.shape[1], sl.data_ptr(), 2, 2, 128,
        ctypes.c_float(inp.softmax_scale), 1, meta.data_ptr(), ns.data_ptr(), 4096, out.data_ptr(),
        lse.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    assert st == mla.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
