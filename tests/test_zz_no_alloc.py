"""kvq_paged_decode_noalloc (no workspace argument, the library's own per-GPU
scratch) against kvq_paged_decode with a caller workspace: the same kernels
and plan, so the outputs must be bit-identical.  Two calls in a row, the
second smaller, on the dense and the sparse-V path; a call whose workspace
would exceed the scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from synth.gpu import stage
from kvq_testlib import say

pytestmark = pytest.mark.gpu


def _both(kvq, st, w, S=None):
    """(workspace call, no-alloc call) outputs over the first S sequences."""
    S = w.num_seqs if S is None else S
    q, bt, ln = st.q[:S], st.bt_dev[:S].contiguous(), st.lens_dev[:S]
    inv = synth.inv_sqrt_d(w.head_dim)
    need = kvq.decode_workspace_bytes(st.layout, S, w.num_q_heads, bt.shape[1], w.sliding_window,
                                      w.sparse_v_threshold)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    ref = kvq.paged_decode(st.layout, q, st.k_pool, st.v_pool, bt, ln, inv, w.sliding_window,
                           w.sparse_v_threshold, st.k_scale, st.v_scale, workspace=ws)
    out = torch.full_like(ref, float("nan"))
    kvq.paged_decode_noalloc(st.layout, q, st.k_pool, st.v_pool, bt, ln, inv, w.sliding_window,
                             w.sparse_v_threshold, st.k_scale, st.v_scale, out=out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("kf,vf,thr,win", [("fp8", "turbo2", 0.0, 0), ("bf16", "turbo4", 1e-3, 0),
                                           ("turbo3", "turbo3", 1e-3, 700), ("turbo4", "turbo8", 0.0, 0)])
def test_noalloc_matches_workspace_call(gpu_lib, kf, vf, thr, win):
    w = synth.small(9100 + synth.FORMATS.index(kf) * 7 + synth.FORMATS.index(vf), lens=[3000, 0, 1, 517, 2048, 90],
                    num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16, k_format=kf, v_format=vf,
                    sparse_v_threshold=thr, sliding_window=win)
    say(f"case no-alloc decode {kf}/{vf} thr {thr} window {win}")
    st = stage(w, gpu_lib, "cuda", write_tail=0)
    for S in (w.num_seqs, 3):   # the second call is smaller: fewer sequences, fewer splits
        ref, out = _both(gpu_lib, st, w, S)
        assert torch.isfinite(ref).all()
        assert torch.equal(ref, out), f"no-alloc decode differs from the workspace call (S={S})"


def test_noalloc_refuses_oversized_call(gpu_lib):
    lib = gpu_lib.load()
    lay = gpu_lib.pool_layout("fp8", "turbo2", 16, 8, 128)
    # 1024 sequences of up to 32768 positions: the dense workspace is about 270 MB
    st = lib.kvq_paged_decode_noalloc(ctypes.byref(lay), None, None, None, None, None, None, 2048, 1024, 32,
                                      ctypes.c_float(0.088), 32 * 128, 0, ctypes.c_float(0.0), ctypes.c_float(1.0),
                                      ctypes.c_float(1.0), None)
    assert st == -4   # KVQ_ERR_WORKSPACE, nothing launched
