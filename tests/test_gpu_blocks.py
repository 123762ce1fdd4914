"""The host block manager driving the GPU path: appends (with a fork and its
copy on write), a rollback, and a decode over the manager's block tables,
against the oracle doing the same steps with its own block model, writer and
decode."""
import zlib

import numpy as np
import pytest
import torch

import paged_quantized_kv_kvq_amd as kvq
import synth
from kvq_testlib import check_decode, say
from oracle import codecs as ocodecs
from oracle import decode as odecode
from oracle import layout as olayout
from oracle import write as owrite
from oracle.blocks import Blocks

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kf,vf,bs,thr", [("turbo4", "turbo3", 16, 0.0), ("bf16", "nvfp4", 32, 1e-3),
                                          ("fp8", "turbo8", 16, 0.0)])
def test_block_manager_drives_write_and_decode(gpu_lib, kf, vf, bs, thr):
    nkv, hd, G, nb = 2, 128, 4, 48
    say(f"case blocks {kf}/{vf} bs{bs} thr{thr}")
    lay = gpu_lib.pool_layout(kf, vf, bs, nkv, hd)
    ks, vs = olayout.pool_layout(kf, vf, bs, nkv, hd)
    bm, model = kvq.BlockManager(nb, bs), Blocks(nb, bs)
    kp = gpu_lib.alloc_pool(lay, "k", nb, fill=0x7F)
    vp = gpu_lib.alloc_pool(lay, "v", nb, fill=0x7F)
    okp = np.full(nb * ks.block_stride_bytes, 0x7F, np.uint8)
    ovp = np.full(nb * vs.block_stride_bytes, 0x7F, np.uint8)
    rng = np.random.default_rng(zlib.crc32(f"{kf}/{vf}/{bs}".encode()))
    kscale = vscale = float(np.float32(60.0 / 448.0))

    def copy_block(src, dst):
        for pool, opool, stride in ((kp, okp, ks.block_stride_bytes), (vp, ovp, vs.block_stride_bytes)):
            pool.view(nb, stride)[dst] = pool.view(nb, stride)[src]
            opool.reshape(nb, stride)[dst] = opool.reshape(nb, stride)[src]

    def append(seq, n):
        slots, cow = bm.append(seq, n)
        mslots, mcow = model.append(seq, n)
        assert slots.tolist() == mslots and cow == mcow
        if cow[0] >= 0:
            copy_block(*cow)
        x = rng.standard_normal((2, n, nkv, hd)).astype(np.float32) * 3
        bits = ocodecs.bf16_round_bits(x)
        key = torch.from_numpy(bits[0].view(np.int16)).view(torch.bfloat16).cuda()
        val = torch.from_numpy(bits[1].view(np.int16)).view(torch.bfloat16).cuda()
        gpu_lib.reshape_and_cache(lay, key, val, kp, vp, torch.from_numpy(slots).cuda(), kscale, vscale)
        owrite.reshape_and_cache(ks, vs, bits[0], bits[1], okp, ovp, np.asarray(mslots, np.int64), kscale, vscale)
        return cow

    a = bm.seq_new()
    assert model.seq_new() == a
    append(a, 100)
    b = bm.seq_fork(a)
    assert model.seq_fork(a) == b
    cow = append(b, 30)                        # the shared, partly filled last block is copied first
    assert cow[0] >= 0
    append(a, 7)
    assert bm.popn(a, 20) == model.popn(a, 20) == 20
    append(a, 5)                               # rewrites positions 87..91
    c = bm.seq_new()
    assert model.seq_new() == c
    append(c, 40)
    d = bm.seq_fork(c)
    assert model.seq_fork(c) == d
    bm.seq_free(c)
    model.seq_free(c)
    append(d, 9)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), okp) and np.array_equal(vp.cpu().numpy(), ovp)

    seqs = [a, b, d]
    mb = 16
    bt, lens = bm.table(seqs, mb)
    rows, mlens = model.table(seqs, mb)
    assert bt.tolist() == rows and lens.tolist() == mlens
    q = ocodecs.bf16_round_bits(rng.standard_normal((len(seqs), nkv * G, hd)).astype(np.float32))
    inv = synth.inv_sqrt_d(hd)
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    need = gpu_lib.decode_workspace_bytes(lay, len(seqs), nkv * G, mb, 0, thr)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    out = gpu_lib.paged_decode(lay, qd, kp, vp, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(), inv, 0,
                               thr, kscale, vscale, workspace=ws)
    torch.cuda.synchronize()
    ref = odecode.paged_decode(ks, vs, q, okp, ovp, np.asarray(rows, np.int32), np.asarray(mlens), inv, 0, thr,
                               kscale, vscale, detail=True)
    e, rel, namb = check_decode(out.cpu().numpy(), ref, list(range(len(seqs))), "blocks")
    say(f"  ok blocks {kf}/{vf}: max-abs {e:.2e} rel-L2 {rel:.2e} ambiguous {namb}")
