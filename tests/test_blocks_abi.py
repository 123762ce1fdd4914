"""The library's host block manager (include/kvq_blocks.h) against the
oracle model, call by call, on the host (no GPU)."""
import ctypes
import random
import subprocess
import sys

import numpy as np
import pytest

import paged_quantized_kv_kvq_amd as kvq
from oracle.blocks import Blocks, Exhausted

EXHAUSTED, INVALID, HOST_MEMORY = -6, -1, -7


def _same(bm: kvq.BlockManager, m: Blocks):
    assert bm.num_free() == len(m.free)
    assert [bm.ref_count(b) for b in range(m.num_blocks)] == m.count
    ids = sorted(m.seqs)
    if ids:
        mb = max(len(t) for _, t in m.seqs.values()) + 2
        bt, lens = bm.table(ids, mb)
        rows, mlens = m.table(ids, mb)
        assert bt.tolist() == rows and lens.tolist() == mlens


@pytest.mark.parametrize("seed,nb,bs", [(1, 40, 4), (2, 17, 1), (3, 64, 16), (4, 9, 3)])
def test_library_matches_model(seed, nb, bs):
    rng = random.Random(seed)
    bm, m = kvq.BlockManager(nb, bs), Blocks(nb, bs)
    for step in range(1500):
        op = rng.random()
        live = sorted(m.seqs)
        if op < 0.12 or not live:
            assert bm.seq_new() == m.seq_new()
        elif op < 0.22:
            p = rng.choice(live)
            assert bm.seq_fork(p) == m.seq_fork(p)
        elif op < 0.32:
            s = rng.choice(live)
            bm.seq_free(s)
            m.seq_free(s)
        elif op < 0.75:
            s, n = rng.choice(live), rng.randint(0, 3 * bs + 2)
            try:
                want = m.append(s, n)
            except Exhausted:
                with pytest.raises(kvq.KvqError) as e:
                    bm.append(s, n)
                assert e.value.status == EXHAUSTED
            else:
                slots, cow = bm.append(s, n)
                assert slots.tolist() == want[0] and cow == want[1]
        elif op < 0.85:
            sub = rng.sample(live, rng.randint(1, len(live)))
            cnt = [rng.randint(0, bs + 1) for _ in sub]
            try:
                want = m.append_many(sub, cnt)
            except Exhausted:
                with pytest.raises(kvq.KvqError) as e:
                    bm.append_many(sub, cnt)
                assert e.value.status == EXHAUSTED
            else:
                slots, cow = bm.append_many(sub, cnt)
                assert slots.tolist() == want[0] and [tuple(p) for p in cow.tolist()] == want[1]
        elif op < 0.97:
            s, n = rng.choice(live), rng.randint(0, 2 * bs + 1)
            assert bm.popn(s, n) == m.popn(s, n)
        else:
            bm.reset()
            m.reset()
        if step % 10 == 0:
            _same(bm, m)
    _same(bm, m)


def test_argument_checks():
    lib = kvq.load()
    h = ctypes.c_void_p()
    assert lib.kvq_blocks_create(0, 16, ctypes.byref(h)) == INVALID
    assert lib.kvq_blocks_create(8, 0, ctypes.byref(h)) == INVALID
    assert lib.kvq_blocks_create(1 << 31, 16, ctypes.byref(h)) == INVALID
    assert lib.kvq_blocks_create(8, 16, None) == INVALID
    bm = kvq.BlockManager(4, 16)
    s = bm.seq_new()
    for call in (lambda: bm.seq_free(s + 1), lambda: bm.seq_fork(7), lambda: bm.popn(3, 1),
                 lambda: bm.ref_count(4), lambda: bm.append(s + 5, 1), lambda: bm.seq_len(2)):
        with pytest.raises(kvq.KvqError) as e:
            call()
        assert e.value.status == INVALID
    bm.append(s, 40)                                     # 3 blocks
    with pytest.raises(kvq.KvqError):
        bm.table([s], 2)                                 # does not fit
    with pytest.raises(kvq.KvqError) as e:
        bm.append(s, 100)
    assert e.value.status == EXHAUSTED and bm.seq_len(s) == (40, 3) and bm.num_free() == 1
    assert kvq.load().kvq_status_string(EXHAUSTED) == b"no free block left"


def test_one_block_id_serves_every_layer_pool():
    # per-layer formats and dims: each layer's pools hold num_blocks blocks of
    # their own stride, and a slot from the manager addresses the same block
    # in every one of them
    bm = kvq.BlockManager(10, 16)
    s = bm.seq_new()
    slots, _ = bm.append(s, 20)
    for kf, vf, nkv, hd in [("bf16", "turbo4", 8, 128), ("turbo3", "turbo8", 4, 256), ("nvfp4", "fp8", 2, 64)]:
        lay = kvq.pool_layout(kf, vf, 16, nkv, hd)
        blocks = slots // 16
        assert np.all(blocks * lay.k_block_stride_bytes + lay.k_block_stride_bytes <= 10 * lay.k_block_stride_bytes)
        assert np.all(blocks * lay.v_block_stride_bytes + lay.v_block_stride_bytes <= 10 * lay.v_block_stride_bytes)


def test_append_many_rejects_repeats_and_unknown_ids():
    bm = kvq.BlockManager(8, 4)
    a, b = bm.seq_new(), bm.seq_new()
    for seqs in ([a, a], [a, 5]):
        with pytest.raises(kvq.KvqError) as e:
            bm.append_many(seqs, [1, 1])
        assert e.value.status == INVALID
    assert bm.num_free() == 8 and bm.seq_len(a) == (0, 0)
    slots, cow = bm.append_many([b, a], [5, 1])
    assert slots.tolist() == [0, 1, 2, 3, 4, 8] and cow.tolist() == [[-1, -1], [-1, -1]]


def test_host_allocation_failure_is_a_status():
    # a manager of 2^31 - 1 blocks needs 16 GiB of host tables; under a 3 GiB
    # address-space limit its allocation fails, and the library must turn
    # that into a status instead of letting the C++ exception cross the C
    # interface (which would abort the process)
    code = (
        "import ctypes, resource, sys\n"
        "resource.setrlimit(resource.RLIMIT_AS, (3 << 30, 3 << 30))\n"
        "lib = ctypes.CDLL(sys.argv[1])\n"
        "h = ctypes.c_void_p()\n"
        "big = lib.kvq_blocks_create(ctypes.c_uint32(0x7FFFFFFF), ctypes.c_uint32(16), ctypes.byref(h))\n"
        "ok = lib.kvq_blocks_create(ctypes.c_uint32(64), ctypes.c_uint32(16), ctypes.byref(h))\n"
        "lib.kvq_blocks_destroy(h)\n"
        "print(big, ok)\n")
    kvq.load()
    out = subprocess.run([sys.executable, "-c", code, kvq._LIB_PATH], capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == [str(HOST_MEMORY), "0"]
    assert kvq.load().kvq_status_string(HOST_MEMORY) == b"host memory exhausted"
