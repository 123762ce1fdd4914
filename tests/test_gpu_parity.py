"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Write: pool bytes (slots, packed codes, scale bytes) bit-exact.  Decode:
max-abs <= 2e-3 and rel-L2 <= 1e-3 against the fp64 oracle, on the same
seeded inputs.  Pools are poison-filled and unused page-table entries point
at a poison block, and the decode workspace starts as NaN, so a stray read
shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

import synth
from synth.gpu import stage
from kvq_testlib import OracleCache, check_decode, say, timed

pytestmark = pytest.mark.gpu

FMTS = list(synth.FORMATS)
ALL_PAIRS = [(k, v) for k in FMTS for v in FMTS]


def _decode(kvq, st, out=None):
    w = st.w
    need = kvq.decode_workspace_bytes(st.layout, w.num_seqs, w.num_q_heads, st.bt.shape[1], w.sliding_window,
                                      w.sparse_v_threshold)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes
    return kvq.paged_decode(st.layout, st.q, st.k_pool, st.v_pool, st.bt_dev, st.lens_dev,
                            synth.inv_sqrt_d(w.head_dim), w.sliding_window, w.sparse_v_threshold,
                            st.k_scale, st.v_scale, out=out, workspace=ws)


def run(kvq, w, seqs=None, tail=None, label="", from_window=False, check_pools=True):
    seqs = list(range(w.num_seqs)) if seqs is None else list(seqs)
    say(f"case {label}: {w}")
    st = stage(w, kvq, "cuda", keep_host=seqs, write_tail=tail)
    if st.tail_slots.numel():
        kvq.reshape_and_cache(st.layout, st.tail_key, st.tail_value, st.k_pool, st.v_pool, st.tail_slots,
                              st.k_scale, st.v_scale)
    out = _decode(kvq, st)
    torch.cuda.synchronize()
    out_np = out.cpu().numpy()
    ora = OracleCache(st, seqs, from_window=from_window)
    if check_pools:
        ora.compare_pools(st)
    ref = ora.decode(st, synth.inv_sqrt_d(w.head_dim))
    e, rel, namb = check_decode(out_np, ref, seqs, label)
    say(f"  ok {label}: max-abs {e:.2e} rel-L2 {rel:.2e} ambiguous {namb}")
    return st, out


LENS = [0, 1, 15, 16, 17, 300, 1100]


@pytest.mark.parametrize("kf,vf", ALL_PAIRS)
def test_pairs_dense(gpu_lib, kf, vf):
    w = synth.small(1000 + FMTS.index(kf) * 5 + FMTS.index(vf), lens=LENS, num_q_heads=8, num_kv_heads=2,
                    head_dim=128, block_size=16, k_format=kf, v_format=vf)
    run(gpu_lib, w, tail=3, label=f"{kf}/{vf} dense")


@pytest.mark.parametrize("hd", [64, 256])
@pytest.mark.parametrize("kf,vf", [("bf16", "bf16"), ("fp8", "turbo2"), ("turbo3", "turbo3"),
                                   ("turbo4", "turbo3"), ("bf16", "turbo4"), ("turbo2", "fp8"), ("turbo8", "turbo8"),
                                   ("turbo4", "turbo8"), ("nvfp4", "nvfp4")])
def test_head_dims(gpu_lib, kf, vf, hd):
    w = synth.small(2000 + hd + FMTS.index(kf) * 5 + FMTS.index(vf), lens=[5, 64, 700], num_q_heads=4,
                    num_kv_heads=2, head_dim=hd, block_size=16, k_format=kf, v_format=vf)
    run(gpu_lib, w, tail=2, label=f"{kf}/{vf} hd{hd}")


@pytest.mark.parametrize("g", [1, 2, 8])
@pytest.mark.parametrize("kf,vf", [("bf16", "turbo4"), ("fp8", "turbo2"), ("turbo4", "turbo3"), ("turbo3", "turbo8"),
                                   ("nvfp4", "turbo4")])
def test_group_sizes(gpu_lib, kf, vf, g):
    w = synth.small(3000 + g * 10 + FMTS.index(kf) * 5 + FMTS.index(vf), lens=[33, 517, 260], num_q_heads=2 * g,
                    num_kv_heads=2, head_dim=128, block_size=16, k_format=kf, v_format=vf)
    run(gpu_lib, w, tail=1, label=f"{kf}/{vf} G{g}")


@pytest.mark.parametrize("bs", [1, 2, 32, 128])
def test_block_sizes(gpu_lib, bs):
    w = synth.small(4000 + bs, lens=[1, 77, 600, 257], num_q_heads=8, num_kv_heads=4, head_dim=128,
                    block_size=bs, k_format="fp8", v_format="turbo4")
    run(gpu_lib, w, tail=2, label=f"bs{bs}")


@pytest.mark.parametrize("hkv", [3, 6, 12, 16])
@pytest.mark.parametrize("kf,vf", [("bf16", "turbo4"), ("turbo4", "turbo3")])
def test_kv_head_counts(gpu_lib, kf, vf, hkv):
    # the dense matrix-core kernel serves up to eight kv heads per workgroup:
    # 3 and 6 in one workgroup, 12 as two of 6, 16 as two of 8
    w = synth.small(4500 + hkv * 10 + FMTS.index(kf) * 5 + FMTS.index(vf), lens=[70, 333, 16], num_q_heads=2 * hkv,
                    num_kv_heads=hkv, head_dim=128, block_size=16, k_format=kf, v_format=vf)
    run(gpu_lib, w, tail=2, label=f"{kf}/{vf} Hkv{hkv}")


@pytest.mark.parametrize("bs", [2, 32, 64])
@pytest.mark.parametrize("kf,vf", [("turbo2", "fp8"), ("turbo3", "turbo2"), ("turbo8", "turbo8"), ("nvfp4", "turbo3")])
def test_block_sizes_turbo_k(gpu_lib, kf, vf, bs):
    # chunks that start inside a page (block_size > 16) on the turbo-K matrix-core path
    w = synth.small(4700 + bs + FMTS.index(kf) * 5 + FMTS.index(vf), lens=[1, 95, 640, 300], num_q_heads=8,
                    num_kv_heads=4, head_dim=128, block_size=bs, k_format=kf, v_format=vf)
    run(gpu_lib, w, tail=2, label=f"{kf}/{vf} bs{bs}")


@pytest.mark.parametrize("thr", [1e-3, 0.05])
@pytest.mark.parametrize("kf,vf", [("bf16", "turbo4"), ("turbo3", "turbo3"), ("fp8", "fp8"), ("bf16", "bf16"),
                                   ("turbo4", "turbo2"), ("turbo4", "turbo8"), ("turbo8", "turbo3"), ("nvfp4", "nvfp4"),
                                   ("bf16", "nvfp4")])
def test_sparse_v(gpu_lib, kf, vf, thr):
    w = synth.small(5000 + int(thr * 1e4) + FMTS.index(kf) * 5 + FMTS.index(vf), lens=[0, 1, 40, 1500, 2100],
                    num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, k_format=kf, v_format=vf,
                    sparse_v_threshold=thr)
    run(gpu_lib, w, tail=2, label=f"{kf}/{vf} thr{thr}")


@pytest.mark.parametrize("win,thr", [(1, 0.0), (100, 0.0), (700, 1e-3), (5000, 0.0)])
def test_sliding_window(gpu_lib, win, thr):
    w = synth.small(6000 + win, lens=[0, 50, 333, 1600], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    block_size=16, k_format="turbo3", v_format="turbo4", sliding_window=win,
                    sparse_v_threshold=thr)
    run(gpu_lib, w, tail=1, label=f"window {win} thr {thr}")


def test_student_t_values(gpu_lib):
    w = synth.small(7000, lens=[900, 31], num_q_heads=16, num_kv_heads=4, head_dim=256, block_size=16,
                    k_format="turbo3", v_format="turbo3", dist="student_t5", outliers=False,
                    sparse_v_threshold=1e-3, sliding_window=512)
    run(gpu_lib, w, tail=4, label="student-t turbo3")


def test_decode_is_deterministic(gpu_lib):
    w = synth.small(8000, lens=[1000, 3000], num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                    k_format="bf16", v_format="turbo4", sparse_v_threshold=1e-3)
    st = stage(w, gpu_lib, "cuda", write_tail=0)
    a = _decode(gpu_lib, st).clone()
    b = _decode(gpu_lib, st)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and torch.equal(a, b)
    w2 = w.scaled(sparse_v_threshold=0.0)
    st.w = w2
    a = _decode(gpu_lib, st).clone()
    b = _decode(gpu_lib, st)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and torch.equal(a, b)


def test_nvfp4_write_ties_and_saturation(gpu_lib):
    # crafted rows: E2M1 ties at every binade (group absmax 6 * 2^k gives the
    # exact scale 2^k), saturation (absmax whose E4M3 scale rounds down),
    # zero and tiny groups, signed zeros; bytes must equal the oracle's
    from oracle import codecs as ocodecs
    from oracle import layout as olayout
    from oracle import write as owrite
    hd, nkv, bs, nb = 128, 2, 16, 4
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5,
                     -5.0, -0.0], np.float32)
    rng = np.random.default_rng(5)
    x = np.zeros((4, nkv, hd), np.float32)
    for h in range(nkv):
        for gi in range(hd // 16):
            x[0, h, gi * 16:(gi + 1) * 16] = rng.permutation(ties) * np.float32(2.0 ** (gi - 3 + 2 * h))
    x[1] = rng.standard_normal((nkv, hd)) * 2
    x[1, :, ::16] = 7.0                       # scale E4M3(7/6) = 1.125: 7 / 1.125 saturates to 6
    x[2, 0, :16] = -1e-30                     # scale underflows to 0: zero nibbles
    x[2, 1] = -0.0
    x[3] = rng.standard_normal((nkv, hd)) * 3
    bits = ocodecs.bf16_round_bits(x)
    lay = gpu_lib.pool_layout("nvfp4", "nvfp4", bs, nkv, hd)
    ks, vs = olayout.pool_layout("nvfp4", "nvfp4", bs, nkv, hd)
    slots = np.array([5, 17, 33, 62], np.int64)
    kp = gpu_lib.alloc_pool(lay, "k", nb, fill=0x7F)
    vp = gpu_lib.alloc_pool(lay, "v", nb, fill=0x7F)
    key = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    gpu_lib.reshape_and_cache(lay, key, key.clone(), kp, vp, torch.from_numpy(slots).cuda(), 1.0, 1.0)
    torch.cuda.synchronize()
    ok_ = np.full(nb * ks.block_stride_bytes, 0x7F, np.uint8)
    ov_ = np.full(nb * vs.block_stride_bytes, 0x7F, np.uint8)
    owrite.reshape_and_cache(ks, vs, bits, bits, ok_, ov_, slots)
    assert np.array_equal(kp.cpu().numpy(), ok_) and np.array_equal(vp.cpu().numpy(), ov_)


def _write_and_compare(kvq, kf, vf, hd, nkv, bs, kbits, vbits, slots, nb, k_scale=1.0, v_scale=1.0):
    """Write host bf16 bit rows [T, nkv, hd] through the library and the
    oracle into poison-filled pools; every pool byte must be equal."""
    from oracle import layout as olayout
    from oracle import write as owrite
    lay = kvq.pool_layout(kf, vf, bs, nkv, hd)
    ks, vs = olayout.pool_layout(kf, vf, bs, nkv, hd)
    kp = kvq.alloc_pool(lay, "k", nb, fill=0x7F)
    vp = kvq.alloc_pool(lay, "v", nb, fill=0x7F)
    key = torch.from_numpy(np.ascontiguousarray(kbits).view(np.int16)).view(torch.bfloat16).cuda()
    val = torch.from_numpy(np.ascontiguousarray(vbits).view(np.int16)).view(torch.bfloat16).cuda()
    kvq.reshape_and_cache(lay, key, val, kp, vp, torch.from_numpy(slots).cuda(), k_scale, v_scale)
    torch.cuda.synchronize()
    ok_ = np.full(nb * ks.block_stride_bytes, 0x7F, np.uint8)
    ov_ = np.full(nb * vs.block_stride_bytes, 0x7F, np.uint8)
    owrite.reshape_and_cache(ks, vs, kbits, vbits, ok_, ov_, slots, k_scale, v_scale)
    for side, g, o in (("K", kp.cpu().numpy(), ok_), ("V", vp.cpu().numpy(), ov_)):
        if not np.array_equal(g, o):
            bad = np.flatnonzero(g != o)
            raise AssertionError(f"{side} pool differs from the oracle at {bad.size} bytes, first {bad[:8].tolist()}")


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 0.37109375), (0.0123456789, 1.0)])
def test_fp8_write_every_bf16_pattern(gpu_lib, k_scale, v_scale):
    # every finite bf16 bit pattern (+-0, subnormals, the largest finites)
    # through both fp8 sides, at scale 1 and at scales that are not powers of
    # two (RN32(x / scale) then E4M3 with the clamp at 448); bytes bit-exact
    hd, nkv, bs = 128, 2, 16
    pat = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    pat = pat[((pat >> 7) & 0xFF) != 0xFF]                  # drop inf / NaN
    T = (pat.size + nkv * hd - 1) // (nkv * hd)
    kb = np.resize(pat, T * nkv * hd).reshape(T, nkv, hd)
    vb = np.roll(kb.ravel(), 1000).reshape(T, nkv, hd)
    nb = (T + bs - 1) // bs + 2
    slots = np.random.default_rng(7050).permutation(nb * bs)[:T].astype(np.int64)
    say(f"case fp8 write of {pat.size} bf16 patterns, scales {k_scale} / {v_scale}")
    _write_and_compare(gpu_lib, "fp8", "fp8", hd, nkv, bs, kb, vb, slots, nb, k_scale, v_scale)


def _crafted_rows(nkv, hd, seed):
    """bf16 bit rows that reach the grouped-scale formats' edge cases."""
    from oracle import codecs as ocodecs
    rng = np.random.default_rng(seed)
    rows = [
        np.ones(hd),                                  # rotates to (sqrt d, 0, ...): all-zero groups after the first
        np.full(hd, -0.0),                            # signed zeros everywhere
        np.zeros(hd),
        rng.standard_normal(hd) * 0.004,              # subnormal E4M3 group scales (< 2^-6)
        rng.standard_normal(hd) * 3e-5,               # group scales that underflow to 0
        rng.standard_normal(hd) * 1500.0,             # group scales clamped at 448
        np.eye(1, hd, 3).ravel() * 4.0,               # rotates to a constant: every element at the group max
        np.where(np.arange(hd) == 7, 3000.0, rng.standard_normal(hd) * 1e-3),   # one huge element
        rng.standard_normal(hd) * 1e-39,              # bf16 denormals
        np.repeat(rng.standard_normal(hd // 16) * 2.0, 16) * np.tile([1.0, -1.0], hd // 2),
    ]
    x = np.stack([np.stack([r if h == 0 else r[::-1] for h in range(nkv)]) for r in rows]).astype(np.float32)
    return ocodecs.bf16_round_bits(x)


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("kf,vf", [("turbo2", "turbo3"), ("turbo4", "turbo8"), ("turbo8", "turbo2"),
                                   ("turbo3", "turbo4")])
def test_turbo_write_crafted_rows(gpu_lib, kf, vf, hd):
    # all-zero groups, +-0, subnormal and underflowing E4M3 scales, scales
    # clamped at 448, every element at its group's max, a single huge element,
    # bf16 denormals; pool bytes (codes and scale bytes) bit-exact
    nkv, bs = 2, 16
    kb = _crafted_rows(nkv, hd, 7060 + hd)
    vb = kb[::-1].copy()
    T = kb.shape[0]
    nb = 4
    slots = np.random.default_rng(7061).permutation(nb * bs)[:T].astype(np.int64)
    say(f"case crafted write {kf}/{vf} hd{hd}")
    _write_and_compare(gpu_lib, kf, vf, hd, nkv, bs, kb, vb, slots, nb)


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("T", [1024, 1025])
@pytest.mark.parametrize("kf,vf", [("turbo4", "turbo3"), ("bf16", "fp8"), ("nvfp4", "turbo8"), ("turbo2", "bf16")])
def test_write_row_count_switch(gpu_lib, kf, vf, T, hd):
    # the write takes one wave per side up to 2048 (token, kv head) rows and
    # one wave for both sides above: 1024 tokens x 2 kv heads is the last
    # count of the first form, 1025 the first of the second; scattered slots
    # with about one in eight skipped (-1); pool bytes must equal the oracle's
    from oracle import layout as olayout
    from oracle import write as owrite
    nkv, bs = 2, 16
    nb = (T + bs - 1) // bs + 3
    say(f"case write {kf}/{vf} T={T} hd{hd}")
    rng = np.random.default_rng([7100, T, FMTS.index(kf), FMTS.index(vf), hd])
    kx = rng.standard_normal((T, nkv, hd)).astype(np.float32)
    vx = rng.standard_normal((T, nkv, hd)).astype(np.float32)
    kx[:, :, 5] *= 20.0
    kb = torch.from_numpy(kx).to(torch.bfloat16)
    vb = torch.from_numpy(vx).to(torch.bfloat16)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[rng.random(T) < 0.125] = -1
    k_scale = float(np.float32(kb.float().abs().max().item() / 448.0))
    v_scale = float(np.float32(vb.float().abs().max().item() / 448.0))
    lay = gpu_lib.pool_layout(kf, vf, bs, nkv, hd)
    ks, vs = olayout.pool_layout(kf, vf, bs, nkv, hd)
    kp = gpu_lib.alloc_pool(lay, "k", nb, fill=0x7F)
    vp = gpu_lib.alloc_pool(lay, "v", nb, fill=0x7F)
    gpu_lib.reshape_and_cache(lay, kb.cuda(), vb.cuda(), kp, vp, torch.from_numpy(slots).cuda(), k_scale, v_scale)
    torch.cuda.synchronize()
    ok_ = np.full(nb * ks.block_stride_bytes, 0x7F, np.uint8)
    ov_ = np.full(nb * vs.block_stride_bytes, 0x7F, np.uint8)
    owrite.reshape_and_cache(ks, vs, kb.view(torch.int16).numpy().view(np.uint16),
                             vb.view(torch.int16).numpy().view(np.uint16), ok_, ov_, slots, k_scale, v_scale)
    assert np.array_equal(kp.cpu().numpy(), ok_), "K pool differs from the oracle"
    assert np.array_equal(vp.cpu().numpy(), ov_), "V pool differs from the oracle"


# eight kv heads (the dense matrix-core pass's widest workgroup): every V
# format behind bf16 / fp8 K, at several shapes
EIGHT_V = ["bf16", "fp8", "turbo2", "turbo3", "turbo4", "turbo8", "nvfp4"]


@pytest.mark.parametrize("vf", EIGHT_V)
@pytest.mark.parametrize("kf", ["fp8", "bf16"])
def test_eight_kv_heads_formats(gpu_lib, kf, vf):
    hd = 64 if vf == "bf16" else 128    # V rows of at most 128 bytes
    w = synth.small(9300 + FMTS.index(kf) * 7 + FMTS.index(vf), lens=[0, 1, 15, 17, 300, 2100, 4133],
                    num_q_heads=32, num_kv_heads=8, head_dim=hd, block_size=16, k_format=kf, v_format=vf)
    run(gpu_lib, w, tail=2, label=f"Hkv8 {kf}/{vf} hd{hd}")


@pytest.mark.parametrize("g,hd,bs,win", [(1, 128, 16, 0), (2, 64, 32, 0), (8, 128, 16, 0), (4, 256, 16, 0),
                                         (4, 128, 64, 0), (4, 128, 32, 333), (8, 64, 16, 1000), (2, 256, 128, 0)])
def test_eight_kv_heads_shapes(gpu_lib, g, hd, bs, win):
    kf = "fp8" if hd == 256 else "bf16"
    w = synth.small(9400 + g * 100 + hd + bs + win, lens=[5, 64, 700, 1999, 3000], num_q_heads=8 * g,
                    num_kv_heads=8, head_dim=hd, block_size=bs, k_format=kf, v_format="turbo2",
                    sliding_window=win)
    run(gpu_lib, w, tail=1, label=f"Hkv8 G{g} hd{hd} bs{bs} W{win}")


# sparse-V with eight kv heads (bf16 / fp8 K rows of 64..256 bytes): several
# splits per sequence, every group size, windows that start inside a chunk,
# both thresholds
@pytest.mark.parametrize("kf,vf,hd,g,bs,win,thr", [
    ("bf16", "turbo4", 128, 4, 16, 0, 1e-3),
    ("bf16", "turbo4", 128, 4, 16, 0, 0.05),
    ("bf16", "bf16", 64, 1, 16, 0, 1e-3),
    ("bf16", "nvfp4", 64, 8, 32, 0, 0.05),
    ("fp8", "turbo2", 128, 2, 16, 333, 1e-3),
    ("fp8", "turbo8", 256, 4, 128, 0, 1e-3),
    ("fp8", "fp8", 64, 8, 16, 1000, 0.05),
    ("bf16", "turbo3", 128, 8, 64, 700, 1e-3),
    ("fp8", "turbo4", 128, 4, 32, 0, 1e-3),
])
def test_sparse_eight_kv_heads(gpu_lib, kf, vf, hd, g, bs, win, thr):
    w = synth.small(9600 + FMTS.index(kf) * 7 + FMTS.index(vf) + hd + 10 * g + bs + win, num_q_heads=8 * g,
                    lens=[0, 1, 15, 17, 511, 512, 513, 1500, 4133], num_kv_heads=8, head_dim=hd, block_size=bs,
                    k_format=kf, v_format=vf, sliding_window=win, sparse_v_threshold=thr)
    run(gpu_lib, w, tail=2, label=f"sparse Hkv8 {kf}/{vf} hd{hd} G{g} bs{bs} W{win} thr{thr}")


def _lens(seed, n, hi, zeros=0.1):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, hi + 1, n)
    lens[rng.random(n) < zeros] = 0
    return [int(x) for x in lens]


# sparse-V over many short sequences (and empty ones), with and without a
# window; block tables sized far beyond the sequences; thousands of sequences
@pytest.mark.parametrize("win", [0, 50])
def test_sparse_many_short_sequences(gpu_lib, win):
    w = synth.small(9700 + win, lens=_lens(9700 + win, 300, 200), num_q_heads=32, num_kv_heads=8, head_dim=128,
                    block_size=16, k_format="bf16", v_format="turbo4", sliding_window=win, sparse_v_threshold=1e-3)
    run(gpu_lib, w, tail=1, label=f"sparse 300 seqs W{win}")


def test_sparse_oversized_block_tables(gpu_lib):
    w = synth.small(9710, lens=_lens(9710, 64, 100), num_q_heads=16, num_kv_heads=8, head_dim=64, block_size=32,
                    k_format="fp8", v_format="turbo2", sparse_v_threshold=1e-3)
    w = w.scaled(seq_len=(1, 32768))   # block tables sized for 32768 positions
    run(gpu_lib, w, tail=1, label="sparse, oversized block tables")


def test_sparse_thousands_of_sequences(gpu_lib):
    w = synth.small(9720, lens=_lens(9720, 4200, 24), num_q_heads=8, num_kv_heads=8, head_dim=64, block_size=16,
                    k_format="bf16", v_format="bf16", sparse_v_threshold=0.05)
    run(gpu_lib, w, tail=0, label="sparse 4200 seqs")
