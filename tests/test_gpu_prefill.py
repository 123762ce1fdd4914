"""GPU parity of chunked prefill (kvq_paged_prefill, through the C ABI) against
the oracle's bottom-right causal attention, on pools written by the library.
Bars as for decode: max-abs <= 2e-3 and rel-L2 <= 1e-3 against fp64."""
import numpy as np
import pytest
import torch

import synth
from synth.gpu import stage
from kvq_testlib import MAX_ABS, REL_L2, OracleCache, say
from oracle import codecs as ocodecs
from oracle import prefill as oprefill

pytestmark = pytest.mark.gpu


def run_prefill(kvq, w, chunks, window=0, seed=0, label="", q_pad=0):
    say(f"case prefill {label}: {w} chunks {chunks}")
    seqs = list(range(w.num_seqs))
    st = stage(w, kvq, "cuda", keep_host=seqs, write_tail=0)
    C = np.minimum(np.asarray(chunks), st.lens)
    qs = np.concatenate([[0], np.cumsum(C)]).astype(np.int32)
    T = int(qs[-1])
    rng = np.random.default_rng(seed)
    q = ocodecs.bf16_round_bits(rng.standard_normal((T, w.num_q_heads, w.head_dim)).astype(np.float32))
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    if q_pad:  # rows with a larger stride: the same values inside a wider buffer
        wide = torch.zeros((T, w.num_q_heads + q_pad, w.head_dim), dtype=torch.bfloat16, device="cuda")
        wide[:, :w.num_q_heads] = qd
        qd = wide[:, :w.num_q_heads]
    mq = max(1, int(C.max()))
    need = kvq.prefill_workspace_bytes(st.layout, w.num_seqs, w.num_q_heads, st.bt.shape[1], mq, window)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")    # NaN bytes
    out = torch.full((T, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    inv = synth.inv_sqrt_d(w.head_dim)
    kvq.paged_prefill(st.layout, qd, st.k_pool, st.v_pool, st.bt_dev, st.lens_dev, torch.from_numpy(qs).cuda(), mq,
                      inv, window, st.k_scale, st.v_scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    ora = OracleCache(st, seqs)
    _, o64 = oprefill.paged_prefill(ora.ks, ora.vs, q, qs, ora.kp, ora.vp, ora.bt, st.lens, inv, window,
                                    st.k_scale, st.v_scale, seqs=seqs)
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    err = np.abs(g - o64)
    rel = np.sqrt(((g - o64) ** 2).sum() / max((o64 ** 2).sum(), 1e-300))
    assert err.max() <= MAX_ABS, f"{label}: max-abs {err.max():.3e}"
    assert rel <= REL_L2, f"{label}: rel-L2 {rel:.3e}"
    say(f"  ok prefill {label}: {T} queries, max-abs {err.max():.2e} rel-L2 {rel:.2e}")


LENS = [1, 17, 300, 1100, 2500]
CHUNKS = [1, 17, 37, 128, 600]   # the 17-long sequence is a whole prompt


@pytest.mark.parametrize("kf,vf", [("bf16", "turbo4"), ("fp8", "turbo2"), ("turbo4", "turbo3"), ("turbo8", "turbo8"),
                                   ("nvfp4", "nvfp4"), ("turbo3", "turbo8"), ("fp8", "fp8"), ("bf16", "nvfp4"),
                                   ("turbo2", "turbo4")])
def test_prefill_pairs(gpu_lib, kf, vf):
    w = synth.small(9000 + len(kf) * 7 + len(vf), lens=LENS, num_q_heads=8, num_kv_heads=2, head_dim=128,
                    block_size=16, k_format=kf, v_format=vf)
    run_prefill(gpu_lib, w, CHUNKS, seed=1, label=f"{kf}/{vf}")


@pytest.mark.parametrize("g", [1, 2, 8])
@pytest.mark.parametrize("kf,vf", [("bf16", "turbo4"), ("turbo4", "turbo3")])
def test_prefill_group_sizes(gpu_lib, kf, vf, g):
    w = synth.small(9100 + g * 10 + len(kf), lens=[40, 700, 333], num_q_heads=2 * g, num_kv_heads=2, head_dim=128,
                    block_size=16, k_format=kf, v_format=vf)
    run_prefill(gpu_lib, w, [40, 150, 9], seed=g, label=f"{kf}/{vf} G{g}")


@pytest.mark.parametrize("hd", [64, 256])
@pytest.mark.parametrize("kf,vf", [("fp8", "turbo2"), ("turbo4", "turbo4"), ("nvfp4", "turbo3")])
def test_prefill_head_dims(gpu_lib, kf, vf, hd):
    w = synth.small(9200 + hd + len(kf), lens=[90, 517], num_q_heads=8, num_kv_heads=2, head_dim=hd, block_size=16,
                    k_format=kf, v_format=vf)
    run_prefill(gpu_lib, w, [90, 64], seed=hd, label=f"{kf}/{vf} hd{hd}")


@pytest.mark.parametrize("win", [1, 100, 700])
def test_prefill_window(gpu_lib, win):
    w = synth.small(9300 + win, lens=[50, 333, 1600], num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                    k_format="turbo3", v_format="turbo4", sliding_window=win)
    run_prefill(gpu_lib, w, [50, 200, 900], window=win, seed=win, label=f"window {win}")


@pytest.mark.parametrize("bs", [32, 64])
def test_prefill_block_sizes(gpu_lib, bs):
    w = synth.small(9400 + bs, lens=[77, 600, 1000], num_q_heads=8, num_kv_heads=4, head_dim=128, block_size=bs,
                    k_format="fp8", v_format="turbo4")
    run_prefill(gpu_lib, w, [77, 33, 250], seed=bs, label=f"bs{bs}")


def test_prefill_empty_chunks_and_strided_q(gpu_lib):
    # an empty sequence, sequences without new queries between others, and q rows
    # whose stride is wider than Hq x hd
    w = synth.small(9500, lens=[300, 0, 64, 129, 17], num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                    k_format="turbo4", v_format="turbo8")
    run_prefill(gpu_lib, w, [33, 0, 0, 129, 5], seed=3, label="empty chunks, strided q", q_pad=3)


def test_prefill_long_chunk_sampled_rows(gpu_lib):
    # a 4096-query chunk at the end of 16384 positions and a 1000-query chunk of
    # a 9000-long sequence: 1024 tiles, tiles whose key range spans two splits
    # of 8192; sampled query rows (chunk edges, tile and split boundaries, random)
    w = synth.small(9600, lens=[16384, 9000], num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                    k_format="bf16", v_format="turbo3")
    say(f"case prefill long chunk: {w}")
    st = stage(w, gpu_lib, "cuda", keep_host=[0, 1], write_tail=0)
    C = np.array([4096, 1000])
    qs = np.array([0, 4096, 5096], np.int32)
    rng = np.random.default_rng(11)
    q = ocodecs.bf16_round_bits(rng.standard_normal((5096, w.num_q_heads, w.head_dim)).astype(np.float32))
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    inv = synth.inv_sqrt_d(w.head_dim)
    out = gpu_lib.paged_prefill(st.layout, qd, st.k_pool, st.v_pool, st.bt_dev, st.lens_dev, torch.from_numpy(qs).cuda(),
                                4096, inv)
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 3, 4, 5, 4095, 4094, 4096, 4097, 5095, 2047, 2048, 3807, 3808]) |
                  set(int(x) for x in rng.choice(5096, 24, replace=False)))
    ora = OracleCache(st, [0, 1])
    _, o64 = oprefill.paged_prefill(ora.ks, ora.vs, q, qs, ora.kp, ora.vp, ora.bt, st.lens, inv, 0,
                                    st.k_scale, st.v_scale, rows=set(rows))
    g = out.cpu().numpy()[rows].astype(np.float64)
    r = o64[rows]
    err = np.abs(g - r).max()
    rel = np.sqrt(((g - r) ** 2).sum() / (r ** 2).sum())
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert err <= MAX_ABS and rel <= REL_L2, f"long chunk: max-abs {err:.2e} rel-L2 {rel:.2e}"
    say(f"  ok prefill long chunk: {len(rows)} sampled rows, max-abs {err:.2e} rel-L2 {rel:.2e}")


# block_size < 4, which the tile kernel does not take: every query runs as a
# decode row through the decode kernels
@pytest.mark.parametrize("kf,vf,hd,bs", [("bf16", "turbo4", 128, 1), ("fp8", "turbo2", 128, 2),
                                         ("turbo4", "bf16", 128, 1), ("turbo8", "turbo8", 256, 2),
                                         ("turbo3", "turbo3", 64, 1), ("nvfp4", "fp8", 256, 2)])
def test_prefill_as_decode_rows(gpu_lib, kf, vf, hd, bs):
    w = synth.small(9800 + hd + bs + len(kf) * 3 + len(vf), lens=[1, 17, 300, 700], num_q_heads=8, num_kv_heads=2,
                    head_dim=hd, block_size=bs, k_format=kf, v_format=vf)
    run_prefill(gpu_lib, w, [1, 17, 40, 100], seed=hd + bs, label=f"rows {kf}/{vf} hd{hd} bs{bs}")


def test_prefill_as_decode_rows_window_and_empty(gpu_lib):
    w = synth.small(9850, lens=[300, 0, 64, 129, 17], num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=2,
                    k_format="turbo4", v_format="bf16")
    run_prefill(gpu_lib, w, [33, 0, 0, 129, 5], window=50, seed=5, label="rows, window 50, empty chunks", q_pad=2)


# the tile kernel (block_size >= 4): every K and V format, the three head
# sizes, every group size, block sizes around its key chunks, windows around
# chunk edges
TILE_V = ["bf16", "fp8", "turbo2", "turbo3", "turbo4", "turbo8", "nvfp4"]


@pytest.mark.parametrize("kf", TILE_V)
@pytest.mark.parametrize("vf", TILE_V)
def test_prefill_tiles_formats(gpu_lib, kf, vf):
    w = synth.small(9900 + TILE_V.index(vf) * 7 + TILE_V.index(kf), lens=[1, 17, 300, 1100, 2500], num_q_heads=16,
                    num_kv_heads=4, head_dim=128, block_size=16, k_format=kf, v_format=vf, outliers=True)
    run_prefill(gpu_lib, w, [1, 17, 37, 200, 600], seed=7, label=f"tiles {kf}/{vf}")


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("rot", [False, True])
def test_prefill_tiles_shapes(gpu_lib, hd, g, rot):
    if rot:
        kf = "turbo3" if g in (1, 4) else "turbo8"
    else:
        kf = "bf16" if g in (1, 4) else "fp8"
    vf = {64: "turbo3", 128: "nvfp4", 256: "turbo4"}[hd]
    w = synth.small(9950 + hd + g + 500 * rot, lens=[40, 700, 333], num_q_heads=2 * g, num_kv_heads=2, head_dim=hd,
                    block_size=16, k_format=kf, v_format=vf)
    run_prefill(gpu_lib, w, [40, 150, 9], seed=g + hd, label=f"tiles {kf}/{vf} hd{hd} G{g}")


@pytest.mark.parametrize("bs", [4, 8, 128, 512])
@pytest.mark.parametrize("kf", ["bf16", "turbo4"])
def test_prefill_tiles_block_sizes(gpu_lib, bs, kf):
    w = synth.small(9970 + bs + len(kf), lens=[77, 600, 1000, 5], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    block_size=bs, k_format=kf, v_format="turbo4")
    run_prefill(gpu_lib, w, [77, 33, 250, 5], seed=bs, label=f"tiles {kf} bs{bs}")


@pytest.mark.parametrize("win", [1, 63, 64, 65, 700])
def test_prefill_tiles_window(gpu_lib, win):
    w = synth.small(9990 + win, lens=[50, 333, 1600], num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                    k_format="fp8", v_format="turbo8", sliding_window=win)
    run_prefill(gpu_lib, w, [50, 200, 900], window=win, seed=win, label=f"tiles window {win}")


def test_prefill_tiles_empty_chunks_and_strided_q(gpu_lib):
    w = synth.small(9995, lens=[300, 0, 64, 129, 17], num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=4,
                    k_format="bf16", v_format="bf16")
    run_prefill(gpu_lib, w, [33, 0, 0, 129, 5], window=50, seed=5, label="tiles, window 50, empty chunks", q_pad=2)


# key splits: a grid of few tiles over long key ranges splits each range and
# merges the splits' partials; many sequences fill the grid without splits
@pytest.mark.parametrize("kf,vf,win", [("bf16", "turbo4", 0), ("turbo4", "turbo3", 0), ("fp8", "bf16", 3000),
                                       ("nvfp4", "turbo8", 0)])
def test_prefill_tiles_split_long(gpu_lib, kf, vf, win):
    w = synth.small(9700 + len(kf) + len(vf) + win, lens=[12000, 33], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    block_size=16, k_format=kf, v_format=vf, sliding_window=win)
    run_prefill(gpu_lib, w, [300, 33], window=win, seed=9, label=f"tiles split {kf}/{vf} window {win}")


def test_prefill_tiles_many_sequences_no_split(gpu_lib):
    lens = [int(x) for x in np.random.default_rng(77).integers(60, 400, 48)]
    w = synth.small(9760, lens=lens, num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                    k_format="bf16", v_format="turbo4")
    run_prefill(gpu_lib, w, [min(L, 100) for L in lens], seed=3, label="tiles, 48 sequences, no split")
