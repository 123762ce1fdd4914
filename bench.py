"""Benchmark: paged quantized KV write + paged decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--also 3]

A step is one pass of the whole hot path over one batch: every sequence's new
token is written into the paged pools (kvq_reshape_and_cache, scattered slots)
and then every sequence decodes one token over its pages (kvq_paged_decode).
Inputs are seeded synthetic data of the workload's shapes, staged in HBM
before the timed region.  Prints one JSON line: the headline workload
(bf16 K / turbo4 V with the sparse-V skip) at the top level, and the second
target workload (fp8 K / turbo2 V, dense, 128 x 32768) under
"configs" (--also 0: none).

value      effective KV GB/s: K+V bytes of every attended (position, kv head)
           at the storage formats' sizes (the dense-window bytes), per step
           time.  The sparse path skips most V rows, so this counts bytes it
           never reads; pct_hbm_peak and roofline.frac count only what must
           move.  Step and decode times are medians of per-step HIP events;
           between steps a 1 GiB scratch read evicts L2 and the MALL (--warm:
           no eviction), outside the timed region.
roofline   the decode call (sparse: score pass, V pass; dense: split pass,
           merge) timed with HIP events on the stream the library
           launches on; algorithmic bytes = K of every attended position + V
           of every (position, kv head) some head of the group keeps (counted
           from the stored K) + q + out + the page-table entries and lengths
           read.  `traffic` = HBM bytes per decode call from the committed
           rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the same sources.
roofline_alu  the same call against the fp32 VALU ceiling of the build
           (packed fp32 off: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz
           = 78.6 TFLOP/s).
stream_read_ref  libkvq_probe.so's page-read kernel over the same page size,
           pages in shuffled order, nothing computed: the practical read
           ceiling of this GPU for the pool's access pattern; `lds_direct`
           is the same read with the pages loaded straight into LDS.
cpu_baseline  the CPU oracle timed on a sample of the same workload, in
           worker processes (one per core of the process's CPU set, at most
           16); its outputs are also checked against the GPU's (parity).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from synth.gpu import stage  # noqa: E402

HBM_PEAK_GBS = 8000.0
VALU_PEAK_TFLOPS = 78.6       # fp32 VALU without packed math: 256 x 4 x 16 x 2 x 2.4e9
MFMA_BF16_TFLOPS = 2500.0     # dense matrix peaks of MI355X
MFMA_F32_TFLOPS = 157.3
ROW_BYTES = {"bf16": lambda hd: 2 * hd, "fp8": lambda hd: hd, "turbo4": lambda hd: hd // 2 + hd // 16,
             "turbo3": lambda hd: hd * 3 // 8 + hd // 16, "turbo2": lambda hd: hd // 4 + hd // 16,
             "turbo8": lambda hd: hd + hd // 8, "nvfp4": lambda hd: hd // 2 + hd // 16}
METRIC = "paged-decode effective KV GB/s (% of HBM peak) + decode tokens/s, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_quantized_kv_kvq_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _k_rows(st, w, kvq, j: torch.Tensor, pages: torch.Tensor) -> torch.Tensor:
    """Stored K of positions j of one sequence as fp32 [Hkv, hd, P], read
    back from the pool bytes with plain torch ops (turbo: in the rotated
    basis, codes -> centroid x E4M3 group scale, turbo8 E4M3 value x BF16
    group scale; nvfp4, not rotated: E2M1 value x E4M3 group scale; fp8:
    E4M3 x k_scale)."""
    Hkv, hd, bs = w.num_kv_heads, w.head_dim, w.block_size
    lay = st.layout
    stride, data = int(lay.k_block_stride_bytes), int(lay.k_data_section_bytes)
    pages = pages.long()
    rows = (j % bs)[:, None] * Hkv + torch.arange(Hkv, device="cuda")[None, :]    # [P, Hkv]
    base = pages[:, None] * stride                                                # [P, 1]
    pool = st.k_pool
    if w.k_format == "bf16":
        off = (base + rows * 2 * hd)[:, :, None] + torch.arange(0, 2 * hd, 2, device="cuda")
        lo, hi = pool[off].int(), pool[off + 1].int()
        k = ((lo | (hi << 8)) << 16).view(torch.float32)
    elif w.k_format == "fp8":
        off = (base + rows * hd)[:, :, None] + torch.arange(hd, device="cuda")
        k = pool[off].view(torch.float8_e4m3fn).float() * st.k_scale
    elif w.k_format == "turbo8":
        i = torch.arange(hd, device="cuda")
        off = (base + rows * hd)[:, :, None] + i
        soff = (base + data + rows * (hd // 8))[:, :, None] + 2 * (i // 16)
        sc = ((pool[soff].int() | (pool[soff + 1].int() << 8)) << 16).view(torch.float32)
        k = pool[off].view(torch.float8_e4m3fn).float() * sc
    else:
        bits = int(w.k_format[-1])
        rb = hd * bits // 8
        i = torch.arange(hd, device="cuda")
        bit = i * bits
        off = (base + rows * rb)[:, :, None] + (bit // 8)
        word = pool[off].int() | (pool[off + 1].int() << 8)
        code = (word >> (bit % 8)) & ((1 << bits) - 1)
        if w.k_format == "nvfp4":  # E2M1 value of each nibble
            cen = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], device="cuda")
        else:
            cen = torch.as_tensor(kvq.codebook(w.k_format)["centroids"], device="cuda")
        soff = (base + data + rows * (hd // 16))[:, :, None] + i // 16
        sq = pool[soff].view(torch.float8_e4m3fn).float()
        k = cen[code.long()] * sq
    return k.permute(1, 2, 0).contiguous()


def _hadamard(n: int) -> torch.Tensor:
    h = torch.ones(1, 1, dtype=torch.float64)
    while h.shape[0] < n:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    return h / math.sqrt(n)


def kept_rows(st, w, kvq) -> int:
    """(position, kv head) pairs whose V some query head of the group keeps.

    Measurement bookkeeping only (plain torch on the device): scores from the
    K actually stored in the pool, in fp32 (turbo K: the query rotated by
    the orthonormal Hadamard matrix, which leaves the scores unchanged).
    """
    S, G, Hkv, hd = w.num_seqs, w.group, w.num_kv_heads, w.head_dim
    P = _attended(st, w)
    if w.sparse_v_threshold <= 0.0:
        return int(P.sum()) * Hkv
    bs = w.block_size
    total = 0
    inv = synth.inv_sqrt_d(hd)
    rot = _hadamard(hd).float().cuda() if w.k_format.startswith("turbo") else None
    for s in range(S):
        L = int(st.lens[s])
        j0 = max(0, L - w.sliding_window) if w.sliding_window else 0
        if L <= j0:
            continue
        j = torch.arange(j0, L, device="cuda")
        K = _k_rows(st, w, kvq, j, st.bt_dev[s, (j // bs)])       # [Hkv, hd, P]
        q = st.q[s].float().view(Hkv, G, hd)
        if rot is not None:
            q = torch.matmul(q, rot)
        sc = torch.matmul(q.contiguous(), K) * inv                  # [Hkv, G, P]
        p = torch.softmax(sc, dim=-1)
        total += int((p > w.sparse_v_threshold).any(dim=1).sum())
    return total


def stream_read_reference(page_bytes: int, total_bytes: int = 4 << 30) -> dict:
    """libkvq_probe.so's page-read kernel: pages of `page_bytes` (rounded down to
    a multiple of 1 KiB) in shuffled order over `total_bytes`, read whole,
    nothing computed (a reference ceiling, not a kernel of this path)."""
    import ctypes
    path = os.path.join(ROOT, "paged_quantized_kv_kvq_amd", "libkvq_probe.so")
    if not os.path.exists(path):
        return {"kernel": "page_read_kernel", "gbs": None, "note": "libkvq_probe.so not built"}
    lib = ctypes.CDLL(path)
    lib.kvq_probe_page_read.restype = ctypes.c_double
    lib.kvq_probe_page_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    pb = max(1024, page_bytes // 1024 * 1024)
    n = total_bytes // pb
    pool = torch.ones(n * pb, dtype=torch.uint8, device="cuda")
    pages = torch.randperm(n, generator=torch.Generator().manual_seed(5)).to(torch.int32).cuda()
    sink = torch.zeros(n, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    reps = 10
    sec = lib.kvq_probe_page_read(pool.data_ptr(), pages.data_ptr(), n, pb, 64, reps, sink.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    gbs = round(reps * n * pb / sec / 1e9, 1) if sec > 0 else None
    rec = {"kernel": "page_read_kernel (libkvq_probe.so)", "page_bytes": pb, "pages": n, "gbs": gbs,
           "frac_of_peak": None if gbs is None else round(gbs / HBM_PEAK_GBS, 4)}
    # the same pages read straight into LDS through a ring of three stages
    if hasattr(lib, "kvq_probe_page_read_lds") and pb * 3 <= 160 * 1024:
        lib.kvq_probe_page_read_lds.restype = ctypes.c_double
        lib.kvq_probe_page_read_lds.argtypes = lib.kvq_probe_page_read.argtypes
        sec = lib.kvq_probe_page_read_lds(pool.data_ptr(), pages.data_ptr(), n, pb, 64, reps, sink.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
        lds = round(reps * n * pb / sec / 1e9, 1) if sec > 0 else None
        rec["lds_direct"] = {"kernel": "page_read_lds_kernel (libkvq_probe.so)", "gbs": lds,
                             "frac_of_peak": None if lds is None else round(lds / HBM_PEAK_GBS, 4)}
    del pool, pages, sink
    return rec


def _attended(st, w) -> np.ndarray:
    L = st.lens.astype(np.int64)
    if w.sliding_window:
        return np.minimum(L, w.sliding_window)
    return L


def decode_kernels(w) -> str:
    """The launches of one decode call for this workload."""
    if w.sparse_v_threshold > 0:
        return "kvq_paged_decode: scores_kernel + sparse_v_kernel"
    bits = {"bf16": 16, "fp8": 8, "turbo2": 2, "turbo3": 3, "turbo4": 4, "turbo8": 8, "nvfp4": 4}
    hd = w.head_dim
    kqb = hd * bits[w.k_format] // 32  # K bytes per lane and chunk in the matrix-core kernel
    if w.k_format.startswith("turbo") or w.k_format == "nvfp4":  # per-16 group scales
        shape_ok = kqb % 4 == 0 and kqb <= 32 and hd // 4 >= 16
    else:
        shape_ok = kqb <= 64 and kqb % 16 == 0
    mfma = shape_ok and hd * bits[w.v_format] // 8 <= 128 and w.block_size >= 16
    return "kvq_paged_decode: " + ("split_mfma_kernel" if mfma else "split_kernel") + " + merge_kernel"


def traffic_from_profile(workload: str, step: str = "decode"):
    """HBM bytes per decode (or prefill) call from the committed rocprofv3
    counter summary, or None when the kernel sources changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{step}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_(?:decode|call):\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_b or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def host_block_manager(kvq, w, lens: np.ndarray, steps: int = 200) -> dict:
    """Host cost of the library's block manager for this workload's decode
    step: one position appended to every sequence (one batched call), then the
    block tables exported; the C calls alone, on buffers made once."""
    import ctypes
    S, bs = len(lens), w.block_size
    nb = int(sum((int(L) + steps + bs - 1) // bs for L in lens)) + S
    bm = kvq.BlockManager(nb, bs)
    ids = np.array([bm.seq_new() for _ in range(S)], np.uint32)
    bm.append_many(ids, np.maximum(lens.astype(np.int64) - 1, 0))
    mb = int((int(lens.max()) + steps + bs - 1) // bs)
    lib = kvq.load()
    ones = np.ones(S, np.uint32)
    slots, cow = np.zeros(S, np.int64), np.zeros((S, 2), np.int32)
    bt, ln = np.zeros((S, mb), np.int32), np.zeros(S, np.int32)
    PU, PI = ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_int32)
    pid, pone = ids.ctypes.data_as(PU), ones.ctypes.data_as(PU)
    pslot, pcow = slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), cow.ctypes.data_as(PI)
    pbt, pln = bt.ctypes.data_as(PI), ln.ctypes.data_as(PI)
    ta = tt = 0.0
    for _ in range(steps):
        t0 = time.perf_counter()
        rc = lib.kvq_blocks_append_many(bm._h, pid, pone, S, pslot, pcow)
        t1 = time.perf_counter()
        rc |= lib.kvq_blocks_table(bm._h, pid, S, mb, pbt, pln)
        t2 = time.perf_counter()
        assert rc == 0
        ta += t1 - t0
        tt += t2 - t1
    return {"append_us_per_step": round(ta / steps * 1e6, 2), "table_us_per_step": round(tt / steps * 1e6, 2),
            "sequences": S, "max_blocks_per_seq": mb, "steps": steps}


def cpu_workers() -> int:
    """Worker processes for the oracle baseline: the process's CPU set, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_worker(job):
    """One worker of the CPU baseline (a spawned process: plain numpy, no GPU):
    build the pools of its sequences with everything but the step's positions
    (untimed), wait for the others, then time the step (write of the new
    positions, fp64 decode of every q head)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import decode as odecode
    from oracle import layout as olayout
    from oracle import write as owrite
    d, seqs, barrier = job["dir"], job["seqs"], job["barrier"]
    ks, vs = olayout.pool_layout(job["k_format"], job["v_format"], job["bs"], job["hkv"], job["hd"])
    bs, tail = job["bs"], job["tail"]
    lens = np.load(os.path.join(d, "lens.npy"))
    bt_all = np.load(os.path.join(d, "bt.npy"))
    q = np.load(os.path.join(d, "q.npy"))
    remap, bt = {}, np.full_like(bt_all, -1)
    for s in seqs:
        for b in bt_all[s, :(int(lens[s]) + bs - 1) // bs]:
            remap.setdefault(int(b), len(remap))
    for s in seqs:
        nb = (int(lens[s]) + bs - 1) // bs
        bt[s, :nb] = [remap[int(b)] for b in bt_all[s, :nb]]
    kp = np.zeros((len(remap) + 1) * ks.block_stride_bytes, np.uint8)
    vp = np.zeros((len(remap) + 1) * vs.block_stride_bytes, np.uint8)
    kv = {s: (np.load(os.path.join(d, f"k{s}.npy"), mmap_mode="r"), np.load(os.path.join(d, f"v{s}.npy"),
                                                                          mmap_mode="r")) for s in seqs}
    with threadpool_limits(1):
        for s in seqs:
            K, V = kv[s]
            L = int(lens[s])
            pos = np.arange(max(0, L - tail))
            owrite.reshape_and_cache(ks, vs, np.asarray(K[pos]), np.asarray(V[pos]), kp, vp,
                                     bt[s, pos // bs].astype(np.int64) * bs + pos % bs, job["k_scale"], job["v_scale"])
        barrier.wait()
        t0 = time.perf_counter()
        for s in seqs:
            K, V = kv[s]
            L = int(lens[s])
            pos = np.arange(max(0, L - tail), L)
            owrite.reshape_and_cache(ks, vs, np.asarray(K[pos]), np.asarray(V[pos]), kp, vp,
                                     bt[s, pos // bs].astype(np.int64) * bs + pos % bs, job["k_scale"], job["v_scale"])
        res = odecode.paged_decode(ks, vs, q, kp, vp, bt, lens, job["inv"], job["window"], job["thr"],
                                   job["k_scale"], job["v_scale"], seqs=seqs, detail=True)
        dt = time.perf_counter() - t0
    _, o64, band, n_amb = res
    return dt, seqs, o64[seqs], band[seqs], n_amb[seqs]


def cpu_baseline(st, w, seqs, out_gpu: np.ndarray) -> dict:
    """The oracle on a sample of the same workload, spread over worker
    processes; its outputs also check the GPU's on the sample (the decode
    bars: max-abs 2e-3 plus the sparse-V band, rel-L2 1e-3)."""
    import multiprocessing as mp
    import shutil
    import tempfile
    nproc = min(cpu_workers(), len(seqs))
    base = "/dev/shm" if os.path.isdir("/dev/shm") else None
    d = tempfile.mkdtemp(prefix="kvq_bench_", dir=base)
    try:
        np.save(os.path.join(d, "lens.npy"), st.lens)
        np.save(os.path.join(d, "bt.npy"), st.bt)
        np.save(os.path.join(d, "q.npy"), st.q.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        for s in seqs:
            K, V = st.host_kv[s]
            np.save(os.path.join(d, f"k{s}.npy"), K)
            np.save(os.path.join(d, f"v{s}.npy"), V)
        ctx = mp.get_context("spawn")
        mgr = ctx.Manager()
        barrier = mgr.Barrier(nproc)
        # longest sequences first, dealt round-robin: the workers' shares stay even
        order = sorted(seqs, key=lambda s: -int(st.lens[s]))
        parts = [order[i::nproc] for i in range(nproc)]
        jobs = [dict(dir=d, seqs=sorted(p), barrier=barrier, k_format=w.k_format, v_format=w.v_format,
                     bs=w.block_size, hkv=w.num_kv_heads, hd=w.head_dim, tail=w.write_tail,
                     inv=synth.inv_sqrt_d(w.head_dim), window=w.sliding_window, thr=w.sparse_v_threshold,
                     k_scale=st.k_scale, v_scale=st.v_scale) for p in parts]
        with ctx.Pool(nproc) as pool:
            results = pool.map(_oracle_worker, jobs)
        mgr.shutdown()
    finally:
        shutil.rmtree(d, ignore_errors=True)
    wall = max(r[0] for r in results)
    att = int(_attended(st, w)[seqs].sum())
    kv_bytes = att * w.num_kv_heads * (ROW_BYTES[w.k_format](w.head_dim) + ROW_BYTES[w.v_format](w.head_dim))
    # parity of the GPU output on the sample
    emax, num, den, namb, ok = 0.0, 0.0, 0.0, 0, True
    for _, ss, o64, band, n_amb in results:
        g = out_gpu[ss].astype(np.float64)
        err = np.abs(g - o64)
        ok &= bool(np.all(err <= 2e-3 + band))
        emax = max(emax, float(err.max()) if err.size else 0.0)
        clean = n_amb == 0
        num += float(((g - o64) ** 2)[clean].sum())
        den += float((o64 ** 2)[clean].sum())
        namb += int(n_amb.sum())
    rel = math.sqrt(num / den) if den > 0 else 0.0
    ok &= rel <= 1e-3
    return {"value": round(kv_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": nproc, "kind": "oracle",
            "sample": f"{len(seqs)} of {w.num_seqs} sequences ({att} attended positions): write of their new "
                      f"token(s) + fp64 decode of all {w.num_q_heads} q heads, {nproc} worker processes, "
                      f"{wall:.2f} s wall (the slowest worker)",
            "parity": {"sequences": len(seqs), "max_abs": emax, "rel_l2": rel, "ambiguous": namb, "ok": ok}}


def prefill_main(args, kvq, w):
    """Chunked prefill step: write the chunks' K/V (the held-back last
    write_tail positions of every sequence), then their queries attend."""
    ncpu = 1 if args.cpu_seqs is None else args.cpu_seqs
    keep = range(min(ncpu, w.num_seqs)) if ncpu else ()
    st = stage(w, kvq, "cuda", keep_host=keep, log=log)
    S, Hq, Hkv, hd, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    C = np.minimum(w.write_tail, st.lens).astype(np.int64)
    qs = np.concatenate([[0], np.cumsum(C)]).astype(np.int32)
    T, mq = int(qs[-1]), int(C.max())
    q = synth.prefill_queries(w, T, "cuda")
    qs_dev = torch.from_numpy(qs).cuda()
    inv = synth.inv_sqrt_d(hd)
    mb = st.bt.shape[1]
    ws = torch.empty(max(16, kvq.prefill_workspace_bytes(st.layout, S, Hq, mb, mq, w.sliding_window)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((T, Hq, hd), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    scratch = None if args.warm else torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def step(ev=None):
        if scratch is not None:
            torch.sum(scratch, dim=0, out=sink)
        if ev:
            ev[0].record(stream)
        kvq.reshape_and_cache(st.layout, st.tail_key, st.tail_value, st.k_pool, st.v_pool, st.tail_slots,
                              st.k_scale, st.v_scale, stream=stream)
        if ev:
            ev[1].record(stream)
        kvq.paged_prefill(st.layout, q, st.k_pool, st.v_pool, st.bt_dev, st.lens_dev, qs_dev, mq, inv,
                          w.sliding_window, st.k_scale, st.v_scale, out=out, workspace=ws, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    att = np.array([e[1].elapsed_time(e[2]) for e in ev])
    stp = np.array([e[0].elapsed_time(e[2]) for e in ev])
    att_ms, ms_step = float(np.median(att)), float(np.median(stp))
    assert torch.isfinite(out).all(), "non-finite prefill output"
    del scratch
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
    # algorithmic work: query i of a chunk of C at the end of L positions
    # attends L - C + i + 1 keys (or the window); Q.K and P.V are 2 hd flops
    # each per (query head, key).  Bytes: every sequence's attended K and V
    # rows once (a lower bound), and what tiles of qt queries read by design.
    kb, vb = ROW_BYTES[w.k_format](hd), ROW_BYTES[w.v_format](hd)
    keys = 0
    tile_keys = 0
    # block_size >= 4 runs on the tile kernel: 128 (query, head) rows per
    # tile, 64 at head_dim 256 or with a rotated K side; smaller blocks run
    # every query as a decode row
    rot_k = w.k_format in ("turbo2", "turbo3", "turbo4", "turbo8")
    tiles = bs >= 4
    rows = (64 if rot_k or hd > 128 else 128) if tiles else Hq // Hkv
    qt = max(1, rows // (Hq // Hkv))
    for L, c in zip(st.lens.astype(np.int64), C):
        p = L - c + np.arange(c)
        lo = np.maximum(0, p + 1 - w.sliding_window) if w.sliding_window else np.zeros_like(p)
        keys += int((p + 1 - lo).sum())
        for t0_ in range(0, int(c), qt):
            hi = int(p[min(t0_ + qt, c) - 1]) + 1
            tile_keys += hi - int(lo[t0_])
    flops = 4 * keys * Hq * hd
    min_bytes = int(sum(int(L) for L in st.lens)) * Hkv * (kb + vb)
    tile_bytes = tile_keys * Hkv * (kb + vb)
    tflops = flops / (att_ms * 1e-3) / 1e12
    if tiles:
        # P.V on bf16 matrix cores with its weights (and a V side that is not
        # a bf16 value) as bf16 hi + lo pairs: 3 products per algorithmic one
        # (2 when V is exact in bf16); Q.K on bf16 ones, or on fp32 ones for a
        # rotated K side.  Half the algorithmic flops each.
        pv_products = 2 if w.v_format in ("bf16", "fp8", "nvfp4") else 3
        qk_peak = MFMA_F32_TFLOPS if rot_k else MFMA_BF16_TFLOPS
        peak = 1.0 / (0.5 / qk_peak + 0.5 / MFMA_BF16_TFLOPS)
        peak_basis = (f"half the flops (Q.K) at {qk_peak}, half (P.V) at {MFMA_BF16_TFLOPS}; P.V issues "
                      f"{pv_products} bf16 products per algorithmic product (hi/lo pairs), counted once")
        issued = flops / 2 * (1 + pv_products)
        # time the issued matrix instructions take at peak, over the kernel time
        busy_s = (flops / 2 / qk_peak + flops / 2 * pv_products / MFMA_BF16_TFLOPS) / 1e12
        kernel = "kvq_paged_prefill: prefill_tile_kernel"
    else:
        peak = MFMA_F32_TFLOPS
        peak_basis = f"every flop at {MFMA_F32_TFLOPS} (decode rows: fp32 matrix cores or VALU)"
        issued = flops
        busy_s = flops / MFMA_F32_TFLOPS / 1e12
        kernel = "kvq_paged_prefill: decode kernels over one row per query"
    rec = {
        "metric": "chunked-prefill query tokens/s over the quantized paged cache, 1 GPU",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "k_format": w.k_format, "v_format": w.v_format, "num_seqs": S,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": hd, "block_size": bs,
                   "seq_lens": list(w.seq_len), "chunk": w.write_tail, "query_rows": T, "parallelism": "1 GPU"},
        "prefill_ms": round(att_ms, 4),
        "write_ms": round(float(np.median(stp - att)), 4),
        "wall_s_timed_loop": round(elapsed, 3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "peak_basis": peak_basis,
                     "frac": round(tflops / peak, 4), "traffic": traffic_from_profile(w.name, "prefill"),
                     "kernel": kernel, "algorithmic_flops": flops, "issued_matrix_flops": int(issued),
                     "issued_busy_frac": round(busy_s / (att_ms * 1e-3), 4)},
        "kv_bytes": {"once_per_sequence": min_bytes, "read_by_tiles": tile_bytes, "queries_per_tile": qt,
                     "gbs_once_per_sequence": round(min_bytes / (att_ms * 1e-3) / 1e9, 1),
                     "gbs_read_by_tiles": round(tile_bytes / (att_ms * 1e-3) / 1e9, 1)},
        "kernel_source_sha256": kernel_source_hash(),
    }
    if ncpu:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = prefill_cpu_baseline(st, w, q, qs, min(ncpu, 1), inv)  # ~10-20 s each
    print(json.dumps(rec), flush=True)


def prefill_cpu_baseline(st, w, q, qs, n_seqs: int, inv: float):
    """Oracle prefill (fp64) of the first n_seqs sequences' chunks, one thread."""
    from oracle import layout as olayout
    from oracle import prefill as oprefill
    from oracle import write as owrite
    from threadpoolctl import threadpool_limits
    seqs = list(range(n_seqs))
    ks, vs = olayout.pool_layout(w.k_format, w.v_format, w.block_size, w.num_kv_heads, w.head_dim)
    bs = w.block_size
    remap = {}
    for s in seqs:
        for b in st.bt[s, :(int(st.lens[s]) + bs - 1) // bs]:
            remap.setdefault(int(b), len(remap))
    n = len(remap) + 1
    kp = np.zeros(n * ks.block_stride_bytes, np.uint8)
    vp = np.zeros(n * vs.block_stride_bytes, np.uint8)
    bt = np.full_like(st.bt, -1)
    for s in seqs:
        nb = (int(st.lens[s]) + bs - 1) // bs
        bt[s, :nb] = [remap[int(b)] for b in st.bt[s, :nb]]
        K, V = st.host_kv[s]
        pos = np.arange(int(st.lens[s]))
        owrite.reshape_and_cache(ks, vs, K[pos], V[pos], kp, vp, bt[s, pos // bs].astype(np.int64) * bs + pos % bs,
                                 st.k_scale, st.v_scale)
    qb = q.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        oprefill.paged_prefill(ks, vs, qb, qs, kp, vp, bt, st.lens, inv, w.sliding_window, st.k_scale, st.v_scale,
                               seqs=seqs)
        dt = time.perf_counter() - t0
    rows = int(qs[n_seqs] - qs[0])
    return {"value": round(rows / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_seqs} of {w.num_seqs} sequences ({rows} query rows): fp64 prefill attention of all "
                      f"{w.num_q_heads} q heads, one thread, {dt:.1f} s (the chunk's write is not in the sample)"}


def page_bytes(w) -> int:
    """K + V bytes of one page of the pools (block_size positions, every kv head)."""
    return w.block_size * w.num_kv_heads * (ROW_BYTES[w.k_format](w.head_dim) + ROW_BYTES[w.v_format](w.head_dim))


def measure_decode(kvq, w, args, cpu_seqs) -> dict:
    """Stage workload w, time K write + decode steps, and return its record."""
    keep = list(cpu_seqs)
    t0 = time.time()
    st = stage(w, kvq, "cuda", keep_host=keep, log=log)
    log(f"staged {w.name} in {time.time() - t0:.1f}s: {int(st.lens.sum())} positions, "
        f"{st.num_blocks} blocks, tail batch {st.tail_slots.numel()} tokens")
    hd, Hkv = w.head_dim, w.num_kv_heads
    inv = synth.inv_sqrt_d(hd)
    mb = st.bt.shape[1]
    ws = torch.empty(max(16, kvq.decode_workspace_bytes(st.layout, w.num_seqs, w.num_q_heads, mb,
                                                        w.sliding_window, w.sparse_v_threshold)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((w.num_seqs, w.num_q_heads, hd), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def write():
        kvq.reshape_and_cache(st.layout, st.tail_key, st.tail_value, st.k_pool, st.v_pool, st.tail_slots,
                              st.k_scale, st.v_scale, stream=stream)

    def decode():
        kvq.paged_decode(st.layout, st.q, st.k_pool, st.v_pool, st.bt_dev, st.lens_dev, inv, w.sliding_window,
                         w.sparse_v_threshold, st.k_scale, st.v_scale, out=out, workspace=ws, stream=stream)

    # Between steps a 1 GiB scratch read evicts L2 and the MALL (outside the
    # timed region), so every step reads the pools from HBM.  A read leaves
    # the caches full of clean lines; a write would leave dirty ones that the
    # next step would pay to write back.
    scratch = None if args.warm else torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def evict():
        if scratch is not None:
            torch.sum(scratch, dim=0, out=sink)

    for _ in range(args.warmup):
        evict()
        write()
        decode()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evict()
        ev[i][0].record(stream)
        write()
        ev[i][1].record(stream)
        decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dec = np.array([e[1].elapsed_time(e[2]) for e in ev])
    stp = np.array([e[0].elapsed_time(e[2]) for e in ev])
    dec_ms = float(np.median(dec))
    ms_step = float(np.median(stp))
    assert torch.isfinite(out).all(), "non-finite decode output"
    del scratch

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    att = _attended(st, w)
    positions = int(att.sum())
    kb, vb = ROW_BYTES[w.k_format](hd), ROW_BYTES[w.v_format](hd)
    kv_dense = positions * Hkv * (kb + vb)
    kept = kept_rows(st, w, kvq)
    alg = (positions * Hkv * kb + kept * vb + w.num_seqs * w.num_q_heads * hd * (2 + 4)
           + sum(int(math.ceil(int(L) / w.block_size)) for L in att) * 4 + w.num_seqs * 4)
    achieved = alg / (dec_ms * 1e-3) / 1e9
    G = w.group
    flops = positions * Hkv * G * (2 * hd + 1) + kept * G * 2 * hd   # QK + exp per position-head, PV per kept
    value = kv_dense / (ms_step * 1e-3) / 1e9
    traffic = traffic_from_profile(w.name)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "value_basis": "dense-window K+V bytes / step time (write + decode)",
        "unit": "GB/s",
        "ms_per_step": round(ms_step, 4),
        "config": {"workload": w.name, "k_format": w.k_format, "v_format": w.v_format,
                   "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": Hkv, "head_dim": hd,
                   "block_size": w.block_size, "seq_lens": list(w.seq_len), "attended_positions": positions,
                   "sparse_v_threshold": w.sparse_v_threshold, "sliding_window": w.sliding_window,
                   "write_tokens_per_step": int(st.tail_slots.numel()), "parallelism": "1 GPU"},
        "pct_hbm_peak": round(100.0 * achieved / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "decode_ms": round(dec_ms, 4),
        "decode_ms_p10_p90": [round(float(np.percentile(dec, 10)), 4), round(float(np.percentile(dec, 90)), 4)],
        "write_ms": round(float(np.median(stp - dec)), 4),
        "caches": "warm" if args.warm else "cold: 1 GiB scratch read between steps, outside the timed region",
        "wall_s_timed_loop": round(elapsed, 3),
        "kept_v_fraction": round(kept / max(1, positions * Hkv), 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic, 0),
                     "kernel": decode_kernels(w),
                     "algorithmic_bytes": alg},
        "roofline_alu": {"bound": "alu", "achieved": round(flops / (dec_ms * 1e-3) / 1e12, 3),
                         "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (dec_ms * 1e-3) / 1e12 / VALU_PEAK_TFLOPS, 4),
                         "algorithmic_flops": flops},
    }
    if keep:
        log(f"timing the CPU oracle on {len(keep)} sequences of {w.name} ...")
        rec["cpu_baseline"] = cpu_baseline(st, w, keep, out.cpu().numpy())
    rec["_lens"] = st.lens
    del st, ws, out
    torch.cuda.empty_cache()
    return rec


# sequences of each workload the CPU baseline times (bounded: about 10-30 s of
# single-core oracle work): every sequence of the headline workload, 16 of
# the 128 x 32768 one, the first 8 elsewhere
CPU_SAMPLE = {2: 64, 3: 16}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--also", type=int, default=None,
                    help="a second decode workload measured in the same line (default: 3 with workload 2; 0: none)")
    ap.add_argument("--cpu-seqs", type=int, default=None, help="sequences in the oracle sample (0: skip)")
    ap.add_argument("--warm", action="store_true", help="no cache eviction between steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU: this path has no multi-GPU step (asked for {args.gpus}); "
              "each GPU would serve its own sequences or kv heads with no exchange", file=sys.stderr)
        sys.exit(2)
    import paged_quantized_kv_kvq_amd as kvq
    kvq.load()
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    if w.prefill:
        return prefill_main(args, kvq, w)
    also = args.also if args.also is not None else (3 if args.workload == 2 else 0)

    def sample(wl):
        n = args.cpu_seqs if args.cpu_seqs is not None else CPU_SAMPLE.get(wl.wid, 8)
        return range(min(n, wl.num_seqs))

    head = measure_decode(kvq, w, args, sample(w))
    lens = head.pop("_lens")
    rec = {"metric": METRIC, "value": head.pop("value"), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic"}
    head.pop("metric")
    rec.update(head)
    rec["stream_read_ref"] = stream_read_reference(page_bytes(w))
    rec["kernel_source_sha256"] = kernel_source_hash()
    rec["host_block_manager"] = host_block_manager(kvq, w, lens)
    if also:
        w2 = synth.WORKLOADS[also]
        sec = measure_decode(kvq, w2, args, sample(w2))
        sec.pop("_lens")
        sec.pop("metric")
        sec["stream_read_ref"] = stream_read_reference(page_bytes(w2))
        rec["configs"] = {w2.name: sec}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
