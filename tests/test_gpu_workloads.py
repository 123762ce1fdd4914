"""GPU parity at the benchmark workloads' full sizes.

Each workload is staged exactly as the benchmark stages it (whole pool, all
sequences, the timed step's write batch in its shuffled slot order) and
decoded through the same C-ABI call with the same arguments.  The oracle then
rebuilds only a few sampled sequences (shortest, longest, last, middle,
sequences 1, 3 and 7, seeded picks; for the sliding-window workload only the
pages inside the window) and checks
them element by element: written pool bytes bit-exact, decode outputs to the
same max-abs / relative-L2 bar as the small cases.  Properties that hold at
any size are checked on every sequence: all outputs finite, the decode
repeatable bit for bit, and the write idempotent (writing the same batch
again leaves the pool bytes unchanged).
"""
import numpy as np
import pytest
import torch

import synth
from synth.gpu import stage
from kvq_testlib import OracleCache, check_decode, say, timed

pytestmark = pytest.mark.gpu


def _sample(lens: np.ndarray, wid: int, extra: int = 1):
    """Shortest, longest, last, middle, sequences 1, 3 and 7 (units are dealt to
    the 8 XCDs in turn, so these cover several residues mod 8 even when every
    length is equal), plus `extra` seeded picks."""
    S = len(lens)
    picks = {int(np.argmin(lens)), int(np.argmax(lens)), S - 1, S // 2} | {s for s in (1, 3, 7) if s < S}
    want = len(picks) + extra
    rng = np.random.default_rng(wid)
    for s in rng.permutation(len(lens)):
        if len(picks) >= want:
            break
        picks.add(int(s))
    return sorted(picks)


def _decode(kvq, st):
    w = st.w
    need = kvq.decode_workspace_bytes(st.layout, w.num_seqs, w.num_q_heads, st.bt.shape[1], w.sliding_window,
                                      w.sparse_v_threshold)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes
    return kvq.paged_decode(st.layout, st.q, st.k_pool, st.v_pool, st.bt_dev, st.lens_dev,
                            synth.inv_sqrt_d(w.head_dim), w.sliding_window, w.sparse_v_threshold,
                            st.k_scale, st.v_scale, workspace=ws)


# sequences the oracle rebuilds per workload (its cost grows with their length)
EXTRA = {1: 0, 2: 1, 3: 0, 4: 1, 5: 1, 6: 0, 7: 0, 8: 0, 9: 0}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", sorted(synth.WORKLOADS))
def test_workload_full_size(gpu_lib, wid):
    w = synth.WORKLOADS[wid]
    lens = synth.seq_lens(w)
    seqs = _sample(lens, wid, EXTRA[wid])
    say(f"workload {wid} ({w.name}): {w.num_seqs} seqs, lens {lens.min()}..{lens.max()}, oracle seqs {seqs}")
    with timed(f"stage workload {wid}"):
        st = stage(w, gpu_lib, "cuda", keep_host=seqs)
    if w.prefill:
        return _prefill_full_size(gpu_lib, w, st, seqs)
    with timed(f"write {st.tail_slots.numel()} tokens + decode"):
        if st.tail_slots.numel():
            gpu_lib.reshape_and_cache(st.layout, st.tail_key, st.tail_value, st.k_pool, st.v_pool,
                                      st.tail_slots, st.k_scale, st.v_scale)
        out = _decode(gpu_lib, st).clone()
        again = _decode(gpu_lib, st)
        torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "non-finite decode output"
    assert torch.equal(out, again), "decode is not repeatable"
    if st.tail_slots.numel():
        kb, vb = st.k_pool.clone(), st.v_pool.clone()
        gpu_lib.reshape_and_cache(st.layout, st.tail_key, st.tail_value, st.k_pool, st.v_pool,
                                  st.tail_slots, st.k_scale, st.v_scale)
        torch.cuda.synchronize()
        assert torch.equal(kb, st.k_pool) and torch.equal(vb, st.v_pool), "rewrite changed the pool"
        del kb, vb
    out_np = out.cpu().numpy()
    with timed(f"oracle for {len(seqs)} sequences"):
        ora = OracleCache(st, seqs, from_window=bool(w.sliding_window))
        ora.compare_pools(st)
        ref = ora.decode(st, synth.inv_sqrt_d(w.head_dim))
    e, rel, namb = check_decode(out_np, ref, seqs, f"workload {wid}")
    say(f"  ok workload {wid}: max-abs {e:.2e} rel-L2 {rel:.2e} ambiguous {namb}")


def _prefill_full_size(kvq, w, st, seqs):
    """The bench's prefill step (write the chunks, then their queries attend),
    checked on the sampled sequences' query rows against the oracle prefill."""
    from kvq_testlib import MAX_ABS, REL_L2
    from oracle import prefill as oprefill
    C = np.minimum(w.write_tail, st.lens).astype(np.int64)
    qs = np.concatenate([[0], np.cumsum(C)]).astype(np.int32)
    T, mq = int(qs[-1]), int(C.max())
    q = synth.prefill_queries(w, T, "cuda")
    inv = synth.inv_sqrt_d(w.head_dim)
    need = kvq.prefill_workspace_bytes(st.layout, w.num_seqs, w.num_q_heads, st.bt.shape[1], mq, w.sliding_window)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    with timed(f"write {st.tail_slots.numel()} tokens + prefill of {T} queries"):
        kvq.reshape_and_cache(st.layout, st.tail_key, st.tail_value, st.k_pool, st.v_pool, st.tail_slots,
                              st.k_scale, st.v_scale)
        out = kvq.paged_prefill(st.layout, q, st.k_pool, st.v_pool, st.bt_dev, st.lens_dev,
                                torch.from_numpy(qs).cuda(), mq, inv, w.sliding_window, st.k_scale, st.v_scale,
                                workspace=ws).clone()
        again = kvq.paged_prefill(st.layout, q, st.k_pool, st.v_pool, st.bt_dev, st.lens_dev,
                                  torch.from_numpy(qs).cuda(), mq, inv, w.sliding_window, st.k_scale, st.v_scale,
                                  workspace=ws)
        torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.equal(out, again)
    with timed(f"oracle prefill for {len(seqs)} sequences"):
        ora = OracleCache(st, seqs)
        ora.compare_pools(st)
        qb = q.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        _, o64 = oprefill.paged_prefill(ora.ks, ora.vs, qb, qs, ora.kp, ora.vp, ora.bt, st.lens, inv,
                                        w.sliding_window, st.k_scale, st.v_scale, seqs=seqs)
    rows = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in seqs])
    g = out.cpu().numpy()[rows].astype(np.float64)
    r = o64[rows]
    err = np.abs(g - r).max()
    rel = np.sqrt(((g - r) ** 2).sum() / (r ** 2).sum())
    assert err <= MAX_ABS and rel <= REL_L2, f"prefill workload: max-abs {err:.2e} rel-L2 {rel:.2e}"
    say(f"  ok workload {w.wid} (prefill): {len(rows)} query rows, max-abs {err:.2e} rel-L2 {rel:.2e}")
