"""Chunked prefill against the oracle beyond the c4a bf16 case: c128a chunks
(unaligned start, a chunk straddling a 128-token boundary, a chunk whose
queries see more than 4096 compressed rows), window-only layers, an E4M3
attention cache, and the full 4096-token chunk at 61440 checked end to end
(every query's top-k set and output, every emitted row, the raw ring and
the compressor state after the chunk), with the oracle using only rows it
computed itself.

Prefill is defined as the sequence of decode steps ("ds4.c を読み解く (#3)",
section 3: chunks keep absolute compressor boundaries); the oracle runs the
whole history at once, the GPU in chunks.
"""
import numpy as np
import pytest

import oracle as O
from harness import (BF16_TOL, FP8_TOL, assert_close, dev, device_layer, oracle_layer, oracle_seq_from_bytes,
                     oracle_seq_from_init, sets_equal, topk_margin)
from test_gpu_contract import _check_chunk_state, _prefill_sampled, chunk_bytes, gpu_bytes_seq
from test_gpu_parity import cpu, log, out_values
from workloads import get_config, make_layer_weights, make_prefill_inputs
from workloads import gen as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MARGIN = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_kv_sparse_amd  # noqa: F401


def _chunked(cfg, pos0, chunks, sample_every=97, all_queries=False):
    """Prefill ``chunks`` consecutive chunks from a drawn cache at pos0; after
    each chunk its rows, the window state and the raw ring are compared with
    the oracle's history run, and the chunk's edge queries, its queries at
    row boundaries and every ``sample_every``-th one (or all) are compared:
    top-k sets on the GPU's index bytes, outputs with the GPU's lists."""
    T_all = sum(chunks)
    wts = make_layer_weights(cfg)
    inp = make_prefill_inputs(cfg, pos0=pos0, T=T_all)
    L = oracle_layer(cfg, wts)
    seq = oracle_seq_from_init(L, inp.cache, 0)
    seq.feed(pos0, inp.x, inp.u)
    r = cfg.ratio
    qI, w = (inp.qI.copy(), inp.w.copy()) if r == 4 else (None, None)
    dl = device_layer(cfg, wts, inp.cache, max_chunk=max(chunks))
    tol = FP8_TOL if cfg.kv_fmt == "e4m3" else BF16_TOL
    p0 = pos0
    for ci, T in enumerate(chunks):
        a = p0 - pos0
        want = set(range(T)) if all_queries else ({0, 1, T - 1} | set(range(0, T, sample_every)))
        if r:
            want |= {n for n in range(T) if (p0 + n + 1) % r == 0 and n % 3 == 0} if r == 4 else \
                    {n for n in range(T) if (p0 + n + 1) % r in (0, 1)}
        want = sorted(n for n in want if 0 <= n < T)
        if r == 4:
            for n in want:
                for att in range(40):
                    if topk_margin(seq.index_scores(p0 + n, qI[a + n], w[a + n]), cfg.top_k) > MARGIN:
                        break
                    nq, nw = G.draw_query_index(cfg, 1, sub=20000 + a + n, attempt=att + 1)
                    qI[a + n], w[a + n] = nq[0], nw[0]
        sl = slice(a, a + T)
        out, tk = dl.prefill(0, p0, dev(inp.x[sl]), dev(inp.u[sl]), dev(inp.q[sl]),
                             None if qI is None else dev(qI[sl]), None if w is None else dev(w[sl]))
        torch.cuda.synchronize()
        assert cpu(dl.status)[0] == 0 and cpu(dl.n_tokens)[0] == p0 + T
        log(f"[{cfg.name}] chunk {ci} pos0={p0} T={T}: {len(want)} queries")
        _check_chunk_state(cfg, dl, seq, p0, T)
        og = out_values(out, cfg.act_fmt)
        tkg = cpu(tk) if tk is not None else None
        cb = chunk_bytes(dl)
        bseq = oracle_seq_from_bytes(L, None, cb[1], cb[2], 0)
        for n in want:
            p = p0 + n
            if r == 4:
                sc = bseq.index_scores(p, qI[a + n], w[a + n])
                assert sets_equal(tkg[n], O.topk_select(sc, cfg.top_k)), f"top-k of query {p}"
            sel = None if tkg is None else tkg[n]
            ref = gpu_bytes_seq(L, cfg, cb, p, p0).attend(p, inp.q[a + n], sel)
            assert_close(og[n], ref, tol, f"{cfg.name} output p={p}, GPU bytes")
            if cfg.kv_fmt != "e4m3":
                assert_close(og[n], seq.attend(p, inp.q[a + n], sel), tol, f"{cfg.name} output p={p}, oracle rows")
        p0 += T


def test_c128a_chunked_prefill_unaligned():
    """c128a chunks of 1, 37, 1000 and 4096 tokens from position 5157 (37
    tokens into a 128-token window, whose first tokens come from the state)."""
    cfg = get_config("c3").with_(batch=1, comp_cap=128, ctx_range=None, seed=91, name="c128a_chunks")
    _chunked(cfg, 128 * 40 + 37, (1, 37, 1000, 4096), sample_every=211)


def test_c128a_prefill_beyond_4096_visible_rows():
    """One c128a chunk at position 524877 (4100 rows visible), straddling the
    128-token boundary at 525056: queries before, at and after the row that
    closes there each attend more than 4096 compressed rows in one split."""
    cfg = get_config("c3").with_(batch=1, ctx_range=None, seed=92, name="c128a_4100_rows")
    _prefill_sampled(cfg, pos0=4100 * 128 + 77, T=300, sample={0, 1, 177, 178, 179, 180, 298, 299})


def test_window_only_chunked_prefill_fp8():
    """Ratio-0 layer with an E4M3 cache: chunks of 37, 1 and 300 tokens from
    position 90 (windows still holding drawn rows), every query compared."""
    cfg = get_config("c5_swa").with_(batch=1, seed=93, name="swa_chunks")
    _chunked(cfg, 90, (37, 1, 300), all_queries=True)


def test_c4a_chunked_prefill_fp8():
    """c4a with the E4M3 attention cache: chunks of 4096, 1000, 37 and 1
    tokens from position 10001 (one token into a stride block)."""
    cfg = get_config("c5").with_(batch=1, comp_cap=4096, seed=94, name="c4a_fp8_chunks")
    _chunked(cfg, 10001, (4096, 1000, 37, 1), sample_every=173)


@pytest.mark.timeout(1200)
def test_c4_prefill_chunk_full_chain():
    """The 4096-token chunk at 61440, every query, the oracle on its own rows
    (no GPU byte enters its scores or outputs).

    * every emitted row, the raw ring and the compressor state after the chunk;
    * top-k: the GPU's set must contain every row whose oracle score is above
      the oracle's k-th by more than 2 delta and only rows within 2 delta
      below it, delta being the largest score change the GPU's stored rows
      make (plus fp32 key rounding): the GPU ranks by scores of its own rows,
      which differ from the oracle's by at most delta, so this is exactly the
      set of rankings those rows allow.  Where no score lies within that band
      of the k-th, the set is unique and must be equal;
    * outputs: the oracle's attention with its own rows over the GPU's list,
      within the bf16 tolerance."""
    cfg = get_config("c4")
    wts = make_layer_weights(cfg)
    inp = make_prefill_inputs(cfg)
    T, p0, k = inp.T, inp.pos0, cfg.top_k
    L = oracle_layer(cfg, wts)
    seq = oracle_seq_from_init(L, inp.cache, 0)
    seq.feed(p0, inp.x, inp.u)
    dl = device_layer(cfg, wts, inp.cache, max_chunk=T)
    out, tk = dl.prefill(0, p0, dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w))
    torch.cuda.synchronize()
    log("[c4 chain] chunk done")
    _check_chunk_state(cfg, dl, seq, p0, T)
    log("[c4 chain] rows, ring and state match")
    og, tkg = out_values(out, cfg.act_fmt), cpu(tk)
    Vmax = (p0 + T) // 4
    own = seq.idx_matrix(Vmax)                                     # oracle's own stored values
    gpu_rows = O.decode_values(cpu(dl.idx)[0][:Vmax], cfg.idx_fmt)
    equal_sets, worst = 0, 0.0
    for n in range(T):
        p = p0 + n
        V = (p + 1) // 4
        qh = O.cast_values(O.rope_tail(O.decode_values(inp.qI[n], cfg.act_fmt), p, L.base_comp, 64), cfg.idx_fmt)
        s_own = O.indexer_scores(qh, inp.w[n], own[:V])
        s_gpu = O.indexer_scores(qh, inp.w[n], gpu_rows[:V])
        smax = float(np.max(np.abs(s_own)))
        delta = float(np.max(np.abs(s_own - s_gpu))) + 1e-5 * smax
        worst = max(worst, delta / smax)
        kth = np.sort(s_own)[::-1][k - 1]
        g = tkg[n][tkg[n] >= 0]
        assert len(g) == k and len(set(g.tolist())) == k, f"query {p}: not {k} distinct rows"
        must = np.nonzero(s_own > kth + 2 * delta)[0]
        assert np.all(np.isin(must, g)), f"query {p}: a row clearly in the top-k is missing"
        assert np.all(s_own[g] >= kth - 2 * delta), f"query {p}: a row clearly outside the top-k was selected"
        ref_set = O.topk_select(s_own, k)
        equal_sets += int(np.array_equal(np.sort(g), ref_set))
        if int(np.sum(np.abs(s_own - kth) <= 2 * delta)) == 1:
            assert np.array_equal(np.sort(g), ref_set), f"query {p}: unique top-k set differs"
        ref = seq.attend(p, inp.q[n], tkg[n])
        assert_close(og[n], ref, BF16_TOL, f"c4 output p={p}")
        if n % 512 == 0:
            log(f"[c4 chain] {n + 1}/{T} queries checked")
    log(f"[c4 chain] top-k sets equal to the oracle's own in {equal_sets}/{T} queries; "
        f"largest score change from stored rows {worst:.2e} of max|s|")
    assert worst < 1e-2
