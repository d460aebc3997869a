"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Each stage is checked in isolation on identical bytes (the oracle reads the
cache the GPU wrote, and is fed the GPU's own top-k list for the attention),
and the chained runs (C1 from token 0) compare whole histories.  Bars:
top-k sets bit-exact on tie-free inputs; rows and outputs within
2e-2 rel + 1e-3 abs (5e-2 rel when the K=V cache is fp8); fp8 codes within one
step of the oracle's encoding.
"""
import numpy as np
import pytest

import oracle as O
from harness import (BF16_TOL, FP8_TOL, assert_close, compare_fp4_rows, compare_rows, dev, device_layer,
                     fp4_query_fragile, oracle_layer, oracle_seq_from_bytes, oracle_seq_from_init, sets_equal,
                     tie_free_queries, topk_margin)
from workloads import get_config, make_decode_inputs, make_layer_weights, make_prefill_inputs
from workloads import gen as G
from workloads.configs import TWO_LANE_FLAG

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MARGIN = 1e-4   # tie-free rule: gap between k-th and (k+1)-th score > MARGIN * max|s|


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_kv_sparse_amd  # noqa: F401  (fails loudly if libckv.so is missing)


def log(msg):
    print(msg, flush=True)


def cpu(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_values(t, fmt):
    a = cpu(t)
    return O.decode_values(a, fmt)


def run_decode_stage_checks(cfg, inp, wts, tol):
    """One decode step at full size: compressor, indexer and attention each
    compared with the oracle on the bytes the GPU holds."""
    B, d = cfg.batch, cfg.head_dim
    log(f"[decode] {cfg.name} B={B} p={inp.pos[:4]}")
    dl = device_layer(cfg, wts, inp.cache)
    pos_d = dev(inp.pos)
    x, u, q = dev(inp.x), dev(inp.u), dev(inp.q)
    dl.compress_decode(x, u, pos_d)
    torch.cuda.synchronize()
    assert int(dl.status.abs().sum()) == 0
    L = oracle_layer(cfg, wts)
    raw_g, comp_g, idx_g = check_compressor(cfg, inp, dl, L)

    # --- indexer on the GPU's own cache bytes
    topk_d = None
    bseqs = [oracle_seq_from_bytes(L, raw_g[b], None if comp_g is None else comp_g[b],
                                   None if idx_g is None else idx_g[b], int(inp.pos[b]) + 1) for b in range(B)]
    if cfg.ratio == 4:
        qI, w = tie_free_queries(cfg, bseqs, inp.pos, inp.qI, inp.w)
        topk_d = torch.empty((B, cfg.top_k), dtype=torch.int32, device="cuda")
        dl.indexer_decode(dev(qI), dev(w), pos_d, topk_d)
        torch.cuda.synchronize()
        check_topk(cfg, inp, bseqs, qI, w, cpu(topk_d))
    # --- attention with the GPU's top-k list
    out = dl.new_out(B)
    dl.attn_decode(q, pos_d, topk_d, out)
    torch.cuda.synchronize()
    check_attention(cfg, inp, bseqs, None if topk_d is None else cpu(topk_d), out, tol)
    return dl


def check_topk(cfg, inp, bseqs, qI, w, tk):
    for b in range(cfg.batch):
        ref = O.topk_select(bseqs[b].index_scores(int(inp.pos[b]), qI[b], w[b]), cfg.top_k)
        assert sets_equal(tk[b], ref), f"top-k set differs for sequence {b}"
        n = int((tk[b] >= 0).sum())
        assert np.all(tk[b][:n] == np.sort(tk[b][:n])) and np.all(tk[b][n:] == -1)


def check_attention(cfg, inp, bseqs, tk, out, tol):
    og = out_values(out, cfg.act_fmt)
    for b in range(cfg.batch):
        ref = bseqs[b].attend(int(inp.pos[b]), inp.q[b], None if tk is None else tk[b])
        assert_close(og[b], ref, tol, f"attention output b={b}")


def check_idx_row(cfg, rec, pre, what):
    """A stored indexer row vs the oracle's value before the format's rounding."""
    if cfg.idx_fmt == "fp4":
        compare_fp4_rows(rec, pre, what)
    else:
        assert_close(O.decode_values(rec, cfg.idx_fmt), pre, BF16_TOL, what)


def check_compressor(cfg, inp, dl, L):
    """Compressor + raw insertion of one decode step vs the oracle run from
    the drawn state; returns the cache bytes the GPU holds."""
    B, d = cfg.batch, cfg.head_dim
    raw_g = cpu(dl.raw)
    comp_g = cpu(dl.comp) if dl.comp is not None else None
    idx_g = cpu(dl.idx) if dl.idx is not None else None
    for b in range(B):
        p = int(inp.pos[b])
        seq = oracle_seq_from_init(L, inp.cache, b)
        seq.feed(p, inp.x[b][None], inp.u[b][None])
        z, _, _ = seq.raw_row(p)
        compare_rows(raw_g[b, p % cfg.swa], z, cfg.kv_fmt, d, cfg.n_rot, f"raw row b={b}")
        if cfg.ratio and (p + 1) % cfg.ratio == 0:
            i = (p + 1) // cfg.ratio - 1
            compare_rows(comp_g[b, i], seq.comp_row(i)[0], cfg.kv_fmt, d, cfg.n_rot, f"comp row {i} b={b}")
            if cfg.ratio == 4:
                check_idx_row(cfg, idx_g[b, i], seq.idx_row(i)[0], f"idx row {i} b={b}")
        if cfg.ratio:
            W = cfg.window
            kap = seq.kap[p]
            st = cpu(dl.st_kv)[b, p % W]
            assert_close(st, kap, (1e-4, 1e-5), f"state kappa b={b}")
    return raw_g, comp_g, idx_g


def run_decode_step_checks(cfg, inp, wts, tol):
    """ckv_decode_step (one call for the whole step) vs the oracle.  The
    indexer query is made tie-free on the cache the separate compressor call
    leaves; the fused call then runs on a fresh copy of the drawn cache, and
    its compressor rows, top-k set (on the bytes it wrote) and attention output
    are checked; its top-k list must also equal the separate calls' list."""
    B = cfg.batch
    log(f"[decode_step] {cfg.name} B={B} p={inp.pos[:4]}")
    L = oracle_layer(cfg, wts)
    pos_d = dev(inp.pos)
    x, u, q = dev(inp.x), dev(inp.u), dev(inp.q)
    qI, w = inp.qI, inp.w
    ref_dl = device_layer(cfg, wts, inp.cache)
    topk_a = None
    if cfg.ratio == 4:
        ref_dl.compress_decode(x, u, pos_d)
        torch.cuda.synchronize()
        seqs_a = [oracle_seq_from_bytes(L, cpu(ref_dl.raw)[b], cpu(ref_dl.comp)[b], cpu(ref_dl.idx)[b],
                                        int(inp.pos[b]) + 1) for b in range(B)]
        qI, w = tie_free_queries(cfg, seqs_a, inp.pos, inp.qI, inp.w)
        topk_a = torch.empty((B, cfg.top_k), dtype=torch.int32, device="cuda")
        ref_dl.indexer_decode(dev(qI), dev(w), pos_d, topk_a)
        torch.cuda.synchronize()
    dl = device_layer(cfg, wts, inp.cache)
    out, topk = dl.decode_step(x, u, q, dev(qI) if cfg.ratio == 4 else None,
                               dev(w) if cfg.ratio == 4 else None, pos_d)
    torch.cuda.synchronize()
    assert int(dl.status.abs().sum()) == 0
    raw_g, comp_g, idx_g = check_compressor(cfg, inp, dl, L)
    bseqs = [oracle_seq_from_bytes(L, raw_g[b], None if comp_g is None else comp_g[b],
                                   None if idx_g is None else idx_g[b], int(inp.pos[b]) + 1) for b in range(B)]
    tk = None
    if cfg.ratio == 4:
        tk = cpu(topk)
        for b in range(B):
            m = topk_margin(bseqs[b].index_scores(int(inp.pos[b]), qI[b], w[b]), cfg.top_k)
            assert m > 1e-6, f"query {b} not tie-free on the fused call's bytes (margin {m})"
        check_topk(cfg, inp, bseqs, qI, w, tk)
        # where both calls stored identical indexer rows, the lists must match exactly
        same = np.all(idx_g.reshape(B, -1) == cpu(ref_dl.idx).reshape(B, -1), axis=1)
        log(f"  identical indexer rows in {int(same.sum())}/{B} sequences")
        assert np.array_equal(tk[same], cpu(topk_a)[same]), "fused and separate top-k lists differ"
        ws = dl.ws[:L_sync_bytes(dl)]
        assert int(ws.view(torch.int32).abs().sum()) == 0, "sync region not left zero"
    check_attention(cfg, inp, bseqs, tk, out, tol)


def test_c5_c4a_fp4_indexer_decode_full_size():
    """The 16 x 131072-token c4a decode with the fp4 indexer cache, stage by
    stage: compressor rows (fp4 records against the oracle's encoding), top-k
    on the stored records, attention."""
    cfg = get_config("c5_fp4idx")
    run_decode_stage_checks(cfg, make_decode_inputs(cfg), make_layer_weights(cfg), FP8_TOL)


def test_c2_c4a_decode_full_size():
    cfg = get_config("c2")
    run_decode_stage_checks(cfg, make_decode_inputs(cfg), make_layer_weights(cfg), BF16_TOL)


def test_c5_c4a_fp8_decode_full_size():
    cfg = get_config("c5")
    run_decode_stage_checks(cfg, make_decode_inputs(cfg), make_layer_weights(cfg), FP8_TOL)


@pytest.mark.parametrize("name", ["c2_small", "c5_two_lane"])
def test_two_lane_decode(name):
    """Two-lane compressors (CKV_FLAG_TWO_LANE): the separate calls' stages
    against the oracle, then the single-call step (fused: both lanes'
    projection columns in the scan launch, the two-lane compressor in the
    selection block), whose top-k list must equal the separate calls'."""
    if name == "c2_small":
        cfg = get_config("c2").with_(batch=3, comp_cap=1024, top_k=128, seed=87, flags=TWO_LANE_FLAG,
                                     name="two_lane_c2_small")
        inp = make_decode_inputs(cfg, n_ctx=np.array([4000, 2501, 130], np.int64))
    else:
        cfg = get_config(name)
        inp = make_decode_inputs(cfg)
    wts = make_layer_weights(cfg)
    assert cfg.two_lane and wts.wkv.shape[0] == 2 * cfg.head_dim and wts.ape.shape == (4, 2 * cfg.head_dim)
    tol = FP8_TOL if cfg.kv_fmt == "e4m3" else BF16_TOL
    run_decode_stage_checks(cfg, inp, wts, tol)
    run_decode_step_checks(cfg, inp, wts, tol)


def test_c3_c128a_decode_full_size():
    cfg = get_config("c3")
    # force a few sequences onto a c128a boundary so the step emits a row
    n = G.context_lengths(cfg)
    n[:3] = (n[:3] // 128) * 128
    inp = make_decode_inputs(cfg, n_ctx=n)
    run_decode_stage_checks(cfg, inp, make_layer_weights(cfg), BF16_TOL)


def test_c5_c128a_and_swa_layers_decode():
    for name in ("c5_c128a", "c5_swa"):
        cfg = get_config(name)
        run_decode_stage_checks(cfg, make_decode_inputs(cfg), make_layer_weights(cfg), FP8_TOL)


def test_c5_decode_step_oracle_own_rows():
    """The C5 c4a step at full size with the oracle on its own rows: it runs
    this step's compressor itself from the drawn state (raw row, compressed
    row, indexer row) and scores, selects and attends over its own bytes; no
    GPU byte enters its scores or outputs.

    * top-k: the GPU's set must contain every row whose oracle score is above
      the oracle's k-th by more than 2 delta and only rows within 2 delta
      below it, delta being the largest score change the GPU's stored rows
      make (plus fp32 key rounding); where no score lies within that band of
      the k-th the set is unique and must be equal;
    * outputs: the oracle's attention with its own rows over the GPU's list,
      within the fp8 tolerance widened, element by element, by the change the
      GPU's stored rows make to that attention (the rows this step computes
      may differ by one E4M3 code: up to 1/8 of an element)."""
    cfg = get_config("c5")
    inp = make_decode_inputs(cfg)
    wts = make_layer_weights(cfg)
    L = oracle_layer(cfg, wts)
    B, k = cfg.batch, cfg.top_k
    own = []
    for b in range(B):
        sq = oracle_seq_from_init(L, inp.cache, b)
        sq.feed(int(inp.pos[b]), inp.x[b][None], inp.u[b][None])
        own.append(sq)
    dl = device_layer(cfg, wts, inp.cache)
    out, topk = dl.decode_step(dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w), dev(inp.pos))
    torch.cuda.synchronize()
    assert int(dl.status.abs().sum()) == 0
    raw_g, comp_g, idx_g = cpu(dl.raw), cpu(dl.comp), cpu(dl.idx)
    tkg, og = cpu(topk), out_values(out, cfg.act_fmt)
    unique = equal = 0
    for b in range(B):
        p = int(inp.pos[b])
        s_own = own[b].index_scores(p, inp.qI[b], inp.w[b])
        on_gpu_rows = oracle_seq_from_bytes(L, raw_g[b], comp_g[b], idx_g[b], p + 1)
        s_gpu = on_gpu_rows.index_scores(p, inp.qI[b], inp.w[b])
        smax = float(np.max(np.abs(s_own)))
        delta = float(np.max(np.abs(s_own - s_gpu))) + 1e-5 * smax
        kth = np.sort(s_own)[::-1][k - 1]
        g = tkg[b][tkg[b] >= 0]
        assert len(g) == k and len(set(g.tolist())) == k, f"sequence {b}: not {k} distinct rows"
        assert np.all(np.isin(np.nonzero(s_own > kth + 2 * delta)[0], g)), f"sequence {b}: a clear top-k row missing"
        assert np.all(s_own[g] >= kth - 2 * delta), f"sequence {b}: a row clearly outside the top-k selected"
        ref_set = O.topk_select(s_own, k)
        equal += int(np.array_equal(np.sort(g), ref_set))
        if int(np.sum(np.abs(s_own - kth) <= 2 * delta)) == 1:
            unique += 1
            assert np.array_equal(np.sort(g), ref_set), f"sequence {b}: unique top-k set differs"
        ref = own[b].attend(p, inp.q[b], tkg[b])
        row_change = np.abs(on_gpu_rows.attend(p, inp.q[b], tkg[b]) - ref)
        bad = np.abs(og[b] - ref) > FP8_TOL[1] + FP8_TOL[0] * np.abs(ref) + row_change
        assert not bad.any(), (f"c5 own-rows output b={b}: {int(bad.sum())} outside the band; "
                               f"first {np.argwhere(bad)[:3].tolist()}")
    log(f"[c5 own rows] sets equal to the oracle's in {equal}/{B} sequences ({unique} unique by the band rule)")


@pytest.mark.parametrize("name", ["c2", "c5", "c3", "c5_swa", "c5_fp4idx"])
def test_decode_step_full_size(name):
    """The single-call decode step at full size: fused on the c4a layers,
    the three separate calls on c128a and sliding-window-only layers."""
    cfg = get_config(name)
    run_decode_step_checks(cfg, make_decode_inputs(cfg), make_layer_weights(cfg),
                           FP8_TOL if cfg.kv_fmt == "e4m3" else BF16_TOL)


@pytest.mark.parametrize("cap,n", [(40000, (159000, 100001)), (1022, (4088, 2050))])
def test_decode_selection_beyond_one_block(cap, n):
    """Caches the one-block selection does not take (more than 32768 rows, or
    a capacity that is not a multiple of 4): the chunked classify + finish
    selection, through the stage calls and the single-call step."""
    cfg = get_config("c5").with_(batch=2, comp_cap=cap, seed=17, name=f"cap{cap}")
    inp = make_decode_inputs(cfg, n_ctx=np.array(n, np.int64))
    wts = make_layer_weights(cfg)
    run_decode_stage_checks(cfg, inp, wts, FP8_TOL)
    run_decode_step_checks(cfg, inp, wts, FP8_TOL)


@pytest.mark.parametrize("fmt,idx_fmt", [("bf16", "bf16"), ("e4m3", "bf16"), ("e4m3", "fp4")])
def test_decode_step_short_contexts(fmt, idx_fmt):
    """Fused step on short and ragged contexts: V <= k, the first rows,
    positions that close a row and positions that do not."""
    base = get_config("c2")
    cfg = base.with_(batch=8, comp_cap=512, kv_fmt=fmt, idx_fmt=idx_fmt, idx_heads=8, idx_dim=128, top_k=64,
                     seed=13, name=f"step_short_{fmt}_{idx_fmt}")
    n = np.array([1, 3, 4, 8, 259, 260, 1023, 2047], np.int64)
    run_decode_step_checks(cfg, make_decode_inputs(cfg, n_ctx=n), make_layer_weights(cfg),
                           FP8_TOL if fmt == "e4m3" else BF16_TOL)


@pytest.mark.parametrize("ratio,fmt,idx_fmt", [(4, "bf16", "bf16"), (4, "e4m3", "bf16"), (4, "bf16", "fp4"),
                                                (128, "bf16", "bf16"), (0, "bf16", "bf16")])
def test_short_contexts_and_ragged_batch(ratio, fmt, idx_fmt):
    """Positions below the window and the top-k size (V <= k, raw window < 128,
    row 0's empty slots), mixed per sequence."""
    base = get_config("c2")
    cfg = base.with_(ratio=ratio, batch=8, comp_cap={4: 512, 128: 64, 0: 0}[ratio], kv_fmt=fmt, idx_fmt=idx_fmt,
                     idx_heads=8 if ratio == 4 else 0, idx_dim=128 if ratio == 4 else 0,
                     top_k=64 if ratio == 4 else 0, seed=11, name=f"short_r{ratio}_{fmt}_{idx_fmt}")
    n = np.array([1, 4, 8, 100, 129, 260, 1024, 2047 if ratio != 128 else 8192], np.int64)
    run_decode_stage_checks(cfg, make_decode_inputs(cfg, n_ctx=n), make_layer_weights(cfg),
                            FP8_TOL if fmt == "e4m3" else BF16_TOL)


def test_bad_position_sets_status_and_spares_others():
    cfg = get_config("c2").with_(batch=4, comp_cap=64, top_k=16, seed=12, name="badpos")
    inp = make_decode_inputs(cfg, n_ctx=np.array([20, 40, 60, 80]))
    wts = make_layer_weights(cfg)
    dl = device_layer(cfg, wts, inp.cache)
    pos = inp.pos.copy()
    pos[1] = -1            # invalid position
    pos[2] = 64 * 4 + 3    # closes row 64: beyond comp_cap
    dl.n_tokens[2] = pos[2]   # in sequence, so that the capacity check is what refuses it
    raw_before = cpu(dl.raw).copy()
    dl.compress_decode(dev(inp.x), dev(inp.u), dev(pos))
    torch.cuda.synchronize()
    st = cpu(dl.status)
    assert st[0] == 0 and st[3] == 0
    assert st[1] & 1 and st[2] & 2
    raw_after = cpu(dl.raw)
    np.testing.assert_array_equal(raw_after[1], raw_before[1])       # untouched
    assert not np.array_equal(raw_after[0], raw_before[0])


@pytest.mark.parametrize("flags", [0, TWO_LANE_FLAG])
def test_c1_full_history_decode_chain(flags):
    """C1 from token 0: 1024 compress_append steps, then index + attend at 1023;
    every stored row and the output compared with the oracle's history run
    (one-lane and two-lane compressors)."""
    cfg = get_config("c1").with_(flags=flags)
    wts = make_layer_weights(cfg)
    T = cfg.n_ctx
    x, u, q, qI, w = G.make_token_stream(cfg, T)
    dl = device_layer(cfg, wts)
    L = oracle_layer(cfg, wts)
    seq = O.OracleSequence(L)
    seq.feed(0, x, u)
    xd, ud = dev(x), dev(u)
    for p in range(T):
        dl.compress_decode(xd[p:p + 1], ud[p:p + 1], dev(np.array([p], np.int32)), B=1)
    torch.cuda.synchronize()
    log("[c1] compressed 1024 tokens")
    comp_g, idx_g, raw_g = cpu(dl.comp)[0], cpu(dl.idx)[0], cpu(dl.raw)[0]
    for i in range(T // 4):
        compare_rows(comp_g[i], seq.comp_row(i)[0], "f32", cfg.head_dim, cfg.n_rot, f"comp row {i}")
        assert_close(idx_g[i], seq.idx_row(i)[0], BF16_TOL, f"idx row {i}")
    for t in range(T - 128, T):
        compare_rows(raw_g[t % 128], seq.raw_row(t)[0], "f32", cfg.head_dim, cfg.n_rot, f"raw {t}")
    p = T - 1
    qI1, w1 = tie_free_queries(cfg, [seq], [p], qI[p:p + 1], w[p:p + 1])
    pos_d = dev(np.array([p], np.int32))
    topk_d = torch.empty((1, cfg.top_k), dtype=torch.int32, device="cuda")
    dl.indexer_decode(dev(qI1), dev(w1), pos_d, topk_d, B=1)
    out = dl.new_out(1)
    dl.attn_decode(dev(q[p:p + 1]), pos_d, topk_d, out, B=1)
    torch.cuda.synchronize()
    ref = seq.query(p, q[p], qI1[0], w1[0])
    assert sets_equal(cpu(topk_d)[0], ref["topk"])
    assert_close(cpu(out)[0], ref["out_f64"], BF16_TOL, "c1 output")


@pytest.mark.parametrize("chunks,flags", [((1024,), 0), ((37, 1, 500, 486), 0), ((37, 1, 500, 486), TWO_LANE_FLAG)])
def test_c1_prefill_chunks_equal_sequential_decode(chunks, flags):
    """Chunked prefill from token 0 in chunks of varying size: stored rows and
    every query's output against the oracle (prefill = sequential decode);
    one-lane and two-lane compressors."""
    cfg = get_config("c1").with_(flags=flags)
    wts = make_layer_weights(cfg)
    T = sum(chunks)
    x, u, q, qI, w = G.make_token_stream(cfg, T)
    L = oracle_layer(cfg, wts)
    seq = O.OracleSequence(L)
    seq.feed(0, x, u)
    # tie-free per query: redraw q^I rows whose margin is too small
    qI, w = qI.copy(), w.copy()
    for p in range(T):
        for a in range(40):
            if topk_margin(seq.index_scores(p, qI[p], w[p]), cfg.top_k) > MARGIN:
                break
            nq, nw = G.draw_query_index(cfg, 1, sub=5000 + p, attempt=a + 1)
            qI[p], w[p] = nq[0], nw[0]
    dl = device_layer(cfg, wts, max_chunk=max(chunks))
    outs, tks = [], []
    p0 = 0
    for c in chunks:
        o, tk = dl.prefill(0, p0, dev(x[p0:p0 + c]), dev(u[p0:p0 + c]), dev(q[p0:p0 + c]), dev(qI[p0:p0 + c]),
                           dev(w[p0:p0 + c]))
        torch.cuda.synchronize()
        outs.append(cpu(o))
        tks.append(cpu(tk))
        p0 += c
    log(f"[c1 prefill] chunks {chunks} done")
    outs, tks = np.concatenate(outs), np.concatenate(tks)
    comp_g, idx_g = cpu(dl.comp)[0], cpu(dl.idx)[0]
    for i in range(T // 4):
        compare_rows(comp_g[i], seq.comp_row(i)[0], "f32", cfg.head_dim, cfg.n_rot, f"comp row {i}")
        assert_close(idx_g[i], seq.idx_row(i)[0], BF16_TOL, f"idx row {i}")
    st = cpu(dl.st_kv)[0]
    for t in range(T - 8, T):
        assert_close(st[t % 8], seq.kap[t], (1e-4, 1e-5), f"state {t}")
    for p in range(T):
        ref = seq.query(p, q[p], qI[p], w[p])
        assert sets_equal(tks[p], ref["topk"]), f"top-k of query {p}"
        assert_close(outs[p], ref["out_f64"], BF16_TOL, f"output of query {p}")


@pytest.mark.parametrize("name", ["c4", "c4_fp4idx", "c4_two_lane"])
def test_c4_prefill_chunk_sampled(name):
    """4096-token chunk at 61440 (compressor windows straddle the chunk edge):
    every emitted row, and sampled queries' top-k and outputs."""
    cfg = get_config(name)
    wts = make_layer_weights(cfg)
    inp = make_prefill_inputs(cfg)
    L = oracle_layer(cfg, wts)
    seq = oracle_seq_from_init(L, inp.cache, 0)
    seq.feed(inp.pos0, inp.x, inp.u)
    T, p0 = inp.T, inp.pos0
    sample = sorted({0, 1, 2, 3, 4, 127, 128, 1000, 2047, 2048, 3001, T - 5, T - 2, T - 1})
    qI, w = inp.qI.copy(), inp.w.copy()
    for n in sample:
        for a in range(40):
            if not (cfg.idx_fmt == "fp4" and fp4_query_fragile(L, p0 + n, qI[n])) and \
                    topk_margin(seq.index_scores(p0 + n, qI[n], w[n]), cfg.top_k) > MARGIN:
                break
            nq, nw = G.draw_query_index(cfg, 1, sub=9000 + n, attempt=a + 1)
            qI[n], w[n] = nq[0], nw[0]
    dl = device_layer(cfg, wts, inp.cache, max_chunk=T)
    out, tk = dl.prefill(0, p0, dev(inp.x), dev(inp.u), dev(inp.q), dev(qI), dev(w))
    torch.cuda.synchronize()
    log("[c4] prefill chunk done")
    comp_g, idx_g = cpu(dl.comp)[0], cpu(dl.idx)[0]
    for i in range(p0 // 4, (p0 + T) // 4, 37):
        compare_rows(comp_g[i], seq.comp_row(i)[0], cfg.kv_fmt, cfg.head_dim, cfg.n_rot, f"comp row {i}")
        check_idx_row(cfg, idx_g[i], seq.idx_row(i)[0], f"idx row {i}")
    i = p0 // 4   # the row whose window straddles the chunk edge
    compare_rows(comp_g[i], seq.comp_row(i)[0], cfg.kv_fmt, cfg.head_dim, cfg.n_rot, "edge row")
    og, tkg = out_values(out, cfg.act_fmt), cpu(tk)
    bseq = oracle_seq_from_bytes(L, None, comp_g, idx_g, 0)
    for n in sample:
        p = p0 + n
        # raw rows and rows of the chunk from the oracle's history; top-k on the GPU's index bytes
        sc = bseq.index_scores(p, qI[n], w[n])
        assert sets_equal(tkg[n], O.topk_select(sc, cfg.top_k)), f"top-k of query {n}"
        ref = seq.attend(p, inp.q[n], tkg[n])
        assert_close(og[n], ref, BF16_TOL, f"output of query {n}")


@pytest.mark.parametrize("idx_fmt", ["bf16", "fp4"])
def test_indexer_score_stage_keys(idx_fmt):
    """ckv_indexer_score_decode alone: keys decode to the oracle's scores."""
    from compressed_kv_sparse_amd import _lib as L
    cfg = get_config("c5").with_(batch=4, comp_cap=4096, seed=31, idx_fmt=idx_fmt, name=f"score_stage_{idx_fmt}")
    inp = make_decode_inputs(cfg, n_ctx=np.array([16384, 9001, 4100, 333]))
    wts = make_layer_weights(cfg)
    Lo = oracle_layer(cfg, wts)
    qI, w = inp.qI.copy(), inp.w.copy()
    for b in range(cfg.batch):   # fp4: queries whose MXFP4 codes cannot flip between fp32 and fp64
        a = 0
        while idx_fmt == "fp4" and fp4_query_fragile(Lo, int(inp.pos[b]), qI[b]):
            a += 1
            assert a < 40, f"no robust fp4 query for sequence {b}"
            nq, nw = G.draw_query_index(cfg, 1, sub=b, attempt=a)
            qI[b], w[b] = nq[0], nw[0]
    dl = device_layer(cfg, wts, inp.cache)
    # one guard row after the batch's [B, comp_cap] keys must stay untouched
    keys_g = torch.zeros((cfg.batch + 1, cfg.comp_cap), dtype=torch.int32, device="cuda")
    keys = keys_g[:cfg.batch]
    rc = L.indexer_score_decode(dl.desc, dl.cache, dev(qI), dev(w), dev(inp.pos), cfg.batch, keys,
                                torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    kg = cpu(keys).view(np.uint32)
    for b in range(cfg.batch):
        p = int(inp.pos[b])
        V = (p + 1) // 4
        k = kg[b, :V]
        bits = np.where(k & 0x80000000, k & 0x7FFFFFFF, ~k).astype(np.uint32)
        sc = bits.view(np.float32).astype(np.float64)
        seq = oracle_seq_from_bytes(Lo, cpu(dl.raw)[b], cpu(dl.comp)[b], cpu(dl.idx)[b], p + 1)
        ref = seq.index_scores(p, qI[b], w[b])
        assert np.max(np.abs(sc - ref)) <= 1e-4 * np.max(np.abs(ref)), f"scores b={b}"
    assert np.all(cpu(keys_g[cfg.batch]) == 0), "keys written past the batch's rows"


def test_score_timing_hook_brackets_one_launch():
    """ckv_time_next_score: the armed launch gives the same keys as an unarmed
    one, stamps both events (positive elapsed time, under a second), and the
    arming is used up by that launch."""
    from compressed_kv_sparse_amd import _lib as L
    cfg = get_config("c5").with_(batch=2, comp_cap=4096, seed=33, name="score_timing")
    inp = make_decode_inputs(cfg, n_ctx=np.array([16384, 5000]))
    dl = device_layer(cfg, make_layer_weights(cfg), inp.cache)
    qI, w, pos = dev(inp.qI), dev(inp.w), dev(inp.pos)
    st = torch.cuda.current_stream().cuda_stream
    plain = torch.zeros((cfg.batch, cfg.comp_cap), dtype=torch.int32, device="cuda")
    timed = torch.zeros_like(plain)
    assert L.indexer_score_decode(dl.desc, dl.cache, qI, w, pos, cfg.batch, plain, st) == 0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    torch.cuda.synchronize()
    assert L.time_next_score(a, b) == 0
    assert L.indexer_score_decode(dl.desc, dl.cache, qI, w, pos, cfg.batch, timed, st) == 0
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    assert 0.0 < ms < 1000.0, ms
    assert torch.equal(plain, timed)
    # disarmed: a further launch leaves the events where they were
    assert L.indexer_score_decode(dl.desc, dl.cache, qI, w, pos, cfg.batch, timed, st) == 0
    torch.cuda.synchronize()
    assert a.elapsed_time(b) == ms


@pytest.mark.parametrize("case", ["all_equal", "integer_ties"])
def test_decode_topk_with_exact_ties(case):
    """Top-k under exact score ties, where the lowest-index rule decides.
    all_equal: zero head weights make every score 0 -- the threshold bin holds
    every row (the exhaustive fallback select).  integer_ties: indexer rows and
    queries with small-integer entries and integer weights make every score an
    integer that fp32 and fp64 both hold exactly, with hundreds of rows per
    value -- the candidate select must apply the index rule among the keys
    equal to the k-th.  Compared bit-exactly with the oracle's full sort."""
    cfg = get_config("c5").with_(batch=2, comp_cap=16384, kv_fmt="bf16", seed=41, name=f"ties_{case}")
    n = np.array([65536, 40000])
    inp = make_decode_inputs(cfg, n_ctx=n)
    wts = make_layer_weights(cfg)
    rng = np.random.default_rng(7)
    c = inp.cache
    qI = inp.qI.copy()
    w = inp.w.copy()
    if case == "all_equal":
        w[:] = 0.0
    else:
        vals = np.array([-2.0, -1.0, 0.0, 1.0, 2.0], np.float32)
        c.idx[:] = G.bf16_bits_of_draw(rng.choice(vals, size=c.idx.shape).astype(np.float32))
        qI_f = rng.choice(vals, size=qI.shape).astype(np.float32)
        qI_f[..., cfg.idx_dim - 64:] = 0.0      # the rotated tail would make scores non-integer
        qI = G.bf16_bits_of_draw(qI_f)
        w = rng.integers(0, 3, size=w.shape).astype(np.float32)
    dl = device_layer(cfg, wts, c)
    topk = torch.empty((cfg.batch, cfg.top_k), dtype=torch.int32, device="cuda")
    L = oracle_layer(cfg, wts)
    for rep in range(2):     # twice: the first call must leave the workspace counters zero
        dl.indexer_decode(dev(qI), dev(w), dev(inp.pos), topk)
        torch.cuda.synchronize()
        tk = cpu(topk)
        for b in range(cfg.batch):
            p = int(inp.pos[b])
            seq = oracle_seq_from_bytes(L, cpu(dl.raw)[b], cpu(dl.comp)[b], cpu(dl.idx)[b], p + 1)
            sc = seq.index_scores(p, qI[b], w[b])
            ref = O.topk_select(sc, cfg.top_k)
            if case == "integer_ties":
                assert np.all(sc == np.round(sc)), "scores are not exact integers"
                kth = np.sort(sc)[::-1][cfg.top_k - 1]
                assert int((sc == kth).sum()) > 1, "no tie at the k-th score"
            assert np.array_equal(tk[b], np.sort(ref)), f"{case}: top-k differs for b={b} (rep {rep})"
    ws = dl.ws[:L_sync_bytes(dl)]
    assert int(ws.view(torch.int32).abs().sum()) == 0, "sync region not left zero"


@pytest.mark.parametrize("case", ["all_equal", "integer_ties"])
def test_prefill_topk_with_exact_ties(case):
    """The prefill indexer (score GEMM + per-query select) under exact ties:
    ckv_indexer_topk_prefill on a chunk of 300 queries at 39700 over stored
    index rows with small-integer entries, integer weights and a zero rotated
    tail, so every score is an integer both fp32 and fp64 hold exactly
    (all_equal: zero weights, every score 0).  Sampled queries' lists
    against the oracle's full sort, bit-exact (lowest index first among
    equal scores)."""
    from compressed_kv_sparse_amd import _lib as LIB
    cfg = get_config("c5").with_(batch=1, comp_cap=16384, kv_fmt="bf16", seed=43, name=f"pf_ties_{case}")
    inp = make_decode_inputs(cfg, n_ctx=np.array([40000]))
    wts = make_layer_weights(cfg)
    rng = np.random.default_rng(11)
    c = inp.cache
    T, pos0 = 300, 39700
    vals = np.array([-2.0, -1.0, 0.0, 1.0, 2.0], np.float32)
    c.idx[:] = G.bf16_bits_of_draw(rng.choice(vals, size=c.idx.shape).astype(np.float32))
    qI_f = rng.choice(vals, size=(T, cfg.idx_heads, cfg.idx_dim)).astype(np.float32)
    qI_f[..., cfg.idx_dim - 64:] = 0.0
    qI = G.bf16_bits_of_draw(qI_f)
    if case == "all_equal":
        w = np.zeros((T, cfg.idx_heads), np.float32)
    else:
        w = rng.integers(0, 3, size=(T, cfg.idx_heads)).astype(np.float32)
    dl = device_layer(cfg, wts, c, max_chunk=T)
    topk = torch.full((T, cfg.top_k), -7, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert LIB.indexer_topk_prefill(dl.desc, dl.cache, dev(qI), dev(w), 0, pos0, T, topk, dl.ws, dl.ws_bytes,
                                    st) == 0
    torch.cuda.synchronize()
    tk = cpu(topk)
    L = oracle_layer(cfg, wts)
    bseq = oracle_seq_from_bytes(L, None, cpu(dl.comp)[0], cpu(dl.idx)[0], 0)
    for n in sorted({0, 1, 63, 64, 150, 255, 256, T - 2, T - 1} | set(range(7, T, 41))):
        p = pos0 + n
        sc = bseq.index_scores(p, qI[n], w[n])
        ref = np.sort(O.topk_select(sc, cfg.top_k))
        assert np.all(sc == np.round(sc)), "scores are not exact integers"
        kth = np.sort(sc)[::-1][cfg.top_k - 1]
        assert int((sc == kth).sum()) > 1, "no tie at the k-th score"
        assert np.array_equal(tk[n], ref), f"{case}: top-k of query {n} differs"


def L_sync_bytes(dl):
    from compressed_kv_sparse_amd import _lib as L
    return L.workspace_sync_bytes(dl.desc, L.CKV_MODE_DECODE, dl.batch)
