"""GPU parity of the next-token sampler (gpt2_sample, and generation with sampling) against the
oracle's sample_filter / sample_next on the same seeded fp32 logits, uniform numbers and histories.

The GPU applies the penalty and the temperature in fp32 and sums probability mass in 2^-40 fixed
point; the oracle works in fp64. A decision that hinges on a comparison closer than the rounding of
those sums (u within DELTA of a step of the CDF, a cumulative mass within DELTA of top_p) may fall
either way, so for every row:
  * the sampled token equals the oracle's draw at (u, top_p), or at one of u +- DELTA combined with
    top_p +- DELTA (the only results the definition allows at that rounding level);
  * the kept-set size lies between the oracle's sizes at top_p - DELTA and top_p + DELTA;
and at least 95% of the rows must match the oracle's (u, top_p) result exactly. Decisions that do
not involve mass (top-k, argmax, ties, -inf, vocabulary bounds) must match exactly.
"""
import numpy as np
import pytest
import torch

from oracle import gpt2_oracle as O
from decoder_only_transformer_gpt2_amd import synth

pytestmark = pytest.mark.gpu

DELTA = 1e-4


@pytest.fixture(scope="session")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from decoder_only_transformer_gpt2_amd import gpt2
    gpt2.lib()  # raises when the library has not been built
    return gpt2


def log(msg):
    print(msg, flush=True)


def run_gpu(g, logits, u, hist, T, k, p, pen, ld=None, ws=True):
    B, V = logits.shape
    ld = V if ld is None else ld
    buf = torch.full((B, ld), float("nan"), dtype=torch.float32)
    buf[:, :V] = torch.from_numpy(logits)
    lg = buf.cuda()[:, :V]
    h = torch.from_numpy(np.ascontiguousarray(hist)).cuda() if hist is not None and hist.shape[1] else None
    n_kept = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    out = g.sample(lg, torch.from_numpy(u).cuda(), history=h, temperature=T, top_k=k, top_p=p,
                   repetition_penalty=pen, n_kept=n_kept, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64), n_kept.cpu().numpy().astype(np.int64)


def check_rows(g, logits, u, hist, T, k, p, pen, ld=None, min_exact=0.95):
    B, V = logits.shape
    log(f"  sample B={B} V={V} ld={ld} T={T} k={k} p={p} pen={pen}")
    tok, kept = run_gpu(g, logits, u, hist, T, k, p, pen, ld)
    # the one-workgroup-per-row path (no workspace) gives the same tokens and kept-set sizes
    tok1, kept1 = run_gpu(g, logits, u, hist, T, k, p, pen, ld, ws=None)
    assert np.array_equal(tok, tok1) and np.array_equal(kept, kept1)
    assert np.all((tok >= 0) & (tok < V))
    exact = 0
    for b in range(B):
        row = logits[b:b + 1].astype(np.float64)
        hb = None if hist is None else hist[b:b + 1]
        ref = int(O.sample_next(row, u[b:b + 1], hb, T, k, p, pen)[0])
        _, keep = O.sample_filter(row, hb, T, k, p, pen)
        n_ref = int(keep.sum())
        if tok[b] == ref and kept[b] == n_ref:
            exact += 1
            continue
        ps = sorted({p, min(1.0, p + DELTA), max(DELTA, p - DELTA)}) if p < 1.0 else [1.0]
        sizes = [int(O.sample_filter(row, hb, T, k, pp, pen)[1].sum()) for pp in ps]
        assert min(sizes) <= kept[b] <= max(sizes), (b, kept[b], sizes)
        allowed = {int(O.sample_next(row, np.array([uu]), hb, T, k, pp, pen)[0])
                   for uu in (max(0.0, u[b] - DELTA), float(u[b]), min(1.0 - 1e-12, u[b] + DELTA)) for pp in ps}
        assert tok[b] in allowed, (b, tok[b], ref, allowed)
    log(f"    exact rows {exact}/{B}")
    assert exact >= min_exact * B
    return tok, kept


# the knobs of the pages' generation example: temperature 0.7, top-k 50, top-p 0.95, penalty 1.2
PAGE_KNOBS = dict(T=0.7, k=50, p=0.95, pen=1.2)


def test_sample_gpt2_vocab_page_knobs(g):
    logits, u, hist = synth.make_sampling_inputs(32, 50257, n_hist=64, n_peaked=16)
    check_rows(g, logits, u, hist, **PAGE_KNOBS)


@pytest.mark.parametrize("T,k,p,pen", [
    (1.0, 0, 1.0, 1.0),      # plain softmax draw over the whole vocabulary
    (1.0, 0, 0.9, 1.0),      # top-p alone
    (0.8, 1000, 1.0, 1.0),   # top-k alone, wide
    (1.3, 0, 0.5, 1.0),      # top-p in the bulk of a flattened distribution
    (0.5, 40, 0.8, 2.0),     # every knob, strong penalty
])
def test_sample_gpt2_vocab_knobs(g, T, k, p, pen):
    logits, u, hist = synth.make_sampling_inputs(24, 50257, n_hist=100, n_peaked=12)
    check_rows(g, logits, u, hist, T, k, p, pen)


def test_sample_top_k_one_is_argmax(g):
    logits, u, _ = synth.make_sampling_inputs(16, 50257, n_peaked=4)
    tok, kept = run_gpu(g, logits, u, None, 1.0, 1, 1.0, 1.0)
    assert np.array_equal(tok, O.argmax_first(logits.astype(np.float64)))
    assert np.all(kept == 1)


@pytest.mark.parametrize("V", [1, 7, 64, 1000, 1025, 8193, 50257, 65536])
def test_sample_ragged_vocab(g, V):
    logits, u, hist = synth.make_sampling_inputs(6, V, n_hist=9, n_peaked=3)
    check_rows(g, logits, u, hist, T=0.8, k=min(20, V), p=0.9, pen=1.3)


def test_sample_strided_rows(g):
    logits, u, hist = synth.make_sampling_inputs(8, 3000, n_hist=5, n_peaked=2)
    check_rows(g, logits, u, hist, T=0.9, k=100, p=0.9, pen=1.1, ld=3000 + 37)


def test_sample_ties_exact(g):
    """Integer-valued logits: many exact ties. top-k keeps every tie of the k-th value (sizes
    compared exactly); the draw among ties follows vocabulary order."""
    rng = np.random.Generator(np.random.PCG64(11))
    logits = np.round(rng.standard_normal((8, 4000)) * 2.0).astype(np.float32)
    u = rng.random(8).astype(np.float32)
    tok, kept = run_gpu(g, logits, u, None, 1.0, 10, 1.0, 1.0)
    for b in range(8):
        _, keep = O.sample_filter(logits[b:b + 1].astype(np.float64), top_k=10)
        assert kept[b] == keep.sum() and keep[0, tok[b]]
    check_rows(g, logits, u, None, T=1.0, k=10, p=1.0, pen=1.0)


def test_sample_long_candidate_lists(g):
    """Rows whose screened candidate list is long: a plateau of equal logits at the top (hundreds
    or thousands of tokens tie above the bound) sends the row to the general path; both paths and
    the oracle agree."""
    rng = np.random.Generator(np.random.PCG64(14))
    logits = (rng.standard_normal((6, 50257)) * 2.0).astype(np.float32)
    for b, width in enumerate((300, 600, 2000, 5000, 20000, 50257)):
        ids = rng.choice(50257, size=width, replace=False)
        logits[b, ids] = 7.0
    u = rng.random(6).astype(np.float32)
    check_rows(g, logits, u, None, T=1.0, k=50, p=1.0, pen=1.0)
    check_rows(g, logits, u, None, T=0.7, k=50, p=0.9, pen=1.0)


def test_sample_masked_vocab(g):
    """-inf logits (a masked vocabulary) are never drawn and do not upset the thresholds."""
    logits, u, _ = synth.make_sampling_inputs(8, 5000, n_peaked=2)
    rng = np.random.Generator(np.random.PCG64(12))
    mask = rng.random(logits.shape) < 0.7
    logits[mask] = -np.inf
    tok, _ = run_gpu(g, logits, u, None, 1.0, 0, 1.0, 1.0)
    assert not np.any(mask[np.arange(8), tok])
    check_rows(g, logits, u, None, T=0.7, k=30, p=0.95, pen=1.0)
    check_rows(g, logits, u, None, T=1.0, k=0, p=1.0, pen=1.0)


def test_sample_u_extremes(g):
    """u = 0 draws the first kept token in vocabulary order; u just below 1 the last one."""
    logits, _, _ = synth.make_sampling_inputs(4, 2000, n_peaked=2)
    for uu in (0.0, np.float32(1.0) - np.float32(2.0 ** -24)):
        u = np.full(4, uu, dtype=np.float32)
        tok, _ = run_gpu(g, logits, u, None, 1.0, 25, 1.0, 1.0)
        for b in range(4):
            _, keep = O.sample_filter(logits[b:b + 1].astype(np.float64), top_k=25)
            kept_ids = np.nonzero(keep[0])[0]
            assert tok[b] == (kept_ids[0] if uu == 0.0 else kept_ids[-1]), (uu, b)


def test_sample_history_edge_ids(g):
    """Repeated, negative and out-of-vocabulary history ids: each valid id is penalised once."""
    logits, u, _ = synth.make_sampling_inputs(6, 3000, n_peaked=6)
    top = np.argsort(-logits, axis=1)[:, :6].astype(np.int32)
    hist = np.concatenate([top, top, np.full((6, 3), -5, np.int32), np.full((6, 2), 3000, np.int32)], axis=1)
    check_rows(g, logits, u, hist, T=1.0, k=8, p=1.0, pen=3.0)
    check_rows(g, logits, u, hist, T=0.6, k=0, p=0.9, pen=0.5)


def test_sample_frequencies_on_a_grid(g):
    """4096 copies of one row drawn at u = (i + 0.5) / 4096: each token's share of the draws is its
    probability over the kept set to within 1/4096 plus the rounding window."""
    N, V = 4096, 700
    logits, _, _ = synth.make_sampling_inputs(1, V, n_peaked=1)
    rows = np.repeat(logits, N, axis=0)
    u = ((np.arange(N) + 0.5) / N).astype(np.float32)
    for T, k, p in ((1.0, 0, 1.0), (0.7, 50, 0.95)):
        tok, _ = run_gpu(g, rows, u, None, T, k, p, 1.0)
        z, keep = O.sample_filter(logits.astype(np.float64), None, T, k, p)
        q = np.where(keep[0], np.exp(z[0] - z[0][keep[0]].max()), 0.0)
        q /= q.sum()
        freq = np.bincount(tok, minlength=V) / N
        assert np.abs(freq - q).max() <= 1.0 / N + 2 * DELTA, (T, k, p)
        assert not np.any(freq[~keep[0]])


def test_sample_errors(g):
    lg = torch.zeros((2, 10), device="cuda")
    u = torch.zeros((2,), device="cuda")
    with pytest.raises(g.GPT2Error):
        g.sample(lg, u, temperature=0.0)
    with pytest.raises(g.GPT2Error):
        g.sample(lg, u, top_p=0.0)
    with pytest.raises(g.GPT2Error):
        g.sample(torch.zeros((1, 70000), device="cuda"), u[:1])


def test_generate_sampled_f32_teacher_forced(g):
    """Generation with sampling on the fp32 GPT-2 small: at every step the new token is the
    oracle's draw from the oracle's logits for the GPU's own prefix, with the whole sequence so far
    as the penalty history (the rounding window as above)."""
    w = synth.make_weights(synth.GPT2_SMALL, bf16=False)
    s = synth.GPT2_SMALL
    m = g.GPT2(g.ModelConfig(n_vocab=s.n_vocab, n_ctx=s.n_ctx, d_model=s.d_model, n_head=s.n_head,
                             n_layer=s.n_layer, d_mlp=s.d_mlp, dtype="f32"))
    m.load_numpy(w)
    prompt = synth.make_tokens(2, 4)
    n_new = 5
    u = np.random.Generator(np.random.PCG64(13)).random((n_new, 2)).astype(np.float32)
    knobs = dict(temperature=0.05, top_k=50, top_p=0.95, repetition_penalty=1.2)
    out = m.generate(torch.from_numpy(prompt).cuda(), n_new, do_sample=True, u=torch.from_numpy(u).cuda(),
                     **knobs).cpu().numpy()
    log(f"  sampled {out.tolist()}")
    assert np.array_equal(out[:, :4], prompt)
    exact = 0
    for i in range(n_new):
        prefix = out[:, :4 + i]
        lg = O.forward(w, prefix, s.n_head, s.n_layer)[:, -1]
        ref = O.sample_next(lg, u[i], prefix, 0.05, 50, 0.95, 1.2)
        for b in range(2):
            if out[b, 4 + i] == ref[b]:
                exact += 1
                continue
            allowed = {int(O.sample_next(lg[b:b + 1], np.array([uu]), prefix[b:b + 1], 0.05, 50, pp, 1.2)[0])
                       for uu in (u[i, b] - DELTA, u[i, b] + DELTA) for pp in (0.95 - DELTA, 0.95 + DELTA)}
            assert out[b, 4 + i] in allowed, (i, b)
    assert exact >= 2 * n_new - 1
