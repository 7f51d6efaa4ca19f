"""GPU parity of the decode attention over an MLA sub-pool's dense latent view
(ukv_mla_decode_attention): floating point, within the fp32 error bound the
oracle derives per request and head for the kernel's arithmetic (exact bf16
products, fp32 sums, weights split into two bf16 parts: relative error
2^-16), and bit-exact where the arithmetic is exact (one position per
request).  Queries that are zero but for a few dims make the bound tight
enough to catch a weight kept at bf16 precision on short requests; dense
queries check the scores over the whole 576-wide row.  The bound takes the
longest sum chain any split of a request can form, from its length alone, so
no test depends on how the kernel cuts the batch into spans; the span
structure itself is checked exactly with zero queries over small-integer
latents, where every float32 partial sum is exact.

The pool holds Irwin-Hall bf16 values generated bit-identically on the device
and on the host, so the oracle reads the same bytes without any copy back.
"""
import numpy as np
import pytest
import torch

import store_gather_amd as U
import ukv_workloads as W
from oracle import attention as A
from parity_util import log, to_dev
from test_gpu_attention import GaussPair, check_exact_mean, requests

pytestmark = pytest.mark.gpu

LAT, VD = 576, 512


def bound_terms(n):
    """The longest fp32 sum chain any split of n positions can form when each weight
    enters the value product as two bf16 parts: from the request's length alone, so the
    bound holds however the kernel cuts the batch into spans.  (Where that bound is too
    loose to see a lost or doubled span of a long request, the exact zero-query tests
    below see it.)"""
    return A.chain_terms_any_split(n, parts_per_weight=2)


@pytest.fixture(autouse=True)
def _name(request):
    log(f"\n[gpu] {request.node.name}")
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


def queries(seed, R, hq, sparse=False):
    q = W.irwin_hall_bf16_host(seed, 0, 2 * R * hq * LAT).reshape(R, hq, LAT).copy()
    if sparse:  # zero but for a few dims in the value part and past it
        keep = np.zeros(LAT, bool)
        keep[[0, 77, 300, 511, 512, 540, 575]] = True
        q[:, :, ~keep] = 0
    return q


def run_mla(pair, layer, q_bits, bt, lens, window, scale, max_len, sub=0, workspace=None):
    q = torch.from_numpy(q_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    out = U.ukv_mla_decode_attention(pair.gpu, sub, layer, q, to_dev(bt), to_dev(lens), max_len, window, scale,
                                     workspace=workspace)
    return out.cpu().numpy().astype(np.float64), U.ukv_pool_error_flags(pair.gpu)


def oracle_mla(pair, layer, q_bits, bt, lens, window, scale, max_len, sub=0, requests=None):
    return A.decode_attention(pair.orc, sub, layer, q_bits, bt, lens, window, scale, max_len, read=pair.read,
                              requests=requests, bound_terms=bound_terms,
                              v_dim=VD, weight_rel=A.BF16_SPLIT_REL)


def check_close(got, exp, bound, what):
    err = np.abs(got - exp)
    worst = float(err.max()) if err.size else 0.0
    log(f"  {what}: max |err| {worst:.3e}, min bound {float(bound[bound > 0].min()) if (bound > 0).any() else 0:.3e}")
    assert (err <= bound[:, :, None]).all(), f"{what}: error {worst} above the fp32 bound"


LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 255, 256, 257, 600, 0, 1000, 2000, 47]


@pytest.mark.parametrize("hq,ps", [(16, 64), (32, 16), (16, 1)])
@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("sparse", [False, True])
def test_mla_decode_attention_parity(hq, ps, window, sparse):
    lens = np.array(LENS, dtype=np.int32)
    P = int(sum((int(n) + ps - 1) // ps for n in lens)) + 4
    pair = GaussPair([W.mla(3, P)], ps, seed=hq + ps)
    pages = requests(5, P, ps, lens)
    req = W.padded_table(pages)
    bt, ef = pair.orc.build_page_table(0, req, lens)
    assert ef == frozenset()
    q = queries(40 + hq, lens.size, hq, sparse)
    scale = A.default_scale(192)
    max_len = int(lens.max())
    for layer in (0, 2):
        got, gf = run_mla(pair, layer, q, bt, lens, window, scale, max_len)
        exp, ef, bound = oracle_mla(pair, layer, q, bt, lens, window, scale, max_len)
        assert gf == ef == frozenset()
        check_close(got, exp, bound, f"layer {layer}")
        assert np.array_equal(got[lens == 0], np.zeros_like(got[lens == 0]))
        assert np.isfinite(got).all()


SPAN_SHAPES = [(512, 16, 8192, 0), (1, 16, 60000, 0), (300, 16, 40, 0), (96, 32, 8000, 0), (8, 48, 2000, 700),
               (130, 16, 3000, 0)]


def span_batch(num_reqs, len_hi):
    g = np.random.default_rng(num_reqs + len_hi)
    lens = g.integers(1, len_hi, size=num_reqs, endpoint=True).astype(np.int32)
    lens[0] = len_hi
    if num_reqs == 130:
        lens[g.choice(num_reqs - 1, 30, replace=False) + 1] = 0
    return lens


@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("num_reqs,hq,len_hi,window", SPAN_SHAPES)
def test_mla_decode_attention_span_shapes(num_reqs, hq, len_hi, window, sparse):
    """Batches that cut the balanced split differently: ~2,000-position spans over 512
    requests, one request merged from 235 spans, spans that cross a dozen tiny
    requests, two and three head groups (one with a window), and empty requests among
    the rest; sampled requests checked (shared pages keep the pool small)."""
    ps = 64
    lens = span_batch(num_reqs, len_hi)
    P = 700
    pair = GaussPair([W.mla(1, P)], ps, seed=num_reqs)
    pages = requests(4, P, ps, lens, share=True)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    q = queries(num_reqs, num_reqs, hq, sparse)
    scale = A.default_scale(192)
    got, gf = run_mla(pair, 0, q, bt, lens, window, scale, len_hi)
    sample = sorted({0, min(1, num_reqs - 1), num_reqs // 2, num_reqs - 1, int(np.argmin(lens))})
    exp, ef, bound = oracle_mla(pair, 0, q, bt, lens, window, scale, len_hi, requests=sample)
    assert np.array_equal(got[lens == 0], np.zeros_like(got[lens == 0]))
    assert gf == ef == frozenset()
    check_close(got[sample], exp[sample], bound[sample], f"{num_reqs} requests up to {len_hi}")
    assert np.isfinite(got).all()


@pytest.mark.parametrize("num_reqs,hq,len_hi,window", SPAN_SHAPES + [(1, 16, 60000, 9000), (4096, 16, 64, 0)])
def test_mla_decode_attention_span_merge_exact(num_reqs, hq, len_hi, window):
    """Zero queries over small-integer latents: every weight is 1 (both of its bf16
    parts exact) and every float32 partial sum exact, so each output is the mean of the
    request's value fronts up to one division, whatever the balanced split.  A span lost,
    counted twice or merged into the wrong request shows at any length (on the CPU the
    same tolerance rejects a dropped 16-position tile or 256-position span of a
    60,000-position request).  Every request of every span shape is checked."""
    ps = 64
    lens = span_batch(num_reqs, len_hi)
    P = 700
    pair = GaussPair([W.mla(1, P)], ps, seed=num_reqs + 3, ints=True)
    pages = requests(4, P, ps, lens, share=True)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    q = np.zeros((num_reqs, hq, LAT), np.uint16)
    got, gf = run_mla(pair, 0, q, bt, lens, window, 0.3, len_hi)
    exp, ef = A.decode_attention(pair.orc, 0, 0, q, bt, lens, window, 0.3, len_hi, v_dim=VD, uniform=True)
    assert gf == ef == frozenset()
    check_exact_mean(got, exp, f"{num_reqs} requests up to {len_hi}")


def test_mla_decode_attention_single_position_is_exact():
    """window = 1 keeps only the last position: the output is the front of that latent
    row, exactly, for any length and either head count."""
    ps = 64
    lens = np.array([1, 16, 17, 32, 33, 256, 257, 700, 1023], dtype=np.int32)
    P = int(sum((int(n) + ps - 1) // ps for n in lens)) + 2
    pair = GaussPair([W.mla(2, P)], ps, seed=5)
    pages = requests(7, P, ps, lens)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    for hq in (16, 64):
        q = queries(hq, lens.size, hq)
        got, gf = run_mla(pair, 1, q, bt, lens, 1, 0.7, int(lens.max()))
        exp, ef = A.decode_attention(pair.orc, 0, 1, q, bt, lens, 1, 0.7, v_dim=VD)
        assert gf == ef == frozenset()
        assert np.array_equal(got, exp)


def test_mla_decode_attention_conditions():
    ps, hq = 16, 16
    lens = np.array([40, 300, 40, 0, 90, 600], dtype=np.int32)
    P = 80
    pair = GaussPair([W.mla(4, P)], ps, seed=8)  # 4 blocks per page: entries off a page start exist
    pages = requests(3, P, ps, lens)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    q = queries(1, lens.size, hq)
    scale = A.default_scale(192)
    good, gf = run_mla(pair, 0, q, bt, lens, 0, scale, 600)
    assert gf == frozenset()
    bpp = pair.orc.plan.subs[0].blocks_per_page
    for bad in (-1, 1, P * bpp, int(bt[1, 0]) + bpp // 2):
        b = bt.copy()
        b[1, 17] = bad
        got, gf = run_mla(pair, 0, q, b, lens, 0, scale, 600)
        exp, ef = A.decode_attention(pair.orc, 0, 0, q, b, lens, 0, scale, 600, v_dim=VD)
        assert gf == ef == {"bad_block"}
        assert np.array_equal(got[1], np.zeros_like(got[1]))
        assert np.array_equal(np.delete(got, 1, 0), np.delete(good, 1, 0))
    # the same bad entry outside a window is never read
    b = bt.copy()
    b[5, 2] = -1
    got, gf = run_mla(pair, 0, q, b, lens, 128, scale, 600)
    assert gf == frozenset()
    # table narrower than a request, and a request past max_seq_len
    got, gf = run_mla(pair, 0, q, np.ascontiguousarray(bt[:, :10]), lens, 0, scale, 600)
    exp, ef = A.decode_attention(pair.orc, 0, 0, q, bt[:, :10], lens, 0, scale, 600, v_dim=VD)
    assert gf == ef == {"bad_block"}
    assert np.array_equal(got[[1, 5]], np.zeros_like(got[[1, 5]]))
    assert np.array_equal(got[[0, 2, 3, 4]], good[[0, 2, 3, 4]])
    got, gf = run_mla(pair, 0, q, bt, lens, 0, scale, 300)
    exp, ef = A.decode_attention(pair.orc, 0, 0, q, bt, lens, 0, scale, 300, v_dim=VD)
    assert gf == ef == {"layout"}
    assert np.array_equal(got[5], np.zeros_like(got[5])) and np.array_equal(got[:5], good[:5])
    got, gf = run_mla(pair, 0, q, bt, lens, 0, scale, 0)
    assert gf == {"layout"} and not got.any()


def test_mla_decode_attention_host_errors():
    pair = GaussPair([W.mha(2, 2, 128, 8), W.mla(2, 8), W.mla(2, 8, latent_dim=512)], 16, seed=1, host=False)
    q = torch.zeros((2, 16, LAT), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(U.UkvError, match="not MLA"):
        U.ukv_mla_decode_attention(pair.gpu, 0, 0, q, bt, lens, 16, 0, 0.1)
    with pytest.raises(U.UkvError, match="layer"):
        U.ukv_mla_decode_attention(pair.gpu, 1, 2, q, bt, lens, 16, 0, 0.1)
    with pytest.raises(U.UkvError, match="supported"):
        U.ukv_mla_decode_attention(pair.gpu, 2, 0, q, bt, lens, 16, 0, 0.1)
    with pytest.raises(U.UkvError, match="supported"):
        U.ukv_mla_decode_attention(pair.gpu, 1, 0, q, bt, lens, 16, 0, 0.1, v_dim=576)
    with pytest.raises(U.UkvError, match="multiple of 16"):
        U.ukv_mla_decode_attention(pair.gpu, 1, 0, torch.zeros((2, 8, LAT), dtype=torch.bfloat16, device="cuda"),
                                   bt, lens, 16, 0, 0.1)
    with pytest.raises(U.UkvError, match="workspace"):
        U.ukv_mla_decode_attention(pair.gpu, 1, 0, q, bt, lens, 16, 0, 0.1,
                                   workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(U.UkvError, match="not finite"):
        U.ukv_mla_decode_attention(pair.gpu, 1, 0, q, bt, lens, 16, 0, float("nan"))
    assert U.ukv_mla_decode_attention_workspace_bytes(pair.gpu, 1, 2, 8, VD, 16, 0) == 0
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


@pytest.mark.parametrize("sparse", [False, True])
def test_mla_decode_attention_full_hybrid_sampled(sparse):
    """The hybrid workload's MLA sub-pool at full size (24 layers, 576-wide latents,
    page 64, 128 requests of 256-16,384 positions, ~28 GiB) with 16 query heads: all
    layers run, six sampled requests checked on two layers; then zero queries over
    small-integer latents, every request checked against its exact mean."""
    w = W.hybrid()
    ps = w.page_size
    shape = w.shapes[1]
    lens = w.req_lens[1]
    pair = GaussPair([shape], ps, seed=33, host=False)
    req = W.padded_table(w.req_pages[1])
    bt_dev = U.ukv_build_page_table(pair.gpu, 0, to_dev(req), to_dev(lens))
    bt, ef = pair.orc.build_page_table(0, req, lens)
    assert np.array_equal(bt_dev.cpu().numpy(), bt) and ef == frozenset()
    R, hq = lens.size, 16
    q = queries(78, R, hq, sparse)
    qd = torch.from_numpy(q.view(np.int16)).to("cuda").view(torch.bfloat16)
    scale = A.default_scale(192)
    max_len = int(lens.max())
    ws = torch.empty(U.ukv_mla_decode_attention_workspace_bytes(pair.gpu, 0, R, hq, VD, max_len, 0),
                     dtype=torch.uint8, device="cuda")
    sample = sorted({0, R - 1, int(np.argmax(lens)), int(np.argmin(lens)), 50, 99})
    for layer in range(shape.layer_num):
        out = U.ukv_mla_decode_attention(pair.gpu, 0, layer, qd, bt_dev, to_dev(lens), max_len, 0, scale,
                                         workspace=ws)
        if layer in (0, shape.layer_num - 1):
            got = out.cpu().numpy().astype(np.float64)
            exp, ef, bound = oracle_mla(pair, layer, q, bt, lens, 0, scale, max_len, requests=sample)
            assert ef == frozenset()
            check_close(got[sample], exp[sample], bound[sample], f"layer {layer}")
            assert np.isfinite(got).all()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    if sparse:
        return
    pair.set_values(ints=True)
    q0 = np.zeros_like(q)
    out = U.ukv_mla_decode_attention(pair.gpu, 0, 11, torch.zeros_like(qd), bt_dev, to_dev(lens), max_len, 0, scale,
                                     workspace=ws)
    exp, ef = A.decode_attention(pair.orc, 0, 11, q0, bt, lens, 0, scale, max_len, v_dim=VD,
                                 read_words=pair.read_words, uniform=True)
    assert ef == frozenset()
    check_exact_mean(out.cpu().numpy().astype(np.float64), exp, "layer 11, every request")
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


@pytest.mark.parametrize("where", ["late", "first", "moderate"])
def test_mla_decode_attention_dominant_scores(where):
    """Scores far apart: one position's score exceeds the rest by ~1,000 (log2 units) late in
    a request (past the first tile, so the weights' reference is outgrown and the kernel
    takes its max-first pass), or in the first tile, or a later tile exceeds the first by
    ~30 (weights up to 2^30 against the first tile's reference)."""
    ps, hq = 16, 16
    lens = np.array([700, 300, 45, 2000], dtype=np.int32)
    P = int(sum((int(n) + ps - 1) // ps for n in lens)) + 4
    pair = GaussPair([W.mla(2, P)], ps, seed=17)
    pages = requests(9, P, ps, lens)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    q = queries(3, lens.size, hq)
    dim = 540  # a rotary dim: the planted values change scores, not values
    big = {"late": 100.0, "first": 100.0, "moderate": 24.0}[where]
    q[:, :, dim] = np.float32(big).view(np.uint32) >> 16  # bf16 bits of an exact value
    rb = pair.orc.row_bytes(0)
    for r, n in enumerate(lens):
        j = {"late": int(n) - 5, "first": 3, "moderate": int(n) // 2}[where]
        kid = int(pages[r][j // ps]) * pair.orc.plan.subs[0].blocks_per_page * ps + j % ps
        off = pair.orc.view_base(0, 1, 0) + kid * rb + 2 * dim
        bits = np.array([np.float32(big).view(np.uint32) >> 16], dtype=np.uint16).view(np.uint8)
        pair.orc.raw[off: off + 2] = bits
        pair.gpu.raw[off: off + 2] = torch.from_numpy(bits.copy()).to("cuda")
    scale = A.default_scale(192)
    got, gf = run_mla(pair, 1, q, bt, lens, 0, scale, int(lens.max()))
    exp, ef, bound = oracle_mla(pair, 1, q, bt, lens, 0, scale, int(lens.max()))
    assert gf == ef == frozenset()
    check_close(got, exp, bound, where)
    assert np.isfinite(got).all()
    if where != "moderate":  # one position takes (nearly) all the weight
        assert np.abs(got - exp).max() < 1e-5
