"""GPU parity of the read path: the prefix-only page-table build (integer work,
bit-exact) and the decode attention over the dense views (floating point,
within the fp32 error bound the oracle derives per request and head, and
bit-exact where the arithmetic is exact: one position per request).

The pool holds Irwin-Hall bf16 values generated bit-identically on the device
and on the host (ukv_workloads.irwin_hall_*), so the oracle reads the same
bytes without copying anything back from the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import store_gather_amd as U
import ukv_workloads as W
from oracle import attention as A
from parity_util import log, ospecs, round8, to_dev

pytestmark = pytest.mark.gpu

# The fp32 bound takes the longest sum chain that any split of a request's positions
# can form, from the request's length alone: it holds however the kernel divides the
# work, and retuning that split changes no test.  Where a long request's bound is too
# loose to see a lost or doubled piece of the split, the exact zero-query tests below
# (every fp32 partial sum exact) see it.
BOUND_TERMS = A.chain_terms_any_split


@pytest.fixture(autouse=True)
def _name(request):
    log(f"\n[gpu] {request.node.name}")
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


class GaussPair:
    """A GPU pool and an oracle pool over identical bf16 bytes: Irwin-Hall values, or
    small integers (``ints=True``: float32 sums of them are exact)."""

    def __init__(self, shapes, ps, seed=21, host=True, ints=False):
        self.shapes = list(shapes)
        self.ps = ps
        self.seed = seed
        plan = U.ukv_pool_plan(self.shapes, ps)
        n = round8(int(plan.required_bytes))
        self.gpu = U.allocate_pool(self.shapes, ps, device="cuda", extra_bytes=n - int(plan.required_bytes))
        self.host = host
        self.set_values(ints)

    def set_values(self, ints):
        """(Re)fill both sides from one stream: the device pool on the device, the
        oracle's in host memory (or, for an addresses-only oracle, on demand)."""
        seed, n = self.seed, self.gpu.raw.numel()
        if ints:
            W.small_int_fill_device(self.gpu.raw, seed)
            gen = W.small_int_bf16_host
            self.read_words = lambda idx: W.small_int_bf16_words(seed, idx)
        else:
            W.irwin_hall_fill_device(self.gpu.raw, seed)
            gen = W.irwin_hall_bf16_host
            self.read_words = None
        if self.host:
            self.orc = oracle.OraclePool(ospecs(self.shapes), self.ps, gen(seed, 0, n).view(np.uint8).copy())
            self.read = None
        else:
            self.orc = oracle.OraclePool(ospecs(self.shapes), self.ps, addresses_only=True)
            self.read = lambda off, nbytes: gen(seed, off, nbytes)


def requests(seed, P, ps, lens, share=False):
    """Per-request physical pages from a permutation of pages 1..P-1 (cyclic when shared)."""
    perm = W.page_permutation(seed, P)
    perm = perm[perm != 0]
    out, at = [], 0
    for n in lens:
        k = (int(n) + ps - 1) // ps
        if not share:
            assert at + k <= perm.size
        out.append(perm[(at + np.arange(k)) % perm.size])
        at += k
    return out


def run_attention(pair, layer, q_bits, bt, lens, window, scale, max_len, sub=0):
    q = torch.from_numpy(q_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    out = U.ukv_decode_attention(pair.gpu, sub, layer, q, to_dev(bt), to_dev(lens), max_len, window, scale)
    return out.cpu().numpy().astype(np.float64), U.ukv_pool_error_flags(pair.gpu)


def check_close(got, exp, bound, what):
    err = np.abs(got - exp)
    worst = float(err.max()) if err.size else 0.0
    log(f"  {what}: max |err| {worst:.3e}, min bound {float(bound[bound > 0].min()) if (bound > 0).any() else 0:.3e}")
    assert (err <= bound[:, :, None]).all(), f"{what}: error {worst} above the fp32 bound"


# ---------------------------------------------------------------------------
# prefix-only page table
# ---------------------------------------------------------------------------

def test_build_page_table_parity():
    ps, P = 16, 300
    pair = GaussPair([W.mha(4, 2, 64, P)], ps)
    g = np.random.default_rng(3)
    lens = g.integers(0, 40 * ps, size=77).astype(np.int32)
    lens[:4] = [0, 1, ps, ps + 1]
    width = 45
    req = g.integers(-2, P + 5, size=(lens.size, width)).astype(np.int32)  # past-the-prefix entries: garbage
    out = U.ukv_build_page_table(pair.gpu, 0, to_dev(req), to_dev(lens))
    exp, ef = pair.orc.build_page_table(0, req, lens)
    assert np.array_equal(out.cpu().numpy(), exp)
    assert U.ukv_pool_error_flags(pair.gpu) == ef == {"slot_range"}
    # in range, through a v2p table, in place
    req = g.integers(0, P, size=(lens.size, width)).astype(np.int32)
    v2p = g.permutation(P).astype(np.int32)
    v2p[g.choice(P, 20, replace=False)] = -1
    d = to_dev(req)
    U.ukv_build_page_table(pair.gpu, 0, d, to_dev(lens), out=d, v2p=to_dev(v2p))
    exp, ef = pair.orc.build_page_table(0, req, lens, v2p)
    assert np.array_equal(d.cpu().numpy(), exp) and ef == frozenset()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    # a prefix wider than the table
    lens2 = lens.copy()
    lens2[5] = width * ps + 1
    out = U.ukv_build_page_table(pair.gpu, 0, to_dev(req), to_dev(lens2))
    exp, ef = pair.orc.build_page_table(0, req, lens2)
    assert np.array_equal(out.cpu().numpy(), exp)
    assert U.ukv_pool_error_flags(pair.gpu) == ef == {"layout"}
    # empty batch: nothing launched
    U.ukv_build_page_table(pair.gpu, 0, to_dev(np.zeros((0, 3), np.int32)), to_dev(np.zeros(0, np.int32)))
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------

LENS = [1, 2, 15, 16, 17, 63, 255, 256, 257, 511, 600, 0, 1000, 33]


@pytest.mark.parametrize("hkv,group,d,ps", [(2, 4, 128, 16), (8, 4, 128, 16), (2, 1, 64, 4), (1, 8, 256, 16),
                                            (3, 2, 128, 1), (2, 8, 64, 32)])
@pytest.mark.parametrize("window", [0, 100])
def test_decode_attention_parity(hkv, group, d, ps, window):
    lens = np.array(LENS, dtype=np.int32)
    need = int(sum((int(n) + ps - 1) // ps for n in lens))
    P = need + 8
    pair = GaussPair([W.mha(3, hkv, d, P)], ps, seed=hkv * 100 + d)
    pages = requests(2, P, ps, lens)
    req = W.padded_table(pages)
    bt, ef = pair.orc.build_page_table(0, req, lens)
    assert ef == frozenset()
    assert np.array_equal(U.ukv_build_page_table(pair.gpu, 0, to_dev(req), to_dev(lens)).cpu().numpy(), bt)
    hq = hkv * group
    q = W.irwin_hall_bf16_host(99, 0, 2 * lens.size * hq * d).reshape(lens.size, hq, d)
    scale = A.default_scale(d)
    max_len = int(lens.max())
    for layer in (0, 2):
        got, gf = run_attention(pair, layer, q, bt, lens, window, scale, max_len)
        exp, ef, bound = A.decode_attention(pair.orc, 0, layer, q, bt, lens, window, scale, max_len,
                                            bound_terms=BOUND_TERMS)
        assert gf == ef == frozenset()
        check_close(got, exp, bound, f"layer {layer}")
        assert np.array_equal(got[lens == 0], np.zeros_like(got[lens == 0]))


@pytest.mark.parametrize("num_reqs,len_hi,window", [(128, 3000, 0), (64, 3000, 0), (256, 2100, 0), (256, 4000, 700),
                                                    (32, 9000, 0)])
def test_decode_attention_parity_unit_sizes(num_reqs, len_hi, window):
    """Batches whose size makes the kernel pick 768-, 384-, 1024-, 512- and 512-position units."""
    ps, hkv, group, d = 16, 8, 4, 128
    g = np.random.default_rng(num_reqs + len_hi)
    lens = g.integers(1, len_hi, size=num_reqs, endpoint=True).astype(np.int32)
    lens[0] = len_hi
    P = 2500
    pair = GaussPair([W.mha(1, hkv, d, P)], ps, seed=num_reqs)
    pages = requests(4, P, ps, lens, share=True)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    q = W.irwin_hall_bf16_host(8, 0, 2 * num_reqs * hkv * group * d).reshape(num_reqs, hkv * group, d)
    scale = A.default_scale(d)
    got, gf = run_attention(pair, 0, q, bt, lens, window, scale, len_hi)
    exp, ef, bound = A.decode_attention(pair.orc, 0, 0, q, bt, lens, window, scale, len_hi,
                                        bound_terms=BOUND_TERMS)
    assert gf == ef == frozenset()
    check_close(got, exp, bound, f"{num_reqs} requests up to {len_hi}")


def check_exact_mean(got, exp, what):
    """Zero-query outputs against the exact mean of the attended values (oracle/attention.py:
    exact_mean_tolerance): every weight is 1 and every float32 partial sum of small
    integers is exact, so only the final division rounds."""
    tol = A.exact_mean_tolerance(exp)
    off = np.abs(got - exp) > tol
    log(f"  {what}: max |err| {float(np.abs(got - exp).max()):.3e}, elements off the exact mean: {int(off.sum())}")
    assert not off.any(), f"{what}: {int(off.sum())} elements off the exact mean, first at {np.argwhere(off)[0]}"


@pytest.mark.parametrize("num_reqs,len_hi,window", [(128, 3000, 0), (64, 3000, 0), (256, 2100, 0), (256, 4000, 700),
                                                    (32, 9000, 0), (256, 8192, 0), (1, 60000, 0), (3, 60000, 5000)])
def test_decode_attention_unit_merge_exact(num_reqs, len_hi, window):
    """Zero queries over small-integer values: the output is the mean of the attended V
    rows up to one division, whatever the kernel's split into units, so a unit lost,
    counted twice or merged into the wrong request shows at any length (on the CPU the
    same tolerance rejects a dropped 16-position tile of an 8,192-position request).
    Every request is checked: the batch shapes that pick each unit size, the decode
    batch's shape, and 60,000-position requests."""
    ps, hkv, group, d = 16, 8, 4, 128
    g = np.random.default_rng(num_reqs + len_hi + 1)
    lens = g.integers(1, len_hi, size=num_reqs, endpoint=True).astype(np.int32)
    lens[0] = len_hi
    P = 2500
    pair = GaussPair([W.mha(1, hkv, d, P)], ps, seed=num_reqs + 7, ints=True)
    pages = requests(4, P, ps, lens, share=True)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    q = np.zeros((num_reqs, hkv * group, d), np.uint16)
    got, gf = run_attention(pair, 0, q, bt, lens, window, 0.5, len_hi)
    exp, ef = A.decode_attention(pair.orc, 0, 0, q, bt, lens, window, 0.5, len_hi, uniform=True)
    assert gf == ef == frozenset()
    check_exact_mean(got, exp, f"{num_reqs} requests up to {len_hi}")


@pytest.mark.parametrize("hkv,group,d", [(2, 4, 128), (1, 2, 64), (2, 8, 256)])
def test_decode_attention_single_position_is_exact(hkv, group, d):
    """window = 1 keeps only the last position: the output is that V row, exactly, for any length."""
    ps = 16
    lens = np.array([1, 16, 17, 256, 257, 700, 1023], dtype=np.int32)
    P = int(sum((int(n) + ps - 1) // ps for n in lens)) + 2
    pair = GaussPair([W.mha(2, hkv, d, P)], ps, seed=5)
    pages = requests(7, P, ps, lens)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    hq = hkv * group
    q = W.irwin_hall_bf16_host(4, 0, 2 * lens.size * hq * d).reshape(lens.size, hq, d)
    got, gf = run_attention(pair, 1, q, bt, lens, 1, 0.7, int(lens.max()))
    exp, ef = A.decode_attention(pair.orc, 0, 1, q, bt, lens, 1, 0.7)
    assert gf == ef == frozenset()
    assert np.array_equal(got, exp)


def test_decode_attention_conditions():
    ps, hkv, group, d = 16, 2, 4, 128
    lens = np.array([40, 300, 40, 0, 90, 600], dtype=np.int32)
    P = 80
    pair = GaussPair([W.mha(1, hkv, d, P)], ps, seed=8)
    pages = requests(3, P, ps, lens)
    bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
    q = W.irwin_hall_bf16_host(1, 0, 2 * lens.size * hkv * group * d).reshape(lens.size, hkv * group, d)
    scale = A.default_scale(d)
    good, gf = run_attention(pair, 0, q, bt, lens, 0, scale, 600)
    assert gf == frozenset()
    bpp = pair.orc.plan.subs[0].blocks_per_page
    for bad in (-1, 1, P * bpp, int(bt[1, 0]) + bpp // 2):
        b = bt.copy()
        b[1, 17] = bad  # inside request 1's second chunk
        got, gf = run_attention(pair, 0, q, b, lens, 0, scale, 600)
        exp, ef = A.decode_attention(pair.orc, 0, 0, q, b, lens, 0, scale, 600)
        assert gf == ef == {"bad_block"}
        assert np.array_equal(got[1], np.zeros_like(got[1]))
        assert np.array_equal(np.delete(got, 1, 0), np.delete(good, 1, 0))
    # the same bad entry outside a window is never read
    b = bt.copy()
    b[5, 2] = -1
    got, gf = run_attention(pair, 0, q, b, lens, 128, scale, 600)
    assert gf == frozenset()
    # table narrower than a request, and a request past max_seq_len
    got, gf = run_attention(pair, 0, q, np.ascontiguousarray(bt[:, :10]), lens, 0, scale, 600)
    exp, ef = A.decode_attention(pair.orc, 0, 0, q, bt[:, :10], lens, 0, scale, 600)
    assert gf == ef == {"bad_block"}
    assert np.array_equal(got[[1, 5]], np.zeros_like(got[[1, 5]]))
    assert np.array_equal(got[[0, 2, 3, 4]], good[[0, 2, 3, 4]])
    got, gf = run_attention(pair, 0, q, bt, lens, 0, scale, 300)
    exp, ef = A.decode_attention(pair.orc, 0, 0, q, bt, lens, 0, scale, 300)
    assert gf == ef == {"layout"}
    assert np.array_equal(got[5], np.zeros_like(got[5])) and np.array_equal(got[:5], good[:5])
    # max_seq_len 0: every non-empty request is past the bound, no chunk kernel runs
    got, gf = run_attention(pair, 0, q, bt, lens, 0, scale, 0)
    assert gf == {"layout"} and not got.any()


def test_decode_attention_host_errors():
    pair = GaussPair([W.mha(2, 2, 128, 8), W.mla(2, 8)], 16, seed=1, host=False)
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(U.UkvError, match="not MHA"):
        U.ukv_decode_attention(pair.gpu, 1, 0, q, bt, lens, 16, 0, 0.1)
    with pytest.raises(U.UkvError, match="layer"):
        U.ukv_decode_attention(pair.gpu, 0, 2, q, bt, lens, 16, 0, 0.1)
    with pytest.raises(U.UkvError, match="multiple of head_num"):
        U.ukv_decode_attention(pair.gpu, 0, 0, q[:, :3].contiguous(), bt, lens, 16, 0, 0.1)
    with pytest.raises(U.UkvError, match="supported"):
        U.ukv_decode_attention(pair.gpu, 0, 0, torch.zeros((2, 6, 128), dtype=torch.bfloat16, device="cuda"), bt,
                               lens, 16, 0, 0.1)
    with pytest.raises(U.UkvError, match="workspace"):
        U.ukv_decode_attention(pair.gpu, 0, 0, q, bt, lens, 16, 0, 0.1,
                               workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(U.UkvError, match="not finite"):
        U.ukv_decode_attention(pair.gpu, 0, 0, q, bt, lens, 16, 0, float("inf"))
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


def test_decode_attention_full_decode_8b_sampled():
    """Llama-3-8B-shape decode batch at full size (8 GiB pool, 256 requests of 1-8 K
    positions, 32 query heads on 8 KV heads), every request's output checked for
    six sampled requests on two layers; all layers run."""
    w = W.decode_8b()
    ps = w.page_size
    lens = w.req_lens[0]
    pair = GaussPair(w.shapes, ps, seed=31, host=False)
    req = W.padded_table(w.req_pages[0])
    bt_dev = U.ukv_build_page_table(pair.gpu, 0, to_dev(req), to_dev(lens))
    bt, ef = pair.orc.build_page_table(0, req, lens)  # the oracle reads its own table
    assert np.array_equal(bt_dev.cpu().numpy(), bt) and ef == frozenset()
    R, hq, d = lens.size, 32, 128
    q = W.irwin_hall_bf16_host(77, 0, 2 * R * hq * d).reshape(R, hq, d)
    qd = torch.from_numpy(q.view(np.int16)).to("cuda").view(torch.bfloat16)
    scale = A.default_scale(d)
    max_len = int(lens.max())
    ws = torch.empty(U.ukv_decode_attention_workspace_bytes(pair.gpu, 0, R, hq, max_len, 0), dtype=torch.uint8, device="cuda")
    sample = sorted({0, R - 1, int(np.argmax(lens)), int(np.argmin(lens)), 101, 177})
    for layer in range(32):
        out = U.ukv_decode_attention(pair.gpu, 0, layer, qd, bt_dev, to_dev(lens), max_len, 0, scale, workspace=ws)
        if layer in (0, 31):
            got = out.cpu().numpy().astype(np.float64)
            exp, ef, bound = A.decode_attention(pair.orc, 0, layer, q, bt, lens, 0, scale, max_len, read=pair.read,
                                                requests=sample, bound_terms=BOUND_TERMS)
            assert ef == frozenset()
            check_close(got[sample], exp[sample], bound[sample], f"layer {layer}")
            assert np.isfinite(got).all()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    # the same batch on small-integer values with zero queries: every request exact
    pair.set_values(ints=True)
    q0 = np.zeros_like(q)
    out = U.ukv_decode_attention(pair.gpu, 0, 5, torch.zeros_like(qd), bt_dev, to_dev(lens), max_len, 0, scale,
                                 workspace=ws)
    exp, ef = A.decode_attention(pair.orc, 0, 5, q0, bt, lens, 0, scale, max_len, read_words=pair.read_words,
                                 uniform=True)
    assert ef == frozenset()
    check_exact_mean(out.cpu().numpy().astype(np.float64), exp, "layer 5, every request")
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
