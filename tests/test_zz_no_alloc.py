"""The allocation-free decode attention (ukv_decode_attention_noalloc) against the
workspace entry point it mirrors: the same kernels, so the outputs must be equal bit for
bit, on two calls in a row on one GPU, the second with a smaller batch (the fixed
scratch keeps the first call's partials, which the second must not read)."""
import numpy as np
import pytest
import torch

import store_gather_amd as U
import ukv_workloads as W
from oracle import attention as A
from parity_util import log, to_dev
from test_gpu_attention import GaussPair, requests

pytestmark = pytest.mark.gpu


def test_noalloc_decode_attention_matches_the_workspace_entry_point():
    ps, hkv, group, d = 16, 8, 4, 128
    P = 2500
    pair = GaussPair([W.mha(2, hkv, d, P)], ps, seed=61, host=False)
    g = np.random.default_rng(61)
    for call, (num_reqs, len_hi, window, layer) in enumerate([(256, 8192, 0, 1), (40, 3000, 500, 0)]):
        log(f"\n[gpu] no-alloc call {call}: {num_reqs} requests up to {len_hi}, window {window}")
        lens = g.integers(0, len_hi, size=num_reqs, endpoint=True).astype(np.int32)
        lens[0] = len_hi
        pages = requests(call + 3, P, ps, lens, share=True)
        bt, _ = pair.orc.translate_pages(0, W.padded_table(pages))
        hq = hkv * group
        q = W.irwin_hall_bf16_host(call + 70, 0, 2 * num_reqs * hq * d).reshape(num_reqs, hq, d)
        qd = torch.from_numpy(q.view(np.int16)).to("cuda").view(torch.bfloat16)
        btd, lend = to_dev(bt), to_dev(lens)
        need = U.ukv_decode_attention_workspace_bytes(pair.gpu, 0, num_reqs, hq, len_hi, window)
        assert 0 < need <= 64 << 20
        ref = U.ukv_decode_attention(pair.gpu, 0, layer, qd, btd, lend, len_hi, window, A.default_scale(d))
        out = torch.full_like(ref, float("nan"))
        U.ukv_decode_attention_noalloc(pair.gpu, 0, layer, qd, btd, lend, len_hi, window, A.default_scale(d), out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {call}: outputs differ"
        assert torch.isfinite(out).all()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


def test_noalloc_decode_attention_rejects_a_batch_past_the_scratch():
    pair = GaussPair([W.mha(1, 8, 128, 64)], 16, seed=62, host=False)
    num_reqs, hq, max_len = 4096, 32, 16384
    assert U.ukv_decode_attention_workspace_bytes(pair.gpu, 0, num_reqs, hq, max_len, 0) > 64 << 20
    q = torch.zeros((num_reqs, hq, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((num_reqs, 1), dtype=torch.int32, device="cuda")
    lens = torch.zeros(num_reqs, dtype=torch.int32, device="cuda")
    out = torch.zeros((num_reqs, hq, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(U.UkvError, match="fixed scratch"):
        U.ukv_decode_attention_noalloc(pair.gpu, 0, 0, q, bt, lens, max_len, 0, 0.1, out=out)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
