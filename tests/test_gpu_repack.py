"""GPU parity of the tail re-pack (lowram_repack) against the CPU oracle.

Each case compresses a prefill on the GPU (and evicts first where the
workload composes eviction), then packs the oldest chunk of the tail into a
new chunk.  Stage isolation as for compress: the new coefficients are checked
against the oracle's own rounding (at most one unit in the last place, rarely),
and everything after them -- landmark, residual set, CSR, residual rows -- is
checked bit for bit against the oracle continuing from the GPU's stored
coefficients.  A decode step on the grown cache with the shortened tail is
then compared with the oracle's decode on the same cache.
"""
import math

import numpy as np
import pytest
import torch

from oracle import lowram_oracle as O
from synth import gen
from synth.configs import BF16, COMPOSED_128K, I8, LLAMA8B_32K, QWEN4B_64K, TINY, small
from tests.harness import (bf16_ulp_diff, cache_to_host, dims_of, f32_of, model_of, to_dev,
                           to_host, upload, within_tol)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-fp32": TINY.replace(T=80),
    "llama8b-small": small(LLAMA8B_32K, k=6, T=160),
    "qwen4b-small": small(QWEN4B_64K, k=3, T=300),
    "composed-small": small(COMPOSED_128K, k=3, T=140),
}


def P():
    import decode_attention_compressed_amd as pkg
    return pkg


def new_res_of(s) -> int:
    """Residual rows the new chunk keeps: the prefill's fraction rho of C."""
    return min(s.C, int(math.ceil(s.rho * s.C - 1e-9)))


@pytest.fixture(scope="module", params=list(CASES))
def grown(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = CASES[request.param]
    print(f"\n[repack case] {request.param}: {s}", flush=True)
    inp = gen.make(s)
    dev = upload(inp)
    d = dims_of(s)
    cache = P().alloc_cache(d)
    P().compress(d, model_of(dev), dev["k"], dev["v"], cache)
    if s.evict_keep < 1.0:
        cache, d, _ = P().evict(d, model_of(dev), cache, to_dev(inp["obs_q"]), s.keep_chunks)
    torch.cuda.synchronize()
    m = new_res_of(s)
    dst, d2 = P().repack(d, model_of(dev), cache, dev["k_tail"], dev["v_tail"], m)
    torch.cuda.synchronize()
    return dict(name=request.param, s=s, inp=inp, dev=dev, d=d, d2=d2, m=m, src=cache_to_host(cache),
                dst=dst, host=cache_to_host(dst))


def oracle_repack(g, stored=True):
    s, inp, d, C = g["s"], g["inp"], g["d"], g["s"].C
    kt, vt = inp["k_tail"][:, :, :, :C], inp["v_tail"][:, :, :, :C]
    sc = g["host"]["coeff"][:, d.n_ctx:] if stored else None
    return O.repack(g["src"], inp, kt, vt, s, g["m"], stored_coeff=sc)


def test_repack_coefficients_match_oracle_rounding(grown):
    s, host, N = grown["s"], grown["host"], grown["d"].n_ctx
    ref = oracle_repack(grown, stored=False)
    got, want = host["coeff"][:, N:], ref["coeff"][:, N:]
    if s.coeff == I8:
        diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
        assert diff.max() <= 1 and np.mean(diff > 0) < 1e-3
    elif s.coeff == BF16:
        ulp = bf16_ulp_diff(got, want)
        assert ulp.max() <= 1 and np.mean(ulp > 0) < 1e-3, (ulp.max(), np.mean(ulp > 0))
    else:
        g, o = got.astype(np.float64), want.astype(np.float64)
        assert np.max(np.abs(g - o) / np.maximum(np.abs(o), 1e-30)) <= 2 ** -23


def test_repack_stages_bit_exact(grown):
    s, host, src, d, m = grown["s"], grown["host"], grown["src"], grown["d"], grown["m"]
    N, n_c = d.n_ctx, d.n_ctx // s.C
    ref = oracle_repack(grown)
    assert np.array_equal(host["coeff"][:, :N], src["coeff"])
    assert np.array_equal(host["landmark"], ref["landmark"])
    assert np.array_equal(host["res_ptr"], ref["res_ptr"])
    for name in ("coeff_scale", "res_scale"):
        if src.get(name) is not None:
            assert np.array_equal(host[name].view(np.uint16), src[name].view(np.uint16))
    for i in np.ndindex(host["res_ptr"].shape[:3]):
        live = int(src["res_ptr"][i][n_c])
        n = int(host["res_ptr"][i][-1])
        assert n == live + m
        assert np.array_equal(host["res_idx"][i][:n], ref["res_idx"][i][:n])
        assert np.array_equal(host["res_val"][i][:live], src["res_val"][i][:live])
        assert not np.any(host["res_idx"][i][n:]) and not np.any(host["res_val"][i][n:])
        got, want = host["res_val"][i][live:n], ref["res_val"][i][live:n]
        if s.resid == I8:
            assert np.max(np.abs(got.astype(np.int32) - want.astype(np.int32)), initial=0) <= 1
        elif s.resid == BF16:
            assert bf16_ulp_diff(got, want).max(initial=0) <= 1
        else:
            assert np.allclose(got, want, rtol=2 ** -23, atol=0)


def test_repack_residual_rows_rarely_differ(grown):
    """Across the whole case, residual rows off by one unit are rare."""
    s, host, src, d = grown["s"], grown["host"], grown["src"], grown["d"]
    if s.resid not in (I8, BF16):
        pytest.skip("float32 rows are compared to 2^-23 above")
    ref = oracle_repack(grown)
    n_c = d.n_ctx // s.C
    off = tot = 0
    for i in np.ndindex(host["res_ptr"].shape[:3]):
        live, n = int(src["res_ptr"][i][n_c]), int(host["res_ptr"][i][-1])
        got, want = host["res_val"][i][live:n], ref["res_val"][i][live:n]
        diff = (np.abs(got.astype(np.int32) - want.astype(np.int32)) if s.resid == I8
                else bf16_ulp_diff(got, want))
        off += int(np.sum(diff > 0))
        tot += diff.size
    assert off <= max(1, tot // 1000), (off, tot)


def test_decode_after_repack_matches_oracle(grown):
    s, inp, dev, d2 = grown["s"], grown["inp"], grown["dev"], grown["d2"]
    C = s.C
    kt = dev["k_tail"][:, :, :, C:].contiguous()
    vt = dev["v_tail"][:, :, :, C:].contiguous()
    inp2 = dict(inp, k_tail=inp["k_tail"][:, :, :, C:], v_tail=inp["v_tail"][:, :, :, C:])
    n_c2 = d2.n_ctx // C
    for layer in range(s.G):
        for top_k in (min(s.k, n_c2), n_c2):
            d = P().with_(d2, top_k=top_k)
            q = dev["q"][1, layer].contiguous()
            sel = torch.full((s.B, s.Hkv, top_k), -1, dtype=torch.int32, device="cuda")
            out = P().decode_attn(d, layer, model_of(dev), grown["dst"], q, kt, vt, sel_out=sel)
            torch.cuda.synchronize()
            ref, rsel = O.decode_layer(grown["host"], inp2, s, layer, inp["q"][1, layer], top_k,
                                       N=d2.n_ctx)
            assert np.array_equal(to_host(sel), rsel), (layer, top_k)
            ok, worst = within_tol(f32_of(out), ref)
            assert ok, f"layer {layer} top_k {top_k}: worst |err|/tol {worst:.3f}"


def test_repack_twice_and_from_empty():
    """Two re-packs in a row, the first from an empty float cache (N = 0),
    against two oracle re-packs; then decode over all chunks on the result."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = TINY.replace(N=0, T=2 * TINY.C + 16, k=2)
    print(f"\n[repack case] empty-twice: {s}", flush=True)
    inp = gen.make(s)
    dev = upload(inp)
    d = dims_of(s, n_res=0)
    empty = P().alloc_cache(d)
    m = new_res_of(s)
    one, d1 = P().repack(d, model_of(dev), empty, dev["k_tail"], dev["v_tail"], m)
    kt1 = dev["k_tail"][:, :, :, s.C:].contiguous()
    vt1 = dev["v_tail"][:, :, :, s.C:].contiguous()
    two, d2 = P().repack(d1, model_of(dev), one, kt1, vt1, m + 3)
    torch.cuda.synchronize()
    h1, h2 = cache_to_host(one), cache_to_host(two)
    src0 = {k: v for k, v in cache_to_host(empty).items()}
    C = s.C
    r1 = O.repack(src0, inp, inp["k_tail"][:, :, :, :C], inp["v_tail"][:, :, :, :C], s, m,
                  stored_coeff=h1["coeff"][:, :C])
    r2 = O.repack(h1, inp, inp["k_tail"][:, :, :, C:2 * C], inp["v_tail"][:, :, :, C:2 * C], s, m + 3,
                  stored_coeff=h2["coeff"][:, C:2 * C])
    for h, r in ((h1, r1), (h2, r2)):
        assert np.array_equal(h["landmark"], r["landmark"])
        assert np.array_equal(h["res_ptr"], r["res_ptr"])
        assert np.array_equal(h["res_idx"], r["res_idx"])
        assert np.allclose(h["res_val"], r["res_val"], rtol=2 ** -23, atol=0)
    assert np.array_equal(h2["res_ptr"][..., -1], np.full(h2["res_ptr"].shape[:3], 2 * m + 3))
    kt2 = dev["k_tail"][:, :, :, 2 * C:].contiguous()
    vt2 = dev["v_tail"][:, :, :, 2 * C:].contiguous()
    inp2 = dict(inp, k_tail=inp["k_tail"][:, :, :, 2 * C:], v_tail=inp["v_tail"][:, :, :, 2 * C:])
    dd = P().with_(d2, top_k=2)
    for layer in range(s.G):
        out = P().decode_attn(dd, layer, model_of(dev), two, dev["q"][0, layer].contiguous(), kt2, vt2)
        torch.cuda.synchronize()
        ref, _ = O.decode_layer(h2, inp2, s, layer, inp["q"][0, layer], 2, N=2 * C)
        ok, worst = within_tol(f32_of(out), ref)
        assert ok, worst

