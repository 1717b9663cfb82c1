"""The allocation-free decode entry point (lowram_decode_attn_noalloc) against
lowram_decode_attn, called through the C ABI: two calls in a row on one GPU,
the second with a smaller input, must give the same selection and the same
output bits as the workspace-taking call (and so meet the oracle bar that
call meets); a request above the static scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import lowram_oracle as O
from synth import gen
from synth.configs import LLAMA8B_32K, MISTRAL7B_16K, small
from tests.harness import cache_to_host, dims_of, f32_of, model_of, to_host, upload, within_tol


def P():
    import decode_attention_compressed_amd as pkg
    return pkg


def test_noalloc_refuses_a_workspace_above_its_scratch():
    L = P()._lib
    big = dims_of(MISTRAL7B_16K.replace(B=1024))
    assert P().workspace_bytes(big, L.OP_DECODE) > L.NOALLOC_SCRATCH_BYTES
    FAKE = 1 << 20
    m = L.Model(FAKE, FAKE, FAKE, FAKE, FAKE)
    c = L.Cache(FAKE, None, FAKE, FAKE, FAKE, FAKE, None)
    st = L.lib().lowram_decode_attn_noalloc(ctypes.byref(big), 0, ctypes.byref(m), ctypes.byref(c), FAKE, FAKE,
                                             FAKE, FAKE, None, None)
    assert st == L.E_WORKSPACE
    assert "static scratch" in L.lib().lowram_last_error().decode()


def _noalloc(d, layer, model, cache, q, kt, vt, out, sel):
    L = P()._lib
    api = P().api
    qp, ktp, vtp = api._decode_common(d, q, kt, vt)
    st = L.lib().lowram_decode_attn_noalloc(
        ctypes.byref(d), layer, ctypes.byref(api.model_struct(d, model)), ctypes.byref(api.cache_struct(d, cache)),
        qp, ktp, vtp, api._ptr(out, api.TORCH_DT[d.act], tuple(q.shape), "out"),
        api._ptr(sel, torch.int32, (d.batch, d.heads_kv, P().k_eff(d)), "sel_out"), api._stream(None))
    L.check(st)


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    cases = [small(LLAMA8B_32K, B=2, N=4096, k=6, T=40), small(LLAMA8B_32K, B=1, N=1024, k=3, T=16)]
    sizes = []
    for i, s in enumerate(cases):
        print(f"\n[noalloc] call {i}: {s}", flush=True)
        inp = gen.make(s, steps=1)
        dev = upload(inp)
        d = dims_of(s)
        sizes.append(P().workspace_bytes(d, P()._lib.OP_DECODE))
        cache = P().alloc_cache(d)
        P().compress(d, model_of(dev), dev["k"], dev["v"], cache)
        layer = s.G - 1
        q = dev["q"][0, layer].contiguous()
        kk = P().k_eff(d)
        sel_a = torch.full((s.B, s.Hkv, kk), -1, dtype=torch.int32, device="cuda")
        sel_b = torch.full_like(sel_a, -2)
        out_a = P().decode_attn(d, layer, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], sel_out=sel_a)
        out_b = torch.full_like(out_a, float("nan"))
        _noalloc(d, layer, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], out_b, sel_b)
        torch.cuda.synchronize()
        assert torch.equal(sel_a, sel_b), i
        assert torch.equal(out_a, out_b), i
        ref, rsel = O.decode_layer(cache_to_host(cache), inp, s, layer, inp["q"][0, layer], s.k)
        assert np.array_equal(to_host(sel_b), rsel)
        ok, worst = within_tol(f32_of(out_b), ref)
        assert ok, f"call {i}: worst |err|/tol {worst:.3f}"
    assert sizes[1] < sizes[0] <= P()._lib.NOALLOC_SCRATCH_BYTES
