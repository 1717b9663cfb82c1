"""GPU parity at the workloads' full sizes, with the launch configuration the
benchmark times.  The oracle checks what it can compute one piece at a time:
every chunk selection (cheap in float64), the outputs of one layer call, the
residual sets of sampled (b, layer, head) triples from the stored
coefficients, and sampled coefficient rows."""
import numpy as np
import pytest
import torch

from oracle import lowram_oracle as O
from synth import gen
from synth.configs import COMPOSED_128K, I8, LLAMA8B_32K, MISTRAL7B_16K, QWEN4B_64K
from tests.harness import (bf16_ulp_diff, cache_to_host, dims_of, f32_of, model_of, to_dev, to_host,
                           upload, within_tol)

pytestmark = pytest.mark.gpu

FULL = {
    "llama8b-32k": LLAMA8B_32K,
    "qwen4b-64k": QWEN4B_64K,
    "composed-int8-evict-128k": COMPOSED_128K,
    "mistral7b-16k-b16": MISTRAL7B_16K,
}


def P():
    import decode_attention_compressed_amd as pkg
    return pkg


@pytest.fixture(scope="module", params=list(FULL))
def full(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = FULL[request.param]
    print(f"\n[full] {request.param}: generating {s}", flush=True)
    inp = gen.make(s, steps=1)
    dev = upload(inp)
    d = dims_of(s)
    cache = P().alloc_cache(d)
    P().compress(d, model_of(dev), dev["k"], dev["v"], cache)
    torch.cuda.synchronize()
    pre = cache_to_host(cache)
    keep = None
    if s.evict_keep < 1.0:
        cache, d, keep = P().evict(d, model_of(dev), cache, to_dev(inp["obs_q"]), s.keep_chunks)
        torch.cuda.synchronize()
        keep = to_host(keep)
    print(f"[full] {request.param}: compressed", flush=True)
    yield dict(s=s, inp=inp, dev=dev, d=d, cache=cache, pre=pre, host=cache_to_host(cache), keep=keep)
    del dev, cache
    torch.cuda.empty_cache()


def test_full_selection_and_outputs(full):
    s, inp, dev, d, cache, host = (full[k] for k in ("s", "inp", "dev", "d", "cache", "host"))
    U_all = O.decode(inp["basis"], s.act)
    for layer in range(s.G):
        q = dev["q"][0, layer].contiguous()
        sel = torch.empty((s.B, s.Hkv, P().k_eff(d)), dtype=torch.int32, device="cuda")
        out = P().decode_attn(d, layer, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], sel_out=sel)
        torch.cuda.synchronize()
        sel_h = to_host(sel)
        qn = O.decode(inp["q"][0, layer], s.act)
        for b in range(s.B):
            for h in range(s.Hkv):
                sc = O.chunk_scores(host["landmark"][b], U_all[b], qn[b], layer, h, s.Hq, s.Hkv, s.dh)
                assert np.array_equal(sel_h[b, h], O.select_chunks(sc, s.k)), (layer, b, h)
        if layer in (0, s.G - 1):
            ref, rsel = O.decode_layer(host, inp, s, layer, inp["q"][0, layer], s.k, N=d.n_ctx)
            assert np.array_equal(rsel, sel_h)
            ok, worst = within_tol(f32_of(out), ref)
            assert ok, f"layer {layer}: worst |err|/tol {worst:.3f}"


def test_full_eviction_matches_oracle(full):
    """The composed workload's eviction at full size (1024 -> 256 chunks per
    sequence): kept chunks, coefficients, landmarks, CSR pointers and every
    live residual row against the oracle's eviction of the same stored cache."""
    s, inp, pre, host, d = (full[k] for k in ("s", "inp", "pre", "host", "d"))
    if s.evict_keep >= 1.0:
        pytest.skip("no eviction in this workload")
    ref = O.evict(pre, inp, s, inp["obs_q"], s.keep_chunks)
    assert np.array_equal(full["keep"], ref["keep"])
    assert np.array_equal(host["coeff"], ref["coeff"])
    assert np.array_equal(host["landmark"], ref["landmark"])
    assert np.array_equal(host["res_ptr"], ref["res_ptr"])
    live = ref["res_ptr"][..., -1]
    assert d.n_res == live.max()  # the evicted cache is sized to the largest head's rows
    for i in np.ndindex(live.shape):
        n = live[i]
        assert np.array_equal(host["res_idx"][i][:n], ref["res_idx"][i][:n]), i
        assert np.array_equal(host["res_val"][i][:n], ref["res_val"][i][:n]), i


def test_full_residual_sets_sampled(full):
    s, inp, pre = full["s"], full["inp"], full["pre"]
    rng = np.random.default_rng(7)
    for _ in range(2):
        b, l, h = int(rng.integers(s.B)), int(rng.integers(s.G)), int(rng.integers(s.Hkv))
        cdeq = O.coeff_deq(pre, b, s.coeff)
        U = O.decode(inp["basis"][b], s.act)
        khat = cdeq @ O.basis_slice(U, l, h, s.Hkv, s.dh).T
        w = [O.decode(inp[n][b, l, h], s.act) for n in ("w1", "b1", "w2", "b2")]
        vhat = O.predict(khat, *w)
        e = O.l2_errors(O.decode(inp["v"][b, l, h], s.act), vhat)
        R = O.topk_indices(e, s.n_res)
        assert np.array_equal(pre["res_idx"][b, l, h], R), (b, l, h)
        assert np.array_equal(pre["res_ptr"][b, l, h], O.csr_pointers(R, s.C, s.n_c))
        delta = O.decode(inp["v"][b, l, h], s.act)[R] - vhat[R]
        if s.resid == I8:
            q, sc = O.quantise(delta, axis=0)
            assert np.array_equal(pre["res_scale"][b, l, h].view(np.uint16), sc.view(np.uint16))
            assert np.max(np.abs(pre["res_val"][b, l, h].astype(int) - q.astype(int))) <= 1
        else:
            assert bf16_ulp_diff(pre["res_val"][b, l, h], O.round_to(delta, s.resid)).max() <= 1


def test_full_coefficients_sampled(full):
    s, inp, pre = full["s"], full["inp"], full["pre"]
    rng = np.random.default_rng(11)
    b = s.B - 1
    toks = np.sort(rng.choice(s.N, size=256, replace=False))
    k = O.decode(inp["k"][b][:, :, toks], s.act)             # [G][Hkv][256][dh]
    kcat = k.transpose(2, 0, 1, 3).reshape(len(toks), -1)
    c = O.project(kcat, O.decode(inp["basis"][b], s.act))
    if s.coeff == I8:
        q = np.clip(np.rint(c / pre["coeff_scale"][b].astype(np.float64)), -127, 127)
        assert np.max(np.abs(pre["coeff"][b][toks].astype(int) - q.astype(int))) <= 1
    else:
        assert bf16_ulp_diff(pre["coeff"][b][toks], O.round_to(c, s.coeff)).max() <= 1
    j = int(rng.integers(s.n_c))
    assert np.array_equal(pre["landmark"][b][j], O.landmarks(O.coeff_deq(pre, b, s.coeff)[j * s.C:(j + 1) * s.C], s.C)[0])
