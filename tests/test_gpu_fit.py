"""GPU parity of the test-time predictor fit (lowram_fit_predictor) against the
CPU oracle.

The starting weights are the generator's predictor perturbed by seeded noise
and stored in act dtype (a stand-in for a meta-learned starting point), so
the descent has work to do.  The GPU runs float32 gradients and master
weights, the oracle float64; both round once at the end.  Bar: the losses
agree to 1e-4 relative, and the fitted weights are within one unit in the
last place of the act dtype, with such differences rare.
"""
import numpy as np
import pytest
import torch

from oracle import lowram_oracle as O
from synth import gen
from synth.configs import BF16, COMPOSED_128K, LLAMA8B_32K, QWEN4B_64K, TINY, small
from tests.harness import bf16_ulp_diff, cache_to_host, dims_of, model_of, to_dev, to_host, upload

pytestmark = pytest.mark.gpu

NAMES = ("w1", "b1", "w2", "b2")
CASES = {
    "tiny-fp32": (TINY, 4, 0.05),
    "llama8b-small": (small(LLAMA8B_32K, N=1024), 4, 0.01),
    "qwen4b-small": (small(QWEN4B_64K, N=1024), 3, 0.005),
    "composed-small": (small(COMPOSED_128K, N=1024, evict_keep=1.0), 3, 0.01),
}


def P():
    import decode_attention_compressed_amd as pkg
    return pkg


def perturbed_init(inp, s, scale=0.3, seed=7):
    """The generator's predictor plus scale * N(0, std of each tensor), stored."""
    rng = np.random.default_rng(seed)
    init = {}
    for n in NAMES:
        w = O.decode(inp[n], s.act)
        std = float(np.std(w)) or 1.0
        init[n] = O.round_to(w + scale * std * rng.standard_normal(w.shape), s.act)
    return init


def assert_weights_close(got, want, init, act, what):
    """GPU and oracle round the same descent, float32 against float64: before
    rounding they differ by a small fraction of the accumulated update, after
    it by at most one unit in the last place more.  In bf16, elements that
    differ at all must be rare."""
    g = O.decode(got, act)
    w = O.decode(want, act)
    w0 = O.decode(init, act)
    if act == BF16:
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(w), 1e-30))) - 7)
    else:
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(w), 1e-30))) - 23)
    allowed = ulp + 1e-3 * np.abs(w - w0) + 1e-7 * np.max(np.abs(w))
    err = np.abs(g - w)
    assert np.all(err <= allowed), (what, float(np.max(err / allowed)))
    if act == BF16:  # float32 results differ in the last bits almost everywhere
        assert np.mean(g != w) < 2e-3, (what, float(np.mean(g != w)))


@pytest.fixture(scope="module", params=list(CASES))
def fitted(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s, steps, lr = CASES[request.param]
    print(f"\n[fit case] {request.param}: steps {steps} lr {lr} {s}", flush=True)
    inp = gen.make(s)
    init = perturbed_init(inp, s)
    dev = upload(inp)
    model = dict(model_of(dev))
    for n in NAMES:
        model[n] = to_dev(init[n], s.act)
    d = dims_of(s)
    out, loss = P().fit_predictor(d, model, dev["k"], dev["v"], steps, lr)
    torch.cuda.synchronize()
    return dict(name=request.param, s=s, steps=steps, lr=lr, inp=inp, init=init, dev=dev, model=model,
                d=d, out=out, loss=to_host(loss), host={n: to_host(out[n]) for n in NAMES})


def test_fit_matches_oracle(fitted):
    s, inp = fitted["s"], fitted["inp"]
    ref = O.fit_predictor(inp, s, fitted["steps"], fitted["lr"], init=fitted["init"])
    assert np.allclose(fitted["loss"], ref["loss"], rtol=1e-4, atol=0), \
        np.max(np.abs(fitted["loss"] - ref["loss"]) / ref["loss"])
    assert np.all(ref["loss"][..., -1] < ref["loss"][..., 0])  # the descent did something
    for n in NAMES:
        assert_weights_close(fitted["host"][n], ref[n], fitted["init"][n], s.act, n)


def test_fit_is_deterministic_and_in_place_equal(fitted):
    s, d, dev = fitted["s"], fitted["d"], fitted["dev"]
    model = {k: (v.clone() if k in NAMES else v) for k, v in fitted["model"].items()}
    out2, loss2 = P().fit_predictor(d, model, dev["k"], dev["v"], fitted["steps"], fitted["lr"], out=model)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(model[n], fitted["out"][n]), n
    assert np.array_equal(to_host(loss2), fitted["loss"])


def test_fit_zero_steps_keeps_weights(fitted):
    s, d, dev = fitted["s"], fitted["d"], fitted["dev"]
    out, loss = P().fit_predictor(d, fitted["model"], dev["k"], dev["v"], 0, fitted["lr"])
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(out[n], fitted["model"][n]), n
    assert np.allclose(to_host(loss)[..., 0], fitted["loss"][..., 0], rtol=0, atol=0)


def test_compress_and_decode_with_fitted_predictor(fitted):
    """The fitted weights feed compress and decode; both stay at parity."""
    s, d, dev, inp = fitted["s"], fitted["d"], fitted["dev"], fitted["inp"]
    model = dict(fitted["model"])
    model.update(fitted["out"])
    cache = P().alloc_cache(d)
    P().compress(d, model, dev["k"], dev["v"], cache)
    torch.cuda.synchronize()
    host = cache_to_host(cache)
    inp2 = dict(inp)
    inp2.update(fitted["host"])
    ref = O.compress(inp2, s, stored={"coeff": host["coeff"], "coeff_scale": host.get("coeff_scale")})
    assert np.array_equal(host["res_idx"], ref["res_idx"])
    assert np.array_equal(host["landmark"], ref["landmark"])
    q = dev["q"][0, 0].contiguous()
    out = P().decode_attn(d, 0, model, cache, q, dev["k_tail"], dev["v_tail"])
    torch.cuda.synchronize()
    want, _ = O.decode_layer(host, inp2, s, 0, inp["q"][0, 0], s.k)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 2e-3 + 1e-2 * np.abs(want))
