"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Sizes: every workload shape with a reduced batch and context so that the
oracle finishes in seconds, while each case still spans several 128-token
tiles, several chunks per split and ragged tails.  Stage isolation: the oracle
continues from the bits the GPU stored (coefficients, then the whole cache),
so selections must be bit-exact; float outputs must satisfy
|gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise.
"""
import numpy as np
import pytest
import torch

from oracle import lowram_oracle as O
from synth import gen
from synth.configs import (BF16, COMPOSED_128K, F32, I8, LLAMA8B_32K, MISTRAL7B_16K, QWEN4B_64K,
                           TINY, small)
from tests.harness import (bf16_ulp_diff, cache_to_host, dims_of, f32_of, model_of, to_dev,
                           to_host, upload, within_tol)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-fp32": TINY,
    "llama8b-small": small(LLAMA8B_32K, k=6, T=100),
    "mistral7b-small": small(MISTRAL7B_16K, k=5, T=64),
    "qwen4b-small": small(QWEN4B_64K, k=3, T=200),
    "composed-small": small(COMPOSED_128K, k=3, T=72),
}


def P():
    import decode_attention_compressed_amd as pkg
    return pkg


def sync():
    torch.cuda.synchronize()


@pytest.fixture(scope="module", params=list(CASES))
def run(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = CASES[request.param]
    print(f"\n[case] {request.param}: {s}", flush=True)
    inp = gen.make(s)
    dev = upload(inp)
    d = dims_of(s)
    cache = P().alloc_cache(d)
    P().compress(d, model_of(dev), dev["k"], dev["v"], cache)
    sync()
    return dict(name=request.param, s=s, inp=inp, dev=dev, d=d, cache=cache, host=cache_to_host(cache))


def test_coefficients_match_oracle_rounding(run):
    s, inp, host = run["s"], run["inp"], run["host"]
    ref = O.compress(inp, s)
    if s.coeff == I8:
        assert np.array_equal(host["coeff_scale"].view(np.uint16), ref["coeff_scale"].view(np.uint16))
        diff = np.abs(host["coeff"].astype(np.int32) - ref["coeff"].astype(np.int32))
        assert diff.max() <= 1 and np.mean(diff > 0) < 1e-4
    elif s.coeff == BF16:
        ulp = bf16_ulp_diff(host["coeff"], ref["coeff"])
        assert ulp.max() <= 1 and np.mean(ulp > 0) < 1e-4, (ulp.max(), np.mean(ulp > 0))
    else:
        g, o = host["coeff"].astype(np.float64), ref["coeff"].astype(np.float64)
        assert np.max(np.abs(g - o) / np.maximum(np.abs(o), 1e-30)) <= 2 ** -23


def test_compress_stages_bit_exact(run):
    """Landmarks, residual sets, CSR pointers and residual rows from the GPU's
    stored coefficients."""
    s, inp, host = run["s"], run["inp"], run["host"]
    ref = O.compress(inp, s, stored={"coeff": host["coeff"], "coeff_scale": host.get("coeff_scale")})
    assert np.array_equal(host["landmark"], ref["landmark"])
    assert np.array_equal(host["res_idx"], ref["res_idx"])
    assert np.array_equal(host["res_ptr"], ref["res_ptr"])
    if s.resid == I8:
        assert np.array_equal(host["res_scale"].view(np.uint16), ref["res_scale"].view(np.uint16))
        diff = np.abs(host["res_val"].astype(np.int32) - ref["res_val"].astype(np.int32))
        assert diff.max() <= 1 and np.mean(diff > 0) < 1e-4
    elif s.resid == BF16:
        ulp = bf16_ulp_diff(host["res_val"], ref["res_val"])
        assert ulp.max() <= 1 and np.mean(ulp > 0) < 1e-4
    else:
        assert np.allclose(host["res_val"], ref["res_val"], rtol=2 ** -23, atol=0)


def test_residual_sets_end_to_end(run):
    """Oracle from raw K/V with its own rounding: the residual sets agree."""
    s, inp, host = run["s"], run["inp"], run["host"]
    ref = O.compress(inp, s)
    inter = sum(len(np.intersect1d(host["res_idx"][i], ref["res_idx"][i]))
                for i in np.ndindex(host["res_idx"].shape[:3]))
    total = host["res_idx"].size
    assert inter / max(total, 1) > 0.999


def evicted(run):
    """(dims, device cache, host cache, token count) the decode steps run on."""
    s, d = run["s"], run["d"]
    if s.evict_keep >= 1.0:
        return d, run["cache"], run["host"], s.N
    if "evicted" not in run:
        dev = run["dev"]
        obs = to_dev(run["inp"]["obs_q"])
        dst, d2, keep = P().evict(d, model_of(dev), run["cache"], obs, s.keep_chunks)
        sync()
        run["evicted"] = (d2, dst, cache_to_host(dst), to_host(keep))
    d2, dst, hdst, keep = run["evicted"]
    return d2, dst, hdst, d2.n_ctx


def test_eviction_matches_oracle(run):
    s = run["s"]
    if s.evict_keep >= 1.0:
        pytest.skip("no eviction in this workload")
    d2, dst, hdst, N2 = evicted(run)
    keep = run["evicted"][3]
    ref = O.evict(run["host"], run["inp"], s, run["inp"]["obs_q"], s.keep_chunks)
    assert np.array_equal(keep, ref["keep"])
    assert np.array_equal(hdst["coeff"], ref["coeff"])
    assert np.array_equal(hdst["landmark"], ref["landmark"])
    assert np.array_equal(hdst["res_ptr"], ref["res_ptr"])
    for i in np.ndindex(hdst["res_ptr"].shape[:3]):
        n = hdst["res_ptr"][i][-1]
        assert np.array_equal(hdst["res_idx"][i][:n], ref["res_idx"][i][:n])
        assert np.array_equal(hdst["res_val"][i][:n], ref["res_val"][i][:n])


def decode_both(run, step, layer, top_k=None, tail=True):
    s = run["s"]
    d, cache, hcache, N = evicted(run)
    if top_k is not None:
        d = P().with_(d, top_k=top_k)
    if not tail:
        d = P().with_(d, n_tail=0)
    dev = run["dev"]
    q = dev["q"][step, layer].contiguous()
    kk = P().k_eff(d)
    sel = torch.full((s.B, s.Hkv, kk), -1, dtype=torch.int32, device="cuda")
    kt = dev["k_tail"] if tail else None
    vt = dev["v_tail"] if tail else None
    out = P().decode_attn(d, layer, model_of(dev), cache, q, kt, vt, sel_out=sel)
    sync()
    inp = run["inp"] if tail else dict(run["inp"], k_tail=run["inp"]["k_tail"][:, :, :, :0],
                                        v_tail=run["inp"]["v_tail"][:, :, :, :0])
    ref, rsel = O.decode_layer(hcache, inp, s, layer, run["inp"]["q"][step, layer], d.top_k, N=N)
    return f32_of(out), to_host(sel), ref, rsel


def test_decode_matches_oracle(run):
    s = run["s"]
    for step in range(2):
        for layer in range(s.G):
            out, sel, ref, rsel = decode_both(run, step, layer)
            assert np.array_equal(sel, rsel), (step, layer)
            ok, worst = within_tol(out, ref)
            assert ok, f"step {step} layer {layer}: worst |err|/tol {worst:.3f}"


@pytest.mark.parametrize("which", ["all", "clamp", "tail-only", "no-tail", "one"])
def test_decode_edge_cases(run, which):
    s = run["s"]
    n_c = evicted(run)[0].n_ctx // s.C
    kw = {"all": dict(top_k=n_c), "clamp": dict(top_k=n_c + 7), "tail-only": dict(top_k=0),
          "no-tail": dict(tail=False), "one": dict(top_k=1)}[which]
    out, sel, ref, rsel = decode_both(run, 1, s.G - 1, **kw)
    assert np.array_equal(sel, rsel)
    if which in ("all", "clamp"):
        assert np.array_equal(sel[0, 0], np.arange(n_c))
    ok, worst = within_tol(out, ref)
    assert ok, worst


def test_decode_is_deterministic(run):
    s = run["s"]
    d, cache, _, _ = evicted(run)
    dev = run["dev"]
    q = dev["q"][0, 0].contiguous()
    outs = [P().decode_attn(d, 0, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"]).clone() for _ in range(2)]
    sync()
    assert torch.equal(outs[0], outs[1])


def test_staged_calls_equal_fused_call(run):
    s = run["s"]
    d, cache, _, _ = evicted(run)
    dev = run["dev"]
    q = dev["q"][1, 0].contiguous()
    ws = P().workspace(d, P()._lib.OP_DECODE)
    out1 = torch.empty_like(q)
    call = P().DecodeCall(d, 0, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], out1, ws)
    call.select(); call.attend(); call.combine()
    out2 = P().decode_attn(d, 0, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"])
    sync()
    assert torch.equal(out1, out2)


def test_dense_comparator_matches_oracle(run):
    s = run["s"]
    dev, inp = run["dev"], run["inp"]
    kd = torch.cat([dev["k"], dev["k_tail"]], dim=3).contiguous()
    vd = torch.cat([dev["v"], dev["v_tail"]], dim=3).contiguous()
    d = run["d"]
    for layer in (0, s.G - 1):
        q = dev["q"][0, layer].contiguous()
        out = P().dense_decode_attn(d, q, kd, vd, layer)
        sync()
        K = np.concatenate([O.decode(inp["k"][:, layer], s.act), O.decode(inp["k_tail"][:, layer], s.act)], axis=2)
        V = np.concatenate([O.decode(inp["v"][:, layer], s.act), O.decode(inp["v_tail"][:, layer], s.act)], axis=2)
        ref = O.dense_decode_layer(O.decode(inp["q"][0, layer], s.act), K, V, s.Hq, s.Hkv)
        ok, worst = within_tol(f32_of(out), ref)
        assert ok, worst


# ---------------------------------------------------------------------------
# special shapes
# ---------------------------------------------------------------------------
def _roundtrip(s, top_k, edit=None):
    inp = gen.make(s)
    if edit is not None:
        edit(inp, s)
    dev = upload(inp)
    d = dims_of(s, top_k=top_k)
    cache = P().alloc_cache(d)
    P().compress(d, model_of(dev), dev["k"], dev["v"], cache)
    q = dev["q"][0, 1].contiguous()
    sel = torch.empty((s.B, s.Hkv, P().k_eff(d)), dtype=torch.int32, device="cuda")
    out = P().decode_attn(d, 1, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], sel_out=sel)
    sync()
    host = cache_to_host(cache)
    ref, rsel = O.decode_layer(host, inp, s, 1, inp["q"][0, 1], top_k)
    return f32_of(out), to_host(sel), ref, rsel, host, inp


@pytest.mark.parametrize("name,shape,top_k", [
    ("mha", small(LLAMA8B_32K, Hq=8, Hkv=8, B=1, N=1024, T=32), 3),
    ("no-residuals", small(LLAMA8B_32K, B=1, N=1024, rho=0.0, T=16), 4),
    ("all-residuals", small(LLAMA8B_32K, B=1, N=1024, rho=1.0, T=16), 4),
    ("fp32-g8", TINY.replace(Hq=16, N=512, rho=0.5, T=1), 3),
    ("int8-ragged", small(COMPOSED_128K, B=1, N=2048, evict_keep=1.0, n_obs=0, T=5), 7),
    # selection paths: radix top-k inside the fused scorer (256 < n_c <= 1024),
    # the three-kernel scorer (n_c > 1024), two and four rank segments per lane
    # one rank block (r <= 64) and n_c <= 256: the score kernel ranks its own
    # scores, here at the most chunks it takes and at a ragged count
    ("self-ranked-nc-256", TINY.replace(N=16384, T=8), 9),
    ("self-ranked-nc-197", TINY.replace(N=197 * 64, T=8), 37),
    ("nc-512", TINY.replace(N=32768, T=8), 9),
    ("nc-2048-unfused", TINY.replace(N=131072, T=8), 11),
    ("rank-1024", small(LLAMA8B_32K, B=1, N=1024, r=1024, T=16), 3),
    ("rank-2048", small(LLAMA8B_32K, B=1, N=1024, r=2048, T=16), 3),
    # the chained kernel's own top-k with eight key slots per lane (256 < n_c <= 512),
    # a ragged last slot and a full one
    # the per-chunk kernel's share of the tail: fewer tail tokens than splits (two
    # splits get one token, three get none), and one split with a ragged 70-token tail
    ("mfma-tail-2-of-5", small(QWEN4B_64K, B=1, N=2048, T=2), 5),
    ("mfma-tail-70-k1", small(QWEN4B_64K, B=1, N=1024, T=70), 1),
    # the chained kernel's other compiled (rank, hidden width, codes)
    ("chain-r256", small(LLAMA8B_32K, B=1, N=2048, r=256, T=16), 4),
    ("chain-f128", small(LLAMA8B_32K, B=1, N=2048, F=128, T=16), 4),
    ("chain-int8-r512", small(COMPOSED_128K, B=1, N=2048, evict_keep=1.0, n_obs=0, r=512, T=16), 4),
    ("chain-nc-320", small(LLAMA8B_32K, B=1, Hq=8, Hkv=2, N=40960, T=16), 9),
    ("chain-nc-512", small(LLAMA8B_32K, B=1, Hq=8, Hkv=2, N=65536, T=16), 9),
    # above 512 chunks the chained kernel reads the selection of the separate top-k
    ("chain-nc-1024", small(LLAMA8B_32K, B=1, Hq=8, Hkv=2, N=131072, T=16), 9),
    # the absorbed kernel (head dim 256): 6 score blocks in its shared launch
    # (padded to 8 idle-ended workgroups before the A tiles), and above 256
    # chunks, where it reads the selection of the separate top-k
    ("absorb-sel-pad", small(QWEN4B_64K, B=1, Hq=4, Hkv=1, N=2048, T=16), 3),
    ("absorb-nc-320", small(QWEN4B_64K, B=1, Hq=4, Hkv=1, N=81920, T=16), 5),
    # int8 codes on the absorbed path: the rank scales folded into A and q~
    ("absorb-int8", small(QWEN4B_64K, B=1, N=2048, T=40, coeff=I8, resid=I8), 4),
    # its other compiled rank (r = 512), and two query heads per kv head
    ("absorb-r512", small(QWEN4B_64K, B=1, N=2048, T=24, r=512), 3),
    ("absorb-g2", small(QWEN4B_64K, B=2, Hq=8, N=2048, T=24), 3),
    # peaked softmax: keys of norm ~100 and queries x16 give logits in the
    # hundreds, on each attend kernel (chained bf16 and int8, absorbed at head
    # dim 256, per-chunk matrix-core at g = 8, vector).  The value model's first
    # layer is scaled by 1 / key_scale, so hidden activations and values keep
    # their usual size.
    ("peaked-chain", small(LLAMA8B_32K, B=1, N=2048, T=40, key_scale=8.0, q_scale=16.0, w1_scale=0.125), 5),
    ("peaked-chain-int8", small(COMPOSED_128K, B=1, N=2048, evict_keep=1.0, n_obs=0, T=40,
                                key_scale=8.0, q_scale=16.0, w1_scale=0.125), 5),
    ("peaked-absorb", small(QWEN4B_64K, B=1, N=2048, T=40, key_scale=6.0, q_scale=16.0, w1_scale=1 / 6.0), 3),
    ("peaked-mfma-g8", small(QWEN4B_64K, B=1, Hq=32, N=2048, T=40, key_scale=6.0, q_scale=16.0,
                             w1_scale=1 / 6.0), 3),
    ("peaked-valu", TINY.replace(key_scale=12.5, q_scale=16.0, w1_scale=0.08), 4),
])
def test_special_shapes(name, shape, top_k):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {name}: {shape}", flush=True)
    if name.startswith("absorb") or name.startswith("chain"):
        assert P().decode_kernel(dims_of(shape, top_k=top_k)) == name.split("-")[0]
    out, sel, ref, rsel, host, inp = _roundtrip(shape, top_k)
    assert np.array_equal(sel, rsel)
    ok, worst = within_tol(out, ref)
    assert ok, f"worst |err|/tol {worst:.3f}"
    if name.startswith("peaked"):  # the regime is reached: logits span hundreds
        qn = O.decode(inp["q"][0, 1], shape.act)[0, 0]
        kn = O.decode(inp["k_tail"][0, 1, 0], shape.act)
        assert np.ptp(kn @ qn) / np.sqrt(shape.dh) > 100
        assert np.max(np.linalg.norm(kn, axis=-1)) > 60
    if shape.rho == 1.0:
        assert np.array_equal(host["res_idx"][0, 0, 0], np.arange(shape.N))


# ---------------------------------------------------------------------------
# equal chunk scores: the selection takes the lower chunk index first
# ---------------------------------------------------------------------------
def _copy_chunks(src_of):
    """An input edit that makes chunk j's keys and values those of chunk
    src_of(j), so their coefficients, landmarks and scores are equal."""
    def edit(inp, s):
        for name in ("k", "v"):
            x = inp[name]
            for j in range(s.N // s.C):
                i = src_of(j)
                if i != j:
                    x[:, :, :, j * s.C:(j + 1) * s.C] = x[:, :, :, i * s.C:(i + 1) * s.C]
    return edit


@pytest.mark.parametrize("name,shape,top_k,src_of", [
    # pairs of equal chunks, an odd k splits the pair at the threshold
    ("pairs", small(LLAMA8B_32K, B=1, N=2048, T=16), 5, lambda j: j - j % 2),
    # every chunk equal: the first k chunks
    ("all-equal", small(LLAMA8B_32K, B=1, N=2048, T=16), 6, lambda j: 0),
    # runs of three equal chunks over 320 chunks (eight key slots per lane)
    ("triples-nc-320", small(LLAMA8B_32K, B=1, Hq=8, Hkv=2, N=40960, T=16), 10, lambda j: j - j % 3),
    # the absorbed kernel (head dim 256) ranks the scores in its own prologue
    ("absorb-pairs", small(QWEN4B_64K, B=1, N=4096, T=16), 5, lambda j: j - j % 2),
    ("absorb-all-equal", small(QWEN4B_64K, B=1, N=4096, T=16), 6, lambda j: 0),
    # the score kernel ranking its own scores (r <= 64, n_c <= 256)
    ("valu-pairs", TINY.replace(N=8192, T=16), 7, lambda j: j - j % 2),
    ("valu-all-equal", TINY.replace(N=4096, T=16), 6, lambda j: 0),
])
def test_selection_ties(name, shape, top_k, src_of):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] ties {name}: {shape}", flush=True)
    assert P().decode_kernel(dims_of(shape, top_k=top_k)) == {"absorb": "absorb", "valu": "valu"}.get(
        name.split("-")[0], "chain")
    out, sel, ref, rsel, host, inp = _roundtrip(shape, top_k, edit=_copy_chunks(src_of))
    lm = host["landmark"][0]
    assert any(np.array_equal(lm[j], lm[src_of(j)]) for j in range(1, lm.shape[0]) if src_of(j) != j)
    assert np.array_equal(sel, rsel)
    if name.endswith("all-equal"):
        assert np.array_equal(sel[0, 0], np.arange(top_k))
    ok, worst = within_tol(out, ref)
    assert ok, worst


# ---------------------------------------------------------------------------
# the chained kernel with four 64-token tiles per wave: one split per (b, h)
# once B * Hkv >= 256 (here 32 x 8), 16 of 24 chunks = 32 tiles over 8 waves
# (a 2-layer group keeps the host's input generation short)
# ---------------------------------------------------------------------------
def test_chain_four_tiles_per_wave_every_layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = small(MISTRAL7B_16K, B=32, G=2, N=3072, k=16, T=24)
    print(f"\n[case] chain-4-tiles-per-wave: {s}", flush=True)
    inp = gen.make(s, steps=1)
    dev = upload(inp)
    d = dims_of(s)
    assert P().decode_kernel(d) == "chain"
    # one split per (b, h): the partials hold B * Hkv * g rows of (4 + F + dh) floats
    parts = P().workspace_bytes(d, P()._lib.OP_DECODE)
    assert parts >= s.B * s.Hkv * s.g * (4 + s.F + s.dh) * 4
    cache = P().alloc_cache(d)
    P().compress(d, model_of(dev), dev["k"], dev["v"], cache)
    sync()
    host = cache_to_host(cache)
    for layer in range(s.G):
        q = dev["q"][0, layer].contiguous()
        sel = torch.full((s.B, s.Hkv, s.k), -1, dtype=torch.int32, device="cuda")
        out = P().decode_attn(d, layer, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], sel_out=sel)
        sync()
        ref, rsel = O.decode_layer(host, inp, s, layer, inp["q"][0, layer], s.k)
        assert np.array_equal(to_host(sel), rsel), layer
        ok, worst = within_tol(f32_of(out), ref)
        assert ok, f"layer {layer}: worst |err|/tol {worst:.3f}"


# ---------------------------------------------------------------------------
# large hidden activations: keys of norm ~100 fed to the unscaled value model
# give SiLU outputs of ~30 and values of ~30.  The hidden activations enter the
# p-weighted hidden sum as fp16 (11 significant bits), so an output element
# near zero carries ~2^-12 |H| |W2 row| of rounding, a few times the 2e-3
# absolute floor of the bar.  Measured and reported, not a parity case.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,shape,top_k", [
    ("large-hidden-chain", small(LLAMA8B_32K, B=1, N=2048, T=40, key_scale=8.0, q_scale=16.0), 5),
])
def test_large_hidden_activations_error_is_bounded(name, shape, top_k):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {name}: {shape}", flush=True)
    out, sel, ref, rsel, host, inp = _roundtrip(shape, top_k)
    assert np.array_equal(sel, rsel)
    # relative to the data's scale the error stays at fp16 level
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(out - ref))
    print(f"[case] {name}: max |err| {err:.3e}, max |out| {scale:.2f}, err / scale {err / scale:.2e}", flush=True)
    assert err <= 2.0 ** -9 * scale
