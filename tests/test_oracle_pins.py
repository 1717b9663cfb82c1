"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: printed
values (tests/golden), closed forms, textbook identities, brute force on tiny
inputs, or a library routine a special case reduces to.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import lowram_oracle as O
from synth import gen
from synth.configs import F64, BF16, I8, QWEN4B_64K, Shape, small

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny64(**kw) -> Shape:
    base = dict(name="pin", cfg_id=90, B=1, G=2, Hq=4, Hkv=2, dh=8, r=8, F=16, N=64, C=8,
                k=2, T=4, rho=0.25, act=F64, coeff=F64, resid=F64, steps=2)
    base.update(kw)
    return Shape(**base)


def kcat_of(inp, s, b):
    k = O.decode(inp["k"][b], s.act)
    return k.transpose(2, 0, 1, 3).reshape(s.N, -1)


def recon_keys(cache, inp, s, b, l, h):
    """k_hat rows written out with einsum, independent of the oracle's matmul path."""
    U = O.decode(inp["basis"][b], s.act)
    r0 = (l * s.Hkv + h) * s.dh
    c = O.coeff_deq(cache, b, s.coeff)
    return np.einsum("tr,dr->td", c, U[r0:r0 + s.dh])


def mlp_explicit(x, w1, b1, w2, b2):
    out = np.zeros((x.shape[0], w2.shape[0]))
    for t in range(x.shape[0]):
        pre = np.array([sum(w1[f, d] * x[t, d] for d in range(x.shape[1])) + b1[f] for f in range(w1.shape[0])])
        hid = pre * (1.0 / (1.0 + np.exp(-pre)))
        out[t] = w2 @ hid + b2
    return out


def sdpa64(q, k, v):
    """torch's scaled_dot_product_attention in float64 on the CPU (library routine)."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(v))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def test_bf16_rounding_golden():
    with open(os.path.join(GOLDEN, "bf16_rounding.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    xs = np.array([float.fromhex(a) for a, _ in rows])
    want = np.array([int(b, 16) for _, b in rows], dtype=np.uint16)
    got = O.to_bf16_bits(xs)
    assert np.array_equal(got, want), list(zip(rows, [hex(g) for g in got]))


def test_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.to_bf16_bits(x32.astype(np.float64))
    assert np.array_equal(got, want)
    back = O.from_bf16_bits(got)
    assert np.array_equal(back, torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy())


def test_f16_matches_numpy():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-18, 11, 200000))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)
    assert np.array_equal(O.to_f16(x).view(np.uint16), ref.view(np.uint16))
    # ties to even at 11 significant bits, single rounding from float64
    assert O.to_f16(np.array([1 + 2.0 ** -11]))[0] == np.float16(1.0)
    assert O.to_f16(np.array([1 + 2.0 ** -11 + 2.0 ** -40]))[0] == np.float16(1 + 2.0 ** -10)


# ---------------------------------------------------------------------------
# keys: projection and reconstruction
# ---------------------------------------------------------------------------
def test_basis_is_orthonormal():
    s = tiny64(r=20)
    inp = gen.make(s)
    U = O.decode(inp["basis"][0], s.act)
    assert np.max(np.abs(U.T @ U - np.eye(s.r))) < 1e-12


def test_full_rank_reconstructs_keys_exactly():
    s = tiny64(r=32)  # r = D
    inp = gen.make(s)
    cache = O.compress(inp, s)
    for l in range(s.G):
        for h in range(s.Hkv):
            k = O.decode(inp["k"][0, l, h], s.act)
            kh = recon_keys(cache, inp, s, 0, l, h)
            assert np.max(np.abs(kh - k)) <= 1e-12 * np.max(np.abs(k))


@pytest.mark.parametrize("r", [1, 5, 13])
def test_eckart_young(r):
    s = tiny64(r=r, N=96, C=8)
    inp = gen.make(s)
    K = kcat_of(inp, s, 0)
    _, sig, vt = np.linalg.svd(K, full_matrices=False)
    inp["basis"] = vt[:r].T[None].copy()
    cache = O.compress(inp, s)
    err = 0.0
    for l in range(s.G):
        for h in range(s.Hkv):
            k = O.decode(inp["k"][0, l, h], s.act)
            err += np.sum((recon_keys(cache, inp, s, 0, l, h) - k) ** 2)
    assert err == pytest.approx(np.sum(sig[r:] ** 2), rel=1e-9, abs=1e-9)


# ---------------------------------------------------------------------------
# values: predictor and residuals
# ---------------------------------------------------------------------------
def test_predictor_matches_explicit_mlp():
    s = tiny64(N=16, C=8)
    inp = gen.make(s)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, s.dh))
    w1, b1, w2, b2 = (O.decode(inp[n][0, 1, 0], s.act) for n in ("w1", "b1", "w2", "b2"))
    assert np.allclose(O.predict(x, w1, b1, w2, b2), mlp_explicit(x, w1, b1, w2, b2), rtol=1e-13, atol=1e-13)


def test_zero_first_layer_gives_b2():
    s = tiny64()
    inp = gen.make(s)
    inp["w1"][:] = 0.0
    inp["b1"][:] = 0.0
    cache = O.compress(inp, s)
    for l in range(s.G):
        for h in range(s.Hkv):
            v = O.decode(inp["v"][0, l, h], s.act)
            b2 = O.decode(inp["b2"][0, l, h], s.act)
            assert np.allclose(cache["errors"][0, l, h], np.sum((v - b2) ** 2, axis=1), rtol=1e-13)


def test_noise_free_full_rank_needs_no_residual():
    s = tiny64(r=32)
    inp = gen.make(s, noise_scale=0.0)
    cache = O.compress(inp, s)
    assert np.max(cache["errors"]) < 1e-20
    assert np.max(np.abs(cache["res_val"])) < 1e-10


def test_all_residuals_give_exact_values():
    s = tiny64(r=32, rho=1.0)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    for l in range(s.G):
        for h in range(s.Hkv):
            k = recon_keys(cache, inp, s, 0, l, h)
            w = [O.decode(inp[n][0, l, h], s.act) for n in ("w1", "b1", "w2", "b2")]
            vhat = mlp_explicit(k, *w)
            idx = cache["res_idx"][0, l, h]
            assert np.array_equal(idx, np.arange(s.N))
            v = O.decode(inp["v"][0, l, h], s.act)
            assert np.max(np.abs(vhat + O.decode(cache["res_val"][0, l, h], s.resid) - v)) < 1e-12


def test_residual_set_is_brute_force_topk():
    s = tiny64(N=48, C=8, rho=0.3)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    for l in range(s.G):
        for h in range(s.Hkv):
            e = cache["errors"][0, l, h]
            want = sorted(sorted(range(s.N), key=lambda t: (-e[t], t))[:s.n_res])
            assert list(cache["res_idx"][0, l, h]) == want
            ptr = cache["res_ptr"][0, l, h]
            for j in range(s.n_c + 1):
                assert ptr[j] == sum(1 for t in want if t < j * s.C)


def test_topk_ties_go_to_lower_index():
    key = np.array([1.0, 5.0, 3.0, 5.0, 2.0, 5.0])
    assert list(O.topk_indices(key, 1)) == [1]
    assert list(O.topk_indices(key, 2)) == [1, 3]
    assert list(O.topk_indices(key, 4)) == [1, 2, 3, 5]
    assert list(O.topk_indices(key, 99)) == [0, 1, 2, 3, 4, 5]
    rng = np.random.default_rng(4)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        key = rng.integers(0, 5, n).astype(np.float64)
        k = int(rng.integers(0, n + 2))
        want = sorted(sorted(range(n), key=lambda t: (-key[t], t))[:k])
        assert list(O.topk_indices(key, k)) == want


def test_duplicated_tokens_tie_to_lower_index():
    s = tiny64(N=32, C=8, rho=0.125)  # n_res = 4
    inp = gen.make(s)
    # token 20 becomes an exact copy of token 3 in every layer and head
    for name in ("k", "v"):
        inp[name][:, :, :, 20] = inp[name][:, :, :, 3]
    # make their error the largest: push their value far off
    inp["v"][:, :, :, 3] += 50.0
    inp["v"][:, :, :, 20] = inp["v"][:, :, :, 3]
    s1 = s.replace(rho=1.0 / 32)  # n_res = 1: exactly one of the two tied tokens
    cache = O.compress(inp, s1)
    assert cache["errors"][0, 0, 0, 3] == cache["errors"][0, 0, 0, 20]
    assert np.all(cache["res_idx"][..., 0] == 3)


def test_outlier_tokens_all_get_residuals():
    s = small(QWEN4B_64K, B=1, N=16 * 256)
    inp = gen.make(s)
    assert inp["outliers"].shape[1] == round(0.01 * s.N)
    cache = O.compress(inp, s)
    for l in range(s.G):
        for h in range(s.Hkv):
            assert set(inp["outliers"][0].tolist()) <= set(cache["res_idx"][0, l, h].tolist())


# ---------------------------------------------------------------------------
# chunk scorer and selection
# ---------------------------------------------------------------------------
def test_chunk_score_equals_mean_token_score():
    s = tiny64(N=64, C=8, r=12)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    q = O.decode(inp["q"][0, 1, 0], s.act)  # step 0, layer 1, b 0
    for h in range(s.Hkv):
        kh = recon_keys(cache, inp, s, 0, 1, h)
        grp = [g for g in range(s.Hq) if g * s.Hkv // s.Hq == h]
        per_tok = sum(kh @ q[g] for g in grp)
        want = per_tok.reshape(s.n_c, s.C).mean(axis=1)
        got = O.chunk_scores(cache["landmark"][0], O.decode(inp["basis"][0], s.act), q, 1, h,
                             s.Hq, s.Hkv, s.dh)
        assert np.allclose(got, want, rtol=1e-6, atol=1e-6 * np.max(np.abs(want)))


def test_selection_is_brute_force_and_ties_lower_chunk():
    s = tiny64(N=64, C=8, r=12, k=3)
    inp = gen.make(s)
    # chunk 6 becomes a copy of chunk 2, so their landmarks (and scores) are equal
    inp["k"][:, :, :, 48:56] = inp["k"][:, :, :, 16:24]
    cache = O.compress(inp, s)
    assert np.array_equal(cache["landmark"][0, 6], cache["landmark"][0, 2])
    U = O.decode(inp["basis"][0], s.act)
    for step in range(2):
        q = O.decode(inp["q"][step, 0, 0], s.act)
        for h in range(s.Hkv):
            sc = O.chunk_scores(cache["landmark"][0], U, q, 0, h, s.Hq, s.Hkv, s.dh)
            assert sc[6] == sc[2]
            for k in range(0, s.n_c + 2):
                want = sorted(sorted(range(s.n_c), key=lambda j: (-sc[j], j))[:k])
                assert list(O.select_chunks(sc, k)) == want


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _independent_decode(cache, inp, s, l, q, sel):
    """Brute force: rebuild the selected keys/values with einsum and explicit
    loops, append the tail, attend with torch's SDPA in float64."""
    out = np.zeros((s.B, s.Hq, s.dh))
    for b in range(s.B):
        qb = O.decode(q[b], s.act)
        for h in range(s.Hkv):
            kh = recon_keys(cache, inp, s, b, l, h)
            w = [O.decode(inp[n][b, l, h], s.act) for n in ("w1", "b1", "w2", "b2")]
            toks = [j * s.C + i for j in sel[b, h] for i in range(s.C)]
            vh = mlp_explicit(kh[toks], *w) if toks else np.zeros((0, s.dh))
            resid = dict(zip(cache["res_idx"][b, l, h][: cache["res_ptr"][b, l, h][-1]].tolist(),
                             O.resid_deq(cache, b, l, h, s.resid)))
            for i, t in enumerate(toks):
                if t in resid:
                    vh[i] = vh[i] + resid[t]
            keys = np.concatenate([kh[toks], O.decode(inp["k_tail"][b, l, h], s.act)])
            vals = np.concatenate([vh, O.decode(inp["v_tail"][b, l, h], s.act)])
            for g in range(s.Hq):
                if g * s.Hkv // s.Hq == h:
                    out[b, g] = sdpa64(qb[g], keys, vals)
    return out


@pytest.mark.parametrize("k", [1, 3, 8])
def test_decode_matches_brute_force(k):
    s = tiny64(N=64, C=8, r=12, k=k, B=2)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    for l in range(s.G):
        out, sel = O.decode_layer(cache, inp, s, l, inp["q"][0, l], k)
        assert sel.shape == (s.B, s.Hkv, min(k, s.n_c))
        want = _independent_decode(cache, inp, s, l, inp["q"][0, l], sel)
        assert np.allclose(out, want, rtol=1e-11, atol=1e-12)


def test_exact_cache_all_chunks_equals_dense_attention():
    s = tiny64(r=32, rho=1.0, B=2)  # r = D and residuals on every token: exact K/V
    inp = gen.make(s)
    cache = O.compress(inp, s)
    for l in range(s.G):
        q = inp["q"][1, l]
        out, sel = O.decode_layer(cache, inp, s, l, q, s.n_c)
        assert np.array_equal(sel[0, 0], np.arange(s.n_c))
        for b in range(s.B):
            for g in range(s.Hq):
                h = g * s.Hkv // s.Hq
                K = np.concatenate([inp["k"][b, l, h], inp["k_tail"][b, l, h]])
                V = np.concatenate([inp["v"][b, l, h], inp["v_tail"][b, l, h]])
                assert np.allclose(out[b, g], sdpa64(q[b, g], K, V), rtol=1e-10, atol=1e-11)


def test_mha_reduces_to_per_head_attention():
    s = tiny64(Hq=2, Hkv=2, r=32, rho=1.0)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    q = inp["q"][0, 0]
    out, _ = O.decode_layer(cache, inp, s, 0, q, s.n_c)
    for g in range(2):
        K = np.concatenate([inp["k"][0, 0, g], inp["k_tail"][0, 0, g]])
        V = np.concatenate([inp["v"][0, 0, g], inp["v_tail"][0, 0, g]])
        assert np.allclose(out[0, g], sdpa64(q[0, g], K, V), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("Hq,Hkv", [(16, 4), (8, 2), (6, 3), (4, 4)])
def test_dense_decode_layer_matches_torch_gqa_attention(Hq, Hkv):
    """The uncompressed comparator's attention equals torch's scaled dot-product
    attention (float64, CPU), whose enable_gqa mode maps query head g to kv head
    g // (Hq / Hkv) by itself: a head-mapping or scale slip fails here."""
    rng = np.random.default_rng(Hq * 10 + Hkv)
    B, n, dh = 2, 37, 16
    q = rng.standard_normal((B, Hq, dh)) * 2.0
    k = rng.standard_normal((B, Hkv, n, dh))
    v = rng.standard_normal((B, Hkv, n, dh))
    out = O.dense_decode_layer(q, k, v, Hq, Hkv)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(k), torch.from_numpy(v),
        enable_gqa=True)[:, :, 0, :].numpy()
    assert np.allclose(out, want, rtol=1e-12, atol=1e-13)
    if Hq != Hkv:  # a wrong grouping (interleaved heads) would differ
        perm = np.array([g % Hkv for g in range(Hq)])
        wrong = np.stack([[O.softmax_attend(q[b, g], k[b, perm[g]], v[b, perm[g]]) for g in range(Hq)]
                          for b in range(B)])
        assert not np.allclose(wrong, want)


def test_tail_only_and_no_tail():
    s = tiny64(B=1)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    q = inp["q"][0, 0]
    out, sel = O.decode_layer(cache, inp, s, 0, q, 0)  # k = 0: the tail alone
    assert sel.shape[-1] == 0
    for g in range(s.Hq):
        h = g * s.Hkv // s.Hq
        assert np.allclose(out[0, g], sdpa64(q[0, g], inp["k_tail"][0, 0, h], inp["v_tail"][0, 0, h]))
    s0 = s.replace(T=0)
    inp0 = gen.make(s0)
    cache0 = O.compress(inp0, s0)
    out0, sel0 = O.decode_layer(cache0, inp0, s0, 1, inp0["q"][0, 1], 2)
    want = _independent_decode(cache0, inp0, s0, 1, inp0["q"][0, 1], sel0)
    assert np.allclose(out0, want, rtol=1e-11, atol=1e-12)
    with pytest.raises(ValueError):
        O.decode_layer(cache0, inp0, s0, 0, inp0["q"][0, 0], 0)


# ---------------------------------------------------------------------------
# storage accounting
# ---------------------------------------------------------------------------
def test_mkv_golden_llama8b():
    with open(os.path.join(GOLDEN, "mkv_llama8b_32k.json")) as f:
        g = json.load(f)
    total = g["B"] * O.m_kv(g["L"], g["Hkv"], g["dh"], g["N"], g["s_bytes"])
    assert total == g["expected_bytes"] == 16 * 2 ** 30
    assert abs(total / 1e9 - g["printed_GB"]) / g["printed_GB"] < 0.08


def test_value_side_ratio_near_printed_4x():
    with open(os.path.join(GOLDEN, "value_ratio_4x.json")) as f:
        g = json.load(f)
    N = 4096
    dense_v = N * g["dh"] * g["s_bytes"]
    resid = math.ceil(g["rho"] * N) * (g["dh"] * g["s_bytes"] + 4)
    assert abs(dense_v / resid / g["printed_ratio"] - 1) < g["tolerance_rel"]


def test_compressed_bytes_counts_each_stored_tensor():
    s = tiny64(coeff=F64, resid=F64)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    stored = (cache["coeff"][0].nbytes + inp["basis"][0].nbytes
              + sum(inp[n][0].nbytes for n in ("w1", "b1", "w2", "b2"))
              + cache["res_val"][0].nbytes + cache["res_idx"][0].nbytes
              + cache["res_ptr"][0].nbytes + cache["landmark"][0].nbytes)
    assert O.compressed_bytes(s.G, s.Hkv, s.dh, s.N, s.C, s.r, s.F, s.n_res, s.act, s.coeff, s.resid) == stored


def _stored_nbytes(cache, inp, b, n_rows=None):
    """Bytes of every array one sequence's compressed group stores, read off
    the arrays themselves (residual arrays cut to n_rows rows per head)."""
    sl = (lambda a: a) if n_rows is None else (lambda a: a[..., :n_rows] if a.ndim == 3 else a[:, :, :n_rows])
    total = cache["coeff"][b].nbytes + inp["basis"][b].nbytes + cache["landmark"][b].nbytes
    total += sum(inp[n][b].nbytes for n in ("w1", "b1", "w2", "b2"))
    total += sl(cache["res_idx"][b]).nbytes + sl(cache["res_val"][b]).nbytes + cache["res_ptr"][b].nbytes
    for name in ("coeff_scale", "res_scale"):
        if cache.get(name) is not None:
            total += cache[name][b].nbytes
    return total


@pytest.mark.parametrize("coeff,resid", [(I8, I8), (BF16, I8), (I8, BF16), (BF16, BF16)])
def test_compressed_bytes_counts_scales_of_int8_caches(coeff, resid):
    """Int8 and mixed caches: the formula equals the summed nbytes of every
    stored array, the fp16 coefficient and residual scales included."""
    s = tiny64(act=BF16, coeff=coeff, resid=resid, dh=16, r=16, N=128, C=16, B=2)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    assert (cache.get("coeff_scale") is not None) == (coeff == I8)
    assert (cache.get("res_scale") is not None) == (resid == I8)
    for b in range(s.B):
        assert O.compressed_bytes(s.G, s.Hkv, s.dh, s.N, s.C, s.r, s.F, s.n_res, s.act, s.coeff,
                                  s.resid) == _stored_nbytes(cache, inp, b)


def test_evicted_cache_bytes_capacity_and_live_rows():
    """After eviction each head keeps the rows of its kept chunks.  Sized to
    the largest head's rows, the cache's arrays hold exactly the formula's
    bytes at that capacity; counting live rows only gives the formula with
    rows = their sum.  The live count is at most the capacity."""
    s = tiny64(act=BF16, coeff=I8, resid=I8, dh=16, r=16, N=256, C=16, B=2, n_obs=3, rho=0.25)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    keep = 5
    ev = O.evict(cache, inp, s, inp["obs_q"], keep)
    N2 = keep * s.C
    for b in range(s.B):
        live = ev["res_ptr"][b, :, :, keep]
        cap = int(live.max())
        assert O.compressed_bytes(s.G, s.Hkv, s.dh, N2, s.C, s.r, s.F, cap, s.act, s.coeff,
                                  s.resid) == _stored_nbytes(ev, inp, b, n_rows=cap)
        by_rows = O.compressed_bytes(s.G, s.Hkv, s.dh, N2, s.C, s.r, s.F, cap, s.act, s.coeff, s.resid,
                                     rows=int(live.sum()))
        spare = (s.G * s.Hkv * cap - int(live.sum())) * (s.dh * 1 + 4)
        assert by_rows == _stored_nbytes(ev, inp, b, n_rows=cap) - spare


def test_composed_workload_ratios():
    """The composed int8 workload against a dense bf16 cache of its 131072
    tokens: 28.4x before eviction; after keeping a quarter of the chunks, the
    formula gives 90.8x when the kept chunks carry a quarter of each head's
    residual rows (the expected share for rows spread evenly over chunks).
    Both figures are derived independently from the workload sizes."""
    from synth.configs import COMPOSED_128K as s
    dense = O.m_kv(s.G, s.Hkv, s.dh, s.N, 2)
    assert dense == 2 * 2 ** 30
    before = O.compressed_bytes(s.G, s.Hkv, s.dh, s.N, s.C, s.r, s.F, s.n_res, s.act, s.coeff, s.resid)
    assert dense / before == pytest.approx(28.4, abs=0.05)
    N2 = s.keep_chunks * s.C
    after = O.compressed_bytes(s.G, s.Hkv, s.dh, N2, s.C, s.r, s.F, s.n_res, s.act, s.coeff, s.resid,
                               rows=s.G * s.Hkv * s.n_res // 4)
    assert dense / after == pytest.approx(90.8, abs=0.1)


# ---------------------------------------------------------------------------
# quantisation
# ---------------------------------------------------------------------------
def test_int8_quantisation_bounds():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((500, 7)) * np.array([1e-3, 0.1, 1, 10, 100, 3e3, 0.0])
    q, s16 = O.quantise(x, axis=0)
    s = s16.astype(np.float64)
    assert q.dtype == np.int8 and s16.dtype == np.float16
    assert np.all(np.abs(q) <= 127)
    deq = O.dequantise(q, s16, axis=0)
    amax = np.max(np.abs(x), axis=0)
    bound = s / 2 + np.maximum(amax - 127 * s, 0) + 1e-300
    assert np.all(np.abs(deq - x) <= bound[None, :] * (1 + 1e-12))
    assert np.all(q[:, 6] == 0) and s[6] == 0
    grid = np.arange(-127, 128)[:, None] * s[None, :5]
    q2, s2 = O.quantise(grid, axis=0)
    assert np.array_equal(s2, s16[:5])
    assert np.array_equal(O.dequantise(q2, s2, axis=0), grid)


# ---------------------------------------------------------------------------
# eviction
# ---------------------------------------------------------------------------
def test_eviction_keeps_top_chunks_by_group_score():
    s = tiny64(N=128, C=8, r=12, coeff=F64, n_obs=3, B=2)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    keep = 4
    new = O.evict(cache, inp, s, inp["obs_q"], keep)
    for b in range(s.B):
        acc = np.zeros(s.n_c)
        for w in range(s.n_obs):
            for l in range(s.G):
                q = O.decode(inp["obs_q"][w, b, l], s.act)
                for h in range(s.Hkv):
                    kh = recon_keys(cache, inp, s, b, l, h)
                    grp = [g for g in range(s.Hq) if g * s.Hkv // s.Hq == h]
                    acc += sum(kh @ q[g] for g in grp).reshape(s.n_c, s.C).mean(axis=1)
        assert np.allclose(new["acc"][b], acc, rtol=1e-6, atol=1e-6 * np.max(np.abs(acc)))
        order = sorted(range(s.n_c), key=lambda j: (-acc[j], j))
        gap = acc[order[keep - 1]] - acc[order[keep]]
        assert gap > 1e-4 * np.max(np.abs(acc))
        assert list(new["keep"][b]) == sorted(order[:keep])
        # kept coefficients and residuals map back to the original tokens
        for jn, jo in enumerate(new["keep"][b]):
            assert np.array_equal(new["coeff"][b, jn * s.C:(jn + 1) * s.C], cache["coeff"][b, jo * s.C:(jo + 1) * s.C])
        for l in range(s.G):
            for h in range(s.Hkv):
                n = new["res_ptr"][b, l, h, keep]
                old = dict(zip(cache["res_idx"][b, l, h].tolist(), cache["res_val"][b, l, h]))
                for e in range(n):
                    t = int(new["res_idx"][b, l, h, e])
                    jo = new["keep"][b][t // s.C]
                    assert np.array_equal(new["res_val"][b, l, h, e], old[jo * s.C + t % s.C])
                assert n == sum(1 for t in old if t // s.C in set(new["keep"][b].tolist()))


def test_eviction_keep_all_is_identity():
    s = tiny64(N=64, C=8, n_obs=2)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    new = O.evict(cache, inp, s, inp["obs_q"], s.n_c)
    for name in ("coeff", "landmark", "res_ptr", "res_idx", "res_val"):
        assert np.array_equal(new[name], cache[name]), name


# ---------------------------------------------------------------------------
# tail growth: re-pack of the oldest C tail tokens as a new chunk
# ---------------------------------------------------------------------------
def _tail_chunk(inp, lo, C):
    return inp["k_tail"][:, :, :, lo:lo + C], inp["v_tail"][:, :, :, lo:lo + C]


def _grown(inp, C):
    """The same sequences with the first C tail tokens moved into the prefill."""
    g = dict(inp)
    for a in ("k", "v"):
        g[a] = np.concatenate([inp[a], inp[a + "_tail"][:, :, :, :C]], axis=3)
        g[a + "_tail"] = inp[a + "_tail"][:, :, :, C:]
    return g


@pytest.mark.parametrize("dt", [F64, BF16])
def test_repack_without_residuals_equals_compress_of_longer_prefill(dt):
    s = tiny64(T=12, B=2, act=dt, coeff=dt, resid=dt)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    new = O.repack(cache, inp, *_tail_chunk(inp, 0, s.C), s, m=0)
    ref = O.compress(_grown(inp, s.C), tiny64(T=4, N=72, B=2, act=dt, coeff=dt, resid=dt))
    assert np.array_equal(new["coeff"], ref["coeff"])
    assert np.array_equal(new["landmark"], ref["landmark"])
    assert np.allclose(new["repack_errors"], ref["errors"][..., s.N:], rtol=1e-12, atol=0)
    # no new residuals: the old CSR with its last pointer repeated
    assert np.array_equal(new["res_ptr"][..., :-1], cache["res_ptr"])
    assert np.array_equal(new["res_ptr"][..., -1], cache["res_ptr"][..., -1])
    assert np.array_equal(new["res_idx"], cache["res_idx"])
    assert np.array_equal(new["res_val"], cache["res_val"])


def test_repack_residuals_are_brute_force_topk_of_the_new_chunk():
    s = tiny64(T=12, B=2, act=BF16, coeff=BF16, resid=BF16)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    m, C, N, n_c = 3, s.C, s.N, s.n_c
    kt, vt = _tail_chunk(inp, 0, C)
    new = O.repack(cache, inp, kt, vt, s, m)
    assert new["res_idx"].shape[-1] == s.n_res + m
    for b in range(s.B):
        U = O.decode(inp["basis"][b], s.act)
        kcat = O.decode(kt[b], s.act).transpose(2, 0, 1, 3).reshape(C, -1)
        c = np.einsum("dr,td->tr", U, kcat)
        cst = O.decode(new["coeff"][b, N:], s.coeff)
        assert np.all(np.abs(cst - c) <= np.abs(c) * 2.0 ** -8)
        assert np.allclose(new["landmark"][b, n_c], cst.mean(axis=0), rtol=1e-6, atol=1e-7)
        for l in range(s.G):
            for h in range(s.Hkv):
                r0 = (l * s.Hkv + h) * s.dh
                kh = np.einsum("tr,dr->td", cst, U[r0:r0 + s.dh])
                w = [O.decode(inp[n][b, l, h], s.act) for n in ("w1", "b1", "w2", "b2")]
                v = O.decode(vt[b, l, h], s.act)
                d = v - mlp_explicit(kh, *w)
                e = new["repack_errors"][b, l, h]
                assert np.allclose(e, np.sum(d * d, axis=1), rtol=1e-12)
                want = sorted(sorted(range(C), key=lambda t: (-e[t], t))[:m])
                op, ptr = cache["res_ptr"][b, l, h], new["res_ptr"][b, l, h]
                live = int(op[n_c])
                assert np.array_equal(ptr[:n_c + 1], op) and ptr[n_c + 1] == live + m
                assert list(new["res_idx"][b, l, h, live:live + m]) == [N + t for t in want]
                assert np.array_equal(new["res_idx"][b, l, h, :live], cache["res_idx"][b, l, h, :live])
                assert np.array_equal(new["res_val"][b, l, h, :live], cache["res_val"][b, l, h, :live])
                got = O.decode(new["res_val"][b, l, h, live:live + m], s.resid)
                assert np.all(np.abs(got - d[want]) <= np.abs(d[want]) * 2.0 ** -8)


def test_repacked_exact_cache_equals_dense_attention():
    s = tiny64(r=32, rho=1.0, B=2, T=12)  # r = D, every token keeps its residual
    inp = gen.make(s)
    cache = O.compress(inp, s)
    new = O.repack(cache, inp, *_tail_chunk(inp, 0, s.C), s, m=s.C)
    s2 = tiny64(r=32, rho=1.0, B=2, T=4, N=72)
    g = _grown(inp, s.C)
    for l in range(s.G):
        q = inp["q"][1, l]
        out, sel = O.decode_layer(new, g, s2, l, q, s2.n_c)
        assert np.array_equal(sel[0, 0], np.arange(s2.n_c))
        for b in range(s.B):
            for gq in range(s.Hq):
                h = gq * s.Hkv // s.Hq
                K = np.concatenate([inp["k"][b, l, h], inp["k_tail"][b, l, h]])
                V = np.concatenate([inp["v"][b, l, h], inp["v_tail"][b, l, h]])
                assert np.allclose(out[b, gq], sdpa64(q[b, gq], K, V), rtol=1e-10, atol=1e-11)


def test_repack_twice_matches_exact_attention_after_eviction():
    # eviction leaves spare residual capacity; two re-packs append after the live entries
    s = tiny64(r=32, rho=1.0, B=2, T=20, N=64, n_obs=2)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    keep = 5
    ev = O.evict(cache, inp, s, inp["obs_q"], keep)
    kt, vt = _tail_chunk(inp, 0, s.C)
    s1 = tiny64(r=32, rho=1.0, B=2, T=12, N=keep * s.C)
    one = O.repack(ev, inp, kt, vt, s1, m=s.C)
    kt2, vt2 = _tail_chunk(inp, s.C, s.C)
    s2 = tiny64(r=32, rho=1.0, B=2, T=4, N=(keep + 1) * s.C)
    two = O.repack(one, inp, kt2, vt2, s2, m=s.C)
    assert two["res_idx"].shape[-1] == s.N + 2 * s.C
    g = dict(inp)
    g["k_tail"], g["v_tail"] = inp["k_tail"][:, :, :, 2 * s.C:], inp["v_tail"][:, :, :, 2 * s.C:]
    s3 = tiny64(r=32, rho=1.0, B=2, T=4, N=(keep + 2) * s.C)
    for l in range(s.G):
        q = inp["q"][0, l]
        out, _ = O.decode_layer(two, g, s3, l, q, keep + 2)
        for b in range(s.B):
            toks = np.concatenate([np.arange(j * s.C, (j + 1) * s.C) for j in ev["keep"][b]])
            for gq in range(s.Hq):
                h = gq * s.Hkv // s.Hq
                K = np.concatenate([inp["k"][b, l, h][toks], inp["k_tail"][b, l, h]])
                V = np.concatenate([inp["v"][b, l, h][toks], inp["v_tail"][b, l, h]])
                assert np.allclose(out[b, gq], sdpa64(q[b, gq], K, V), rtol=1e-10, atol=1e-11)


def test_repack_int8_keeps_scales_and_reproduces_prefill_codes():
    s = tiny64(T=12, B=2, act=BF16, coeff=I8, resid=I8)
    inp = gen.make(s)
    cache = O.compress(inp, s)
    C, N, n_c = s.C, s.N, s.n_c
    # the prefill's own first chunk, re-packed, gives back its stored codes and landmark
    again = O.repack(cache, inp, inp["k"][:, :, :, :C], inp["v"][:, :, :, :C], s, m=2)
    assert np.array_equal(again["coeff"][:, N:], cache["coeff"][:, :C])
    assert np.array_equal(again["landmark"][:, n_c], cache["landmark"][:, 0])
    assert np.array_equal(again["coeff_scale"], cache["coeff_scale"])
    assert np.array_equal(again["res_scale"], cache["res_scale"])
    # new tokens: round-to-nearest codes on the old scales, clamped to +-127
    kt, vt = _tail_chunk(inp, 0, C)
    new = O.repack(cache, inp, kt, vt, s, m=3)
    n_in = n_out = 0
    for b in range(s.B):
        U = O.decode(inp["basis"][b], s.act)
        kcat = O.decode(kt[b], s.act).transpose(2, 0, 1, 3).reshape(C, -1)
        c = np.einsum("dr,td->tr", U, kcat)
        sc = cache["coeff_scale"][b].astype(np.float64)[None, :]
        q = new["coeff"][b, N:].astype(np.float64)
        inside = np.abs(c) <= 127 * sc
        assert np.all(np.abs(q) <= 127)
        assert np.all(np.abs(q * sc - c)[inside] <= (sc / 2 * (1 + 1e-12) + 0 * c)[inside])
        assert np.all((q == 127 * np.sign(c))[~inside])
        for l in range(s.G):
            for h in range(s.Hkv):
                live = int(cache["res_ptr"][b, l, h, n_c])
                rs = cache["res_scale"][b, l, h].astype(np.float64)[None, :]
                dq = new["res_val"][b, l, h, live:live + 3].astype(np.float64)
                R = new["res_idx"][b, l, h, live:live + 3] - N
                r0 = (l * s.Hkv + h) * s.dh
                kh = np.einsum("tr,dr->td", q * sc, U[r0:r0 + s.dh])
                w = [O.decode(inp[n][b, l, h], s.act) for n in ("w1", "b1", "w2", "b2")]
                d = (O.decode(vt[b, l, h], s.act) - mlp_explicit(kh, *w))[R]
                ok = np.abs(d) <= 127 * rs
                assert np.all(np.abs(dq) <= 127)
                assert np.all(np.abs(dq * rs - d)[ok] <= (rs / 2 * (1 + 1e-9) + 0 * d)[ok])
                assert np.all((dq == 127 * np.sign(d))[~ok])
                n_in += int(ok.sum()); n_out += int((~ok).sum())
    assert n_in > 0 and n_out > 0  # both the rounding and the clamp are exercised


# ---------------------------------------------------------------------------
# test-time fitting of the value predictor
# ---------------------------------------------------------------------------
def _mlp_case(seed=11, N=40, dh=8, F=16):
    rng = np.random.default_rng(seed)
    khat = rng.standard_normal((N, dh))
    v = rng.standard_normal((N, dh))
    w = [rng.standard_normal((F, dh)) / np.sqrt(dh), 0.1 * rng.standard_normal(F),
         rng.standard_normal((dh, F)) / np.sqrt(F), 0.1 * rng.standard_normal(dh)]
    return khat, v, w


def test_predictor_gradient_matches_torch_autograd():
    khat, v, w = _mlp_case()
    loss, grads = O.predictor_loss_grad(khat, v, *w)
    wt = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in w]
    kt, vt = torch.from_numpy(khat), torch.from_numpy(v)
    pred = torch.nn.functional.silu(kt @ wt[0].T + wt[1]) @ wt[2].T + wt[3]
    lt = ((pred - vt) ** 2).sum(dim=1).mean()
    lt.backward()
    assert loss == pytest.approx(lt.item(), rel=1e-13)
    for g, x in zip(grads, wt):
        assert np.allclose(g, x.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_predictor_gradient_matches_finite_differences():
    khat, v, w = _mlp_case(seed=12)
    _, grads = O.predictor_loss_grad(khat, v, *w)
    rng = np.random.default_rng(3)
    eps = 1e-6
    for i in range(4):
        d = rng.standard_normal(w[i].shape)
        wp = [x.copy() for x in w]
        wm = [x.copy() for x in w]
        wp[i] = wp[i] + eps * d
        wm[i] = wm[i] - eps * d
        fd = (O.predictor_loss_grad(khat, v, *wp)[0] - O.predictor_loss_grad(khat, v, *wm)[0]) / (2 * eps)
        assert fd == pytest.approx(float(np.sum(grads[i] * d)), rel=1e-7, abs=1e-10)


def test_fit_zero_steps_keeps_weights_and_reports_the_error():
    s = tiny64(B=2)
    inp = gen.make(s)
    fit = O.fit_predictor(inp, s, steps=0, lr=0.1)
    cache = O.compress(inp, s)
    for n in ("w1", "b1", "w2", "b2"):
        assert np.array_equal(fit[n], inp[n])
    # loss = mean over tokens of the compress-side squared errors
    assert np.allclose(fit["loss"][..., 0], cache["errors"].mean(axis=-1), rtol=1e-12)


def test_fit_stationary_at_an_exact_predictor():
    s = tiny64(r=32)  # r = D: k_hat = k
    inp = gen.make(s, noise_scale=0.0)
    fit = O.fit_predictor(inp, s, steps=3, lr=0.5)
    assert np.max(fit["loss"]) < 1e-24
    for n in ("w1", "b1", "w2", "b2"):
        assert np.max(np.abs(fit[n] - inp[n])) < 1e-12


def test_fit_descends_and_equals_explicit_gradient_steps():
    s = tiny64(B=1, G=1, Hkv=1, Hq=2)
    inp = gen.make(s)
    lr, steps = 0.05, 6
    fit = O.fit_predictor(inp, s, steps=steps, lr=lr)
    L = fit["loss"][0, 0, 0]
    assert np.all(np.diff(L) < 0), L
    # the same steps written out with torch autograd from the oracle's k_hat
    U = O.decode(inp["basis"][0], s.act)
    kcat = kcat_of(inp, s, 0)
    khat = torch.from_numpy(np.einsum("tr,dr->td", np.einsum("td,dr->tr", kcat, U), U[:s.dh]))
    v = torch.from_numpy(O.decode(inp["v"][0, 0, 0], s.act))
    wt = [torch.from_numpy(O.decode(inp[n][0, 0, 0], s.act)).clone() for n in ("w1", "b1", "w2", "b2")]
    for st in range(steps):
        for x in wt:
            x.requires_grad_(True)
        lt = ((torch.nn.functional.silu(khat @ wt[0].T + wt[1]) @ wt[2].T + wt[3] - v) ** 2).sum(1).mean()
        assert lt.item() == pytest.approx(L[st], rel=1e-11)
        gs = torch.autograd.grad(lt, wt)
        wt = [(x - lr * g).detach() for x, g in zip(wt, gs)]
    for n, x in zip(("w1", "b1", "w2", "b2"), wt):
        assert np.allclose(fit[n][0, 0, 0], x.numpy(), rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------------------
# the group key basis at prefill
# ---------------------------------------------------------------------------
def test_key_basis_is_eckart_young_optimal():
    s = tiny64(B=2, r=8, N=64)
    inp = gen.make(s)
    U, lam = O.key_basis(inp, s)
    for b in range(s.B):
        kcat = kcat_of(inp, s, b)
        sv = np.linalg.svd(kcat, compute_uv=False)          # library SVD, not the Gram
        tail = np.sum(sv[s.r:] ** 2)
        res = np.sum((kcat - kcat @ U[b] @ U[b].T) ** 2)
        assert res == pytest.approx(tail, rel=1e-9)
        assert np.allclose(lam[b], sv[:s.r] ** 2, rtol=1e-10)
        assert np.allclose(U[b].T @ U[b], np.eye(s.r), atol=1e-12)
        assert np.all(np.diff(lam[b]) <= 0)
        # columns are eigenvectors of the Gram matrix, largest entry positive
        G = kcat.T @ kcat
        assert np.allclose(G @ U[b], U[b] * lam[b][None, :], atol=1e-9 * lam[b][0])
        assert np.all(U[b][np.argmax(np.abs(U[b]), axis=0), np.arange(s.r)] > 0)
    assert np.allclose(O.residual_energy(inp, s, U),
                       [np.sum(np.linalg.svd(kcat_of(inp, s, b), compute_uv=False)[s.r:] ** 2) /
                        np.sum(kcat_of(inp, s, b) ** 2) for b in range(s.B)], rtol=1e-9)


def test_key_basis_spans_exactly_low_rank_keys():
    s = tiny64(r=8, key_cols=6)          # keys drawn in a 6-dim subspace of D = 32
    inp = gen.make(s)
    U, lam = O.key_basis(inp, s)
    assert np.max(O.residual_energy(inp, s, U)) < 1e-24
    assert lam[0, 6] < 1e-12 * lam[0, 0]  # eigh resolves zero to about eps * ||G||
    # the generator's frame lies in the span of the leading 6 directions
    F = O.decode(inp["basis"][0], s.act)[:, :6]
    assert np.allclose(U[0][:, :6] @ (U[0][:, :6].T @ F), F, atol=1e-10)


def test_key_basis_full_rank_is_complete():
    s = tiny64(r=32)
    inp = gen.make(s)
    U, _ = O.key_basis(inp, s)
    assert np.allclose(U[0] @ U[0].T, np.eye(32), atol=1e-12)
    assert np.max(O.residual_energy(inp, s, U)) < 1e-25
