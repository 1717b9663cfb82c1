"""The C ABI on the host: exported symbols, storage accounting, workspace
sizing and every validation path.  No call here reaches a kernel launch, so
these run without a GPU (fake device pointers are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import lowram_oracle as O
from synth.configs import ALL, COMPOSED_128K, LLAMA8B_32K, QWEN4B_64K, TINY
from tests.harness import dims_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

P = pytest.importorskip("decode_attention_compressed_amd")
L = P._lib

FAKE = 1 << 20  # a 256-byte aligned fake device address; never dereferenced


def header_functions():
    with open(os.path.join(ROOT, "include", "lowram.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(lowram_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(L.SIGNATURES) == set(names)


@pytest.mark.parametrize("s", ALL, ids=lambda s: s.name)
def test_cache_bytes_match_accounting(s):
    d = dims_of(s)
    comp, dense = P.cache_bytes(d)
    assert dense == O.m_kv(s.G, s.Hkv, s.dh, s.N, O.DTYPE_BYTES[s.act])
    assert comp == O.compressed_bytes(s.G, s.Hkv, s.dh, s.N, s.C, s.r, s.F, s.n_res, s.act, s.coeff, s.resid)


def test_llama_ratio_and_composed_ratio():
    c, dn = P.cache_bytes(dims_of(LLAMA8B_32K))
    assert dn / c == pytest.approx(7.008, abs=1e-3)
    c, dn = P.cache_bytes(dims_of(TINY))
    assert dn / c == pytest.approx(3.006, abs=1e-3)
    # the composed int8 workload before eviction, its scales counted
    c, dn = P.cache_bytes(dims_of(COMPOSED_128K))
    assert dn / c == pytest.approx(28.4, abs=0.05)
    s = COMPOSED_128K
    assert c == O.compressed_bytes(s.G, s.Hkv, s.dh, s.N, s.C, s.r, s.F, s.n_res, s.act, s.coeff, s.resid)
    assert c - P.cache_bytes(dims_of(s.replace(coeff="bf16", resid="bf16")))[0] == \
        (s.r * 2 + s.G * s.Hkv * s.dh * 2) - s.N * s.r - s.G * s.Hkv * s.n_res * s.dh


@pytest.mark.parametrize("s", ALL, ids=lambda s: s.name)
def test_workspace_sizes_are_positive_and_aligned(s):
    d = dims_of(s)
    for op in (L.OP_COMPRESS, L.OP_DECODE, L.OP_EVICT, L.OP_DENSE, L.OP_REPACK, L.OP_FIT, L.OP_BASIS):
        n = P.workspace_bytes(d, op)
        assert n > 0 and n % 256 == 0


def call_decode(d, layer=0, ws_bytes=None, q=FAKE, out=FAKE, sel=None, ws=FAKE, model=None, cache=None):
    lib = L.lib()
    m = model or L.Model(FAKE, FAKE, FAKE, FAKE, FAKE)
    c = cache or L.Cache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    need = P.workspace_bytes(d, L.OP_DECODE) if ws_bytes is None else ws_bytes
    return lib.lowram_decode_attn(ctypes.byref(d), layer, ctypes.byref(m), ctypes.byref(c), q, FAKE,
                                  FAKE, out, sel, ws, need, None)


def status_of(fn):
    try:
        fn()
    except P.LowramError as e:
        return e.status
    return L.OK


def base_dims(**kw):
    d = dims_of(LLAMA8B_32K.replace(B=1, N=1024))
    return P.with_(d, **kw)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), L.E_UNSUPPORTED),
    (dict(n_ctx=1000), L.E_INVALID),            # not a multiple of the chunk
    (dict(n_res=5000), L.E_INVALID),            # more residuals than tokens
    (dict(heads_q=30), L.E_INVALID),            # not a multiple of heads_kv
    (dict(heads_q=8 * 17), L.E_UNSUPPORTED),    # more than 16 query heads per kv head
    (dict(rank=520), L.E_UNSUPPORTED),          # not a multiple of 16
    (dict(rank=8192), L.E_UNSUPPORTED),
    (dict(hidden=100), L.E_UNSUPPORTED),
    (dict(batch=0), L.E_INVALID),
    (dict(chunk=0), L.E_INVALID),
    (dict(top_k=-1), L.E_INVALID),
    (dict(act=L.F32), L.E_UNSUPPORTED),         # f32 act with bf16 coefficients
    (dict(coeff=L.F16), L.E_UNSUPPORTED),
    (dict(act=7), L.E_UNSUPPORTED),
])
def test_bad_dims_rejected_before_launch(kw, status):
    d = base_dims(**kw)
    assert status_of(lambda: P.workspace_bytes(d, L.OP_DECODE)) == status
    assert call_decode(d, ws_bytes=1 << 30) == status
    assert L.lib().lowram_last_error()


def test_decode_argument_errors():
    d = base_dims()
    assert call_decode(d, layer=4) == L.E_INVALID
    assert call_decode(d, layer=-1) == L.E_INVALID
    assert call_decode(d, ws_bytes=P.workspace_bytes(d, L.OP_DECODE) - 256) == L.E_WORKSPACE
    assert call_decode(d, ws=FAKE + 16) == L.E_INVALID    # workspace not 256-byte aligned
    assert call_decode(d, q=FAKE + 2) == L.E_INVALID      # q not 16-byte aligned
    assert call_decode(d, q=None) == L.E_INVALID
    assert call_decode(d, out=None) == L.E_INVALID
    assert call_decode(d, sel=FAKE + 4) == L.E_INVALID
    nothing = P.with_(d, top_k=0, n_tail=0)
    assert call_decode(nothing) == L.E_INVALID
    no_cache = L.Cache(None, None, None, None, None, None, None)
    assert call_decode(d, cache=no_cache) == L.E_INVALID
    i8 = P.with_(d, coeff=L.I8)
    assert call_decode(i8, cache=L.Cache(FAKE, None, FAKE, FAKE, FAKE, FAKE, None)) == L.E_INVALID


def test_compress_and_evict_argument_errors():
    lib = L.lib()
    d = base_dims()
    m = L.Model(FAKE, FAKE, FAKE, FAKE, FAKE)
    c = L.Cache(FAKE, None, FAKE, FAKE, FAKE, FAKE, None)
    need = P.workspace_bytes(d, L.OP_COMPRESS)
    assert lib.lowram_compress(ctypes.byref(d), ctypes.byref(m), None, FAKE, ctypes.byref(c), FAKE, need, None) == L.E_INVALID
    assert lib.lowram_compress(ctypes.byref(d), ctypes.byref(m), FAKE, FAKE, ctypes.byref(c), FAKE, need - 1, None) == L.E_WORKSPACE
    empty = P.with_(d, n_ctx=0, n_res=0)
    assert lib.lowram_compress(ctypes.byref(empty), ctypes.byref(m), FAKE, FAKE, ctypes.byref(c), FAKE, need, None) == L.E_INVALID
    dst = L.Cache(FAKE * 2, None, FAKE * 2, FAKE * 2, FAKE * 2, FAKE * 2, None)
    ne = P.workspace_bytes(d, L.OP_EVICT)
    n_c = d.n_ctx // d.chunk
    def ev(keep, dst_=dst, n_obs=1, cap=d.n_res, keep_out=None, live=None):
        dp = ctypes.byref(dst_) if dst_ is not None else None
        return lib.lowram_evict(ctypes.byref(d), ctypes.byref(m), ctypes.byref(c), FAKE, n_obs, keep, cap,
                                dp, keep_out, live, FAKE, ne, None)
    assert ev(0) == L.E_INVALID
    assert ev(n_c + 1) == L.E_INVALID
    assert ev(2, n_obs=-1) == L.E_INVALID
    assert ev(2, dst_=c) == L.E_INVALID        # in-place eviction is refused
    assert ev(2, cap=-1) == L.E_INVALID        # dst capacity outside [0, n_res]
    assert ev(2, cap=d.n_res + 1) == L.E_INVALID
    assert ev(2, dst_=None) == L.E_INVALID     # nothing to write
    assert ev(2, dst_=None, live=FAKE + 4) == L.E_INVALID  # unaligned live_out


def test_repack_argument_errors():
    lib = L.lib()
    d = P.with_(base_dims(), n_tail=base_dims().chunk + 3)
    m = L.Model(FAKE, FAKE, FAKE, FAKE, FAKE)
    src = L.Cache(FAKE, None, FAKE, FAKE, FAKE, FAKE, None)
    dst = L.Cache(FAKE * 2, None, FAKE * 2, FAKE * 2, FAKE * 2, FAKE * 2, None)
    need = P.workspace_bytes(d, L.OP_REPACK)

    def rp(d_=d, n_new=2, dst_=dst, k=FAKE, ws=FAKE, have=need, src_=src):
        return lib.lowram_repack(ctypes.byref(d_), ctypes.byref(m), ctypes.byref(src_), k, FAKE, n_new,
                                 ctypes.byref(dst_), ws, have, None)

    assert rp(n_new=-1) == L.E_INVALID
    assert rp(n_new=d.chunk + 1) == L.E_INVALID             # more rows than the chunk has
    assert rp(d_=P.with_(d, n_tail=d.chunk - 1)) == L.E_INVALID  # no full chunk in the tail
    assert rp(k=None) == L.E_INVALID
    assert rp(k=FAKE + 8) == L.E_INVALID                     # k_tail not 16-byte aligned
    assert rp(have=need - 1) == L.E_WORKSPACE
    assert rp(ws=FAKE + 64) == L.E_INVALID
    for shared in range(4):                                  # dst sharing src storage
        fields = [FAKE * 2, None, FAKE * 2, FAKE * 2, FAKE * 2, FAKE * 2, None]
        fields[(0, 2, 3, 5)[shared]] = FAKE
        assert rp(dst_=L.Cache(*fields)) == L.E_INVALID
    i8 = P.with_(d, coeff=L.I8)
    assert rp(d_=i8) == L.E_INVALID                          # int8 without coefficient scales
    assert rp(d_=P.with_(i8, n_ctx=0, n_res=0)) == L.E_INVALID  # int8 needs a prefill's scales
    full = P.with_(d, n_ctx=(1 << 22), n_res=0)               # the grown cache would exceed n_ctx limits
    assert rp(d_=full) != L.OK


def test_fit_argument_errors():
    lib = L.lib()
    d = base_dims()
    m = L.Model(FAKE, FAKE, FAKE, FAKE, FAKE)
    out = L.Predictor(FAKE, FAKE, FAKE, FAKE)
    need = P.workspace_bytes(d, L.OP_FIT)

    def fit(d_=d, steps=2, lr=0.1, out_=out, k=FAKE, have=need, loss=None):
        return lib.lowram_fit_predictor(ctypes.byref(d_), ctypes.byref(m), k, FAKE, steps, lr,
                                        ctypes.byref(out_) if out_ is not None else None, loss, FAKE,
                                        have, None)

    assert fit(steps=-1) == L.E_INVALID
    assert fit(lr=-0.5) == L.E_INVALID
    assert fit(lr=float("nan")) == L.E_INVALID
    assert fit(out_=None) == L.E_INVALID
    assert fit(out_=L.Predictor(FAKE, None, FAKE, FAKE)) == L.E_INVALID
    assert fit(k=None) == L.E_INVALID
    assert fit(loss=FAKE + 4) == L.E_INVALID                  # loss not 16-byte aligned
    assert fit(have=need - 1) == L.E_WORKSPACE
    assert fit(d_=P.with_(d, n_ctx=0, n_res=0)) == L.E_INVALID  # no tokens to fit on
    # the workspace holds float32 activations of every token
    Z = d.batch * d.layers * d.heads_kv
    assert need >= 4 * Z * d.n_ctx * (2 * d.hidden + 2 * d.head_dim)


def test_key_basis_argument_errors():
    lib = L.lib()
    d = base_dims()
    need = P.workspace_bytes(d, L.OP_BASIS)

    def kb(d_=d, it=4, k=FAKE, out=FAKE, have=need):
        return lib.lowram_key_basis(ctypes.byref(d_), k, it, out, FAKE, have, None)

    assert kb(it=-1) == L.E_INVALID
    assert kb(k=None) == L.E_INVALID
    assert kb(out=FAKE + 2) == L.E_INVALID
    assert kb(have=need - 1) == L.E_WORKSPACE
    assert kb(d_=P.with_(d, n_ctx=0, n_res=0)) == L.E_INVALID
    wide = P.with_(d, layers=8, heads_kv=8, heads_q=8, head_dim=256)   # D = 16384
    assert kb(d_=wide) == L.E_UNSUPPORTED
    D = d.layers * d.heads_kv * d.head_dim
    assert need >= 4 * d.batch * (D * D + 2 * d.rank * D)


def test_reuse_argument_errors():
    lib = L.lib()
    d = base_dims()
    m = L.Model(FAKE, FAKE, FAKE, FAKE, FAKE)
    c = L.Cache(FAKE, None, FAKE, FAKE, FAKE, FAKE, None)
    need = P.workspace_bytes(d, L.OP_DECODE)
    tile = P.reuse_tile_bytes(d)
    assert tile == 128 * d.head_dim * 2                                  # 128 rebuilt keys, fp16

    def call(reuse, d_=d):
        return lib.lowram_decode_attn_reuse(ctypes.byref(d_), 0, ctypes.byref(m), ctypes.byref(c), FAKE, FAKE, FAKE,
                                            FAKE, None, ctypes.byref(reuse) if reuse is not None else None,
                                            None, FAKE, need, None)

    assert call(None) == L.E_INVALID
    assert call(L.Reuse(FAKE, FAKE, FAKE, FAKE, 0)) == L.E_INVALID         # no slots
    assert call(L.Reuse(FAKE, FAKE, FAKE, FAKE, 257)) == L.E_INVALID       # above the slot limit
    assert call(L.Reuse(None, FAKE, FAKE, FAKE, 8)) == L.E_INVALID
    assert call(L.Reuse(FAKE, FAKE, FAKE + 4, FAKE, 8)) == L.E_INVALID     # misaligned stamps
    other = P.with_(d, head_dim=64)                                          # not a chain shape
    assert call(L.Reuse(FAKE, FAKE, FAKE, FAKE, 8), d_=other) == L.E_UNSUPPORTED
    n = ctypes.c_size_t(0)
    assert lib.lowram_reuse_tile_bytes(ctypes.byref(other), ctypes.byref(n)) == L.E_UNSUPPORTED
    # the slot assignment stages at most 512 selected chunks in LDS: a larger
    # top-k on a chained shape is refused before anything is enqueued
    big = P.with_(d, n_ctx=1024 * d.chunk, top_k=513, n_res=0)
    assert P.decode_kernel(big) == "chain"
    need_big = P.workspace_bytes(big, L.OP_DECODE)
    st = lib.lowram_decode_attn_reuse(ctypes.byref(big), 0, ctypes.byref(m), ctypes.byref(c), FAKE, FAKE, FAKE,
                                      FAKE, None, ctypes.byref(L.Reuse(FAKE, FAKE, FAKE, FAKE, 8)), None, FAKE,
                                      need_big, None)
    assert st == L.E_UNSUPPORTED
    assert "512" in L.lib().lowram_last_error().decode()


def test_dense_argument_errors():
    lib = L.lib()
    d = P.with_(base_dims(), n_ctx=1000, chunk=7)   # the comparator ignores chunking
    need = P.workspace_bytes(d, L.OP_DENSE)
    assert need > 0
    ok_stride = d.heads_kv * 1000 * d.head_dim
    assert lib.lowram_dense_decode_attn(ctypes.byref(d), FAKE, FAKE, FAKE, 0, ok_stride, FAKE, FAKE, need, None) == L.E_INVALID
    assert lib.lowram_dense_decode_attn(ctypes.byref(P.with_(d, batch=2)), FAKE, FAKE, FAKE, 1000, 10, FAKE, FAKE, need, None) == L.E_INVALID


def test_status_strings():
    lib = L.lib()
    for s in range(5):
        assert lib.lowram_status_string(s)


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "decode_attention_compressed_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+(oracle|synth)\b", text, re.M), f
    ora = open(os.path.join(ROOT, "oracle", "lowram_oracle.py")).read()
    assert not re.search(r"^\s*(from|import)\s+(decode_attention_compressed_amd|synth|torch)\b", ora, re.M)


@pytest.mark.parametrize("name,path", [("tiny-fp32", "valu"), ("llama8b-32k", "chain"), ("mistral7b-16k", "chain"),
                                       ("qwen4b-64k", "absorb"), ("composed-int8-evict-128k", "chain")])
def test_decode_kernel_per_workload(name, path):
    from synth.configs import BY_NAME
    s = BY_NAME[name]
    # decode runs on the cache after eviction
    assert P.decode_kernel(dims_of(s, n_ctx=s.N_after)) == path


def test_decode_kernel_tail_only_and_errors():
    d = dims_of(TINY)
    assert P.decode_kernel(P.with_(d, top_k=0)) == "none"
    assert L.lib().lowram_decode_kernel(ctypes.byref(d), None) == L.E_INVALID


def _decode_ws_expected(s, n_part):
    """Decode workspace of the plan: selection, rank-block partial scores,
    summed scores, then n_part split partials per (b, h) of g (4 + F + dh) floats."""
    up = lambda x: (x + 255) // 256 * 256
    n_c, g, k = s.N // s.C, s.Hq // s.Hkv, min(s.k, s.N // s.C)
    nrb = (s.r + 63) // 64
    return (up(4 * s.B * s.Hkv * max(k, 1)) + up(8 * s.B * s.Hkv * nrb * n_c) + up(8 * s.B * s.Hkv * n_c)
            + up(4 * s.B * s.Hkv * n_part * g * (4 + s.F + s.dh)))


def test_decode_workspace_counts_the_partials_of_each_attend_kernel():
    up = lambda x: (x + 255) // 256 * 256
    # qwen4b-64k runs the absorbed kernel: 4 splits of 16 slices per (b, h) for
    # 256 workgroups over the four quarters of F, a chunk row and three tail rows
    # per split, then A = W1 U (fp16 [B][Hkv][F][r]) and q~ (fp16 hi/lo [B][Hkv][2][4][r])
    s = QWEN4B_64K
    assert P.decode_kernel(dims_of(s)) == "absorb"
    absorbed = up(2 * s.B * s.Hkv * s.F * s.r) + up(2 * s.B * s.Hkv * 2 * 4 * s.r)
    assert P.workspace_bytes(dims_of(s), L.OP_DECODE) == _decode_ws_expected(s, 4 * 4) + absorbed
    # eight query heads per kv head: the per-chunk matrix-core kernel, one partial
    # per selected chunk, each carrying a share of the tail (no separate tail
    # partial), then the select stage's logit operand: 16-bit hi/lo columns of
    # U^T q_g, [B][Hkv][2][16][r]
    s8 = QWEN4B_64K.replace(Hq=32)
    assert P.decode_kernel(dims_of(s8)) == "mfma"
    assert P.workspace_bytes(dims_of(s8), L.OP_DECODE) == (_decode_ws_expected(s8, s8.k)
                                                           + up(2 * s8.B * s8.Hkv * 2 * 16 * s8.r))
    # nothing selected: one tail partial per (b, h)
    d0 = P.with_(dims_of(s), top_k=0)
    assert P.workspace_bytes(d0, L.OP_DECODE) == _decode_ws_expected(s.replace(k=0), 1)
    # tiny-fp32 runs the vector kernel: one partial per token range of each
    # selected chunk (4 ranges of 16 tokens: 8 (b, h, chunk) units are far
    # below 256 workgroups) plus the tail's
    s = TINY
    assert P.workspace_bytes(dims_of(s), L.OP_DECODE) == _decode_ws_expected(s, 4 * s.k + 1)
    # with enough units (B = 64: 512) each chunk is one workgroup again
    s64 = TINY.replace(B=64)
    assert P.workspace_bytes(dims_of(s64), L.OP_DECODE) == _decode_ws_expected(s64, s64.k + 1)
