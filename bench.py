"""Benchmark of the compressed-KV decode step on one MI355X.

One step = one new query per sequence through every layer of an xKV group
(G lowram_decode_attn calls: chunk select, rebuild-and-attend, combine) on the
Llama-3.1-8B-shaped workload: B=4, 32 q / 8 kv heads, d_h=128, 4-layer group,
rank 512, predictor 128-256-128, residuals on 12.5% of tokens, 32K context,
chunks of 128, top-32 chunks, 128-token uncompressed tail, bf16.  Inputs are
seeded synthetic data resident in HBM before the timed region.

Prints one JSON line: seq-steps/s, the roofline of the rebuild-and-attend
kernel (HIP events on its stream), the dense bf16 comparator on the same
queries (x vs dense), and the CPU oracle on a bounded sample.  After the
decode step it also times, outside the headline: the tail re-pack, the
predictor fit, the key basis, and (with --reuse) reuse of rebuilt chunks on
correlated queries; then the other workloads of the method's configurations
(tiny fp32, Mistral-7B-shaped at B = 16 and 64, Qwen-4B-shaped d_h = 256, and
the composed int8 + eviction case), each with its step time, attend kernel,
dense comparator and compression ratio under "other_workloads" (--configs
none skips them).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
CSRC = os.path.join(ROOT, "decode_attention_compressed_amd", "csrc")
# the source file of each attend kernel (its code hash keys the stored counters)
ATTEND_SRC = {"chain": "k_attend_chain.hip", "absorb": "k_attend_absorb.hip", "mfma": "k_attend_mfma.hip",
              "valu": "k_decode.hip"}


# the other workloads of the method's configurations, timed after the headline
DEFAULT_CONFIGS = "tiny-fp32,mistral7b-16k:16,mistral7b-16k:64,qwen4b-64k,composed-int8-evict-128k"


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", "attend_traffic_" + workload.replace("-", "_") + ".json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama8b-32k")
    ap.add_argument("--batch", type=int, default=0, help="override the batch (e.g. 16/32/64 for mistral7b-16k)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle leg")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches (for counter runs)")
    ap.add_argument("--no-fit", action="store_true", help="skip timing the predictor fit")
    ap.add_argument("--fit-steps", type=int, default=4)
    ap.add_argument("--no-basis", action="store_true", help="skip timing the key basis")
    ap.add_argument("--basis-iterations", type=int, default=8)
    ap.add_argument("--reuse", action="store_true",
                    help="also time reuse of rebuilt chunks (lowram_decode_attn_reuse, off the default decode path)")
    ap.add_argument("--no-reuse", action="store_true", help="(the default) do not time reuse")
    ap.add_argument("--reuse-rho", type=float, default=0.95, help="step-to-step query correlation for the reuse timing")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times: a kernel of known "
                         "traffic that scales hardware byte counters")
    ap.add_argument("--configs", default=DEFAULT_CONFIGS,
                    help="comma-separated workload[:batch] list timed after the headline ('none' skips): "
                         "each gets its step time, attend kernel, dense comparator and compression ratio")
    ap.add_argument("--config-steps", type=int, default=16, help="timed steps per other workload")
    ap.add_argument("--bw-probe", action="store_true",
                    help="only report the HBM bandwidth torch's own reduction and copy kernels reach "
                         "on 2 GiB (what a plain streaming kernel attains on this GPU), then exit")
    return ap.parse_args()


def bw_probe():
    """Read (sum) and read+write (copy) bandwidth of torch's own kernels over a
    2 GiB bf16 buffer, eager, 10 launches each after 3 untimed ones."""
    import torch
    x = torch.ones((2 << 30) // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        x.sum()
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn, nbytes in (("sum_read", lambda: x.sum(), x.numel() * 2),
                             ("copy_read_write", lambda: y.copy_(x), 2 * x.numel() * 2)):
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 10 * 1e-3
        res[name + "_gbps"] = round(nbytes / t / 1e9, 1)
    print(json.dumps({"bw_probe": res, "hbm_peak_gbps": HBM_PEAK_GBPS}))


def attend_accounting(s, sel, res_ptr, layer, kernel="chain"):
    """Algorithmic HBM bytes and FLOPs of one rebuild-and-attend launch.

    bytes: the union over kv heads of the selected coefficient tiles (each
    read once per sequence), the layer's basis slice and first predictor
    layer, residual rows (+int32 index) and CSR pointers of the selected
    chunks, the layer's tail K/V, the queries and the chunk scores the kernel
    ranks for its own top-k.  The absorbed kernel (head dim 256) reads the
    first layer in its absorbed form A = W1 U_{l,h} (F r values) and q~ (g r)
    in place of the basis slice and W1, and its selection comes from the
    separate top-k (no scores read).
    flops: per selected token-head the cheaper exact form of the product
    chain: 2(d_h r + F d_h + g d_h + g F) (rebuilt key, hidden layer, logits,
    p-weighted hidden sum) or, absorbed, 2(F r + g r + g F); plus the tail's
    4 T d_h per query head."""
    B, Hkv, C, r, dh, F, T = s.B, s.Hkv, s.C, s.r, s.dh, s.F, s.T
    sa, sc, sr = 2, (1 if s.coeff == "i8" else 2), (1 if s.resid == "i8" else 2)
    g = s.Hq // Hkv
    union = sum(len(np.unique(sel[b])) for b in range(B))
    nbytes = union * C * r * sc
    if s.coeff == "i8":
        nbytes += B * r * 2
    if kernel == "absorb":
        nbytes += B * Hkv * (F * r + 2 * 4 * r) * sa + B * Hkv * F * sa
    else:
        nbytes += B * Hkv * dh * r * sa + B * Hkv * (F * dh + F) * sa
    rows = 0
    for b in range(B):
        for h in range(Hkv):
            p = res_ptr[b, layer, h]
            rows += int(np.sum(p[sel[b, h] + 1] - p[sel[b, h]]))
    nbytes += rows * (dh * sr + 4) + B * Hkv * sel.shape[-1] * 8
    if s.resid == "i8":
        nbytes += B * Hkv * dh * 2
    nbytes += 2 * B * Hkv * T * dh * sa + B * s.Hq * dh * sa
    if kernel == "chain":
        nbytes += B * Hkv * (s.N_after // C) * 8
    per_tok = min(dh * r + F * dh + g * dh + g * F, F * r + g * r + g * F)
    flops = B * Hkv * sel.shape[-1] * C * 2 * per_tok + B * s.Hq * T * dh * 4
    return nbytes, flops, union


def step_bytes(s, attend_b):
    """Whole-step extras beyond the attend kernel: landmarks read by the
    scorer, basis slice read by the scorer, W2/b2 and partial-free output."""
    B, Hkv, dh, r, F = s.B, s.Hkv, s.dh, s.r, s.F
    n_c = s.N_after // s.C
    return attend_b + B * n_c * r * 4 + B * Hkv * dh * r * 2 + B * Hkv * (dh * F + dh) * 2 + B * s.Hq * dh * 2


def kernel_code_hash(path):
    """sha256 of a source file's code: comment lines and blank lines left out,
    so that the counters stay valid across edits of comments only."""
    keep = []
    for line in open(path, encoding="utf-8"):
        s = line.strip()
        if s and not s.startswith("//"):
            keep.append(line.rstrip())
    return hashlib.sha256("\n".join(keep).encode()).hexdigest()


def traffic_for_current_kernel(workload, kern):
    """HBM bytes per attend launch measured by rocprofv3 counters for this
    workload, if they were taken on the current source of its attend kernel."""
    path = traffic_file(workload)
    if kern not in ATTEND_SRC or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("workload") != workload or t.get("kernel_sha256") != kernel_code_hash(os.path.join(CSRC, ATTEND_SRC[kern])):
        return None
    return t.get("bytes_per_launch")


def repack_bytes(s, d, live_rows, m):
    """Algorithmic HBM bytes of one re-pack call: the existing cache read once and
    written once into the grown cache, plus the new chunk (C tail tokens of K and
    V, the basis, the predictor, and the rows it writes)."""
    cb = 1 if s.coeff == "i8" else (4 if s.act == "f32" else 2)
    rb = s.dh * (1 if s.resid == "i8" else (4 if s.act == "f32" else 2))
    ab = 4 if s.act == "f32" else 2
    N, C, n_c, lh = d.n_ctx, s.C, d.n_ctx // s.C, s.G * s.Hkv
    old = N * s.r * cb + n_c * s.r * 4 + live_rows * (rb + 4) + lh * (n_c + 1) * 4
    new = (2 * lh * C * s.dh * ab + s.D * s.r * ab + lh * (2 * s.F * s.dh + s.F + s.dh) * ab
           + C * s.r * cb + s.r * 4 + lh * m * (rb + 4) + lh * 4)
    return s.B * (2 * old + new)


def time_repack(P, s, d, model, cache, dev, ev, reps=5):
    """Time lowram_repack (oldest C tail tokens -> one new chunk) on this cache."""
    import torch
    if d.n_tail < s.C:
        return None
    m = min(s.C, int(math.ceil(s.rho * s.C - 1e-9)))
    d2 = P.with_(d, n_ctx=d.n_ctx + s.C, n_res=d.n_res + m, n_tail=d.n_tail - s.C)
    dst = P.alloc_cache(d2)
    for name in ("coeff_scale", "res_scale"):
        if name in cache:
            dst[name] = cache[name]
    ws = P.workspace(d, P._lib.OP_REPACK)
    P.repack(d, model, cache, dev["k_tail"], dev["v_tail"], m, dst=dst, ws=ws)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        P.repack(d, model, cache, dev["k_tail"], dev["v_tail"], m, dst=dst, ws=ws)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    live = int(cache["res_ptr"][..., -1].sum().item()) // s.B
    nbytes = repack_bytes(s, d, live, m)
    del dst, ws
    log(f"repack {us:.1f} us/call ({us / s.C:.2f} us per decode step amortised over C = {s.C})")
    return {"us_per_call": round(us, 1), "amortised_us_per_step": round(us / s.C, 3), "new_res_rows": m,
            "algorithmic_bytes": int(nbytes), "hbm_gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "how": f"{reps} eager calls between HIP events; once per C decode steps"}


def time_fit(P, s, d, model, dev, ev, steps=4, lr=0.01):
    """Time lowram_fit_predictor (gradient descent on the prefill, once per
    context) into side buffers; the benchmarked predictor is left as it is."""
    import torch
    Z = s.B * s.G * s.Hkv
    flops = Z * (steps * 10 * s.N * s.F * s.dh + 4 * s.N * s.F * s.dh + 2 * s.N * s.r * s.dh)
    ws = P.workspace(d, P._lib.OP_FIT)
    out, loss = P.fit_predictor(d, model, dev["k"], dev["v"], 0, lr, ws=ws)  # warm-up
    torch.cuda.synchronize()
    ev[0].record()
    out, loss = P.fit_predictor(d, model, dev["k"], dev["v"], steps, lr, out=out, ws=ws)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    L = loss.cpu().numpy()
    tf = flops / (ms * 1e-3) / 1e12
    ws_gb = ws.numel() / 1e9
    del ws, out
    torch.cuda.empty_cache()
    log(f"fit {steps} steps in {ms:.1f} ms ({tf:.1f} TFLOP/s fp32), loss {L[..., 0].mean():.4f} -> {L[..., -1].mean():.4f}")
    return {"steps": steps, "lr": lr, "ms": round(ms, 2), "algorithmic_flops": int(flops),
            "tflops": round(tf, 2), "bound": "mfma", "peak_tflops": FP32_PEAK_TFLOPS,
            "frac": round(tf / FP32_PEAK_TFLOPS, 4), "workspace_gb": round(ws_gb, 2),
            "loss_first_mean": round(float(L[..., 0].mean()), 5), "loss_last_mean": round(float(L[..., -1].mean()), 5),
            "how": "one call between HIP events after a zero-step warm-up; float32 products on the matrix cores "
                   "(v_mfma_f32_16x16x4_f32, the fp32 peak), bound by the traffic of their fp32 activations"}


def time_basis(P, s, d, dev, ev, iterations=8):
    """Time lowram_key_basis on the prefill keys (once per context) and report
    how much key energy its basis leaves out next to the basis the inputs carry."""
    import torch
    D = s.G * s.Hkv * s.dh
    flops = s.B * (s.N * D * D + iterations * 2 * s.r * D * D)   # upper-triangle Gram + G Q products
    ws = P.workspace(d, P._lib.OP_BASIS)
    out = P.key_basis(d, dev["k"], 0, ws=ws)  # warm-up
    torch.cuda.synchronize()
    ev[0].record()
    out = P.key_basis(d, dev["k"], iterations, out=out, ws=ws)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    tf = flops / (ms * 1e-3) / 1e12
    # energy outside span(U) on a sample of tokens, for the GPU basis and the given one
    n = min(s.N, 4096)
    kc = dev["k"][:, :, :, :n].float().permute(0, 3, 1, 2, 4).reshape(s.B, n, D)
    def resid(U):
        U = U.float()
        rec = (kc @ U) @ U.transpose(1, 2)
        return float(((kc - rec) ** 2).sum() / (kc ** 2).sum())
    r_gpu, r_given = resid(out), resid(dev["basis"])
    del ws, out, kc
    torch.cuda.empty_cache()
    log(f"basis {iterations} iterations in {ms:.1f} ms ({tf:.1f} TFLOP/s fp32), residual energy {r_gpu:.2e} (given basis {r_given:.2e})")
    return {"iterations": iterations, "ms": round(ms, 2), "algorithmic_flops": int(flops), "tflops": round(tf, 2),
            "bound": "mfma", "peak_tflops": FP32_PEAK_TFLOPS, "frac": round(tf / FP32_PEAK_TFLOPS, 4),
            "residual_energy": r_gpu, "residual_energy_given_basis": r_given, "sample_tokens": n,
            "how": "one call between HIP events after a zero-iteration warm-up; fp32 products on the matrix cores "
                   "against the fp32 peak (the Gram matrix of bf16 keys on bf16 matrix cores, fp32 sums)"}


def time_reuse(P, s, d, model, cache, dev, rho=0.95, steps=32, slots_per_k=2):
    """Decode steps on a stream of correlated queries, plain and with reuse of
    rebuilt chunks (slot table of slots_per_k * k chunks per head), each
    captured in one HIP graph and replayed after a warm-up replay."""
    import torch
    from synth import gen
    from tests.harness import to_dev
    if P.decode_kernel(d) != "chain":
        return None
    k = P.k_eff(d)
    qs = to_dev(gen.make_correlated_queries(s, steps, rho), s.act)
    table = P.alloc_reuse(d, slots_per_k * k)
    ws = P.workspace(d, P._lib.OP_DECODE)
    out = torch.empty((s.B, s.Hq, s.dh), dtype=qs.dtype, device="cuda")
    hits = torch.zeros((steps, s.G, s.B, s.Hkv), dtype=torch.int32, device="cuda")

    def run(use_reuse):
        for st in range(steps):
            for l in range(s.G):
                q = qs[st, l]
                if use_reuse:
                    P.decode_attn_reuse(d, l, model, cache, q, dev["k_tail"], dev["v_tail"], table, out=out,
                                        hits_out=hits[st, l], ws=ws)
                else:
                    P.decode_attn(d, l, model, cache, q, dev["k_tail"], dev["v_tail"], out=out, ws=ws)

    res = {}
    for name, flag in (("plain", False), ("reuse", True)):
        run(flag)  # eager warm-up (fills the table)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(flag)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / steps
        del g
    hit_rate = float(hits.sum().item()) / (steps * s.G * s.B * s.Hkv * k)
    del table, ws
    torch.cuda.empty_cache()
    log(f"reuse rho {rho}: plain {res['plain']:.1f} us/step, reuse {res['reuse']:.1f} us/step, hit rate {hit_rate:.3f}")
    return {"rho": rho, "slots": slots_per_k * k, "steps": steps, "hit_rate": round(hit_rate, 4),
            "us_per_step_plain": round(res["plain"], 1), "us_per_step_reuse": round(res["reuse"], 1),
            "speedup": round(res["plain"] / res["reuse"], 3),
            "how": "correlated queries q_s = rho q_(s-1) + sqrt(1 - rho^2) xi; both paths captured in one HIP graph "
                   "each; the step time includes the reuse path's separate selection and slot kernels"}


def cpu_baseline(s, host, inp, budget_s):
    from oracle import lowram_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    steps = 0
    while True:
        for layer in range(s.G):
            O.decode_layer(host, inp, s, layer, inp["q"][steps % inp["q"].shape[0], layer], s.k, N=s.N_after)
        steps += 1
        if time.perf_counter() - t0 >= budget_s or steps >= 8:
            break
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    out = {"value": s.B * steps / dt, "unit": "seq-steps/s", "cores": int(threads), "kind": "oracle",
           "cpu_model": model,
           "sample": f"{steps} full decode step(s) ({s.G} layers x B={s.B}) of the {s.name} workload, "
                     f"float64 numpy oracle, {dt:.1f} s"}
    try:  # the same oracle on one thread: one layer call of the same workload
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            O.decode_layer(host, inp, s, 0, inp["q"][0, 0], s.k, N=s.N_after)
            d1 = time.perf_counter() - t1
        out["single_thread"] = {"value": s.B / (s.G * d1), "unit": "seq-steps/s", "cores": 1,
                                "sample": f"one layer call (B={s.B}), {d1:.2f} s, scaled to a {s.G}-layer step"}
    except Exception as e:  # pragma: no cover
        out["single_thread"] = {"value": None, "error": str(e)}
    return out


class Workload:
    """One workload on the GPU: inputs drawn and uploaded, the cache compressed
    (and evicted where the workload evicts), and pre-marshalled decode calls for
    n_q query sets."""

    def __init__(self, P, s, n_q, quiet=False):
        import torch
        from synth import gen
        from tests.harness import dims_of, model_of, to_dev, upload
        from decode_attention_compressed_amd.api import TORCH_DT

        self.s, self.n_q = s, n_q
        t0 = time.perf_counter()

        def gen_progress(done, total):  # large batches take a while to draw on the host
            if not quiet and total >= 16 and (done % 8 == 0 or done == total):
                log(f"generated {done}/{total} sequences")
        self.inp = gen.make(s, steps=n_q, progress=gen_progress)
        self.gen_s = time.perf_counter() - t0
        log(f"{s.name} B={s.B}: generated inputs in {self.gen_s:.1f} s")
        self.dev = dev = upload(self.inp)
        self.d = d = dims_of(s)
        self.model = model = model_of(dev)
        self.cache = P.alloc_cache(d)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        P.compress(d, model, dev["k"], dev["v"], self.cache)
        ev[1].record()
        torch.cuda.synchronize()
        self.compress_ms = ev[0].elapsed_time(ev[1])
        log(f"compress {self.compress_ms:.1f} ms")
        self.comp_bytes, self.dense_bytes = P.cache_bytes(dims_of(s))   # as compressed, before any eviction
        self.evicted = None
        if s.evict_keep < 1.0:
            self.cache, self.d, _ = P.evict(d, model, self.cache, to_dev(self.inp["obs_q"]), s.keep_chunks)
            d = self.d
            torch.cuda.synchronize()
            # against the dense bf16 cache of all s.N tokens: the evicted cache as
            # allocated (every head sized to the largest head's kept rows), and by
            # the rows the kept chunks actually hold
            comp_ev, _ = P.cache_bytes(d)
            live = float(self.cache["res_ptr"][..., -1].sum().item()) / s.B
            row_b = s.dh * (1 if s.resid == "i8" else 2) + 4
            comp_live = comp_ev - (s.G * s.Hkv * d.n_res - live) * row_b
            self.evicted = {
                "n_ctx": d.n_ctx, "res_rows_capacity": d.n_res, "res_rows_live_per_seq": live,
                "compressed_bytes_per_seq": comp_ev, "ratio_vs_dense_bf16": round(self.dense_bytes / comp_ev, 2),
                "ratio_vs_dense_bf16_live_rows": round(self.dense_bytes / comp_live, 2),
                "dense_bytes_per_seq": self.dense_bytes,
                "how": f"dense = M_KV of the {s.N}-token context in bf16; compressed = the evicted cache "
                       f"({d.n_ctx} tokens) with its residual arrays as allocated, or counting live rows only"}
            log(f"evicted cache: {self.evicted['ratio_vs_dense_bf16']}x as allocated, "
                f"{self.evicted['ratio_vs_dense_bf16_live_rows']}x by live rows")
        kk = P.k_eff(d)
        self.ws = P.workspace(d, P._lib.OP_DECODE)
        self.out = torch.empty((s.B, s.Hq, s.dh), dtype=TORCH_DT[d.act], device="cuda")
        self.sels = [[torch.empty((s.B, s.Hkv, kk), dtype=torch.int32, device="cuda") for _ in range(s.G)]
                     for _ in range(n_q)]
        self.calls = [[P.DecodeCall(d, l, model, self.cache, dev["q"][i, l], dev["k_tail"], dev["v_tail"],
                                    self.out, self.ws, self.sels[i][l]) for l in range(s.G)] for i in range(n_q)]

    def step(self, i):
        for c in self.calls[i % self.n_q]:
            c()


def time_steps(W, steps, warmup, use_graph=True):
    """Mean step time (ms) of `steps` decode steps: captured in one HIP graph
    and replayed (eager launches if capture is off or fails).  Returns
    (ms per step, the graph or None)."""
    import torch
    for i in range(warmup):
        W.step(i)
    torch.cuda.synchronize()
    graph = None
    try:
        if not use_graph:
            raise RuntimeError("disabled by --no-graph")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                W.step(i)
        graph.replay()
        torch.cuda.synchronize()
    except Exception as e:  # capture unsupported: time eager launches instead
        log(f"graph capture failed ({e}); timing eager launches")
        graph = None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(steps):
            W.step(i)
    ev[1].record()
    torch.cuda.synchronize()
    ms_step = ev[0].elapsed_time(ev[1]) / steps
    log(f"{W.s.name}: {steps} steps -> {ms_step * 1e3:.1f} us/step (graph={graph is not None})")
    return ms_step, graph


def step_distribution(W, steps):
    """p50/p90 of single steps: a one-step graph replayed with HIP events around
    each replay (each figure includes one replay launch)."""
    import torch
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        W.step(0)
    g1.replay()
    torch.cuda.synchronize()
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a_, b_ in pev:
        a_.record()
        g1.replay()
        b_.record()
    torch.cuda.synchronize()
    per = np.array([a_.elapsed_time(b_) for a_, b_ in pev]) * 1e3
    dist = {"us_p50": round(float(np.median(per)), 1), "us_p90": round(float(np.percentile(per, 90)), 1),
            "us_min": round(float(per.min()), 1), "n": int(per.size),
            "how": "one-step graph replayed with HIP events around each replay (adds the replay launch)"}
    log(f"per-step: p50 {dist['us_p50']} us, p90 {dist['us_p90']} us")
    del g1
    return dist


def time_attend(P, W, n_time):
    """The rebuild-and-attend kernel alone: HIP events on its stream around each
    attend launch of n_time steps (select and combine run outside the events),
    against its algorithmic bytes and FLOPs.  Returns (roofline dict, bytes per
    launch, union of selected chunks per sequence)."""
    import torch
    from tests.harness import to_host
    s, d = W.s, W.d
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_time * s.G)]
    k = 0
    for i in range(n_time):
        for c in W.calls[i]:
            c.select()
            evs[k][0].record(stream)
            c.attend()
            evs[k][1].record(stream)
            c.combine()
            k += 1
    torch.cuda.synchronize()
    attend_ms = np.array([a.elapsed_time(b) for a, b in evs])
    host_ptr = to_host(W.cache["res_ptr"])
    kern = P.decode_kernel(d)
    acc = [attend_accounting(s, to_host(W.sels[i][l]), host_ptr, l, kern) for i in range(n_time) for l in range(s.G)]
    a_bytes = np.mean([a[0] for a in acc])
    a_flops = np.mean([a[1] for a in acc])
    union = np.mean([a[2] for a in acc]) / s.B
    t_attend = attend_ms.mean() * 1e-3
    gbps = a_bytes / t_attend / 1e9
    tflops = a_flops / t_attend / 1e12
    t_hbm, t_mfma = a_bytes / (HBM_PEAK_GBPS * 1e9), a_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = traffic_for_current_kernel(s.name, kern)
    kname = {"chain": "k_attend_chain (top-k + rebuild-and-attend)", "mfma": "k_attend_mfma (rebuild-and-attend)",
             "absorb": "k_attend_absorb (absorbed first layer; A = W1 U formed with the selection)",
             "valu": "k_attend_valu (rebuild-and-attend)", "none": "tail only"}[kern]
    roof.update({"kernel": kname, "avg_launch_us": round(t_attend * 1e6, 2),
                 "algorithmic_bytes_per_launch": int(a_bytes), "algorithmic_flops_per_launch": int(a_flops),
                 "mfma_tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                 "hbm_gbps": round(gbps, 1), "roof_time_us": round(max(t_hbm, t_mfma) * 1e6, 2),
                 "frac_of_binding_roof": round(max(t_hbm, t_mfma) / t_attend, 4)})
    log(f"attend {t_attend * 1e6:.1f} us/launch, {gbps:.0f} GB/s, {tflops:.1f} TF/s, union {union:.1f} chunks/seq")
    return roof, a_bytes, union


def time_dense(P, W, steps, use_graph):
    """The dense bf16 comparator on the same queries, timed like the compressed
    step: `steps` steps of G layer calls captured in one HIP graph."""
    import torch
    s, d, dev = W.s, W.d, W.dev
    kd = torch.cat([dev["k"], dev["k_tail"]], dim=3).contiguous()
    vd = torch.cat([dev["v"], dev["v_tail"]], dim=3).contiguous()
    dws = P.dense_workspace(d, kd.shape[3])
    dout = torch.empty_like(W.out)

    def dense_step(i):
        for l in range(s.G):
            P.dense_decode_attn(d, dev["q"][i % W.n_q, l], kd, vd, l, out=dout, ws=dws)

    for i in range(2):
        dense_step(i)
    torch.cuda.synchronize()
    dgraph = None
    if use_graph:
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph):
            for i in range(steps):
                dense_step(i)
        dgraph.replay()
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    if dgraph is not None:
        dgraph.replay()
    else:
        for i in range(steps):
            dense_step(i)
    ev[1].record()
    torch.cuda.synchronize()
    dense_ms = ev[0].elapsed_time(ev[1]) / steps
    dense_bytes_step = 2 * s.B * s.G * s.Hkv * kd.shape[3] * s.dh * 2 + 2 * s.B * s.G * s.Hq * s.dh * 2
    ideal_ms = dense_bytes_step / (HBM_PEAK_GBPS * 1e9) * 1e3
    gb = dense_bytes_step / (dense_ms * 1e-3) / 1e9
    log(f"dense {dense_ms * 1e3:.1f} us/step, {gb:.0f} GB/s ({gb / HBM_PEAK_GBPS:.1%} of HBM peak)")
    how = "captured in one HIP graph like the compressed step" if dgraph is not None else "eager launches"
    del kd, vd, dgraph, dws, dout
    torch.cuda.empty_cache()
    return {"ms_per_step": round(dense_ms, 4), "hbm_gbps": round(gb, 1),
            "hbm_frac": round(gb / HBM_PEAK_GBPS, 4), "ideal_ms_per_step": round(ideal_ms, 4),
            "kernel": "k_dense_mfma (bf16 split-K) + combine, " + how}


def other_workloads(P, spec, steps, warmup, use_graph):
    """The other workloads of the method's configurations, each in the same
    launch configuration as the headline (HIP-graph-timed steps, attend kernel
    events, dense comparator): one compact record per (workload, batch)."""
    import torch
    from synth.configs import BY_NAME
    rows = []
    for item in spec:
        name, _, batch = item.partition(":")
        s = BY_NAME[name]
        if batch:
            s = s.replace(B=int(batch))
        W = Workload(P, s, n_q=min(steps, 16), quiet=True)
        ms_step, graph = time_steps(W, steps, warmup, use_graph)
        roof, _, union = time_attend(P, W, min(steps, W.n_q))
        del graph
        dense = time_dense(P, W, steps, use_graph)
        row = {"workload": s.name, "B": s.B, "us_per_step": round(ms_step * 1e3, 1),
               "seq_steps_per_s": round(s.B / (ms_step * 1e-3), 1), "attend_kernel": P.decode_kernel(W.d),
               "attend_us": roof["avg_launch_us"], "attend_bound": roof["bound"],
               "attend_frac_of_binding_roof": roof["frac_of_binding_roof"],
               "attend_hbm_frac": round(roof["hbm_gbps"] / HBM_PEAK_GBPS, 4), "attend_mfma_frac": roof["mfma_frac"],
               "dense_us_per_step": round(dense["ms_per_step"] * 1e3, 1), "dense_hbm_frac": dense["hbm_frac"],
               "x_vs_dense": round(dense["ms_per_step"] / ms_step, 3),
               "compression_ratio": round(W.dense_bytes / W.comp_bytes, 3),
               "selected_chunk_union_per_seq": round(float(union), 1), "gen_s": round(W.gen_s, 1)}
        if W.evicted:
            row["ratio_after_eviction"] = W.evicted["ratio_vs_dense_bf16"]
            row["ratio_after_eviction_live_rows"] = W.evicted["ratio_vs_dense_bf16_live_rows"]
        log(f"{s.name} B={s.B}: {row['us_per_step']} us/step, {row['x_vs_dense']}x vs dense")
        rows.append(row)
        del W
        torch.cuda.empty_cache()
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path shards over "
              "sequences with no exchange, so N GPUs run N independent copies).", file=sys.stderr)
        sys.exit(2)
    if args.bw_probe:
        bw_probe()
        return
    import torch

    import decode_attention_compressed_amd as P
    from synth.configs import BY_NAME
    from tests.harness import cache_to_host, dims_of

    s = BY_NAME[args.workload]
    if args.batch:
        s = s.replace(B=args.batch)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev_name = torch.cuda.get_device_name(0)
    log(f"workload {s.name}: {s}")
    n_q = min(64, max(args.steps, 1))
    W = Workload(P, s, n_q)
    d, model, cache, dev, inp = W.d, W.model, W.cache, W.dev, W.inp
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    # ---- timed region: K steps captured in one HIP graph -------------------
    ms_step, graph = time_steps(W, args.steps, args.warmup, use_graph=not args.no_graph)
    graph_used = graph is not None
    step_dist = step_distribution(W, args.steps) if graph_used else None
    del graph

    # ---- attend-kernel timing with events on its stream ------------------------
    roof, a_bytes, union = time_attend(P, W, min(args.steps, n_q))

    # ---- dense comparator on the same queries, timed like the compressed step
    dense = None if args.no_dense else time_dense(P, W, args.steps, use_graph=graph_used)

    # ---- once-per-context and optional paths, timed after the decode step ------
    repack = time_repack(P, s, d, model, cache, dev, ev)
    fit = None if args.no_fit else time_fit(P, s, dims_of(s), model, dev, ev, steps=args.fit_steps)
    basis = None if args.no_basis else time_basis(P, s, dims_of(s), dev, ev, iterations=args.basis_iterations)
    reuse = time_reuse(P, s, d, model, cache, dev, rho=args.reuse_rho) if args.reuse and not args.no_reuse else None

    # ---- CPU oracle on a bounded sample ---------------------------------------
    cpu = None
    if not args.no_cpu:
        host = cache_to_host(cache)
        cpu = cpu_baseline(s, host, inp, args.cpu_seconds)
        log(f"cpu oracle {cpu['value']:.3f} seq-steps/s on {cpu['cores']} threads, "
            f"{cpu['single_thread'].get('value') or 0:.3f} on one")

    if args.copy_ref_mib:
        src = torch.ones((args.copy_ref_mib << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):  # an elementwise kernel: reads and writes the buffer once each
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"copy reference: 3 x {args.copy_ref_mib} MiB")
        del src, dst

    # ---- the other workloads, after the headline's own figures ------------------
    step_b = step_bytes(s, a_bytes) * s.G
    comp_bytes, dense_bytes, evicted, compress_ms = W.comp_bytes, W.dense_bytes, W.evicted, W.compress_ms
    del W, d, model, cache, dev, inp
    torch.cuda.empty_cache()
    spec = [] if args.configs in ("", "none") else args.configs.split(",")
    others = other_workloads(P, spec, args.config_steps, 4, use_graph=not args.no_graph) if spec else None

    result = {
        "metric": "decode-attn seq-steps/s and HBM GB/s (% peak) at Llama-8B shape 32K; x vs dense",
        "value": round(s.B / (ms_step * 1e-3), 1),
        "unit": "seq-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16"}[s.act],
        "data": "synthetic (seeded spectrum-decayed keys, MLP+Student-t values, N(0,1) queries)",
        "config": {"workload": s.name, "B": s.B, "G": s.G, "Hq": s.Hq, "Hkv": s.Hkv, "dh": s.dh,
                   "r": s.r, "F": s.F, "N": s.N_after, "C": s.C, "top_k": s.k, "T": s.T,
                   "rho": s.rho, "coeff": s.coeff, "resid": s.resid, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_hbm_gbps": round(step_b / (ms_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_b / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "x_vs_dense": round(dense["ms_per_step"] / ms_step, 3) if dense else None,
        "x_vs_dense_at_hbm_peak": round(dense["ideal_ms_per_step"] / ms_step, 3) if dense else None,
        "dense": dense,
        "compression_ratio": round(dense_bytes / comp_bytes, 3),
        "evicted": evicted,
        "selected_chunk_union_per_seq": round(float(union), 1),
        "compress_ms": round(compress_ms, 2),
        "repack": repack,
        "fit": fit,
        "basis": basis,
        "reuse": reuse,
        "step_time_distribution": step_dist,
        "graph": graph_used,
        "other_workloads": others,
        "device": dev_name,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
