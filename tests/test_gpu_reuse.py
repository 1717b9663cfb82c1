"""GPU tests of reuse of rebuilt chunks across decode steps
(lowram_decode_attn_reuse).

A stream of correlated queries (successive steps tend to pick the same chunks)
runs through the plain decode and through the reuse path with a slot table.
At every step and layer:
- the outputs and selections are equal bit for bit (the operands read back
  are the bits the kernel computes);
- the hit counts and the table contents equal a host model of the documented
  slot policy.
With few slots the policy evicts and drops chunks, with many it keeps them all.
The plain decode itself is at parity with the oracle (test_gpu_parity); one
step here is also checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

from oracle import lowram_oracle as O
from synth import gen
from synth.configs import COMPOSED_128K, LLAMA8B_32K, small
from tests.harness import cache_to_host, dims_of, model_of, to_dev, to_host, upload, within_tol

pytestmark = pytest.mark.gpu

STEPS = 6
CASES = {
    "llama8b-small": small(LLAMA8B_32K, k=6, T=100),
    "composed-small": small(COMPOSED_128K, k=3, T=72),
    # 1024 chunks: the kernel reads the separate top-k's selection and stages
    # all of it for the slot assignment
    "chain-nc-1024": small(LLAMA8B_32K, B=1, Hq=8, Hkv=2, N=131072, T=16, k=9),
}


def P():
    import decode_attention_compressed_amd as pkg
    return pkg


class SlotModel:
    """Host model of the slot policy for one (b, l, h) table."""

    def __init__(self, slots):
        self.chunk = [-1] * slots
        self.stamp = [0] * slots
        self.clock = 0

    def step(self, sel):
        self.clock += 1
        t, used, hits, codes = self.clock, set(), 0, []
        for c in sel:
            if c in self.chunk:
                j = self.chunk.index(c)
                used.add(j)
                self.stamp[j] = t
                hits += 1
                codes.append(("hit", j))
            else:
                codes.append(None)
        for i, c in enumerate(sel):
            if codes[i] is not None:
                continue
            free = [j for j in range(len(self.chunk)) if j not in used]
            if not free:
                codes[i] = ("none", -1)
                continue
            j = min(free, key=lambda x: (self.stamp[x], x))
            used.add(j)
            self.chunk[j] = int(c)
            self.stamp[j] = t
            codes[i] = ("store", j)
        return hits


@pytest.fixture(scope="module", params=list(CASES))
def stream(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = CASES[request.param]
    print(f"\n[reuse case] {request.param}: {s}", flush=True)
    inp = gen.make(s)
    dev = upload(inp)
    d = dims_of(s)
    cache = P().alloc_cache(d)
    P().compress(d, model_of(dev), dev["k"], dev["v"], cache)
    if s.evict_keep < 1.0:
        cache, d, _ = P().evict(d, model_of(dev), cache, to_dev(inp["obs_q"]), s.keep_chunks)
    torch.cuda.synchronize()
    assert P().decode_kernel(d) == "chain", P().decode_kernel(d)
    qs = gen.make_correlated_queries(s, STEPS, rho=0.9)
    return dict(name=request.param, s=s, inp=inp, dev=dev, d=d, cache=cache, qs=qs, qdev=to_dev(qs, s.act))


@pytest.mark.parametrize("slots_per_k", [0.5, 1.0, 3.0])
def test_reuse_equals_plain_decode_and_the_slot_policy(stream, slots_per_k):
    s, d, dev, cache = stream["s"], stream["d"], stream["dev"], stream["cache"]
    k = P().k_eff(d)
    slots = max(1, int(slots_per_k * k))
    table = P().alloc_reuse(d, slots)
    models = {(b, l, h): SlotModel(slots) for b in range(s.B) for l in range(s.G) for h in range(s.Hkv)}
    total_hits = 0
    for st in range(STEPS):
        for l in range(s.G):
            q = stream["qdev"][st, l].contiguous()
            sel_a = torch.empty((s.B, s.Hkv, k), dtype=torch.int32, device="cuda")
            sel_b = torch.empty_like(sel_a)
            hits = torch.full((s.B, s.Hkv), -1, dtype=torch.int32, device="cuda")
            out_a = P().decode_attn(d, l, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], sel_out=sel_a)
            out_b = P().decode_attn_reuse(d, l, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], table,
                                          sel_out=sel_b, hits_out=hits)
            torch.cuda.synchronize()
            assert torch.equal(out_a, out_b), (st, l)
            assert torch.equal(sel_a, sel_b), (st, l)
            sel, hh = to_host(sel_b), to_host(hits)
            for b in range(s.B):
                for h in range(s.Hkv):
                    want = models[(b, l, h)].step([int(c) for c in sel[b, h]])
                    assert hh[b, h] == want, (st, l, b, h, hh[b, h], want)
                    total_hits += want
        chunk, _ = P().reuse_current(table)
        for (b, l, h), m in models.items():
            assert list(chunk[b, l, h]) == m.chunk, (st, b, l, h)
        assert np.all(to_host(table["clock"]) == st + 1)
    assert total_hits > 0  # correlated queries do revisit chunks


def test_reuse_step_matches_oracle(stream):
    s, d, dev, cache, inp = stream["s"], stream["d"], stream["dev"], stream["cache"], stream["inp"]
    table = P().alloc_reuse(d, 2 * P().k_eff(d))
    host = cache_to_host(cache)
    for st in range(2):  # the second call reads back what the first stored
        q = stream["qdev"][st, 0].contiguous()
        out = P().decode_attn_reuse(d, 0, model_of(dev), cache, q, dev["k_tail"], dev["v_tail"], table)
        torch.cuda.synchronize()
        want, _ = O.decode_layer(host, inp, s, 0, stream["qs"][st, 0], d.top_k, N=d.n_ctx)
        ok, worst = within_tol(out.float().cpu().numpy().astype(np.float64), want)
        assert ok, f"step {st}: worst |err|/tol {worst:.3f}"
