"""h2o_prefill_no_alloc, through the C ABI, against h2o_prefill_with_output and
h2o_prefill on the same prompts: two calls in a row on each ctx, the second
with a smaller prompt, must leave bit-identical outputs and cache states, and
the decode steps after them must agree bit for bit too."""
import pytest
import torch

from synth import WORKLOADS
from synth.stage import stage_decode, stage_prompt

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _state(c):
    # scores and positions everywhere; rows and row scales of live slots only
    live = c.pos >= 0
    st = [c.score, c.pos, c.k_slots.view(torch.uint8)[live], c.v_slots.view(torch.uint8)[live]]
    if c.k_scale is not None:
        st += [c.k_scale[live], c.v_scale[live]]
    return [x.clone() for x in st]


def _same(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name,cache_kind,prompts", [
    ("opt6.7b", "input", (512, 200)),
    ("opt6.7b", "e4m3", (512, 77)),
    # 3584 units x 1024 positions: 29.4 MB of the 32 MiB buffer
    ("opt30b", "input", (1024, 300)),
])
def test_no_alloc_prefill_equals_prefill(name, cache_kind, prompts):
    from kv_cache_eviction_02_amd import H2OCache
    wl = WORKLOADS[name]
    dtype = torch.bfloat16
    print(f"[no_alloc] {name} cache={cache_kind} prompts={prompts}", flush=True)
    ref = H2OCache(wl.batch, wl.heads, wl.head_dim, wl.recent, wl.heavy, max(prompts), dtype, wl.scale,
                   cache=cache_kind)
    # max_prompt = 0: h2o_create allocates no device memory for this ctx
    na = H2OCache(wl.batch, wl.heads, wl.head_dim, wl.recent, wl.heavy, 0, dtype, wl.scale, cache=cache_kind,
                  decode_split=1)
    for P in prompts:
        q, k, v = stage_prompt(wl, "cuda", prompt=P)
        o_ref = ref.prefill(q, k, v, output=True)
        o_na = na.prefill(q, k, v, output=True, no_alloc=True)
        torch.cuda.synchronize()
        assert torch.equal(o_ref, o_na)
        _same(_state(ref), _state(na))
        assert ref.position() == na.position() == (P, min(P, wl.k))
        ref.prefill(q, k, v)
        na.prefill(q, k, v, no_alloc=True)
        _same(_state(ref), _state(na))
        # the ctx decodes on from the state the no-allocation prefill left
        dq, dk, dv = stage_decode(wl, 0, 3, "cuda", prompt=P)
        for s in range(3):
            a = [x.clone() for x in ref.step(dq[s], dk[s], dv[s])]
            b = [x.clone() for x in na.step(dq[s], dk[s], dv[s])]
            _same(a, b)
        _same(_state(ref), _state(na))
        del q, k, v, o_ref, o_na
    ref.close()
    na.close()
