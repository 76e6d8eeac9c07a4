"""The whole layer (route -> align -> gate/up -> down -> combine) captured as one
HIP graph: every replay equals the eager call bit for bit, with eager work and
synchronisations between the replays, and a replay after the inputs are
updated in place follows the new inputs.  Small-batch and large-batch kernels,
int8 per-column and int4 act-order weights."""
import pytest

import gen
import weight_only_quantized_topk_amd as wq
from tests.gpu_common import dev_u16, need_gpu, say, torch

pytestmark = pytest.mark.gpu

W8 = gen.CFG2.with_(name="w8-graph", E=8, topk=2, K=512, N=384)
W4AO = gen.CFG3.with_(name="w4ao-graph", E=8, topk=2, K=512, N=384)
SPECS = {"w8": (W8, 520), "w4ao": (W4AO, 521)}
_packed = {}


def packed(key):
    if key not in _packed:
        spec, seed = SPECS[key]
        wts = gen.make_moe_weights(spec, seed_config=seed)
        act = torch.float16 if spec.act == "f16" else torch.bfloat16
        _packed[key] = (spec, wq.pack_moe(spec.bits, wts.w1q, wts.s1, wts.w2q, wts.s2, act, spec.group_size,
                                          wts.g1, wts.g2))
    return _packed[key]


def inputs(spec, M, seed):
    toks = gen.make_tokens(spec, M, seed_config=seed)
    return dev_u16(toks.x, spec.act), torch.from_numpy(toks.logits).cuda()


@pytest.mark.parametrize("key,M", [("w8", 5), ("w8", 300), ("w4ao", 40), ("w4ao", 600)])
def test_graph_replay_matches_eager(key, M):
    need_gpu()
    spec, p = packed(key)
    say("graph", key, M)
    x, lg = inputs(spec, M, 900 + M)
    eager = wq.MoERunner(p, M, spec.topk, spec.renormalize)
    ref = eager(x, lg).clone()
    torch.cuda.synchronize()

    r = wq.MoERunner(p, M, spec.topk, spec.renormalize)
    assert r.bs == eager.bs
    xs, ls = x.clone(), lg.clone()
    r.capture(xs, ls)
    for _ in range(3):
        out = r.replay().clone()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        eager(x, lg)  # eager work on the same stream between replays
        torch.cuda.synchronize()

    x2, lg2 = inputs(spec, M, 950 + M)
    ref2 = eager(x2, lg2).clone()
    xs.copy_(x2)
    ls.copy_(lg2)
    out2 = r.replay().clone()
    torch.cuda.synchronize()
    assert torch.equal(out2, ref2)
    assert not torch.equal(ref2, ref)
