"""fp_prefill_noalloc (the entry point for callers that cannot allocate)
against the three-call path with a caller-allocated workspace, through the C
ABI, on two calls in a row on one GPU, the second with a smaller layer.  Both
run the same kernels, so the outputs must be bit-identical; the second call
also shows that the first call's leftovers in the shared scratch buffer do
not leak into a later, smaller problem."""
import pytest
import torch

from block_sparse_long_04_amd import _lib
from block_sparse_long_04_amd.inputs import CONFIGS, make_layer
from tests.parity_util import require_gpu, say

pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, B, tau, **scales):
    out = torch.empty(q.shape, dtype=torch.float32 if q.dtype == torch.float32 else torch.bfloat16,
                      device=q.device)
    prob = _lib.make_problem(q, k, v, out, B, tau, **scales)
    _lib.fp_prefill_noalloc(prob, _lib.current_stream(q.device))
    return out


@pytest.mark.parametrize("dtype,d,B", [("bf16", 128, 128), ("fp8", 128, 128), ("bf16", 64, 64)])
def test_noalloc_matches_the_three_calls(dtype, d, B):
    dev = require_gpu()
    outs = []
    for L, Hq, Hkv, tau in ((9000, 16, 4, 0.1), (1500, 8, 2, 0.05)):
        cfg = CONFIGS["c2"].with_(seq_len=L, num_q_heads=Hq, num_kv_heads=Hkv, dtype=dtype,
                                  head_dim=d, block_size=B)
        say(f"[noalloc {dtype} d={d} B={B}] L={L} Hq={Hq} Hkv={Hkv} tau={tau}")
        lay = make_layer(cfg, device=dev, keep_fp32=False)
        sc = dict(q_scale=lay.q_scale, k_scale=lay.k_scale, v_scale=lay.v_scale)
        pf = _lib.Prefill(lay.q, lay.k, lay.v, block_size=B, threshold=tau, **sc)
        ref = pf.run()
        got = _noalloc(lay.q, lay.k, lay.v, B, tau, **sc)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), float((got.float() - ref.float()).abs().max())
        assert torch.isfinite(got.float()).all()
        outs.append(got)
    say("    bit-identical on both calls")

