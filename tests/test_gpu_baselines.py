"""The dense decode baselines the bench compares against ("Where Activation
Sparsity and KV-Cache Sparsity Cross in LLM Decoding", "The Attention
Baseline"): masked (eager matmul + mask + softmax) and fused (SDPA) attention,
over the whole cache and over the 30 % sink-plus-recent window, checked
against the fp64 oracle so the speedups the bench reports compare equal
results.  Both baselines are PyTorch's kernels with bf16 outputs (and bf16
probabilities in the masked one), so their bound is looser than the
library's: |out| stays below ~4 on these inputs, where a bf16 half-ulp is
2^-8, plus 2^-9 relative error on each probability."""
import math

import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from gpu_util import banner, dev, host, need_gpu

pytestmark = pytest.mark.gpu

TOL_BF16_OUT = 1.5e-2


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rand(shape, seed):
    return synth.bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("nn", [2048, 32768])
def test_masked_and_fused_baselines_match_oracle(nn):
    banner(f"attention baselines vs oracle n={nn}")
    hq, hkv, d = 32, 8, 128
    G = hq // hkv
    scale = 1.0 / math.sqrt(d)
    q, k, v = _rand((hq, d), 51), _rand((hkv, nn, d), 52), _rand((hkv, nn, d), 53)
    w = int(round(0.3 * nn))
    recent = w - 4
    tail = nn - recent
    sink_idx = np.tile(np.arange(4, dtype=np.int32), (hkv, 1))
    sink_cnt = np.full(hkv, 4, np.int32)
    ref_d, _ = oracle.attend_dense(q, k, v, nn)
    ref_w, _ = oracle.attend_sparse(q, k, v, nn, sink_idx, sink_cnt, tail)
    qt, kt, vt = dev(q), dev(k), dev(v)
    kw = torch.cat([kt[:, :4], kt[:, tail:]], 1).contiguous()
    vw = torch.cat([vt[:, :4], vt[:, tail:]], 1).contiguous()
    mask = torch.zeros((nn, 1), device="cuda")
    outs = {
        "masked_dense": bench.masked_decode(qt, kt, vt, nn, scale, mask),
        "masked_window": bench.masked_decode(qt, kw, vw, w, scale),
        "fused_dense": bench.fused_decode(qt, kt, vt, nn, scale),
        "fused_window": bench.fused_decode(qt, kw, vw, w, scale),
    }
    torch.cuda.synchronize()
    for name, o in outs.items():
        got = host(o.float()).reshape(hq, d)
        ref = ref_d if name.endswith("dense") else ref_w
        err = np.abs(got - ref).max()
        assert err <= TOL_BF16_OUT, (name, err)
