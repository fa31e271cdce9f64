"""GPU test of the allocation-free decode entry point
(mllm_decode_rope_store_attn_noalloc): two calls in a row through the C ABI,
the second with fewer entries and a smaller cache, each against the
workspace entry point (mllm_decode_rope_store_attn) on an identical copy of
the inputs and the cache.  The two share their kernels and plan, so the bar is
bit-for-bit equality of the output and of every cache byte.
"""
import numpy as np
import pytest
import torch

import gpu_harness as H
import positions_aware_cached_amd as pac
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")


def _pair(cfg):
    """Two device copies of one decode step's inputs and cache."""
    inp = workloads.draw_decode(cfg, device="cuda")
    other = dict(inp)
    for k in ("q", "k_new", "v_new", "Kc", "Vc"):
        other[k] = inp[k].clone()
    return H.DecodeRun(inp, cfg), H.DecodeRun(other, cfg)


def _noalloc(run):
    hm = np.concatenate([run.pos_h, run.rows_h])
    pac.decode_rope_store_attn_noalloc(run.cache, 0, run.q, run.k_new, run.v_new, run.pos,
                                       run.rows, run.out, run.cfg["base"], host_mirror=hm,
                                       status=run.status)
    torch.cuda.synchronize()


def test_noalloc_matches_workspace_call_twice():
    cases = [("llama3_8b", workloads.config("llama3_8b")),
             ("smaller", workloads.config("llama3_8b", A=12, S=16, C=1024, seed=7,
                                          pos=("uniform", 0, 1023), rows="subset"))]
    for name, cfg in cases:
        H.log(f"no-alloc decode vs workspace decode: {name} A={cfg['A']} C={cfg['C']}")
        ref, got = _pair(cfg)
        ref.run(kernel=0)
        _noalloc(got)
        assert int(ref.status.item()) == 0 and int(got.status.item()) == 0
        assert torch.equal(ref.out.view(torch.int16), got.out.view(torch.int16)), name
        assert torch.equal(ref.Kc.view(torch.int16), got.Kc.view(torch.int16)), name
        assert torch.equal(ref.Vc.view(torch.int16), got.Vc.view(torch.int16)), name
        del ref, got
        torch.cuda.empty_cache()
