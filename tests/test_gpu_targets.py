"""The decode path's targets at the 13B shape (40 heads x 128, fp16, 16-token blocks, 30 sequences of
128..2048 tokens), timed on the GPU the way bench.py times them: paged decode attention sustains at
least 70 % of the MI355X's 8 TB/s HBM peak on its algorithmic bytes, and costs at most 15 % more
than the contiguous-cache kernel of the same design on the same data."""
import argparse

import pytest
import torch

import bench
from paged_kv_cache_416_amd import kernels

from harness import say

pytestmark = pytest.mark.gpu


def test_decode_13b_meets_hbm_and_indirection_targets():
    w, P, flags = bench.make_workload("13b")
    args = argparse.Namespace(replicas=3, steps=100)
    st = bench.Setup(w, args, "cuda:0", "none")
    ws = kernels.alloc_workspace(w.num_seqs, w.num_q_heads, w.head_dim, st.max_ctx, P, st.dev)
    stream = torch.cuda.current_stream()

    def attend(i):
        r = i % args.replicas
        kernels.paged_attention_decode(st.out, st.q, st.ks[r], st.vs[r], st.tb, st.ctx_dev, st.max_ctx, w.scale, P, ws,
                                       flags)

    for i in range(30):
        attend(i)
    us = bench.timed_launches(attend, args.steps, stream)
    frac = st.unique_b / (us * 1e-6) / (bench.PEAK_HBM_GBS * 1e9)
    cont = bench.contiguous_leg(w, P, args, st.dev, st.dt, us, flags)
    say(f"[13B targets] {us:.1f} us per launch, {100 * frac:.1f} % of HBM peak; paged over contiguous "
        f"{100 * cont['paged_over_contiguous']:+.1f} %")
    assert frac >= 0.70, f"{100 * frac:.1f} % of HBM peak, below 70 %"
    assert cont["paged_over_contiguous"] <= 0.15, f"paged costs {100 * cont['paged_over_contiguous']:.1f} % more"
