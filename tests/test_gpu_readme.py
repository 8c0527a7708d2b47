"""The README's usage example runs as written, and its output matches the oracle on the cache the
step left behind (the step writes each sequence's new row, then attends over it)."""
import os
import re

import numpy as np
import pytest

import oracle
from harness import assert_close, say

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_example_runs_and_matches_oracle():
    import torch

    blocks = re.findall(r"```python\n(.*?)```", open(README).read(), re.S)
    assert len(blocks) == 1
    torch.manual_seed(0)
    env = {}
    say("  README example")
    exec(compile(blocks[0], README, "exec"), env)
    torch.cuda.synchronize()
    c, out, q = env["c"], env["out"], env["q"]
    tables, lens, D = env["tables"], env["lens"], env["D"]
    # both sequences hold the 100 prompt rows and then their own new row
    assert lens.cpu().tolist() == [101, 101]
    for s, slot in enumerate(env["slots"]):
        b, o = int(slot) // c.block_size, int(slot) % c.block_size
        assert torch.equal(c.k[b, :, o].view(torch.int16), env["new_k"][s].view(torch.int16))
    ref = oracle.paged_attention(q.view(torch.int16).cpu().numpy(), c.k.view(torch.int16).cpu().numpy(),
                                 c.v.view(torch.int16).cpu().numpy(), tables.cpu().numpy(), lens.cpu().numpy(),
                                 D ** -0.5, "bf16")
    assert np.isfinite(ref).all()
    assert_close(out, ref, "bf16", "README example")
