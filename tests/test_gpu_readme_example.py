"""The README's serving-loop example, run as written: the block manager's
prefix cache, copy-on-write, prefill, decode and the shared-prefix decode
wired together through the Python binding."""
import os
import re

import numpy as np
import pytest

from tests.helpers import assert_close
from paged_kv_cache_101_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _example_code():
    with open(os.path.join(ROOT, "README.md")) as fh:
        text = fh.read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    code = [b for b in blocks if "BlockManager(" in b]
    assert len(code) == 1, "the README holds one serving-loop example"
    return code[0]


@pytest.mark.gpu
def test_readme_serving_loop(gpu):
    ns = {}
    exec(compile(_example_code(), "README.md (serving-loop example)", "exec"), ns)
    import torch
    torch.cuda.synchronize()
    # request 2 reused request 1's four full system-prompt blocks
    starts, shared = ns["starts"], ns["shared"]
    assert list(starts) == [0, 2] and list(shared) == [4]
    assert ns["bm"].prefix_cache_stats()[1] == 64
    for rid, o in ns["prefill_out"].items():
        assert torch.isfinite(o.float()).all(), rid
    out, out_shared = ns["out"], ns["out_shared"]
    assert torch.isfinite(out.float()).all()
    # the shared-prefix call computes the same attention as plain decode
    assert_close(W.to_numpy(out_shared).astype(np.float64), W.to_numpy(out).astype(np.float64),
                 "f16", "shared-prefix against plain decode")
    # every block went back to the pool
    assert ns["bm"].num_free_blocks == ns["num_blocks"] - 1
