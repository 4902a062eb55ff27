"""The README's Python example, run as written on the GPU, then checked against the oracle."""
import os
import re

import numpy as np
import pytest
import torch

from oracle import paged_ref as ref
from tests.gpu_util import ATOL, RTOL, assert_close, raw, widen

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _example() -> str:
    blocks = re.findall(r"```python\n(.*?)```", open(README).read(), flags=re.S)
    assert len(blocks) == 1, "the README holds one Python example"
    return blocks[0]


def test_readme_example_matches_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ns = {}
    exec(compile(_example(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    tables = ns["bm"].block_tables(range(len(ns["lens"])))
    want = ref.decode_ref(raw(ns["q"]), raw(ns["k_cache"]), raw(ns["v_cache"]), tables,
                          np.asarray(ns["lens"], np.int32), 1 / np.sqrt(ns["D"]), "bf16")
    assert_close(widen(ns["out"]), want, ATOL, RTOL, "README example")
