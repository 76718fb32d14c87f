"""The seeded input generator is bitwise device-independent: K, V and q drawn
on the GPU equal those drawn on the CPU.  The parity tests rely on this when
they draw the oracle's inputs on the GPU (fast) and copy them to the host:
the values are then exactly the CPU generator's."""
import sys

import numpy as np
import pytest
import torch

from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import synthetic  # noqa: E402


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy()


@pytest.mark.parametrize("name", ["tiny", "llama8b", "llama70b", "mixed", "kivi"])
def test_generator_same_bits_on_cpu_and_gpu(name):
    """First, middle and last positions of the last sequence (the largest
    counters the workload uses), plus the queries."""
    w = synthetic.WORKLOADS[name]
    lens = synthetic.seq_lens(w)
    b = len(lens) - 1
    n = int(lens[b])
    say("generator", name)
    for pos0 in sorted({0, max(0, n // 2 - 300), max(0, n - 600)}):
        m = min(600, n - pos0)
        kc, vc = synthetic.gen_kv(w, b, pos0, m, "cpu")
        kg, vg = synthetic.gen_kv(w, b, pos0, m, "cuda")
        assert np.array_equal(bits(kc), bits(kg)), (name, pos0)
        assert np.array_equal(bits(vc), bits(vg)), (name, pos0)
    kc, vc = synthetic.gen_new_kv(w, b, 4, "cpu")
    kg, vg = synthetic.gen_new_kv(w, b, 4, "cuda")
    assert np.array_equal(bits(kc), bits(kg)) and np.array_equal(bits(vc), bits(vg))
    assert np.array_equal(bits(synthetic.gen_q(w, "cpu")), bits(synthetic.gen_q(w, "cuda")))
