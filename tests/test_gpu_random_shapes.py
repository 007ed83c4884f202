"""Seeded random layer shapes on the GPU against the oracle (needs an MI355X).

Twelve shapes drawn once from a fixed seed, spread over the shape space the ABI accepts for
each expert dtype (bf16 and FP8: d % 256 == 0 and d_ff % 128 == 0; fp32: multiples of 64):
token counts 1..700, 1..96 routed experts, K up to min(N_r, 16), 0..3 shared experts. Each
runs the whole step and is checked as the edge cases are (routing, counts, permutation and
bias bit for bit outside the tie band; output within the output tolerances).
"""
import numpy as np
import pytest

from mixture_experts_layer_26_amd import inputs as I
from tests.test_gpu_edges import MID, _w, run_layer_case

pytestmark = pytest.mark.gpu


def _shapes(n=12, seed=20261203):
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        ffn = ["bf16", "fp8", "f32"][i % 3]
        if ffn == "f32":
            d = int(rng.choice([64, 128, 192, 320]))
            d_ff = int(rng.choice([64, 128, 192]))
            base = I.WORKLOADS["tiny_f32"]
        else:
            d = int(rng.choice([256, 512, 768, 1024]))
            d_ff = int(rng.choice([128, 256, 384, 640]))
            base = MID
        n_r = int(rng.integers(1, 97))
        k = int(rng.integers(1, min(n_r, 16) + 1))
        kw = dict(T=int(rng.integers(1, 701)), d=d, n_routed=n_r, top_k=k, n_shared=int(rng.integers(0, 4)),
                  d_ff=d_ff, seed=3000 + i)
        if ffn == "fp8":
            kw["ffn"] = "fp8"
        name = f"r{i}_{ffn}_T{kw['T']}_d{d}_nr{n_r}_k{k}_ns{kw['n_shared']}_ff{d_ff}"
        out[name] = _w(name, base=base, **kw)
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("name", list(SHAPES))
def test_random_shape(name):
    w = SHAPES[name]
    run_layer_case(w, I.make_b(w), name)
