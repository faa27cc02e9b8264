"""The Longformer layer (``lf_layer_forward``) against the fp64 layer oracle.

Tolerance (bf16 activations between the steps, fp32 GEMM accumulation, bf16
output): max-abs 5e-2 and mean-abs 5e-3 over the output, whose LayerNorm rows
have unit scale.  The output rounding alone is up to 2^-9 of |out| (about 8e-3 at
|out| = 4), and each of the stored intermediates (the QKV and first feed-forward
GEMM outputs, q, k, v, attention output, x1, feed-forward activations) adds a
rounding of the same relative size before the next step.
"""

import numpy as np
import pytest
import torch

from oracle import layer_oracle as lo
from tests.gpu_common import log

pytestmark = pytest.mark.gpu

TOL_MAX = 5e-2
TOL_MEAN = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_sequence_longformer_amd import binding

    binding.load_library()
    yield


def _weights(E, F, seed, scale=0.05):
    rng = np.random.default_rng(seed)
    W = {
        "w_qkv": rng.standard_normal((3 * E, E)) * scale, "b_qkv": rng.standard_normal(3 * E) * scale,
        "w_o": rng.standard_normal((E, E)) * scale, "b_o": rng.standard_normal(E) * scale,
        "ln1_g": 1.0 + rng.standard_normal(E) * 0.1, "ln1_b": rng.standard_normal(E) * 0.1,
        "w_1": rng.standard_normal((F, E)) * scale, "b_1": rng.standard_normal(F) * scale,
        "w_2": rng.standard_normal((E, F)) * scale, "b_2": rng.standard_normal(E) * scale,
        "ln2_g": 1.0 + rng.standard_normal(E) * 0.1, "ln2_b": rng.standard_normal(E) * 0.1,
    }
    return {k: torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16) for k, v in W.items()}


# (name, B, L, E, F, w, dil, globals, pad lengths, causal)
CASES = [
    ("small_dil", 2, 300, 128, 256, 16, [1, 2], [0, 150], [300, 211], False),
    ("roberta_like_1024", 1, 1024, 768, 3072, 128, [1] * 12, list(range(8)), None, False),
    ("causal_small", 1, 400, 256, 512, 32, [1, 1, 2, 2], [5, 300], None, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_forward(case):
    from sparse_long_sequence_longformer_amd import binding

    name, B, L, E, F, w, dil, G, lens, causal = case
    log(f"case layer {name}: B={B} L={L} hidden={E} ffn={F} w={w}")
    x = torch.from_numpy(np.random.default_rng(len(name)).standard_normal((B, L, E), dtype=np.float32)).bfloat16()
    W = _weights(E, F, len(name) + 1)
    pad = None if lens is None else (np.arange(L)[None, :] >= np.asarray(lens)[:, None]).astype(np.uint8)
    out = binding.layer_forward(x.cuda(), {k: v.cuda() for k, v in W.items()}, w, dil, G,
                                None if pad is None else torch.from_numpy(pad).cuda(), causal=causal)
    torch.cuda.synchronize()
    ref = lo.layer_forward(x, W, E // 64, w, dil, G, pad, causal=causal)
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    log(f"  {name}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} (max |ref| {np.abs(ref).max():.2f})")
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN
