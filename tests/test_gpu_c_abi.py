"""The C-ABI from plain C: ``lf_abi_check`` (built from
``sparse_long_sequence_longformer_amd/csrc/lf_abi_check.c`` by the package build, linked
against liblfattn.so and the HIP runtime only) runs one forward with its own device
memory, outside Python and torch.  Its output is compared with the fp64 oracle at the
bf16 bar (max-abs 2e-2, mean-abs 2e-3), and a call with w = -1 must fail with
LF_ERR_INVALID_ARG before anything is enqueued."""

import os
import struct
import subprocess

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd import build as pkg_build
from sparse_long_sequence_longformer_amd.workloads import make_custom
from tests.gpu_common import compare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(pkg_build.ABI_CHECK):
        pytest.fail("lf_abi_check is not built (run __graft_entry__.build())")
    yield


def _write_problem(path, q, k, v, w, dil, G, pad):
    B, H, L, d = q.shape
    with open(path, "wb") as f:
        f.write(struct.pack("<7i", B, H, L, d, w, len(G), 0 if pad is None else 1))
        f.write(np.asarray(dil, dtype="<i4").tobytes())
        f.write(np.asarray(G, dtype="<i4").tobytes())
        if pad is not None:
            f.write(np.ascontiguousarray(pad, dtype=np.uint8).tobytes())
        for t in (q, k, v):
            f.write(t.contiguous().view(torch.int16).numpy().astype("<i2").tobytes())


def _run(args):
    log(f"  running {' '.join(os.path.basename(a) for a in args)}")
    return subprocess.run(args, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)


def test_c_program_forward(tmp_path):
    B, H, L, w = 2, 3, 500, 40
    dil, G = [1, 2, 3], [0, 9, 250, 9]
    pad = (np.arange(L)[None, :] >= np.asarray([500, 333])[:, None]).astype(np.uint8)
    log(f"case C caller: B={B} H={H} L={L} w={w} dil={dil} G={G} padded")
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=21)
    src, dst = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    _write_problem(src, q, k, v, w, dil, G, pad)
    res = _run([pkg_build.ABI_CHECK, src, dst])
    log("  " + res.stdout.strip())
    assert res.returncode == 0, res.stdout
    raw = np.fromfile(dst, dtype="<i2")
    assert raw.size == B * H * L * 64
    out = torch.from_numpy(raw.astype(np.int16)).view(torch.bfloat16).reshape(B, H, L, 64)
    compare(out, orc.attention(q, k, v, w, dil, G, pad), "bf16", "C caller out")


def test_c_program_rejects_bad_window(tmp_path):
    q, k, v = make_custom(1, 1, 64, dtype="bf16", seed=22)
    src = str(tmp_path / "in.bin")
    _write_problem(src, q, k, v, 4, [1], [], None)
    res = _run([pkg_build.ABI_CHECK, src, str(tmp_path / "unused.bin"), "bad-w"])
    log("  " + res.stdout.strip())
    assert res.returncode == 0 and "bad w:" in res.stdout, res.stdout
