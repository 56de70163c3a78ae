"""hsa_forward_noalloc (the entry point that allocates nothing, with the
library's static device scratch) against hsa_forward with a caller
workspace: the same bits, on two calls in a row, the second with a smaller
input, through the C ABI."""
import numpy as np
import pytest
import torch

from hierarchical_index_sparse_amd import _lib, datagen, pipeline
from hierarchical_index_sparse_amd.workloads import Workload

pytestmark = pytest.mark.gpu


def _case(name, batch, L, nq, B, m, k, Hq, Hkv, nL=1, dI=128):
    return Workload(name=name, batch=batch, seq_len=L, n_q=nq, d_index=dI, block=B, top_m=m, top_k=k,
                    n_heads_q=Hq, n_heads_kv=Hkv, n_landmarks=nL)


def _both(w):
    inp = datagen.make_inputs(w)
    dev = pipeline.to_device(inp)
    shape = _lib.shape_of(w)
    need = _lib.hsa_sparse_workspace_size(shape, _lib.HSA_SPARSE_OP_FORWARD)
    assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES
    ref = pipeline.to_host(pipeline.run_forward(w, dev))
    out = pipeline.alloc_outputs(w)
    _lib.hsa_forward_noalloc(shape, dev["qI"], dev["kI"], dev.get("W"), 0, out["S"], dev["Q"], dev["K"], dev["V"],
                             out["blk"], out["tok"], out["O"], out["lse"])
    got = pipeline.to_host(out)
    for key in ("S", "blk", "tok", "O", "lse"):
        assert np.array_equal(got[key], ref[key], equal_nan=True), f"{w.name}: {key} differs from hsa_forward's"


@pytest.mark.parametrize("first,second", [
    # prefill (token scores and lists in the scratch), then a smaller decode
    # step (split attention partials in the scratch)
    (_case("prefill_first", 2, 6000, 700, 64, 12, 300, 16, 2), _case("decode_second", 3, 5000, 1, 32, 8, 128, 8, 1)),
    # a long-context decode with landmarks (many splits), then a smaller one
    (_case("decode_lm_first", 2, 200000, 1, 128, 64, 2048, 16, 1, nL=4),
     _case("decode_lm_second", 1, 9000, 1, 16, 6, 40, 4, 2, nL=2, dI=64)),
])
def test_noalloc_matches_forward_twice(first, second):
    _both(first)
    _both(second)
    torch.cuda.synchronize()


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    w = _case("too_big", 1, 65536, 65536, 128, 64, 2048, 16, 1)
    shape = _lib.shape_of(w)
    assert _lib.hsa_sparse_workspace_size(shape, _lib.HSA_SPARSE_OP_FORWARD) > _lib.NOALLOC_SCRATCH_BYTES
    lib = _lib.load()
    fake = 256  # never dereferenced: the size check comes before any launch
    st = lib.hsa_forward_noalloc(_lib.ctypes.byref(shape), fake, fake, None, 0, fake, fake, fake, fake, None, None,
                                 fake, None, None)
    assert _lib.STATUS[st] == "WORKSPACE_TOO_SMALL"
    assert b"static scratch" in lib.hsa_sparse_last_error()
