"""The C ABI on the host: the library loads, exports every declared entry
point, sizes workspaces, and rejects bad arguments before any HIP call (so
these run without a GPU; no compute is launched)."""
import ctypes
import os
import re

import pytest

from hierarchical_index_sparse_amd import _lib
from hierarchical_index_sparse_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsa_sparse.h")

FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(hsa_[a-z_0-9]+)\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("hsa_block_summary", "hsa_block_topm", "hsa_token_topk", "hsa_sparse_attn", "hsa_forward",
              "hsa_sparse_workspace_size", "hsa_sparse_strerror", "hsa_sparse_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(_lib.EXPORTS)


def test_strerror(lib):
    assert lib.hsa_sparse_strerror(0) == b"success"
    assert lib.hsa_sparse_strerror(3) == b"workspace too small"
    assert lib.hsa_sparse_strerror(99) == b"unknown status"


def shape(**kw):
    base = dict(batch=1, seq_len=4096, n_q=4096, d_index=64, block=64, top_m=8, top_k=256,
                n_heads_q=1, n_heads_kv=1, head_dim=128, n_landmarks=1)
    base.update(kw)
    return _lib.make_shape(**base)


def call_attn(lib, s, ws_bytes=1 << 40, O=FAKE):
    return lib.hsa_sparse_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, O, None, FAKE, ws_bytes, None)


def call_forward(lib, s, ws_bytes=1 << 40, W=None, qI=FAKE):
    return lib.hsa_forward(ctypes.byref(s), qI, FAKE, W, 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None,
                           FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), 2),
    (dict(n_heads_q=3, n_heads_kv=2), 1),
    (dict(n_heads_q=64, n_heads_kv=2), 2),
    (dict(top_k=0), 1),
    (dict(n_q=5000), 1),
    # kv row offsets are 31-bit: seq_len * n_heads_kv * 256 must stay below 2^31
    (dict(seq_len=1 << 22, n_q=1, n_heads_q=16, n_heads_kv=2), 2),
    (dict(seq_len=(1 << 23) - 1, n_q=1, n_heads_q=16, n_heads_kv=1, top_k=1 << 20), 0),
])
def test_attention_validation(lib, kw, status):
    if status == 0:
        # valid: the call would launch, so only the shape check is exercised
        # (zero queries: nothing is enqueued)
        assert call_attn(lib, shape(**dict(kw, batch=0))) == 0
        return
    assert call_attn(lib, shape(**kw)) == status
    assert lib.hsa_sparse_last_error() != b""


def test_attention_null_output(lib):
    assert call_attn(lib, shape(), O=None) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(top_m=1), 1),
    (dict(top_k=0), 1),
    (dict(d_index=96), 2),
    (dict(block=48), 2),
    (dict(block=256), 2),
    (dict(block=4), 2),
    (dict(n_landmarks=3), 2),
    (dict(seq_len=128 * 40000, n_q=1, block=128), 2),
    (dict(seq_len=1 << 20, n_q=1, block=128, top_m=512, top_k=4096), 2),
    (dict(batch=-1), 1),
])
def test_forward_validation(lib, kw, status):
    assert call_forward(lib, shape(**kw)) == status


def test_forward_needs_landmark_weights(lib):
    assert call_forward(lib, shape(n_landmarks=4)) == 1
    assert call_forward(lib, shape(), qI=None) == 1


def test_workspace_too_small(lib):
    s = shape()
    need = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_FORWARD)
    assert need > 0
    assert call_forward(lib, s, ws_bytes=need - 1) == 3
    assert b"workspace" in lib.hsa_sparse_last_error()
    st = lib.hsa_token_topk(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, 0, None)
    assert st == 3


def test_summary_validation(lib):
    s = shape(top_m=0, top_k=0)  # selection fields are not read by the summary step
    assert lib.hsa_block_summary(ctypes.byref(s), FAKE, None, -1, FAKE, None) == 1
    assert lib.hsa_block_summary(ctypes.byref(shape(n_landmarks=2)), FAKE, None, 0, FAKE, None) == 1
    assert lib.hsa_block_summary(ctypes.byref(shape(d_index=32)), FAKE, None, 0, FAKE, None) == 2


def test_empty_inputs_are_no_ops(lib):
    # nothing to do: returns OK without touching memory or the GPU
    for kw in (dict(batch=0), dict(n_q=0)):
        s = shape(**kw)
        assert lib.hsa_block_topm(ctypes.byref(s), None, None, None, None, 0, None) == 0
        assert lib.hsa_token_topk(ctypes.byref(s), None, None, None, None, None, 0, None) == 0
        assert lib.hsa_sparse_attn(ctypes.byref(s), None, None, None, None, None, None, None, 0, None) == 0


def test_workspace_sizes(lib):
    for w in WORKLOADS.values():
        s = _lib.shape_of(w)
        nqt = w.batch * w.n_q
        topm = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_BLOCK_TOPM)
        assert topm >= nqt * w.n_blocks * 4
        topk = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_TOKEN_TOPK)
        if w.top_k >= w.top_m * w.block:
            assert topk == 0
        else:
            assert topk >= nqt * w.top_m * w.block * 4
        fwd = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_FORWARD)
        assert fwd >= nqt * (w.top_m + w.top_k) * 4 + max(topm, topk)
        assert fwd % 256 == 0
    assert lib.hsa_sparse_workspace_size(None, _lib.HSA_SPARSE_OP_FORWARD) == 0
    assert lib.hsa_sparse_workspace_size(ctypes.byref(shape()), 42) == 0


def call_flat(lib, s, ws_bytes=1 << 44, tok=FAKE):
    return lib.hsa_flat_topk(ctypes.byref(s), FAKE, FAKE, tok, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), 1),
    (dict(d_index=32), 2),
    (dict(n_q=5000), 1),
    (dict(seq_len=65536, n_q=1, top_k=8193), 2),        # list longer than the LDS stage
    (dict(seq_len=8000, n_q=1, top_k=8193), 0),         # keeps everything: no select
    (dict(seq_len=200000, n_q=1, top_k=8192), 0),       # several merge levels
    (dict(seq_len=4096, n_q=16, block=0, top_m=0), 0),  # block fields are not read
])
def test_flat_validation(lib, kw, status):
    if status == 0:
        assert call_flat(lib, shape(**dict(kw, batch=0))) == 0
        assert lib.hsa_sparse_workspace_size(ctypes.byref(shape(**kw)), _lib.HSA_SPARSE_OP_FLAT_TOPK) >= 0
        return
    assert call_flat(lib, shape(**kw)) == status
    assert lib.hsa_sparse_last_error() != b""


def test_flat_workspace(lib):
    # every causal score in fp32, rows padded to a multiple of 4; plus two
    # ping-pong buffers of chunk winners (8-byte pairs and a count per list)
    # when a query's candidates span several 8192-token chunks
    s = shape(batch=2, seq_len=4097, n_q=3, top_k=100)
    need = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_FLAT_TOPK)
    assert need >= 2 * 3 * 4100 * 4 and need % 256 == 0
    s = shape(batch=1, seq_len=70000, n_q=2, top_k=1000)
    need = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_FLAT_TOPK)
    assert need >= 2 * 70000 * 4 + 2 * (2 * 9 * 1000 * 8)
    assert call_flat(lib, s, ws_bytes=need - 1) == 3
    assert lib.hsa_sparse_workspace_size(ctypes.byref(shape(top_k=5000)), _lib.HSA_SPARSE_OP_FLAT_TOPK) == 0
    assert lib.hsa_flat_topk(ctypes.byref(shape(batch=0)), None, None, None, None, 0, None) == 0


def test_decode_step_validation(lib):
    def call(s, lens=FAKE):
        return lib.hsa_decode_step(ctypes.byref(s), lens, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                                   None, FAKE, 1 << 40, None)
    assert call(shape(n_q=2)) == 1          # one new query per sequence
    assert call(shape(n_q=1), lens=None) == 1
    assert call(shape(n_q=1, head_dim=64)) == 2
    assert call(shape(batch=0, n_q=1), lens=None) == 0
    s = shape(n_q=1)
    need = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_FORWARD)
    assert lib.hsa_decode_step(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                               None, FAKE, need - 1, None) == 3


def test_three_level_validation(lib):
    def fwd(s, group=16, m2=8, S2=FAKE, sup=FAKE, ws=1 << 40, lens=None):
        return lib.hsa_forward_3level(ctypes.byref(s), lens, group, m2, FAKE, FAKE, None, 0, FAKE, S2, FAKE, FAKE,
                                      FAKE, sup, None, None, FAKE, None, FAKE, ws, None)

    def sel(s, group=16, m2=8, ws=1 << 40):
        return lib.hsa_block_topm_3level(ctypes.byref(s), group, m2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)

    s = shape()
    assert fwd(s, group=12) == 2             # not a power of two
    assert fwd(s, group=8192) == 2           # above 4096
    assert fwd(s, group=0) == 2
    assert fwd(s, m2=1) == 1                 # first and last super-block are kept
    assert fwd(s, group=64, m2=256) == 2     # 16384 level-2 candidates > 8192
    assert fwd(s, S2=None) == 1
    assert fwd(s, sup=None) == 1
    assert fwd(shape(head_dim=64)) == 2
    assert fwd(s, lens=FAKE) == 1            # per-sequence lengths need one query per sequence
    assert b"n_q == 1" in lib.hsa_sparse_last_error()
    need = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_FORWARD)
    assert fwd(s, ws=need - 1) == 3
    assert sel(s, group=3) == 2 and sel(s, m2=0) == 1
    need = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_BLOCK_TOPM)
    # level 1 scores ceil(nb / group) super-blocks: the block top-m size is enough
    assert sel(s, group=1, ws=need - 1) == 3
    assert b"workspace" in lib.hsa_sparse_last_error()
    assert sel(shape(batch=0), ws=0) == 0
    assert lib.hsa_super_summary(ctypes.byref(s), 16, FAKE, -1, FAKE, None) == 1
    assert lib.hsa_super_summary(ctypes.byref(s), 5, FAKE, 0, FAKE, None) == 2
    assert lib.hsa_super_summary(ctypes.byref(shape(batch=0)), 16, None, 0, None, None) == 0
    # start past the last super-block (4096 / 64 = 64 blocks, 4 super-blocks of 16): nothing to do
    assert lib.hsa_super_summary(ctypes.byref(s), 16, None, 4, None, None) == 0
    assert lib.hsa_super_summary(ctypes.byref(s), 16, None, 3, None, None) == 1


def test_per_head_validation(lib):
    def fwd(s, ws=1 << 40, W=None, LK=FAKE):
        return lib.hsa_forward_heads(ctypes.byref(s), None, W, 0, FAKE, FAKE, FAKE, LK, None, FAKE, None, FAKE, ws,
                                     None)

    base = dict(n_q=1, block=64, top_m=8, n_heads_q=8, n_heads_kv=2, d_index=0, top_k=0)
    assert fwd(shape(**dict(base, top_m=1))) == 1
    assert fwd(shape(**dict(base, head_dim=64))) == 2
    assert fwd(shape(**dict(base, block=96))) == 2
    assert fwd(shape(**dict(base, n_heads_kv=3))) == 1            # does not divide 8
    assert fwd(shape(**dict(base, n_heads_q=32, n_heads_kv=32))) == 2  # more than 16 kv heads
    assert fwd(shape(**dict(base, top_m=4096, block=64))) == 2   # 262144 tokens per head
    assert fwd(shape(**dict(base, n_landmarks=4))) == 1          # needs landmark_W
    assert fwd(shape(**base), LK=None) == 1
    s = shape(**base)
    need = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_FORWARD_HEADS)
    # chunk lists + token lists (top_m * block per query head) + scratch
    rows = 1 * 1 * 8
    assert need >= rows * 8 * 4 + rows * 8 * 64 * 4
    assert fwd(s, ws=need - 1) == 3
    sel = lib.hsa_sparse_workspace_size(ctypes.byref(s), _lib.HSA_SPARSE_OP_HEAD_TOPM)
    assert sel >= rows * 64 * 4  # fp32 score per (query, head, chunk): 4096 / 64 chunks
    assert lib.hsa_head_topm(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, sel - 1, None) == 3
    # landmarks read no selection fields
    t = shape(**dict(base, top_m=0))
    assert lib.hsa_head_landmarks(ctypes.byref(t), FAKE, None, -1, FAKE, None) == 1
    assert lib.hsa_head_landmarks(ctypes.byref(shape(**dict(base, n_landmarks=2))), FAKE, None, 0, FAKE, None) == 1
    assert lib.hsa_head_landmarks(ctypes.byref(t), None, None, 64, None, None) == 0  # past the last chunk
    assert lib.hsa_forward_heads(ctypes.byref(shape(**dict(base, batch=0))), None, None, 0, None, None, None, None,
                                 None, None, None, None, 0, None) == 0
    # per-sequence lengths take one query per sequence
    assert lib.hsa_forward_heads(ctypes.byref(shape(**dict(base, n_q=2))), FAKE, None, 0, FAKE, FAKE, FAKE, FAKE,
                                 None, FAKE, None, FAKE, 1 << 40, None) == 1


def test_kernel_event_validation(lib):
    Ev = ctypes.c_void_p * 80
    a, b = Ev(), Ev()
    assert lib.hsa_sparse_set_kernel_events(a, b, 65) == 1      # at most 64 kernels
    assert lib.hsa_sparse_set_kernel_events(a, None, 4) == 1
    assert lib.hsa_sparse_set_kernel_events(None, None, 0) == 0  # off
    assert lib.hsa_sparse_last_kernels() == b""
    # NULL events are allowed: kernels are then named but not timed
    assert lib.hsa_sparse_set_kernel_events(a, b, 4) == 0
    assert lib.hsa_sparse_set_kernel_events(None, None, 0) == 0


def test_header_is_a_c_abi(tmp_path):
    # a pedantic C99 translation unit includes the header alone, takes the
    # address of every declared entry point and links against the library
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = tmp_path / "abi.c"
    src.write_text('#include "hsa_sparse.h"\n#include <stdio.h>\ntypedef void (*fn_t)(void);\n'
                   "int main(void) {\n  fn_t fns[] = {\n" + ",\n".join(f"    (fn_t)&{n}" for n in names) +
                   '\n  };\n  printf("%d\\n", (int)(sizeof(fns) / sizeof(fns[0])));\n  return 0;\n}\n')
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.dirname(HEADER), str(src),
                        "-L", lib_dir, "-lhsa_sparse", "-Wl,--allow-shlib-undefined", "-o", str(tmp_path / "abi")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
