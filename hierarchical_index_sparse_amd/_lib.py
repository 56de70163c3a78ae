"""ctypes binding of libhsa_sparse.so (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch
tensors that already live on the GPU (torch is used for device memory and
streams only).  bf16 tensors may be ``torch.bfloat16`` or 16-bit integer
views of the same bits.  There is no fallback: if the shared library is
missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhsa_sparse.so")

HSA_SPARSE_OP_BLOCK_SUMMARY = 0
HSA_SPARSE_OP_BLOCK_TOPM = 1
HSA_SPARSE_OP_TOKEN_TOPK = 2
HSA_SPARSE_OP_SPARSE_ATTN = 3
HSA_SPARSE_OP_FORWARD = 4
HSA_SPARSE_OP_FLAT_TOPK = 5
HSA_SPARSE_OP_HEAD_TOPM = 6
HSA_SPARSE_OP_FORWARD_HEADS = 7
HSA_SPARSE_OP_BLOCK_SCORE_MAX = 8

STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE_TOO_SMALL", 4: "HIP_ERROR"}

EXPORTS = ("hsa_sparse_workspace_size", "hsa_sparse_strerror", "hsa_sparse_last_error",
           "hsa_block_summary", "hsa_block_topm", "hsa_token_topk", "hsa_sparse_attn", "hsa_forward",
           "hsa_sparse_set_stage_events", "hsa_flat_topk", "hsa_decode_step", "hsa_super_summary",
           "hsa_block_topm_3level", "hsa_forward_3level", "hsa_head_landmarks", "hsa_head_topm",
           "hsa_forward_heads", "hsa_sparse_set_kernel_events", "hsa_sparse_last_kernels", "hsa_forward_noalloc",
           "hsa_block_score_max")

# bytes of the device array hsa_forward_noalloc uses as its scratch
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


class HsaSparseShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seq_len", "n_q", "d_index", "block", "n_landmarks", "top_m", "top_k",
        "n_heads_q", "n_heads_kv", "head_dim")] + [("scale", ctypes.c_float)]


class HsaSparseError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.status_name}: {detail}")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m hierarchical_index_sparse_amd.build_lib`")
    lib = ctypes.CDLL(path)
    P, S, I32, SZ = ctypes.c_void_p, ctypes.POINTER(HsaSparseShape), ctypes.c_int32, ctypes.c_size_t
    lib.hsa_sparse_workspace_size.argtypes = [S, ctypes.c_int]
    lib.hsa_sparse_workspace_size.restype = SZ
    lib.hsa_sparse_strerror.argtypes = [ctypes.c_int]
    lib.hsa_sparse_strerror.restype = ctypes.c_char_p
    lib.hsa_sparse_last_error.argtypes = []
    lib.hsa_sparse_last_error.restype = ctypes.c_char_p
    lib.hsa_block_summary.argtypes = [S, P, P, I32, P, P]
    lib.hsa_block_topm.argtypes = [S, P, P, P, P, SZ, P]
    lib.hsa_block_score_max.argtypes = [S, P, P, P, P, SZ, P]
    lib.hsa_token_topk.argtypes = [S, P, P, P, P, P, SZ, P]
    lib.hsa_sparse_attn.argtypes = [S, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_forward.argtypes = [S, P, P, P, I32, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_forward_noalloc.argtypes = [S, P, P, P, I32, P, P, P, P, P, P, P, P, P]
    lib.hsa_sparse_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.hsa_flat_topk.argtypes = [S, P, P, P, P, SZ, P]
    lib.hsa_decode_step.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_super_summary.argtypes = [S, I32, P, I32, P, P]
    lib.hsa_block_topm_3level.argtypes = [S, I32, I32, P, P, P, P, P, P, SZ, P]
    lib.hsa_forward_3level.argtypes = [S, P, I32, I32, P, P, P, I32, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_head_landmarks.argtypes = [S, P, P, I32, P, P]
    lib.hsa_head_topm.argtypes = [S, P, P, P, P, SZ, P]
    lib.hsa_forward_heads.argtypes = [S, P, P, I32, P, P, P, P, P, P, P, P, SZ, P]
    EV = ctypes.POINTER(ctypes.c_void_p)
    lib.hsa_sparse_set_kernel_events.argtypes = [EV, EV, ctypes.c_int]
    lib.hsa_sparse_last_kernels.argtypes = []
    lib.hsa_sparse_last_kernels.restype = ctypes.c_char_p
    for name in ("hsa_block_summary", "hsa_block_topm", "hsa_token_topk", "hsa_sparse_attn", "hsa_forward",
                 "hsa_sparse_set_stage_events", "hsa_flat_topk", "hsa_decode_step", "hsa_forward_noalloc",
                 "hsa_block_score_max"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def make_shape(batch, seq_len, n_q, d_index, block, top_m, top_k, n_heads_q=1, n_heads_kv=1,
               head_dim=128, n_landmarks=1, scale=None) -> HsaSparseShape:
    if scale is None:
        scale = head_dim ** -0.5
    return HsaSparseShape(batch, seq_len, n_q, d_index, block, n_landmarks, top_m, top_k,
                          n_heads_q, n_heads_kv, head_dim, scale)


def shape_of(w) -> HsaSparseShape:
    """Shape struct of a workloads.Workload."""
    return make_shape(w.batch, w.seq_len, w.n_q, w.d_index, w.block, w.top_m, w.top_k,
                      w.n_heads_q, w.n_heads_kv, w.head_dim, w.n_landmarks, w.scale)


def _ptr(t, name, dtypes, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)
_F32 = (torch.float32,)
_I8 = (torch.int8,)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        lib = load()
        raise HsaSparseError(status, where, lib.hsa_sparse_last_error().decode())


def hsa_sparse_workspace_size(shape: HsaSparseShape, op: int) -> int:
    return int(load().hsa_sparse_workspace_size(ctypes.byref(shape), op))


def _workspace(shape, op, ws, device):
    need = hsa_sparse_workspace_size(shape, op)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def hsa_block_summary(shape, kI, W, start_block, S, stream=None):
    st = load().hsa_block_summary(ctypes.byref(shape), _ptr(kI, "kI", _BF16), _ptr(W, "W", _I8, True),
                                  int(start_block), _ptr(S, "S", _BF16), _stream(stream))
    _check(st, "hsa_block_summary")


def hsa_block_topm(shape, qI, S, blk, workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_BLOCK_TOPM, workspace, qI.device)
    st = load().hsa_block_topm(ctypes.byref(shape), _ptr(qI, "qI", _BF16), _ptr(S, "S", _BF16),
                               _ptr(blk, "blk", _I32), ws.data_ptr(), nbytes, _stream(stream))
    _check(st, "hsa_block_topm")


def hsa_token_topk(shape, qI, kI, blk, tok, workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_TOKEN_TOPK, workspace, qI.device)
    st = load().hsa_token_topk(ctypes.byref(shape), _ptr(qI, "qI", _BF16), _ptr(kI, "kI", _BF16),
                               _ptr(blk, "blk", _I32), _ptr(tok, "tok", _I32), ws.data_ptr(), nbytes,
                               _stream(stream))
    _check(st, "hsa_token_topk")


def hsa_decode_step(shape, seq_lens, qI, kI, W, S, Q, K, V, blk_out, tok_out, O, lse, workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_FORWARD, workspace, Q.device)
    st = load().hsa_decode_step(ctypes.byref(shape), _ptr(seq_lens, "seq_lens", _I32), _ptr(qI, "qI", _BF16),
                                _ptr(kI, "kI", _BF16), _ptr(W, "W", _I8, True), _ptr(S, "S", _BF16),
                                _ptr(Q, "Q", _BF16), _ptr(K, "K", _BF16), _ptr(V, "V", _BF16),
                                _ptr(blk_out, "blk_out", _I32, True), _ptr(tok_out, "tok_out", _I32, True),
                                _ptr(O, "O", _F32), _ptr(lse, "lse", _F32, True), ws.data_ptr(), nbytes,
                                _stream(stream))
    _check(st, "hsa_decode_step")


def hsa_flat_topk(shape, qI, kI, tok, workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_FLAT_TOPK, workspace, qI.device)
    st = load().hsa_flat_topk(ctypes.byref(shape), _ptr(qI, "qI", _BF16), _ptr(kI, "kI", _BF16),
                              _ptr(tok, "tok", _I32), ws.data_ptr(), nbytes, _stream(stream))
    _check(st, "hsa_flat_topk")


def hsa_sparse_attn(shape, Q, K, V, tok, O, lse=None, workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_SPARSE_ATTN, workspace, Q.device)
    st = load().hsa_sparse_attn(ctypes.byref(shape), _ptr(Q, "Q", _BF16), _ptr(K, "K", _BF16),
                                _ptr(V, "V", _BF16), _ptr(tok, "tok", _I32), _ptr(O, "O", _F32),
                                _ptr(lse, "lse", _F32, True), ws.data_ptr(), nbytes, _stream(stream))
    _check(st, "hsa_sparse_attn")


def hsa_forward(shape, qI, kI, W, summary_start_block, S, Q, K, V, blk_out, tok_out, O, lse=None,
                workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_FORWARD, workspace, Q.device)
    st = load().hsa_forward(ctypes.byref(shape), _ptr(qI, "qI", _BF16), _ptr(kI, "kI", _BF16),
                            _ptr(W, "W", _I8, True), int(summary_start_block), _ptr(S, "S", _BF16),
                            _ptr(Q, "Q", _BF16), _ptr(K, "K", _BF16), _ptr(V, "V", _BF16),
                            _ptr(blk_out, "blk_out", _I32, True), _ptr(tok_out, "tok_out", _I32, True),
                            _ptr(O, "O", _F32), _ptr(lse, "lse", _F32, True), ws.data_ptr(), nbytes,
                            _stream(stream))
    _check(st, "hsa_forward")


def hsa_block_score_max(shape, qI, S, out, workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_BLOCK_SCORE_MAX, workspace, qI.device)
    st = load().hsa_block_score_max(ctypes.byref(shape), _ptr(qI, "qI", _BF16), _ptr(S, "S", _BF16),
                                    _ptr(out, "out", _F32), ws.data_ptr(), nbytes, _stream(stream))
    _check(st, "hsa_block_score_max")


def hsa_forward_noalloc(shape, qI, kI, W, summary_start_block, S, Q, K, V, blk_out, tok_out, O, lse=None,
                        stream=None):
    st = load().hsa_forward_noalloc(ctypes.byref(shape), _ptr(qI, "qI", _BF16), _ptr(kI, "kI", _BF16),
                                    _ptr(W, "W", _I8, True), int(summary_start_block), _ptr(S, "S", _BF16),
                                    _ptr(Q, "Q", _BF16), _ptr(K, "K", _BF16), _ptr(V, "V", _BF16),
                                    _ptr(blk_out, "blk_out", _I32, True), _ptr(tok_out, "tok_out", _I32, True),
                                    _ptr(O, "O", _F32), _ptr(lse, "lse", _F32, True), _stream(stream))
    _check(st, "hsa_forward_noalloc")


def hsa_super_summary(shape, group, S, start_super, S2, stream=None):
    st = load().hsa_super_summary(ctypes.byref(shape), int(group), _ptr(S, "S", _BF16), int(start_super),
                                  _ptr(S2, "S2", _BF16), _stream(stream))
    _check(st, "hsa_super_summary")


def hsa_block_topm_3level(shape, group, top_m2, qI, S, S2, sup, blk, workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_BLOCK_TOPM, workspace, qI.device)
    st = load().hsa_block_topm_3level(ctypes.byref(shape), int(group), int(top_m2), _ptr(qI, "qI", _BF16),
                                      _ptr(S, "S", _BF16), _ptr(S2, "S2", _BF16), _ptr(sup, "sup", _I32),
                                      _ptr(blk, "blk", _I32), ws.data_ptr(), nbytes, _stream(stream))
    _check(st, "hsa_block_topm_3level")


def hsa_forward_3level(shape, group, top_m2, qI, kI, W, summary_start_block, S, S2, Q, K, V, sup_out, blk_out,
                       tok_out, O, lse=None, workspace=None, stream=None, seq_lens=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_FORWARD, workspace, Q.device)
    st = load().hsa_forward_3level(ctypes.byref(shape), _ptr(seq_lens, "seq_lens", _I32, True), int(group),
                                   int(top_m2), _ptr(qI, "qI", _BF16),
                                   _ptr(kI, "kI", _BF16), _ptr(W, "W", _I8, True), int(summary_start_block),
                                   _ptr(S, "S", _BF16), _ptr(S2, "S2", _BF16), _ptr(Q, "Q", _BF16),
                                   _ptr(K, "K", _BF16), _ptr(V, "V", _BF16), _ptr(sup_out, "sup_out", _I32),
                                   _ptr(blk_out, "blk_out", _I32, True), _ptr(tok_out, "tok_out", _I32, True),
                                   _ptr(O, "O", _F32), _ptr(lse, "lse", _F32, True), ws.data_ptr(), nbytes,
                                   _stream(stream))
    _check(st, "hsa_forward_3level")


def hsa_head_landmarks(shape, K, W, start_block, LK, stream=None):
    st = load().hsa_head_landmarks(ctypes.byref(shape), _ptr(K, "K", _BF16), _ptr(W, "W", _I8, True),
                                   int(start_block), _ptr(LK, "LK", _BF16), _stream(stream))
    _check(st, "hsa_head_landmarks")


def hsa_head_topm(shape, Q, LK, blk, workspace=None, stream=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_HEAD_TOPM, workspace, Q.device)
    st = load().hsa_head_topm(ctypes.byref(shape), _ptr(Q, "Q", _BF16), _ptr(LK, "LK", _BF16),
                              _ptr(blk, "blk", _I32), ws.data_ptr(), nbytes, _stream(stream))
    _check(st, "hsa_head_topm")


def hsa_forward_heads(shape, W, summary_start_block, Q, K, V, LK, blk_out, O, lse=None, workspace=None,
                      stream=None, seq_lens=None):
    ws, nbytes = _workspace(shape, HSA_SPARSE_OP_FORWARD_HEADS, workspace, Q.device)
    st = load().hsa_forward_heads(ctypes.byref(shape), _ptr(seq_lens, "seq_lens", _I32, True),
                                  _ptr(W, "W", _I8, True), int(summary_start_block),
                                  _ptr(Q, "Q", _BF16), _ptr(K, "K", _BF16), _ptr(V, "V", _BF16),
                                  _ptr(LK, "LK", _BF16), _ptr(blk_out, "blk_out", _I32, True), _ptr(O, "O", _F32),
                                  _ptr(lse, "lse", _F32, True), ws.data_ptr(), nbytes, _stream(stream))
    _check(st, "hsa_forward_heads")


def hsa_sparse_set_kernel_events(start, stop):
    """start, stop: equal-length lists of raw hipEvent_t handles (ints; None
    entries are not recorded), or None to stop recording."""
    lib = load()
    if start is None:
        _check(lib.hsa_sparse_set_kernel_events(None, None, 0), "hsa_sparse_set_kernel_events")
        return
    n = len(start)
    a = (ctypes.c_void_p * n)(*start)
    b = (ctypes.c_void_p * n)(*stop)
    _check(lib.hsa_sparse_set_kernel_events(a, b, n), "hsa_sparse_set_kernel_events")


def hsa_sparse_last_kernels():
    return load().hsa_sparse_last_kernels().decode().split(",")


def hsa_sparse_set_stage_events(events):
    """events: 5 raw hipEvent_t handles (ints; None entries are not recorded),
    or None to stop recording."""
    lib = load()
    if events is None:
        _check(lib.hsa_sparse_set_stage_events(None, 0), "hsa_sparse_set_stage_events")
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib.hsa_sparse_set_stage_events(arr, len(events)), "hsa_sparse_set_stage_events")
