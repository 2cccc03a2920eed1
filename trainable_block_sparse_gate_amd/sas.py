"""ctypes binding of ``libsas.so``: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module only
turns torch device tensors into pointers, allocates outputs with torch, and
passes torch's current stream.  It raises if the library is not built.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsas.so")

SAS_BF16, SAS_F32 = 0, 1
GATE_HIST, GATE_ALL, GATE_SIGMOID, GATE_RAW, GATE_STE = 0, 1, 2, 3, 4
GATE_INNER, GATE_OUTER = 0, 1  # gate position
KV_CONTIGUOUS, KV_PAGED = 0, 1
SUMMARY_F32, SUMMARY_BF16 = 0, 1
BLOCK = 64
ABI_VERSION = 2  # the header's SAS_ABI_VERSION these structs follow

STATUS = {0: "SAS_OK", -1: "SAS_ERR_NULL", -2: "SAS_ERR_SHAPE", -3: "SAS_ERR_DTYPE",
          -4: "SAS_ERR_ALIGN", -5: "SAS_ERR_UNSUPPORTED", -6: "SAS_ERR_WORKSPACE",
          -7: "SAS_ERR_HIP"}

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = ["sas_gate_topk", "sas_fwd", "sas_bwd_workspace_size", "sas_bwd", "sas_bwd_prepare",
           "sas_bwd_dq", "sas_bwd_dkdv", "sas_gate_bwd",
           "sas_pool_keys", "sas_decode_append", "sas_decode_select", "sas_decode_workspace_size", "sas_decode",
           "sas_status_string", "sas_last_error", "sas_abi_version"]


class SasError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
        ("total_qblocks", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
        ("budget_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("cu_seqlens", ctypes.c_void_p), ("cu_qblocks", ctypes.c_void_p),
        ("cu_seqlens_host", ctypes.c_void_p), ("cu_qblocks_host", ctypes.c_void_p),
        ("gate_position", ctypes.c_int32),
    ]


class DecodeProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
        ("budget_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("nblk_stride", ctypes.c_int32),
        ("scale", ctypes.c_float), ("seqlens", ctypes.c_void_p),
        ("seqlens_host", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
        ("summary_dtype", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Load libsas.so (in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with trainable_block_sparse_gate_amd.build "
                "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P, DP = ctypes.POINTER(Problem), ctypes.POINTER(DecodeProblem)
        sigs = {
            "sas_gate_topk": [P, vp, i64, i32, vp, vp, vp, vp],
            "sas_fwd": [P, vp, vp, vp, vp, vp, vp, vp, vp],
            "sas_bwd_workspace_size": [P],
            "sas_bwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "sas_bwd_prepare": [P, vp, vp, sz, vp],
            "sas_bwd_dq": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "sas_bwd_dkdv": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "sas_gate_bwd": [P, vp, i64, i32, vp, vp, vp, vp, vp],
            "sas_pool_keys": [DP, vp, vp, vp],
            "sas_decode_append": [DP, vp, vp, vp, vp, vp, vp],
            "sas_decode_select": [DP, vp, vp, vp, vp, vp, vp, vp],
            "sas_decode_workspace_size": [DP],
            "sas_decode": [DP, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "sas_status_string": [i32],
            "sas_last_error": [],
            "sas_abi_version": [],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = i32
        L.sas_bwd_workspace_size.restype = sz
        L.sas_decode_workspace_size.restype = sz
        L.sas_status_string.restype = ctypes.c_char_p
        L.sas_last_error.restype = ctypes.c_char_p
        if L.sas_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.sas_abi_version()}, the binding "
                               f"expects {ABI_VERSION}: rebuild the library")
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise SasError(status, lib().sas_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Varlen:
    """A packed varlen problem: owns the device and host copies of
    cu_seqlens / cu_qblocks and the ctypes struct that points at them."""

    def __init__(self, lengths, hq, hkv, head_dim, budget_blocks, dtype="bf16",
                 out_dtype=None, scale=None, device="cuda", gate_position=0):
        import torch
        self.lengths = [int(x) for x in lengths]
        cu = np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)
        nb = [(n + BLOCK - 1) // BLOCK for n in self.lengths]
        cuq = np.concatenate([[0], np.cumsum(nb)]).astype(np.int32)
        self.cu_host, self.cuq_host = cu, cuq
        self.cu_dev = torch.tensor(cu, device=device)
        self.cuq_dev = torch.tensor(cuq, device=device)
        self.hq, self.hkv, self.d, self.Kb = hq, hkv, head_dim, budget_blocks
        self.T, self.QB = int(cu[-1]), int(cuq[-1])
        self.max_blocks = max(nb) if nb else 0
        out_dtype = out_dtype or dtype
        self.dtype, self.out_dtype = dtype, out_dtype
        self.scale = float(scale if scale is not None else 1.0 / np.sqrt(head_dim))
        code = {"bf16": SAS_BF16, "f32": SAS_F32}
        self.s = Problem(len(self.lengths), self.T, self.QB, hq, hkv, head_dim, BLOCK,
                         budget_blocks, code[dtype], code[out_dtype], self.scale,
                         self.cu_dev.data_ptr(), self.cuq_dev.data_ptr(),
                         cu.ctypes.data, cuq.ctypes.data, int(gate_position))
        self.gate_position = int(gate_position)

    @property
    def ref(self):
        return ctypes.byref(self.s)

    def torch_dtype(self, which="in"):
        import torch
        d = self.dtype if which == "in" else self.out_dtype
        return torch.bfloat16 if d == "bf16" else torch.float32


def gate_topk(prob: Varlen, logits, mode=GATE_HIST, out=None):
    """sas_gate_topk -> (sel_idx int32 [hkv,QB,Kb], sel_loggate f32, gate_lse f32)."""
    import torch
    dev = logits.device
    if out is None:
        out = (torch.empty((prob.hkv, prob.QB, prob.Kb), dtype=torch.int32, device=dev),
               torch.empty((prob.hkv, prob.QB, prob.Kb), dtype=torch.float32, device=dev),
               torch.empty((prob.hkv, prob.QB), dtype=torch.float32, device=dev))
    sel, lg, lse = out
    _check(lib().sas_gate_topk(prob.ref, _ptr(logits), logits.shape[-1], mode, _ptr(sel),
                               _ptr(lg), _ptr(lse), _stream()))
    return sel, lg, lse


def fwd(prob: Varlen, q, k, v, sel_idx, sel_lg, out=None):
    """sas_fwd -> (o [T,hq,d] in the output dtype, lse f32 [hq,T])."""
    import torch
    if out is None:
        out = (torch.empty((prob.T, prob.hq, prob.d), dtype=prob.torch_dtype("out"),
                           device=q.device),
               torch.empty((prob.hq, prob.T), dtype=torch.float32, device=q.device))
    o, lse = out
    _check(lib().sas_fwd(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(sel_idx), _ptr(sel_lg),
                         _ptr(o), _ptr(lse), _stream()))
    return o, lse


def bwd_workspace_bytes(prob: Varlen):
    return int(lib().sas_bwd_workspace_size(prob.ref))


def bwd(prob: Varlen, q, k, v, o, dO, lse, sel_idx, sel_lg, workspace=None):
    """sas_bwd -> (dq, dk, dv, d_loggate), all fp32."""
    import torch
    dev = q.device
    dq = torch.empty((prob.T, prob.hq, prob.d), dtype=torch.float32, device=dev)
    dk = torch.empty((prob.T, prob.hkv, prob.d), dtype=torch.float32, device=dev)
    dv = torch.empty((prob.T, prob.hkv, prob.d), dtype=torch.float32, device=dev)
    dlg = torch.empty(sel_idx.shape, dtype=torch.float32, device=dev)
    nbytes = bwd_workspace_bytes(prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().sas_bwd(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                         _ptr(sel_idx), _ptr(sel_lg), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlg),
                         _ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dv, dlg


def bwd_phases(prob: Varlen, q, k, v, o, dO, lse, sel_idx, sel_lg, out, workspace,
               marks=None):
    """sas_bwd_prepare, sas_bwd_dq and sas_bwd_dkdv into preallocated
    outputs out = (dq, dk, dv, dlg).  `marks`, if given, is called with a
    phase name before each phase and with "end" after the last (used to
    record timing events between phases)."""
    dq, dk, dv, dlg = out
    L, st, ws, n = lib(), _stream(), _ptr(workspace), workspace.numel()
    if marks:
        marks("prepare")
    _check(L.sas_bwd_prepare(prob.ref, _ptr(sel_idx), ws, n, st))
    if marks:
        marks("dq")
    _check(L.sas_bwd_dq(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                        _ptr(sel_idx), _ptr(sel_lg), _ptr(dq), _ptr(dlg), ws, n, st))
    if marks:
        marks("dkdv")
    _check(L.sas_bwd_dkdv(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse),
                          _ptr(sel_lg), _ptr(dk), _ptr(dv), ws, n, st))
    if marks:
        marks("end")


def gate_bwd(prob: Varlen, logits, sel_idx, gate_lse, dlg, mode=GATE_HIST, out=None):
    """sas_gate_bwd -> d_logits f32, shaped like logits."""
    import torch
    if out is None:
        out = torch.empty(logits.shape, dtype=torch.float32, device=logits.device)
    _check(lib().sas_gate_bwd(prob.ref, _ptr(logits), logits.shape[-1], mode, _ptr(sel_idx),
                              _ptr(gate_lse), _ptr(dlg), _ptr(out), _stream()))
    return out


class Decode:
    """A decode problem: owns seqlens (device + host), the page table and
    the ctypes struct."""

    def __init__(self, seqlens, hq, hkv, head_dim, budget_blocks, paged, max_seqlen,
                 page_table=None, num_pages=0, out_dtype="bf16", scale=None, device="cuda",
                 nblk_stride=None, summary_dtype="f32"):
        import torch
        self.seqlens = [int(x) for x in seqlens]
        self.sl_host = np.array(self.seqlens, np.int32)
        self.sl_dev = torch.tensor(self.sl_host, device=device)
        self.hq, self.hkv, self.d, self.Kb = hq, hkv, head_dim, budget_blocks
        self.batch = len(self.seqlens)
        self.paged = paged
        # summary row stride: history blocks of the longest sequence, rounded
        # up to a multiple of 4 (the library then reads summaries as float4)
        self.nblk_stride = -(-max(1, max((n - 1) // BLOCK for n in self.seqlens)) // 4) * 4
        if nblk_stride is not None:
            self.nblk_stride = int(nblk_stride)
        self.pt_dev = None
        max_pages = 0
        if paged:
            pt = np.ascontiguousarray(page_table, np.int32)
            self.pt_dev = torch.tensor(pt, device=device)
            max_pages = pt.shape[1]
        self.out_dtype = out_dtype
        self.scale = float(scale if scale is not None else 1.0 / np.sqrt(head_dim))
        self.s = DecodeProblem(
            self.batch, hq, hkv, head_dim, BLOCK, budget_blocks, SAS_BF16,
            SAS_BF16 if out_dtype == "bf16" else SAS_F32,
            KV_PAGED if paged else KV_CONTIGUOUS, max_seqlen, max_pages, num_pages,
            self.nblk_stride, self.scale, self.sl_dev.data_ptr(), self.sl_host.ctypes.data,
            self.pt_dev.data_ptr() if paged else None,
            SUMMARY_BF16 if summary_dtype == "bf16" else SUMMARY_F32)
        self.summary_dtype = summary_dtype

    @property
    def ref(self):
        return ctypes.byref(self.s)


def pool_keys(prob: Decode, k_cache):
    import torch
    ksum = torch.empty((prob.batch, prob.hkv, prob.d, prob.nblk_stride),
                       dtype=torch.bfloat16 if prob.summary_dtype == "bf16" else torch.float32,
                       device=k_cache.device)
    _check(lib().sas_pool_keys(prob.ref, _ptr(k_cache), _ptr(ksum), _stream()))
    return ksum


def decode_append(prob: Decode, k_new, v_new, k_cache, v_cache, ksum):
    """sas_decode_append: write the new token (prob.seqlens count it) into
    the caches and, when it opens a block, the finished block's summary."""
    _check(lib().sas_decode_append(prob.ref, _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(ksum), _stream()))


def decode_select(prob: Decode, q, ksum, out=None):
    """sas_decode_select -> (sel_idx, sel_loggate, gate_lse, scores)."""
    import torch
    dev = q.device
    rows = prob.batch * prob.hkv
    if out is None:
        out = (torch.empty((rows, prob.Kb), dtype=torch.int32, device=dev),
               torch.empty((rows, prob.Kb), dtype=torch.float32, device=dev),
               torch.empty((rows,), dtype=torch.float32, device=dev),
               torch.empty((prob.batch, prob.hkv, prob.nblk_stride), dtype=torch.float32,
                           device=dev))
    sel, lg, lse, scores = out
    _check(lib().sas_decode_select(prob.ref, _ptr(q), _ptr(ksum), _ptr(scores), _ptr(sel),
                                   _ptr(lg), _ptr(lse), _stream()))
    return sel, lg, lse, scores


def decode_workspace_bytes(prob: Decode):
    return int(lib().sas_decode_workspace_size(prob.ref))


def decode(prob: Decode, q, k_cache, v_cache, sel_idx, sel_lg, workspace=None, out=None):
    """sas_decode -> (o [B,hq,d], lse f32 [B,hq])."""
    import torch
    dev = q.device
    if out is None:
        out = (torch.empty((prob.batch, prob.hq, prob.d),
                           dtype=torch.bfloat16 if prob.out_dtype == "bf16" else torch.float32,
                           device=dev),
               torch.empty((prob.batch, prob.hq), dtype=torch.float32, device=dev))
    o, lse = out
    nbytes = decode_workspace_bytes(prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().sas_decode(prob.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sel_idx),
                            _ptr(sel_lg), _ptr(o), _ptr(lse), _ptr(workspace),
                            workspace.numel(), _stream()))
    return o, lse
