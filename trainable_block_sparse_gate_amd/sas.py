"""ctypes binding of ``libsas.so``: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module only
turns torch device tensors into pointers, allocates outputs with torch, and
passes torch's current stream.  It raises if the library is not built.

The library sees raw pointers, so before every call the binding checks each
tensor against the problem: dtype, device, contiguity and shape.  A tensor
that does not match raises SasError (SAS_ERR_NULL, _DTYPE or _SHAPE) and
nothing is launched.
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
SUMMARY_F32, SUMMARY_BF16, SUMMARY_FP8 = 0, 1, 2
BLOCK = 64
ABI_VERSION = 6  # the header's SAS_ABI_VERSION these structs follow

STATUS = {0: "SAS_OK", -1: "SAS_ERR_NULL", -2: "SAS_ERR_SHAPE", -3: "SAS_ERR_DTYPE",
          -4: "SAS_ERR_ALIGN", -5: "SAS_ERR_UNSUPPORTED", -6: "SAS_ERR_WORKSPACE",
          -7: "SAS_ERR_HIP"}

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = ["sas_gate_topk", "sas_fwd", "sas_bwd_workspace_size", "sas_bwd", "sas_bwd_prepare",
           "sas_bwd_dq", "sas_bwd_dkdv", "sas_gate_bwd",
           "sas_pool_keys", "sas_decode_append", "sas_decode_select_workspace_size",
           "sas_decode_select", "sas_pool_coarse", "sas_decode_select_hier_workspace_size",
           "sas_decode_select_hier", "sas_decode_workspace_size",
           "sas_decode", "sas_decode_noalloc",
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
        ("summary_dtype", ctypes.c_int32), ("page_table_host", ctypes.c_void_p),
        ("num_splits", ctypes.c_int32),
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
            "sas_decode_append": [DP, vp, vp, vp, vp, vp, vp, vp],
            "sas_pool_coarse": [DP, vp, vp, vp],
            "sas_decode_select_hier_workspace_size": [DP, i32],
            "sas_decode_select_hier": [DP, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp],
            "sas_decode_select_workspace_size": [DP],
            "sas_decode_select": [DP, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "sas_decode_workspace_size": [DP],
            "sas_decode": [DP, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "sas_decode_noalloc": [DP, vp, vp, vp, vp, vp, vp, vp, vp],
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
        L.sas_decode_select_workspace_size.restype = sz
        L.sas_decode_select_hier_workspace_size.restype = sz
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


ERR_NULL, ERR_SHAPE, ERR_DTYPE = -1, -2, -3


def _need(t, name, dtype, shape):
    """Check one tensor argument: a tensor of `dtype`, contiguous, of exactly
    `shape` (an entry None accepts any size along that axis).  That it is on
    the GPU is checked by _gpu, after every argument's dtype and shape."""
    import torch
    if t is None:
        raise SasError(ERR_NULL, f"{name} is None")
    if not isinstance(t, torch.Tensor):
        raise SasError(ERR_SHAPE, f"{name} must be a torch tensor (got {type(t).__name__})")
    if t.dtype != dtype:
        raise SasError(ERR_DTYPE, f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != len(shape) or any(w is not None and int(a) != int(w)
                                    for a, w in zip(t.shape, shape)):
        raise SasError(ERR_SHAPE, f"{name} has shape {tuple(t.shape)}, expected "
                       f"{tuple('*' if w is None else w for w in shape)}")
    if not t.is_contiguous():
        raise SasError(ERR_SHAPE, f"{name} must be contiguous")


def _gpu(*tensors):
    """Every tensor argument (None skipped) is on the same GPU."""
    devs = {t.device for t in tensors if t is not None}
    for dv in devs:
        if dv.type != "cuda":
            raise SasError(ERR_SHAPE, f"tensor arguments must be on a GPU (got {dv})")
    if len(devs) > 1:
        raise SasError(ERR_SHAPE, f"tensor arguments are on different devices: {sorted(map(str, devs))}")


def _torch_dtype(code):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}[code]


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
        return _torch_dtype(self.dtype if which == "in" else self.out_dtype)

    # argument checks (raise SasError before anything reaches the library)
    def check_logits(self, logits, name):
        import torch
        _need(logits, name, torch.float32, (self.hkv, self.QB, None))
        if logits.shape[-1] < max(1, self.max_blocks):
            raise SasError(ERR_SHAPE, f"{name}: row length {logits.shape[-1]} < blocks of the "
                           f"longest sequence ({self.max_blocks})")

    def check_selection(self, sel_idx, sel_lg):
        import torch
        _need(sel_idx, "sel_idx", torch.int32, (self.hkv, self.QB, self.Kb))
        _need(sel_lg, "sel_loggate", torch.float32, (self.hkv, self.QB, self.Kb))

    def check_qkv(self, q, k, v):
        dt = self.torch_dtype("in")
        _need(q, "q", dt, (self.T, self.hq, self.d))
        _need(k, "k", dt, (self.T, self.hkv, self.d))
        _need(v, "v", dt, (self.T, self.hkv, self.d))

    def check_bwd_inputs(self, q, k, v, o, dO, lse, sel_idx, sel_lg, workspace):
        import torch
        self.check_qkv(q, k, v)
        self.check_selection(sel_idx, sel_lg)
        _need(o, "o", self.torch_dtype("out"), (self.T, self.hq, self.d))
        _need(dO, "dO", self.torch_dtype("out"), (self.T, self.hq, self.d))
        _need(lse, "lse", torch.float32, (self.hq, self.T))
        _need(workspace, "workspace", torch.uint8, (None,))


def gate_topk(prob: Varlen, logits, mode=GATE_HIST, out=None):
    """sas_gate_topk -> (sel_idx int32 [hkv,QB,Kb], sel_loggate f32, gate_lse f32)."""
    import torch
    prob.check_logits(logits, "logits")
    dev = logits.device
    if out is None:
        out = (torch.empty((prob.hkv, prob.QB, prob.Kb), dtype=torch.int32, device=dev),
               torch.empty((prob.hkv, prob.QB, prob.Kb), dtype=torch.float32, device=dev),
               torch.empty((prob.hkv, prob.QB), dtype=torch.float32, device=dev))
    sel, lg, lse = out
    prob.check_logits(logits, "logits")
    prob.check_selection(sel, lg)
    _need(lse, "gate_lse", torch.float32, (prob.hkv, prob.QB))
    _gpu(logits, sel, lg, lse)
    _check(lib().sas_gate_topk(prob.ref, _ptr(logits), logits.shape[-1], mode, _ptr(sel),
                               _ptr(lg), _ptr(lse), _stream()))
    return sel, lg, lse


def fwd(prob: Varlen, q, k, v, sel_idx, sel_lg, out=None):
    """sas_fwd -> (o [T,hq,d] in the output dtype, lse f32 [hq,T])."""
    import torch
    prob.check_qkv(q, k, v)
    prob.check_selection(sel_idx, sel_lg)
    if out is None:
        out = (torch.empty((prob.T, prob.hq, prob.d), dtype=prob.torch_dtype("out"),
                           device=q.device),
               torch.empty((prob.hq, prob.T), dtype=torch.float32, device=q.device))
    o, lse = out
    _need(o, "o", prob.torch_dtype("out"), (prob.T, prob.hq, prob.d))
    _need(lse, "lse", torch.float32, (prob.hq, prob.T))
    _gpu(q, k, v, sel_idx, sel_lg, o, lse)
    _check(lib().sas_fwd(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(sel_idx), _ptr(sel_lg),
                         _ptr(o), _ptr(lse), _stream()))
    return o, lse


def bwd_workspace_bytes(prob: Varlen):
    return int(lib().sas_bwd_workspace_size(prob.ref))


def bwd(prob: Varlen, q, k, v, o, dO, lse, sel_idx, sel_lg, workspace=None):
    """sas_bwd -> (dq, dk, dv, d_loggate), all fp32."""
    import torch
    if workspace is not None:
        prob.check_bwd_inputs(q, k, v, o, dO, lse, sel_idx, sel_lg, workspace)
    else:
        prob.check_bwd_inputs(q, k, v, o, dO, lse, sel_idx, sel_lg,
                              torch.empty(0, dtype=torch.uint8))
    dev = q.device
    dq = torch.empty((prob.T, prob.hq, prob.d), dtype=torch.float32, device=dev)
    dk = torch.empty((prob.T, prob.hkv, prob.d), dtype=torch.float32, device=dev)
    dv = torch.empty((prob.T, prob.hkv, prob.d), dtype=torch.float32, device=dev)
    dlg = torch.empty(sel_idx.shape, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(prob), 1), dtype=torch.uint8, device=dev)
    _gpu(q, k, v, o, dO, lse, sel_idx, sel_lg, dq, dk, dv, dlg, workspace)
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
    import torch
    prob.check_bwd_inputs(q, k, v, o, dO, lse, sel_idx, sel_lg, workspace)
    _need(dq, "dq", torch.float32, (prob.T, prob.hq, prob.d))
    _need(dk, "dk", torch.float32, (prob.T, prob.hkv, prob.d))
    _need(dv, "dv", torch.float32, (prob.T, prob.hkv, prob.d))
    _need(dlg, "d_loggate", torch.float32, (prob.hkv, prob.QB, prob.Kb))
    _gpu(q, k, v, o, dO, lse, sel_idx, sel_lg, dq, dk, dv, dlg, workspace)
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
    prob.check_logits(logits, "logits")
    _need(sel_idx, "sel_idx", torch.int32, (prob.hkv, prob.QB, prob.Kb))
    _need(gate_lse, "gate_lse", torch.float32, (prob.hkv, prob.QB))
    _need(dlg, "d_loggate", torch.float32, (prob.hkv, prob.QB, prob.Kb))
    if out is None:
        out = torch.empty(logits.shape, dtype=torch.float32, device=logits.device)
    _need(out, "d_logits", torch.float32, tuple(logits.shape))
    _gpu(logits, sel_idx, gate_lse, dlg, out)
    _check(lib().sas_gate_bwd(prob.ref, _ptr(logits), logits.shape[-1], mode, _ptr(sel_idx),
                              _ptr(gate_lse), _ptr(dlg), _ptr(out), _stream()))
    return out


class Decode:
    """A decode problem: owns seqlens (device + host), the page table and
    the ctypes struct."""

    def __init__(self, seqlens, hq, hkv, head_dim, budget_blocks, paged, max_seqlen,
                 page_table=None, num_pages=0, out_dtype="bf16", scale=None, device="cuda",
                 nblk_stride=None, summary_dtype="f32", num_splits=0):
        import torch
        self.seqlens = [int(x) for x in seqlens]
        self.sl_host = np.array(self.seqlens, np.int32)
        self.sl_dev = torch.tensor(self.sl_host, device=device)
        self.hq, self.hkv, self.d, self.Kb = hq, hkv, head_dim, budget_blocks
        self.batch = len(self.seqlens)
        self.paged = paged
        # blocks per summary / score row: history blocks of the longest
        # sequence, rounded up to whole 64-block summary tiles
        self.nblk_stride = -(-max(1, max((n - 1) // BLOCK for n in self.seqlens)) // 64) * 64
        if nblk_stride is not None:
            self.nblk_stride = int(nblk_stride)
        self.pt_dev = None
        self.pt_host = None
        max_pages = 0
        if paged:
            pt = np.ascontiguousarray(page_table, np.int32)
            self.pt_host = pt
            self.pt_dev = torch.tensor(pt, device=device)
            max_pages = pt.shape[1]
        self.max_seqlen, self.num_pages = int(max_seqlen), int(num_pages)
        self.out_dtype = out_dtype
        self.scale = float(scale if scale is not None else 1.0 / np.sqrt(head_dim))
        self.s = DecodeProblem(
            self.batch, hq, hkv, head_dim, BLOCK, budget_blocks, SAS_BF16,
            SAS_BF16 if out_dtype == "bf16" else SAS_F32,
            KV_PAGED if paged else KV_CONTIGUOUS, max_seqlen, max_pages, num_pages,
            self.nblk_stride, self.scale, self.sl_dev.data_ptr(), self.sl_host.ctypes.data,
            self.pt_dev.data_ptr() if paged else None,
            {"f32": SUMMARY_F32, "bf16": SUMMARY_BF16, "fp8": SUMMARY_FP8}[summary_dtype],
            self.pt_host.ctypes.data if paged else None, int(num_splits))
        self.summary_dtype = summary_dtype

    # argument checks (raise SasError before anything reaches the library)
    def check_q(self, q):
        import torch
        _need(q, "q", torch.bfloat16, (self.batch, self.hq, self.d))

    def check_cache(self, cache, name):
        import torch
        if self.paged:
            _need(cache, name, torch.bfloat16, (self.num_pages, self.hkv, BLOCK, self.d))
        else:
            _need(cache, name, torch.bfloat16, (self.batch, self.hkv, self.max_seqlen, self.d))

    def summary_shape(self):
        """The tiled summary layout: [batch][hkv][tile of 64 blocks][16-byte
        piece][block in tile][channel in piece]."""
        epp = 16 // {"f32": 4, "bf16": 2, "fp8": 1}[self.summary_dtype]
        return (self.batch, self.hkv, self.nblk_stride // 64, self.d // epp, 64, epp)

    def coarse_shape(self):
        """Super-block summaries: the tiled layout with cstride super-blocks
        per row (nblk_stride / 8 rounded up to whole 64-entry tiles)."""
        epp = 16 // {"f32": 4, "bf16": 2, "fp8": 1}[self.summary_dtype]
        cstride = -(-(self.nblk_stride // COARSE_BLOCKS) // 64) * 64
        return (self.batch, self.hkv, cstride // 64, self.d // epp, 64, epp)

    def check_coarse(self, csum):
        _need(csum, "csum", _torch_dtype(self.summary_dtype), self.coarse_shape())

    def check_summaries(self, ksum):
        _need(ksum, "ksum", _torch_dtype(self.summary_dtype), self.summary_shape())

    def check_selection(self, sel_idx, sel_lg, lg_optional=False):
        import torch
        rows = self.batch * self.hkv
        _need(sel_idx, "sel_idx", torch.int32, (rows, self.Kb))
        if sel_lg is not None or not lg_optional:
            _need(sel_lg, "sel_loggate", torch.float32, (rows, self.Kb))

    @property
    def ref(self):
        return ctypes.byref(self.s)


def pool_keys(prob: Decode, k_cache):
    import torch
    prob.check_cache(k_cache, "k_cache")
    ksum = torch.empty(prob.summary_shape(),
                       dtype=_torch_dtype(prob.summary_dtype), device=k_cache.device)
    _gpu(k_cache, ksum)
    _check(lib().sas_pool_keys(prob.ref, _ptr(k_cache), _ptr(ksum), _stream()))
    return ksum


def summaries_by_block(ksum):
    """A [batch][hkv][block][channel] view (copy) of tiled summaries, for
    inspection: the library's layout is [batch][hkv][tile][piece][block in
    tile][channel in piece]."""
    B, hkv, nt, npc, bt, epp = ksum.shape
    return ksum.permute(0, 1, 2, 4, 3, 5).reshape(B, hkv, nt * bt, npc * epp)


def decode_append(prob: Decode, k_new, v_new, k_cache, v_cache, ksum, csum=None):
    """sas_decode_append: write the new token (prob.seqlens count it) into
    the caches and, when it opens a block, the finished block's summary (and,
    with csum, the summary of a super-block that block completes)."""
    import torch
    _need(k_new, "k_new", torch.bfloat16, (prob.batch, prob.hkv, prob.d))
    _need(v_new, "v_new", torch.bfloat16, (prob.batch, prob.hkv, prob.d))
    prob.check_cache(k_cache, "k_cache")
    prob.check_cache(v_cache, "v_cache")
    prob.check_summaries(ksum)
    if csum is not None:
        prob.check_coarse(csum)
    _gpu(k_new, v_new, k_cache, v_cache, ksum, csum)
    _check(lib().sas_decode_append(prob.ref, _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(ksum), _ptr(csum), _stream()))


COARSE_BLOCKS = 8  # the header's SAS_COARSE_BLOCKS


def pool_coarse(prob: Decode, ksum):
    """sas_pool_coarse -> super-block summaries (the tiled layout)."""
    import torch
    prob.check_summaries(ksum)
    csum = torch.empty(prob.coarse_shape(), dtype=_torch_dtype(prob.summary_dtype),
                       device=ksum.device)
    _gpu(ksum, csum)
    _check(lib().sas_pool_coarse(prob.ref, _ptr(ksum), _ptr(csum), _stream()))
    return csum


def decode_select_hier_workspace_bytes(prob: Decode, coarse_keep):
    return int(lib().sas_decode_select_hier_workspace_size(prob.ref, int(coarse_keep)))


def decode_select_hier(prob: Decode, q, ksum, csum, coarse_keep, out=None, workspace=None):
    """sas_decode_select_hier -> (sel_idx, sel_loggate, gate_lse, scores);
    scores are written for the candidate blocks only."""
    import torch
    prob.check_q(q)
    prob.check_summaries(ksum)
    prob.check_coarse(csum)
    dev = q.device
    rows = prob.batch * prob.hkv
    if out is None:
        out = (torch.empty((rows, prob.Kb), dtype=torch.int32, device=dev),
               torch.empty((rows, prob.Kb), dtype=torch.float32, device=dev),
               torch.empty((rows,), dtype=torch.float32, device=dev),
               torch.empty((prob.batch, prob.hkv, prob.nblk_stride), dtype=torch.float32,
                           device=dev))
    sel, lg, lse, scores = out
    prob.check_selection(sel, lg)
    _need(lse, "gate_lse", torch.float32, (rows,))
    _need(scores, "scores", torch.float32, (prob.batch, prob.hkv, prob.nblk_stride))
    if workspace is None:
        workspace = torch.empty(max(decode_select_hier_workspace_bytes(prob, coarse_keep), 1),
                                dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, (None,))
    _gpu(q, ksum, csum, sel, lg, lse, scores, workspace)
    _check(lib().sas_decode_select_hier(prob.ref, _ptr(q), _ptr(ksum), _ptr(csum),
                                        int(coarse_keep), _ptr(scores), _ptr(sel), _ptr(lg),
                                        _ptr(lse), _ptr(workspace), workspace.numel(),
                                        _stream()))
    return sel, lg, lse, scores


def decode_select_workspace_bytes(prob: Decode):
    return int(lib().sas_decode_select_workspace_size(prob.ref))


def decode_select_workspace(prob: Decode, device="cuda"):
    """A workspace for sas_decode_select (any contents; reusable)."""
    import torch
    return torch.empty(max(decode_select_workspace_bytes(prob), 1), dtype=torch.uint8,
                       device=device)


def decode_select(prob: Decode, q, ksum, out=None, workspace=None):
    """sas_decode_select -> (sel_idx, sel_loggate, gate_lse, scores)."""
    import torch
    prob.check_q(q)
    prob.check_summaries(ksum)
    dev = q.device
    rows = prob.batch * prob.hkv
    if out is None:
        out = (torch.empty((rows, prob.Kb), dtype=torch.int32, device=dev),
               torch.empty((rows, prob.Kb), dtype=torch.float32, device=dev),
               torch.empty((rows,), dtype=torch.float32, device=dev),
               torch.empty((prob.batch, prob.hkv, prob.nblk_stride), dtype=torch.float32,
                           device=dev))
    sel, lg, lse, scores = out
    prob.check_selection(sel, lg)
    _need(lse, "gate_lse", torch.float32, (rows,))
    _need(scores, "scores", torch.float32, (prob.batch, prob.hkv, prob.nblk_stride))
    if workspace is None:
        workspace = decode_select_workspace(prob, dev)
    _need(workspace, "workspace", torch.uint8, (None,))
    _gpu(q, ksum, sel, lg, lse, scores, workspace)
    _check(lib().sas_decode_select(prob.ref, _ptr(q), _ptr(ksum), _ptr(scores), _ptr(sel),
                                   _ptr(lg), _ptr(lse), _ptr(workspace), workspace.numel(),
                                   _stream()))
    return sel, lg, lse, scores


def decode_workspace_bytes(prob: Decode):
    return int(lib().sas_decode_workspace_size(prob.ref))


def decode(prob: Decode, q, k_cache, v_cache, sel_idx, sel_lg, workspace=None, out=None):
    """sas_decode -> (o [B,hq,d], lse f32 [B,hq])."""
    import torch
    prob.check_q(q)
    prob.check_cache(k_cache, "k_cache")
    prob.check_cache(v_cache, "v_cache")
    prob.check_selection(sel_idx, sel_lg, lg_optional=True)
    dev = q.device
    if out is None:
        out = (torch.empty((prob.batch, prob.hq, prob.d),
                           dtype=torch.bfloat16 if prob.out_dtype == "bf16" else torch.float32,
                           device=dev),
               torch.empty((prob.batch, prob.hq), dtype=torch.float32, device=dev))
    o, lse = out
    if workspace is None:
        workspace = torch.empty(max(decode_workspace_bytes(prob), 1), dtype=torch.uint8,
                                device=dev)
    _need(o, "o", _torch_dtype(prob.out_dtype), (prob.batch, prob.hq, prob.d))
    if lse is not None:
        _need(lse, "lse", torch.float32, (prob.batch, prob.hq))
    _need(workspace, "workspace", torch.uint8, (None,))
    _gpu(q, k_cache, v_cache, sel_idx, sel_lg, o, lse, workspace)
    _check(lib().sas_decode(prob.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sel_idx),
                            _ptr(sel_lg), _ptr(o), _ptr(lse), _ptr(workspace),
                            workspace.numel(), _stream()))
    return o, lse


DECODE_SCRATCH_BYTES = 4 << 20  # the header's SAS_DECODE_SCRATCH_BYTES


def decode_noalloc(prob: Decode, q, k_cache, v_cache, sel_idx, sel_lg, out):
    """sas_decode_noalloc into the caller's out = (o, lse): the library
    allocates nothing and takes no workspace (split partials go to its
    fixed per-device scratch)."""
    import torch
    prob.check_q(q)
    prob.check_cache(k_cache, "k_cache")
    prob.check_cache(v_cache, "v_cache")
    prob.check_selection(sel_idx, sel_lg, lg_optional=True)
    o, lse = out
    _need(o, "o", _torch_dtype(prob.out_dtype), (prob.batch, prob.hq, prob.d))
    if lse is not None:
        _need(lse, "lse", torch.float32, (prob.batch, prob.hq))
    _gpu(q, k_cache, v_cache, sel_idx, sel_lg, o, lse)
    _check(lib().sas_decode_noalloc(prob.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(sel_idx), _ptr(sel_lg), _ptr(o), _ptr(lse), _stream()))
    return o, lse
