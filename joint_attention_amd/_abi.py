"""Python binding of libjoint_attn (ctypes).  Argument marshalling only.

Every function here checks tensor placement/dtype/shape, allocates outputs with torch
when the caller gives none, and calls the C entry point of the same name on the
current HIP stream.  All arithmetic runs in the library's gfx950 kernels; there is no
fallback path.  If the shared library is missing, calls raise instead of computing.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# JOINT_ATTN_LIB overrides the shared object (e.g. an alternative build of the kernels)
LIB_PATH = os.environ.get("JOINT_ATTN_LIB") or os.path.join(HERE, "libjoint_attn.so")

JA_OK, JA_EINVAL, JA_EUNSUPPORTED, JA_EHIP, JA_ESCRATCH = 0, 1, 2, 3, 4
JA_LAYOUT_BHND, JA_LAYOUT_BHDN = 0, 1
JA_MAX_STREAMS = 16
JA_MAX_HEAD_ELEMS = 1 << 30
JA_QK_BLOCK = 128
JA_HI_CHANNELS = 16
JA_SPARSE_BLOCK, JA_SPARSE_MAX_N = 128, 131072
JA_SPARSE_PLAN_MAX = 2097152
JA_FP8_PLAIN, JA_FP8_SPLIT, JA_FP8_REPAIR = 0, 1, 2
JA_REPAIR_MAX_N = 131072
JA_REPAIR_TILE = 64
JA_SCRATCH_BYTES = 64 << 20

EXPORTS = ("joint_attn_strerror", "joint_attn_last_hip_error", "joint_attn_vt_ld",
           "joint_attn_pack", "joint_attn_fwd_bf16", "joint_attn_fwd_bf16_sparse",
           "joint_attn_sparse_plan_bytes", "joint_attn_sparse_plan",
           "joint_attn_fwd_bf16_sparse_planned",
           "joint_attn_fwd_bf16_splitkv", "joint_attn_fwd_bf16_splitkv_workspace",
           "joint_attn_fwd_bf16_splitkv_suggest", "joint_attn_fwd_bf16_splitkv_noalloc",
           "joint_attn_fwd_bf16_streams", "joint_attn_fwd_bf16_streams_splitkv",
           "joint_attn_fwd_bf16_streams_splitkv_workspace",
           "joint_attn_quant_fp8", "joint_attn_quant_fp8_streams",
           "joint_attn_fwd_fp8", "joint_attn_fwd_fp8_splitkv", "joint_attn_fwd_fp8_splitkv_workspace",
           "joint_attn_fwd_fp8_splitkv_suggest", "joint_attn_repair_count",
           "joint_attn_quant_fp8_repair",
           "joint_attn_fwd_fp8_repair")

_lock = threading.Lock()
_lib = None


class JointAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        lib_ = _lib
        msg = lib_.joint_attn_strerror(status).decode() if lib_ is not None else str(status)
        extra = " (hipError %d)" % hip_error if status == JA_EHIP else ""
        super().__init__("%s failed: %s%s" % (fn, msg, extra))
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library once and declare every export's signature."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libjoint_attn.so is not built (%s); run "
                               "`python -m joint_attention_amd.build`" % path)
        # torch first: it ships its own HIP runtime under the same soname as the system's,
        # and the first one loaded serves the whole process (the library's dependency
        # resolved first would leave torch without a usable runtime)
        import torch  # noqa: F401
        h = ctypes.CDLL(path)
        P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        h.joint_attn_strerror.restype = ctypes.c_char_p
        h.joint_attn_strerror.argtypes = [I]
        h.joint_attn_last_hip_error.restype = I
        h.joint_attn_last_hip_error.argtypes = []
        h.joint_attn_vt_ld.restype = I64
        h.joint_attn_vt_ld.argtypes = [I64]
        h.joint_attn_pack.restype = I
        h.joint_attn_pack.argtypes = [I, P, P, I, I, I, I, I64, P, P, P]
        h.joint_attn_fwd_bf16.restype = I
        h.joint_attn_fwd_bf16.argtypes = [P, P, P, I, I, I64, I, I64, F, P, P, P]
        h.joint_attn_fwd_bf16_sparse.restype = I
        h.joint_attn_fwd_bf16_sparse.argtypes = [P, P, P, I, I, I64, I, I64, P, F, P, P, P]
        h.joint_attn_sparse_plan_bytes.restype = I64
        h.joint_attn_sparse_plan_bytes.argtypes = [I, I, I64]
        h.joint_attn_sparse_plan.restype = I
        h.joint_attn_sparse_plan.argtypes = [P, I, I, I64, P, I64, P]
        h.joint_attn_fwd_bf16_sparse_planned.restype = I
        h.joint_attn_fwd_bf16_sparse_planned.argtypes = [P, P, P, I, I, I64, I, I64, P, P, F, P,
                                                         P, P]
        h.joint_attn_fwd_bf16_splitkv_workspace.restype = I64
        h.joint_attn_fwd_bf16_splitkv_workspace.argtypes = [I, I, I64, I, I]
        h.joint_attn_fwd_bf16_splitkv_suggest.restype = I
        h.joint_attn_fwd_bf16_splitkv_suggest.argtypes = [I, I, I64, I]
        h.joint_attn_fwd_bf16_splitkv.restype = I
        h.joint_attn_fwd_bf16_splitkv.argtypes = [P, P, P, I, I, I64, I, I64, F, I, P, I64, P, P,
                                                  P]
        h.joint_attn_fwd_bf16_splitkv_noalloc.restype = I
        h.joint_attn_fwd_bf16_splitkv_noalloc.argtypes = [P, P, P, I, I, I64, I, I64, F, I, P, P,
                                                          P]
        h.joint_attn_fwd_bf16_streams.restype = I
        h.joint_attn_fwd_bf16_streams.argtypes = [I, P, P, P, P, I, I, I, F,
                                                  P, P, P, P]
        h.joint_attn_fwd_bf16_streams_splitkv_workspace.restype = I64
        h.joint_attn_fwd_bf16_streams_splitkv_workspace.argtypes = [I, I, I64, I, I, I]
        h.joint_attn_fwd_bf16_streams_splitkv.restype = I
        h.joint_attn_fwd_bf16_streams_splitkv.argtypes = [I, P, P, P, P, I, I, I, F, I, I, P, I64,
                                                          P, P, P, P]
        h.joint_attn_quant_fp8.restype = I
        h.joint_attn_quant_fp8.argtypes = [P, P, P, I, I, I64, I, I64, I, P, P, P, P, P, P,
                                           P, P, P, P, P]
        h.joint_attn_quant_fp8_streams.restype = I
        h.joint_attn_quant_fp8_streams.argtypes = [I, P, P, P, P, I, I, I, I64, I, P, P, P, P, P,
                                                   P, P, P, P, P, P, P]
        h.joint_attn_fwd_fp8.restype = I
        h.joint_attn_fwd_fp8.argtypes = [P, P, P, P, P, P, I, I, I64, I, I64, F, I, P, P, P, P,
                                         P]
        h.joint_attn_fwd_fp8_splitkv_workspace.restype = I64
        h.joint_attn_fwd_fp8_splitkv_workspace.argtypes = [I, I, I64, I, I]
        h.joint_attn_fwd_fp8_splitkv_suggest.restype = I
        h.joint_attn_fwd_fp8_splitkv_suggest.argtypes = [I, I, I64, I, I]
        h.joint_attn_fwd_fp8_splitkv.restype = I
        h.joint_attn_fwd_fp8_splitkv.argtypes = [P, P, P, P, P, P, I, I, I64, I, I64, F, I, P, P, I,
                                                 P, I64, P, P, P]
        h.joint_attn_repair_count.restype = I64
        h.joint_attn_repair_count.argtypes = [I64, ctypes.c_double]
        h.joint_attn_quant_fp8_repair.restype = I
        h.joint_attn_quant_fp8_repair.argtypes = [P, P, P, I, I, I64, I, I64, I64, P, P, P, P, P,
                                                  P, P, P, P, P, P, P]
        h.joint_attn_fwd_fp8_repair.restype = I
        h.joint_attn_fwd_fp8_repair.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I64, I, I, I64,
                                                I, I64, F, P, P, P]
        _lib = h
        return h


def _check(fn: str, status: int):
    if status != JA_OK:
        raise JointAttnError(fn, status, load().joint_attn_last_hip_error())


def _torch():
    import torch
    return torch


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, dtype, name: str, ndim: int):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-D tensor" % (name, ndim))


def joint_attn_vt_ld(N: int) -> int:
    return int(load().joint_attn_vt_ld(int(N)))


def joint_attn_pack(streams, layout: str = "bhnd", ld: int | None = None, out=None):
    """Concatenate per-stream bf16 [B, L_s, H, D] tensors along tokens.

    layout "bhnd" -> [B, H, N, D] (Q, K); "bhdn" -> [B, H, D, ld] (V; ld defaults to
    joint_attn_vt_ld(N), padding zeroed).  Returns (packed, offsets list of n+1 ints).
    """
    torch = _torch()
    streams = list(streams)
    if not 1 <= len(streams) <= JA_MAX_STREAMS:
        raise ValueError("need 1..%d streams" % JA_MAX_STREAMS)
    for i, s in enumerate(streams):
        _need(s, torch.bfloat16, "stream %d" % i, 4)
    B, _, H, D = streams[0].shape
    for s in streams:
        if s.shape[0] != B or s.shape[2] != H or s.shape[3] != D or s.device != streams[0].device:
            raise ValueError("streams must share B, H, D and the device")
    N = sum(int(s.shape[1]) for s in streams)
    lay = {"bhnd": JA_LAYOUT_BHND, "bhdn": JA_LAYOUT_BHDN}[layout]
    if lay == JA_LAYOUT_BHDN:
        ld = joint_attn_vt_ld(N) if ld is None else int(ld)
        shape = (B, H, D, ld)
    else:
        ld = 0
        shape = (B, H, N, D)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=streams[0].device)
    elif tuple(out.shape) != shape:
        raise ValueError("out must have shape %s" % (shape,))
    _need(out, torch.bfloat16, "out", 4)
    ptrs = (ctypes.c_void_p * len(streams))(*[s.data_ptr() if s.numel() else None for s in streams])
    lens = (ctypes.c_int64 * len(streams))(*[int(s.shape[1]) for s in streams])
    offs = (ctypes.c_int64 * (len(streams) + 1))()
    st = load().joint_attn_pack(len(streams), ptrs, lens, B, H, D, lay, ld,
                                out.data_ptr() if out.numel() else None, offs, _stream(out))
    _check("joint_attn_pack", st)
    return out, list(offs)


def joint_attn_fwd_bf16(q, k, vt, softmax_scale: float | None = None, out=None,
                        return_lse: bool = False):
    """q, k: bf16 [B, H, N, D]; vt: bf16 [B, H, D, ldv].  Returns O [B, N, H, D]
    (and lse [B, H, N] fp32 if asked)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.bfloat16, n, 4)
    B, H, N, D = q.shape
    if tuple(k.shape) != (B, H, N, D) or vt.shape[:3] != (B, H, D):
        raise ValueError("k must match q; vt must be [B, H, D, ldv]")
    ldv = int(vt.shape[3])
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out", 4)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    st = load().joint_attn_fwd_bf16(q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H, N, D, ldv,
                                    scale, out.data_ptr(),
                                    lse.data_ptr() if lse is not None else None, _stream(q))
    _check("joint_attn_fwd_bf16", st)
    return (out, lse) if return_lse else out


def joint_attn_fwd_bf16_sparse(q, k, vt, block_mask, softmax_scale: float | None = None,
                               out=None, return_lse: bool = False):
    """Block-sparse attention: q, k bf16 [B, H, N, D]; vt bf16 [B, H, D, ldv]; block_mask
    uint8 [B, H, nb, nb] with nb = ceil(N / JA_SPARSE_BLOCK), nonzero = attended.  Returns
    O [B, N, H, D] (and lse [B, H, N])."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.bfloat16, n, 4)
    B, H, N, D = q.shape
    nb = -(-N // JA_SPARSE_BLOCK)
    _need(block_mask, torch.uint8, "block_mask", 4)
    if tuple(block_mask.shape) != (B, H, nb, nb):
        raise ValueError("block_mask must be [B, H, %d, %d]" % (nb, nb))
    if tuple(k.shape) != (B, H, N, D) or vt.shape[:3] != (B, H, D):
        raise ValueError("k must match q; vt must be [B, H, D, ldv]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out", 4)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    st = load().joint_attn_fwd_bf16_sparse(q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H, N, D,
                                           int(vt.shape[3]), block_mask.data_ptr(), scale,
                                           out.data_ptr(), _ptr(lse), _stream(q))
    _check("joint_attn_fwd_bf16_sparse", st)
    return (out, lse) if return_lse else out


def joint_attn_sparse_plan(block_mask, N: int, out=None):
    """Dispatch plan of joint_attn_fwd_bf16_sparse_planned for a uint8 block mask
    [B, H, nb, nb] (nb = ceil(N / JA_SPARSE_BLOCK)): an int32 tensor [B * H * nb]."""
    torch = _torch()
    _need(block_mask, torch.uint8, "block_mask", 4)
    B, H, nb = int(block_mask.shape[0]), int(block_mask.shape[1]), -(-int(N) // JA_SPARSE_BLOCK)
    if tuple(block_mask.shape) != (B, H, nb, nb):
        raise ValueError("block_mask must be [B, H, %d, %d]" % (nb, nb))
    nbytes = int(load().joint_attn_sparse_plan_bytes(B, H, int(N)))
    if nbytes < 0:
        raise ValueError("no plan for B=%d H=%d N=%d (limits JA_SPARSE_MAX_N, JA_SPARSE_PLAN_MAX)"
                         % (B, H, N))
    if out is None:
        out = torch.empty((nbytes // 4,), dtype=torch.int32, device=block_mask.device)
    _need(out, torch.int32, "out", 1)
    st = load().joint_attn_sparse_plan(block_mask.data_ptr(), B, H, int(N), out.data_ptr(),
                                       out.numel() * 4, _stream(block_mask))
    _check("joint_attn_sparse_plan", st)
    return out


def joint_attn_fwd_bf16_sparse_planned(q, k, vt, block_mask, plan,
                                       softmax_scale: float | None = None, out=None,
                                       return_lse: bool = False):
    """joint_attn_fwd_bf16_sparse with the workgroup order of joint_attn_sparse_plan
    (same results, bit for bit).  plan: int32 [B * H * nb] from that call."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.bfloat16, n, 4)
    B, H, N, D = q.shape
    nb = -(-N // JA_SPARSE_BLOCK)
    _need(block_mask, torch.uint8, "block_mask", 4)
    _need(plan, torch.int32, "plan", 1)
    if tuple(block_mask.shape) != (B, H, nb, nb):
        raise ValueError("block_mask must be [B, H, %d, %d]" % (nb, nb))
    if plan.numel() != B * H * nb:
        raise ValueError("plan must have B * H * nb = %d entries" % (B * H * nb))
    if tuple(k.shape) != (B, H, N, D) or vt.shape[:3] != (B, H, D):
        raise ValueError("k must match q; vt must be [B, H, D, ldv]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out", 4)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    st = load().joint_attn_fwd_bf16_sparse_planned(
        q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H, N, D, int(vt.shape[3]),
        block_mask.data_ptr(), plan.data_ptr(), scale, out.data_ptr(), _ptr(lse), _stream(q))
    _check("joint_attn_fwd_bf16_sparse_planned", st)
    return (out, lse) if return_lse else out


def joint_attn_fwd_bf16_splitkv(q, k, vt, softmax_scale: float | None = None,
                                n_split: int | None = None, workspace=None, out=None,
                                return_lse: bool = False):
    """joint_attn_fwd_bf16 with split keys (for grids too small to fill the GPU).  n_split
    defaults to the library's suggestion; workspace (a device tensor of at least the
    required bytes) is allocated here if not given."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.bfloat16, n, 4)
    B, H, N, D = q.shape
    if tuple(k.shape) != (B, H, N, D) or vt.shape[:3] != (B, H, D):
        raise ValueError("k must match q; vt must be [B, H, D, ldv]")
    lib = load()
    if n_split is None:
        n_split = lib.joint_attn_fwd_bf16_splitkv_suggest(B, H, N, D)
    need = int(lib.joint_attn_fwd_bf16_splitkv_workspace(B, H, N, D, int(n_split)))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out", 4)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib.joint_attn_fwd_bf16_splitkv(q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H, N, D,
                                         int(vt.shape[3]), scale, int(n_split),
                                         workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(),
                                         out.data_ptr(), _ptr(lse), _stream(q))
    _check("joint_attn_fwd_bf16_splitkv", st)
    return (out, lse) if return_lse else out


def joint_attn_fwd_bf16_splitkv_noalloc(q, k, vt, softmax_scale: float | None = None,
                                        n_split: int | None = None, out=None, lse=None):
    """joint_attn_fwd_bf16_splitkv with the partial results in the library's static scratch
    (no workspace; the library allocates nothing).  Pass `out` (and `lse`, fp32
    [B, H, N], if wanted) to allocate nothing here either."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.bfloat16, n, 4)
    B, H, N, D = q.shape
    if tuple(k.shape) != (B, H, N, D) or vt.shape[:3] != (B, H, D):
        raise ValueError("k must match q; vt must be [B, H, D, ldv]")
    lib = load()
    if n_split is None:
        n_split = lib.joint_attn_fwd_bf16_splitkv_suggest(B, H, N, D)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out", 4)
    if lse is not None:
        _need(lse, torch.float32, "lse", 3)
    st = lib.joint_attn_fwd_bf16_splitkv_noalloc(q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H,
                                                 N, D, int(vt.shape[3]), scale, int(n_split),
                                                 out.data_ptr(), _ptr(lse), _stream(q))
    _check("joint_attn_fwd_bf16_splitkv_noalloc", st)
    return out


def _streams(q_streams, k_streams, v_streams):
    """Checks of per-stream bf16 [B, L_s, H, D] tensors; returns (lists, B, H, D, N, ctypes
    pointer arrays and lengths)."""
    torch = _torch()
    qs, ks, vs = list(q_streams), list(k_streams), list(v_streams)
    n = len(qs)
    if not 1 <= n <= JA_MAX_STREAMS or len(ks) != n or len(vs) != n:
        raise ValueError("need 1..%d streams, the same number for q, k and v" % JA_MAX_STREAMS)
    B, _, H, D = qs[0].shape
    dev = qs[0].device
    for i in range(n):
        for t, nm in ((qs[i], "q"), (ks[i], "k"), (vs[i], "v")):
            _need(t, torch.bfloat16, "%s stream %d" % (nm, i), 4)
            if (t.shape[0], t.shape[2], t.shape[3]) != (B, H, D) or t.shape[1] != qs[i].shape[1] \
                    or t.device != dev:
                raise ValueError("streams must share B, H, D, lengths per stream and device")
    N = sum(int(x.shape[1]) for x in qs)
    ptr = lambda lst: (ctypes.c_void_p * n)(*[x.data_ptr() if x.numel() else None for x in lst])
    lens = (ctypes.c_int64 * n)(*[int(x.shape[1]) for x in qs])
    return qs, B, H, D, N, dev, ptr(qs), ptr(ks), ptr(vs), lens


def joint_attn_fwd_bf16_streams(q_streams, k_streams, v_streams,
                                softmax_scale: float | None = None, out=None,
                                return_lse: bool = False):
    """Attention over the concatenation of per-stream bf16 [B, L_s, H, D] tensors, read in
    place.  Returns (O [B, N, H, D], offsets) (and lse [B, H, N] if asked)."""
    torch = _torch()
    qs, B, H, D, N, dev, pq, pk, pv, lens = _streams(q_streams, k_streams, v_streams)
    n = len(qs)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", 4)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_lse else None
    offs = (ctypes.c_int64 * (n + 1))()
    st = load().joint_attn_fwd_bf16_streams(n, pq, pk, pv, lens, B, H, D, scale,
                                            out.data_ptr() if out.numel() else None,
                                            lse.data_ptr() if lse is not None else None, offs,
                                            _stream(out))
    _check("joint_attn_fwd_bf16_streams", st)
    return (out, list(offs), lse) if return_lse else (out, list(offs))


def joint_attn_fwd_bf16_streams_splitkv(q_streams, k_streams, v_streams,
                                        softmax_scale: float | None = None,
                                        n_split: int | None = None, pack_v: int = 1,
                                        workspace=None, out=None, return_lse: bool = False):
    """joint_attn_fwd_bf16_streams with split keys.  pack_v = 1 transposes V into the
    workspace first (faster forward), 0 reads V in place too.  n_split defaults to the
    library's suggestion; the workspace is allocated here if not given.  Returns
    (O, offsets) (and lse if asked)."""
    torch = _torch()
    qs, B, H, D, N, dev, pq, pk, pv, lens = _streams(q_streams, k_streams, v_streams)
    n = len(qs)
    lib = load()
    if n_split is None:
        n_split = lib.joint_attn_fwd_bf16_splitkv_suggest(B, H, N, D)
    need = int(lib.joint_attn_fwd_bf16_streams_splitkv_workspace(B, H, N, D, int(n_split),
                                                                 int(pack_v)))
    if need < 0:
        raise ValueError("invalid sizes, n_split or pack_v")
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", 4)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_lse else None
    offs = (ctypes.c_int64 * (n + 1))()
    st = lib.joint_attn_fwd_bf16_streams_splitkv(
        n, pq, pk, pv, lens, B, H, D, scale, int(n_split), int(pack_v), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), out.data_ptr() if out.numel() else None,
        lse.data_ptr() if lse is not None else None, offs, _stream(out))
    _check("joint_attn_fwd_bf16_streams_splitkv", st)
    return (out, list(offs), lse) if return_lse else (out, list(offs))


class Fp8Tensors:
    """Outputs of joint_attn_quant_fp8 (device tensors); the split-mode fields are None
    outside mode 1, the token-repair fields (q_err, k_err, q_sel, k_sel, n_repair and the
    unquantised q, k the forward needs) None outside mode 2."""

    def __init__(self, mode, q8, k8, v8t, q_scale, k_scale, v_scale, q_hi=None, k_hi=None,
                 hi_idx=None, ch_amax=None):
        self.mode = mode
        self.q8, self.k8, self.v8t = q8, k8, v8t
        self.q_scale, self.k_scale, self.v_scale = q_scale, k_scale, v_scale
        self.q_hi, self.k_hi, self.hi_idx, self.ch_amax = q_hi, k_hi, hi_idx, ch_amax
        self.q_err = self.k_err = self.q_sel = self.k_sel = self.v8t_sel = None
        self.q_src = self.k_src = None
        self.n_repair = 0


def _ptr(t):
    return t.data_ptr() if t is not None else None


def joint_attn_quant_fp8(q, k, vt, mode: int = JA_FP8_PLAIN, out: Fp8Tensors | None = None
                         ) -> Fp8Tensors:
    """q, k: bf16 [B, H, N, D]; vt: bf16 [B, H, D, ldv] -> Fp8Tensors (codes as uint8).
    `out` (from an earlier call with the same shapes and mode) is reused if given."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.bfloat16, n, 4)
    B, H, N, D = q.shape
    ldv = int(vt.shape[3])
    dev = q.device
    nblk = -(-N // JA_QK_BLOCK)
    if out is not None:
        if (out.mode != mode or tuple(out.q8.shape) != (B, H, N, D)
                or tuple(out.v8t.shape) != (B, H, D, ldv)):
            raise ValueError("joint_attn_quant_fp8: `out` does not match the inputs or mode")
    else:
        out = _alloc_fp8(mode, B, H, N, D, ldv, nblk, dev)
    st = load().joint_attn_quant_fp8(
        q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H, N, D, ldv, int(mode),
        out.q8.data_ptr(), out.k8.data_ptr(), out.v8t.data_ptr(), out.q_scale.data_ptr(),
        out.k_scale.data_ptr(), out.v_scale.data_ptr(), _ptr(out.q_hi), _ptr(out.k_hi),
        _ptr(out.hi_idx), _ptr(out.ch_amax), _stream(q))
    _check("joint_attn_quant_fp8", st)
    return out


def joint_attn_quant_fp8_streams(q_streams, k_streams, v_streams, mode: int = JA_FP8_PLAIN,
                                 out: Fp8Tensors | None = None):
    """joint_attn_quant_fp8 on the concatenation of per-stream bf16 [B, L_s, H, D] tensors,
    read in place.  Returns (Fp8Tensors, offsets)."""
    torch = _torch()
    qs, ks, vs = list(q_streams), list(k_streams), list(v_streams)
    n = len(qs)
    if not 1 <= n <= JA_MAX_STREAMS or len(ks) != n or len(vs) != n:
        raise ValueError("need 1..%d streams, the same number for q, k and v" % JA_MAX_STREAMS)
    B, _, H, D = qs[0].shape
    dev = qs[0].device
    for i in range(n):
        for t, nm in ((qs[i], "q"), (ks[i], "k"), (vs[i], "v")):
            _need(t, torch.bfloat16, "%s stream %d" % (nm, i), 4)
            if (t.shape[0], t.shape[2], t.shape[3]) != (B, H, D) or t.shape[1] != qs[i].shape[1] \
                    or t.device != dev:
                raise ValueError("streams must share B, H, D, lengths per stream and device")
    N = sum(int(x.shape[1]) for x in qs)
    ldv = joint_attn_vt_ld(N)
    nblk = -(-N // JA_QK_BLOCK)
    if out is not None:
        if out.mode != mode or tuple(out.q8.shape) != (B, H, N, D) \
                or tuple(out.v8t.shape) != (B, H, D, ldv):
            raise ValueError("joint_attn_quant_fp8_streams: `out` does not match the inputs or mode")
    else:
        out = _alloc_fp8(mode, B, H, N, D, ldv, nblk, dev)
    ptr = lambda lst: (ctypes.c_void_p * n)(*[x.data_ptr() if x.numel() else None for x in lst])
    lens = (ctypes.c_int64 * n)(*[int(x.shape[1]) for x in qs])
    offs = (ctypes.c_int64 * (n + 1))()
    st = load().joint_attn_quant_fp8_streams(
        n, ptr(qs), ptr(ks), ptr(vs), lens, B, H, D, ldv, int(mode), _ptr(out.q8), _ptr(out.k8),
        _ptr(out.v8t), _ptr(out.q_scale), _ptr(out.k_scale), _ptr(out.v_scale), _ptr(out.q_hi),
        _ptr(out.k_hi), _ptr(out.hi_idx), _ptr(out.ch_amax), offs, _stream(qs[0]))
    _check("joint_attn_quant_fp8_streams", st)
    return out, list(offs)


def _alloc_fp8(mode, B, H, N, D, ldv, nblk, dev) -> Fp8Tensors:
    torch = _torch()
    out = Fp8Tensors(
        mode,
        torch.empty((B, H, N, D), dtype=torch.uint8, device=dev),
        torch.empty((B, H, N, D), dtype=torch.uint8, device=dev),
        torch.empty((B, H, D, ldv), dtype=torch.uint8, device=dev),
        torch.empty((B, H, nblk), dtype=torch.float32, device=dev),
        torch.empty((B, H, nblk), dtype=torch.float32, device=dev),
        torch.empty((B, H, D), dtype=torch.float32, device=dev))
    if mode == JA_FP8_SPLIT:
        out.q_hi = torch.empty((B, H, N, JA_HI_CHANNELS), dtype=torch.bfloat16, device=dev)
        out.k_hi = torch.empty((B, H, N, JA_HI_CHANNELS), dtype=torch.bfloat16, device=dev)
        out.hi_idx = torch.empty((B, H, JA_HI_CHANNELS), dtype=torch.int32, device=dev)
        out.ch_amax = torch.empty((B, H, 2, D), dtype=torch.float32, device=dev)
    return out


def joint_attn_fwd_fp8_splitkv(t: Fp8Tensors, softmax_scale: float | None = None,
                               n_split: int | None = None, workspace=None, out=None,
                               return_lse: bool = False):
    """joint_attn_fwd_fp8 (modes 0 and 1) with the last round's query tiles split into
    key ranges.  n_split defaults to the library's suggestion; workspace (a device tensor
    of at least the required bytes) is allocated here if not given."""
    torch = _torch()
    if t.mode not in (JA_FP8_PLAIN, JA_FP8_SPLIT):
        raise ValueError("joint_attn_fwd_fp8_splitkv: modes 0 and 1 only")
    for x, n in ((t.q8, "q8"), (t.k8, "k8"), (t.v8t, "v8t")):
        _need(x, torch.uint8, n, 4)
    B, H, N, D = t.q8.shape
    ldv = int(t.v8t.shape[3])
    lib = load()
    if n_split is None:
        n_split = lib.joint_attn_fwd_fp8_splitkv_suggest(B, H, N, D, int(t.mode))
    need = int(lib.joint_attn_fwd_fp8_splitkv_workspace(B, H, N, D, int(n_split)))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=t.q8.device)
    if workspace.device != t.q8.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=t.q8.device)
    _need(out, torch.bfloat16, "out", 4)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=t.q8.device) if return_lse else None
    st = lib.joint_attn_fwd_fp8_splitkv(
        t.q8.data_ptr(), t.k8.data_ptr(), t.v8t.data_ptr(), t.q_scale.data_ptr(),
        t.k_scale.data_ptr(), t.v_scale.data_ptr(), B, H, N, D, ldv, scale, int(t.mode),
        _ptr(t.q_hi), _ptr(t.k_hi), int(n_split), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), out.data_ptr(), _ptr(lse), _stream(t.q8))
    _check("joint_attn_fwd_fp8_splitkv", st)
    return (out, lse) if return_lse else out


def joint_attn_repair_count(N: int, rho: float) -> int:
    """Tokens repaired per (b, h) and operand: ceil(rho * N)."""
    n = int(load().joint_attn_repair_count(int(N), float(rho)))
    if n < 0:
        raise ValueError("joint_attn_repair_count: need N >= 0 and 0 <= rho <= 1")
    return n


def joint_attn_quant_fp8_repair(q, k, vt, rho: float = 0.005, out: Fp8Tensors | None = None
                                ) -> Fp8Tensors:
    """Token-repair quantisation (mode JA_FP8_REPAIR): the plain codes and scales plus,
    per (b, h) and operand, the ceil(rho N) tokens of largest residual.  The result keeps
    q and k (the forward reads the repaired tokens' exact values from them)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.bfloat16, n, 4)
    B, H, N, D = q.shape
    ldv = int(vt.shape[3])
    n_rep = joint_attn_repair_count(N, rho)
    nblk = -(-N // JA_QK_BLOCK)
    if out is not None:
        if (out.mode != JA_FP8_REPAIR or tuple(out.q8.shape) != (B, H, N, D)
                or tuple(out.v8t.shape) != (B, H, D, ldv) or out.n_repair != n_rep):
            raise ValueError("joint_attn_quant_fp8_repair: `out` does not match the inputs")
    else:
        out = _alloc_fp8(JA_FP8_REPAIR, B, H, N, D, ldv, nblk, q.device)
        out.q_err = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        out.k_err = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        out.q_sel = torch.empty((B, H, n_rep), dtype=torch.int32, device=q.device)
        out.k_sel = torch.empty((B, H, n_rep), dtype=torch.int32, device=q.device)
        ldr = -(-n_rep // JA_REPAIR_TILE) * JA_REPAIR_TILE
        out.v8t_sel = torch.empty((B, H, D, ldr), dtype=torch.uint8, device=q.device)
        out.n_repair = n_rep
    out.q_src, out.k_src = q, k
    st = load().joint_attn_quant_fp8_repair(
        q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, H, N, D, ldv, n_rep,
        out.q8.data_ptr(), out.k8.data_ptr(), out.v8t.data_ptr(), out.q_scale.data_ptr(),
        out.k_scale.data_ptr(), out.v_scale.data_ptr(), out.q_err.data_ptr(),
        out.k_err.data_ptr(), _ptr(out.q_sel) if n_rep else None,
        _ptr(out.k_sel) if n_rep else None, _ptr(out.v8t_sel) if n_rep else None, _stream(q))
    _check("joint_attn_quant_fp8_repair", st)
    return out


def joint_attn_fwd_fp8_repair(t: Fp8Tensors, softmax_scale: float | None = None, out=None,
                              return_lse: bool = False):
    """fp8 attention with the repaired tokens of joint_attn_quant_fp8_repair.  Returns O
    bf16 [B, N, H, D] (and lse)."""
    torch = _torch()
    if t.mode != JA_FP8_REPAIR or t.q_src is None or t.k_src is None:
        raise ValueError("joint_attn_fwd_fp8_repair needs joint_attn_quant_fp8_repair's result")
    B, H, N, D = t.q8.shape
    ldv = int(t.v8t.shape[3])
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=t.q8.device)
    _need(out, torch.bfloat16, "out", 4)
    # the key correction reads and rewrites lse: always computed
    lse = torch.empty((B, H, N), dtype=torch.float32, device=t.q8.device)
    n_rep = int(t.n_repair)
    st = load().joint_attn_fwd_fp8_repair(
        t.q8.data_ptr(), t.k8.data_ptr(), t.v8t.data_ptr(), t.q_scale.data_ptr(),
        t.k_scale.data_ptr(), t.v_scale.data_ptr(), t.q_src.data_ptr(), t.k_src.data_ptr(),
        _ptr(t.q_sel) if n_rep else None, _ptr(t.k_sel) if n_rep else None,
        _ptr(t.v8t_sel) if n_rep else None, n_rep, B, H, N, D, ldv, scale, out.data_ptr(),
        lse.data_ptr(), _stream(t.q8))
    _check("joint_attn_fwd_fp8_repair", st)
    return (out, lse) if return_lse else out


def joint_attn_fwd_fp8(t: Fp8Tensors, softmax_scale: float | None = None, out=None,
                       return_lse: bool = False):
    """fp8 attention on joint_attn_quant_fp8's outputs (its mode; mode JA_FP8_REPAIR goes
    to joint_attn_fwd_fp8_repair).  Returns O bf16 [B, N, H, D] (and lse)."""
    torch = _torch()
    if t.mode == JA_FP8_REPAIR:
        return joint_attn_fwd_fp8_repair(t, softmax_scale, out, return_lse)
    for x, n in ((t.q8, "q8"), (t.k8, "k8"), (t.v8t, "v8t")):
        _need(x, torch.uint8, n, 4)
    for x, n in ((t.q_scale, "q_scale"), (t.k_scale, "k_scale"), (t.v_scale, "v_scale")):
        _need(x, torch.float32, n, 3)
    B, H, N, D = t.q8.shape
    ldv = int(t.v8t.shape[3])
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=t.q8.device)
    _need(out, torch.bfloat16, "out", 4)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=t.q8.device) if return_lse else None
    st = load().joint_attn_fwd_fp8(
        t.q8.data_ptr(), t.k8.data_ptr(), t.v8t.data_ptr(), t.q_scale.data_ptr(),
        t.k_scale.data_ptr(), t.v_scale.data_ptr(), B, H, N, D, ldv, scale, int(t.mode),
        _ptr(t.q_hi), _ptr(t.k_hi), out.data_ptr(), _ptr(lse), _stream(t.q8))
    _check("joint_attn_fwd_fp8", st)
    return (out, lse) if return_lse else out
