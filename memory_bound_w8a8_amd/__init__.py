"""Python binding of libfp8bq (W8A8 block-FP8 linear layer on MI355X).

Argument marshalling only: every step runs in the HIP kernels of
libfp8bq.so, called through its C ABI (include/fp8bq.h). torch supplies
device memory and the current stream. There is no fallback: if the library
is missing or cannot run, the calls raise.

    a_q, a_s = quant_act(a)              # a: bf16 [M, K] on the GPU
    w_q, w_s = quant_weight(w)           # w: fp32 [N, K] on the GPU
    c = gemm(a_q, a_s, w_q, w_s)         # c: bf16 [M, N]

Two-stage vocabulary scoring (coarse FP8 logits, exact top-k, exact BF16
rescoring of the survivors):

    pick, idx, scores = two_stage(h, w_q, w_s, w_bf16, k)
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8bq.so")

FP8BQ_OK = 0
PATH_NONE, PATH_STREAM, PATH_TILED = 0, 1, 2
# tile shapes of the tiled kernel (tokens x weight rows), for gemm_forced
PATH_TILED_128x128, PATH_TILED_128x256, PATH_TILED_192x256, PATH_TILED_256x256 = 3, 4, 5, 6
PATH_TILED_64x128, PATH_TILED_128x64, PATH_TILED_64x64 = 7, 8, 9
PATH_NAMES = {PATH_NONE: "none", PATH_STREAM: "stream", PATH_TILED: "tiled",
              PATH_TILED_128x128: "tiled 128x128", PATH_TILED_128x256: "tiled 128x256",
              PATH_TILED_192x256: "tiled 192x256", PATH_TILED_256x256: "tiled 256x256",
              PATH_TILED_64x128: "tiled 64x128", PATH_TILED_128x64: "tiled 128x64", PATH_TILED_64x64: "tiled 64x64"}


# Every symbol the C ABI exports (kept in step with include/fp8bq.h).
EXPORTS = (
    "fp8bq_quant_act",
    "fp8bq_quant_weight",
    "fp8bq_gemm",
    "fp8bq_gemm_path",
    "fp8bq_gemm_forced",
    "fp8bq_gemm_workspace_bytes",
    "fp8bq_gemm_ws",
    "fp8bq_gemm_ws_forced",
    "fp8bq_gemm_tile_shape",
    "fp8bq_gemm_fused",
    "fp8bq_gemm_w8a16",
    "fp8bq_topk_workspace_bytes",
    "fp8bq_topk_bf16",
    "fp8bq_topk_bf16_noalloc",
    "fp8bq_rescore_bf16",
    "fp8bq_mb_read",
    "fp8bq_mb_empty",
    "fp8bq_mb_mfma_e4m3",
    "fp8bq_mb_mfma_e4m3_data",
    "fp8bq_mb_mfma_e4m3_scaled",
    "fp8bq_status_string",
)


class Fp8bqError(RuntimeError):
    """A nonzero status returned by libfp8bq."""

    def __init__(self, call: str, status: int):
        super().__init__(f"{call}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfp8bq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m memory_bound_w8a8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, fp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        L.fp8bq_quant_act.argtypes = [i64, i64, vp, vp, fp, vp]
        L.fp8bq_quant_weight.argtypes = [i64, i64, fp, vp, fp, vp]
        L.fp8bq_gemm.argtypes = [i64, i64, i64, vp, fp, vp, fp, vp, vp]
        L.fp8bq_gemm_forced.argtypes = [ctypes.c_int, i64, i64, i64, vp, fp, vp, fp, vp, vp]
        L.fp8bq_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8bq_gemm_workspace_bytes.restype = i64
        L.fp8bq_gemm_ws.argtypes = [i64, i64, i64, vp, fp, vp, fp, vp, vp, i64, vp]
        L.fp8bq_gemm_ws_forced.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, fp, vp, fp, vp, vp, i64, vp]
        L.fp8bq_gemm_path.argtypes = [i64, i64, i64]
        L.fp8bq_gemm_tile_shape.argtypes = [i64, i64, i64]
        L.fp8bq_gemm_w8a16.argtypes = [i64, i64, i64, vp, vp, fp, vp, vp]
        L.fp8bq_gemm_fused.argtypes = [i64, i64, i64, vp, vp, fp, vp, vp]
        L.fp8bq_topk_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8bq_topk_workspace_bytes.restype = i64
        L.fp8bq_topk_bf16.argtypes = [i64, i64, i64, vp, vp, i64, vp, vp, vp]
        L.fp8bq_topk_bf16_noalloc.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.fp8bq_rescore_bf16.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        ci = ctypes.c_int
        L.fp8bq_mb_read.argtypes = [vp, i64, ci, vp, vp]
        L.fp8bq_mb_empty.argtypes = [ci, ci, vp]
        L.fp8bq_mb_mfma_e4m3.argtypes = [ci, ci, ci, vp, vp]
        L.fp8bq_mb_mfma_e4m3_data.argtypes = [ci, ci, vp, vp, vp]
        L.fp8bq_mb_mfma_e4m3_scaled.argtypes = [ci, ci, vp, ctypes.c_float, vp, vp]
        L.fp8bq_status_string.argtypes = [ctypes.c_int]
        L.fp8bq_status_string.restype = ctypes.c_char_p
        for name in ("fp8bq_quant_act", "fp8bq_quant_weight", "fp8bq_gemm", "fp8bq_gemm_forced", "fp8bq_gemm_path",
                     "fp8bq_gemm_ws", "fp8bq_gemm_ws_forced",
                     "fp8bq_gemm_tile_shape",
                     "fp8bq_gemm_w8a16", "fp8bq_gemm_fused", "fp8bq_topk_bf16", "fp8bq_topk_bf16_noalloc",
                     "fp8bq_rescore_bf16",
                     "fp8bq_mb_read", "fp8bq_mb_empty", "fp8bq_mb_mfma_e4m3", "fp8bq_mb_mfma_e4m3_data",
                     "fp8bq_mb_mfma_e4m3_scaled"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fp8bq_status_string(int(status)).decode()


def _check(call: str, status: int) -> None:
    if status != FP8BQ_OK:
        raise Fp8bqError(call, status)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _codes(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {ndim}-d tensor")


def quant_act(a: torch.Tensor):
    """bf16 [M, K] -> (uint8 e4m3fn codes [M, K], fp32 scales [M, K/128])."""
    _need(a, "a", torch.bfloat16, 2)
    m, k = a.shape
    a_q = torch.empty((m, k), dtype=torch.uint8, device=a.device)
    a_s = torch.empty((m, k // 128 if k % 128 == 0 else 0), dtype=torch.float32, device=a.device)
    with torch.cuda.device(a.device):
        _check("fp8bq_quant_act", lib().fp8bq_quant_act(m, k, _ptr(a), _ptr(a_q), _ptr(a_s), _stream(a)))
    return a_q, a_s


def quant_weight(w: torch.Tensor):
    """fp32 [N, K] -> (uint8 codes [N, K], fp32 scales [ceil(N/128), K/128])."""
    _need(w, "w", torch.float32, 2)
    n, k = w.shape
    w_q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    w_s = torch.empty(((n + 127) // 128, k // 128 if k % 128 == 0 else 0), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        _check("fp8bq_quant_weight", lib().fp8bq_quant_weight(n, k, _ptr(w), _ptr(w_q), _ptr(w_s), _stream(w)))
    return w_q, w_s


def _gemm_args(a_q, a_s, w_q, w_s, out):
    a_q, w_q = _codes(a_q), _codes(w_q)
    _need(a_q, "a_q", torch.uint8, 2)
    _need(w_q, "w_q", torch.uint8, 2)
    _need(a_s, "a_s", torch.float32, 2)
    _need(w_s, "w_s", torch.float32, 2)
    m, k = a_q.shape
    n, k2 = w_q.shape
    if k != k2:
        raise ValueError(f"K mismatch: a_q has {k}, w_q has {k2}")
    groups = k // 128
    if tuple(a_s.shape) != (m, groups) or tuple(w_s.shape) != ((n + 127) // 128, groups):
        raise ValueError(f"scale shapes {tuple(a_s.shape)}, {tuple(w_s.shape)} do not match M={m}, N={n}, K={k}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    else:
        _need(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (m, n):
            raise ValueError(f"out must be [{m}, {n}]")
    return a_q, w_q, m, n, k, out


def gemm(a_q, a_s, w_q, w_s, out=None) -> torch.Tensor:
    """Block-scaled FP8 GEMM: C[m, n] = sum over K of A[m, k] W[n, k], bf16 [M, N]."""
    a_q, w_q, m, n, k, out = _gemm_args(a_q, a_s, w_q, w_s, out)
    with torch.cuda.device(a_q.device):
        st = lib().fp8bq_gemm(m, n, k, _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), _ptr(out), _stream(a_q))
    _check("fp8bq_gemm", st)
    return out


def _bf16_act_args(a, w_q, w_s, out):
    w_q = _codes(w_q)
    _need(a, "a", torch.bfloat16, 2)
    _need(w_q, "w_q", torch.uint8, 2)
    _need(w_s, "w_s", torch.float32, 2)
    m, k = a.shape
    n, k2 = w_q.shape
    if k != k2:
        raise ValueError(f"K mismatch: a has {k}, w_q has {k2}")
    if tuple(w_s.shape) != ((n + 127) // 128, k // 128):
        raise ValueError(f"weight scale shape {tuple(w_s.shape)} does not match N={n}, K={k}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    else:
        _need(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (m, n):
            raise ValueError(f"out must be [{m}, {n}]")
    return w_q, m, n, k, out


def gemm_w8a16(a: torch.Tensor, w_q, w_s, out=None) -> torch.Tensor:
    """Weight-only block-FP8 GEMM: bf16 activation [M, K] (M <= 16) times the
    block-FP8 weight, bf16 [M, N]."""
    w_q, m, n, k, out = _bf16_act_args(a, w_q, w_s, out)
    with torch.cuda.device(a.device):
        st = lib().fp8bq_gemm_w8a16(m, n, k, _ptr(a), _ptr(w_q), _ptr(w_s), _ptr(out), _stream(a))
    _check("fp8bq_gemm_w8a16", st)
    return out


def gemm_fused(a: torch.Tensor, w_q, w_s, out=None) -> torch.Tensor:
    """Activation quantisation and block-FP8 GEMM in one launch: bf16 [M, K]
    (M <= 8) -> bf16 [M, N], bitwise gemm(*quant_act(a), w_q, w_s)."""
    w_q, m, n, k, out = _bf16_act_args(a, w_q, w_s, out)
    with torch.cuda.device(a.device):
        st = lib().fp8bq_gemm_fused(m, n, k, _ptr(a), _ptr(w_q), _ptr(w_s), _ptr(out), _stream(a))
    _check("fp8bq_gemm_fused", st)
    return out


def gemm_forced(path: int, a_q, a_s, w_q, w_s, out=None) -> torch.Tensor:
    """gemm() on a chosen kernel path or tile shape (PATH_STREAM needs M <= 128)."""
    a_q, w_q, m, n, k, out = _gemm_args(a_q, a_s, w_q, w_s, out)
    with torch.cuda.device(a_q.device):
        st = lib().fp8bq_gemm_forced(int(path), m, n, k, _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), _ptr(out),
                                     _stream(a_q))
    _check("fp8bq_gemm_forced", st)
    return out


def gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    """Device workspace bytes gemm_ws() uses for its K-split plan on (M, N, K)
    (0: no split); raises on invalid sizes."""
    st = lib().fp8bq_gemm_workspace_bytes(int(m), int(n), int(k))
    if st < 0:
        raise Fp8bqError("fp8bq_gemm_workspace_bytes", st)
    return st


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace: contiguous uint8 tensor")
    return workspace


def gemm_ws(a_q, a_s, w_q, w_s, out=None, workspace=None) -> torch.Tensor:
    """gemm() with a device workspace (uint8 tensor; allocated here when
    None), which lets 65..~256-token calls split each tile's K range over
    several workgroups (fp8bq_gemm_ws)."""
    a_q, w_q, m, n, k, out = _gemm_args(a_q, a_s, w_q, w_s, out)
    workspace = _workspace(gemm_workspace_bytes(m, n, k), a_q.device, workspace)
    with torch.cuda.device(a_q.device):
        st = lib().fp8bq_gemm_ws(m, n, k, _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), _ptr(out), _ptr(workspace),
                                 workspace.numel(), _stream(a_q))
    _check("fp8bq_gemm_ws", st)
    return out


def gemm_ws_forced(path: int, split: int, a_q, a_s, w_q, w_s, out=None, workspace=None) -> torch.Tensor:
    """gemm_ws() with the tile shape (a PATH_TILED_* value) and the number of
    K parts forced (split == 1: gemm_forced)."""
    a_q, w_q, m, n, k, out = _gemm_args(a_q, a_s, w_q, w_s, out)
    workspace = _workspace(int(split) * m * n * 4 if split > 1 else 0, a_q.device, workspace)
    with torch.cuda.device(a_q.device):
        st = lib().fp8bq_gemm_ws_forced(int(path), int(split), m, n, k, _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s),
                                        _ptr(out), _ptr(workspace), workspace.numel(), _stream(a_q))
    _check("fp8bq_gemm_ws_forced", st)
    return out


def gemm_path(m: int, n: int, k: int) -> int:
    """Kernel path fp8bq_gemm takes for (M, N, K); raises on invalid sizes."""
    st = lib().fp8bq_gemm_path(int(m), int(n), int(k))
    if st < 0:
        raise Fp8bqError("fp8bq_gemm_path", st)
    return st


def topk_workspace_bytes(m: int, v: int, k: int) -> int:
    """Device workspace bytes topk() needs for (M, V, k); raises on sizes the
    library rejects."""
    st = lib().fp8bq_topk_workspace_bytes(int(m), int(v), int(k))
    if st < 0:
        raise Fp8bqError("fp8bq_topk_workspace_bytes", st)
    return st


def topk(logits: torch.Tensor, k: int, workspace: torch.Tensor = None):
    """Exact top-k of each row of bf16 logits [M, V] (1 <= k <= 256): int32
    indices [M, k], best first (equal values: lower index first), and their
    bf16 values. `workspace` (uint8, on the device) is allocated if absent."""
    _need(logits, "logits", torch.bfloat16, 2)
    m, v = logits.shape
    need = topk_workspace_bytes(m, v, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=logits.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    idx = torch.empty((m, k), dtype=torch.int32, device=logits.device)
    val = torch.empty((m, k), dtype=torch.bfloat16, device=logits.device)
    with torch.cuda.device(logits.device):
        st = lib().fp8bq_topk_bf16(m, v, int(k), _ptr(logits), _ptr(workspace), workspace.numel(), _ptr(idx),
                                   _ptr(val), _stream(logits))
    _check("fp8bq_topk_bf16", st)
    return idx, val


# Bytes of the library's static scratch array used by topk_noalloc.
TOPK_SCRATCH_BYTES = 4 << 20


def topk_noalloc(logits: torch.Tensor, k: int, idx: torch.Tensor, val: torch.Tensor):
    """topk() into caller-provided outputs (int32 idx [M, k], bf16 val [M, k])
    through the entry point that allocates nothing: its workspace is the
    library's static per-GPU scratch array (calls on one GPU must not
    overlap). Returns (idx, val)."""
    _need(logits, "logits", torch.bfloat16, 2)
    _need(idx, "idx", torch.int32, 2)
    _need(val, "val", torch.bfloat16, 2)
    m, v = logits.shape
    if tuple(idx.shape) != (m, k) or tuple(val.shape) != (m, k):
        raise ValueError(f"idx and val must be [{m}, {k}]")
    with torch.cuda.device(logits.device):
        st = lib().fp8bq_topk_bf16_noalloc(m, v, int(k), _ptr(logits), _ptr(idx), _ptr(val), _stream(logits))
    _check("fp8bq_topk_bf16_noalloc", st)
    return idx, val


def rescore(h: torch.Tensor, w: torch.Tensor, idx: torch.Tensor):
    """Exact scores of survivors: h bf16 [M, K], w bf16 [V, K], idx int32
    [M, k] -> (fp32 scores [M, k], int32 pick [M]: the best survivor, ties to
    the lower index)."""
    _need(h, "h", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 2)
    _need(idx, "idx", torch.int32, 2)
    m, kdim = h.shape
    v, k2 = w.shape
    if k2 != kdim:
        raise ValueError(f"K mismatch: h has {kdim}, w has {k2}")
    if idx.shape[0] != m:
        raise ValueError(f"idx has {idx.shape[0]} rows, h has {m}")
    k = idx.shape[1]
    scores = torch.empty((m, k), dtype=torch.float32, device=h.device)
    pick = torch.empty((m,), dtype=torch.int32, device=h.device)
    with torch.cuda.device(h.device):
        st = lib().fp8bq_rescore_bf16(m, kdim, v, k, _ptr(h), _ptr(w), _ptr(idx), _ptr(scores), _ptr(pick),
                                      _stream(h))
    _check("fp8bq_rescore_bf16", st)
    return scores, pick


# Largest token count whose coarse logits two_stage() takes from the fused
# launch (the fused entry point serves up to 8 tokens); beyond it,
# quantisation + GEMM, bitwise the same logits.
TWO_STAGE_FUSED_MAX_M = 8


def two_stage(h: torch.Tensor, w_q, w_s, w_bf16: torch.Tensor, k: int, workspace: torch.Tensor = None):
    """Two-stage vocabulary scoring of hidden states h bf16 [M, K]: coarse
    logits by the block-FP8 GEMM of the quantised h against (w_q, w_s),
    their exact top-k, exact scores of those k against the bf16 projection
    w_bf16 [V, K]. Returns (pick int32 [M], idx int32 [M, k], scores fp32
    [M, k])."""
    _need(h, "h", torch.bfloat16, 2)
    if h.shape[0] <= TWO_STAGE_FUSED_MAX_M:
        logits = gemm_fused(h, w_q, w_s)
    else:
        logits = gemm(*quant_act(h), w_q, w_s)
    idx, _ = topk(logits, k, workspace)
    scores, pick = rescore(h, w_bf16, idx)
    return pick, idx, scores


# Measurement kernels (the machine's own ceilings for the roofline figures).

def mb_read(buf: torch.Tensor, grid: int = 256, sink: torch.Tensor = None) -> torch.Tensor:
    """Streaming read of a contiguous GPU buffer (size a multiple of 16
    bytes); returns the per-workgroup XOR words (uint32 viewed as int32)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("mb_read: buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(grid, dtype=torch.int32, device=buf.device)
    _check("fp8bq_mb_read", lib().fp8bq_mb_read(_ptr(buf), nbytes, int(grid), _ptr(sink), _stream(buf)))
    return sink


def mb_empty(grid: int, block: int, device=None) -> None:
    """One launch of an empty kernel on the current stream."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    _check("fp8bq_mb_empty", lib().fp8bq_mb_empty(int(grid), int(block), torch.cuda.current_stream(dev).cuda_stream))


def mb_mfma(grid: int, iters: int, code: int = 0x38, sink: torch.Tensor = None, device=None) -> torch.Tensor:
    """grid x 4 waves x 8 x iters FP8 16x16x128 MFMAs; returns the per-thread
    sums (fp32 [grid * 256], each 4096 * iters * decode(code)^2)."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    if sink is None:
        sink = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    _check("fp8bq_mb_mfma_e4m3",
           lib().fp8bq_mb_mfma_e4m3(int(grid), int(iters), int(code), _ptr(sink), torch.cuda.current_stream(dev).cuda_stream))
    return sink


MB_MFMA_DATA_BYTES = 32768


def mb_mfma_data(grid: int, iters: int, codes: torch.Tensor, sink: torch.Tensor = None) -> torch.Tensor:
    """The MFMA loop of mb_mfma with operands read from `codes` (uint8
    [32768] on the GPU, e4m3 codes without NaN codes; see the header for the
    layout); returns the per-thread sums (fp32 [grid * 256])."""
    if codes.dtype != torch.uint8 or codes.numel() != MB_MFMA_DATA_BYTES or not codes.is_contiguous():
        raise ValueError("codes: contiguous uint8 tensor of 32768 bytes")
    if sink is None:
        sink = torch.empty(grid * 256, dtype=torch.float32, device=codes.device)
    _check("fp8bq_mb_mfma_e4m3_data",
           lib().fp8bq_mb_mfma_e4m3_data(int(grid), int(iters), _ptr(codes), _ptr(sink),
                                         torch.cuda.current_stream(codes.device).cuda_stream))
    return sink


def mb_mfma_scaled(grid: int, iters: int, codes: torch.Tensor, scale: float, sink: torch.Tensor = None) -> torch.Tensor:
    """mb_mfma_data's operands in the block-scaled GEMM's inner loop: every
    MFMA from zero, its results folded into running sums by 4 fp32 FMAs with
    `scale`; returns the per-thread sums (fp32 [grid * 256], `scale` times
    mb_mfma_data's)."""
    if codes.dtype != torch.uint8 or codes.numel() != MB_MFMA_DATA_BYTES or not codes.is_contiguous():
        raise ValueError("codes: contiguous uint8 tensor of 32768 bytes")
    if sink is None:
        sink = torch.empty(grid * 256, dtype=torch.float32, device=codes.device)
    _check("fp8bq_mb_mfma_e4m3_scaled",
           lib().fp8bq_mb_mfma_e4m3_scaled(int(grid), int(iters), _ptr(codes), float(scale), _ptr(sink),
                                           torch.cuda.current_stream(codes.device).cuda_stream))
    return sink
