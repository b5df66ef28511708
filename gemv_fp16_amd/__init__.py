"""Python binding for libgemvfp16 (fp16 GEMM-NT, split-K GEMM, GEMV on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgemvfp16.so``; torch supplies device memory and the stream.
The functions carry the C-ABI names (include/gemvfp16.h).  A missing library
raises at the first call; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GEMVFP16_LIB names another build of the same library (the diagnostic
# variants of build.py); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("GEMVFP16_LIB") or os.path.join(_HERE, "libgemvfp16.so")

GF_OK, GF_ERR_INVALID_ARG, GF_ERR_HIP, GF_ERR_UNSUPPORTED, GF_ERR_TOO_LARGE = 0, 1, 2, 3, 4
GF_SPLITK_ATOMIC, GF_SPLITK_TWOPASS, GF_SPLITK_F16 = 0, 1, 2

EXPORTS = (
    "gemm_f16_nt", "gemm_f16_nt_splitk", "gemv_f16",
    "gemm_f16_nt_splitk_workspace_bytes", "gemm_f16_nt_splitk_ex", "gemm_f16_nt_splitk_f16",
    "gemm_f16_nt_cfg", "gemv_f16_cfg", "gemm_f16", "gemm_f16_nn", "gemm_f16_tn", "gemm_f16_cfg",
    "gemm_f16_nt_skinny", "gf_skinny_config_count", "gf_skinny_config_get", "gf_skinny_default_config",
    "gemm_f16_nt_splitk_cfg", "gemm_f16_nt_splitk_noalloc", "gf_noalloc_scratch_bytes",
    "gf_gemm_config_count", "gf_gemm_config_get", "gf_gemv_config_count", "gf_gemv_config_get",
    "gf_gemm_default_config", "gf_gemv_default_config", "gf_status_string",
    "sp24_compress_f16", "gemm_sp_f16_nt", "gemm_sp_f16_nt_cfg", "gf_sp_config_count",
    "gf_sp_config_get", "gf_sp_default_config",
)


class SkinnyCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("blocks", "unroll", "waves", "stages")]


class GemmCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("block_m", "block_n", "block_k", "stages", "threads", "raster", "schedule")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class SpCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("block_m", "block_n", "stages", "raster")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class GemvCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("rows_per_wave", "unroll", "waves", "blocks")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgemvfp16.so is not built (python -m gemv_fp16_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.gemm_f16_nt.argtypes = [vp, vp, vp, ci, ci, ci, vp]
    L.gemm_f16_nt_splitk.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp]
    L.gemv_f16.argtypes = [vp, vp, vp, ci, ci, vp]
    L.gemm_f16_nt_splitk_workspace_bytes.argtypes = [ci, ci, ci]
    L.gemm_f16_nt_splitk_workspace_bytes.restype = sz
    L.gemm_f16_nt_splitk_ex.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, vp, sz, vp]
    L.gemm_f16_nt_splitk_f16.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp, sz, vp]
    L.gemm_f16_nt_splitk_noalloc.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp]
    L.gf_noalloc_scratch_bytes.argtypes = []
    L.gf_noalloc_scratch_bytes.restype = sz
    L.gemm_f16.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, vp]
    L.gemm_f16_nt_skinny.argtypes = [vp, vp, vp, ci, ci, ci, ctypes.POINTER(SkinnyCfg), vp]
    L.gemm_f16_nt_splitk_cfg.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, vp, sz, ctypes.POINTER(GemmCfg), vp]
    L.gf_skinny_config_get.argtypes = [ci, ctypes.POINTER(SkinnyCfg)]
    L.gf_skinny_default_config.argtypes = [ci, ci, ci, ctypes.POINTER(SkinnyCfg)]
    L.gemm_f16_nn.argtypes = [vp, vp, vp, ci, ci, ci, vp]
    L.gemm_f16_tn.argtypes = [vp, vp, vp, ci, ci, ci, vp]
    L.gemm_f16_cfg.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ctypes.POINTER(GemmCfg), vp]
    L.gemm_f16_nt_cfg.argtypes = [vp, vp, vp, ci, ci, ci, ctypes.POINTER(GemmCfg), vp]
    L.gemv_f16_cfg.argtypes = [vp, vp, vp, ci, ci, ctypes.POINTER(GemvCfg), vp]
    L.gf_gemm_config_get.argtypes = [ci, ctypes.POINTER(GemmCfg)]
    L.gf_gemv_config_get.argtypes = [ci, ctypes.POINTER(GemvCfg)]
    L.gf_gemm_default_config.argtypes = [ci, ci, ci, ctypes.POINTER(GemmCfg)]
    L.gf_gemv_default_config.argtypes = [ci, ci, ctypes.POINTER(GemvCfg)]
    L.sp24_compress_f16.argtypes = [vp, vp, vp, ci, ci, vp]
    L.gemm_sp_f16_nt.argtypes = [vp, vp, vp, vp, ci, ci, ci, vp]
    L.gemm_sp_f16_nt_cfg.argtypes = [vp, vp, vp, vp, ci, ci, ci, ctypes.POINTER(SpCfg), vp]
    L.gf_sp_config_get.argtypes = [ci, ctypes.POINTER(SpCfg)]
    L.gf_sp_default_config.argtypes = [ci, ci, ci, ctypes.POINTER(SpCfg)]
    L.gf_status_string.argtypes = [ci]
    L.gf_status_string.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("gemm_f16_nt_splitk_workspace_bytes", "gf_noalloc_scratch_bytes", "gf_status_string"):
            getattr(L, name).restype = ci
    _lib = L
    return L


def status_string(rc: int) -> str:
    return lib().gf_status_string(rc).decode()


def _check(rc: int, what: str) -> None:
    if rc != GF_OK:
        raise RuntimeError("%s: %s" % (what, status_string(rc)))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _alloc(stream, fn):
    """Allocate a tensor that the call enqueued on `stream` will use: under
    that stream, so that torch's caching allocator does not hand the block
    to another stream's work while the call may still be running."""
    import torch
    if stream is None:
        return fn()
    with torch.cuda.stream(stream if isinstance(stream, torch.cuda.Stream)
                           else torch.cuda.ExternalStream(int(stream))):
        return fn()


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype and not (dtype == torch.int16 and t.dtype == getattr(torch, "uint16", None)):
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# configs
# ---------------------------------------------------------------------------

def gemm_configs() -> list[tuple[dict, bool]]:
    """Every GEMM tile config in the library, with whether a kernel exists."""
    L, out = lib(), []
    for i in range(L.gf_gemm_config_count()):
        c = GemmCfg()
        rc = L.gf_gemm_config_get(i, ctypes.byref(c))
        out.append((c.as_dict(), rc == GF_OK))
    return out


def gemv_configs() -> list[dict]:
    L, out = lib(), []
    for i in range(L.gf_gemv_config_count()):
        c = GemvCfg()
        _check(L.gf_gemv_config_get(i, ctypes.byref(c)), "gf_gemv_config_get")
        out.append(c.as_dict())
    return out


def gemm_default_config(M: int, N: int, K: int) -> dict:
    c = GemmCfg()
    _check(lib().gf_gemm_default_config(M, N, K, ctypes.byref(c)), "gf_gemm_default_config")
    return c.as_dict()


def gemv_default_config(N: int, K: int) -> dict:
    c = GemvCfg()
    _check(lib().gf_gemv_default_config(N, K, ctypes.byref(c)), "gf_gemv_default_config")
    return c.as_dict()


# ---------------------------------------------------------------------------
# operations on torch tensors
# ---------------------------------------------------------------------------

def _gemm_shapes(A, B):
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("A must be (M, K) and B (N, K)")
    return A.shape[0], B.shape[0], A.shape[1]


def gemm_f16_nt(A, B, C=None, stream=None, cfg: dict | None = None):
    """C = A . B^T (fp16 in, fp32 accumulate, fp16 out).  Returns C."""
    import torch
    M, N, K = _gemm_shapes(A, B)
    if C is None:
        C = _alloc(stream, lambda: torch.empty((M, N), dtype=torch.float16, device=A.device))
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be (M, N)")
    args = (_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"), _dev(C, torch.float16, "C"),
            M, N, K)
    if cfg is None:
        _check(lib().gemm_f16_nt(*args, _stream(stream)), "gemm_f16_nt")
    else:
        c = GemmCfg(**cfg)
        _check(lib().gemm_f16_nt_cfg(*args, ctypes.byref(c), _stream(stream)), "gemm_f16_nt_cfg")
    return C


def gemm_f16(A, B, C=None, a_kmajor: bool = False, b_kmajor: bool = False, stream=None,
             cfg: dict | None = None):
    """C = op(A) . op(B) with fp32 accumulation, fp16 out.  A is (M, K), or
    (K, M) when a_kmajor; B is (N, K), or (K, N) when b_kmajor.  Returns C."""
    import torch
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    K, M = (A.shape[0], A.shape[1]) if a_kmajor else (A.shape[1], A.shape[0])
    Kb, N = (B.shape[0], B.shape[1]) if b_kmajor else (B.shape[1], B.shape[0])
    if K != Kb:
        raise ValueError("A and B disagree on K (%d vs %d)" % (K, Kb))
    if C is None:
        C = _alloc(stream, lambda: torch.empty((M, N), dtype=torch.float16, device=A.device))
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be (M, N)")
    args = (_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"), _dev(C, torch.float16, "C"),
            M, N, K, int(bool(a_kmajor)), int(bool(b_kmajor)))
    if cfg is None:
        _check(lib().gemm_f16(*args, _stream(stream)), "gemm_f16")
    else:
        c = GemmCfg(**cfg)
        _check(lib().gemm_f16_cfg(*args, ctypes.byref(c), _stream(stream)), "gemm_f16_cfg")
    return C


def gemm_f16_nt_skinny(A, B, C=None, stream=None, cfg: dict | None = None):
    """C = A . B^T for 1 <= M <= 64 rows of A through the skinny kernel
    (17 to 64 rows: the LDS-staged form only, K % 512 == 0)."""
    import torch
    M, N, K = _gemm_shapes(A, B)
    if C is None:
        C = _alloc(stream, lambda: torch.empty((M, N), dtype=torch.float16, device=A.device))
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be (M, N)")
    c = ctypes.byref(SkinnyCfg(**cfg)) if cfg is not None else None
    _check(lib().gemm_f16_nt_skinny(_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"),
                                    _dev(C, torch.float16, "C"), M, N, K, c, _stream(stream)),
           "gemm_f16_nt_skinny")
    return C


def skinny_configs() -> list:
    L = lib()
    out = []
    for i in range(L.gf_skinny_config_count()):
        c = SkinnyCfg()
        _check(L.gf_skinny_config_get(i, ctypes.byref(c)), "gf_skinny_config_get")
        out.append({"blocks": c.blocks, "unroll": c.unroll, "waves": c.waves, "stages": c.stages})
    return out


def skinny_default_config(M: int, N: int, K: int) -> dict:
    c = SkinnyCfg()
    _check(lib().gf_skinny_default_config(M, N, K, ctypes.byref(c)), "gf_skinny_default_config")
    return {"blocks": c.blocks, "unroll": c.unroll, "waves": c.waves, "stages": c.stages}


def gemm_f16_nn(A, B, C=None, stream=None):
    """C = A . B with A (M, K) and B (K, N), both row-major."""
    return gemm_f16(A, B, C, False, True, stream)


def gemm_f16_tn(A, B, C=None, stream=None):
    """C = A^T . B with A (K, M) and B (K, N), both row-major."""
    return gemm_f16(A, B, C, True, True, stream)


def gemm_f16_nt_splitk_workspace_bytes(M: int, N: int, split_k: int) -> int:
    return int(lib().gemm_f16_nt_splitk_workspace_bytes(M, N, split_k))


def gemm_f16_nt_splitk(A, B, C32=None, split_k: int = 4, stream=None):
    """C32 = A . B^T in fp32 via split-K with fp32 atomic combine."""
    import torch
    M, N, K = _gemm_shapes(A, B)
    if C32 is None:
        C32 = _alloc(stream, lambda: torch.empty((M, N), dtype=torch.float32, device=A.device))
    if tuple(C32.shape) != (M, N):
        raise ValueError("C32 must be (M, N)")
    _check(lib().gemm_f16_nt_splitk(_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"),
                                    _dev(C32, torch.float32, "C32"), M, N, K, split_k,
                                    _stream(stream)), "gemm_f16_nt_splitk")
    return C32


def gemm_f16_nt_splitk_ex(A, B, C32=None, split_k: int = 4, mode: int = GF_SPLITK_TWOPASS,
                          workspace=None, stream=None):
    """Split-K with mode GF_SPLITK_ATOMIC or GF_SPLITK_TWOPASS (deterministic).

    In two-pass mode a workspace (fp32 CUDA tensor of at least
    gemm_f16_nt_splitk_workspace_bytes bytes) is allocated if not given."""
    import torch
    M, N, K = _gemm_shapes(A, B)
    if C32 is None:
        C32 = _alloc(stream, lambda: torch.empty((M, N), dtype=torch.float32, device=A.device))
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if mode == GF_SPLITK_TWOPASS:
        need = gemm_f16_nt_splitk_workspace_bytes(M, N, split_k)
        if workspace is None:
            workspace = _alloc(stream, lambda: torch.empty(max(1, need // 4), dtype=torch.float32,
                                                           device=A.device))
        ws_ptr = _dev(workspace, torch.float32, "workspace")
        ws_bytes = workspace.numel() * 4
    _check(lib().gemm_f16_nt_splitk_ex(_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"),
                                       _dev(C32, torch.float32, "C32"), M, N, K, split_k, mode,
                                       ws_ptr, ws_bytes, _stream(stream)), "gemm_f16_nt_splitk_ex")
    return C32




def gemm_f16_nt_splitk_noalloc(A, B, C32, split_k: int = 4, stream=None):
    """Two-pass split-K into the caller's C32 (fp32, M x N) with the slice
    partials in the library's fixed scratch: neither the library nor this
    binding allocates anything.  Calls that overlap on one GPU race."""
    import torch
    M, N, K = _gemm_shapes(A, B)
    if tuple(C32.shape) != (M, N):
        raise ValueError("C32 must be (M, N)")
    _check(lib().gemm_f16_nt_splitk_noalloc(_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"),
                                            _dev(C32, torch.float32, "C32"), M, N, K, split_k,
                                            _stream(stream)), "gemm_f16_nt_splitk_noalloc")
    return C32


def gemm_f16_nt_splitk_cfg(A, B, C, split_k: int, mode: int, cfg: dict, workspace, stream=None):
    """Split-K with an explicit tile config; C is fp32 (atomic / two-pass) or
    fp16 (GF_SPLITK_F16).  The workspace (fp32 CUDA tensor) is required."""
    import torch
    M, N, K = _gemm_shapes(A, B)
    cdt = torch.float16 if mode == GF_SPLITK_F16 else torch.float32
    c = GemmCfg(**cfg)
    _check(lib().gemm_f16_nt_splitk_cfg(_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"),
                                        _dev(C, cdt, "C"), M, N, K, split_k, mode,
                                        _dev(workspace, torch.float32, "workspace"),
                                        workspace.numel() * 4, ctypes.byref(c), _stream(stream)),
           "gemm_f16_nt_splitk_cfg")
    return C


def gemm_f16_nt_splitk_f16(A, B, C=None, split_k: int = 4, workspace=None, stream=None):
    """Split-K with an fp16 output: the fp32 slice partials (workspace, fp32
    CUDA tensor, allocated if not given) are summed in ascending slice order
    and rounded once to fp16.  Returns C (M x N fp16)."""
    import torch
    M, N, K = _gemm_shapes(A, B)
    if C is None:
        C = _alloc(stream, lambda: torch.empty((M, N), dtype=torch.float16, device=A.device))
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be (M, N)")
    need = gemm_f16_nt_splitk_workspace_bytes(M, N, split_k)
    if workspace is None:
        workspace = _alloc(stream, lambda: torch.empty(max(1, need // 4), dtype=torch.float32,
                                                       device=A.device))
    _check(lib().gemm_f16_nt_splitk_f16(_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"),
                                        _dev(C, torch.float16, "C"), M, N, K, split_k,
                                        _dev(workspace, torch.float32, "workspace"),
                                        workspace.numel() * 4, _stream(stream)),
           "gemm_f16_nt_splitk_f16")
    return C


def gemv_f16(W, x, y=None, stream=None, cfg: dict | None = None):
    """y = W . x (fp16 in, fp32 accumulate, fp16 out).  Returns y."""
    import torch
    if W.dim() != 2 or x.dim() != 1 or W.shape[1] != x.shape[0]:
        raise ValueError("W must be (N, K) and x (K,)")
    N, K = W.shape
    if y is None:
        y = _alloc(stream, lambda: torch.empty((N,), dtype=torch.float16, device=W.device))
    if tuple(y.shape) != (N,):
        raise ValueError("y must be (N,)")
    args = (_dev(W, torch.float16, "W"), _dev(x, torch.float16, "x"), _dev(y, torch.float16, "y"), N, K)
    if cfg is None:
        _check(lib().gemv_f16(*args, _stream(stream)), "gemv_f16")
    else:
        c = GemvCfg(**cfg)
        _check(lib().gemv_f16_cfg(*args, ctypes.byref(c), _stream(stream)), "gemv_f16_cfg")
    return y


# ---------------------------------------------------------------------------
# pre-marshalled calls: the checks and pointer extraction happen once, so a
# timing loop pays only the ctypes call per launch
# ---------------------------------------------------------------------------

def prepare_gemm_f16_nt(A, B, C, stream=None, cfg: dict | None = None):
    """Zero-argument callable that launches C = A . B^T on `stream`."""
    import torch
    M, N, K = _gemm_shapes(A, B)
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be (M, N)")
    args = (_dev(A, torch.float16, "A"), _dev(B, torch.float16, "B"), _dev(C, torch.float16, "C"),
            M, N, K)
    s = _stream(stream)
    L = lib()
    if cfg is None:
        fn = L.gemm_f16_nt

        def call():
            rc = fn(*args, s)
            if rc:
                _check(rc, "gemm_f16_nt")
    else:
        c = GemmCfg(**cfg)
        ref = ctypes.byref(c)
        fn = L.gemm_f16_nt_cfg

        def call():
            rc = fn(*args, ref, s)
            if rc:
                _check(rc, "gemm_f16_nt_cfg")
    call.keep = (A, B, C, args)
    return call


def prepare_gemv_f16(W, x, y, stream=None, cfg: dict | None = None):
    """Zero-argument callable that launches y = W . x on `stream`."""
    import torch
    if W.dim() != 2 or x.dim() != 1 or W.shape[1] != x.shape[0] or tuple(y.shape) != (W.shape[0],):
        raise ValueError("W must be (N, K), x (K,), y (N,)")
    N, K = W.shape
    args = (_dev(W, torch.float16, "W"), _dev(x, torch.float16, "x"), _dev(y, torch.float16, "y"), N, K)
    s = _stream(stream)
    L = lib()
    if cfg is None:
        fn = L.gemv_f16

        def call():
            rc = fn(*args, s)
            if rc:
                _check(rc, "gemv_f16")
    else:
        c = GemvCfg(**cfg)
        ref = ctypes.byref(c)
        fn = L.gemv_f16_cfg

        def call():
            rc = fn(*args, ref, s)
            if rc:
                _check(rc, "gemv_f16_cfg")
    call.keep = (W, x, y, args)
    return call


# ---------------------------------------------------------------------------
# 2:4 structured sparsity
# ---------------------------------------------------------------------------

def sp24_compress_f16(A, A_sparse=None, E=None, stream=None):
    """Compress A (M, K) fp16, K % 16 == 0, into A_sparse (M, K/2) fp16 and
    E (M, K/16) int16 metadata words.  Returns (A_sparse, E)."""
    import torch
    if A.dim() != 2:
        raise ValueError("A must be (M, K)")
    M, K = A.shape
    if A_sparse is None:
        A_sparse = _alloc(stream, lambda: torch.empty((M, K // 2), dtype=torch.float16, device=A.device))
    if E is None:
        E = _alloc(stream, lambda: torch.empty((M, K // 16), dtype=torch.int16, device=A.device))
    if tuple(A_sparse.shape) != (M, K // 2) or tuple(E.shape) != (M, K // 16):
        raise ValueError("A_sparse must be (M, K/2) and E (M, K/16)")
    _check(lib().sp24_compress_f16(_dev(A, torch.float16, "A"), _dev(A_sparse, torch.float16, "A_sparse"),
                                   _dev(E, torch.int16, "E"), M, K, _stream(stream)), "sp24_compress_f16")
    return A_sparse, E


def _sp_args(A_sparse, E, B, C, stream=None):
    import torch
    if A_sparse.dim() != 2 or E.dim() != 2 or B.dim() != 2:
        raise ValueError("A_sparse must be (M, K/2), E (M, K/16), B (N, K)")
    M, K = A_sparse.shape[0], 2 * A_sparse.shape[1]
    N = B.shape[0]
    if B.shape[1] != K or tuple(E.shape) != (M, K // 16):
        raise ValueError("A_sparse must be (M, K/2), E (M, K/16), B (N, K)")
    if C is None:
        C = _alloc(stream, lambda: torch.empty((M, N), dtype=torch.float16, device=B.device))
    if tuple(C.shape) != (M, N):
        raise ValueError("C must be (M, N)")
    args = (_dev(A_sparse, torch.float16, "A_sparse"), _dev(E, torch.int16, "E"), _dev(B, torch.float16, "B"),
            _dev(C, torch.float16, "C"), M, N, K)
    return C, args


def gemm_sp_f16_nt(A_sparse, E, B, C=None, stream=None, cfg: dict | None = None):
    """C = decompress(A_sparse, E) . B^T (fp16 in, fp32 accumulate, fp16 out)."""
    C, args = _sp_args(A_sparse, E, B, C, stream)
    if cfg is None:
        _check(lib().gemm_sp_f16_nt(*args, _stream(stream)), "gemm_sp_f16_nt")
    else:
        c = SpCfg(**cfg)
        _check(lib().gemm_sp_f16_nt_cfg(*args, ctypes.byref(c), _stream(stream)), "gemm_sp_f16_nt_cfg")
    return C


def prepare_gemm_sp_f16_nt(A_sparse, E, B, C, stream=None, cfg: dict | None = None):
    """Zero-argument callable that launches the sparse product on `stream`."""
    C, args = _sp_args(A_sparse, E, B, C, stream)
    s = _stream(stream)
    L = lib()
    c = SpCfg(**cfg) if cfg is not None else None
    ref = ctypes.byref(c) if c is not None else None
    fn = L.gemm_sp_f16_nt_cfg

    def call():
        rc = fn(*args, ref, s)
        if rc:
            _check(rc, "gemm_sp_f16_nt_cfg")
    call.keep = (A_sparse, E, B, C, args, c)
    return call


def sp_configs() -> list[dict]:
    L, out = lib(), []
    for i in range(L.gf_sp_config_count()):
        c = SpCfg()
        _check(L.gf_sp_config_get(i, ctypes.byref(c)), "gf_sp_config_get")
        out.append(c.as_dict())
    return out


def sp_default_config(M: int, N: int, K: int) -> dict:
    c = SpCfg()
    _check(lib().gf_sp_default_config(M, N, K, ctypes.byref(c)), "gf_sp_default_config")
    return c.as_dict()

