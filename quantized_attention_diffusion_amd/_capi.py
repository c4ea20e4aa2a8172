"""ctypes binding of libsage_attn.so.  Argument marshalling only: every step of the
computation runs in the library's HIP kernels; torch supplies device memory and the
current stream.  The functions carry the C entry points' names."""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["SageError", "lib_path", "load", "sage_last_error", "sage_kernel_info",
           "sage_padded_tokens", "sage_workspace_bytes", "sage_workspace_bytes_ex",
           "sage_quant_scratch_bytes", "sage_quant_qk", "sage_attn_fwd_prequant", "sage_attn_fwd",
           "sage_attn_fwd_ex", "sage_quant_qk_ex", "sage_debug_qk_i32", "sage_debug_qk_i32_ex", "sage_debug_e4m3",
           "sage_select_scratch_bytes", "sage_block_select", "sage_workspace_bytes_sparse",
           "sage_attn_fwd_sparse", "sage_density_schedule", "sage_attn_fwd_noalloc",
           "NOALLOC_SCRATCH_BYTES", "EXPORTS", "STATUS", "SAGE_PV_FP8", "SAGE_PV_BF16", "SAGE_QK_PER_TOKEN",
           "SAGE_K_BLOCK_MEAN", "mode_bits"]

HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(HERE, "libsage_attn.so")

STATUS = {0: "SAGE_OK", -1: "SAGE_EINVAL", -2: "SAGE_EUNSUPPORTED", -3: "SAGE_EALIGN",
          -4: "SAGE_EWORKSPACE", -5: "SAGE_EHIP"}

EXPORTS = ["sage_last_error", "sage_kernel_info", "sage_padded_tokens",
           "sage_quant_scratch_bytes", "sage_workspace_bytes", "sage_workspace_bytes_ex",
           "sage_quant_qk", "sage_quant_qk_ex", "sage_attn_fwd_prequant", "sage_attn_fwd",
           "sage_attn_fwd_ex", "sage_select_scratch_bytes", "sage_block_select",
           "sage_workspace_bytes_sparse", "sage_attn_fwd_sparse", "sage_debug_qk_i32",
           "sage_debug_qk_i32_ex", "sage_debug_e4m3", "sage_attn_fwd_noalloc",
           "sage_density_schedule"]

NOALLOC_SCRATCH_BYTES = 64 << 20        # SAGE_NOALLOC_SCRATCH_BYTES

SAGE_PV_FP8, SAGE_PV_BF16, SAGE_QK_PER_TOKEN, SAGE_K_BLOCK_MEAN = 0, 1, 2, 4


def mode_bits(pv: str = "fp8", per_token: bool = False, k_block_mean: bool = False) -> int:
    """The C mode bits for P.V precision ``pv`` ('fp8' or 'bf16'), per-token Q/K scales
    and block-residual K."""
    if pv not in ("fp8", "bf16"):
        raise ValueError(f"pv must be 'fp8' or 'bf16', got {pv!r}")
    return ((SAGE_PV_BF16 if pv == "bf16" else 0) | (SAGE_QK_PER_TOKEN if per_token else 0) |
            (SAGE_K_BLOCK_MEAN if k_block_mean else 0))


class SageError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {message}")


class sage_strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class sage_info(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("kv_tile", ctypes.c_int),
                ("quant_block", ctypes.c_int), ("token_align", ctypes.c_int),
                ("p_scale", ctypes.c_float), ("d_supported_mask", ctypes.c_int),
                ("arch", ctypes.c_char * 16)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "sage_last_error": (ctypes.c_char_p, []),
    "sage_kernel_info": (_I, [ctypes.POINTER(sage_info)]),
    "sage_padded_tokens": (ctypes.c_int64, [_I]),
    "sage_quant_scratch_bytes": (_I, [_I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "sage_workspace_bytes": (_I, [_I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "sage_workspace_bytes_ex": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "sage_quant_qk": (_I, [_P, _P, _P, ctypes.POINTER(sage_strides), ctypes.POINTER(sage_strides),
                           ctypes.POINTER(sage_strides), _I, _I, _I, _I,
                           _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sage_quant_qk_ex": (_I, [_P, _P, _P, ctypes.POINTER(sage_strides), ctypes.POINTER(sage_strides),
                              ctypes.POINTER(sage_strides), _I, _I, _I, _I, _I,
                              _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sage_attn_fwd_prequant": (_I, [_P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(sage_strides),
                                    _I, _I, _I, _I, ctypes.c_float, _P]),
    "sage_attn_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float,
                           ctypes.POINTER(sage_strides), _P, _P, _SZ]),
    "sage_attn_fwd_ex": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float,
                              ctypes.POINTER(sage_strides), _I, _P, _P, _SZ]),
    "sage_select_scratch_bytes": (_I, [_I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "sage_block_select": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "sage_workspace_bytes_sparse": (_I, [_I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "sage_attn_fwd_sparse": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float,
                                  ctypes.POINTER(sage_strides), ctypes.c_float, _P, _P, _SZ]),
    "sage_debug_qk_i32": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "sage_debug_qk_i32_ex": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "sage_debug_e4m3": (_I, [_P, _P, ctypes.c_int64, _P]),
    "sage_density_schedule": (_I, [_I, _I, ctypes.c_float, ctypes.c_float, ctypes.POINTER(ctypes.c_float)]),
    "sage_attn_fwd_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float,
                                   ctypes.POINTER(sage_strides), _P]),
}

_lib = None


def load():
    """Load the built library (raises if it has not been built: there is no other path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is missing: build it with "
                              "`python -m quantized_attention_diffusion_amd.build`")
        lib = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise SageError(status, sage_last_error())


def sage_last_error() -> str:
    return load().sage_last_error().decode()


def sage_kernel_info() -> dict:
    info = sage_info()
    _check(load().sage_kernel_info(ctypes.byref(info)))
    return dict(block_m=info.block_m, kv_tile=info.kv_tile, quant_block=info.quant_block,
                token_align=info.token_align, p_scale=info.p_scale,
                d_supported=[64 * (i + 1) for i in range(8) if info.d_supported_mask >> i & 1],
                arch=info.arch.decode())


def sage_padded_tokens(N: int) -> int:
    return int(load().sage_padded_tokens(N))


def sage_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    n = _SZ()
    _check(load().sage_workspace_bytes(B, H, N, d, ctypes.byref(n)))
    return n.value


def sage_workspace_bytes_ex(B: int, H: int, N: int, d: int, mode: int = 0) -> int:
    n = _SZ()
    _check(load().sage_workspace_bytes_ex(B, H, N, d, int(mode), ctypes.byref(n)))
    return n.value


def sage_quant_scratch_bytes(B: int, H: int, N: int, d: int) -> int:
    n = _SZ()
    _check(load().sage_quant_scratch_bytes(B, H, N, d, ctypes.byref(n)))
    return n.value


# ------------------------------------------------------------------ marshalling
def _dims(t: torch.Tensor, layout: str):
    """(B, H, N, d) and the element strides of a 4-D view in ``layout`` ('bnhd' or
    'bhnd')."""
    if t.dim() != 4:
        raise ValueError(f"expected a 4-D tensor, got shape {tuple(t.shape)}")
    if t.stride(3) != 1:
        raise ValueError("the channel dimension must be contiguous")
    if layout == "bnhd":
        B, N, H, d = t.shape
        st = sage_strides(t.stride(0), t.stride(2), t.stride(1))
    elif layout == "bhnd":
        B, H, N, d = t.shape
        st = sage_strides(t.stride(0), t.stride(1), t.stride(2))
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return (B, H, N, d), st


def _bf16_cuda(name, t):
    if t.dtype != torch.bfloat16 or t.device.type != "cuda":
        raise TypeError(f"{name} must be a bfloat16 CUDA tensor (got {t.dtype} on {t.device})")


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _quant_specs(B, H, N, d, mode=0) -> dict:
    """(shape, dtype) of every quantised operand of sage_quant_qk_ex in ``mode``."""
    npad = sage_padded_tokens(N)
    nsc = npad if mode & SAGE_QK_PER_TOKEN else npad // 64
    vdt = torch.bfloat16 if mode & SAGE_PV_BF16 else torch.uint8
    return dict(
        q_i8=((B, H, npad, d), torch.int8),
        q_scale=((B, H, nsc), torch.float32),
        k_i8=((B, H, npad, d), torch.int8),
        k_scale=((B, H, nsc), torch.float32),
        k_mean=((B, H, npad // 64, d) if mode & SAGE_K_BLOCK_MEAN else (B, H, d), torch.bfloat16),
        v_f8=((B, H, d, npad), vdt),
        v_scale=((B, H, d), torch.float32),
    )


def _alloc_quant(B, H, N, d, dev, mode=0):
    return {name: torch.empty(shape, dtype=dt, device=dev)
            for name, (shape, dt) in _quant_specs(B, H, N, d, mode).items()}


def _check_quant_out(o: dict, B, H, N, d, dev, mode):
    """A caller-supplied operand dict must match the layout of ``mode`` exactly: the
    library writes that many bytes into each buffer."""
    for name, (shape, dt) in _quant_specs(B, H, N, d, mode).items():
        t = o.get(name)
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"out[{name!r}] is missing")
        if t.dtype != dt or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"out[{name!r}] must be a contiguous {dt} tensor of shape {tuple(shape)} on "
                             f"{dev} for mode {mode} (got {t.dtype} {tuple(t.shape)} on {t.device})")


def sage_quant_qk(q, k, v, layout: str = "bnhd", out: dict | None = None,
                  scratch: torch.Tensor | None = None) -> dict:
    """Quantise Q, K, V (bf16 CUDA views in ``layout``).  Returns the dict of quantised
    operands (padded layouts of the C header) plus 'N'."""
    return sage_quant_qk_ex(q, k, v, 0, layout=layout, out=out, scratch=scratch, _entry="sage_quant_qk")


def sage_quant_qk_ex(q, k, v, mode: int, layout: str = "bnhd", out: dict | None = None,
                     scratch: torch.Tensor | None = None, _entry: str = "sage_quant_qk_ex") -> dict:
    """sage_quant_qk with mode bits (per-token scales, bf16 V).  The dict also holds
    'mode'."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _bf16_cuda(n, t)
    (B, H, N, d), sq = _dims(q, layout)
    dk, sk = _dims(k, layout)
    dv, sv = _dims(v, layout)
    if dk != (B, H, N, d) or dv != (B, H, N, d):
        raise ValueError("q, k and v must have the same shape")
    dev = q.device
    if out is not None:
        _check_quant_out(out, B, H, N, d, dev, mode)
    o = out if out is not None else _alloc_quant(B, H, N, d, dev, mode)
    if scratch is None:
        scratch = torch.empty(sage_quant_scratch_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    ptrs = (o["q_i8"].data_ptr(), o["q_scale"].data_ptr(), o["k_i8"].data_ptr(),
            o["k_scale"].data_ptr(), o["k_mean"].data_ptr(), o["v_f8"].data_ptr(),
            o["v_scale"].data_ptr(), scratch.data_ptr(), scratch.numel(), _stream(dev))
    head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(sq), ctypes.byref(sk),
            ctypes.byref(sv), B, H, N, d)
    if _entry == "sage_quant_qk":
        _check(load().sage_quant_qk(*head, *ptrs))
    else:
        _check(load().sage_quant_qk_ex(*head, int(mode), *ptrs))
    o["N"] = N
    o["mode"] = int(mode)
    return o


def _scale_arg(sm_scale) -> float:
    """None selects the library's default 1/sqrt(d) (passed as 0)."""
    return 0.0 if sm_scale is None else float(sm_scale)


def sage_attn_fwd_prequant(quant: dict, out: torch.Tensor | None = None,
                           sm_scale: float | None = None, layout: str = "bnhd") -> torch.Tensor:
    """Attention on operands produced by :func:`sage_quant_qk` (mode 0: the C entry
    point takes 64-token scales and FP8 V only).  Returns ``out``."""
    if int(quant.get("mode", 0)) != 0:
        raise ValueError(f"sage_attn_fwd_prequant takes mode-0 operands (got mode {quant['mode']}); "
                         "use sage_attn_fwd_ex for the other modes")
    B, H, npad, d = quant["q_i8"].shape
    N = int(quant["N"])
    dev = quant["q_i8"].device
    if out is None:
        shape = (B, N, H, d) if layout == "bnhd" else (B, H, N, d)
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _bf16_cuda("out", out)
    dims, so = _dims(out, layout)
    if dims != (B, H, N, d):
        raise ValueError(f"out has dims {dims}, expected {(B, H, N, d)}")
    sm = _scale_arg(sm_scale)
    _check(load().sage_attn_fwd_prequant(
        quant["q_i8"].data_ptr(), quant["q_scale"].data_ptr(), quant["k_i8"].data_ptr(),
        quant["k_scale"].data_ptr(), quant["v_f8"].data_ptr(), quant["v_scale"].data_ptr(),
        out.data_ptr(), ctypes.byref(so), B, H, N, d, sm, _stream(dev)))
    return out


def sage_attn_fwd(q, k, v, out: torch.Tensor | None = None, sm_scale: float | None = None,
                  layout: str = "bnhd", workspace: torch.Tensor | None = None) -> torch.Tensor:
    """O = softmax(Q K^T * sm_scale) V by the quantised path.  q, k, v, out: bf16 CUDA
    views in ``layout`` ('bnhd' = [B, N, H, d], 'bhnd' = [B, H, N, d]); any strides with
    a contiguous channel dimension (e.g. slices of a fused qkv tensor)."""
    return sage_attn_fwd_ex(q, k, v, out=out, sm_scale=sm_scale, layout=layout,
                            workspace=workspace, _entry="sage_attn_fwd")


def sage_attn_fwd_ex(q, k, v, out: torch.Tensor | None = None, sm_scale: float | None = None,
                     layout: str = "bnhd", workspace: torch.Tensor | None = None,
                     pv: str = "fp8", per_token: bool = False, k_block_mean: bool = False,
                     _entry: str = "sage_attn_fwd_ex") -> torch.Tensor:
    """sage_attn_fwd with options: ``pv`` = 'fp8' (speed, the default path) or 'bf16'
    (P rounded to bf16, V unquantised); ``per_token``: one INT8 scale per Q and K token;
    ``k_block_mean``: block-residual K (FP8 P.V only)."""
    mode = mode_bits(pv, per_token, k_block_mean)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _bf16_cuda(n, t)
    (B, H, N, d), sq = _dims(q, layout)
    dk, sk = _dims(k, layout)
    dv, sv = _dims(v, layout)
    if dk != (B, H, N, d) or dv != (B, H, N, d):
        raise ValueError("q, k and v must have the same shape")
    dev = q.device
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    _bf16_cuda("out", out)
    do, so = _dims(out, layout)
    if do != (B, H, N, d):
        raise ValueError("out must have the shape of q")
    if workspace is None:
        workspace = torch.empty(sage_workspace_bytes_ex(B, H, N, d, mode), dtype=torch.uint8, device=dev)
    sm = _scale_arg(sm_scale)
    strides = (sage_strides * 4)(sq, sk, sv, so)
    if _entry == "sage_attn_fwd":
        _check(load().sage_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    B, H, N, d, sm, strides, _stream(dev), workspace.data_ptr(),
                                    workspace.numel()))
    else:
        _check(load().sage_attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       B, H, N, d, sm, strides, mode, _stream(dev),
                                       workspace.data_ptr(), workspace.numel()))
    return out


def sage_attn_fwd_noalloc(q, k, v, out: torch.Tensor, sm_scale: float | None = None,
                          layout: str = "bnhd") -> torch.Tensor:
    """sage_attn_fwd without a workspace argument: the library's own device array
    serves (at most NOALLOC_SCRATCH_BYTES of workspace; calls on one device must not
    overlap).  ``out`` is the caller's; nothing is allocated."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _bf16_cuda(n, t)
    (B, H, N, d), sq = _dims(q, layout)
    dk, sk = _dims(k, layout)
    dv, sv = _dims(v, layout)
    do, so = _dims(out, layout)
    if dk != (B, H, N, d) or dv != (B, H, N, d) or do != (B, H, N, d):
        raise ValueError("q, k, v and out must have the same shape")
    strides = (sage_strides * 4)(sq, sk, sv, so)
    _check(load().sage_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        B, H, N, d, _scale_arg(sm_scale), strides, _stream(q.device)))
    return out


def sage_select_scratch_bytes(B: int, H: int, N: int, d: int) -> int:
    n = _SZ()
    _check(load().sage_select_scratch_bytes(B, H, N, d, ctypes.byref(n)))
    return n.value


def sage_workspace_bytes_sparse(B: int, H: int, N: int, d: int) -> int:
    n = _SZ()
    _check(load().sage_workspace_bytes_sparse(B, H, N, d, ctypes.byref(n)))
    return n.value


def sage_block_select(quant: dict, density: float, return_importance: bool = False):
    """Kept key tiles of every query block for ``density`` from the operands of
    :func:`sage_quant_qk`: (tile_count int32 [B, H, nqb], tile_list int32 [B, H, nqb, T]
    whose rows start with the tile_count kept tiles in ascending order), plus the fp64
    importance matrix [B, H, nqb, T] from the scratch with ``return_importance``."""
    B, H, npad, d = quant["q_i8"].shape
    N = int(quant["N"])
    dev = quant["q_i8"].device
    nt = npad // sage_kernel_info()["kv_tile"]
    count = torch.zeros((B, H, nt), dtype=torch.int32, device=dev)
    lists = torch.full((B, H, nt, nt), -1, dtype=torch.int32, device=dev)
    scratch = torch.empty(sage_select_scratch_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    _check(load().sage_block_select(
        quant["q_i8"].data_ptr(), quant["q_scale"].data_ptr(), quant["k_i8"].data_ptr(),
        quant["k_scale"].data_ptr(), B, H, N, d, float(density), count.data_ptr(), lists.data_ptr(),
        scratch.data_ptr(), scratch.numel(), _stream(dev)))
    if not return_importance:
        return count, lists
    sums_bytes = -(-2 * B * H * (npad // 64) * 2 * d // 256) * 256     # code sums as two int8 digits
    imp = scratch[sums_bytes:sums_bytes + B * H * nt * nt * 8].view(torch.float64).reshape(B, H, nt, nt)
    return count, lists, imp


def sage_density_schedule(step: int, n_steps: int, tau_start: float, tau_end: float = 1.0) -> float:
    """Density of sampling step ``step`` of ``n_steps``, moving linearly from tau_start
    (first step) to tau_end (last step); see the C header."""
    tau = ctypes.c_float(0.0)
    _check(load().sage_density_schedule(int(step), int(n_steps), ctypes.c_float(tau_start),
                                        ctypes.c_float(tau_end), ctypes.byref(tau)))
    return tau.value


def sage_attn_fwd_sparse(q, k, v, density: float, out: torch.Tensor | None = None,
                         sm_scale: float | None = None, layout: str = "bnhd",
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Block-sparse sage_attn_fwd: each block of 128 queries visits the key tiles of
    largest importance, a fraction ``density`` of them (1 gives the dense result)."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _bf16_cuda(n, t)
    (B, H, N, d), sq = _dims(q, layout)
    dk, sk = _dims(k, layout)
    dv, sv = _dims(v, layout)
    if dk != (B, H, N, d) or dv != (B, H, N, d):
        raise ValueError("q, k and v must have the same shape")
    dev = q.device
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    _bf16_cuda("out", out)
    do, so = _dims(out, layout)
    if do != (B, H, N, d):
        raise ValueError("out must have the shape of q")
    if workspace is None:
        workspace = torch.empty(sage_workspace_bytes_sparse(B, H, N, d), dtype=torch.uint8, device=dev)
    sm = _scale_arg(sm_scale)
    strides = (sage_strides * 4)(sq, sk, sv, so)
    _check(load().sage_attn_fwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       B, H, N, d, sm, strides, float(density), _stream(dev),
                                       workspace.data_ptr(), workspace.numel()))
    return out


def sage_debug_qk_i32(q_i8, k_i8, N: int, b: int, h: int, q_block: int, kv_tile: int,
                      n_q_blocks: int = 1, n_kv_tiles: int = 1) -> torch.Tensor:
    """Int32 S tiles of head (b, h) from the quantised operands (see the C header)."""
    B, H, npad, d = q_i8.shape
    info = sage_kernel_info()
    s = torch.empty((n_q_blocks * info["block_m"], n_kv_tiles * info["kv_tile"]),
                    dtype=torch.int32, device=q_i8.device)
    _check(load().sage_debug_qk_i32(q_i8.data_ptr(), k_i8.data_ptr(), B, H, N, d, b, h,
                                    q_block, kv_tile, n_q_blocks, n_kv_tiles, s.data_ptr(),
                                    _stream(q_i8.device)))
    return s


def sage_debug_qk_i32_ex(q_i8, k_i8, N: int, b: int, h: int, q_block: int, kv_tile: int,
                         n_q_blocks: int = 1, n_kv_tiles: int = 1, mode: int = 0) -> torch.Tensor:
    """sage_debug_qk_i32 through the attention body that ``mode`` (SAGE_* bits) selects."""
    B, H, npad, d = q_i8.shape
    info = sage_kernel_info()
    s = torch.empty((n_q_blocks * info["block_m"], n_kv_tiles * info["kv_tile"]),
                    dtype=torch.int32, device=q_i8.device)
    _check(load().sage_debug_qk_i32_ex(q_i8.data_ptr(), k_i8.data_ptr(), B, H, N, d, b, h,
                                       q_block, kv_tile, n_q_blocks, n_kv_tiles, int(mode),
                                       s.data_ptr(), _stream(q_i8.device)))
    return s


def sage_debug_e4m3(x: torch.Tensor) -> torch.Tensor:
    """Device fp32 -> e4m3 codes (the conversion used for V)."""
    if x.dtype != torch.float32 or x.device.type != "cuda" or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 CUDA tensor")
    y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(load().sage_debug_e4m3(x.data_ptr(), y.data_ptr(), x.numel(), _stream(x.device)))
    return y
