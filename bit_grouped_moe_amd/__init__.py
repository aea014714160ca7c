"""Python binding of libgq (grouped MoE matmul on 4-bit packed experts, MI355X).

The functions below carry the names of the C entry points declared in
``include/gq.h`` and only marshal arguments: they check tensor shapes,
dtypes, devices and contiguity, allocate outputs with torch when the caller
passes none, and call the library on torch's current stream.  Every step of
the computation runs in the HIP kernels of ``libgq.so``; there is no CPU or
PyTorch fallback.  If the library is missing, every call raises.

Build the library with ``python -m bit_grouped_moe_amd.build``.
"""

import ctypes
import os
from collections import namedtuple

import torch

__all__ = [
    "GQError", "load_library", "library_path", "EXPORTED_SYMBOLS", "TILE_M",
    "gq_route_max_tiles", "gq_route_sort", "gq_nf4_decode", "gq_mxfp4_decode",
    "gq_nf4_grouped_gemv", "gq_mxfp4_grouped_gemv", "gq_nf4_grouped_gemm",
    "gq_mxfp4_grouped_gemm", "gq_nf4_grouped_dgrad", "gq_mxfp4_grouped_dgrad",
    "gq_nf4_grouped_gemv_swiglu", "gq_nf4_grouped_gemm_swiglu", "gq_nf4_grouped_gemv_down_combine",
    "gq_moe_combine", "gq_act_split_e4m3", "gq_mxfp4_grouped_gemm_scaled",
    "gq_mxfp4_grouped_gemv_swiglu", "gq_mxfp4_grouped_gemm_scaled_swiglu",
    "gq_mxfp4_grouped_gemm_scaled_swiglu_split",
    "gq_mxfp4_grouped_gemv_down_combine", "gq_nf4_grouped_gemv_host", "gq_mxfp4_grouped_gemv_host",
    "OSS_ALPHA", "OSS_LIMIT", "Route",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
TILE_M = 256                       # the tile height the grouped GEMM kernels use
OSS_ALPHA = 1.702                  # gpt-oss gated unit: sigmoid slope
OSS_LIMIT = 7.0                    # gpt-oss gated unit: clamp

EXPORTED_SYMBOLS = (
    "gq_status_string", "gq_route_max_tiles", "gq_route_sort", "gq_nf4_decode",
    "gq_mxfp4_decode", "gq_nf4_grouped_gemv", "gq_mxfp4_grouped_gemv", "gq_nf4_grouped_gemm",
    "gq_mxfp4_grouped_gemm", "gq_nf4_grouped_dgrad", "gq_mxfp4_grouped_dgrad",
    "gq_nf4_grouped_gemv_swiglu", "gq_nf4_grouped_gemm_swiglu", "gq_nf4_grouped_gemv_down_combine",
    "gq_moe_combine", "gq_act_split_e4m3", "gq_mxfp4_grouped_gemm_scaled",
    "gq_mxfp4_grouped_gemv_swiglu", "gq_mxfp4_grouped_gemm_scaled_swiglu",
    "gq_mxfp4_grouped_gemm_scaled_swiglu_split",
    "gq_mxfp4_grouped_gemv_down_combine", "gq_nf4_grouped_gemv_host", "gq_mxfp4_grouped_gemv_host",
)

_i32, _i64, _p, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
_SIGNATURES = {
    "gq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gq_route_max_tiles": (_i32, [_i32, _i32, _i32, _i32]),
    "gq_route_sort": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _p, _p, _p, _i32, _p, _p]),
    "gq_nf4_decode": (ctypes.c_int, [_p, _p, _i64, _i32, _p, _p, _p]),
    "gq_mxfp4_decode": (ctypes.c_int, [_p, _p, _i64, _i32, _p, _p, _p]),
    "gq_nf4_grouped_gemv": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _p, _i32,
                                           _p, _p, _p]),
    "gq_mxfp4_grouped_gemv": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _p, _i32,
                                             _p, _p, _p]),
    "gq_nf4_grouped_gemm": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _i32, _p,
                                           _p, _p, _p, _p, _i32, _i32, _p, _p]),
    "gq_mxfp4_grouped_gemm": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _i32, _p,
                                             _p, _p, _p, _p, _i32, _i32, _p, _p]),
    "gq_nf4_grouped_dgrad": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _p, _p,
                                            _p, _p, _i32, _i32, _p, _p]),
    "gq_mxfp4_grouped_dgrad": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _p, _p,
                                              _p, _p, _i32, _i32, _p, _p]),
    "gq_nf4_grouped_gemv_swiglu": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _p,
                                                  _i32, _p, _p]),
    "gq_nf4_grouped_gemm_swiglu": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _i32,
                                                  _p, _p, _p, _p, _i32, _i32, _p, _p]),
    "gq_nf4_grouped_gemv_down_combine": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32,
                                                        _p, _i32, _p, _p, _p]),
    "gq_moe_combine": (ctypes.c_int, [_p, _i32, _i32, _i32, _i64, _p, _p, _p]),
    "gq_act_split_e4m3": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _p]),
    "gq_mxfp4_grouped_gemm_scaled": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32,
                                                    _p, _p, _p, _p, _p, _i32, _i32, _p, _p]),
    "gq_nf4_grouped_gemv_host": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _p,
                                                _i32, _p, _p, _p]),
    "gq_mxfp4_grouped_gemv_host": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _p,
                                                  _i32, _p, _p, _p]),
    "gq_mxfp4_grouped_gemv_down_combine": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32,
                                                          _i32, _p, _i32, _p, _p, _p]),
    "gq_mxfp4_grouped_gemv_swiglu": (ctypes.c_int, [_p, _i32, _i32, _i64, _p, _p, _i32, _i32, _p,
                                                    _i32, _f32, _f32, _p, _p]),
    "gq_mxfp4_grouped_gemm_scaled_swiglu": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _i32,
                                                           _i32, _i32, _f32, _f32, _p, _p, _p,
                                                           _p, _i32, _i32, _p, _p]),
    "gq_mxfp4_grouped_gemm_scaled_swiglu_split": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p,
                                                                 _i32, _i32, _i32, _f32, _f32,
                                                                 _p, _p, _p, _p, _i32, _i32, _p,
                                                                 _p, _p]),
}

_lib = None


class GQError(RuntimeError):
    """A libgq call returned a nonzero status, or the library is missing."""

    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


def library_path():
    return os.environ.get("GQ_LIBRARY", os.path.join(_HERE, "libgq.so"))


def load_library():
    """Load libgq.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise GQError(f"libgq.so not found at {path}; build it with "
                      "`python -m bit_grouped_moe_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status, what):
    if status != 0:
        lib = load_library()
        raise GQError(f"{what}: {lib.gq_status_string(status).decode()} (status {status})", status)


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


Route = namedtuple("Route", "expert_offsets sorted_pairs tiles num_tiles max_tiles tile_m "
                            "rows topk num_experts")


def gq_route_max_tiles(rows, topk, num_experts, tile_m=TILE_M):
    return int(load_library().gq_route_max_tiles(rows, topk, num_experts, tile_m))


def gq_route_sort(topk_ids, num_experts, tile_m=TILE_M, expert_offsets=None, sorted_pairs=None,
                  tiles=None, num_tiles=None):
    """Group the (token, slot) pairs of ``topk_ids`` int32 [rows, topk] by expert."""
    lib = load_library()
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    rows, topk = topk_ids.shape
    dev = topk_ids.device
    max_tiles = gq_route_max_tiles(rows, topk, num_experts, tile_m)
    if max_tiles < 0:
        raise GQError("gq_route_max_tiles: invalid arguments", 1)
    if expert_offsets is None:
        expert_offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    if sorted_pairs is None:
        sorted_pairs = torch.empty(rows * topk, dtype=torch.int32, device=dev)
    if tiles is None:
        tiles = torch.empty((max_tiles, 2), dtype=torch.int32, device=dev)
    if num_tiles is None:
        num_tiles = torch.empty(1, dtype=torch.int32, device=dev)
    st = lib.gq_route_sort(_ptr(topk_ids), rows, topk, num_experts, tile_m, _ptr(expert_offsets),
                           _ptr(sorted_pairs), _ptr(tiles), tiles.shape[0], _ptr(num_tiles),
                           _stream(topk_ids))
    _check(st, "gq_route_sort")
    return Route(expert_offsets, sorted_pairs, tiles, num_tiles, tiles.shape[0], tile_m, rows,
                 topk, num_experts)


def gq_nf4_decode(codes, absmax, out_f32=True, out_bf16=True):
    """Decode NF4 codes uint8 [..., K/2] with absmax float32 [..., K/64]."""
    lib = load_library()
    _dev(codes, "codes", torch.uint8)
    _dev(absmax, "absmax", torch.float32)
    K = codes.shape[-1] * 2
    n_rows = codes.numel() // (K // 2) if K else 0
    shape = tuple(codes.shape[:-1]) + (K,)
    f = torch.empty(shape, dtype=torch.float32, device=codes.device) if out_f32 is True else out_f32
    b = torch.empty(shape, dtype=torch.bfloat16, device=codes.device) if out_bf16 is True else out_bf16
    f = None if f is False else f
    b = None if b is False else b
    st = lib.gq_nf4_decode(_ptr(codes), _ptr(absmax), n_rows, K, _ptr(f), _ptr(b), _stream(codes))
    _check(st, "gq_nf4_decode")
    return f, b


def gq_mxfp4_decode(blocks, scales, out_f32=True, out_bf16=True):
    """Decode MXFP4 blocks uint8 [..., K/32, 16] with e8m0 scales uint8 [..., K/32]."""
    lib = load_library()
    _dev(blocks, "blocks", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    K = blocks.shape[-2] * 32
    n_rows = blocks.numel() // (K // 2) if K else 0
    shape = tuple(blocks.shape[:-2]) + (K,)
    f = torch.empty(shape, dtype=torch.float32, device=blocks.device) if out_f32 is True else out_f32
    b = torch.empty(shape, dtype=torch.bfloat16, device=blocks.device) if out_bf16 is True else out_bf16
    f = None if f is False else f
    b = None if b is False else b
    st = lib.gq_mxfp4_decode(_ptr(blocks), _ptr(scales), n_rows, K, _ptr(f), _ptr(b),
                             _stream(blocks))
    _check(st, "gq_mxfp4_decode")
    return f, b


def _x_args(x, name="x"):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be a bf16 device tensor")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return x.shape[0], x.shape[1], x.stride(0)


def _nf4_bank(codes, absmax):
    _dev(codes, "codes", torch.uint8, 3)
    _dev(absmax, "absmax", torch.float32, 3)
    E, N, half = codes.shape
    K = half * 2
    if tuple(absmax.shape) != (E, N, K // 64):
        raise ValueError("absmax must be [E, N, K/64]")
    return E, N, K


def _mx_bank(blocks, scales):
    _dev(blocks, "blocks", torch.uint8, 4)
    _dev(scales, "scales", torch.uint8, 3)
    E, N, nb, sixteen = blocks.shape
    if sixteen != 16 or tuple(scales.shape) != (E, N, nb):
        raise ValueError("blocks must be [E, N, K/32, 16] and scales [E, N, K/32]")
    return E, N, nb * 32


def _out(out, P, N, dev):
    if out is None:
        return torch.empty((P, N), dtype=torch.bfloat16, device=dev)
    _dev(out, "out", torch.bfloat16)
    if out.numel() != P * N:
        raise ValueError("out must hold rows*topk x N elements")
    return out


def _scale(pair_scale, P):
    if pair_scale is None:
        return None
    _dev(pair_scale, "pair_scale", torch.float32)
    if pair_scale.numel() != P:
        raise ValueError("pair_scale must hold one float per pair")
    return pair_scale


def _gemv_pairs(topk_ids, rows):
    """Pair count of a decode GEMV call: ``topk_ids`` must be [rows, topk]
    for the ``rows`` activation rows of x (the kernel reads pair p's row
    p / topk and writes rows*topk output rows)."""
    if topk_ids.dim() != 2 or topk_ids.shape[0] != rows:
        raise ValueError(f"topk_ids must be [rows={rows}, topk] (got {tuple(topk_ids.shape)})")
    return topk_ids.shape[0] * topk_ids.shape[1]


def gq_nf4_grouped_gemv(x, codes, absmax, topk_ids, pair_scale=None, out=None):
    """Decode-time grouped GEMV (<= 256 pairs) on NF4 experts; returns bf16 [rows*topk, N]."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    E, N, Kw = _nf4_bank(codes, absmax)
    if Kw != K:
        raise ValueError("x and codes disagree on K")
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    P = _gemv_pairs(topk_ids, rows)
    out = _out(out, P, N, x.device)
    st = lib.gq_nf4_grouped_gemv(_ptr(x), rows, K, xs, _ptr(codes), _ptr(absmax), E, N,
                                 _ptr(topk_ids), topk_ids.shape[1], _ptr(_scale(pair_scale, P)),
                                 _ptr(out), _stream(x))
    _check(st, "gq_nf4_grouped_gemv")
    return out


def gq_mxfp4_grouped_gemv(x, blocks, scales, topk_ids, pair_scale=None, out=None):
    """Decode-time grouped GEMV (<= 256 pairs) on MXFP4 experts; returns bf16 [rows*topk, N]."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    E, N, Kw = _mx_bank(blocks, scales)
    if Kw != K:
        raise ValueError("x and blocks disagree on K")
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    P = _gemv_pairs(topk_ids, rows)
    out = _out(out, P, N, x.device)
    st = lib.gq_mxfp4_grouped_gemv(_ptr(x), rows, K, xs, _ptr(blocks), _ptr(scales), E, N,
                                   _ptr(topk_ids), topk_ids.shape[1], _ptr(_scale(pair_scale, P)),
                                   _ptr(out), _stream(x))
    _check(st, "gq_mxfp4_grouped_gemv")
    return out


def gq_mxfp4_grouped_gemv_swiglu(x, blocks, scales, topk_ids, alpha=OSS_ALPHA, limit=OSS_LIMIT,
                                 out=None):
    """Decode gate_up GEMV on MXFP4 experts with gpt-oss's gated unit fused:
    blocks [E, 2I, K] with gate row 2j and up row 2j + 1; returns bf16
    [rows*topk, I] = gc * sigmoid(alpha gc) * (uc + 1) (gc = min(gate, limit),
    uc = up clipped to [-limit, limit])."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    E, N2, Kw = _mx_bank(blocks, scales)
    if Kw != K or N2 % 2:
        raise ValueError("x and blocks disagree on K, or the gate_up width is odd")
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    P = _gemv_pairs(topk_ids, rows)
    out = _out(out, P, N2 // 2, x.device)
    st = lib.gq_mxfp4_grouped_gemv_swiglu(_ptr(x), rows, K, xs, _ptr(blocks), _ptr(scales), E, N2,
                                          _ptr(topk_ids), topk_ids.shape[1], float(alpha),
                                          float(limit), _ptr(out), _stream(x))
    _check(st, "gq_mxfp4_grouped_gemv_swiglu")
    return out


def _host_bank(a, b, names):
    """Host-resident bank tensors: CPU, pinned, contiguous (the library maps
    them to device addresses and rejects memory that is not pinned)."""
    for t, n in zip((a, b), names):
        if t.device.type != "cpu" or not t.is_pinned():
            raise ValueError(f"{n} must be a pinned host tensor (pin_memory=True)")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")


def gq_nf4_grouped_gemv_host(x, codes, absmax, topk_ids, pair_scale=None, out=None):
    """Decode GEMV on NF4 experts resident in pinned host memory: codes uint8
    [E, N, K/2] and absmax float32 [E, N, K/64] are pinned CPU tensors; the
    kernel streams the routed experts' bytes over the host link.  x, topk_ids,
    pair_scale and out are device tensors.  Returns bf16 [rows*topk, N]."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    _host_bank(codes, absmax, ("codes", "absmax"))
    if codes.dtype != torch.uint8 or absmax.dtype != torch.float32 or codes.dim() != 3:
        raise ValueError("codes uint8 [E, N, K/2] and absmax float32 [E, N, K/64] expected")
    E, N, half = codes.shape
    if half * 2 != K or tuple(absmax.shape) != (E, N, K // 64):
        raise ValueError("x, codes and absmax disagree on the shapes")
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    P = _gemv_pairs(topk_ids, rows)
    out = _out(out, P, N, x.device)
    st = lib.gq_nf4_grouped_gemv_host(_ptr(x), rows, K, xs, _ptr(codes), _ptr(absmax), E, N,
                                      _ptr(topk_ids), topk_ids.shape[1],
                                      _ptr(_scale(pair_scale, P)), _ptr(out), _stream(x))
    _check(st, "gq_nf4_grouped_gemv_host")
    return out


def gq_mxfp4_grouped_gemv_host(x, blocks, scales, topk_ids, pair_scale=None, out=None):
    """Decode GEMV on MXFP4 experts resident in pinned host memory (blocks
    uint8 [E, N, K/32, 16], scales uint8 [E, N, K/32], pinned CPU tensors)."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    _host_bank(blocks, scales, ("blocks", "scales"))
    if blocks.dtype != torch.uint8 or scales.dtype != torch.uint8 or blocks.dim() != 4:
        raise ValueError("blocks uint8 [E, N, K/32, 16] and scales uint8 [E, N, K/32] expected")
    E, N, nb, sixteen = blocks.shape
    if sixteen != 16 or nb * 32 != K or tuple(scales.shape) != (E, N, nb):
        raise ValueError("x, blocks and scales disagree on the shapes")
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    P = _gemv_pairs(topk_ids, rows)
    out = _out(out, P, N, x.device)
    st = lib.gq_mxfp4_grouped_gemv_host(_ptr(x), rows, K, xs, _ptr(blocks), _ptr(scales), E, N,
                                        _ptr(topk_ids), topk_ids.shape[1],
                                        _ptr(_scale(pair_scale, P)), _ptr(out), _stream(x))
    _check(st, "gq_mxfp4_grouped_gemv_host")
    return out


def _route_ptrs(route):
    return (_ptr(route.expert_offsets), _ptr(route.sorted_pairs), _ptr(route.tiles),
            _ptr(route.num_tiles), route.max_tiles, route.tile_m)


def gq_nf4_grouped_gemm(x, codes, absmax, route, pair_scale=None, out=None):
    """Prefill grouped GEMM on NF4 experts using a ``gq_route_sort`` result."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    E, N, Kw = _nf4_bank(codes, absmax)
    if Kw != K or route.rows != rows or route.num_experts != E:
        raise ValueError("x, codes and route disagree")
    P = rows * route.topk
    out = _out(out, P, N, x.device)
    st = lib.gq_nf4_grouped_gemm(_ptr(x), rows, K, xs, _ptr(codes), _ptr(absmax), E, N,
                                 route.topk, _ptr(_scale(pair_scale, P)), *_route_ptrs(route),
                                 _ptr(out), _stream(x))
    _check(st, "gq_nf4_grouped_gemm")
    return out


def gq_mxfp4_grouped_gemm(x, blocks, scales, route, pair_scale=None, out=None):
    """Prefill grouped GEMM on MXFP4 experts using a ``gq_route_sort`` result."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    E, N, Kw = _mx_bank(blocks, scales)
    if Kw != K or route.rows != rows or route.num_experts != E:
        raise ValueError("x, blocks and route disagree")
    P = rows * route.topk
    out = _out(out, P, N, x.device)
    st = lib.gq_mxfp4_grouped_gemm(_ptr(x), rows, K, xs, _ptr(blocks), _ptr(scales), E, N,
                                   route.topk, _ptr(_scale(pair_scale, P)), *_route_ptrs(route),
                                   _ptr(out), _stream(x))
    _check(st, "gq_mxfp4_grouped_gemm")
    return out


def gq_nf4_grouped_dgrad(dy, codes, absmax, route, out=None):
    """dX = dY . W per pair through NF4 experts; ``route`` from gq_route_sort(pair ids [P, 1])."""
    lib = load_library()
    P, N, ds = _x_args(dy, "dy")
    E, Nw, K = _nf4_bank(codes, absmax)
    if Nw != N or route.rows * route.topk != P or route.topk != 1 or route.num_experts != E:
        raise ValueError("dy, codes and route disagree (route must be built with topk = 1)")
    out = _out(out, P, K, dy.device)
    st = lib.gq_nf4_grouped_dgrad(_ptr(dy), P, N, ds, _ptr(codes), _ptr(absmax), E, K,
                                  *_route_ptrs(route), _ptr(out), _stream(dy))
    _check(st, "gq_nf4_grouped_dgrad")
    return out


def gq_mxfp4_grouped_dgrad(dy, blocks, scales, route, out=None):
    """dX = dY . W per pair through MXFP4 experts; ``route`` from gq_route_sort(pair ids [P, 1])."""
    lib = load_library()
    P, N, ds = _x_args(dy, "dy")
    E, Nw, K = _mx_bank(blocks, scales)
    if Nw != N or route.rows * route.topk != P or route.topk != 1 or route.num_experts != E:
        raise ValueError("dy, blocks and route disagree (route must be built with topk = 1)")
    out = _out(out, P, K, dy.device)
    st = lib.gq_mxfp4_grouped_dgrad(_ptr(dy), P, N, ds, _ptr(blocks), _ptr(scales), E, K,
                                    *_route_ptrs(route), _ptr(out), _stream(dy))
    _check(st, "gq_mxfp4_grouped_dgrad")
    return out


# ---- MoE-layer epilogues ----------------------------------------------------
def gq_nf4_grouped_gemv_swiglu(x, codes, absmax, topk_ids, out=None):
    """Decode gate_up GEMV with SwiGLU fused: codes [E, 2I, K] (gate rows first);
    returns bf16 [rows*topk, I] = silu(gate) * up."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    E, N2, Kw = _nf4_bank(codes, absmax)
    if Kw != K or N2 % 2:
        raise ValueError("x and codes disagree on K, or the gate_up width is odd")
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    P = _gemv_pairs(topk_ids, rows)
    out = _out(out, P, N2 // 2, x.device)
    st = lib.gq_nf4_grouped_gemv_swiglu(_ptr(x), rows, K, xs, _ptr(codes), _ptr(absmax), E, N2,
                                        _ptr(topk_ids), topk_ids.shape[1], _ptr(out), _stream(x))
    _check(st, "gq_nf4_grouped_gemv_swiglu")
    return out


def gq_nf4_grouped_gemm_swiglu(x, codes, absmax, route, out=None):
    """Prefill gate_up GEMM with SwiGLU fused; returns bf16 [rows*topk, I]."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    E, N2, Kw = _nf4_bank(codes, absmax)
    if Kw != K or route.rows != rows or route.num_experts != E or N2 % 2:
        raise ValueError("x, codes and route disagree")
    P = rows * route.topk
    out = _out(out, P, N2 // 2, x.device)
    st = lib.gq_nf4_grouped_gemm_swiglu(_ptr(x), rows, K, xs, _ptr(codes), _ptr(absmax), E, N2,
                                        route.topk, *_route_ptrs(route), _ptr(out), _stream(x))
    _check(st, "gq_nf4_grouped_gemm_swiglu")
    return out


def _weights(topk_weights, rows, topk):
    if topk_weights is None:
        return None
    _dev(topk_weights, "topk_weights", torch.float32)
    if topk_weights.numel() != rows * topk:
        raise ValueError("topk_weights must hold rows x topk floats")
    return topk_weights


def gq_nf4_grouped_gemv_down_combine(act, codes, absmax, topk_ids, topk_weights=None, out=None):
    """Decode down GEMV with the router-weighted combine fused: act bf16 [rows*topk, I]
    (row p is pair p's input), codes [E, H, I]; returns bf16 [rows, H]."""
    lib = load_library()
    P, I, a_s = _x_args(act, "act")
    E, H, Iw = _nf4_bank(codes, absmax)
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    rows, topk = topk_ids.shape
    if Iw != I or rows * topk != P:
        raise ValueError("act, codes and topk_ids disagree")
    out = _out(out, rows, H, act.device)
    st = lib.gq_nf4_grouped_gemv_down_combine(_ptr(act), rows, I, a_s, _ptr(codes), _ptr(absmax),
                                              E, H, _ptr(topk_ids), topk,
                                              _ptr(_weights(topk_weights, rows, topk)), _ptr(out),
                                              _stream(act))
    _check(st, "gq_nf4_grouped_gemv_down_combine")
    return out


def gq_mxfp4_grouped_gemv_down_combine(act, blocks, scales, topk_ids, topk_weights=None,
                                       out=None):
    """Decode down GEMV on MXFP4 experts with the router-weighted combine fused:
    act bf16 [rows*topk, I] (row p is pair p's input), blocks [E, H, I];
    returns bf16 [rows, H]."""
    lib = load_library()
    P, I, a_s = _x_args(act, "act")
    E, H, Iw = _mx_bank(blocks, scales)
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    rows, topk = topk_ids.shape
    if Iw != I or rows * topk != P:
        raise ValueError("act, blocks and topk_ids disagree")
    out = _out(out, rows, H, act.device)
    st = lib.gq_mxfp4_grouped_gemv_down_combine(_ptr(act), rows, I, a_s, _ptr(blocks),
                                                _ptr(scales), E, H, _ptr(topk_ids), topk,
                                                _ptr(_weights(topk_weights, rows, topk)),
                                                _ptr(out), _stream(act))
    _check(st, "gq_mxfp4_grouped_gemv_down_combine")
    return out


def gq_moe_combine(y_pairs, topk, topk_weights=None, out=None):
    """y[t] = sum_s w[t, s] * y_pairs[t*topk + s] (plain sum without weights);
    y_pairs bf16 [rows*topk, H]; returns bf16 [rows, H]."""
    lib = load_library()
    P, H, ys = _x_args(y_pairs, "y_pairs")
    if P % topk:
        raise ValueError("y_pairs must hold rows*topk rows")
    rows = P // topk
    out = _out(out, rows, H, y_pairs.device)
    st = lib.gq_moe_combine(_ptr(y_pairs), rows, topk, H, ys,
                            _ptr(_weights(topk_weights, rows, topk)), _ptr(out), _stream(y_pairs))
    _check(st, "gq_moe_combine")
    return out


# ---- MXFP4 on the block-scaled fp4 matrix instruction ------------------------
def split_sizes(rows, K):
    """Byte shapes of gq_act_split_e4m3's outputs for x [rows, K]:
    (codes [rows, 2*Kp], scales [rows, Kp/16]) with Kp = K rounded up to 64."""
    kp = (K + 63) // 64 * 64
    return (rows, 2 * kp), (rows, kp // 16)


def gq_act_split_e4m3(x, codes=None, scales=None):
    """Two-term e4m3 split of bf16 activations x [rows, K]; returns the
    (codes, scales) uint8 tensors gq_mxfp4_grouped_gemm_scaled takes."""
    lib = load_library()
    rows, K, xs = _x_args(x)
    cshape, sshape = split_sizes(rows, K)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    _dev(codes, "codes", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    if tuple(codes.shape) != cshape or tuple(scales.shape) != sshape:
        raise ValueError(f"split buffers must be {cshape} and {sshape}")
    st = lib.gq_act_split_e4m3(_ptr(x), rows, K, xs, _ptr(codes), _ptr(scales), _stream(x))
    _check(st, "gq_act_split_e4m3")
    return codes, scales


def gq_mxfp4_grouped_gemm_scaled(x_split, blocks, scales, route, pair_scale=None, out=None):
    """Prefill grouped GEMM on MXFP4 experts through the block-scaled fp4
    instruction; ``x_split`` = gq_act_split_e4m3(x) for x [rows, K]."""
    lib = load_library()
    xq, xsc = x_split
    _dev(xq, "x_split codes", torch.uint8, 2)
    _dev(xsc, "x_split scales", torch.uint8, 2)
    E, N, K = _mx_bank(blocks, scales)
    rows = xq.shape[0]
    cshape, sshape = split_sizes(rows, K)
    if tuple(xq.shape) != cshape or tuple(xsc.shape) != sshape:
        raise ValueError("x_split does not match the weights' K")
    if route.rows != rows or route.num_experts != E:
        raise ValueError("x_split and route disagree")
    P = rows * route.topk
    out = _out(out, P, N, xq.device)
    st = lib.gq_mxfp4_grouped_gemm_scaled(_ptr(xq), _ptr(xsc), rows, K, _ptr(blocks),
                                          _ptr(scales), E, N, route.topk,
                                          _ptr(_scale(pair_scale, P)), *_route_ptrs(route),
                                          _ptr(out), _stream(xq))
    _check(st, "gq_mxfp4_grouped_gemm_scaled")
    return out


def gq_mxfp4_grouped_gemm_scaled_swiglu(x_split, blocks, scales, route, alpha=OSS_ALPHA,
                                        limit=OSS_LIMIT, out=None):
    """Prefill gate_up GEMM on the block-scaled fp4 instruction with gpt-oss's
    gated unit in the epilogue: blocks [E, 2I, K] (gate row 2j, up row
    2j + 1); returns bf16 [rows*topk, I]."""
    lib = load_library()
    xq, xsc = x_split
    _dev(xq, "x_split codes", torch.uint8, 2)
    _dev(xsc, "x_split scales", torch.uint8, 2)
    E, N2, K = _mx_bank(blocks, scales)
    if N2 % 2:
        raise ValueError("the gate_up width is odd")
    rows = xq.shape[0]
    cshape, sshape = split_sizes(rows, K)
    if tuple(xq.shape) != cshape or tuple(xsc.shape) != sshape:
        raise ValueError("x_split does not match the weights' K")
    if route.rows != rows or route.num_experts != E:
        raise ValueError("x_split and route disagree")
    P = rows * route.topk
    out = _out(out, P, N2 // 2, xq.device)
    st = lib.gq_mxfp4_grouped_gemm_scaled_swiglu(_ptr(xq), _ptr(xsc), rows, K, _ptr(blocks),
                                                 _ptr(scales), E, N2, route.topk, float(alpha),
                                                 float(limit), *_route_ptrs(route), _ptr(out),
                                                 _stream(xq))
    _check(st, "gq_mxfp4_grouped_gemm_scaled_swiglu")
    return out


def gq_mxfp4_grouped_gemm_scaled_swiglu_split(x_split, blocks, scales, route, alpha=OSS_ALPHA,
                                              limit=OSS_LIMIT, out=None):
    """gq_mxfp4_grouped_gemm_scaled_swiglu with the [rows*topk, I] result
    written as its two-term e4m3 split (the bytes gq_act_split_e4m3 would
    write for it); returns (codes, scales), the down product's x_split.
    ``out``: an optional (codes, scales) pair of the split_sizes shapes."""
    lib = load_library()
    xq, xsc = x_split
    _dev(xq, "x_split codes", torch.uint8, 2)
    _dev(xsc, "x_split scales", torch.uint8, 2)
    E, N2, K = _mx_bank(blocks, scales)
    if N2 % 2:
        raise ValueError("the gate_up width is odd")
    rows = xq.shape[0]
    cshape, sshape = split_sizes(rows, K)
    if tuple(xq.shape) != cshape or tuple(xsc.shape) != sshape:
        raise ValueError("x_split does not match the weights' K")
    if route.rows != rows or route.num_experts != E:
        raise ValueError("x_split and route disagree")
    P = rows * route.topk
    ocs, oss = split_sizes(P, N2 // 2)
    if out is None:
        out = (torch.empty(ocs, dtype=torch.uint8, device=xq.device),
               torch.empty(oss, dtype=torch.uint8, device=xq.device))
    oq, osc = out
    _dev(oq, "out codes", torch.uint8, 2)
    _dev(osc, "out scales", torch.uint8, 2)
    if tuple(oq.shape) != ocs or tuple(osc.shape) != oss:
        raise ValueError(f"out must be uint8 {ocs} and {oss}")
    st = lib.gq_mxfp4_grouped_gemm_scaled_swiglu_split(
        _ptr(xq), _ptr(xsc), rows, K, _ptr(blocks), _ptr(scales), E, N2, route.topk,
        float(alpha), float(limit), *_route_ptrs(route), _ptr(oq), _ptr(osc), _stream(xq))
    _check(st, "gq_mxfp4_grouped_gemm_scaled_swiglu_split")
    return oq, osc
