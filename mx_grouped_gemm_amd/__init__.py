"""MI355X-native grouped block-scaled low-precision GEMM.

Python binding of ``libbsgemm.so`` (the C ABI declared in ``include/bsgemm.h``). It only
marshals arguments: every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream. There is no fallback: if the
library is missing or the device is not gfx950 the calls raise.
"""

import ctypes
import os

import torch

__all__ = [
    "BsgemmError", "ELEM", "SCALE", "OUT", "make_fmt", "bsgemm_build_tiles", "bsgemm_grouped",
    "check_grouped_args", "check_permute_args", "bsgemm_grouped_workspace_size", "bsgemm_grouped_ws",
    "bsgemm_grouped_noalloc",
    "bsgemm_status_string", "bsgemm_route_counts", "bsgemm_quantize_permute", "library_path",
    "load_library",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG_DIR, "libbsgemm.so")
_lib = None

ELEM = {"e4m3": 1, "e2m1": 2}
SCALE = {"blockwise": 1, "mx": 2, "nv": 3}
OUT = {"f32": 1, "bf16": 2, "f16": 3}
OUT_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
EXPORTED = ("bsgemm_build_tiles", "bsgemm_grouped", "bsgemm_status_string", "bsgemm_route_counts",
            "bsgemm_quantize_permute", "bsgemm_grouped_workspace_size", "bsgemm_grouped_ws",
            "bsgemm_grouped_noalloc")


class BsgemmError(RuntimeError):
    def __init__(self, func, status):
        super().__init__(f"{func} failed: {bsgemm_status_string(status)} (status {status})")
        self.status = status


def library_path():
    return _LIB_PATH


def load_library():
    """Load ``libbsgemm.so`` and declare its C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m mx_grouped_gemm_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
    lib.bsgemm_build_tiles.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    lib.bsgemm_build_tiles.restype = ctypes.c_int
    lib.bsgemm_grouped.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, u32, vp]
    lib.bsgemm_grouped.restype = ctypes.c_int
    lib.bsgemm_status_string.argtypes = [ctypes.c_int]
    lib.bsgemm_status_string.restype = ctypes.c_char_p
    lib.bsgemm_route_counts.argtypes = [vp, i32, i32, vp, vp]
    lib.bsgemm_route_counts.restype = ctypes.c_int
    lib.bsgemm_quantize_permute.argtypes = [vp, u32, vp, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp]
    lib.bsgemm_quantize_permute.restype = ctypes.c_int
    lib.bsgemm_grouped_workspace_size.argtypes = [ctypes.POINTER(ctypes.c_size_t)]
    lib.bsgemm_grouped_workspace_size.restype = ctypes.c_int
    lib.bsgemm_grouped_ws.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, u32, vp,
                                      ctypes.c_size_t, vp]
    lib.bsgemm_grouped_ws.restype = ctypes.c_int
    lib.bsgemm_grouped_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, u32, vp]
    lib.bsgemm_grouped_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def bsgemm_status_string(status):
    return load_library().bsgemm_status_string(int(status)).decode()


SCHED_SMALL_M = 1 << 16


def make_fmt(a_elem, b_elem, scale, out, small_m=False):
    """Pack element formats, scale kind and output type into the C ABI's ``fmt`` word
    (``small_m``: the schedule for M-tiles of few rows, blockwise only)."""
    return (ELEM[a_elem] | (ELEM[b_elem] << 4) | (SCALE[scale] << 8) | (OUT[out] << 12)
            | (SCHED_SMALL_M if small_m else 0))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _nbytes(t):
    return t.numel() * t.element_size()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _byte_tensor(t, name, nbytes):
    _need(t.element_size() == 1, f"{name} must hold one byte per element, got {t.dtype}")
    _need(t.numel() >= nbytes, f"{name} holds {t.numel()} bytes, the call needs {nbytes}")


def _f32_tensor(t, name, n):
    _need(t.dtype == torch.float32, f"{name} must be float32, got {t.dtype}")
    _need(t.numel() >= n, f"{name} holds {t.numel()} floats, the call needs {n}")


def _i32_len(t, name, n):
    _need(t.dtype == torch.int32, f"{name} must be int32, got {t.dtype}")
    _need(t.numel() >= n, f"{name} holds {t.numel()} entries, the call needs {n}")


_OUT_NAME = {v: k for k, v in OUT.items()}


def check_grouped_args(A, a_scales, B, b_scales, expert_ids, tile_offsets, C, M, N, K, fmt,
                       num_tiles, num_experts):
    """Check that every tensor is large enough, and of the right type, for the sizes and ``fmt``
    of a ``bsgemm_grouped`` call. The C ABI receives bare pointers and cannot check this: a
    buffer that is too small would be read or written past its end on the GPU. Raises
    ValueError. Sizes or formats the library itself rejects (negative sizes, N or K not a
    multiple of 128, an unknown ``fmt``) are left to its status code."""
    fa, fb, sk, out = fmt & 0xF, (fmt >> 4) & 0xF, (fmt >> 8) & 0xF, (fmt >> 12) & 0xF
    if (M <= 0 or N <= 0 or K <= 0 or N % 128 or K % 128 or num_experts < 1 or num_tiles < 0
            or fa not in (1, 2) or fb not in (1, 2) or sk not in (1, 2, 3) or out not in _OUT_NAME):
        return
    dense = expert_ids is None and tile_offsets is None
    E = 1 if dense else num_experts
    if not dense:
        _need(expert_ids is not None and tile_offsets is not None,
              "expert_ids and tile_offsets are both given or both None")
        _i32_len(expert_ids, "expert_ids", num_tiles)
        _i32_len(tile_offsets, "tile_offsets", num_tiles + 1)
    row_a = K if fa == ELEM["e4m3"] else K // 2
    row_b = K if fb == ELEM["e4m3"] else K // 2
    _byte_tensor(A, "A", M * row_a)
    _byte_tensor(B, "B", E * N * row_b)
    if sk == SCALE["blockwise"]:
        _f32_tensor(a_scales, "a_scales", M * (K // 128))
        _f32_tensor(b_scales, "b_scales", E * (N // 128) * (K // 128))
    else:
        per = 32 if sk == SCALE["mx"] else 16
        _byte_tensor(a_scales, "a_scales", M * (K // per))
        _byte_tensor(b_scales, "b_scales", E * N * (K // per))
    want = OUT_DTYPE[_OUT_NAME[out]]
    _need(C.dtype == want, f"C must be {want} for this fmt, got {C.dtype}")
    _need(C.numel() >= M * N, f"C holds {C.numel()} elements, the call needs {M * N}")


def bsgemm_build_tiles(counts, num_tiles, padded=True, expert_offsets=None, tile_offsets=None,
                       expert_ids=None, stream=None):
    """Token-to-expert tile map from per-expert row counts (int32 device tensor).

    Returns ``(expert_offsets[E+1], tile_offsets[T+1], expert_ids[T])`` int32 device tensors,
    allocated here unless given.
    """
    _dev(counts, "counts", torch.int32)
    E, dev = counts.numel(), counts.device
    if expert_offsets is None:
        expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if tile_offsets is None:
        tile_offsets = torch.empty(num_tiles + 1, dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(max(num_tiles, 1), dtype=torch.int32, device=dev)
    for t, n in ((expert_offsets, "expert_offsets"), (tile_offsets, "tile_offsets"), (expert_ids, "expert_ids")):
        _dev(t, n, torch.int32)
    _i32_len(expert_offsets, "expert_offsets", E + 1)
    _i32_len(tile_offsets, "tile_offsets", num_tiles + 1)
    _i32_len(expert_ids, "expert_ids", num_tiles)
    st = load_library().bsgemm_build_tiles(_ptr(counts), E, int(num_tiles), 1 if padded else 0,
                                           _ptr(expert_offsets), _ptr(tile_offsets),
                                           _ptr(expert_ids), _stream(stream))
    if st != 0:
        raise BsgemmError("bsgemm_build_tiles", st)
    return expert_offsets, tile_offsets, expert_ids[:num_tiles]


def bsgemm_grouped(A, a_scales, B, b_scales, expert_ids, tile_offsets, C, M, N, K, fmt,
                   num_tiles=None, num_experts=None, stream=None):
    """Grouped block-scaled GEMM into ``C`` (see ``include/bsgemm.h``).

    ``expert_ids`` / ``tile_offsets`` may both be None (one dense group). ``num_tiles``
    defaults to ``expert_ids.numel()``, ``num_experts`` to ``B.shape[0]`` for 3-D ``B``.
    """
    for t, n in ((A, "A"), (a_scales, "a_scales"), (B, "B"), (b_scales, "b_scales"), (C, "C")):
        _dev(t, n)
    _dev(expert_ids, "expert_ids", torch.int32)
    _dev(tile_offsets, "tile_offsets", torch.int32)
    if num_tiles is None:
        num_tiles = expert_ids.numel() if expert_ids is not None else 0
    if num_experts is None:
        num_experts = B.shape[0] if B.dim() == 3 else 1
    check_grouped_args(A, a_scales, B, b_scales, expert_ids, tile_offsets, C, int(M), int(N), int(K),
                       int(fmt), int(num_tiles), int(num_experts))
    st = load_library().bsgemm_grouped(
        _ptr(A), _ptr(a_scales), _ptr(B), _ptr(b_scales), _ptr(expert_ids), _ptr(tile_offsets),
        int(num_tiles), _ptr(C), int(M), int(N), int(K), int(num_experts), int(fmt), _stream(stream))
    if st != 0:
        raise BsgemmError("bsgemm_grouped", st)
    return C


def bsgemm_grouped_workspace_size():
    """Bytes of workspace ``bsgemm_grouped_ws`` needs on the current device."""
    n = ctypes.c_size_t(0)
    st = load_library().bsgemm_grouped_workspace_size(ctypes.byref(n))
    if st != 0:
        raise BsgemmError("bsgemm_grouped_workspace_size", st)
    return int(n.value)


def bsgemm_grouped_ws(A, a_scales, B, b_scales, expert_ids, tile_offsets, C, M, N, K, fmt, workspace,
                      num_tiles=None, num_experts=None, stream=None):
    """``bsgemm_grouped`` with a workspace (a contiguous device tensor of at least
    ``bsgemm_grouped_workspace_size()`` bytes) for the split schedule of the last work items."""
    for t, n in ((A, "A"), (a_scales, "a_scales"), (B, "B"), (b_scales, "b_scales"), (C, "C"),
                 (workspace, "workspace")):
        _dev(t, n)
    _dev(expert_ids, "expert_ids", torch.int32)
    _dev(tile_offsets, "tile_offsets", torch.int32)
    if num_tiles is None:
        num_tiles = expert_ids.numel() if expert_ids is not None else 0
    if num_experts is None:
        num_experts = B.shape[0] if B.dim() == 3 else 1
    check_grouped_args(A, a_scales, B, b_scales, expert_ids, tile_offsets, C, int(M), int(N), int(K),
                       int(fmt), int(num_tiles), int(num_experts))
    st = load_library().bsgemm_grouped_ws(
        _ptr(A), _ptr(a_scales), _ptr(B), _ptr(b_scales), _ptr(expert_ids), _ptr(tile_offsets),
        int(num_tiles), _ptr(C), int(M), int(N), int(K), int(num_experts), int(fmt), _ptr(workspace),
        _nbytes(workspace), _stream(stream))
    if st != 0:
        raise BsgemmError("bsgemm_grouped_ws", st)
    return C


def bsgemm_grouped_noalloc(A, a_scales, B, b_scales, expert_ids, tile_offsets, C, M, N, K, fmt,
                           num_tiles=None, num_experts=None, stream=None):
    """``bsgemm_grouped_ws`` with the library's own device scratch instead of a workspace: for
    callers that cannot allocate. Concurrent calls on one GPU race on that scratch."""
    for t, n in ((A, "A"), (a_scales, "a_scales"), (B, "B"), (b_scales, "b_scales"), (C, "C")):
        _dev(t, n)
    _dev(expert_ids, "expert_ids", torch.int32)
    _dev(tile_offsets, "tile_offsets", torch.int32)
    if num_tiles is None:
        num_tiles = expert_ids.numel() if expert_ids is not None else 0
    if num_experts is None:
        num_experts = B.shape[0] if B.dim() == 3 else 1
    check_grouped_args(A, a_scales, B, b_scales, expert_ids, tile_offsets, C, int(M), int(N), int(K),
                       int(fmt), int(num_tiles), int(num_experts))
    st = load_library().bsgemm_grouped_noalloc(
        _ptr(A), _ptr(a_scales), _ptr(B), _ptr(b_scales), _ptr(expert_ids), _ptr(tile_offsets),
        int(num_tiles), _ptr(C), int(M), int(N), int(K), int(num_experts), int(fmt), _stream(stream))
    if st != 0:
        raise BsgemmError("bsgemm_grouped_noalloc", st)
    return C


def bsgemm_route_counts(topk_ids, num_experts, counts=None, stream=None):
    """Picks per expert from int32 top-k ids (device tensor, any shape). Returns ``counts``."""
    _dev(topk_ids, "topk_ids", torch.int32)
    if counts is None:
        counts = torch.empty(num_experts, dtype=torch.int32, device=topk_ids.device)
    _dev(counts, "counts", torch.int32)
    _i32_len(counts, "counts", num_experts)
    st = load_library().bsgemm_route_counts(_ptr(topk_ids), topk_ids.numel(), int(num_experts),
                                            _ptr(counts), _stream(stream))
    if st != 0:
        raise BsgemmError("bsgemm_route_counts", st)
    return counts


def check_permute_args(x, topk_ids, expert_offsets, M, num_experts, dest, qa, a_scales):
    """Size and type checks of a ``bsgemm_quantize_permute`` call that the C ABI cannot make
    (see :func:`check_grouped_args`). Raises ValueError."""
    _need(x.dim() == 2, f"x must be [tokens, K], got shape {tuple(x.shape)}")
    tokens, K = x.shape
    _need(topk_ids.dim() == 2 and topk_ids.shape[0] == tokens,
          f"topk_ids must be [tokens={tokens}, top_k], got shape {tuple(topk_ids.shape)}")
    top_k = topk_ids.shape[1]
    if K <= 0 or K % 128 or M < 0 or num_experts < 1 or top_k < 1:
        return
    _i32_len(expert_offsets, "expert_offsets", num_experts + 1)
    _i32_len(dest, "dest", tokens * top_k)
    _need(tuple(qa.shape) == (M, K), f"qa must be [M={M}, K={K}], got shape {tuple(qa.shape)}")
    _byte_tensor(qa, "qa", M * K)
    _need(tuple(a_scales.shape) == (M, K // 128),
          f"a_scales must be [M={M}, K/128={K // 128}], got shape {tuple(a_scales.shape)}")
    _f32_tensor(a_scales, "a_scales", M * (K // 128))


def bsgemm_quantize_permute(x, topk_ids, expert_offsets, M, num_experts, dest=None, qa=None,
                            a_scales=None, stream=None):
    """Quantise token rows ``x`` ([tokens, K], fp32 or bf16) to e4m3 with 1x128 scales and place
    them at the rows of their top-k picks (``topk_ids`` int32 [tokens, top_k]) in the grouped
    layout given by ``expert_offsets``. Returns (dest, qa, a_scales)."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    _dev(x, "x")
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(expert_offsets, "expert_offsets", torch.int32)
    tokens, K = x.shape
    top_k = topk_ids.shape[1]
    dev = x.device
    if dest is None:
        dest = torch.empty(tokens, top_k, dtype=torch.int32, device=dev)
    if qa is None:
        qa = torch.empty(M, K, dtype=torch.uint8, device=dev)
    if a_scales is None:
        a_scales = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
    for t, n in ((dest, "dest"), (qa, "qa"), (a_scales, "a_scales")):
        _dev(t, n)
    check_permute_args(x, topk_ids, expert_offsets, M, num_experts, dest, qa, a_scales)
    x_dtype = OUT["f32"] if x.dtype == torch.float32 else OUT["bf16"]
    st = load_library().bsgemm_quantize_permute(
        _ptr(x), x_dtype, _ptr(topk_ids), int(tokens), int(top_k), int(K), int(num_experts),
        _ptr(expert_offsets), int(M), _ptr(dest), _ptr(qa), _ptr(a_scales), _stream(stream))
    if st != 0:
        raise BsgemmError("bsgemm_quantize_permute", st)
    return dest, qa, a_scales
