"""Python binding of the densegemm C ABI (``include/densegemm.h``).

Argument marshalling only: tensors become device pointers, leading dimensions
and the current HIP stream; every step of the computation runs in the HIP
library ``libdensegemm.so``.  There is no fallback: if the library is missing
the import of this package fails.

Functions mirror the C entry points:

  select_tile(M, N, K, dtype="bf16", num_cus=0) -> Tile
  shuffle_b_bytes(N, K, dtype="bf16") -> int
  shuffle_b(B, dtype=None, out=None) -> Bs (uint8 device tensor)
  gemm_bf16(A, Bs, N, out=None, tile=None) -> C
  gemm_fp8_scaled(A, Bs, N, scale_a, scale_b, out=None, tile=None) -> C
  gemm_status_string(code) -> str
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, replace

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdensegemm.so")

GEMM_OK = 0
GEMM_ERR_INVALID_VALUE = 1
GEMM_ERR_UNSUPPORTED = 2
GEMM_ERR_HIP = 3

GEMM_BF16 = 0
GEMM_FP8_E4M3 = 1

# bytes of the library's own split-K scratch behind gemm_bf16_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20
READ_PROBE_SLOTS = 32768

GEMM_KERNEL_TILED = 0
GEMM_KERNEL_SKINNY = 1
GEMM_KERNEL_TILED_AB = 2
GEMM_KERNEL_TILED_PP = 3

EXPORTS = ("select_tile", "shuffle_b_bytes", "shuffle_b", "gemm_bf16", "gemm_fp8_scaled",
           "gemm_tile_check", "gemm_status_string", "select_tile_ws", "gemm_workspace_bytes",
           "gemm_bf16_ws", "gemm_fp8_scaled_ws", "gemm_bf16_ex", "gemm_fp8_scaled_ex", "shuffle_b_t",
           "transpose_2d", "gemm_plan", "gemm_bf16_noalloc", "gemm_read_probe")

# gemm_activation
GEMM_ACT_NONE, GEMM_ACT_RELU, GEMM_ACT_SILU, GEMM_ACT_GELU_ERF, GEMM_ACT_GELU_TANH = 0, 1, 2, 3, 4
ACTIVATIONS = {None: GEMM_ACT_NONE, "none": GEMM_ACT_NONE, "relu": GEMM_ACT_RELU,
               "silu": GEMM_ACT_SILU, "gelu": GEMM_ACT_GELU_ERF, "gelu_erf": GEMM_ACT_GELU_ERF,
               "gelu_tanh": GEMM_ACT_GELU_TANH}


class GemmEpilogue(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("scale_m", ctypes.c_void_p),
                ("scale_n", ctypes.c_void_p), ("mul", ctypes.c_void_p),
                ("ld_mul", ctypes.c_int64), ("activation", ctypes.c_int32)]


class GemmTile(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("atom", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("k_split", ctypes.c_int32), ("lds_stages", ctypes.c_int32),
                ("tile_eff", ctypes.c_float), ("wq_eff", ctypes.c_float),
                ("predicted_us", ctypes.c_float), ("stream_k", ctypes.c_int32)]


@dataclass(frozen=True)
class Tile:
    kernel: int
    tile_m: int
    tile_n: int
    tile_k: int = 0
    atom: int = 16
    waves: int = 4
    k_split: int = 1
    lds_stages: int = 0
    tile_eff: float = 0.0
    wq_eff: float = 0.0
    predicted_us: float = 0.0
    stream_k: int = 0

    @property
    def name(self) -> str:
        """e.g. tiled128x128 (4 waves, 16x16 atom), ab256x256w8a32s4k32 (8 waves,
        32x32 atom, 4 stages, 32-element k-tile), tiled128x128a32s3k64sk4 (split
        over 4 K slices); unset fields are omitted."""
        atom = "" if self.atom in (0, 16) else f"a{self.atom}"
        pipe = (f"s{self.lds_stages}" if self.lds_stages else "") + (f"k{self.tile_k}" if self.tile_k else "")
        if self.kernel != GEMM_KERNEL_SKINNY and self.k_split > 1:
            pipe += f"sk{self.k_split}"
        if self.stream_k:
            pipe += "streamk"
        if self.kernel == GEMM_KERNEL_TILED:
            return f"tiled{self.tile_m}x{self.tile_n}" + ("" if self.waves == 4 else f"w{self.waves}") + \
                atom + pipe
        if self.kernel == GEMM_KERNEL_TILED_AB:
            return f"ab{self.tile_m}x{self.tile_n}w{self.waves}" + atom + pipe
        if self.kernel == GEMM_KERNEL_TILED_PP:
            return f"pp{self.tile_m}x{self.tile_n}" + atom + pipe
        return f"skinny{self.tile_m}x{self.tile_n}" + ("" if self.k_split in (0, 4) else f"w{self.k_split}")

    def to_c(self) -> GemmTile:
        return GemmTile(self.kernel, self.tile_m, self.tile_n, self.tile_k, self.atom, self.waves,
                        self.k_split, self.lds_stages, self.tile_eff, self.wq_eff, self.predicted_us,
                        self.stream_k)

    @staticmethod
    def from_c(t: GemmTile) -> "Tile":
        return Tile(t.kernel, t.tile_m, t.tile_n, t.tile_k, t.atom, t.waves, t.k_split,
                    t.lds_stages, t.tile_eff, t.wq_eff, t.predicted_us, t.stream_k)


def tiled(tm: int, tn: int, waves: int = 4, atom: int = 16, stages: int = 0, tile_k: int = 0,
          k_split: int = 1) -> Tile:
    """A rung of the tiled ladder; stages / tile_k (K elements per stage) 0 = any;
    k_split > 1 splits K over that many workgroups (needs a workspace)."""
    return Tile(GEMM_KERNEL_TILED, tm, tn, tile_k=tile_k, atom=atom, waves=waves, k_split=k_split,
                lds_stages=stages)


def tiled_ab(tm: int, tn: int, waves: int = 4, atom: int = 16, stages: int = 0, tile_k: int = 0,
             k_split: int = 1) -> Tile:
    """A rung of the A+B-in-LDS ladder; stages / tile_k 0 = any."""
    return Tile(GEMM_KERNEL_TILED_AB, tm, tn, tile_k=tile_k, atom=atom, waves=waves,
                k_split=k_split, lds_stages=stages)


def tiled_pp(tm: int, tn: int, atom: int = 32, stages: int = 0, tile_k: int = 0,
             k_split: int = 1) -> Tile:
    """A rung of the ping-pong A+B ladder (8 waves); stages / tile_k 0 = any."""
    return Tile(GEMM_KERNEL_TILED_PP, tm, tn, tile_k=tile_k, atom=atom, waves=8, k_split=k_split,
                lds_stages=stages)


def with_stream_k(tile: Tile) -> Tile:
    """The same one-pass tiled / A+B rung as a stream-K launch (needs a
    workspace of workspace_bytes(...) bytes)."""
    if tile.kernel not in (GEMM_KERNEL_TILED, GEMM_KERNEL_TILED_AB):
        raise ValueError("stream-K runs on tiled and A+B rungs")
    return replace(tile, stream_k=1, k_split=1)


def with_split(tile: Tile, k_split: int) -> Tile:
    """The same tiled rung split over k_split K slices."""
    if tile.kernel == GEMM_KERNEL_SKINNY:
        raise ValueError("the skinny kernel splits K inside one workgroup")
    return replace(tile, k_split=k_split)


def skinny(tm: int, tn: int, waves: int = 4) -> Tile:
    """A rung of the skinny ladder; `waves` split K inside one workgroup."""
    return Tile(GEMM_KERNEL_SKINNY, tm, tn, waves=waves, k_split=waves, lds_stages=0)


# The ladders of include/densegemm.h, as (tile_m, tile_n, waves, stages, atom,
# k-tile bytes).  8-wave tiled rungs arrange the waves 2 (M) x 4 (N); A+B
# rungs form 2 x (waves / 2).
TILED_LADDER = [(256, 128, 8, 2, 16, 128), (128, 256, 8, 2, 16, 128), (128, 128, 8, 2, 16, 128)] + \
    [(m, n, 4, 3, 16, 128) for m in (256, 128, 64, 32) for n in (256, 128, 64) if (m, n) != (256, 256)] + \
    [(256, 256, 8, 2, 32, 128), (256, 128, 8, 2, 32, 128), (128, 256, 8, 2, 32, 128),
     (128, 128, 8, 2, 32, 128), (256, 128, 4, 3, 32, 128), (128, 256, 4, 3, 32, 128),
     (128, 128, 4, 3, 32, 128), (64, 256, 4, 3, 32, 128), (64, 128, 4, 3, 32, 128),
     (128, 256, 4, 4, 32, 64), (128, 128, 4, 4, 32, 64), (256, 128, 4, 4, 32, 64)]
AB_LADDER = [(256, 128, 4, 3, 16, 128), (128, 256, 4, 3, 16, 128), (128, 128, 4, 3, 16, 128),
             (256, 256, 8, 2, 32, 128), (256, 256, 4, 2, 32, 128), (256, 128, 8, 3, 32, 128),
             (256, 128, 4, 3, 32, 128), (128, 256, 4, 3, 32, 128), (128, 128, 4, 3, 32, 128),
             (256, 256, 8, 4, 32, 64), (256, 256, 4, 4, 32, 64),
             (256, 128, 8, 6, 32, 64), (128, 256, 4, 6, 32, 64), (256, 256, 8, 4, 16, 64)]
# (tile_m, tile_n, waves splitting K)
# (tile_m, tile_n, stages, atom, k-tile bytes)
PP_LADDER = [(256, 256, 4, 32, 64)]
SKINNY_LADDER = [(m, n, 4) for m in (16, 32, 48, 64) for n in (16, 32, 64)] + \
    [(16, 16, 8), (16, 32, 8), (32, 16, 8), (32, 32, 8), (16, 16, 16), (32, 16, 16)]


def ladder_tiles(dtype="bf16"):
    """Every tiled and A+B rung, fully specified for an element type."""
    e = 2 if _dtype_code(dtype) == GEMM_BF16 else 1
    # e4m3 16 x 16 atoms take 128 K bytes per MFMA: 128-byte k-tiles only
    fits = lambda a, kb: not (e == 1 and a == 16 and kb != 128)  # noqa: E731
    return [tiled(m, n, w, a, st, kb // e) for m, n, w, st, a, kb in TILED_LADDER if fits(a, kb)] + \
        [tiled_ab(m, n, w, a, st, kb // e) for m, n, w, st, a, kb in AB_LADDER if fits(a, kb)] + \
        [tiled_pp(m, n, a, st, kb // e) for m, n, st, a, kb in PP_LADDER]


def all_tiles(M: int, dtype="bf16"):
    """Every rung usable for a GEMM with M rows."""
    t = ladder_tiles(dtype)
    if M <= 64:
        t += [skinny(m, n, w) for m, n, w in SKINNY_LADDER if M <= m < M + 16]
    return t


class GemmError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {gemm_status_string(code)}")
        self.code = code


def _load_lib():
    # Load torch's HIP runtime first.  torch ships its own libamdhip64 (soname
    # libamdhip64.so.7); once it is mapped, this library's dependency on that
    # soname resolves to the same copy, so the memory and streams torch hands
    # us belong to the runtime our kernels launch on.  Loading this library
    # first would map /opt/rocm's runtime as well: two HIP runtimes in one
    # process, and launches on torch's streams fail.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g;"
                          f" g.build()'` (hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.select_tile.argtypes = [I64, I64, I64, ctypes.c_int, ctypes.c_int32, ctypes.POINTER(GemmTile)]
    lib.select_tile.restype = ctypes.c_int
    lib.shuffle_b_bytes.argtypes = [I64, I64, ctypes.c_int]
    lib.shuffle_b_bytes.restype = ctypes.c_size_t
    lib.shuffle_b.argtypes = [P, I64, P, I64, I64, ctypes.c_int, P]
    lib.shuffle_b.restype = ctypes.c_int
    lib.gemm_bf16.argtypes = [P, I64, P, P, I64, I64, I64, I64, ctypes.POINTER(GemmTile), P]
    lib.gemm_bf16.restype = ctypes.c_int
    lib.gemm_fp8_scaled.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64,
                                    ctypes.POINTER(GemmTile), P]
    lib.gemm_fp8_scaled.restype = ctypes.c_int
    lib.select_tile_ws.argtypes = [I64, I64, I64, ctypes.c_int, ctypes.c_int32, ctypes.c_size_t,
                                   ctypes.POINTER(GemmTile)]
    lib.select_tile_ws.restype = ctypes.c_int
    lib.gemm_workspace_bytes.argtypes = [I64, I64, I64, ctypes.c_int, ctypes.POINTER(GemmTile)]
    lib.gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.gemm_bf16_ws.argtypes = [P, I64, P, P, I64, I64, I64, I64, ctypes.POINTER(GemmTile), P,
                                 ctypes.c_size_t, P]
    lib.gemm_bf16_ws.restype = ctypes.c_int
    lib.gemm_fp8_scaled_ws.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64,
                                       ctypes.POINTER(GemmTile), P, ctypes.c_size_t, P]
    lib.gemm_fp8_scaled_ws.restype = ctypes.c_int
    lib.gemm_bf16_ex.argtypes = [P, I64, P, P, I64, I64, I64, I64, ctypes.POINTER(GemmTile),
                                 ctypes.POINTER(GemmEpilogue), P, ctypes.c_size_t, P]
    lib.gemm_bf16_ex.restype = ctypes.c_int
    lib.gemm_fp8_scaled_ex.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64,
                                       ctypes.POINTER(GemmTile), ctypes.POINTER(GemmEpilogue), P,
                                       ctypes.c_size_t, P]
    lib.gemm_fp8_scaled_ex.restype = ctypes.c_int
    lib.shuffle_b_t.argtypes = [P, I64, P, I64, I64, ctypes.c_int, P]
    lib.shuffle_b_t.restype = ctypes.c_int
    lib.transpose_2d.argtypes = [P, I64, P, I64, I64, I64, ctypes.c_int32, P]
    lib.transpose_2d.restype = ctypes.c_int
    lib.gemm_bf16_noalloc.argtypes = [P, I64, P, P, I64, I64, I64, I64, ctypes.POINTER(GemmTile), P]
    lib.gemm_bf16_noalloc.restype = ctypes.c_int
    lib.gemm_plan.argtypes = [I64, I64, I64, ctypes.c_int, ctypes.c_int32, ctypes.c_size_t,
                              ctypes.POINTER(GemmTile), ctypes.POINTER(GemmTile),
                              ctypes.POINTER(I64), ctypes.POINTER(I64)]
    lib.gemm_plan.restype = ctypes.c_int
    lib.gemm_tile_check.argtypes = [ctypes.POINTER(GemmTile), I64, ctypes.c_int]
    lib.gemm_tile_check.restype = ctypes.c_int
    lib.gemm_read_probe.argtypes = [P, ctypes.c_uint64, P, P]
    lib.gemm_read_probe.restype = ctypes.c_int
    lib.gemm_status_string.argtypes = [ctypes.c_int]
    lib.gemm_status_string.restype = ctypes.c_char_p
    return lib


lib = _load_lib()


def gemm_status_string(code: int) -> str:
    return lib.gemm_status_string(int(code)).decode()


def _dtype_code(dtype) -> int:
    if dtype in ("bf16", GEMM_BF16):
        return GEMM_BF16
    if dtype in ("fp8", "e4m3", GEMM_FP8_E4M3):
        return GEMM_FP8_E4M3
    raise ValueError(f"unknown dtype {dtype!r}")


def select_tile(M: int, N: int, K: int, dtype="bf16", num_cus: int = 0,
                workspace_bytes: int = 0) -> Tile:
    """The library's choice; with workspace_bytes > 0, split-K tiles whose
    partials fit are candidates too (select_tile_ws)."""
    t = GemmTile()
    if workspace_bytes:
        st = lib.select_tile_ws(M, N, K, _dtype_code(dtype), num_cus, workspace_bytes, ctypes.byref(t))
    else:
        st = lib.select_tile(M, N, K, _dtype_code(dtype), num_cus, ctypes.byref(t))
    if st != GEMM_OK:
        raise GemmError("select_tile", st)
    return Tile.from_c(t)


def workspace_bytes(M: int, N: int, K: int, dtype, tile: Tile) -> int:
    """Device workspace `tile` needs on M x N x K (0 unless it splits K)."""
    return int(lib.gemm_workspace_bytes(M, N, K, _dtype_code(dtype), ctypes.byref(tile.to_c())))


def plan(M: int, N: int, K: int, dtype="bf16", num_cus: int = 256, workspace_bytes: int = 0):
    """The launches a GEMM with tile=None makes: (first tile, second tile or
    None, columns of the first launch, rows of the first launch).  A second
    launch takes the remaining columns (first columns < N) or the remaining
    rows (first rows < M)."""
    a, b, n, m = GemmTile(), GemmTile(), ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib.gemm_plan(M, N, K, _dtype_code(dtype), num_cus, workspace_bytes, ctypes.byref(a),
                       ctypes.byref(b), ctypes.byref(n), ctypes.byref(m))
    if st != GEMM_OK:
        raise GemmError("gemm_plan", st)
    two = n.value < N or m.value < M
    return Tile.from_c(a), (Tile.from_c(b) if two else None), n.value, m.value


def tile_check(tile: Tile, M: int, dtype="bf16") -> int:
    """Status of forcing `tile` on an M-row GEMM of this dtype (GEMM_OK if a rung)."""
    return int(lib.gemm_tile_check(ctypes.byref(tile.to_c()), M, _dtype_code(dtype)))


def shuffle_b_bytes(N: int, K: int, dtype="bf16") -> int:
    return int(lib.shuffle_b_bytes(N, K, _dtype_code(dtype)))


# ------------------------------------------------------------ torch layer
def _torch():
    import torch
    return torch


def _stream_ptr(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _tensor_dtype_code(t) -> int:
    torch = _torch()
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return GEMM_BF16
    if t.dtype in (torch.uint8, torch.int8, torch.float8_e4m3fn):
        return GEMM_FP8_E4M3
    raise TypeError(f"unsupported element type {t.dtype}")


def _check_rows(name: str, t):
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def shuffle_b(B, dtype=None, out=None):
    """Preshuffle the row-major weight B [N, K] (bf16 or e4m3) into a new (or
    the given) uint8 device tensor of shuffle_b_bytes(N, K) bytes."""
    torch = _torch()
    _check_rows("B", B)
    code = _tensor_dtype_code(B) if dtype is None else _dtype_code(dtype)
    N, K = B.shape
    nbytes = shuffle_b_bytes(N, K, code)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=B.device)
    elif out.numel() * out.element_size() < nbytes:
        raise ValueError("out is too small")
    st = lib.shuffle_b(B.data_ptr(), B.stride(0), out.data_ptr(), N, K, code, _stream_ptr(B))
    if st != GEMM_OK:
        raise GemmError("shuffle_b", st)
    return out


def read_probe(buf, out=None):
    """Read every byte of the contiguous device tensor `buf` once with the
    library's streaming-read probe (a measurement aid: the time floor of a
    kernel that reads the same bytes).  Returns `out`, READ_PROBE_SLOTS
    uint32 values (as int32) whose XOR is the XOR of all 32-bit words of
    buf."""
    torch = _torch()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(READ_PROBE_SLOTS, dtype=torch.int32, device=buf.device)
    elif (not out.is_cuda or out.dtype != torch.int32 or out.numel() < READ_PROBE_SLOTS
          or out.device != buf.device):
        raise ValueError(f"out must be an int32 device tensor of {READ_PROBE_SLOTS} elements "
                         "on buf's device")
    st = lib.gemm_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), _stream_ptr(buf))
    if st != GEMM_OK:
        raise GemmError("gemm_read_probe", st)
    return out


def shuffle_b_t(Bt, dtype=None, out=None):
    """The preshuffled weight of B = Bt^T, from Bt [K, N] (bf16 or e4m3): the
    same bytes as shuffle_b(Bt.T) without materialising the transpose."""
    torch = _torch()
    _check_rows("Bt", Bt)
    code = _tensor_dtype_code(Bt) if dtype is None else _dtype_code(dtype)
    K, N = Bt.shape
    nbytes = shuffle_b_bytes(N, K, code)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=Bt.device)
    elif out.numel() * out.element_size() < nbytes:
        raise ValueError("out is too small")
    st = lib.shuffle_b_t(Bt.data_ptr(), Bt.stride(0), out.data_ptr(), N, K, code, _stream_ptr(Bt))
    if st != GEMM_OK:
        raise GemmError("shuffle_b_t", st)
    return out


def transpose(X, out=None):
    """X^T of a 2-D device tensor of 1- or 2-byte elements, into a new (or the
    given [cols, rows]) tensor of the same dtype."""
    torch = _torch()
    _check_rows("X", X)
    rows, cols = X.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=X.dtype, device=X.device)
    else:
        _check_rows("out", out)
        if tuple(out.shape) != (cols, rows) or out.element_size() != X.element_size():
            raise ValueError("out must be [cols, rows] with X's element size")
    st = lib.transpose_2d(X.data_ptr(), X.stride(0), out.data_ptr(), out.stride(0), rows, cols,
                          X.element_size(), _stream_ptr(X))
    if st != GEMM_OK:
        raise GemmError("transpose_2d", st)
    return out


def grad_input(dY, W, out=None, Ws_t=None, **kw):
    """dX = dY W for a linear layer Y = X W^T (bf16): the GEMM C = A B^T with
    A = dY [M, N_out] and B = W^T, preshuffled by shuffle_b_t(W) (pass it as
    Ws_t to reuse it across calls).  Extra keywords go to gemm_bf16."""
    Bs = shuffle_b_t(W) if Ws_t is None else Ws_t
    return gemm_bf16(dY, Bs, W.shape[1], out=out, **kw)


def grad_weight(dY, X, out=None, **kw):
    """dW = dY^T X for a linear layer Y = X W^T (bf16): A = transpose(dY)
    [N_out, M] and B = X^T, preshuffled by shuffle_b_t(X); the sum runs over
    the M tokens, so M is this GEMM's K and follows its contract (a multiple
    of 16; pad the token dimension with zero rows otherwise).  Extra keywords
    go to gemm_bf16."""
    return gemm_bf16(transpose(dY), shuffle_b_t(X), X.shape[1], out=out, **kw)


def _out(A, N, out):
    torch = _torch()
    M = A.shape[0]
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _check_rows("out", out)
    if tuple(out.shape) != (M, N) or out.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("out must be a bf16 [M, N] view")
    return out


def _check_operands(code: int, A, Bs, N: int, scales=()):
    """Everything the C ABI cannot see behind its plain pointers, checked
    before any launch: A's element type matches the entry point (an e4m3 A
    handed to the bf16 GEMM would have its byte pitch read as a bf16 pitch),
    Bs is a device buffer at least shuffle_b_bytes(N, K) long (the kernels
    size their B bounds from N and K, not from the buffer), and each scale is
    a float32 device tensor with at least one element (a host tensor would
    hand the kernel a host pointer).  Element types are checked first, so
    the checks also run on a machine without a GPU."""
    torch = _torch()
    want = (torch.bfloat16, torch.int16, torch.uint16) if code == GEMM_BF16 else \
        (torch.uint8, torch.int8, torch.float8_e4m3fn)
    fn = "gemm_bf16" if code == GEMM_BF16 else "gemm_fp8_scaled"
    if A.dtype not in want:
        raise ValueError(f"{fn}: A has element type {A.dtype}, expected one of "
                         f"{', '.join(str(d) for d in want)}")
    for name, t in scales:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() < 1:
            raise ValueError(f"{fn}: {name} must be a float32 device tensor with one element")
    if not isinstance(Bs, torch.Tensor):
        raise ValueError(f"{fn}: Bs must be the device tensor shuffle_b returned")
    _check_rows("A", A)
    if not Bs.is_cuda or Bs.device != A.device:
        raise ValueError(f"{fn}: Bs must be a device tensor on A's device")
    if not Bs.is_contiguous():
        raise ValueError(f"{fn}: Bs must be contiguous (the preshuffled layout is dense)")
    need = shuffle_b_bytes(N, A.shape[1], code)
    if Bs.numel() * Bs.element_size() < need:
        raise ValueError(f"{fn}: Bs holds {Bs.numel() * Bs.element_size()} bytes, the "
                         f"preshuffled B of N={N}, K={A.shape[1]} needs {need}")
    for name, t in scales:
        if not t.is_cuda or t.device != A.device:
            raise ValueError(f"{fn}: {name} must be on A's device, not {t.device}")


def _tile_ptr(tile):
    if tile is None:
        return None
    return ctypes.byref(tile.to_c())


def _workspace(A, N: int, K: int, code: int, tile, workspace):
    """(pointer, bytes) of the split-K workspace: the caller's uint8 device
    tensor, or a new one when a forced split-K tile needs it, else none."""
    if workspace is not None:
        if not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if tile is None or tile.kernel == GEMM_KERNEL_SKINNY or (tile.k_split <= 1 and not tile.stream_k):
        return None, 0
    nbytes = workspace_bytes(A.shape[0], N, K, code, tile)
    if nbytes == 0:
        return None, 0
    # torch's caching allocator hands this block out again only to work
    # ordered after ours on the same (current) stream, so it may be freed on
    # return
    ws = _torch().empty(nbytes, dtype=_torch().uint8, device=A.device)
    return ws.data_ptr(), nbytes


def _epilogue(A, N: int, bias, scale_m, scale_n, activation, mul):
    """The gemm_epilogue struct for the given parts, or None when there are none."""
    act = ACTIVATIONS[activation] if not isinstance(activation, int) else activation
    if bias is None and scale_m is None and scale_n is None and mul is None and act == GEMM_ACT_NONE:
        return None
    torch = _torch()
    M = A.shape[0]

    def vec(name, t, n, dtypes):
        if t.dim() != 1 or t.shape[0] != n or t.stride(0) != 1 or not t.is_cuda or t.dtype not in dtypes:
            raise ValueError(f"{name} must be a contiguous device vector of {n} {dtypes[0]}")
        return t.data_ptr()
    e = GemmEpilogue()
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    if bias is not None:
        e.bias = vec("bias", bias, N, bf)
    if scale_m is not None:
        e.scale_m = vec("scale_m", scale_m, M, (torch.float32,))
    if scale_n is not None:
        e.scale_n = vec("scale_n", scale_n, N, (torch.float32,))
    if mul is not None:
        _check_rows("mul", mul)
        if tuple(mul.shape) != (M, N) or mul.dtype not in bf:
            raise ValueError("mul must be a bf16 [M, N] view")
        e.mul = mul.data_ptr()
        e.ld_mul = mul.stride(0)
    e.activation = act
    return e


def gemm_bf16(A, Bs, N: int, out=None, tile: Tile | None = None, workspace=None, *, bias=None,
              scale_m=None, scale_n=None, activation=None, mul=None):
    """C[M, N] = A[M, K] * B[N, K]^T with Bs = shuffle_b(B); returns C (bf16).
    workspace: a uint8 device tensor for split-K (then tile None lets the
    library weigh split-K tiles that fit in it).  Fused epilogue (all
    optional): C = act(acc * scale_m[m] * scale_n[n] + bias[n]) * mul[m, n],
    activation one of ACTIVATIONS; mul may be `out` itself."""
    _check_operands(GEMM_BF16, A, Bs, N)
    C = _out(A, N, out)
    M, K = A.shape
    ws, nbytes = _workspace(A, N, K, GEMM_BF16, tile, workspace)
    epi = _epilogue(A, N, bias, scale_m, scale_n, activation, mul)
    if epi is not None:
        st = lib.gemm_bf16_ex(A.data_ptr(), A.stride(0), Bs.data_ptr(), C.data_ptr(), C.stride(0),
                              M, N, K, _tile_ptr(tile), ctypes.byref(epi), ws, nbytes,
                              _stream_ptr(A))
    elif ws is None:
        st = lib.gemm_bf16(A.data_ptr(), A.stride(0), Bs.data_ptr(), C.data_ptr(), C.stride(0), M,
                           N, K, _tile_ptr(tile), _stream_ptr(A))
    else:
        st = lib.gemm_bf16_ws(A.data_ptr(), A.stride(0), Bs.data_ptr(), C.data_ptr(), C.stride(0),
                              M, N, K, _tile_ptr(tile), ws, nbytes, _stream_ptr(A))
    if st != GEMM_OK:
        raise GemmError("gemm_bf16", st)
    return C


def gemm_fp8_scaled(A, Bs, N: int, scale_a, scale_b, out=None, tile: Tile | None = None,
                    workspace=None, *, bias=None, scale_m=None, scale_n=None, activation=None,
                    mul=None):
    """C = (A * B^T) * scale_a * scale_b for e4m3 A [M, K] and Bs = shuffle_b(B);
    scale_a / scale_b are one-element float32 device tensors.  The fused
    epilogue parts are those of gemm_bf16 (scale_m / scale_n: per-token and
    per-channel fp32 multipliers)."""
    _check_operands(GEMM_FP8_E4M3, A, Bs, N, (("scale_a", scale_a), ("scale_b", scale_b)))
    C = _out(A, N, out)
    M, K = A.shape
    ws, nbytes = _workspace(A, N, K, GEMM_FP8_E4M3, tile, workspace)
    epi = _epilogue(A, N, bias, scale_m, scale_n, activation, mul)
    if epi is not None:
        st = lib.gemm_fp8_scaled_ex(A.data_ptr(), A.stride(0), Bs.data_ptr(), scale_a.data_ptr(),
                                    scale_b.data_ptr(), C.data_ptr(), C.stride(0), M, N, K,
                                    _tile_ptr(tile), ctypes.byref(epi), ws, nbytes,
                                    _stream_ptr(A))
    elif ws is None:
        st = lib.gemm_fp8_scaled(A.data_ptr(), A.stride(0), Bs.data_ptr(), scale_a.data_ptr(),
                                 scale_b.data_ptr(), C.data_ptr(), C.stride(0), M, N, K,
                                 _tile_ptr(tile), _stream_ptr(A))
    else:
        st = lib.gemm_fp8_scaled_ws(A.data_ptr(), A.stride(0), Bs.data_ptr(), scale_a.data_ptr(),
                                    scale_b.data_ptr(), C.data_ptr(), C.stride(0), M, N, K,
                                    _tile_ptr(tile), ws, nbytes, _stream_ptr(A))
    if st != GEMM_OK:
        raise GemmError("gemm_fp8_scaled", st)
    return C


def gemm_bf16_noalloc(A, Bs, N: int, out, tile: Tile | None = None):
    """gemm_bf16 for callers that cannot allocate: split-K partials go to the
    library's fixed scratch array (NOALLOC_SCRATCH_BYTES per GPU), `out` must
    be given, and nothing is allocated.  Calls on one GPU must not overlap."""
    _check_operands(GEMM_BF16, A, Bs, N)
    if out is None:
        raise ValueError("gemm_bf16_noalloc: out must be given (the call allocates nothing)")
    C = _out(A, N, out)
    M, K = A.shape
    st = lib.gemm_bf16_noalloc(A.data_ptr(), A.stride(0), Bs.data_ptr(), C.data_ptr(), C.stride(0),
                               M, N, K, _tile_ptr(tile), _stream_ptr(A))
    if st != GEMM_OK:
        raise GemmError("gemm_bf16_noalloc", st)
    return C
