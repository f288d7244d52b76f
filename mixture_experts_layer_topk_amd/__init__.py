"""Python binding of libmoe (the fused FP8 x FP4 top-k MoE layer for gfx950).

Argument marshalling only: every step runs in the HIP library behind the C ABI
of include/moe.h.  Tensors are torch device tensors; their data pointers and
the current HIP stream are passed through ctypes.  Importing fails loudly when
the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (e.g. a profiling build)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_ETIMEOUT, MOE_ESCRATCH = -5, -6
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
FLAG_NONE, FLAG_NARROW, FLAG_TILED, FLAG_ONE_LAUNCH, FLAG_ONE_KERNEL = 0, 1, 2, 4, 8
FLAG_W13_PREINTERLEAVED, FLAG_W_SCALES_PER_ROW = 16, 32
FLAG_KEEP_INTERMEDIATES, FLAG_DEBUG_SPIN_BOUND = 64, 128
FLAG_WEIGHTS_FP8_BLOCK128 = 256
FLAG_W_STAGED = 512


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("topk", ctypes.c_int32), ("score_fn", ctypes.c_int32),
                ("renorm", ctypes.c_int32)]


class Args(ctypes.Structure):
    _fields_ = [("dims", Dims), ("x", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("w13", ctypes.c_void_p), ("w13_sf", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_sf", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint32),
                ("stage_events", ctypes.c_void_p), ("kernel_events", ctypes.c_void_p)]

NUM_STAGE_EVENTS = 5
STAGES = ("route+quant", "gemm1", "gemm2", "combine")


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("topk_idx", "topk_w", "counts", "offsets", "slot_src", "slot_of",
                 "xq", "xsf", "hq", "hsf", "o", "status", "total")]


# Every symbol include/moe.h declares.
EXPORTS = ("moe_workspace_size", "moe_workspace_layout", "moe_workspace_init", "moe_route",
           "moe_route_noalloc", "moe_quant_act", "moe_pack_weights", "moe_pack_weights_fp8_block128",
           "moe_scales_kmajor", "moe_stage_weights", "moe_forward",
           "moe_check_status", "moe_stream_read", "moe_error_string")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python mixture_experts_layer_topk_amd/build.py`")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.moe_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(sz)]
    lib.moe_workspace_layout.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Layout)]
    lib.moe_workspace_init.argtypes = [vp, sz, vp]
    lib.moe_route.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_route_noalloc.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_quant_act.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.moe_pack_weights.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.moe_pack_weights_fp8_block128.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.moe_scales_kmajor.argtypes = [vp, i64, i32, i32, vp, vp]
    lib.moe_stage_weights.argtypes = [vp, i64, i32, i32, i32, vp, vp]
    lib.moe_forward.argtypes = [ctypes.POINTER(Args), vp]
    lib.moe_check_status.argtypes = [vp, vp]
    lib.moe_stream_read.argtypes = [vp, sz, vp, vp, vp, vp]
    lib.moe_error_string.argtypes = [ctypes.c_int]
    lib.moe_error_string.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("moe_error_string",):
            getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = load_library()


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, _lib.moe_error_string(rc).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dims(T, H, I, E, topk, score_fn=SCORE_SOFTMAX, renorm=True) -> Dims:
    return Dims(int(T), int(H), int(I), int(E), int(topk), int(score_fn), int(bool(renorm)))


def workspace_size(d: Dims) -> int:
    n = ctypes.c_size_t()
    _check(_lib.moe_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def workspace_layout(d: Dims) -> Layout:
    out = Layout()
    _check(_lib.moe_workspace_layout(ctypes.byref(d), ctypes.byref(out)))
    return out


def new_workspace(d: Dims, device="cuda") -> torch.Tensor:
    """Allocate (torch) and zero (library kernel) a workspace for d."""
    ws = torch.empty(workspace_size(d), dtype=torch.uint8, device=device)
    _check(_lib.moe_workspace_init(_ptr(ws), ws.numel(), _stream()))
    return ws


def workspace_init(ws: torch.Tensor):
    _check(_lib.moe_workspace_init(_ptr(ws), ws.numel(), _stream()))


def _bits16(t: torch.Tensor) -> torch.Tensor:
    """BF16 tensors travel as their 16-bit patterns."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def quant_act(x: torch.Tensor):
    """x BF16 [rows, cols] -> (E4M3 codes uint8 [rows, cols], UE8M0 uint8 [rows, cols/32])."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    sf = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _check(_lib.moe_quant_act(_ptr(x), rows, cols, _ptr(q), _ptr(sf), _stream()))
    return q, sf


def pack_weights(w: torch.Tensor):
    """w BF16 [..., rows, cols] -> (packed E2M1 uint8 [..., cols/2], UE8M0 uint8 [..., cols/32])."""
    cols = w.shape[-1]
    rows = w.numel() // cols
    q = torch.empty(w.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=w.device)
    sf = torch.empty(w.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=w.device)
    _check(_lib.moe_pack_weights(_ptr(w), rows, cols, _ptr(q), _ptr(sf), _stream()))
    return q, sf


def pack_weights_fp8_block128(w: torch.Tensor):
    """w BF16 [..., N, K] (N, K multiples of 128) -> (E4M3 codes uint8 [..., N, K], float32
    scales [..., N/128, K/128]): one scale per 128 x 128 block."""
    cols = w.shape[-1]
    rows = w.numel() // cols
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    sf = torch.empty(w.shape[:-2] + (w.shape[-2] // 128, cols // 128), dtype=torch.float32, device=w.device)
    _check(_lib.moe_pack_weights_fp8_block128(_ptr(w), rows, cols, _ptr(q), _ptr(sf), _stream()))
    return q, sf


def scales_kmajor(sf: torch.Tensor, cols: int) -> torch.Tensor:
    """Per-row scales [..., rows, cols/32] -> K-step major [..., cols/128, rows, 4]."""
    rows = sf.shape[-2]
    mats = sf.numel() // (rows * (cols // 32))
    out = torch.empty(sf.shape[:-2] + (cols // 128, rows, 4), dtype=torch.uint8, device=sf.device)
    _check(_lib.moe_scales_kmajor(_ptr(sf), mats, rows, cols, _ptr(out), _stream()))
    return out


def stage_weights(w: torch.Tensor, is_w13: bool) -> torch.Tensor:
    """Packed FP4 codes [..., rows, K/2] in canonical row order (W13: gate rows, then
    up rows) -> the staged layout moe_forward reads with FLAG_W_STAGED (same size)."""
    rows, cols = w.shape[-2], 2 * w.shape[-1]
    mats = w.numel() // (rows * (cols // 2))
    out = torch.empty_like(w)
    _check(_lib.moe_stage_weights(_ptr(w), mats, rows, cols, 1 if is_w13 else 0, _ptr(out), _stream()))
    return out


def prepare_weights(w13: torch.Tensor, w2: torch.Tensor):
    """BF16 expert weights W13 [E, 2I, H] and W2 [E, H, I] -> the four tensors
    moe_forward takes (packed FP4 codes, K-step-major UE8M0 scales)."""
    q13, s13 = pack_weights(w13)
    q2, s2 = pack_weights(w2)
    return q13, scales_kmajor(s13, w13.shape[-1]), q2, scales_kmajor(s2, w2.shape[-1])


def route(d: Dims, logits: torch.Tensor, ws: torch.Tensor):
    """Top-k routing + bucketisation.  Returns a dict of device tensors."""
    T, k, E = d.T, d.topk, d.E
    dev = logits.device
    out = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
               topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
               counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               slot_src=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
               slot_of=torch.empty((T, k), dtype=torch.int32, device=dev))
    _check(_lib.moe_route(ctypes.byref(d), _ptr(logits), _ptr(out["topk_idx"]), _ptr(out["topk_w"]),
                          _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["slot_src"]),
                          _ptr(out["slot_of"]), _ptr(ws), ws.numel(), _stream()))
    return out


def route_noalloc(d: Dims, logits: torch.Tensor):
    """route() without a workspace (moe_route_noalloc: the library's static scratch)."""
    T, k, E = d.T, d.topk, d.E
    dev = logits.device
    out = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
               topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
               counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               slot_src=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
               slot_of=torch.empty((T, k), dtype=torch.int32, device=dev))
    _check(_lib.moe_route_noalloc(ctypes.byref(d), _ptr(logits), _ptr(out["topk_idx"]),
                                  _ptr(out["topk_w"]), _ptr(out["counts"]), _ptr(out["offsets"]),
                                  _ptr(out["slot_src"]), _ptr(out["slot_of"]), _stream()))
    return out


def forward_args(d: Dims, x, w13, w13_sf, w2, w2_sf, y, ws, logits=None, topk_idx=None,
                 topk_w=None, flags=0, stage_events=None, kernel_events=None) -> Args:
    """stage_events: None or a ctypes array of NUM_STAGE_EVENTS hipEvent_t handles;
    kernel_events: None or a ctypes array of 2 handles that take the GEMM1 kernel's
    start and end times."""
    ev = ctypes.cast(stage_events, ctypes.c_void_p) if stage_events is not None else None
    kev = ctypes.cast(kernel_events, ctypes.c_void_p) if kernel_events is not None else None
    return Args(d, _ptr(x), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(w13), _ptr(w13_sf),
                _ptr(w2), _ptr(w2_sf), _ptr(y), _ptr(ws), ws.numel(), flags, ev, kev)


def forward_raw(args: Args, stream=None):
    """Enqueue the layer for prepared arguments (no per-call Python marshalling)."""
    _check(_lib.moe_forward(ctypes.byref(args), stream if stream is not None else _stream()))


def forward(d: Dims, x, w13, w13_sf, w2, w2_sf, ws, logits=None, topk_idx=None, topk_w=None,
            y=None, flags=FLAG_NONE):
    """The whole layer; returns y (BF16 [T, H]).  flags: FLAG_NARROW / FLAG_TILED force
    the GEMM kernel family (default: chosen from the rows per expert); FLAG_ONE_LAUNCH
    runs the tiled GEMMs (or, with FLAG_NARROW, the narrow ones) as one launch with ready
    counters; FLAG_ONE_KERNEL runs the whole layer as one launch (T * topk <= 1024)."""
    if y is None:
        y = torch.empty((d.T, d.H), dtype=torch.bfloat16, device=x.device)
    forward_raw(forward_args(d, x, w13, w13_sf, w2, w2_sf, y, ws, logits, topk_idx, topk_w,
                             flags=flags))
    return y


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None, start=None, stop=None):
    """Read src's bytes once (moe_stream_read: the HBM read ceiling of a footprint);
    start/stop: None or hipEvent_t handles the launch carries."""
    _check(_lib.moe_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), start, stop,
                                stream if stream is not None else _stream()))


def check_status(ws: torch.Tensor) -> int:
    """Synchronise the current stream and return MOE_OK, or MOE_ETIMEOUT when a
    bounded wait of the last forward on ws gave up (errors raise)."""
    rc = _lib.moe_check_status(_ptr(ws), _stream())
    if rc not in (MOE_OK, MOE_ETIMEOUT):
        _check(rc)
    return rc


def intermediates(d: Dims, ws: torch.Tensor, block_fp8: bool = False):
    """Views of the workspace intermediates left by the last forward with ws
    (block_fp8: the forward ran with FLAG_WEIGHTS_FP8_BLOCK128, whose xsf and hsf are
    float32, one per row per 128 elements)."""
    L = workspace_layout(d)
    T, k, E, H, I = d.T, d.topk, d.E, d.H, d.I
    R = T * k

    def view(off, n, dtype, shape):
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype).view(shape)

    if block_fp8:
        xsf = view(L.xsf, T * H // 128, torch.float32, (H // 128, T)).t()
        hsf = view(L.hsf, R * I // 128, torch.float32, (I // 128, R)).t()
    else:
        # scales are K-step major in the workspace; shown here per row
        xsf = view(L.xsf, T * H // 32, torch.uint8, (H // 128, T, 4)).permute(1, 0, 2).reshape(T, H // 32)
        hsf = view(L.hsf, R * I // 32, torch.uint8, (I // 128, R, 4)).permute(1, 0, 2).reshape(R, I // 32)
    return dict(
        topk_idx=view(L.topk_idx, R, torch.int32, (T, k)),
        topk_w=view(L.topk_w, R, torch.float32, (T, k)),
        counts=view(L.counts, E, torch.int32, (E,)),
        offsets=view(L.offsets, E + 1, torch.int32, (E + 1,)),
        slot_src=view(L.slot_src, R, torch.int32, (R,)),
        slot_of=view(L.slot_of, R, torch.int32, (T, k)),
        xq=view(L.xq, T * H, torch.uint8, (T, H)),
        xsf=xsf,
        hq=view(L.hq, R * I, torch.uint8, (R, I)),
        hsf=hsf,
        o=view(L.o, R * H, torch.int16, (R, H)),
        status=view(L.status, 1, torch.int32, (1,)),
    )
