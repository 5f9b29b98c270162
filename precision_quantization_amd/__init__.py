"""MI355X (gfx950) quantization casts: a thin Python binding of libqcast.so.

Each ``qcast_*`` function has the name of the C entry point it calls and does
argument marshalling only: it checks that tensors are on one GPU and
contiguous, allocates outputs that were not given, and passes raw pointers
and torch's current stream. Every step of a cast runs in the HIP kernels; a
missing library raises ``QcastError``.

Outputs: E4M3 codes as ``torch.float8_e4m3fn`` and E5M2 codes as
``torch.float8_e5m2`` (one byte per code), E2M1 codes as ``torch.uint8`` with
two codes per byte (low nibble = even column), E5M6 codes as ``torch.uint8``
with two 12-bit codes per three bytes (a little-endian bit stream), scales as
``torch.float32``. Every cast takes every format; codes are packed along the
rows of its output (``code_shape``): columns for the per-token, SwiGLU,
per-block and per-channel casts, tokens for the transposed per-channel ones.

``per_token_cast(x, fmt='e4m3', num_per_channels=128) -> (out, out_sf)``
mirrors the call shown in the quick start of the page
"DeepSeek开源TileKernels：用Python写的GPU算子逼近硬件性能上限".
"""
import torch

from ._lib import (FMT_E2M1, FMT_E4M3, FMT_E5M2, FMT_E5M6, OUT_BF16, OUT_F32, SF_COL_MAJOR,
                   SF_PACKED_UE8M0, SF_ROUND_POW2, QcastError, check, fmt_id, load)

__all__ = ["qcast_per_token", "qcast_e2m1", "qcast_swiglu_per_token", "qcast_per_block",
           "qcast_per_channel_T", "qcast_cast_back", "qcast_per_token_sf",
           "qcast_swiglu_per_token_sf", "qcast_swiglu_per_token_ex",
           "qcast_swiglu_backward_per_token", "qcast_swiglu_per_channel_T", "qcast_per_channel",
           "qcast_swiglu_per_token_noalloc", "qcast_per_block_sf", "qcast_per_channel_sf",
           "qcast_per_channel_T_sf", "qcast_swiglu_per_channel_T_sf",
           "qcast_swiglu_backward_per_token_sf", "sf_layout_shape", "SF_ROUND_POW2", "SF_COL_MAJOR",
           "SF_PACKED_UE8M0", "qcast_abi_version", "qcast_set_num_cus", "qcast_bench_copy",
           "qcast_bench_check_scale", "qcast_bench_time_next",
           "qcast_bench_per_channel_T_traffic",
           "per_token_cast",
           "QcastError", "FMT_E4M3", "FMT_E2M1", "FMT_E5M2", "FMT_E5M6", "code_shape"]


def _bf16_input(x, name):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise QcastError(1, f"{name} must be a CUDA (HIP) tensor")
    if x.dtype != torch.bfloat16:
        raise QcastError(2, f"{name} must be bfloat16, got {x.dtype}")
    if x.dim() != 2 or not x.is_contiguous():
        raise QcastError(2, f"{name} must be a contiguous 2-D tensor")
    return x


def _gate_up(h, name="h"):
    """A SwiGLU input ``[rows, 2*cols]`` (gate | up): (h, rows, cols). The
    width must be even, or the C ABI would walk h with a row stride one
    element short."""
    if isinstance(h, torch.Tensor) and h.dim() == 2 and h.shape[1] % 2:
        raise QcastError(2, f"{name} must have an even number of columns (gate | up), "
                            f"got {h.shape[1]}")
    h = _bf16_input(h, name)
    rows, two_n = h.shape
    return h, rows, two_n // 2


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or \
            not t.is_contiguous():
        raise QcastError(2, f"{name} must be a contiguous {dtype} tensor of shape {shape} "
                            f"on {device}")
    return t


def _stream(device, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(device).cuda_stream


def _row_weight(row_weight, rows, device):
    if row_weight is None:
        return None
    if not isinstance(row_weight, torch.Tensor) or row_weight.dtype != torch.float32 or \
            tuple(row_weight.shape) != (rows,) or row_weight.device != device or \
            not row_weight.is_contiguous():
        raise QcastError(2, "row_weight must be a contiguous float32 [rows] tensor on h's device")
    return row_weight.data_ptr()


def _counter(clamp_count, device):
    """Device int64 [1] tensor the clamp count is added to (or None)."""
    if clamp_count is None:
        return None
    if not isinstance(clamp_count, torch.Tensor) or clamp_count.dtype != torch.int64 or \
            clamp_count.numel() != 1 or clamp_count.device != device:
        raise QcastError(2, "clamp_count must be a one-element int64 tensor on h's device")
    return clamp_count.data_ptr()


COUNT_WS_BYTES = 8192           # QCAST_COUNT_WS_BYTES
_count_ws_cache = {}


def _count_ws(count_workspace, clamp_count, device, stream_handle):
    """Device pointer of the clamp-count workspace (QCAST_COUNT_WS_BYTES,
    zero between calls): the caller's tensor; none when ``count_workspace``
    is False, when nothing is counted, or (for the default None) under graph
    capture, since a graph may be replayed on any stream; else, for None,
    one int64 tensor kept per device and stream (each call leaves it
    zeroed, and calls on one stream are ordered).

    The first counting call on a (device, stream) allocates that tensor
    (8 KB) and zeroes it with a fill kernel enqueued on the same stream,
    ahead of the cast: nothing waits on the host. Callers that must not
    allocate inside the call pass their own ``count_workspace``, or
    ``False`` (the capped grid, no workspace)."""
    if clamp_count is None or count_workspace is False:
        return None
    if count_workspace is None:
        if torch.cuda.is_current_stream_capturing():
            return None     # a graph may replay on any stream: no shared workspace
        key = (device, stream_handle)
        ws = _count_ws_cache.get(key)
        if ws is None:
            # allocated for, and zeroed on, the stream the cast runs on
            if torch.cuda.current_stream(device).cuda_stream == stream_handle:
                ws = torch.zeros(COUNT_WS_BYTES // 8, dtype=torch.int64, device=device)
            else:
                with torch.cuda.stream(torch.cuda.ExternalStream(stream_handle, device=device)):
                    ws = torch.zeros(COUNT_WS_BYTES // 8, dtype=torch.int64, device=device)
            _count_ws_cache[key] = ws
        return ws.data_ptr()
    if not isinstance(count_workspace, torch.Tensor) or count_workspace.device != device or \
            not count_workspace.is_contiguous() or \
            count_workspace.numel() * count_workspace.element_size() < COUNT_WS_BYTES:
        raise QcastError(2, f"count_workspace must be a contiguous tensor of at least "
                            f"{COUNT_WS_BYTES} bytes on h's device")
    return count_workspace.data_ptr()


def code_shape(fmt, rows, cols):
    """Shape of the uint8/float8 code tensor of a per-token cast."""
    f = fmt_id(fmt)
    if f == FMT_E2M1:
        return (rows, cols // 2)
    if f == FMT_E5M6:
        return (rows, cols // 2 * 3)
    return (rows, cols)


def _code_dtype(f):
    return {FMT_E4M3: torch.float8_e4m3fn, FMT_E5M2: torch.float8_e5m2}.get(f, torch.uint8)


def qcast_per_token(x, fmt="e4m3", group=128, clamp_min=0.0, out=None, out_sf=None,
                    stream=None):
    """Per-token cast of bf16 ``x [rows, cols]``; see include/qcast.h."""
    f = fmt_id(fmt)
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    qshape = code_shape(f, rows, cols)
    out = _out(out, qshape, _code_dtype(f), x.device, "out")
    out_sf = _out(out_sf, (rows, cols // group if group > 0 else 0), torch.float32, x.device,
                  "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_per_token(x.data_ptr(), rows, cols, f, group, clamp_min,
                                     out.data_ptr(), out_sf.data_ptr(), _stream(x.device, stream)),
              "qcast_per_token")
    return out, out_sf


def sf_layout_shape(rows, cols, group, sf_flags):
    """(shape, dtype) of the scale tensor of a layout (include/qcast.h)."""
    groups = cols // group
    rows_pad = (rows + 3) // 4 * 4
    if sf_flags & SF_PACKED_UE8M0:
        shape = (groups // 4, rows_pad) if sf_flags & SF_COL_MAJOR else (rows, groups // 4)
        return shape, torch.int32
    shape = (groups, rows_pad) if sf_flags & SF_COL_MAJOR else (rows, groups)
    return shape, torch.float32


def qcast_per_token_sf(x, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0, out=None,
                       out_sf=None, stream=None):
    """qcast_per_token with a scale-factor layout; out_sf is float32 or int32
    (packed UE8M0 words) of ``sf_layout_shape``."""
    f = fmt_id(fmt)
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    qshape = code_shape(f, rows, cols)
    out = _out(out, qshape, _code_dtype(f), x.device, "out")
    shape, dt = sf_layout_shape(rows, cols, group if group > 0 else 1, sf_flags)
    out_sf = _out(out_sf, shape, dt, x.device, "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_per_token_sf(x.data_ptr(), rows, cols, f, group, clamp_min, sf_flags,
                                        out.data_ptr(), out_sf.data_ptr(),
                                        _stream(x.device, stream)), "qcast_per_token_sf")
    return out, out_sf


def qcast_swiglu_per_token_sf(h, row_weight=None, fmt="e4m3", group=128, clamp_min=0.0,
                              sf_flags=0, out=None, out_sf=None, stream=None):
    """qcast_swiglu_per_token with a scale-factor layout."""
    f = fmt_id(fmt)
    h, rows, cols = _gate_up(h)
    wptr = None
    if row_weight is not None:
        if row_weight.dtype != torch.float32 or tuple(row_weight.shape) != (rows,) or \
                row_weight.device != h.device or not row_weight.is_contiguous():
            raise QcastError(2, "row_weight must be a contiguous float32 [rows] tensor on h's device")
        wptr = row_weight.data_ptr()
    out = _out(out, code_shape(f, rows, cols), _code_dtype(f), h.device, "out")
    shape, dt = sf_layout_shape(rows, cols, group if group > 0 else 1, sf_flags)
    out_sf = _out(out_sf, shape, dt, h.device, "out_sf")
    with torch.cuda.device(h.device):
        check(load().qcast_swiglu_per_token_sf(h.data_ptr(), rows, cols, wptr, f, group, clamp_min,
                                               sf_flags, out.data_ptr(), out_sf.data_ptr(),
                                               _stream(h.device, stream)),
              "qcast_swiglu_per_token_sf")
    return out, out_sf


def qcast_swiglu_per_token_ex(h, row_weight=None, fmt="e4m3", group=128, clamp_min=0.0,
                              sf_flags=0, swiglu_clamp=0.0, clamp_count=None, out=None,
                              out_sf=None, stream=None, count_workspace=None):
    """SwiGLU with the optional clamp (gate <= c, up in [-c, c]) fused with the
    per-token cast. ``clamp_count``: an int64 [1] device tensor to which the
    number of clamped values is added, or None. ``count_workspace``: see
    ``_count_ws`` (the default keeps one per device and stream)."""
    f = fmt_id(fmt)
    h, rows, cols = _gate_up(h)
    wptr = _row_weight(row_weight, rows, h.device)
    cptr = _counter(clamp_count, h.device)
    out = _out(out, code_shape(f, rows, cols), _code_dtype(f), h.device, "out")
    shape, dt = sf_layout_shape(rows, cols, group if group > 0 else 1, sf_flags)
    out_sf = _out(out_sf, shape, dt, h.device, "out_sf")
    with torch.cuda.device(h.device):
        sh = _stream(h.device, stream)
        wsptr = _count_ws(count_workspace, clamp_count, h.device, sh)
        check(load().qcast_swiglu_per_token_ex(h.data_ptr(), rows, cols, wptr, f, group, clamp_min,
                                               sf_flags, swiglu_clamp, out.data_ptr(),
                                               out_sf.data_ptr(), cptr, wsptr, sh),
              "qcast_swiglu_per_token_ex")
    return out, out_sf


def qcast_swiglu_per_token_noalloc(h, row_weight=None, fmt="e4m3", group=128, clamp_min=0.0,
                                   sf_flags=0, swiglu_clamp=0.0, clamp_count=None, out=None,
                                   out_sf=None, stream=None):
    """qcast_swiglu_per_token_ex for callers that cannot allocate: the clamp
    count goes through the library's own device array (include/qcast.h), so
    with ``out`` and ``out_sf`` given nothing is allocated; calls that may
    overlap on one GPU race on that array."""
    f = fmt_id(fmt)
    h, rows, cols = _gate_up(h)
    wptr = _row_weight(row_weight, rows, h.device)
    cptr = _counter(clamp_count, h.device)
    out = _out(out, code_shape(f, rows, cols), _code_dtype(f), h.device, "out")
    shape, dt = sf_layout_shape(rows, cols, group if group > 0 else 1, sf_flags)
    out_sf = _out(out_sf, shape, dt, h.device, "out_sf")
    with torch.cuda.device(h.device):
        check(load().qcast_swiglu_per_token_noalloc(h.data_ptr(), rows, cols, wptr, f, group,
                                                    clamp_min, sf_flags, swiglu_clamp,
                                                    out.data_ptr(), out_sf.data_ptr(), cptr,
                                                    _stream(h.device, stream)),
              "qcast_swiglu_per_token_noalloc")
    return out, out_sf


def qcast_swiglu_backward_per_token(h, dv, row_weight=None, fmt="e4m3", group=128,
                                    clamp_min=0.0, swiglu_clamp=0.0, out=None, out_sf=None,
                                    stream=None):
    """SwiGLU backward fused with the per-token cast of ``[dgate | dup]``:
    ``out [rows, 2*cols]``, ``out_sf [rows, 2*cols/group]``."""
    f = fmt_id(fmt)
    h, rows, cols = _gate_up(h)
    two_n = 2 * cols
    dv = _bf16_input(dv, "dv")
    if tuple(dv.shape) != (rows, cols) or dv.device != h.device:
        raise QcastError(2, f"dv must be [{rows}, {cols}] on h's device")
    wptr = _row_weight(row_weight, rows, h.device)
    out = _out(out, code_shape(f, rows, two_n), _code_dtype(f), h.device, "out")
    out_sf = _out(out_sf, (rows, two_n // group if group > 0 else 0), torch.float32, h.device,
                  "out_sf")
    with torch.cuda.device(h.device):
        check(load().qcast_swiglu_backward_per_token(h.data_ptr(), dv.data_ptr(), rows, cols,
                                                     wptr, f, group, clamp_min, swiglu_clamp,
                                                     out.data_ptr(), out_sf.data_ptr(),
                                                     _stream(h.device, stream)),
              "qcast_swiglu_backward_per_token")
    return out, out_sf


def qcast_swiglu_backward_per_token_sf(h, dv, row_weight=None, fmt="e4m3", group=128,
                                       clamp_min=0.0, sf_flags=0, swiglu_clamp=0.0, out=None,
                                       out_sf=None, stream=None):
    """qcast_swiglu_backward_per_token with a scale-factor layout over the
    rows ``[dgate | dup]`` of 2*cols values (``sf_layout_shape(rows, 2*cols,
    group, sf_flags)``)."""
    f = fmt_id(fmt)
    h, rows, cols = _gate_up(h)
    two_n = 2 * cols
    dv = _bf16_input(dv, "dv")
    if tuple(dv.shape) != (rows, cols) or dv.device != h.device:
        raise QcastError(2, f"dv must be [{rows}, {cols}] on h's device")
    wptr = _row_weight(row_weight, rows, h.device)
    out = _out(out, code_shape(f, rows, two_n), _code_dtype(f), h.device, "out")
    shape, dt = sf_layout_shape(rows, two_n, group if group > 0 else 1, sf_flags)
    out_sf = _out(out_sf, shape, dt, h.device, "out_sf")
    with torch.cuda.device(h.device):
        check(load().qcast_swiglu_backward_per_token_sf(h.data_ptr(), dv.data_ptr(), rows, cols,
                                                        wptr, f, group, clamp_min, sf_flags,
                                                        swiglu_clamp, out.data_ptr(),
                                                        out_sf.data_ptr(),
                                                        _stream(h.device, stream)),
              "qcast_swiglu_backward_per_token_sf")
    return out, out_sf


def qcast_swiglu_per_channel_T_sf(h, row_weight=None, fmt="e4m3", group=128, clamp_min=0.0,
                                  sf_flags=0, swiglu_clamp=0.0, clamp_count=None, out=None,
                                  out_sf=None, stream=None, count_workspace=None):
    """qcast_swiglu_per_channel_T with a scale-factor layout: the per-token
    layouts of the transposed values (``sf_layout_shape(cols, rows, group,
    sf_flags)``: rows are the channels)."""
    f = fmt_id(fmt)
    h, rows, cols = _gate_up(h)
    wptr = _row_weight(row_weight, rows, h.device)
    cptr = _counter(clamp_count, h.device)
    out = _out(out, code_shape(f, cols, rows), _code_dtype(f), h.device, "out")
    shape, dt = sf_layout_shape(cols, rows, group if group > 0 else 1, sf_flags)
    out_sf = _out(out_sf, shape, dt, h.device, "out_sf")
    with torch.cuda.device(h.device):
        sh = _stream(h.device, stream)
        wsptr = _count_ws(count_workspace, clamp_count, h.device, sh)
        check(load().qcast_swiglu_per_channel_T_sf(h.data_ptr(), rows, cols, wptr, f, group,
                                                   clamp_min, sf_flags, swiglu_clamp,
                                                   out.data_ptr(), out_sf.data_ptr(), cptr,
                                                   wsptr, sh),
              "qcast_swiglu_per_channel_T_sf")
    return out, out_sf


def qcast_swiglu_per_channel_T(h, row_weight=None, fmt="e4m3", group=128, clamp_min=0.0,
                               swiglu_clamp=0.0, clamp_count=None, out=None, out_sf=None,
                               stream=None, count_workspace=None):
    """SwiGLU fused with the per-channel cast written transposed:
    ``out [cols, rows]``, ``out_sf [cols, rows/group]``; ``clamp_count`` and
    ``count_workspace`` as in qcast_swiglu_per_token_ex."""
    f = fmt_id(fmt)
    h, rows, cols = _gate_up(h)
    wptr = _row_weight(row_weight, rows, h.device)
    cptr = _counter(clamp_count, h.device)
    out = _out(out, code_shape(f, cols, rows), _code_dtype(f), h.device, "out")
    out_sf = _out(out_sf, (cols, rows // group if group > 0 else 0), torch.float32, h.device,
                  "out_sf")
    with torch.cuda.device(h.device):
        sh = _stream(h.device, stream)
        wsptr = _count_ws(count_workspace, clamp_count, h.device, sh)
        check(load().qcast_swiglu_per_channel_T(h.data_ptr(), rows, cols, wptr, f, group,
                                                clamp_min, swiglu_clamp, out.data_ptr(),
                                                out_sf.data_ptr(), cptr, wsptr, sh),
              "qcast_swiglu_per_channel_T")
    return out, out_sf


def qcast_per_channel(x, fmt="e4m3", group=128, clamp_min=0.0, out=None, out_sf=None,
                      stream=None):
    """Per-channel cast in the input layout: ``out [tokens, channels]``,
    ``out_sf [tokens/group, channels]``."""
    f = fmt_id(fmt)
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    out = _out(out, code_shape(f, rows, cols), _code_dtype(f), x.device, "out")
    out_sf = _out(out_sf, (rows // group if group > 0 else 0, cols), torch.float32, x.device,
                  "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_per_channel(x.data_ptr(), rows, cols, f, group, clamp_min,
                                       out.data_ptr(), out_sf.data_ptr(),
                                       _stream(x.device, stream)), "qcast_per_channel")
    return out, out_sf


def qcast_e2m1(x, group=32, clamp_min=0.0, out=None, out_sf=None, stream=None):
    """Per-token cast to packed E2M1: ``out [rows, cols/2]`` uint8."""
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    out = _out(out, (rows, cols // 2), torch.uint8, x.device, "out")
    out_sf = _out(out_sf, (rows, cols // group if group > 0 else 0), torch.float32, x.device,
                  "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_e2m1(x.data_ptr(), rows, cols, group, clamp_min, out.data_ptr(),
                                out_sf.data_ptr(), _stream(x.device, stream)), "qcast_e2m1")
    return out, out_sf


def qcast_swiglu_per_token(h, row_weight=None, fmt="e4m3", group=128, clamp_min=0.0, out=None,
                           out_sf=None, stream=None):
    """SwiGLU of ``h [rows, 2N]`` (gate | up) times ``row_weight [rows]`` (fp32
    or None), cast per token: ``out [rows, N]``, ``out_sf [rows, N/group]``."""
    f = fmt_id(fmt)
    h, rows, cols = _gate_up(h)
    wptr = None
    if row_weight is not None:
        if row_weight.dtype != torch.float32 or tuple(row_weight.shape) != (rows,) or \
                row_weight.device != h.device or not row_weight.is_contiguous():
            raise QcastError(2, "row_weight must be a contiguous float32 [rows] tensor on h's device")
        wptr = row_weight.data_ptr()
    out = _out(out, code_shape(f, rows, cols), _code_dtype(f), h.device, "out")
    out_sf = _out(out_sf, (rows, cols // group if group > 0 else 0), torch.float32, h.device,
                  "out_sf")
    with torch.cuda.device(h.device):
        check(load().qcast_swiglu_per_token(h.data_ptr(), rows, cols, wptr, f, group, clamp_min,
                                            out.data_ptr(), out_sf.data_ptr(),
                                            _stream(h.device, stream)), "qcast_swiglu_per_token")
    return out, out_sf


def qcast_per_block(x, fmt="e4m3", block=128, clamp_min=0.0, out=None, out_sf=None,
                    stream=None):
    """One scale per ``block x block`` tile: ``out [rows, cols]``,
    ``out_sf [rows/block, cols/block]``."""
    f = fmt_id(fmt)
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    out = _out(out, code_shape(f, rows, cols), _code_dtype(f), x.device, "out")
    out_sf = _out(out_sf, (rows // block if block > 0 else 0, cols // block if block > 0 else 0),
                  torch.float32, x.device, "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_per_block(x.data_ptr(), rows, cols, f, block, clamp_min, out.data_ptr(),
                                     out_sf.data_ptr(), _stream(x.device, stream)),
              "qcast_per_block")
    return out, out_sf


def qcast_per_channel_T(x, fmt="e4m3", group=128, clamp_min=0.0, out=None, out_sf=None,
                        stream=None):
    """Per-channel cast of ``x [tokens, channels]`` written transposed:
    ``out [channels, tokens]``, ``out_sf [channels, tokens/group]``."""
    f = fmt_id(fmt)
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    out = _out(out, code_shape(f, cols, rows), _code_dtype(f), x.device, "out")
    out_sf = _out(out_sf, (cols, rows // group if group > 0 else 0), torch.float32, x.device,
                  "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_per_channel_T(x.data_ptr(), rows, cols, f, group, clamp_min,
                                         out.data_ptr(), out_sf.data_ptr(),
                                         _stream(x.device, stream)), "qcast_per_channel_T")
    return out, out_sf


def qcast_per_block_sf(x, fmt="e4m3", block=128, clamp_min=0.0, sf_flags=0, out=None,
                       out_sf=None, stream=None):
    """qcast_per_block with round_sf (``sf_flags`` 0 or SF_ROUND_POW2);
    ``out_sf [rows/block, cols/block]`` float32."""
    f = fmt_id(fmt)
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    out = _out(out, code_shape(f, rows, cols), _code_dtype(f), x.device, "out")
    out_sf = _out(out_sf, (rows // block if block > 0 else 0, cols // block if block > 0 else 0),
                  torch.float32, x.device, "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_per_block_sf(x.data_ptr(), rows, cols, f, block, clamp_min, sf_flags,
                                        out.data_ptr(), out_sf.data_ptr(),
                                        _stream(x.device, stream)), "qcast_per_block_sf")
    return out, out_sf


def qcast_per_channel_sf(x, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0, out=None,
                         out_sf=None, stream=None):
    """qcast_per_channel with round_sf (``sf_flags`` 0 or SF_ROUND_POW2)."""
    f = fmt_id(fmt)
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    out = _out(out, code_shape(f, rows, cols), _code_dtype(f), x.device, "out")
    out_sf = _out(out_sf, (rows // group if group > 0 else 0, cols), torch.float32, x.device,
                  "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_per_channel_sf(x.data_ptr(), rows, cols, f, group, clamp_min, sf_flags,
                                          out.data_ptr(), out_sf.data_ptr(),
                                          _stream(x.device, stream)), "qcast_per_channel_sf")
    return out, out_sf


def qcast_per_channel_T_sf(x, fmt="e4m3", group=128, clamp_min=0.0, sf_flags=0, out=None,
                           out_sf=None, stream=None):
    """qcast_per_channel_T with a scale-factor layout: the per-token layouts
    of ``x^T`` (``sf_layout_shape(channels, tokens, group, sf_flags)``)."""
    f = fmt_id(fmt)
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    out = _out(out, code_shape(f, cols, rows), _code_dtype(f), x.device, "out")
    shape, dt = sf_layout_shape(cols, rows, group if group > 0 else 1, sf_flags)
    out_sf = _out(out_sf, shape, dt, x.device, "out_sf")
    with torch.cuda.device(x.device):
        check(load().qcast_per_channel_T_sf(x.data_ptr(), rows, cols, f, group, clamp_min,
                                            sf_flags, out.data_ptr(), out_sf.data_ptr(),
                                            _stream(x.device, stream)), "qcast_per_channel_T_sf")
    return out, out_sf


def qcast_cast_back(q, sf, fmt="e4m3", group=128, out_dtype=torch.bfloat16, out=None,
                    stream=None):
    """Dequantize per-token codes ``q`` with scales ``sf [rows, cols/group]``
    to ``out [rows, cols]`` (bf16 or fp32): decode(q) * sf."""
    f = fmt_id(fmt)
    if isinstance(q, torch.Tensor) and q.dim() == 2 and f == FMT_E5M6 and q.shape[1] % 3:
        raise QcastError(2, f"E5M6 codes take three bytes per pair of columns: q's width "
                            f"{q.shape[1]} is not a multiple of 3")
    if not (isinstance(q, torch.Tensor) and q.is_cuda and q.dim() == 2 and q.is_contiguous()):
        raise QcastError(2, "q must be a contiguous 2-D CUDA tensor")
    if q.element_size() != 1:
        raise QcastError(2, "q must hold one byte per element")
    rows = q.shape[0]
    cols = {FMT_E2M1: q.shape[1] * 2, FMT_E5M6: q.shape[1] // 3 * 2}.get(f, q.shape[1])
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise QcastError(4, "out_dtype must be torch.bfloat16 or torch.float32")
    if sf.dtype != torch.float32 or tuple(sf.shape) != (rows, cols // group if group > 0 else 0) \
            or sf.device != q.device or not sf.is_contiguous():
        raise QcastError(2, "sf must be a contiguous float32 [rows, cols/group] tensor on q's device")
    out = _out(out, (rows, cols), out_dtype, q.device, "out")
    od = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    with torch.cuda.device(q.device):
        check(load().qcast_cast_back(q.data_ptr(), sf.data_ptr(), rows, cols, f, group, od,
                                     out.data_ptr(), _stream(q.device, stream)), "qcast_cast_back")
    return out


def qcast_abi_version():
    return load().qcast_abi_version()


def qcast_set_num_cus(n):
    load().qcast_set_num_cus(int(n))


def qcast_bench_copy(src, dst, stream=None):
    """Measurement helper (include/qcast_bench.h): copy src's bytes to dst."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise QcastError(2, "src and dst must be contiguous CUDA tensors")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or src.device != dst.device:
        raise QcastError(2, "src and dst must have the same size on one device")
    with torch.cuda.device(src.device):
        check(load().qcast_bench_copy(src.data_ptr(), dst.data_ptr(), n, _stream(src.device, stream)),
              "qcast_bench_copy")


def qcast_bench_per_channel_T_traffic(x, out=None, stream=None):
    """Measurement helper (include/qcast_bench.h): the loads and qT stores of
    qcast_per_channel_T on bf16 ``x [tokens, channels]`` without its
    arithmetic; ``out [channels, tokens]`` bytes receives meaningless data."""
    x = _bf16_input(x, "x")
    rows, cols = x.shape
    out = _out(out, (cols, rows), torch.uint8, x.device, "out")
    with torch.cuda.device(x.device):
        check(load().qcast_bench_per_channel_T_traffic(x.data_ptr(), rows, cols, out.data_ptr(),
                                                       _stream(x.device, stream)),
              "qcast_bench_per_channel_T_traffic")
    return out


def qcast_bench_check_scale(fmt, first, last, device="cuda:0", stream=None):
    """Self-check helper (include/qcast_bench.h): mismatches of the kernels'
    scale routine against IEEE division over fp32 patterns [first, last];
    returns (sf mismatches, sf_inv mismatches)."""
    dev = torch.device(device)
    counts = torch.empty(2 * 2048, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        check(load().qcast_bench_check_scale(fmt_id(fmt), first, last, counts.data_ptr(),
                                             _stream(dev, stream)), "qcast_bench_check_scale")
        c = counts.view(2048, 2).sum(dim=0, dtype=torch.int64).cpu()
    return int(c[0]), int(c[1])


def qcast_bench_time_next(start_event, stop_event):
    """Measurement helper (include/qcast_bench.h): the next kernel this thread
    launches through the library records these HIP events (raw hipEvent_t
    handles) at its own start and end."""
    check(load().qcast_bench_time_next(start_event, stop_event), "qcast_bench_time_next")


def per_token_cast(x, fmt="e4m3", num_per_channels=128):
    """``(out, out_sf)`` as in the page's quick-start call."""
    if fmt_id(fmt) == FMT_E2M1:
        return qcast_e2m1(x, num_per_channels)
    return qcast_per_token(x, fmt, num_per_channels)
