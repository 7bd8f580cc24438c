"""ctypes binding of libfp8bs.so with the C names, taking torch tensors.

The binding only marshals arguments: it checks dtypes, devices and strides,
allocates outputs with torch (device memory is torch's job here) and passes raw
pointers plus the current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels.  There is no fallback: when the
library is missing the import fails, and a non-zero status raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8bs.so")

FP8BS_OK = 0
GROUP = 128

_c_void_p, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int

_SIGNATURES = {
    "fp8bs_quantize_act_1x128": [_c_void_p, _i64, _i64, _i64, _int, _c_void_p, _i64, _c_void_p, _c_void_p],
    "fp8bs_quantize_act_1x128_routed": [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _i64, _c_void_p,
                                        _c_void_p],
    "fp8bs_quantize_act_1x128_dual": [_c_void_p, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p, _i64,
                                      _c_void_p, _c_void_p],
    "fp8bs_quantize_w_128x128": [_c_void_p, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p],
    "fp8bs_requantize_act_1x128_t": [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p],
    "fp8bs_gemm": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _int, _c_void_p, _i64,
                   _c_void_p],
    "fp8bs_gemm_noalloc": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _int, _c_void_p, _i64,
                           _c_void_p],
    "fp8bs_grouped_gemm": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i64,
                           _i64, _c_void_p, _c_void_p],
    "fp8bs_grouped_gemm_bf16w": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _c_void_p, _i64, _i64,
                                 _c_void_p, _c_void_p, _c_void_p, _int, _c_void_p],
    "fp8bs_gemm_wgrad": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _i64, _int,
                         _c_void_p],
    "fp8bs_moe_route": [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p],
    "fp8bs_moe_permute_quantize": [_c_void_p, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p, _i64,
                                   _c_void_p, _i64, _c_void_p, _i64, _c_void_p],
    "fp8bs_moe_combine": [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _i64,
                          _c_void_p],
}


class Fp8bsError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m fp8_fine_grained_act_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.fp8bs_status_string.argtypes = [ctypes.c_int]
    lib.fp8bs_status_string.restype = ctypes.c_char_p
    lib.fp8bs_moe_max_rows.argtypes = [_i64, _i64, _i64]
    lib.fp8bs_moe_max_rows.restype = ctypes.c_int64
    return lib


raw = _load()
EXPORTED = tuple(_SIGNATURES) + ("fp8bs_status_string", "fp8bs_moe_max_rows")


def status_string(status):
    return raw.fp8bs_status_string(int(status)).decode()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, status):
    if status != FP8BS_OK:
        raise Fp8bsError(fn, status)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return t


def _row_major(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def fp8bs_quantize_act_1x128(x, transpose=0, q=None, scales=None, stream=None):
    """1x128 tile quantization of bf16 x [rows, cols].

    transpose=0: q uint8 [rows, cols], scales f32 [rows, cols/128].
    transpose=1: q uint8 [cols, rows], scales f32 [cols, rows/128] (tiles along rows).
    """
    _dev(x, torch.bfloat16, "x")
    ldx = _row_major(x, "x")
    rows, cols = x.shape
    if transpose:
        qshape, sshape = (cols, rows), (cols, rows // GROUP)
    else:
        qshape, sshape = (rows, cols), (rows, cols // GROUP)
    if q is None:
        q = torch.empty(qshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.float32, device=x.device)
    _dev(q, torch.uint8, "q")
    _dev(scales, torch.float32, "scales")
    ldq = _row_major(q, "q")
    if tuple(q.shape) != qshape or tuple(scales.shape) != sshape or not scales.is_contiguous():
        raise ValueError("output shapes do not match the input")
    st = raw.fp8bs_quantize_act_1x128(x.data_ptr(), rows, cols, ldx, int(bool(transpose)), q.data_ptr(), ldq,
                                      scales.data_ptr(), _stream(stream))
    _check("fp8bs_quantize_act_1x128", st)
    return q, scales


def fp8bs_quantize_act_1x128_routed(x, row_token, q=None, scales=None, stream=None):
    """1x128 tiles along the columns of the rows of bf16 x [rows, cols] whose
    row_token entry (int32 [rows]) is >= 0; the other rows of q and scales are
    left as they are.  Returns (q [rows, cols], scales [rows, cols/128])."""
    _dev(x, torch.bfloat16, "x")
    _dev(row_token, torch.int32, "row_token")
    ldx = _row_major(x, "x")
    rows, cols = x.shape
    if tuple(row_token.shape) != (rows,) or not row_token.is_contiguous():
        raise ValueError("row_token must be a contiguous int32 [rows]")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // GROUP), dtype=torch.float32, device=x.device)
    _dev(q, torch.uint8, "q")
    _dev(scales, torch.float32, "scales")
    ldq = _row_major(q, "q")
    if tuple(q.shape) != (rows, cols) or tuple(scales.shape) != (rows, cols // GROUP) or not scales.is_contiguous():
        raise ValueError("output shapes do not match the input")
    st = raw.fp8bs_quantize_act_1x128_routed(x.data_ptr(), rows, cols, ldx, row_token.data_ptr(), q.data_ptr(), ldq,
                                             scales.data_ptr(), _stream(stream))
    _check("fp8bs_quantize_act_1x128_routed", st)
    return q, scales


def fp8bs_quantize_act_1x128_dual(x, q=None, scales=None, qt=None, scales_t=None, stream=None):
    """Both 1x128 orientations of bf16 x [rows, cols] from one read.

    Returns (q [rows, cols], scales [rows, cols/128], qt [cols, rows], scales_t [cols, rows/128]),
    bit-identical to fp8bs_quantize_act_1x128 with transpose=0 and transpose=1.
    """
    _dev(x, torch.bfloat16, "x")
    ldx = _row_major(x, "x")
    rows, cols = x.shape
    mk = lambda t, shape, dt: torch.empty(shape, dtype=dt, device=x.device) if t is None else t  # noqa: E731
    q = mk(q, (rows, cols), torch.uint8)
    scales = mk(scales, (rows, cols // GROUP), torch.float32)
    qt = mk(qt, (cols, rows), torch.uint8)
    scales_t = mk(scales_t, (cols, rows // GROUP), torch.float32)
    for t, dt, name in ((q, torch.uint8, "q"), (scales, torch.float32, "scales"), (qt, torch.uint8, "qt"),
                        (scales_t, torch.float32, "scales_t")):
        _dev(t, dt, name)
    ldq, ldqt = _row_major(q, "q"), _row_major(qt, "qt")
    if (tuple(q.shape) != (rows, cols) or tuple(qt.shape) != (cols, rows)
            or tuple(scales.shape) != (rows, cols // GROUP) or tuple(scales_t.shape) != (cols, rows // GROUP)
            or not scales.is_contiguous() or not scales_t.is_contiguous()):
        raise ValueError("output shapes do not match the input")
    st = raw.fp8bs_quantize_act_1x128_dual(x.data_ptr(), rows, cols, ldx, q.data_ptr(), ldq, scales.data_ptr(),
                                           qt.data_ptr(), ldqt, scales_t.data_ptr(), _stream(stream))
    _check("fp8bs_quantize_act_1x128_dual", st)
    return q, scales, qt, scales_t


def fp8bs_requantize_act_1x128_t(q, scales, qt=None, scales_t=None, stream=None):
    """Tiles along the rows from a cached activation: q [rows, cols] + scales [rows, cols/128]
    -> qt [cols, rows], scales_t [cols, rows/128]."""
    _dev(q, torch.uint8, "q")
    ldq = _row_major(q, "q")
    _dev(scales, torch.float32, "scales")
    rows, cols = q.shape
    if tuple(scales.shape) != (rows, cols // GROUP) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous [rows, cols/128] tensor")
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=q.device)
    if scales_t is None:
        scales_t = torch.empty((cols, rows // GROUP), dtype=torch.float32, device=q.device)
    _dev(qt, torch.uint8, "qt")
    ldqt = _row_major(qt, "qt")
    _dev(scales_t, torch.float32, "scales_t")
    if tuple(qt.shape) != (cols, rows) or tuple(scales_t.shape) != (cols, rows // GROUP) \
            or not scales_t.is_contiguous():
        raise ValueError("output shapes do not match the input")
    st = raw.fp8bs_requantize_act_1x128_t(q.data_ptr(), scales.data_ptr(), rows, cols, ldq, qt.data_ptr(), ldqt,
                                          scales_t.data_ptr(), _stream(stream))
    _check("fp8bs_requantize_act_1x128_t", st)
    return qt, scales_t


def fp8bs_quantize_w_128x128(w, q=None, scales=None, stream=None):
    """128x128 block quantization of bf16 w [n, k] (or [E, N, K], viewed as [E*N, K])."""
    _dev(w, torch.bfloat16, "w")
    lead = tuple(w.shape[:-2])
    w2 = w.reshape(-1, w.shape[-1]) if w.dim() == 3 else w
    ldw = _row_major(w2, "w")
    n, k = w2.shape
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(lead + (w.shape[-2] // GROUP, k // GROUP), dtype=torch.float32, device=w.device)
    _dev(q, torch.uint8, "q")
    q2 = q.reshape(-1, q.shape[-1]) if q.dim() == 3 else q
    ldq = _row_major(q2, "q")
    if tuple(q2.shape) != (n, k) or scales.numel() != (n // GROUP) * (k // GROUP) or not scales.is_contiguous():
        raise ValueError("output shapes do not match the input")
    st = raw.fp8bs_quantize_w_128x128(w2.data_ptr(), n, k, ldw, q2.data_ptr(), ldq, scales.data_ptr(),
                                      _stream(stream))
    _check("fp8bs_quantize_w_128x128", st)
    return q, scales


def fp8bs_gemm(qa, sa, qb, sb, b_layout=0, c=None, stream=None, _entry="fp8bs_gemm"):
    """bf16 C [m, n] from E4M3 A [m, k] and B ([n, k] for b_layout 0, [k, n] for 1)."""
    for t, nm in ((qa, "qa"), (qb, "qb")):
        _dev(t, torch.uint8, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    for t, nm in ((sa, "sa"), (sb, "sb")):
        _dev(t, torch.float32, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    m, k = qa.shape
    n = qb.shape[0] if b_layout == 0 else qb.shape[1]
    if c is None:
        c = torch.empty((m, n), dtype=torch.bfloat16, device=qa.device)
    _dev(c, torch.bfloat16, "c")
    ldc = _row_major(c, "c")
    st = getattr(raw, _entry)(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(), m, n, k, int(b_layout),
                              c.data_ptr(), ldc, _stream(stream))
    _check(_entry, st)
    return c


def fp8bs_gemm_noalloc(qa, sa, qb, sb, b_layout=0, c=None, stream=None):
    """fp8bs_gemm that never allocates device memory (a split contraction uses the library's fixed array).
    c is allocated here only when the caller passes none."""
    return fp8bs_gemm(qa, sa, qb, sb, b_layout=b_layout, c=c, stream=stream, _entry="fp8bs_gemm_noalloc")


def fp8bs_grouped_gemm(qa, sa, seg_offsets, qb, sb, c=None, stream=None, row_token=None):
    """MoE grouped GEMM: bf16 C [R, n]; qb [E, n, k]; seg_offsets int32 [E+1] on the device.

    row_token (int32 [R] on the device, the routing's row map, or None): when
    given, each 128-row tile's rows after its last routed row are not read and
    their outputs are 0."""
    _dev(qa, torch.uint8, "qa")
    _dev(qb, torch.uint8, "qb")
    _dev(sa, torch.float32, "sa")
    _dev(sb, torch.float32, "sb")
    _dev(seg_offsets, torch.int32, "seg_offsets")
    checked = [(qa, "qa"), (qb, "qb"), (sa, "sa"), (sb, "sb"), (seg_offsets, "seg_offsets")]
    if row_token is not None:
        _dev(row_token, torch.int32, "row_token")
        checked.append((row_token, "row_token"))
    for t, nm in checked:
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    rows, k = qa.shape
    num_e, n = qb.shape[0], qb.shape[1]
    if seg_offsets.numel() != num_e + 1:
        raise ValueError("seg_offsets must have num_experts + 1 entries")
    if row_token is not None and row_token.numel() != rows:
        raise ValueError("row_token must have one entry per row of qa")
    if c is None:
        c = torch.empty((rows, n), dtype=torch.bfloat16, device=qa.device)
    _dev(c, torch.bfloat16, "c")
    if not c.is_contiguous():
        raise ValueError("c must be contiguous")
    st = raw.fp8bs_grouped_gemm(qa.data_ptr(), sa.data_ptr(), seg_offsets.data_ptr(),
                                None if row_token is None else row_token.data_ptr(), num_e, rows, qb.data_ptr(),
                                sb.data_ptr(), n, k, c.data_ptr(), _stream(stream))
    _check("fp8bs_grouped_gemm", st)
    return c


def fp8bs_grouped_gemm_bf16w(qa, sa, seg_offsets, w, c=None, qw=None, sw=None, stream=None, row_token=None,
                             keep_codes=None):
    """MoE grouped GEMM from bf16 expert weights w [E, n, k]: bf16 C [R, n], the same bits as
    fp8bs_grouped_gemm over fp8bs_quantize_w_128x128(w).

    qw (uint8 [E, n, k]) and sw (float32 [E, n/128, k/128]), both or neither.  keep_codes
    (default: True when they are given) stores the weight codes and scales of every expert
    that owns rows there; keep_codes=False uses them as a workspace, storing only the codes
    of experts with more than one 128-row tile (read back by those tiles)."""
    if keep_codes is None:
        keep_codes = qw is not None
    _dev(qa, torch.uint8, "qa")
    _dev(sa, torch.float32, "sa")
    _dev(w, torch.bfloat16, "w")
    _dev(seg_offsets, torch.int32, "seg_offsets")
    checked = [(qa, "qa"), (sa, "sa"), (w, "w"), (seg_offsets, "seg_offsets")]
    if row_token is not None:
        _dev(row_token, torch.int32, "row_token")
        checked.append((row_token, "row_token"))
    if (qw is None) != (sw is None):
        raise ValueError("qw and sw go together")
    if qw is not None:
        _dev(qw, torch.uint8, "qw")
        _dev(sw, torch.float32, "sw")
        checked += [(qw, "qw"), (sw, "sw")]
    for t, nm in checked:
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    rows, k = qa.shape
    if w.dim() != 3 or w.shape[2] != k:
        raise ValueError("w must be [experts, n, k] with the k of qa")
    num_e, n = w.shape[0], w.shape[1]
    if seg_offsets.numel() != num_e + 1:
        raise ValueError("seg_offsets must have num_experts + 1 entries")
    if row_token is not None and row_token.numel() != rows:
        raise ValueError("row_token must have one entry per row of qa")
    if qw is not None and (tuple(qw.shape) != tuple(w.shape) or tuple(sw.shape) != (num_e, n // GROUP, k // GROUP)):
        raise ValueError("qw must be [E, n, k] and sw [E, n/128, k/128]")
    if c is None:
        c = torch.empty((rows, n), dtype=torch.bfloat16, device=qa.device)
    _dev(c, torch.bfloat16, "c")
    if not c.is_contiguous():
        raise ValueError("c must be contiguous")
    st = raw.fp8bs_grouped_gemm_bf16w(qa.data_ptr(), sa.data_ptr(), seg_offsets.data_ptr(),
                                      None if row_token is None else row_token.data_ptr(), num_e, rows,
                                      w.data_ptr(), n, k, c.data_ptr(), None if qw is None else qw.data_ptr(),
                                      None if sw is None else sw.data_ptr(), 1 if keep_codes else 0,
                                      _stream(stream))
    _check("fp8bs_grouped_gemm_bf16w", st)
    return c


def fp8bs_gemm_wgrad(qa, sa, qb, sb, c=None, accumulate=0, stream=None):
    """f32 C [m, n] (+)= A B^T over tokens; A [m, t], B [n, t], per-row scales [*, t/128]."""
    for t, nm in ((qa, "qa"), (qb, "qb")):
        _dev(t, torch.uint8, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    for t, nm in ((sa, "sa"), (sb, "sb")):
        _dev(t, torch.float32, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    m, t_len = qa.shape
    n = qb.shape[0]
    if c is None:
        c = torch.empty((m, n), dtype=torch.float32, device=qa.device)
    _dev(c, torch.float32, "c")
    ldc = _row_major(c, "c")
    st = raw.fp8bs_gemm_wgrad(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(), m, n, t_len,
                              c.data_ptr(), ldc, int(accumulate), _stream(stream))
    _check("fp8bs_gemm_wgrad", st)
    return c


def fp8bs_moe_max_rows(tokens, topk, num_experts):
    """Largest padded row count of the expert-major layout (host only)."""
    r = raw.fp8bs_moe_max_rows(int(tokens), int(topk), int(num_experts))
    if r < 0:
        raise Fp8bsError("fp8bs_moe_max_rows", r)
    return int(r)


def _contig(t, dtype, name):
    _dev(t, dtype, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def fp8bs_moe_route(topk_ids, num_experts, rows_cap=None, seg_offsets=None, slot_rows=None, row_token=None,
                    stream=None):
    """Expert-major padded layout of top-k routing: (seg_offsets [E+1], slot_rows [T, k], row_token [cap])."""
    _contig(topk_ids, torch.int32, "topk_ids")
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [tokens, topk]")
    tokens, topk = topk_ids.shape
    if rows_cap is None:
        rows_cap = fp8bs_moe_max_rows(tokens, topk, num_experts)
    dev = topk_ids.device
    if seg_offsets is None:
        seg_offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    if slot_rows is None:
        slot_rows = torch.empty((tokens, topk), dtype=torch.int32, device=dev)
    if row_token is None:
        row_token = torch.empty(rows_cap, dtype=torch.int32, device=dev)
    for t, nm in ((seg_offsets, "seg_offsets"), (slot_rows, "slot_rows"), (row_token, "row_token")):
        _contig(t, torch.int32, nm)
    if seg_offsets.numel() != num_experts + 1 or tuple(slot_rows.shape) != (tokens, topk) \
            or row_token.numel() != rows_cap:
        raise ValueError("output shapes do not match the routing")
    st = raw.fp8bs_moe_route(topk_ids.data_ptr(), tokens, topk, num_experts, seg_offsets.data_ptr(),
                             slot_rows.data_ptr(), row_token.data_ptr(), rows_cap, _stream(stream))
    _check("fp8bs_moe_route", st)
    return seg_offsets, slot_rows, row_token


def fp8bs_moe_permute_quantize(x, slot_rows, seg_offsets, row_token, q=None, scales=None, stream=None):
    """Dispatch payload: q uint8 [cap, hidden], scales f32 [cap, hidden/128] in expert-major rows."""
    _dev(x, torch.bfloat16, "x")
    ldx = _row_major(x, "x")
    tokens, hidden = x.shape
    for t, nm in ((slot_rows, "slot_rows"), (seg_offsets, "seg_offsets"), (row_token, "row_token")):
        _contig(t, torch.int32, nm)
    if slot_rows.dim() != 2 or slot_rows.shape[0] != tokens:
        raise ValueError("slot_rows must be [tokens, topk]")
    topk = slot_rows.shape[1]
    cap = row_token.numel()
    num_e = seg_offsets.numel() - 1
    if q is None:
        q = torch.empty((cap, hidden), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((cap, hidden // GROUP), dtype=torch.float32, device=x.device)
    _dev(q, torch.uint8, "q")
    ldq = _row_major(q, "q")
    _contig(scales, torch.float32, "scales")
    if tuple(q.shape) != (cap, hidden) or tuple(scales.shape) != (cap, hidden // GROUP):
        raise ValueError("output shapes do not match the row capacity")
    st = raw.fp8bs_moe_permute_quantize(x.data_ptr(), tokens, hidden, ldx, slot_rows.data_ptr(), topk,
                                        seg_offsets.data_ptr(), row_token.data_ptr(), num_e, q.data_ptr(), ldq,
                                        scales.data_ptr(), cap, _stream(stream))
    _check("fp8bs_moe_permute_quantize", st)
    return q, scales


def fp8bs_moe_combine(y, slot_rows, gates, out=None, stream=None):
    """bf16 out [tokens, n] = sum_j gates[t, j] * y[slot_rows[t, j]] (FP32 accumulation)."""
    _dev(y, torch.bfloat16, "y")
    ldy = _row_major(y, "y")
    cap, n = y.shape
    _contig(slot_rows, torch.int32, "slot_rows")
    _contig(gates, torch.float32, "gates")
    if slot_rows.dim() != 2 or tuple(gates.shape) != tuple(slot_rows.shape):
        raise ValueError("slot_rows and gates must both be [tokens, topk]")
    tokens, topk = slot_rows.shape
    if out is None:
        out = torch.empty((tokens, n), dtype=torch.bfloat16, device=y.device)
    _dev(out, torch.bfloat16, "out")
    ldo = _row_major(out, "out")
    if tuple(out.shape) != (tokens, n):
        raise ValueError("out must be [tokens, n]")
    st = raw.fp8bs_moe_combine(y.data_ptr(), ldy, cap, slot_rows.data_ptr(), gates.data_ptr(), tokens, topk, n,
                               out.data_ptr(), ldo, _stream(stream))
    _check("fp8bs_moe_combine", st)
    return out
