"""Python binding of libmoeq (the routed-expert MoE forward over NVFP4 / VQ
expert weights, with an optional BF16 shared expert, for MI355X).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  PyTorch is used for device memory and the current stream.  If
libmoeq.so has not been built, every call raises -- there is no fallback.

Calls (same names as the C ABI in include/moeq.h):
    route_topk(logits, k)                       -> topk_ids, topk_w
    permute(topk_ids, E)                        -> counts, offsets, perm_src, inv_perm
    expert_ffn_q(layer, x, perm_src, offsets, k) -> y_perm
    combine(y_perm, inv_perm, topk_w)           -> out
    shared_ffn(shared, x)                       -> y_shared
    combine_shared(y_perm, inv_perm, topk_w, y_shared) -> out
    forward(layer, x, logits, k, shared=None)   -> all of the above
    layer_forward(layer, x, logits, k)          -> topk_ids, topk_w, out (one C call)
Host packers: quantize_nvfp4, quantize_nvfp4_residual, pack_nvfp4_expert,
pack_nvfp4r_expert, pack_vq_expert, pack_vq8_expert, pack_bf16_expert,
record_bytes, record_table.  Test hook: dequant_q.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeq.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EWORKSPACE = -3
MOE_EHIP = -4

FMT_NVFP4 = 1
FMT_VQ = 2
FMT_VQ8 = 3
FMT_BF16 = 4
FMT_NVFP4R = 5      # nested two-level NVFP4: base plane + residual plane
FMT_VQ8_M1, FMT_VQ8_M2, FMT_VQ8_M3 = 6, 7, 8   # small-codebook VQ at 1 / 2 / 3 bits
FMT_VQ8_RATES = (FMT_VQ8_M1, FMT_VQ8_M2, FMT_VQ8_M3)
FORMATS = (FMT_NVFP4, FMT_VQ, FMT_VQ8, FMT_BF16, FMT_NVFP4R) + FMT_VQ8_RATES


def vq8_rate(fmt, vq8_m):
    """Codes per 8-weight group of a small-codebook VQ format (vq8_m for
    FMT_VQ8), 0 for other formats."""
    if fmt == FMT_VQ8:
        return vq8_m
    if fmt in FMT_VQ8_RATES:
        return fmt - FMT_VQ8_M1 + 1
    return 0
REC_COMPACT, REC_RESIDENT = 0, 1
PROJ_GATE, PROJ_UP, PROJ_DOWN = 0, 1, 2
VQ_NCODE = 65536
VQ8_NCODE = 256
STATIC_WS_BYTES = 32 << 20   # MOE_STATIC_WS_BYTES: moe_layer_forward_static's per-GPU array


class MoeError(RuntimeError):
    def __init__(self, status, fn, detail):
        self.status = status
        super().__init__(f"{fn}: status {status}: {detail}")


class _QLayerC(ctypes.Structure):
    _fields_ = [
        ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
        ("vq8_m", ctypes.c_int32),
        ("fmt_host", ctypes.c_void_p),
        ("rec_dev", ctypes.c_void_p),
        ("nvfp4_w13", ctypes.c_void_p), ("nvfp4_w13_stride", ctypes.c_int64),
        ("nvfp4_w2", ctypes.c_void_p), ("nvfp4_w2_stride", ctypes.c_int64),
        ("vq_w13", ctypes.c_void_p), ("vq_w13_stride", ctypes.c_int64),
        ("vq_w2", ctypes.c_void_p), ("vq_w2_stride", ctypes.c_int64),
        ("vq_codebook", ctypes.c_void_p * 3),
        ("vq_codebook_stride", ctypes.c_int64),
        ("vq8_w13", ctypes.c_void_p), ("vq8_w13_stride", ctypes.c_int64),
        ("vq8_w2", ctypes.c_void_p), ("vq8_w2_stride", ctypes.c_int64),
        ("vq8_codebook", ctypes.c_void_p * 3),
        ("bf16_w13", ctypes.c_void_p), ("bf16_w13_stride", ctypes.c_int64),
        ("bf16_w2", ctypes.c_void_p), ("bf16_w2_stride", ctypes.c_int64),
        ("record_mode", ctypes.c_int32), ("rot_in2_block", ctypes.c_int32),
        ("rot_signs", ctypes.c_void_p),
        ("nvfp4r_w13", ctypes.c_void_p), ("nvfp4r_w13_stride", ctypes.c_int64),
        ("nvfp4r_w2", ctypes.c_void_p), ("nvfp4r_w2_stride", ctypes.c_int64),
        ("nvfp4r_shift", ctypes.c_int32), ("reserved2", ctypes.c_int32),
        ("vq8r_w13", ctypes.c_void_p * 3), ("vq8r_w13_stride", ctypes.c_int64 * 3),
        ("vq8r_w2", ctypes.c_void_p * 3), ("vq8r_w2_stride", ctypes.c_int64 * 3),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_PROTOS = {
    "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_route_topk": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_permute_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "moe_permute": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_permute": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                         _P]),
    "moe_ffn_workspace_bytes": (_SZ, [ctypes.POINTER(_QLayerC), _I64, _I32]),
    "moe_expert_ffn_q": (ctypes.c_int, [ctypes.POINTER(_QLayerC), _P, _P, _P, _I64, _I32, _P,
                                        _P, _SZ, _P]),
    "moe_gateup_workspace_bytes": (_SZ, [ctypes.POINTER(_QLayerC), _I64, _I32]),
    "moe_expert_gateup_q": (ctypes.c_int, [ctypes.POINTER(_QLayerC), _P, _P, _P, _I64, _I32, _P,
                                           _P, _SZ, _P]),
    "moe_expert_down_q": (ctypes.c_int, [ctypes.POINTER(_QLayerC), _P, _P, _I64, _I32, _P, _P]),
    "moe_combine": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _P, _P]),
    "moe_shared_ffn_workspace_bytes": (_SZ, [ctypes.POINTER(_QLayerC), _I64]),
    "moe_shared_ffn": (ctypes.c_int, [ctypes.POINTER(_QLayerC), _P, _I64, _P, _P, _SZ, _P]),
    "moe_combine_shared": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I32, _I32, _P, _P]),
    "moe_layer_forward_workspace_bytes": (_SZ, [ctypes.POINTER(_QLayerC), _I64, _I32]),
    "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(_QLayerC), _P, _P, _I64, _I32, _P, _P,
                                         _P, _P, _P, _SZ, _P]),
    "moe_layer_forward_static": (ctypes.c_int, [ctypes.POINTER(_QLayerC), _P, _P, _I64, _I32,
                                                _P, _P, _P, _P, _P]),
    "moe_layer_forward_shared_workspace_bytes": (_SZ, [ctypes.POINTER(_QLayerC),
                                                       ctypes.POINTER(_QLayerC), _I64, _I32]),
    "moe_layer_forward_shared": (ctypes.c_int, [ctypes.POINTER(_QLayerC),
                                                ctypes.POINTER(_QLayerC), _P, _P, _I64, _I32,
                                                _P, _P, _P, _P, _SZ, _P]),
    "moe_quantize_nvfp4": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "moe_quantize_nvfp4_residual": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P, _P]),
    "moe_pack_nvfp4r_expert": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "moe_record_bytes": (_SZ, [ctypes.c_int, ctypes.c_int, _I32, _I32]),
    "moe_record_bytes_vq8": (_SZ, [ctypes.c_int, _I32, _I32, _I32]),
    "moe_pack_vq8_expert": (ctypes.c_int, [_P] * 6 + [_I32, _I32, _I32, _P, _P]),
    "moe_pack_nvfp4_expert": (ctypes.c_int, [_P] * 6 + [_I32, _I32, _P, _P]),
    "moe_pack_vq_expert": (ctypes.c_int, [_P] * 6 + [_I32, _I32, _P, _P]),
    "moe_pack_bf16_expert": (ctypes.c_int, [_P] * 3 + [_I32, _I32, _P, _P]),
    "moe_rot_sign_bytes": (_SZ, [_I32, _I32]),
    "moe_pack_rot_signs": (ctypes.c_int, [_P] * 5 + [_I32, _I32, _P]),
    "moe_rotate_matrix": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P]),
    "moe_rotate_matrix_blocks": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _I32, _I32, _P]),
    "moe_record_table": (ctypes.c_int, [_P, _I32, _P, _P]),
    "moe_record_table_resident": (ctypes.c_int, [_P, _I32, _P]),
    "moe_dequant_q": (ctypes.c_int, [ctypes.POINTER(_QLayerC), _I32, _I32, _P, _P]),
    "moe_probe_read": (ctypes.c_int, [_P, _SZ, _P, _P]),
}

_lib = None


def lib():
    """The loaded libmoeq (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bit_quantized_moe_route_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status, fn):
    if status != MOE_OK:
        L = lib()
        detail = L.moe_last_error().decode() or L.moe_strerror(status).decode()
        raise MoeError(status, fn, detail)


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# host packers (numpy in, numpy out)
# --------------------------------------------------------------------------

def quantize_nvfp4(w):
    """fp32 [n, kin] -> (codes uint8 [n, kin/2], scales uint8 [n, kin/16])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, kin = w.shape
    codes = np.empty((n, kin // 2), np.uint8)
    scales = np.empty((n, max(kin // 16, 0)), np.uint8)
    _check(lib().moe_quantize_nvfp4(_np_ptr(w), n, kin, _np_ptr(codes), _np_ptr(scales)),
           "moe_quantize_nvfp4")
    return codes, scales


NVFP4R_SHIFT = 8    # default residual-plane exponent of a nested layer


def quantize_nvfp4_residual(w, shift=NVFP4R_SHIFT):
    """fp32 [n, kin] -> ((base codes, base scales), (residual codes, residual
    scales)): the two planes of a nested two-level NVFP4 matrix (the residual
    plane holds the residual times 2^shift)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, kin = w.shape
    out = [np.empty((n, kin // 2), np.uint8), np.empty((n, max(kin // 16, 0)), np.uint8),
           np.empty((n, kin // 2), np.uint8), np.empty((n, max(kin // 16, 0)), np.uint8)]
    _check(lib().moe_quantize_nvfp4_residual(_np_ptr(w), n, kin, shift,
                                             *[_np_ptr(a) for a in out]),
           "moe_quantize_nvfp4_residual")
    return (out[0], out[1]), (out[2], out[3])


def record_bytes(fmt, which, H, I, vq8_m=0):
    if fmt == FMT_VQ8:
        return int(lib().moe_record_bytes_vq8(which, H, I, vq8_m))
    return int(lib().moe_record_bytes(fmt, which, H, I))


def pack_nvfp4_expert(gate, up, down, H, I, w13=None, w2=None):
    """gate/up/down = (codes, scales) canonical NVFP4 -> (w13 record, w2 record)."""
    if w13 is None:
        w13 = np.empty(record_bytes(FMT_NVFP4, 0, H, I), np.uint8)
    if w2 is None:
        w2 = np.empty(record_bytes(FMT_NVFP4, 1, H, I), np.uint8)
    arrs = [np.ascontiguousarray(a, dtype=np.uint8) for pair in (gate, up, down) for a in pair]
    _check(lib().moe_pack_nvfp4_expert(*[_np_ptr(a) for a in arrs], H, I, _np_ptr(w13),
                                       _np_ptr(w2)), "moe_pack_nvfp4_expert")
    return w13, w2


def pack_nvfp4r_expert(base, res, H, I, w13=None, w2=None):
    """base / res = ((codes, scales) of gate, up, down) of the two planes ->
    (w13 record, w2 record) of a nested two-level NVFP4 expert."""
    if w13 is None:
        w13 = np.empty(record_bytes(FMT_NVFP4R, 0, H, I), np.uint8)
    if w2 is None:
        w2 = np.empty(record_bytes(FMT_NVFP4R, 1, H, I), np.uint8)
    b = [np.ascontiguousarray(a, dtype=np.uint8) for pair in base for a in pair]
    r = [np.ascontiguousarray(a, dtype=np.uint8) for pair in res for a in pair]
    bp = (ctypes.c_void_p * 6)(*[a.ctypes.data for a in b])
    rp = (ctypes.c_void_p * 6)(*[a.ctypes.data for a in r])
    _check(lib().moe_pack_nvfp4r_expert(ctypes.cast(bp, ctypes.c_void_p),
                                        ctypes.cast(rp, ctypes.c_void_p), H, I, _np_ptr(w13),
                                        _np_ptr(w2)), "moe_pack_nvfp4r_expert")
    return w13, w2


def pack_vq_expert(gate, up, down, H, I, w13=None, w2=None):
    """gate/up/down = (codes uint16 [n, kin/8], scales fp16 bits uint16 [n])."""
    if w13 is None:
        w13 = np.empty(record_bytes(FMT_VQ, 0, H, I), np.uint8)
    if w2 is None:
        w2 = np.empty(record_bytes(FMT_VQ, 1, H, I), np.uint8)
    arrs = [np.ascontiguousarray(a, dtype=np.uint16) for pair in (gate, up, down) for a in pair]
    _check(lib().moe_pack_vq_expert(*[_np_ptr(a) for a in arrs], H, I, _np_ptr(w13), _np_ptr(w2)),
           "moe_pack_vq_expert")
    return w13, w2


def pack_vq8_expert(gate, up, down, H, I, m, w13=None, w2=None):
    """gate/up/down = (codes uint8 [n, kin/8, m], scales fp16 bits uint16 [n])."""
    if w13 is None:
        w13 = np.empty(record_bytes(FMT_VQ8, 0, H, I, m), np.uint8)
    if w2 is None:
        w2 = np.empty(record_bytes(FMT_VQ8, 1, H, I, m), np.uint8)
    arrs = []
    for codes, scales in (gate, up, down):
        arrs.append(np.ascontiguousarray(codes, dtype=np.uint8))
        arrs.append(np.ascontiguousarray(scales, dtype=np.uint16))
    _check(lib().moe_pack_vq8_expert(*[_np_ptr(a) for a in arrs], H, I, m, _np_ptr(w13),
                                     _np_ptr(w2)), "moe_pack_vq8_expert")
    return w13, w2


def pack_bf16_expert(gate, up, down, H, I, w13=None, w2=None):
    """gate, up [I, H], down [H, I]: bf16 bits (uint16 / int16) or torch
    bfloat16 CPU tensors -> (w13 record, w2 record)."""
    if w13 is None:
        w13 = np.empty(record_bytes(FMT_BF16, 0, H, I), np.uint8)
    if w2 is None:
        w2 = np.empty(record_bytes(FMT_BF16, 1, H, I), np.uint8)
    arrs = []
    for a in (gate, up, down):
        if hasattr(a, "view") and not isinstance(a, np.ndarray):   # torch bfloat16
            a = a.contiguous().view(_torch().int16).numpy()
        arrs.append(np.ascontiguousarray(a).view(np.uint16))
    _check(lib().moe_pack_bf16_expert(*[_np_ptr(a) for a in arrs], H, I, _np_ptr(w13),
                                      _np_ptr(w2)), "moe_pack_bf16_expert")
    return w13, w2


def rot_sign_bytes(H, I):
    return int(lib().moe_rot_sign_bytes(H, I))


def pack_rot_signs(s_in13, s_out_gate, s_out_up, s_in2, s_out2, H, I):
    """One expert's rotation signs (int8 +-1 arrays) -> the packed bits."""
    arrs = [np.ascontiguousarray(a, dtype=np.int8) for a in
            (s_in13, s_out_gate, s_out_up, s_in2, s_out2)]
    out = np.empty(rot_sign_bytes(H, I), np.uint8)
    _check(lib().moe_pack_rot_signs(*[_np_ptr(a) for a in arrs], H, I, _np_ptr(out)),
           "moe_pack_rot_signs")
    return out


def rotate_matrix(w, s_out, s_in, block_out=128, block_in=128):
    """W_rot = R_out W R_in^T (fp32 in and out, fp64 inside), R = signs then
    Hadamard-b / sqrt(b) per block of b (128, or 512 for the input side of a
    wide-variant down matrix): the offline step of a rotated format."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    so = np.ascontiguousarray(s_out, dtype=np.int8)
    si = np.ascontiguousarray(s_in, dtype=np.int8)
    out = np.empty_like(w)
    _check(lib().moe_rotate_matrix_blocks(_np_ptr(w), w.shape[0], w.shape[1], _np_ptr(so),
                                          _np_ptr(si), block_out, block_in, _np_ptr(out)),
           "moe_rotate_matrix_blocks")
    return out


def record_table(fmt_host):
    """(rec [E] int32, experts per format {tag: n for every tag in FORMATS})."""
    fmt_host = np.ascontiguousarray(fmt_host, dtype=np.uint8)
    E = fmt_host.shape[0]
    rec = np.empty(E, np.int32)
    n = np.zeros(max(FORMATS) + 1, np.int32)
    _check(lib().moe_record_table(_np_ptr(fmt_host), E, _np_ptr(rec), _np_ptr(n)),
           "moe_record_table")
    return rec, {f: int(n[f]) for f in FORMATS}


def record_table_resident(fmt_host):
    """rec [E] = fmt << 24 | e (every used pool holds every expert at slot e)."""
    fmt_host = np.ascontiguousarray(fmt_host, dtype=np.uint8)
    rec = np.empty(fmt_host.shape[0], np.int32)
    _check(lib().moe_record_table_resident(_np_ptr(fmt_host), fmt_host.shape[0], _np_ptr(rec)),
           "moe_record_table_resident")
    return rec


# --------------------------------------------------------------------------
# device calls (torch tensors for memory and the current stream)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(dev=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("device tensors required")
        if t is not None and not t.is_contiguous():
            raise ValueError("contiguous tensors required")


class QLayer:
    """A packed expert layer resident on one GPU.

    Holds the device pools, the record table and the codebooks, and the C
    descriptor that points at them.  Build it with `QLayer.build(...)`.
    """

    def __init__(self, E, H, I, fmt_host, device="cuda", vq8_m=0, resident_formats=None,
                 nvfp4r_shift=NVFP4R_SHIFT):
        """resident_formats: None (compact pools: each expert stored in its own
        format only) or a set of format tags whose pools hold every expert at
        slot e, so that set_tiers() can move experts between those formats
        between calls.  With both FMT_NVFP4 and FMT_NVFP4R resident the layer
        is nested: the NVFP4 pools are the NVFP4R records themselves (their
        base planes), so moving an expert between the two tiers changes no
        bytes (set_residual writes a residual plane on its own)."""
        torch = _torch()
        self.E, self.H, self.I = int(E), int(H), int(I)
        self.fmt_host = np.ascontiguousarray(fmt_host, dtype=np.uint8)
        self.resident = frozenset(resident_formats) if resident_formats else None
        _, counts = record_table(self.fmt_host)
        if self.resident is not None:
            if not set(np.unique(self.fmt_host).tolist()) <= self.resident:
                raise ValueError("every expert's format must be one of the resident formats")
            rec = record_table_resident(self.fmt_host)
            sizes = {f: (self.E if f in self.resident else 0) for f in FORMATS}
        else:
            rec = record_table(self.fmt_host)[0]
            sizes = dict(counts)
        self.counts = counts
        if sizes[FMT_VQ8] and vq8_m not in (1, 2, 3):
            raise ValueError("a layer with small-codebook VQ experts needs vq8_m = 1, 2 or 3")
        # the layer's small codebooks per projection: as many as its largest rate
        self.vq8_ncb = max([vq8_m if sizes[FMT_VQ8] else 0]
                           + [vq8_rate(f, 0) for f in FMT_VQ8_RATES if sizes[f]])
        self.vq8_m = int(vq8_m)
        self.nvfp4r_shift = int(nvfp4r_shift)
        self.rec_host = rec
        self.device = torch.device(device)
        self.rec_dev = torch.from_numpy(rec).to(self.device)
        self.stride = {}
        self.pools = {}
        nested = (self.resident is not None and FMT_NVFP4 in self.resident
                  and FMT_NVFP4R in self.resident)
        self.alias = {FMT_NVFP4: FMT_NVFP4R} if nested else {}
        for fmt in sorted(FORMATS, key=lambda f: f in self.alias):
            if fmt in self.alias:
                for which in (0, 1):
                    self.stride[(fmt, which)] = self.stride[(self.alias[fmt], which)]
                    self.pools[(fmt, which)] = self.pools[(self.alias[fmt], which)]
                continue
            n = sizes[fmt]
            for which in (0, 1):
                b = record_bytes(fmt, which, H, I, self.vq8_m) if n else 0
                s = (b + 255) // 256 * 256
                self.stride[(fmt, which)] = s
                self.pools[(fmt, which)] = (torch.empty(n * s, dtype=torch.uint8, device=self.device)
                                            if n else None)
        self.codebooks = [None, None, None]
        self.codebook_stride = 0
        self.codebooks8 = [None, None, None]
        self.rot_signs = None
        self.rot_in2_block = 128
        self._c = None

    def record_index(self, e):
        return int(self.rec_host[e] & 0xFFFFFF)

    def set_tiers(self, fmt_host):
        """Resident layers: move experts between the resident formats.  The
        host tier map is updated in place and the device record table by a
        copy on the current stream, so calls issued afterwards on that stream
        use the new tiers."""
        torch = _torch()
        if self.resident is None:
            raise ValueError("set_tiers needs a layer built with resident_formats")
        new = np.ascontiguousarray(fmt_host, dtype=np.uint8)
        if new.shape != self.fmt_host.shape or not set(np.unique(new).tolist()) <= self.resident:
            raise ValueError("tier map must give every expert one of the resident formats")
        rec = record_table_resident(new)
        self.fmt_host[:] = new          # in place: the C descriptor points at this array
        self.rec_host = rec
        self.rec_dev.copy_(torch.from_numpy(rec))
        self.counts = record_table(self.fmt_host)[1]

    def set_record(self, e, w13, w2, fmt=None, stream=None):
        """Copy one expert's two host records (numpy uint8) into its pool slots
        (fmt: the format of the records; a resident layer holds one per
        resident format)."""
        torch = _torch()
        fmt = int(self.fmt_host[e]) if fmt is None else int(fmt)
        idx = e if self.resident is not None else self.record_index(e)
        for which, rec in ((0, w13), (1, w2)):
            s = self.stride[(fmt, which)]
            dst = self.pools[(fmt, which)][idx * s: idx * s + rec.shape[0]]
            dst.copy_(torch.from_numpy(np.ascontiguousarray(rec)), non_blocking=False)
        self._c = None

    def set_residual(self, e, res13, res2):
        """Nested layers: write the residual planes (NVFP4 records, numpy
        uint8) of expert e's two-level records, leaving their base planes as
        they are."""
        torch = _torch()
        idx = e if self.resident is not None else self.record_index(e)
        for which, rec in ((0, res13), (1, res2)):
            off = record_bytes(FMT_NVFP4, which, self.H, self.I)
            if rec.shape[0] > off:
                raise ValueError("a residual plane is one NVFP4 record")
            s = self.stride[(FMT_NVFP4R, which)]
            dst = self.pools[(FMT_NVFP4R, which)][idx * s + off: idx * s + off + rec.shape[0]]
            dst.copy_(torch.from_numpy(np.ascontiguousarray(rec)), non_blocking=False)
        self._c = None

    def set_codebooks(self, cbs, stride=0):
        """cbs: three uint16 arrays [n_vq_books * 65536, 8] (fp16 bits) for gate,
        up, down; stride = bytes between per-record codebooks (0 = shared)."""
        torch = _torch()
        self.codebooks = [torch.from_numpy(np.ascontiguousarray(c, dtype=np.uint16).view(np.int16))
                          .to(self.device) for c in cbs]
        self.codebook_stride = int(stride)
        self._c = None

    def set_codebooks8(self, cbs):
        """Small-codebook VQ: for gate, up and down, a list of uint16 arrays
        [256, 8] (fp16 bits), codebook 0 first: as many as the layer's largest
        rate (vq8_m, or the largest explicit rate); an expert at rate m reads
        the first m."""
        torch = _torch()
        out = []
        for books in cbs:
            if len(books) != self.vq8_ncb:
                raise ValueError(f"{self.vq8_ncb} codebooks per projection (the largest rate)")
            a = np.ascontiguousarray(np.concatenate([np.asarray(b, dtype=np.uint16) for b in books]))
            if a.shape != (self.vq8_ncb * VQ8_NCODE, 8):
                raise ValueError("codebooks must be [256, 8] each")
            out.append(torch.from_numpy(a.view(np.int16)).to(self.device))
        self.codebooks8 = out
        self._c = None

    def set_rot_signs(self, signs, in2_block=128):
        """Rotated storage: signs uint8 [E, rot_sign_bytes(H, I)] (one row per
        expert from pack_rot_signs); None: the stored matrices are the weights.
        in2_block: the Hadamard block of the down projection's input side (128,
        or 512 for the wide variant)."""
        torch = _torch()
        self.rot_in2_block = in2_block
        if signs is None:
            self.rot_signs = None
        else:
            a = np.ascontiguousarray(signs, dtype=np.uint8)
            if a.shape != (self.E, rot_sign_bytes(self.H, self.I)):
                raise ValueError("rotation signs must be [E, rot_sign_bytes(H, I)]")
            self.rot_signs = torch.from_numpy(a).to(self.device)
        self._c = None

    def c(self):
        if self._c is None:
            d = _QLayerC()
            d.E, d.H, d.I = self.E, self.H, self.I
            d.fmt_host = self.fmt_host.ctypes.data
            d.rec_dev = self.rec_dev.data_ptr()
            d.vq8_m = self.vq8_m
            d.nvfp4r_shift = self.nvfp4r_shift
            d.record_mode = REC_RESIDENT if self.resident is not None else REC_COMPACT
            for fmt, n13, n2 in ((FMT_NVFP4, "nvfp4_w13", "nvfp4_w2"), (FMT_VQ, "vq_w13", "vq_w2"),
                                 (FMT_VQ8, "vq8_w13", "vq8_w2"),
                                 (FMT_BF16, "bf16_w13", "bf16_w2"),
                                 (FMT_NVFP4R, "nvfp4r_w13", "nvfp4r_w2")):
                p13, p2 = self.pools[(fmt, 0)], self.pools[(fmt, 1)]
                setattr(d, n13, p13.data_ptr() if p13 is not None else None)
                setattr(d, n2, p2.data_ptr() if p2 is not None else None)
                setattr(d, n13 + "_stride", self.stride[(fmt, 0)])
                setattr(d, n2 + "_stride", self.stride[(fmt, 1)])
            for i, fmt in enumerate(FMT_VQ8_RATES):
                p13, p2 = self.pools[(fmt, 0)], self.pools[(fmt, 1)]
                d.vq8r_w13[i] = p13.data_ptr() if p13 is not None else None
                d.vq8r_w2[i] = p2.data_ptr() if p2 is not None else None
                d.vq8r_w13_stride[i] = self.stride[(fmt, 0)]
                d.vq8r_w2_stride[i] = self.stride[(fmt, 1)]
            for p in range(3):
                cb = self.codebooks[p]
                d.vq_codebook[p] = cb.data_ptr() if cb is not None else None
            d.vq_codebook_stride = self.codebook_stride
            for p in range(3):
                cb = self.codebooks8[p]
                d.vq8_codebook[p] = cb.data_ptr() if cb is not None else None
            d.rot_signs = self.rot_signs.data_ptr() if self.rot_signs is not None else None
            d.rot_in2_block = self.rot_in2_block
            self._c = d
        return self._c

    def packed_bytes(self, experts):
        """Codes + scales bytes of the given experts (each counted once), plus
        each codebook once if a VQ expert is among them: the bytes a forward
        over those experts must read."""
        tot = 0
        vq = vq8 = False
        vq_books = 0                    # per-record VQ codebooks touched
        for e in set(int(x) for x in experts):
            if self.fmt_host[e] in (FMT_NVFP4, FMT_NVFP4R):
                planes = 2 if self.fmt_host[e] == FMT_NVFP4R else 1
                tot += planes * 3 * (self.H * self.I // 2 + self.H * self.I // 16)
            elif self.fmt_host[e] == FMT_BF16:
                tot += 3 * self.H * self.I * 2
            elif self.fmt_host[e] == FMT_VQ8 or self.fmt_host[e] in FMT_VQ8_RATES:
                vq8 = True
                m = vq8_rate(int(self.fmt_host[e]), self.vq8_m)
                tot += 3 * (self.H * self.I // 8) * m + (2 * self.I + self.H) * 2
            else:
                vq = True
                vq_books += 1
                tot += 3 * (self.H * self.I // 8) * 2 + (2 * self.I + self.H) * 2
        if vq:
            # one shared codebook per projection, or each touched record's own
            tot += 3 * VQ_NCODE * 8 * 2 * (1 if self.codebook_stride == 0 else vq_books)
        if vq8:
            tot += 3 * self.vq8_ncb * VQ8_NCODE * 8 * 2
        return tot


def route_topk(logits, k, topk_ids=None, topk_w=None):
    torch = _torch()
    _need_cuda(logits)
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(_dptr(logits), T, E, k, _dptr(topk_ids), _dptr(topk_w),
                                _stream(logits.device)), "moe_route_topk")
    return topk_ids, topk_w


def permute(topk_ids, E, out=None, ws=None):
    """Stable counting sort of the assignments by expert.  Returns counts,
    offsets, perm_src, inv_perm.  `ws`: from permute_workspace (allocated here
    if needed and not given)."""
    torch = _torch()
    _need_cuda(topk_ids)
    T, k = topk_ids.shape
    dev = topk_ids.device
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev))
    counts, offsets, perm_src, inv_perm = out
    L = lib()
    nws = L.moe_permute_workspace_bytes(T, k, E)
    if ws is None and nws:
        ws = permute_workspace(T, k, E, dev)
    _check(L.moe_permute(_dptr(topk_ids), T, k, E, _dptr(counts), _dptr(offsets),
                         _dptr(perm_src), _dptr(inv_perm), _dptr(ws),
                         ws.numel() if ws is not None else 0, _stream(dev)),
           "moe_permute")
    return counts, offsets, perm_src, inv_perm


def permute_workspace(T, k, E, device="cuda"):
    """Workspace tensor for permute / route_permute at these sizes (None if
    none is needed)."""
    torch = _torch()
    nws = lib().moe_permute_workspace_bytes(T, k, E)
    return torch.empty(nws, dtype=torch.uint8, device=device) if nws else None


def route_permute(logits, k, E=None, out=None, ws=None):
    """route_topk + permute in one call (one launch for T*k <= 64).
    Returns topk_ids, topk_w, counts, offsets, perm_src, inv_perm.  `ws`:
    from permute_workspace (allocated here if needed and not given)."""
    torch = _torch()
    _need_cuda(logits)
    T, E_ = logits.shape
    E = E_ if E is None else E
    dev = logits.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev))
    L = lib()
    nws = L.moe_permute_workspace_bytes(T, k, E)
    if ws is None and nws:
        ws = permute_workspace(T, k, E, dev)
    _check(L.moe_route_permute(_dptr(logits), T, E, k, *[_dptr(t) for t in out], _dptr(ws),
                               ws.numel() if ws is not None else 0, _stream(dev)),
           "moe_route_permute")
    return out


def ffn_workspace(layer, T, k):
    torch = _torch()
    n = lib().moe_ffn_workspace_bytes(ctypes.byref(layer.c()), T, k)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=layer.device)


def expert_ffn_q(layer, x, perm_src, offsets, k, y_perm=None, ws=None):
    """x: bf16 [T, H] tensor (or int16/uint16 holding bf16 bits)."""
    torch = _torch()
    _need_cuda(x, perm_src, offsets)
    T, H = x.shape
    if y_perm is None:
        y_perm = torch.empty((T * k, layer.H), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = ffn_workspace(layer, T, k)
    _check(lib().moe_expert_ffn_q(ctypes.byref(layer.c()), _dptr(x), _dptr(perm_src),
                                  _dptr(offsets), T, k, _dptr(y_perm), _dptr(ws), ws.numel(),
                                  _stream(x.device)), "moe_expert_ffn_q")
    return y_perm


def gateup_workspace(layer, T, k):
    torch = _torch()
    n = lib().moe_gateup_workspace_bytes(ctypes.byref(layer.c()), T, k)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=layer.device)


def expert_gateup_q(layer, x, perm_src, offsets, k, h=None, ws=None):
    """First half of the expert FFN: h = silu(W_gate x) * (W_up x), fp16 [T*k, I]."""
    torch = _torch()
    _need_cuda(x, perm_src, offsets)
    T = x.shape[0]
    if h is None:
        h = torch.empty((T * k, layer.I), dtype=torch.float16, device=x.device)
    if ws is None:
        ws = gateup_workspace(layer, T, k)
    _check(lib().moe_expert_gateup_q(ctypes.byref(layer.c()), _dptr(x), _dptr(perm_src),
                                     _dptr(offsets), T, k, _dptr(h), _dptr(ws), ws.numel(),
                                     _stream(x.device)), "moe_expert_gateup_q")
    return h


def expert_down_q(layer, h, offsets, k, y_perm=None):
    """Second half: y_perm = W_down h, fp32 [T*k, H]."""
    torch = _torch()
    _need_cuda(h, offsets)
    T = h.shape[0] // k
    if y_perm is None:
        y_perm = torch.empty((T * k, layer.H), dtype=torch.float32, device=h.device)
    _check(lib().moe_expert_down_q(ctypes.byref(layer.c()), _dptr(h), _dptr(offsets), T, k,
                                   _dptr(y_perm), _stream(h.device)), "moe_expert_down_q")
    return y_perm


def combine(y_perm, inv_perm, topk_w, out=None):
    torch = _torch()
    _need_cuda(y_perm, inv_perm, topk_w)
    T, k = topk_w.shape
    H = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=y_perm.device)
    _check(lib().moe_combine(_dptr(y_perm), _dptr(inv_perm), _dptr(topk_w), T, k, H, _dptr(out),
                             _stream(y_perm.device)), "moe_combine")
    return out


def shared_workspace(shared, T):
    torch = _torch()
    n = lib().moe_shared_ffn_workspace_bytes(ctypes.byref(shared.c()), T)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=shared.device)


def shared_ffn(shared, x, y=None, ws=None):
    """The shared expert (a one-expert QLayer) on every token: fp32 [T, H]."""
    torch = _torch()
    _need_cuda(x)
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, shared.H), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = shared_workspace(shared, T)
    _check(lib().moe_shared_ffn(ctypes.byref(shared.c()), _dptr(x), T, _dptr(y), _dptr(ws),
                                ws.numel(), _stream(x.device)), "moe_shared_ffn")
    return y


def combine_shared(y_perm, inv_perm, topk_w, y_shared, out=None):
    """combine, then + y_shared (the shared expert's output) per token."""
    torch = _torch()
    _need_cuda(y_perm, inv_perm, topk_w, y_shared)
    T, k = topk_w.shape
    H = y_perm.shape[1]
    if tuple(y_shared.shape) != (T, H) or y_shared.dtype != torch.float32:
        raise ValueError("y_shared must be fp32 [T, H]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=y_perm.device)
    _check(lib().moe_combine_shared(_dptr(y_perm), _dptr(inv_perm), _dptr(topk_w),
                                    _dptr(y_shared), T, k, H, _dptr(out), _stream(y_perm.device)),
           "moe_combine_shared")
    return out


PROBE_BLOCKS = 2048


def probe_read(buf, sink=None):
    """Read a device tensor once with the weight kernels' kind of loads (a
    measurement aid); returns the per-workgroup XOR sink."""
    torch = _torch()
    _need_cuda(buf)
    if sink is None:
        sink = torch.empty(PROBE_BLOCKS, dtype=torch.int32, device=buf.device)
    _check(lib().moe_probe_read(_dptr(buf), buf.numel() * buf.element_size(), _dptr(sink),
                                _stream(buf.device)), "moe_probe_read")
    return sink


def dequant_q(layer, expert, proj):
    torch = _torch()
    n, kin = (layer.H, layer.I) if proj == PROJ_DOWN else (layer.I, layer.H)
    out = torch.empty((n, kin), dtype=torch.float32, device=layer.device)
    _check(lib().moe_dequant_q(ctypes.byref(layer.c()), expert, proj, _dptr(out),
                               _stream(layer.device)), "moe_dequant_q")
    return out


_side_streams = {}


def side_stream(device):
    """A second stream of `device` (default priority), for the shared expert,
    which depends on x only and so can run beside the routed experts."""
    torch = _torch()
    d = torch.device(device)
    key = d.index if d.index is not None else torch.cuda.current_device()
    if key not in _side_streams:
        _side_streams[key] = torch.cuda.Stream(device=d)
    return _side_streams[key]


def layer_workspace(layer, T, k, shared=None):
    """Workspace of layer_forward (with `shared`: of its shared-expert form)."""
    torch = _torch()
    if shared is None:
        n = lib().moe_layer_forward_workspace_bytes(ctypes.byref(layer.c()), T, k)
    else:
        n = lib().moe_layer_forward_shared_workspace_bytes(ctypes.byref(layer.c()),
                                                           ctypes.byref(shared.c()), T, k)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=layer.device)


def layer_forward(layer, x, logits, k, y_shared=None, out=None, ids=None, w=None, ws=None,
                  shared=None):
    """The whole routed layer in one C call (moe_layer_forward): returns
    (topk_ids [T, k] int32, topk_w [T, k] fp32, out [T, H] fp32), with
    y_shared (fp32 [T, H], a shared expert's output) added after the routed
    sum when given.  Decode batches (T*k <= 16, k <= 8) of single-format
    layers run fused in two launches (four for a rotated layer).  With
    `shared` (a one-expert
    layer) instead of y_shared, the shared expert runs in the same C call
    (moe_layer_forward_shared; `ws` from layer_workspace(..., shared=))."""
    torch = _torch()
    _need_cuda(x, logits)
    T = x.shape[0]
    if tuple(logits.shape) != (T, layer.E) or logits.dtype != torch.float32:
        raise ValueError("logits must be fp32 [T, E]")
    if shared is not None and y_shared is not None:
        raise ValueError("give the shared layer or its output y_shared, not both")
    if y_shared is not None:
        _need_cuda(y_shared)
        if tuple(y_shared.shape) != (T, layer.H) or y_shared.dtype != torch.float32:
            raise ValueError("y_shared must be fp32 [T, H]")
    dev = x.device
    if out is None:
        out = torch.empty((T, layer.H), dtype=torch.float32, device=dev)
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if shared is not None:
        if ws is None:
            ws = layer_workspace(layer, T, k, shared=shared)
        _check(lib().moe_layer_forward_shared(ctypes.byref(layer.c()), ctypes.byref(shared.c()),
                                              _dptr(x), _dptr(logits), T, k, _dptr(ids),
                                              _dptr(w), _dptr(out), _dptr(ws), ws.numel(),
                                              _stream(dev)),
               "moe_layer_forward_shared")
        return ids, w, out
    if ws is None:
        ws = layer_workspace(layer, T, k)
    _check(lib().moe_layer_forward(ctypes.byref(layer.c()), _dptr(x), _dptr(logits), T, k,
                                   _dptr(y_shared), _dptr(ids),
                                   _dptr(w), _dptr(out), _dptr(ws), ws.numel(), _stream(dev)),
           "moe_layer_forward")
    return ids, w, out


def layer_forward_static(layer, x, logits, k, y_shared=None, out=None, ids=None, w=None):
    """moe_layer_forward_static: the whole routed layer in one C call with the
    library's own per-GPU workspace (no workspace argument; the call
    allocates nothing).  Pass preallocated out / ids / w to keep this
    function from allocating them.  Returns (topk_ids, topk_w, out)."""
    torch = _torch()
    _need_cuda(x, logits)
    T = x.shape[0]
    if tuple(logits.shape) != (T, layer.E) or logits.dtype != torch.float32:
        raise ValueError("logits must be fp32 [T, E]")
    if y_shared is not None:
        _need_cuda(y_shared)
        if tuple(y_shared.shape) != (T, layer.H) or y_shared.dtype != torch.float32:
            raise ValueError("y_shared must be fp32 [T, H]")
    dev = x.device
    if out is None:
        out = torch.empty((T, layer.H), dtype=torch.float32, device=dev)
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib().moe_layer_forward_static(ctypes.byref(layer.c()), _dptr(x), _dptr(logits), T, k,
                                          _dptr(y_shared), _dptr(ids), _dptr(w), _dptr(out),
                                          _stream(dev)),
           "moe_layer_forward_static")
    return ids, w, out


def forward(layer, x, logits, k, shared=None, overlap=False):
    """route -> permute -> expert FFN -> combine (+ the shared expert's output
    when `shared`, a one-expert QLayer, is given).  With overlap, the shared
    expert runs on side_stream(), forked from and joined back into the current
    stream (so the call stays stream-ordered and can be graph-captured), while
    the routed experts run on the current stream.  (Measured on MI355X: no
    faster in a graph, whose replay ran both branches on one queue, and slower
    eagerly, so it is off by default.)  Returns a dict of every intermediate
    (device tensors)."""
    torch = _torch()
    if shared is not None:
        main = torch.cuda.current_stream(x.device)
        y_sh = torch.empty((x.shape[0], shared.H), dtype=torch.float32, device=x.device)
        sws = shared_workspace(shared, x.shape[0])
        side = side_stream(x.device) if overlap else main
        side.wait_stream(main)
        with torch.cuda.stream(side):
            shared_ffn(shared, x, y_sh, sws)
    ids, w, counts, offsets, perm_src, inv_perm = route_permute(logits, k, layer.E)
    y_perm = expert_ffn_q(layer, x, perm_src, offsets, k)
    r = dict(topk_ids=ids, topk_w=w, counts=counts, offsets=offsets, perm_src=perm_src,
             inv_perm=inv_perm, y_perm=y_perm)
    if shared is None:
        r["out"] = combine(y_perm, inv_perm, w)
    else:
        main.wait_stream(side)
        r["y_shared"] = y_sh
        r["out"] = combine_shared(y_perm, inv_perm, w, y_sh)
    return r
