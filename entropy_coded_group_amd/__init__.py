"""Python binding of libecco, the MI355X (gfx950) Ecco block codec.

A thin ctypes layer over the C ABI declared in include/ecco.h: every function
here has the name of the C entry point it calls and only marshals arguments
(NumPy arrays and torch tensors to pointers, the current torch stream to a
hipStream_t).  All codec work runs in the library's HIP kernels; if the
shared library is missing or fails to load, every call raises.

Device buffers are torch CUDA tensors (device memory and streams are the only
things torch is used for).
"""

import ctypes
import os

import numpy as np

__all__ = [
    "EccoError", "lib", "library_path",
    "ecco_tables_size", "ecco_tables_build", "ecco_tables_validate", "ecco_tables_get",
    "ecco_train_patterns", "ecco_tensor_scale_from_amax", "ecco_amax", "ecco_amax_many", "ecco_encode",
    "ecco_decode", "ecco_decode_speculative", "ecco_decode_segmented", "ecco_encode_many", "ecco_encode_act", "ecco_decode_act",
    "ecco_decode_many",
    "ecco_decode_gemv", "ecco_decode_gemv_many", "ecco_attention_workspace_size",
    "ecco_attention_decode", "ecco_attention_decode_noalloc", "ecco_strerror", "ecco_version",
    "ATTENTION_NOALLOC_MAX_WORKSPACE",
    "STATS_FIELDS", "DECODE_MAX_JOBS", "GEMV_MAX_JOBS", "AMAX_MAX_JOBS", "tables_to_device",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libecco.so")

GROUP = 128
BLOCK_BYTES = 64
STATS_FIELDS = ("groups", "clipped_groups", "clipped_values", "padded_outliers", "pad_bits",
                "fill_bits", "nonfinite_groups")

_ERRORS = {0: "ECCO_OK", -1: "ECCO_EINVAL", -2: "ECCO_EALIGN", -3: "ECCO_ESIZE",
           -4: "ECCO_ETABLES", -5: "ECCO_EHIP", -6: "ECCO_EDEVICE"}


class EccoError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s failed: %s (%s)" % (where, _ERRORS.get(code, code), ecco_strerror(code)))


class TrainOpts(ctypes.Structure):
    _fields_ = [("kmeans_iters", ctypes.c_uint32), ("huff_iters", ctypes.c_uint32),
                ("seed", ctypes.c_uint64), ("max_groups", ctypes.c_uint32), ("threads", ctypes.c_uint32),
                ("n_patterns", ctypes.c_uint32), ("group", ctypes.c_uint32)]


DECODE_MAX_JOBS = 16
GEMV_MAX_JOBS = 16
AMAX_MAX_JOBS = 16
ATTENTION_NOALLOC_MAX_WORKSPACE = 64 << 20


class AmaxJob(ctypes.Structure):
    """ecco_amax_job_t."""
    _fields_ = [("x_dev", ctypes.c_void_p), ("n_values", ctypes.c_uint64), ("amax_dev", ctypes.c_void_p)]


class DecodeJob(ctypes.Structure):
    """ecco_decode_job_t."""
    _fields_ = [("blocks_dev", ctypes.c_void_p), ("y_dev", ctypes.c_void_p), ("tables_dev", ctypes.c_void_p),
                ("n_rows", ctypes.c_uint64), ("groups_per_row", ctypes.c_uint64),
                ("blk_row_stride_blocks", ctypes.c_uint64), ("y_row_stride_elems", ctypes.c_uint64),
                ("tensor_scale", ctypes.c_float), ("reserved", ctypes.c_uint32)]


class EncodeJob(ctypes.Structure):
    """ecco_encode_job_t."""
    _fields_ = [("x_dev", ctypes.c_void_p), ("blocks_dev", ctypes.c_void_p), ("tables_dev", ctypes.c_void_p),
                ("stats_dev", ctypes.c_void_p), ("n_rows", ctypes.c_uint64), ("groups_per_row", ctypes.c_uint64),
                ("x_row_stride_elems", ctypes.c_uint64), ("blk_row_stride_blocks", ctypes.c_uint64),
                ("tensor_scale", ctypes.c_float), ("reserved", ctypes.c_uint32)]


class GemvJob(ctypes.Structure):
    """ecco_gemv_job_t."""
    _fields_ = [("blocks_dev", ctypes.c_void_p), ("tables_dev", ctypes.c_void_p), ("x_dev", ctypes.c_void_p),
                ("y_dev", ctypes.c_void_p), ("out_features", ctypes.c_int64), ("in_features", ctypes.c_int64),
                ("tensor_scale", ctypes.c_float), ("reserved", ctypes.c_uint32)]


_lib = None


def lib():
    """The loaded libecco (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError("libecco.so is not built; run `python -m entropy_coded_group_amd.build`")
        L = ctypes.CDLL(library_path)
        vp, u64, i64, f32, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        sig = {
            "ecco_tables_size": (ctypes.c_size_t, []),
            "ecco_tables_build": (i32, [vp, vp, vp]),
            "ecco_tables_validate": (i32, [vp]),
            "ecco_tables_get": (i32, [vp, vp, vp]),
            "ecco_train_patterns": (i32, [vp, u64, vp, vp]),
            "ecco_tensor_scale_from_amax": (f32, [f32]),
            "ecco_amax": (i32, [vp, u64, vp, vp]),
            "ecco_amax_many": (i32, [vp, ctypes.c_uint32, vp]),
            "ecco_encode": (i32, [vp, u64, u64, u64, u64, vp, f32, vp, vp, vp]),
            "ecco_decode": (i32, [vp, u64, u64, u64, u64, vp, f32, vp, vp]),
            "ecco_decode_speculative": (i32, [vp, u64, u64, u64, u64, vp, f32, vp, vp]),
            "ecco_decode_segmented": (i32, [vp, u64, u64, u64, u64, vp, f32, vp, ctypes.c_uint32, vp]),
            "ecco_encode_many": (i32, [vp, ctypes.c_uint32, vp]),
            "ecco_encode_act": (i32, [vp, u64, u64, u64, u64, vp, f32, vp, vp, vp]),
            "ecco_decode_act": (i32, [vp, u64, u64, u64, u64, vp, f32, vp, vp]),
            "ecco_decode_many": (i32, [vp, ctypes.c_uint32, vp]),
            "ecco_decode_gemv": (i32, [vp, vp, f32, i64, i64, vp, i64, vp, vp]),
            "ecco_decode_gemv_many": (i32, [vp, ctypes.c_uint32, i64, vp]),
            "ecco_attention_workspace_size": (ctypes.c_size_t, [u64, u64, u64, u64]),
            "ecco_attention_decode": (i32, [vp, vp, f32, vp, vp, f32, vp, u64, u64, u64, u64, u64, f32, vp, vp,
                                            vp]),
            "ecco_attention_decode_noalloc": (i32, [vp, vp, f32, vp, vp, f32, vp, u64, u64, u64, u64, u64, f32, vp,
                                                    vp]),
            "ecco_strerror": (ctypes.c_char_p, [i32]),
            "ecco_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc, where):
    if rc != 0:
        raise EccoError(rc, where)


def _ptr(obj):
    """Address of a torch tensor's data or of a NumPy array's buffer."""
    if obj is None:
        return None
    if hasattr(obj, "data_ptr"):
        return obj.data_ptr()
    if isinstance(obj, np.ndarray):
        if not obj.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be C-contiguous")
        return obj.ctypes.data
    if isinstance(obj, int):
        return obj
    raise TypeError("expected a torch tensor, NumPy array or address, got %r" % type(obj))


def _dptr(obj, dense=False):
    """Address of a device argument: a torch tensor on the GPU (dense=True: also
    contiguous, for arguments whose layout the call fixes), or a raw address.
    Host memory handed to a kernel would fault the GPU, so it is refused here."""
    if obj is None or isinstance(obj, int):
        return obj
    if hasattr(obj, "data_ptr"):
        if not obj.is_cuda:
            raise ValueError("device argument must be a GPU tensor, got one on %s" % obj.device)
        if dense and not obj.is_contiguous():
            raise ValueError("this argument must be a contiguous tensor")
        return obj.data_ptr()
    raise TypeError("expected a GPU tensor or a device address, got %r" % type(obj))


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ----------------------------------------------------------------- tables

def ecco_tables_size():
    return int(lib().ecco_tables_size())


def ecco_tables_build(centroids, code_len):
    """centroids [64, 15] float32, code_len [64, 4, 16] uint8 -> host blob (uint8 array)."""
    c = np.ascontiguousarray(centroids, dtype=np.float32)
    l = np.ascontiguousarray(code_len, dtype=np.uint8)
    if c.shape != (64, 15) or l.shape != (64, 4, 16):
        raise ValueError("bad table shapes")
    blob = _aligned_host(ecco_tables_size())
    _check(lib().ecco_tables_build(_ptr(c), _ptr(l), _ptr(blob)), "ecco_tables_build")
    return blob


def ecco_tables_validate(blob):
    return int(lib().ecco_tables_validate(_ptr(np.ascontiguousarray(blob, dtype=np.uint8))))


def ecco_tables_get(blob):
    c = np.zeros((64, 15), np.float32)
    l = np.zeros((64, 4, 16), np.uint8)
    _check(lib().ecco_tables_get(_ptr(np.ascontiguousarray(blob, dtype=np.uint8)), _ptr(c), _ptr(l)),
           "ecco_tables_get")
    return c, l


def ecco_train_patterns(sample_fp16, kmeans_iters=25, huff_iters=10, seed=0, max_groups=0, threads=0,
                        n_patterns=0, group=0):
    """Learn a host blob from an FP16 sample (NumPy float16/uint16 or CPU torch tensor);
    n_patterns distinct patterns (16, 32 or 64; 0 = 64) repeated over the 64 slots."""
    if hasattr(sample_fp16, "numpy"):
        sample_fp16 = sample_fp16.contiguous().numpy()
    s = np.ascontiguousarray(sample_fp16).view(np.uint16).ravel()
    opts = TrainOpts(kmeans_iters, huff_iters, seed, max_groups, threads, n_patterns, group)
    blob = _aligned_host(ecco_tables_size())
    _check(lib().ecco_train_patterns(_ptr(s), s.size, ctypes.byref(opts), _ptr(blob)), "ecco_train_patterns")
    return blob


def ecco_tensor_scale_from_amax(amax):
    return float(np.float32(lib().ecco_tensor_scale_from_amax(float(amax))))


def _aligned_host(n, align=256):
    raw = np.zeros(n + align, np.uint8)
    off = (-raw.ctypes.data) % align
    return raw[off:off + n]


def tables_to_device(blob, device="cuda"):
    """Copy a host blob into a fresh device tensor (torch allocations are 256-byte aligned)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(blob, dtype=np.uint8).copy()).to(device)
    if t.data_ptr() % 256:
        raise RuntimeError("device allocation not 256-byte aligned")
    return t


# ----------------------------------------------------------------- device

def ecco_amax(x, n_values, amax_out, stream=None):
    _check(lib().ecco_amax(_dptr(x), int(n_values), _dptr(amax_out), _stream(stream)), "ecco_amax")


def ecco_amax_many(jobs, stream=None):
    """jobs: a sequence of (x, n_values, amax_out) tuples -- the arguments of
    ecco_amax, one per tensor -- reduced in one launch."""
    arr = (AmaxJob * max(1, len(jobs)))()
    for i, (x, n_values, amax_out) in enumerate(jobs):
        arr[i] = AmaxJob(_dptr(x), int(n_values), _dptr(amax_out))
    _check(lib().ecco_amax_many(ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream(stream)), "ecco_amax_many")


def ecco_encode(x, n_rows, groups_per_row, x_row_stride_elems, blk_row_stride_blocks, tables_dev,
                tensor_scale, blocks, stats=None, stream=None):
    _check(lib().ecco_encode(_dptr(x), int(n_rows), int(groups_per_row), int(x_row_stride_elems),
                             int(blk_row_stride_blocks), _dptr(tables_dev), float(tensor_scale), _dptr(blocks),
                             _dptr(stats), _stream(stream)), "ecco_encode")


def ecco_decode(blocks, n_rows, groups_per_row, blk_row_stride_blocks, y_row_stride_elems, tables_dev,
                tensor_scale, y, stream=None):
    _check(lib().ecco_decode(_dptr(blocks), int(n_rows), int(groups_per_row), int(blk_row_stride_blocks),
                             int(y_row_stride_elems), _dptr(tables_dev), float(tensor_scale), _dptr(y),
                             _stream(stream)), "ecco_decode")


def ecco_decode_speculative(blocks, n_rows, groups_per_row, blk_row_stride_blocks, y_row_stride_elems,
                            tables_dev, tensor_scale, y, stream=None):
    """ecco_decode by the speculative segment method (same output, slower)."""
    _check(lib().ecco_decode_speculative(_dptr(blocks), int(n_rows), int(groups_per_row),
                                         int(blk_row_stride_blocks), int(y_row_stride_elems), _dptr(tables_dev),
                                         float(tensor_scale), _dptr(y), _stream(stream)), "ecco_decode_speculative")


def ecco_decode_segmented(blocks, n_rows, groups_per_row, blk_row_stride_blocks, y_row_stride_elems,
                          tables_dev, tensor_scale, y, lanes_per_block, stream=None):
    """ecco_decode with 2, 4 or 8 lanes per block, each decoding a segment
    speculatively (same output, slower)."""
    _check(lib().ecco_decode_segmented(_dptr(blocks), int(n_rows), int(groups_per_row),
                                       int(blk_row_stride_blocks), int(y_row_stride_elems), _dptr(tables_dev),
                                       float(tensor_scale), _dptr(y), int(lanes_per_block), _stream(stream)),
           "ecco_decode_segmented")


def ecco_encode_many(jobs, stream=None):
    """jobs: a sequence of (x, n_rows, groups_per_row, x_row_stride_elems,
    blk_row_stride_blocks, tables_dev, tensor_scale, blocks, stats) tuples --
    the arguments of ecco_encode, one tuple per tensor -- encoded in one
    launch (stats may be None)."""
    arr = (EncodeJob * max(1, len(jobs)))()
    for i, (x, n_rows, gpr, xstride, bstride, tables_dev, t, blocks, stats) in enumerate(jobs):
        arr[i] = EncodeJob(_dptr(x), _dptr(blocks), _dptr(tables_dev), _dptr(stats), int(n_rows), int(gpr), int(xstride),
                           int(bstride), float(t), 0)
    _check(lib().ecco_encode_many(ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream(stream)),
           "ecco_encode_many")


def ecco_encode_act(x, n_rows, groups_per_row, x_row_stride_elems, blk_row_stride_blocks, tables_dev,
                    tensor_scale, blocks, stats=None, stream=None):
    """ecco_encode for the 2x activation format (groups of 64 values)."""
    _check(lib().ecco_encode_act(_dptr(x), int(n_rows), int(groups_per_row), int(x_row_stride_elems),
                                 int(blk_row_stride_blocks), _dptr(tables_dev), float(tensor_scale), _dptr(blocks),
                                 _dptr(stats), _stream(stream)), "ecco_encode_act")


def ecco_decode_act(blocks, n_rows, groups_per_row, blk_row_stride_blocks, y_row_stride_elems, tables_dev,
                    tensor_scale, y, stream=None):
    """ecco_decode for the 2x activation format (groups of 64 values)."""
    _check(lib().ecco_decode_act(_dptr(blocks), int(n_rows), int(groups_per_row), int(blk_row_stride_blocks),
                                 int(y_row_stride_elems), _dptr(tables_dev), float(tensor_scale), _dptr(y),
                                 _stream(stream)), "ecco_decode_act")


def ecco_decode_many(jobs, stream=None):
    """jobs: a sequence of (blocks, n_rows, groups_per_row, blk_row_stride_blocks,
    y_row_stride_elems, tables_dev, tensor_scale, y) tuples -- the arguments of
    ecco_decode, one tuple per tensor -- decoded in one launch."""
    arr = (DecodeJob * max(1, len(jobs)))()
    for i, (blocks, n_rows, gpr, bstride, ystride, tables_dev, t, y) in enumerate(jobs):
        arr[i] = DecodeJob(_dptr(blocks), _dptr(y), _dptr(tables_dev), int(n_rows), int(gpr), int(bstride),
                           int(ystride), float(t), 0)
    _check(lib().ecco_decode_many(ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream(stream)),
           "ecco_decode_many")


def ecco_decode_gemv(blocks, tables_dev, tensor_scale, out_features, in_features, x, batch, y, stream=None):
    _check(lib().ecco_decode_gemv(_dptr(blocks, True), _dptr(tables_dev), float(tensor_scale), int(out_features),
                                  int(in_features), _dptr(x, True), int(batch), _dptr(y, True), _stream(stream)),
           "ecco_decode_gemv")


def ecco_decode_gemv_many(jobs, batch, stream=None):
    """jobs: a sequence of (blocks, tables_dev, tensor_scale, out_features,
    in_features, x, y) tuples -- the arguments of ecco_decode_gemv, one tuple
    per matrix -- with a common batch."""
    arr = (GemvJob * max(1, len(jobs)))()
    for i, (blocks, tables_dev, t, out_f, in_f, x, y) in enumerate(jobs):
        arr[i] = GemvJob(_dptr(blocks, True), _dptr(tables_dev), _dptr(x, True), _dptr(y, True), int(out_f),
                         int(in_f), float(t), 0)
    _check(lib().ecco_decode_gemv_many(ctypes.cast(arr, ctypes.c_void_p), len(jobs), int(batch), _stream(stream)),
           "ecco_decode_gemv_many")


def ecco_attention_workspace_size(batch, kv_heads, group, seq):
    return int(lib().ecco_attention_workspace_size(int(batch), int(kv_heads), int(group), int(seq)))


def ecco_attention_decode(k_blocks, k_tables_dev, k_scale, v_blocks, v_tables_dev, v_scale, q, batch, kv_heads,
                          group, seq, kv_stride_tokens, scale, workspace, out, stream=None):
    _check(lib().ecco_attention_decode(_dptr(k_blocks), _dptr(k_tables_dev), float(k_scale), _dptr(v_blocks),
                                       _dptr(v_tables_dev), float(v_scale), _dptr(q, True), int(batch), int(kv_heads),
                                       int(group), int(seq), int(kv_stride_tokens), float(scale), _dptr(workspace),
                                       _dptr(out, True), _stream(stream)), "ecco_attention_decode")


def ecco_attention_decode_noalloc(k_blocks, k_tables_dev, k_scale, v_blocks, v_tables_dev, v_scale, q, batch,
                                  kv_heads, group, seq, kv_stride_tokens, scale, out, stream=None):
    """ecco_attention_decode with the library's own static scratch in place of
    a caller workspace (allocates nothing)."""
    _check(lib().ecco_attention_decode_noalloc(_dptr(k_blocks), _dptr(k_tables_dev), float(k_scale), _dptr(v_blocks),
                                               _dptr(v_tables_dev), float(v_scale), _dptr(q, True), int(batch),
                                               int(kv_heads), int(group), int(seq), int(kv_stride_tokens),
                                               float(scale), _dptr(out, True), _stream(stream)),
           "ecco_attention_decode_noalloc")


def ecco_strerror(code):
    return lib().ecco_strerror(int(code)).decode()


def ecco_version():
    return lib().ecco_version().decode()
