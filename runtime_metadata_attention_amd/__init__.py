"""Python binding of libcompilemask (CompileMask hot path for MI355X / gfx950).

The functions below carry the C ABI's names (include/compilemask.h) and only
marshal arguments: every step of the path runs in the library's HIP kernels.
PyTorch supplies device memory and the stream.  Importing works without a
GPU (the spec compiler and the host inspection call run on the CPU), but the
library itself must be built: there is no fallback of any kind.

    spec = cm_spec_compile(text)
    desc = Descriptor(spec, B, N, seg_cap, tiles, device)     # cm_desc_size + cm_desc_init
    # packed batches: Descriptor(spec, 1, T, seg_cap, tiles, device, packed=n_samples)
    # with metadata carrying cu_seqlens
    cm_build_descriptor(spec, device_metadata(md, device), desc)
    cm_attn_fwd(attn_args(q), q, k, v, desc, o, lse)
    cm_attn_bwd(attn_args(q), q, k, v, o, lse, do, desc, dq, dk, dv, ws)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libcompilemask.so")

CM_OK = 0
STATUS = {0: "CM_OK", -1: "CM_ERR_NULL", -2: "CM_ERR_INVALID", -3: "CM_ERR_PARSE", -4: "CM_ERR_MISMATCH",
          -5: "CM_ERR_UNSUPPORTED", -6: "CM_ERR_SIZE", -7: "CM_ERR_HIP"}
SECTIONS = ("header", "sample_err", "row_tkmax", "col_tkmax", "fbm", "bbm", "row_iv", "col_iv", "total")
# every symbol include/compilemask.h declares
EXPORTS = ("cm_spec_compile", "cm_spec_free", "cm_spec_info", "cm_spec_dump", "cm_spec_eval_host",
           "cm_spec_specialize", "cm_spec_codegen",
           "cm_desc_size", "cm_desc_init", "cm_desc_size_packed", "cm_desc_init_packed", "cm_desc_free",
           "cm_desc_offsets", "cm_build_descriptor", "cm_build_blockmask",
           "cm_attn_fwd", "cm_attn_bwd_workspace", "cm_attn_bwd", "cm_attn_bwd_stage",
           "cm_attn_bwd_noalloc", "cm_desc_download", "cm_desc_errors",
           "cm_status_str", "cm_last_error", "cm_version")


class CompileMaskError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


class cm_tiles(ctypes.Structure):
    _fields_ = [("fwd_q", ctypes.c_int32), ("fwd_k", ctypes.c_int32),
                ("bwd_k", ctypes.c_int32), ("bwd_q", ctypes.c_int32)]


class cm_metadata(ctypes.Structure):
    _fields_ = [("scalars", ctypes.c_void_p), ("seg_bounds", ctypes.c_void_p), ("n_seg", ctypes.c_void_p),
                ("refs", ctypes.c_void_p), ("n_scalars", ctypes.c_int32), ("n_refs", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p)]


class cm_attn_args(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int32), ("check", ctypes.c_int32),
                ("precision", ctypes.c_int32)]


CM_CHECK_RUN_BITS = 0
CM_CHECK_ORDINARY_MASKED = 1
CM_CHECK_PREDICATE = 2
CM_CHECK_UNSIGNED = 3
# P / dS operand precision (cm_attn_args.precision)
CM_PRECISION_BF16 = 0
CM_PRECISION_SPLIT = 1
# predicate-baseline families (cm_build_blockmask)
CM_PRED = {"causal": 0, "hstu": 1, "shared_prompt": 2, "retrieval": 3}


_lib = None


def library() -> ctypes.CDLL:
    """Load libcompilemask.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m runtime_metadata_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    sig = {
        "cm_spec_compile": (I32, [ctypes.c_char_p, P(VP)]),
        "cm_spec_free": (None, [VP]),
        "cm_spec_info": (I32, [VP, I32, P(I32), P(I32), P(I32), P(I32)]),
        "cm_spec_dump": (I32, [VP, ctypes.c_char_p, SZ, P(SZ)]),
        "cm_spec_specialize": (I32, [VP]),
        "cm_spec_codegen": (I32, [VP, ctypes.c_char_p, SZ, P(SZ)]),
        "cm_spec_eval_host": (I32, [VP, I32, I32, I32, VP, I32, VP, I32, I32, VP, I32, VP, I32, P(I32),
                                    P(ctypes.c_uint32)]),
        "cm_desc_size": (I32, [VP, I32, I32, I32, P(cm_tiles), P(SZ)]),
        "cm_desc_init": (I32, [VP, I32, I32, I32, P(cm_tiles), VP, SZ, P(VP)]),
        "cm_desc_size_packed": (I32, [VP, I32, I32, I32, P(cm_tiles), P(SZ)]),
        "cm_desc_init_packed": (I32, [VP, I32, I32, I32, P(cm_tiles), VP, SZ, P(VP)]),
        "cm_desc_free": (None, [VP]),
        "cm_desc_offsets": (I32, [VP, P(SZ)]),
        "cm_build_descriptor": (I32, [VP, P(cm_metadata), VP, VP]),
        "cm_build_blockmask": (I32, [I32, P(cm_metadata), VP, VP]),
        "cm_attn_fwd": (I32, [P(cm_attn_args), VP, VP, VP, VP, VP, VP, VP]),
        "cm_attn_bwd_workspace": (I32, [P(cm_attn_args), P(SZ)]),
        "cm_attn_bwd": (I32, [P(cm_attn_args), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]),
        "cm_attn_bwd_stage": (I32, [I32, P(cm_attn_args), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]),
        "cm_attn_bwd_noalloc": (I32, [P(cm_attn_args), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP]),
        "cm_desc_download": (I32, [VP, VP, SZ, VP]),
        "cm_desc_errors": (I32, [VP, P(ctypes.c_uint32), VP, P(I32), VP]),
        "cm_status_str": (ctypes.c_char_p, [I32]),
        "cm_last_error": (ctypes.c_char_p, []),
        "cm_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(st: int, where: str):
    if st != CM_OK:
        raise CompileMaskError(st, where, library().cm_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch

    return int(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------------ spec

class Spec:
    """Owner of a compiled cm_spec handle."""

    def __init__(self, handle: int, text: str):
        self.handle = handle
        self.text = text

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.cm_spec_free(ctypes.c_void_p(self.handle))
            self.handle = None


def cm_spec_compile(text: str) -> Spec:
    h = ctypes.c_void_p()
    _check(library().cm_spec_compile(text.encode(), ctypes.byref(h)), "cm_spec_compile")
    return Spec(h.value, text)


def cm_spec_info(spec: Spec, seg_cap: int) -> Tuple[int, int, int, int]:
    """(K_row, K_col, n_scalars, n_refs)."""
    out = [ctypes.c_int32() for _ in range(4)]
    _check(library().cm_spec_info(spec.handle, seg_cap, *[ctypes.byref(x) for x in out]), "cm_spec_info")
    return tuple(x.value for x in out)


def cm_spec_dump(spec: Spec) -> str:
    need = ctypes.c_size_t()
    _check(library().cm_spec_dump(spec.handle, None, 0, ctypes.byref(need)), "cm_spec_dump")
    buf = ctypes.create_string_buffer(need.value)
    _check(library().cm_spec_dump(spec.handle, buf, need.value, None), "cm_spec_dump")
    return buf.value.decode()


def cm_spec_codegen(spec: Spec) -> str:
    """HIP source of the spec-specialised preprocess kernel."""
    need = ctypes.c_size_t()
    _check(library().cm_spec_codegen(spec.handle, None, 0, ctypes.byref(need)), "cm_spec_codegen")
    buf = ctypes.create_string_buffer(need.value)
    _check(library().cm_spec_codegen(spec.handle, buf, need.value, None), "cm_spec_codegen")
    return buf.value.decode()


def cm_spec_specialize(spec: Spec):
    """Compile (hipRTC) and load the spec-specialised preprocess kernel on the
    current device; later cm_build_descriptor calls with this spec use it."""
    _check(library().cm_spec_specialize(spec.handle), "cm_spec_specialize")


def cm_spec_eval_host(spec: Spec, direction: int, N: int, index: int, scalars: Sequence[int],
                      seg_bounds: Sequence[int], n_seg: int, refs, n_refs: int, cap: int = 4096):
    """Visible runs of one query row (direction 0) or key column (1) of one
    sample, evaluated on the host from the lowered program.  Returns
    (list of (start, end), metadata error bits)."""
    import numpy as np

    sc = np.ascontiguousarray(np.asarray(scalars, np.int32).ravel())
    sb = np.ascontiguousarray(np.asarray(seg_bounds, np.int32).ravel())
    rf = np.ascontiguousarray(np.asarray(refs, np.int32).ravel())
    seg_cap = max(0, len(sb) - 1)
    runs = (ctypes.c_uint32 * (2 * cap))()
    n = ctypes.c_int32()
    err = ctypes.c_uint32()
    _check(library().cm_spec_eval_host(
        spec.handle, direction, N, index,
        sc.ctypes.data if sc.size else None, len(sc),
        sb.ctypes.data if sb.size else None, n_seg, seg_cap,
        rf.ctypes.data if rf.size else None, n_refs,
        runs, cap, ctypes.byref(n), ctypes.byref(err)), "cm_spec_eval_host")
    return [(runs[2 * q], runs[2 * q + 1]) for q in range(n.value)], err.value


# ------------------------------------------------------------------ descriptor

def make_tiles(tiles) -> cm_tiles:
    if isinstance(tiles, cm_tiles):
        return tiles
    return cm_tiles(*[int(x) for x in tiles])


def cm_desc_size(spec: Spec, B: int, N: int, seg_cap: int, tiles) -> int:
    out = ctypes.c_size_t()
    _check(library().cm_desc_size(spec.handle, B, N, seg_cap, ctypes.byref(make_tiles(tiles)), ctypes.byref(out)),
           "cm_desc_size")
    return out.value


def cm_desc_size_packed(spec: Spec, n_samples: int, T: int, seg_cap: int, tiles) -> int:
    out = ctypes.c_size_t()
    _check(library().cm_desc_size_packed(spec.handle, n_samples, T, seg_cap, ctypes.byref(make_tiles(tiles)),
                                         ctypes.byref(out)), "cm_desc_size_packed")
    return out.value


class Descriptor:
    """A cm_desc handle over a torch uint8 device buffer it keeps alive.

    With packed=n_samples (> 0) the descriptor covers one packed sequence of N
    tokens holding n_samples samples (cm_desc_init_packed); B must then be 1."""

    def __init__(self, spec: Spec, B: int, N: int, seg_cap: int, tiles, device=None, buffer=None, packed: int = 0):
        import torch

        self.spec = spec
        self.B, self.N, self.seg_cap, self.packed = B, N, seg_cap, int(packed)
        if self.packed and B != 1:
            raise ValueError("a packed descriptor covers one sequence: B must be 1")
        self.tiles = tuple(int(x) for x in (tiles if not isinstance(tiles, cm_tiles) else
                                            (tiles.fwd_q, tiles.fwd_k, tiles.bwd_k, tiles.bwd_q)))
        if self.packed:
            self.bytes = cm_desc_size_packed(spec, self.packed, N, seg_cap, self.tiles)
        else:
            self.bytes = cm_desc_size(spec, B, N, seg_cap, self.tiles)
        if buffer is None:
            buffer = torch.empty(self.bytes, dtype=torch.uint8, device=device or "cuda")
        self.buffer = buffer
        h = ctypes.c_void_p()
        if self.packed:
            _check(library().cm_desc_init_packed(spec.handle, self.packed, N, seg_cap,
                                                 ctypes.byref(make_tiles(self.tiles)), ctypes.c_void_p(_ptr(buffer)),
                                                 buffer.numel() * buffer.element_size(), ctypes.byref(h)),
                   "cm_desc_init_packed")
        else:
            _check(library().cm_desc_init(spec.handle, B, N, seg_cap, ctypes.byref(make_tiles(self.tiles)),
                                          ctypes.c_void_p(_ptr(buffer)), buffer.numel() * buffer.element_size(),
                                          ctypes.byref(h)), "cm_desc_init")
        self.handle = h.value
        K = cm_spec_info(spec, seg_cap)
        self.K_r, self.K_c = K[0], K[1]

    def offsets(self):
        return cm_desc_offsets(self)

    def words(self):
        """The descriptor as a host numpy uint32 array (synchronises)."""
        return self.buffer[: self.bytes].view(__import__("torch").int32).cpu().numpy().view("uint32")

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.cm_desc_free(ctypes.c_void_p(self.handle))
            self.handle = None


def cm_desc_download(desc: Descriptor, stream=None):
    """The whole descriptor as a host numpy uint32 array (synchronises)."""
    import numpy as np

    out = np.zeros(desc.bytes // 4, np.uint32)
    _check(library().cm_desc_download(desc.handle, out.ctypes.data, out.nbytes, _stream(stream)), "cm_desc_download")
    return out


def cm_desc_errors(desc: Descriptor, stream=None):
    """(OR of every sample's metadata-error bits, per-sample list); synchronises."""
    n = desc.packed if desc.packed else desc.B
    per = (ctypes.c_uint32 * max(1, n))()
    flags, cnt = ctypes.c_uint32(), ctypes.c_int32()
    _check(library().cm_desc_errors(desc.handle, ctypes.byref(flags), per, ctypes.byref(cnt), _stream(stream)),
           "cm_desc_errors")
    return flags.value, [per[i] for i in range(cnt.value)]


def cm_desc_offsets(desc: Descriptor):
    out = (ctypes.c_size_t * 9)()
    _check(library().cm_desc_offsets(desc.handle, out), "cm_desc_offsets")
    return dict(zip(SECTIONS, list(out)))


class DeviceMetadata:
    """Device int32 copies of a metadata object (scalars, seg_bounds, n_seg, refs)."""

    def __init__(self, md, device="cuda"):
        import torch

        def up(a):
            t = torch.as_tensor(a).to(torch.int32).contiguous()
            return t.to(device) if t.numel() else None

        self.scalars = up(md.scalars)
        self.seg_bounds = up(md.seg_bounds)
        self.n_seg = up(md.n_seg)
        self.refs = up(md.refs)
        self.n_scalars = int(md.scalars.shape[1])
        self.n_refs = int(md.refs.shape[2]) if md.refs.ndim == 3 else 0
        cu = getattr(md, "cu_seqlens", None)
        self.cu_seqlens = None if cu is None else up(cu)

    def struct(self) -> cm_metadata:
        return cm_metadata(_ptr(self.scalars), _ptr(self.seg_bounds), _ptr(self.n_seg), _ptr(self.refs),
                           self.n_scalars, self.n_refs, _ptr(self.cu_seqlens))


def device_metadata(md, device="cuda") -> DeviceMetadata:
    return DeviceMetadata(md, device)


def cm_build_blockmask(family, md: DeviceMetadata, desc: Descriptor, stream=None):
    """Predicate baseline: build desc's tile bitmaps by evaluating the family's
    predicate at every element (family: a CM_PRED name or id).  md must stay
    alive until the attention calls (check=CM_CHECK_PREDICATE) have run."""
    fam = CM_PRED[family] if isinstance(family, str) else int(family)
    m = md.struct()
    _check(library().cm_build_blockmask(fam, ctypes.byref(m), desc.handle, _stream(stream)), "cm_build_blockmask")
    desc.pred_md = md  # keep the metadata the descriptor now refers to alive


def cm_build_descriptor(spec: Spec, md: DeviceMetadata, desc: Descriptor, stream=None):
    m = md.struct()
    _check(library().cm_build_descriptor(spec.handle, ctypes.byref(m), desc.handle, _stream(stream)),
           "cm_build_descriptor")


# ------------------------------------------------------------------ attention

def attn_args(q, causal: bool = False, scale: float = 0.0, check: int = CM_CHECK_RUN_BITS,
              precision: int = CM_PRECISION_BF16) -> cm_attn_args:
    """cm_attn_args from a [B, H, N, d] bf16 tensor's shape and strides; `check` selects the partial-tile
    visibility check (CM_CHECK_UNSIGNED and CM_CHECK_ORDINARY_MASKED are the ablation kernels) and
    `precision` the P / dS operand precision (CM_PRECISION_SPLIT: hi + lo bf16 pairs)."""
    B, H, N, d = q.shape
    sb, sh, sn, sd = q.stride()
    if sd != 1:
        raise ValueError("the last dimension must be contiguous")
    return cm_attn_args(B, H, N, d, sb, sh, sn, float(scale), 1 if causal else 0, int(check), int(precision))


def _desc_handle(desc):
    return None if desc is None else desc.handle


def _check_tensors(where: str, args: cm_attn_args, q, lse, **others):
    """The C ABI applies args' shape and strides to every bf16 tensor: check
    that q matches args and that each other tensor has q's shape, strides,
    dtype and device, and lse is a contiguous fp32 [B, H, N] tensor there."""
    import torch

    def bad(msg):
        raise ValueError(f"{where}: {msg}")

    shape = (args.B, args.H, args.N, args.d)
    if tuple(q.shape) != shape:
        bad(f"q has shape {tuple(q.shape)}, args say {shape}")
    if q.dtype != torch.bfloat16:
        bad(f"q must be bfloat16, not {q.dtype}")
    if (args.stride_b, args.stride_h, args.stride_n) != (0, 0, 0) and \
            tuple(q.stride()[:3]) != (args.stride_b, args.stride_h, args.stride_n):
        bad(f"q has strides {q.stride()}, args say {(args.stride_b, args.stride_h, args.stride_n, 1)}")
    if q.stride()[3] != 1:
        bad("the last dimension of q must be contiguous")
    for name, t in others.items():
        if t is None:
            continue
        if tuple(t.shape) != tuple(q.shape):
            bad(f"{name} has shape {tuple(t.shape)}, q has {tuple(q.shape)}")
        if t.dtype != torch.bfloat16:
            bad(f"{name} must be bfloat16, not {t.dtype}")
        if t.stride() != q.stride():
            bad(f"{name} has strides {t.stride()}, q has {q.stride()} (the kernels apply q's strides to every tensor)")
        if t.device != q.device:
            bad(f"{name} is on {t.device}, q on {q.device}")
    if lse is not None:
        if tuple(lse.shape) != shape[:3] or lse.dtype != torch.float32 or not lse.is_contiguous():
            bad(f"lse must be a contiguous float32 tensor of shape {shape[:3]}, not {lse.dtype} {tuple(lse.shape)}")
        if lse.device != q.device:
            bad(f"lse is on {lse.device}, q on {q.device}")
    if not q.is_cuda:
        bad("tensors must be on the GPU")


def cm_attn_fwd(args: cm_attn_args, q, k, v, desc, o, lse, stream=None):
    _check_tensors("cm_attn_fwd", args, q, lse, k=k, v=v, o=o)
    _check(library().cm_attn_fwd(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _desc_handle(desc), _ptr(o),
                                 _ptr(lse), _stream(stream)), "cm_attn_fwd")


def cm_attn_bwd_workspace(args: cm_attn_args) -> int:
    out = ctypes.c_size_t()
    _check(library().cm_attn_bwd_workspace(ctypes.byref(args), ctypes.byref(out)), "cm_attn_bwd_workspace")
    return out.value


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_workspace(where, args, workspace):
    import torch

    if workspace.dtype != torch.float32 or not workspace.is_contiguous():
        raise ValueError(f"{where}: the workspace must be a contiguous float32 tensor")


def cm_attn_bwd(args: cm_attn_args, q, k, v, o, lse, do, desc, dq, dk, dv, workspace, stream=None):
    _check_workspace("cm_attn_bwd", args, workspace)
    _check_tensors("cm_attn_bwd", args, q, lse, k=k, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv)
    _check(library().cm_attn_bwd(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                 _desc_handle(desc), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                 _nbytes(workspace), _stream(stream)), "cm_attn_bwd")


def cm_attn_bwd_stage(stage: int, args: cm_attn_args, q, k, v, o, lse, do, desc, dq, dk, dv, workspace, stream=None):
    _check_workspace("cm_attn_bwd_stage", args, workspace)
    _check_tensors("cm_attn_bwd_stage", args, q, lse, k=k, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv)
    _check(library().cm_attn_bwd_stage(stage, ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       _ptr(do), _desc_handle(desc), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                       _nbytes(workspace), _stream(stream)), "cm_attn_bwd_stage")


CM_NOALLOC_MAX_ROWS = 1 << 21


def cm_attn_bwd_noalloc(args: cm_attn_args, q, k, v, o, lse, do, desc, dq, dk, dv, stream=None):
    """cm_attn_bwd with the library's fixed per-GPU workspace (no workspace
    argument; at most CM_NOALLOC_MAX_ROWS rows B * H * N per call)."""
    _check_tensors("cm_attn_bwd_noalloc", args, q, lse, k=k, v=v, o=o, do=do, dq=dq, dk=dk, dv=dv)
    _check(library().cm_attn_bwd_noalloc(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                         _desc_handle(desc), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)),
           "cm_attn_bwd_noalloc")


def cm_status_str(status: int) -> str:
    return library().cm_status_str(status).decode()


def cm_last_error() -> str:
    return library().cm_last_error().decode()


def cm_version() -> str:
    return library().cm_version().decode()


from . import specs  # noqa: E402,F401
