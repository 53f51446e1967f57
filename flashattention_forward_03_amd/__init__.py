"""Python binding of the gfx950 exact-attention library (``libfa_mi355x.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/fa.h``.  PyTorch provides
device memory and the current stream.  There is no CPU path: if the library
is missing or no GPU is present, calls raise.

Two layers:
  * ``fa_fwd``, ``fa_fwd_gqa``, ``fa_fwd_ex``, ``fa_bwd``, ``fa_decode_paged``,
    ``fa_decode_paged_gqa``, ``fa_decode_workspace_bytes``, ``fa_status_str``,
    ``fa_last_hip_error``: the C entry points with the same names and
    arguments (raw device addresses as ints, stream as int, strides as
    3-tuples or None).
  * ``Pager``: the host page allocator.
  * ``forward`` / ``backward`` / ``decode_paged`` / ``kv_append``: take torch tensors, check them, allocate
    the outputs (and the decode workspace), call the entry point on the
    current stream and raise ``FAError`` on a non-zero status.  The number
    of K/V heads is read from k (or the pools); fewer K/V heads than query
    heads go to the ``_gqa`` entry point; non-contiguous tensors (any strides
    with the head dim contiguous, e.g. a [B, N, H, d] buffer viewed as
    [B, H, N, d]) or a 16-bit O go to ``fa_fwd_ex``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_MI355X_LIB names another build of the library to load instead (the
# host-sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("FA_MI355X_LIB") or os.path.join(_HERE, "libfa_mi355x.so")

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_UNSUPPORTED = 3
FA_ERR_ALIGN = 4
FA_ERR_WORKSPACE = 5
FA_ERR_HIP = 6
FA_ERR_ARG = 7
FA_ERR_NOMEM = 8
FA_ERR_SCRATCH = 9
FA_DTYPE_F16 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F32 = 2

EXPORTED = ("fa_fwd", "fa_fwd_gqa", "fa_fwd_ex", "fa_bwd", "fa_decode_paged", "fa_decode_paged_gqa",
            "fa_decode_paged_noalloc",
            "fa_kv_append", "fa_pager_create", "fa_pager_destroy", "fa_pager_reserve",
            "fa_pager_release", "fa_pager_length", "fa_pager_free_pages", "fa_pager_copy_table",
            "fa_decode_workspace_bytes", "fa_ln_stats", "fa_ln_fold_weights", "fa_ln_linear",
            "fa_linear", "fa_prenorm_attention_workspace_bytes", "fa_prenorm_attention",
            "fa_status_str", "fa_last_hip_error", "fa_version")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: status {status} ({fa_status_str(status)})"
        if status == FA_ERR_HIP:
            msg += f", hipError {fa_last_hip_error()}"
        super().__init__(msg)
        self.status = status


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def load_library():
    """Load ``libfa_mi355x.so`` (built by ``flashattention_forward_03_amd.build``).

    torch is imported first when it is installed: torch ships its own HIP
    runtime, and the library must bind to that same runtime (loaded first,
    the library would pull in a second HIP/HSA runtime and the process would
    hold two).  Raises if two HIP runtimes end up mapped.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m flashattention_forward_03_amd.build")
    try:
        import torch  # noqa: F401  (binds the process to torch's HIP runtime first)
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process: " + ", ".join(runtimes))
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, I, P]
    lib.fa_fwd.restype = I
    lib.fa_fwd_gqa.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, P, I, P]
    lib.fa_fwd_gqa.restype = I
    S3 = ctypes.POINTER(ctypes.c_int64)
    lib.fa_fwd_ex.argtypes = [P, P, P, P, P, I, I, I, I, I, I, S3, S3, S3, S3, F, I, P, I, I, P]
    lib.fa_fwd_ex.restype = I
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, I, P]
    lib.fa_bwd.restype = I
    lib.fa_kv_append.argtypes = [P, P, P, P, I, P, P, P, I, I, I, I, I, I, I, P]
    lib.fa_kv_append.restype = I
    lib.fa_pager_create.argtypes = [I, I, I]
    lib.fa_pager_create.restype = P
    lib.fa_pager_destroy.argtypes = [P]
    lib.fa_pager_destroy.restype = None
    lib.fa_pager_reserve.argtypes = [P, I, I]
    lib.fa_pager_reserve.restype = I
    lib.fa_pager_release.argtypes = [P, I]
    lib.fa_pager_release.restype = I
    lib.fa_pager_length.argtypes = [P, I]
    lib.fa_pager_length.restype = I
    lib.fa_pager_free_pages.argtypes = [P]
    lib.fa_pager_free_pages.restype = I
    lib.fa_pager_copy_table.argtypes = [P, P, Z]
    lib.fa_pager_copy_table.restype = I
    lib.fa_decode_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, Z, P]
    lib.fa_decode_paged.restype = I
    lib.fa_decode_paged_gqa.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, Z, P]
    lib.fa_decode_paged_gqa.restype = I
    lib.fa_decode_paged_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.fa_decode_paged_noalloc.restype = I
    lib.fa_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_decode_workspace_bytes.restype = Z
    lib.fa_ln_stats.argtypes = [P, P, P, I, I, F, I, P]
    lib.fa_ln_stats.restype = I
    lib.fa_ln_fold_weights.argtypes = [P, P, P, P, P, P, P, I, I, I, P]
    lib.fa_ln_fold_weights.restype = I
    lib.fa_ln_linear.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P]
    lib.fa_ln_linear.restype = I
    lib.fa_linear.argtypes = [P, P, P, P, P, I, I, I, I, P]
    lib.fa_linear.restype = I
    lib.fa_prenorm_attention_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_prenorm_attention_workspace_bytes.restype = Z
    lib.fa_prenorm_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, F, I, P, I, P, Z,
                                         P]
    lib.fa_prenorm_attention.restype = I
    lib.fa_status_str.argtypes = [I]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = I
    lib.fa_version.argtypes = []
    lib.fa_version.restype = I
    _lib = lib
    return lib


# ------------------------------------------------------------ C entry points

def fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_lens, dtype, stream) -> int:
    return load_library().fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_lens, dtype,
                                 stream)


def fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, kv_lens, dtype,
               stream) -> int:
    return load_library().fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal,
                                     kv_lens, dtype, stream)


def _strides3(st):
    if st is None:
        return None
    arr = (ctypes.c_int64 * 3)(*[int(x) for x in st])
    return arr


def fa_fwd_ex(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, q_strides, k_strides, v_strides, o_strides,
              scale, causal, kv_lens, dtype, o_dtype, stream) -> int:
    return load_library().fa_fwd_ex(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, _strides3(q_strides),
                                    _strides3(k_strides), _strides3(v_strides),
                                    _strides3(o_strides), scale, causal, kv_lens, dtype, o_dtype,
                                    stream)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H_kv, Nq, Nk, d, scale, causal,
           kv_lens, dtype, stream) -> int:
    return load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H_kv, Nq, Nk, d,
                                 scale, causal, kv_lens, dtype, stream)


def fa_kv_append(k_new, v_new, seq_ids, positions, T, k_pages, v_pages, page_table, S, H_kv, d,
                 page_size, max_pages_per_seq, num_pages, dtype, stream) -> int:
    return load_library().fa_kv_append(k_new, v_new, seq_ids, positions, T, k_pages, v_pages,
                                       page_table, S, H_kv, d, page_size, max_pages_per_seq,
                                       num_pages, dtype, stream)


def fa_pager_create(num_pages, max_seqs, max_pages_per_seq):
    return load_library().fa_pager_create(num_pages, max_seqs, max_pages_per_seq)


def fa_pager_destroy(p) -> None:
    load_library().fa_pager_destroy(p)


def fa_pager_reserve(p, seq, length) -> int:
    return load_library().fa_pager_reserve(p, seq, length)


def fa_pager_release(p, seq) -> int:
    return load_library().fa_pager_release(p, seq)


def fa_pager_length(p, seq) -> int:
    return load_library().fa_pager_length(p, seq)


def fa_pager_free_pages(p) -> int:
    return load_library().fa_pager_free_pages(p)


def fa_pager_copy_table(p, dst, dst_entries) -> int:
    return load_library().fa_pager_copy_table(p, dst, dst_entries)


def fa_decode_paged(q, k_pages, v_pages, page_table, kv_lens, o, lse, S, H, d, page_size,
                    max_pages_per_seq, num_pages, scale, dtype, workspace, workspace_bytes,
                    stream) -> int:
    return load_library().fa_decode_paged(q, k_pages, v_pages, page_table, kv_lens, o, lse, S, H,
                                          d, page_size, max_pages_per_seq, num_pages, scale,
                                          dtype, workspace, workspace_bytes, stream)


def fa_decode_paged_gqa(q, k_pages, v_pages, page_table, kv_lens, o, lse, S, H, H_kv, d,
                        page_size, max_pages_per_seq, num_pages, scale, dtype, workspace,
                        workspace_bytes, stream) -> int:
    return load_library().fa_decode_paged_gqa(q, k_pages, v_pages, page_table, kv_lens, o, lse,
                                              S, H, H_kv, d, page_size, max_pages_per_seq,
                                              num_pages, scale, dtype, workspace,
                                              workspace_bytes, stream)


def fa_decode_paged_noalloc(q, k_pages, v_pages, page_table, kv_lens, o, lse, S, H, H_kv, d,
                            page_size, max_pages_per_seq, num_pages, scale, dtype, stream) -> int:
    return load_library().fa_decode_paged_noalloc(q, k_pages, v_pages, page_table, kv_lens, o,
                                                  lse, S, H, H_kv, d, page_size,
                                                  max_pages_per_seq, num_pages, scale, dtype,
                                                  stream)


def fa_decode_workspace_bytes(S, H, d, max_pages_per_seq, page_size) -> int:
    return int(load_library().fa_decode_workspace_bytes(S, H, d, max_pages_per_seq, page_size))


def fa_ln_stats(x, mean, rstd, T, C, eps, dtype, stream) -> int:
    return load_library().fa_ln_stats(x, mean, rstd, T, C, eps, dtype, stream)


def fa_ln_fold_weights(gamma, beta, w, bias, w_folded, bias_folded, colsum, N, C, dtype,
                       stream) -> int:
    return load_library().fa_ln_fold_weights(gamma, beta, w, bias, w_folded, bias_folded, colsum,
                                             N, C, dtype, stream)


def fa_ln_linear(x, mean, rstd, w_folded, bias_folded, colsum, y, T, C, N, dtype, stream) -> int:
    return load_library().fa_ln_linear(x, mean, rstd, w_folded, bias_folded, colsum, y, T, C, N,
                                       dtype, stream)


def fa_linear(a, w, bias, residual, y, M, K, N, dtype, stream) -> int:
    return load_library().fa_linear(a, w, bias, residual, y, M, K, N, dtype, stream)


def fa_prenorm_attention_workspace_bytes(B, N, H, H_kv, d) -> int:
    return load_library().fa_prenorm_attention_workspace_bytes(B, N, H, H_kv, d)


def fa_prenorm_attention(x, w_qkv_folded, b_qkv_folded, colsum_qkv, w_o, b_o, y, B, N, H, H_kv, d,
                         eps, scale, causal, kv_lens, dtype, workspace, workspace_bytes,
                         stream) -> int:
    return load_library().fa_prenorm_attention(x, w_qkv_folded, b_qkv_folded, colsum_qkv, w_o, b_o,
                                               y, B, N, H, H_kv, d, eps, scale, causal, kv_lens,
                                               dtype, workspace, workspace_bytes, stream)


def fa_status_str(status: int) -> str:
    return load_library().fa_status_str(status).decode()


def fa_last_hip_error() -> int:
    return int(load_library().fa_last_hip_error())


# ------------------------------------------------------------ torch wrappers

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return FA_DTYPE_F16
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")


def _check_dev(name, t, contiguous=True):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (this library has no CPU path)")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not contiguous and t.dim() > 0 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")


def _stream_handle(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def forward(q, k, v, *, scale: Optional[float] = None, causal: bool = False,
            kv_lens=None, stream=None, out=None, out_dtype=None):
    """Exact attention forward: q [B, H, Nq, d], k/v [B, H_kv, Nk, d] f16/bf16
    (H a multiple of H_kv; query head h reads K/V head h // (H // H_kv)).
    The tensors may be strided views (head dim contiguous).

    Returns ``(o, lse)``: o [B, H, Nq, d] in ``out_dtype`` (float32 by
    default, or float16 / bfloat16), lse float32 [B, H, Nq].  ``out``: an
    (o, lse) pair to write into; o may be a strided view, lse contiguous.
    ``kv_lens``: optional int32 GPU tensor [B] of valid key counts.
    """
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_kv, Nk, d] matching q")
    if Hkv < 1 or H % Hkv:
        raise ValueError("the query heads must be a multiple of the K/V heads")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, contiguous=False)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl_ptr = None
    if kv_lens is not None:
        _check_dev("kv_lens", kv_lens)
        if kv_lens.dtype != torch.int32 or tuple(kv_lens.shape) != (B,):
            raise ValueError("kv_lens must be int32 [B]")
        kl_ptr = kv_lens.data_ptr()
    if out is None:
        odt = torch.float32 if out_dtype is None else out_dtype
        o = torch.empty((B, H, Nq, d), dtype=odt, device=q.device)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if out_dtype is not None and o.dtype != out_dtype:
            raise TypeError("out[0] does not have out_dtype")
    if tuple(o.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("out must be (o [B, H, Nq, d], lse [B, H, Nq])")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32")
    _check_dev("o", o, contiguous=False)
    odc = {torch.float32: FA_DTYPE_F32, torch.float16: FA_DTYPE_F16,
           torch.bfloat16: FA_DTYPE_BF16}.get(o.dtype)
    if odc is None:
        raise TypeError(f"o must be float32, float16 or bfloat16, got {o.dtype}")
    plain = (odc == FA_DTYPE_F32 and all(t.is_contiguous() for t in (q, k, v, o)))
    if plain and Hkv == H:
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                    Nq, Nk, d, float(scale), int(bool(causal)), kl_ptr, dt, _stream_handle(stream))
        name = "fa_fwd"
    elif plain:
        st = fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B,
                        H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), kl_ptr, dt,
                        _stream_handle(stream))
        name = "fa_fwd_gqa"
    else:
        st = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                       Hkv, Nq, Nk, d, q.stride()[:3], k.stride()[:3], v.stride()[:3],
                       o.stride()[:3], float(scale), int(bool(causal)), kl_ptr, dt, odc,
                       _stream_handle(stream))
        name = "fa_fwd_ex"
    if st != FA_OK:
        raise FAError(st, name)
    return o, lse


def backward(q, k, v, o, lse, dout, *, scale: Optional[float] = None, causal: bool = False,
             kv_lens=None, stream=None, out=None):
    """Gradients of the forward: q, dout [B, H, Nq, d]; k, v [B, H_kv, Nk, d]
    (f16/bf16, contiguous); o [B, H, Nq, d] and lse [B, H, Nq] float32 from
    the forward on the same inputs.  Returns (dq, dk, dv) float32 (dk, dv
    summed over the query heads sharing a K/V head) and the row term delta
    [B, H, Nq] (D = dO . O, a view of the [2, B, H, Nq] scratch the library
    fills; ``out`` supplies dq, dk, dv and that scratch).
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        _check_dev(name, t)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("k, v must be [B, H_kv, Nk, d] and dout [B, H, Nq, d]")
    if Hkv < 1 or H % Hkv:
        raise ValueError("the query heads must be a multiple of the K/V heads")
    if o.dtype != torch.float32 or tuple(o.shape) != (B, H, Nq, d):
        raise ValueError("o must be float32 [B, H, Nq, d]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be float32 [B, H, Nq]")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype:
        raise TypeError("q, k, v, dout must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl_ptr = None
    if kv_lens is not None:
        _check_dev("kv_lens", kv_lens)
        if kv_lens.dtype != torch.int32 or tuple(kv_lens.shape) != (B,):
            raise ValueError("kv_lens must be int32 [B]")
        kl_ptr = kv_lens.data_ptr()
    if out is None:
        dq = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
        dk = torch.empty((B, Hkv, Nk, d), dtype=torch.float32, device=q.device)
        dv = torch.empty_like(dk)
        delta = torch.empty((2, B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv, delta = out
        if tuple(delta.shape) != (2, B, H, Nq) or delta.dtype != torch.float32 or not delta.is_contiguous():
            raise ValueError("out[3] (the row-term scratch) must be contiguous float32 [2, B, H, Nq]")
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B,
                H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), kl_ptr, dt,
                _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv, delta[0]


class Pager:
    """Host page allocator of a paged KV cache (wraps ``fa_pager_*``): 16-token
    pages handed to sequences from a free list, a page table [max_seqs,
    max_pages] (-1 unused) to copy to the device."""

    def __init__(self, num_pages: int, max_seqs: int, max_pages_per_seq: int):
        self._p = fa_pager_create(num_pages, max_seqs, max_pages_per_seq)
        if not self._p:
            raise ValueError("fa_pager_create failed (sizes)")
        self.num_pages, self.max_seqs, self.max_pages = num_pages, max_seqs, max_pages_per_seq

    def close(self):
        if self._p:
            fa_pager_destroy(self._p)
            self._p = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reserve(self, seq: int, length: int) -> None:
        st = fa_pager_reserve(self._p, seq, length)
        if st != FA_OK:
            raise FAError(st, "fa_pager_reserve")

    def release(self, seq: int) -> None:
        st = fa_pager_release(self._p, seq)
        if st != FA_OK:
            raise FAError(st, "fa_pager_release")

    def length(self, seq: int) -> int:
        return fa_pager_length(self._p, seq)

    def free_pages(self) -> int:
        return fa_pager_free_pages(self._p)

    def table(self):
        import numpy as np

        out = np.empty((self.max_seqs, self.max_pages), dtype=np.int32)
        st = fa_pager_copy_table(self._p, out.ctypes.data, out.size)
        if st != FA_OK:
            raise FAError(st, "fa_pager_copy_table")
        return out


def kv_append(k_new, v_new, seq_ids, positions, k_pages, v_pages, page_table, *, stream=None):
    """Write new tokens' K/V rows [T, H_kv, d] into the pools [num_pages, H_kv,
    16, d] at page_table[seq][pos // 16], row pos % 16 (int32 GPU tensors
    seq_ids [T], positions [T], page_table [S, max_pages])."""
    torch = _torch()
    for name, t in (("k_new", k_new), ("v_new", v_new), ("seq_ids", seq_ids),
                    ("positions", positions), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("page_table", page_table)):
        _check_dev(name, t)
    T, Hkv, d = k_new.shape
    num_pages, Hp, page_size, dp = k_pages.shape
    if v_new.shape != k_new.shape or v_pages.shape != k_pages.shape or (Hp, dp) != (Hkv, d):
        raise ValueError("k_new/v_new [T, H_kv, d] and pools [num_pages, H_kv, 16, d] must match")
    for name, t in (("seq_ids", seq_ids), ("positions", positions)):
        if t.dtype != torch.int32 or tuple(t.shape) != (T,):
            raise ValueError(f"{name} must be int32 [T]")
    if page_table.dtype != torch.int32 or page_table.dim() != 2:
        raise ValueError("page_table must be int32 [S, max_pages]")
    dt = _dtype_code(k_new)
    if v_new.dtype != k_new.dtype or k_pages.dtype != k_new.dtype or v_pages.dtype != k_new.dtype:
        raise TypeError("new rows and pools must share one dtype")
    S, max_pages = page_table.shape
    st = fa_kv_append(k_new.data_ptr(), v_new.data_ptr(), seq_ids.data_ptr(),
                      positions.data_ptr(), T, k_pages.data_ptr(), v_pages.data_ptr(),
                      page_table.data_ptr(), S, Hkv, d, page_size, max_pages, num_pages, dt,
                      _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_kv_append")


def decode_paged(q, k_pages, v_pages, page_table, kv_lens, *, scale: Optional[float] = None,
                 workspace=None, stream=None, out=None):
    """Decode attention: q [S, H, d], pools [num_pages, H_kv, page_size, d] (H a
    multiple of H_kv), page_table int32 [S, max_pages], kv_lens int32 [S].
    Returns (o, lse)."""
    torch = _torch()
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("page_table", page_table), ("kv_lens", kv_lens)):
        _check_dev(name, t)
    S, H, d = q.shape
    num_pages, Hkv, page_size, dp = k_pages.shape
    if dp != d or v_pages.shape != k_pages.shape:
        raise ValueError("pools must be [num_pages, H_kv, page_size, d] matching q")
    if Hkv < 1 or H % Hkv:
        raise ValueError("the query heads must be a multiple of the K/V heads")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.shape[0] != S:
        raise ValueError("page_table must be int32 [S, max_pages]")
    if kv_lens.dtype != torch.int32 or tuple(kv_lens.shape) != (S,):
        raise ValueError("kv_lens must be int32 [S]")
    dt = _dtype_code(q)
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q and the pools must share one dtype")
    max_pages = page_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_decode_workspace_bytes(S, H, d, max_pages, page_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if out is None:
        o = torch.empty((S, H, d), dtype=torch.float32, device=q.device)
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    if Hkv == H:
        st = fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                             page_table.data_ptr(), kv_lens.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), S, H, d, page_size, max_pages, num_pages,
                             float(scale), dt, ws_ptr, ws_bytes, _stream_handle(stream))
    else:
        st = fa_decode_paged_gqa(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                 page_table.data_ptr(), kv_lens.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), S, H, Hkv, d, page_size, max_pages, num_pages,
                                 float(scale), dt, ws_ptr, ws_bytes, _stream_handle(stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_paged" if Hkv == H else "fa_decode_paged_gqa")
    return o, lse


# ------------------------------------------------------ pre-LN block wrappers

def _f32_vec(name, t, n):
    torch = _torch()
    _check_dev(name, t)
    if t.dtype != torch.float32 or tuple(t.shape) != (n,):
        raise ValueError(f"{name} must be float32 [{n}]")
    return t.data_ptr()


def _mat16(name, t, shape):
    _check_dev(name, t)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    return t.data_ptr()


def _call(name, st):
    if st != FA_OK:
        raise FAError(st, name)


def ln_stats(x, eps: float = 1e-5, *, stream=None):
    """Per-row mean and 1/sqrt(var + eps) (fp32 [T]) of x [T, C] f16/bf16."""
    torch = _torch()
    T, C = x.shape
    dt = _dtype_code(x)
    _mat16("x", x, (T, C))
    mean = torch.empty(T, dtype=torch.float32, device=x.device)
    rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _call("fa_ln_stats", fa_ln_stats(x.data_ptr(), mean.data_ptr(), rstd.data_ptr(), T, C,
                                     float(eps), dt, _stream_handle(stream)))
    return mean, rstd


def ln_fold_weights(gamma, beta, w, bias=None, *, stream=None):
    """Fold LayerNorm's gamma and beta into a dense layer w [N, C]: returns
    (w_folded [N, C] in w's dtype, bias_folded fp32 [N], colsum fp32 [N])."""
    torch = _torch()
    N, C = w.shape
    dt = _dtype_code(w)
    _mat16("w", w, (N, C))
    g = _f32_vec("gamma", gamma, C)
    b = _f32_vec("beta", beta, C)
    bp = None if bias is None else _f32_vec("bias", bias, N)
    wf = torch.empty_like(w)
    bf = torch.empty(N, dtype=torch.float32, device=w.device)
    cs = torch.empty(N, dtype=torch.float32, device=w.device)
    _call("fa_ln_fold_weights", fa_ln_fold_weights(g, b, w.data_ptr(), bp, wf.data_ptr(),
                                                   bf.data_ptr(), cs.data_ptr(), N, C, dt,
                                                   _stream_handle(stream)))
    return wf, bf, cs


def ln_linear(x, mean, rstd, folded, *, stream=None, out=None):
    """LayerNorm(x) w^T + bias for x [T, C] from ``ln_stats`` and the
    ``ln_fold_weights`` triple; returns y [T, N] in x's dtype."""
    torch = _torch()
    wf, bf, cs = folded
    T, C = x.shape
    N = wf.shape[0]
    dt = _dtype_code(x)
    if wf.dtype != x.dtype:
        raise TypeError("x and the folded weights must share one dtype")
    _mat16("x", x, (T, C))
    _mat16("w_folded", wf, (N, C))
    y = torch.empty((T, N), dtype=x.dtype, device=x.device) if out is None else out
    _mat16("y", y, (T, N))
    _call("fa_ln_linear", fa_ln_linear(x.data_ptr(), _f32_vec("mean", mean, T),
                                       _f32_vec("rstd", rstd, T), wf.data_ptr(),
                                       _f32_vec("bias_folded", bf, N), _f32_vec("colsum", cs, N),
                                       y.data_ptr(), T, C, N, dt, _stream_handle(stream)))
    return y


def linear(a, w, bias=None, residual=None, *, stream=None, out=None):
    """a [M, K] w [N, K]^T + bias (+ residual [M, N]); returns y [M, N] in a's dtype."""
    torch = _torch()
    M, K = a.shape
    N = w.shape[0]
    dt = _dtype_code(a)
    if w.dtype != a.dtype or (residual is not None and residual.dtype != a.dtype):
        raise TypeError("a, w and residual must share one dtype")
    _mat16("a", a, (M, K))
    _mat16("w", w, (N, K))
    rp = None if residual is None else _mat16("residual", residual, (M, N))
    bp = None if bias is None else _f32_vec("bias", bias, N)
    y = torch.empty((M, N), dtype=a.dtype, device=a.device) if out is None else out
    _mat16("y", y, (M, N))
    _call("fa_linear", fa_linear(a.data_ptr(), w.data_ptr(), bp, rp, y.data_ptr(), M, K, N, dt,
                                 _stream_handle(stream)))
    return y


def prenorm_attention(x, qkv_folded, w_o, b_o, *, B: int, N: int, H: int, H_kv: Optional[int] = None,
                      eps: float = 1e-5, scale: Optional[float] = None, causal: bool = False,
                      kv_lens=None, workspace=None, stream=None, out=None):
    """The pre-LayerNorm attention block y = x + Attn(LN(x) W_qkv^T + b_qkv) W_o^T + b_o.

    x [B*N, C] f16/bf16 (C = H*d); ``qkv_folded`` = ``ln_fold_weights(gamma,
    beta, W_qkv, b_qkv)`` with W_qkv [(H + 2*H_kv)*d, C] (query heads, key
    heads, value heads); w_o [C, C]; b_o fp32 [C] or None.  ``workspace``: a
    uint8 GPU tensor of at least ``fa_prenorm_attention_workspace_bytes``
    bytes (allocated when None).  Returns (y, workspace)."""
    torch = _torch()
    H_kv = H if H_kv is None else H_kv
    T, C = x.shape
    if T != B * N or C % H:
        raise ValueError("x must be [B*N, H*d]")
    d = C // H
    wf, bf, cs = qkv_folded
    R = (H + 2 * H_kv) * d
    dt = _dtype_code(x)
    if wf.dtype != x.dtype or w_o.dtype != x.dtype:
        raise TypeError("x and the weights must share one dtype")
    _mat16("x", x, (T, C))
    _mat16("w_qkv_folded", wf, (R, C))
    _mat16("w_o", w_o, (C, C))
    bo = None if b_o is None else _f32_vec("b_o", b_o, C)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl_ptr = None
    if kv_lens is not None:
        _check_dev("kv_lens", kv_lens)
        if kv_lens.dtype != torch.int32 or tuple(kv_lens.shape) != (B,):
            raise ValueError("kv_lens must be int32 [B]")
        kl_ptr = kv_lens.data_ptr()
    need = fa_prenorm_attention_workspace_bytes(B, N, H, H_kv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check_dev("workspace", workspace)
    y = torch.empty_like(x) if out is None else out
    _mat16("y", y, (T, C))
    _call("fa_prenorm_attention",
          fa_prenorm_attention(x.data_ptr(), wf.data_ptr(), _f32_vec("b_qkv_folded", bf, R),
                               _f32_vec("colsum_qkv", cs, R), w_o.data_ptr(), bo, y.data_ptr(), B,
                               N, H, H_kv, d, float(eps), float(scale), int(bool(causal)), kl_ptr,
                               dt, workspace.data_ptr(), workspace.numel(),
                               _stream_handle(stream)))
    return y, workspace


def prenorm_workspace_views(workspace, B: int, N: int, H: int, H_kv: int, d: int, dtype):
    """Views of the block's stages inside its workspace, in the documented order
    (mean, rstd, qkv, o, lse; each on a 256-byte boundary)."""
    torch = _torch()
    up = lambda v: (v + 255) // 256 * 256
    T, C, R = B * N, H * d, (H + 2 * H_kv) * d
    offs = {}
    o = 0
    for name, nbytes in (("mean", T * 4), ("rstd", T * 4), ("qkv", T * R * 2), ("o", T * C * 2),
                         ("lse", B * H * N * 4)):
        offs[name] = (o, nbytes)
        o += up(nbytes)
    def view(name, dt, shape):
        a, n = offs[name]
        return workspace[a:a + n].view(dt).view(*shape)
    return dict(mean=view("mean", torch.float32, (T,)), rstd=view("rstd", torch.float32, (T,)),
                qkv=view("qkv", dtype, (T, R)), o=view("o", dtype, (T, C)),
                lse=view("lse", torch.float32, (B, H, N)))
