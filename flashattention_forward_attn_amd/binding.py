"""ctypes binding of libfa.so: the C ABI of include/fa.h, one Python function per
C entry point, with the same names.  Argument marshalling only: tensors become
device pointers and sizes, torch's current stream becomes the hipStream_t, and
a non-zero status becomes an exception.  Every step of the computation runs in
the library's HIP kernels.

The library is loaded on first use; if it is missing this raises (there is no
fallback of any kind).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libfa.so")
# the same entry points with the forward kernels built to use one LDS stage
# (a race check for tests; never loaded by the product path)
SINGLE_STAGE_LIBRARY = os.path.join(HERE, "libfa_single_stage.so")

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEAD_DIM", 4: "FA_ERR_SCALE",
                5: "FA_ERR_ALIGN", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_HIP", 8: "FA_ERR_ALIAS",
                9: "FA_ERR_SCRATCH"}
# bytes of the no-allocation decode's static buffer (FA_DECODE_SCRATCH_BYTES)
FA_DECODE_SCRATCH_BYTES = 16 << 20

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load():
    """Load libfa.so (once) and declare the C signatures.  Raises if it is not built."""
    global _lib
    if _lib is None:
        _lib = open_library(LIBRARY)
    return _lib


def open_library(path: str):
    """A ctypes handle on a library exporting the C ABI of include/fa.h, with the
    C signatures declared.  Raises if the file is missing."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m flashattention_forward_attn_amd.build`")
    # torch first: the library must bind to the HIP runtime torch loads, since
    # the tensors, streams and device context it is handed are that runtime's.
    # torch's HIP library asks for its bundled runtime by file name, so a library
    # loaded before torch would bring in the system runtime and torch would then
    # load a second one beside it.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    fwd = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp]
    lib.fa_fwd_bf16.argtypes = fwd
    lib.fa_fwd_f32.argtypes = fwd
    lib.fa_fwd_unfused_bf16.argtypes = fwd[:-1] + [vp, sz, vp]
    lib.fa_fwd_unfused_f32.argtypes = fwd[:-1] + [vp, sz, vp]
    for name in ("fa_fwd_bf16", "fa_fwd_f32", "fa_fwd_unfused_bf16", "fa_fwd_unfused_f32"):
        getattr(lib, name).restype = ctypes.c_int
    lib.fa_unfused_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_unfused_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_bf16.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp, sz, vp]
    lib.fa_bwd_bf16.restype = ctypes.c_int
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_paged_bf16.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_decode_paged_bf16.restype = ctypes.c_int
    lib.fa_decode_paged_bf16_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_decode_paged_bf16_noalloc.restype = ctypes.c_int
    lib.fa_fp8_quantize_bf16.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.fa_fp8_quantize_bf16.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp]
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_fp8_qbf16.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp]
    lib.fa_fwd_fp8_qbf16.restype = ctypes.c_int
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_status_str.restype = ctypes.c_char_p
    return lib


def fa_status_str(status: int) -> str:
    return load().fa_status_str(int(status)).decode()


def _check(status: int) -> None:
    if status != FA_OK:
        raise FAError(status, fa_status_str(status))


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _dims(q):
    if not hasattr(q, "dim") or q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


# Every tensor argument is checked before its address is handed to the library:
# the kernels read and write exactly the documented number of contiguous
# elements of the documented type in device memory, so anything else would make
# them touch memory the caller did not mean.

def _expect(t, name: str, dtype, shape) -> None:
    """dtype, shape and contiguity of one tensor argument."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_one_gpu(**tensors) -> None:
    """All given tensors (None skipped) live on the same GPU."""
    first = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
        if first is None:
            first = t.device
        elif t.device != first:
            raise ValueError(f"{name} is on {t.device} but the other arguments are on {first}")


def _workspace(ws) -> int:
    """Byte size of a workspace tensor (contiguous uint8), 0 for None."""
    import torch
    if ws is None:
        return 0
    _expect(ws, "workspace", torch.uint8, ws.shape)
    return ws.numel()


def _forward_args(q, k, v, o, lse, kv_limit, dtype):
    import torch
    B, H, N, d = _dims(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _expect(t, name, dtype, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if kv_limit is not None:
        _expect(kv_limit, "kv_limit", torch.int32, (B, N))
    return B, H, N, d


def fa_fwd_bf16(q, k, v, o, lse, causal: bool, scale: float, kv_limit=None, stream=None) -> None:
    """Fused forward, bf16 tensors [B, H, N, d]; lse fp32 [B, H, N]; kv_limit int32 [B, N] or None."""
    import torch
    B, H, N, d = _forward_args(q, k, v, o, lse, kv_limit, torch.bfloat16)
    _on_one_gpu(q=q, k=k, v=v, o=o, lse=lse, kv_limit=kv_limit)
    _check(load().fa_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                              float(scale), _ptr(kv_limit), _stream(stream)))


def fa_fwd_f32(q, k, v, o, lse, causal: bool, scale: float, kv_limit=None, stream=None) -> None:
    """Fused forward, fp32 tensors [B, H, N, d]."""
    import torch
    B, H, N, d = _forward_args(q, k, v, o, lse, kv_limit, torch.float32)
    _on_one_gpu(q=q, k=k, v=v, o=o, lse=lse, kv_limit=kv_limit)
    _check(load().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                             float(scale), _ptr(kv_limit), _stream(stream)))


def fa_unfused_workspace_bytes(B: int, H: int, N: int, elem_bytes: int) -> int:
    return int(load().fa_unfused_workspace_bytes(B, H, N, elem_bytes))


def fa_fwd_unfused_bf16(q, k, v, o, lse, causal: bool, scale: float, kv_limit=None, workspace=None,
                        stream=None) -> None:
    """Unfused three-kernel forward (bf16); workspace is a device uint8 tensor."""
    import torch
    B, H, N, d = _forward_args(q, k, v, o, lse, kv_limit, torch.bfloat16)
    nbytes = _workspace(workspace)
    _on_one_gpu(q=q, k=k, v=v, o=o, lse=lse, kv_limit=kv_limit, workspace=workspace)
    _check(load().fa_fwd_unfused_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                      int(bool(causal)), float(scale), _ptr(kv_limit), _ptr(workspace), nbytes,
                                      _stream(stream)))


def fa_fwd_unfused_f32(q, k, v, o, lse, causal: bool, scale: float, kv_limit=None, workspace=None,
                       stream=None) -> None:
    """Unfused three-kernel forward (fp32)."""
    import torch
    B, H, N, d = _forward_args(q, k, v, o, lse, kv_limit, torch.float32)
    nbytes = _workspace(workspace)
    _on_one_gpu(q=q, k=k, v=v, o=o, lse=lse, kv_limit=kv_limit, workspace=workspace)
    _check(load().fa_fwd_unfused_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                     int(bool(causal)), float(scale), _ptr(kv_limit), _ptr(workspace), nbytes,
                                     _stream(stream)))


def fa_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, N))


def fa_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, causal: bool, scale: float, kv_limit=None, workspace=None,
                stream=None) -> None:
    """Backward pass of fa_fwd_bf16: bf16 [B, H, N, d] tensors, lse fp32 [B, H, N]; workspace a device
    uint8 tensor of at least fa_bwd_workspace_bytes(B, H, N) bytes."""
    import torch
    B, H, N, d = _forward_args(q, k, v, o, lse, kv_limit, torch.bfloat16)
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    nbytes = _workspace(workspace)
    _on_one_gpu(q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, kv_limit=kv_limit,
                workspace=workspace)
    _check(load().fa_bwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), B, H, N, d, int(bool(causal)), float(scale), _ptr(kv_limit),
                              _ptr(workspace), nbytes, _stream(stream)))


def attention_backward(q, k, v, o, lse, dout, causal: bool = False, scale: Optional[float] = None,
                       kv_limit=None, stream=None):
    """Allocate dq, dk, dv and the workspace with torch and run the backward pass (bf16).
    Returns (dq, dk, dv)."""
    import torch
    B, H, N, d = _dims(q)
    if scale is None:
        scale = d ** -0.5
    if q.dtype != torch.bfloat16:
        raise TypeError(f"the backward pass takes bf16 tensors, got {q.dtype}")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=q.device)
    fa_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, causal, scale, kv_limit, ws, stream)
    return dq, dk, dv


def fa_decode_workspace_bytes(B: int, H: int, d: int, max_pages: int) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, d, max_pages))


def _decode_shapes(q, k_cache, v_cache, block_table, seq_lens, o, lse):
    """(B, H, d, page_size, max_pages, num_pages) of a paged decode call, after
    checking every tensor's dtype, shape and layout."""
    import torch
    if not all(hasattr(t, "dim") for t in (q, k_cache, block_table)) or q.dim() != 3 or k_cache.dim() != 4 \
            or block_table.dim() != 2:
        raise ValueError("q must be [B, H, d], the caches [num_pages, H, page_size, d], block_table [B, max_pages]")
    B, H, d = (int(x) for x in q.shape)
    num_pages, _, page_size, _ = (int(x) for x in k_cache.shape)
    max_pages = int(block_table.shape[1])
    _expect(q, "q", torch.bfloat16, (B, H, d))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _expect(t, name, torch.bfloat16, (num_pages, H, page_size, d))
    _expect(block_table, "block_table", torch.int32, (B, max_pages))
    _expect(seq_lens, "seq_lens", torch.int32, (B,))
    _expect(o, "o", torch.bfloat16, (B, H, d))
    _expect(lse, "lse", torch.float32, (B, H))
    return B, H, d, page_size, max_pages, num_pages


def fa_decode_paged_bf16(q, k_cache, v_cache, block_table, seq_lens, o, lse, scale: float, workspace=None,
                         stream=None) -> None:
    """Decode over a paged cache: q, o bf16 [B, H, d]; k_cache, v_cache bf16 [num_pages, H, 16, d];
    block_table int32 [B, max_pages]; seq_lens int32 [B]; lse fp32 [B, H]; workspace a device uint8
    tensor of at least fa_decode_workspace_bytes(B, H, d, max_pages) bytes."""
    B, H, d, page_size, max_pages, num_pages = _decode_shapes(q, k_cache, v_cache, block_table, seq_lens, o, lse)
    nbytes = _workspace(workspace)
    _on_one_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seq_lens=seq_lens, o=o, lse=lse,
                workspace=workspace)
    _check(load().fa_decode_paged_bf16(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                       _ptr(o), _ptr(lse), B, H, d, page_size, max_pages, num_pages, float(scale),
                                       _ptr(workspace), nbytes, _stream(stream)))


def fa_decode_paged_bf16_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, lse, scale: float,
                                 stream=None) -> None:
    """fa_decode_paged_bf16 without a workspace: the library's static per-GPU buffer
    of FA_DECODE_SCRATCH_BYTES holds the partials.  Same tensors as fa_decode_paged_bf16."""
    B, H, d, page_size, max_pages, num_pages = _decode_shapes(q, k_cache, v_cache, block_table, seq_lens, o, lse)
    _on_one_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seq_lens=seq_lens, o=o, lse=lse)
    _check(load().fa_decode_paged_bf16_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                               _ptr(seq_lens), _ptr(o), _ptr(lse), B, H, d, page_size, max_pages,
                                               num_pages, float(scale), _stream(stream)))


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale: Optional[float] = None, stream=None):
    """Allocate o, lse and the workspace with torch and run the paged decode (bf16).  Returns (o, lse)."""
    import torch
    B, H, d = (int(x) for x in q.shape)
    if scale is None:
        scale = d ** -0.5
    if q.dtype != torch.bfloat16:
        raise TypeError(f"the paged decode takes bf16 tensors, got {q.dtype}")
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(1, fa_decode_workspace_bytes(B, H, d, int(block_table.shape[1]))), dtype=torch.uint8,
                     device=q.device)
    fa_decode_paged_bf16(q, k_cache, v_cache, block_table, seq_lens, o, lse, scale, ws, stream)
    return o, lse


FP8_Q_TILE, FP8_K_TILE = 32, 64


def fa_fp8_quantize_bf16(x, signs, codes, exps, tile_rows: int, stream=None) -> None:
    """Rotate (signs, Hadamard) and encode a bf16 [B, H, N, d] tensor: codes uint8 [B, H, N, d],
    exps int32 [B, H, ceil(N / tile_rows)]; tile_rows 32 for q, 64 for k."""
    import torch
    B, H, N, d = _dims(x)
    if tile_rows not in (FP8_Q_TILE, FP8_K_TILE):
        raise ValueError(f"tile_rows must be {FP8_Q_TILE} or {FP8_K_TILE}, got {tile_rows}")
    _expect(x, "x", torch.bfloat16, (B, H, N, d))
    _expect(signs, "signs", torch.int8, (d,))
    _expect(codes, "codes", torch.uint8, (B, H, N, d))
    _expect(exps, "exps", torch.int32, (B, H, -(-N // tile_rows)))
    _on_one_gpu(x=x, signs=signs, codes=codes, exps=exps)
    _check(load().fa_fp8_quantize_bf16(_ptr(x), _ptr(signs), _ptr(codes), _ptr(exps), B, H, N, d, int(tile_rows),
                                       _stream(stream)))


def fa_fwd_fp8(q_codes, q_exps, k_codes, k_exps, v, o, lse, causal: bool, scale: float, kv_limit=None,
               stream=None) -> None:
    """Fused forward on E4M3 q and k codes (from fa_fp8_quantize_bf16) and bf16 v."""
    import torch
    B, H, N, d = _dims(v)
    _expect(v, "v", torch.bfloat16, (B, H, N, d))
    _expect(q_codes, "q_codes", torch.uint8, (B, H, N, d))
    _expect(k_codes, "k_codes", torch.uint8, (B, H, N, d))
    _expect(q_exps, "q_exps", torch.int32, (B, H, -(-N // FP8_Q_TILE)))
    _expect(k_exps, "k_exps", torch.int32, (B, H, -(-N // FP8_K_TILE)))
    _expect(o, "o", torch.bfloat16, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if kv_limit is not None:
        _expect(kv_limit, "kv_limit", torch.int32, (B, N))
    _on_one_gpu(q_codes=q_codes, q_exps=q_exps, k_codes=k_codes, k_exps=k_exps, v=v, o=o, lse=lse,
                kv_limit=kv_limit)
    _check(load().fa_fwd_fp8(_ptr(q_codes), _ptr(q_exps), _ptr(k_codes), _ptr(k_exps), _ptr(v), _ptr(o), _ptr(lse),
                             B, H, N, d, int(bool(causal)), float(scale), _ptr(kv_limit), _stream(stream)))


def fa_fwd_fp8_qbf16(q, signs, k_codes, k_exps, v, o, lse, causal: bool, scale: float, kv_limit=None,
                     stream=None) -> None:
    """FP8 forward with q in bf16 (rotated and encoded inside the kernel, the same codes
    fa_fp8_quantize_bf16 would store) and k as codes from fa_fp8_quantize_bf16."""
    import torch
    B, H, N, d = _dims(q)
    _expect(q, "q", torch.bfloat16, (B, H, N, d))
    _expect(signs, "signs", torch.int8, (d,))
    _expect(k_codes, "k_codes", torch.uint8, (B, H, N, d))
    _expect(k_exps, "k_exps", torch.int32, (B, H, -(-N // FP8_K_TILE)))
    _expect(v, "v", torch.bfloat16, (B, H, N, d))
    _expect(o, "o", torch.bfloat16, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if kv_limit is not None:
        _expect(kv_limit, "kv_limit", torch.int32, (B, N))
    _on_one_gpu(q=q, signs=signs, k_codes=k_codes, k_exps=k_exps, v=v, o=o, lse=lse, kv_limit=kv_limit)
    _check(load().fa_fwd_fp8_qbf16(_ptr(q), _ptr(signs), _ptr(k_codes), _ptr(k_exps), _ptr(v), _ptr(o), _ptr(lse),
                                   B, H, N, d, int(bool(causal)), float(scale), _ptr(kv_limit), _stream(stream)))


def fp8_quantize(x, signs, tile_rows: int, stream=None):
    """Allocate and fill (codes, exps) for a bf16 tensor."""
    import torch
    B, H, N, d = _dims(x)
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    exps = torch.empty((B, H, -(-N // tile_rows)), dtype=torch.int32, device=x.device)
    fa_fp8_quantize_bf16(x, signs, codes, exps, tile_rows, stream)
    return codes, exps


def attention_fp8(q, k, v, signs, causal: bool = False, scale: Optional[float] = None, kv_limit=None, stream=None):
    """FP8 forward from bf16 q, k, v: quantise k, then attention with q rotated and
    encoded inside the kernel (the same signs for both).  Returns (o, lse)."""
    import torch
    B, H, N, d = _dims(q)
    if scale is None:
        scale = d ** -0.5
    kc, ke = fp8_quantize(k, signs, FP8_K_TILE, stream)
    o = torch.empty_like(v)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_fp8_qbf16(q, signs, kc, ke, v, o, lse, causal, scale, kv_limit, stream)
    return o, lse


def attention(q, k, v, causal: bool = False, scale: Optional[float] = None, kv_limit=None, unfused: bool = False,
              stream=None):
    """Allocate O and LSE with torch and run the fused (or unfused) forward.

    q, k, v: contiguous device tensors [B, H, N, d], all bf16 or all fp32.
    Returns (o, lse).  The unfused path also allocates its workspace.
    """
    import torch
    B, H, N, d = _dims(q)
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if q.dtype == torch.bfloat16:
        if unfused:
            ws = torch.empty(fa_unfused_workspace_bytes(B, H, N, 2), dtype=torch.uint8, device=q.device)
            fa_fwd_unfused_bf16(q, k, v, o, lse, causal, scale, kv_limit, ws, stream)
        else:
            fa_fwd_bf16(q, k, v, o, lse, causal, scale, kv_limit, stream)
    elif q.dtype == torch.float32:
        if unfused:
            ws = torch.empty(fa_unfused_workspace_bytes(B, H, N, 4), dtype=torch.uint8, device=q.device)
            fa_fwd_unfused_f32(q, k, v, o, lse, causal, scale, kv_limit, ws, stream)
        else:
            fa_fwd_f32(q, k, v, o, lse, causal, scale, kv_limit, stream)
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return o, lse
