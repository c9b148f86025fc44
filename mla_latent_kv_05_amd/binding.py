"""Thin ctypes binding of libmla.so (include/mla_decode.h).

Argument marshalling only: every function checks devices/dtypes/contiguity,
passes raw device pointers plus the current torch stream, and raises
RuntimeError with the library's status text on a non-zero status.  All compute
runs in the HIP kernels of libmla.so; if the library is missing these
functions raise instead of falling back to anything else."""

from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mla_decode.h")

MLA_F32, MLA_BF16, MLA_FP8_E4M3, MLA_INT4, MLA_INT2 = 0, 1, 2, 3, 4
MLA_FLAG_FORCE_GENERIC = 1
MLA_STAGE_ABSORB, MLA_STAGE_ATTEND, MLA_STAGE_MERGE, MLA_STAGE_ALL = 1, 2, 4, 7

_lib = None

_c = ctypes
_SIGS = {
    "mla_status_string": (_c.c_char_p, [_c.c_int]),
    "mla_absorb_q": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int,
                                _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p]),
    "mla_up_proj_v": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int,
                                 _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p]),
    "mla_decode_workspace_bytes": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "mla_decode_absorbed": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p,
                                       _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float,
                                       _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_size_t,
                                       _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "mla_combine_lse": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int,
                                   _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "mla_cache_append": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                    _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float, _c.c_int,
                                    _c.c_int, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "mla_cache_append_workspace_bytes": (_c.c_size_t, [_c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "mla_decode_step": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int,
                                   _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                   _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int, _c.c_void_p, _c.c_size_t,
                                   _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "mla_decode_step_stages": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                          _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int,
                                          _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int,
                                          _c.c_void_p, _c.c_size_t, _c.c_void_p, _c.c_void_p, _c.c_int,
                                          _c.c_void_p]),
    "mla_decode_step_workspace_bytes": (_c.c_size_t, [_c.c_int] * 6),
    "mla_decode_step_noalloc": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                           _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int,
                                           _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int,
                                           _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "mla_gqa_decode": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p,
                                  _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float,
                                  _c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "mla_expand_kv": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                 _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p]),
    "mla_prefill_mha": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                   _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int,
                                   _c.c_void_p]),
}


def lib() -> ctypes.CDLL:
    """Load libmla.so (built in-tree by mla_latent_kv_05_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_05_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/mla_decode.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(mla_\w+)\s*\(", txt, flags=re.M)


def status_string(code: int) -> str:
    return lib().mla_status_string(code).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what}: {status_string(rc)} (status {rc})")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tdt(code: int) -> torch.dtype:
    return {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16}[code]


def _gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _ptr(t):
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------------------


def absorb_q(q_nope: torch.Tensor, w_uk: torch.Tensor, out_dtype: torch.dtype | None = None,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """q_lat[t, i, :] = W^UK_i^T q_nope[t, i, :].  q_nope [T, n_h, d_h] (token
    stride may exceed n_h*d_h), w_uk [n_h*d_h, d_c]."""
    _gpu(q_nope, w_uk)
    T, n_h, d_h = q_nope.shape
    assert q_nope.stride(2) == 1 and q_nope.stride(1) == d_h, "q_nope heads must be packed"
    assert w_uk.is_contiguous() and w_uk.shape[0] == n_h * d_h
    d_c = w_uk.shape[1]
    odt = out_dtype or q_nope.dtype
    if out is None:
        out = torch.empty((T, n_h, d_c), dtype=odt, device=q_nope.device)
    assert out.stride(2) == 1 and out.stride(1) == d_c
    _check(lib().mla_absorb_q(_ptr(q_nope), q_nope.stride(0), _ptr(w_uk), _ptr(out), out.stride(0), T, n_h,
                              d_h, d_c, _dt(q_nope), _dt(w_uk), _dt(out), _stream()), "mla_absorb_q")
    return out


def up_proj_v(o_lat: torch.Tensor, w_uv: torch.Tensor, d_h: int, out_dtype: torch.dtype | None = None,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """o[t, i, :] = W^UV_i o_lat[t, i, :].  o_lat [T, n_h, d_c], w_uv [n_h*d_h, d_c]."""
    _gpu(o_lat, w_uv)
    T, n_h, d_c = o_lat.shape
    assert o_lat.stride(2) == 1 and o_lat.stride(1) == d_c
    assert w_uv.is_contiguous() and w_uv.shape == (n_h * d_h, d_c)
    odt = out_dtype or o_lat.dtype
    if out is None:
        out = torch.empty((T, n_h, d_h), dtype=odt, device=o_lat.device)
    assert out.stride(2) == 1 and out.stride(1) == d_h
    _check(lib().mla_up_proj_v(_ptr(o_lat), o_lat.stride(0), _ptr(w_uv), _ptr(out), out.stride(0), T, n_h, d_c,
                               d_h, _dt(o_lat), _dt(w_uv), _dt(out), _stream()), "mla_up_proj_v")
    return out


def workspace_bytes(B: int, s_q: int, n_h: int, d_c: int, max_blocks_per_seq: int, num_splits: int = 0) -> int:
    n = lib().mla_decode_workspace_bytes(B, s_q, n_h, d_c, max_blocks_per_seq, num_splits)
    if n == 0:
        raise RuntimeError("mla_decode_workspace_bytes: invalid arguments or no HIP device")
    return n


def alloc_workspace(B, s_q, n_h, d_c, max_blocks_per_seq, num_splits=0, device="cuda") -> torch.Tensor:
    n = workspace_bytes(B, s_q, n_h, d_c, max_blocks_per_seq, num_splits)
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode(q_lat: torch.Tensor, q_rope: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, softmax_scale: float, kv_dtype: int | None = None, d_r: int | None = None,
           block_size: int = 64, out_dtype: torch.dtype = torch.bfloat16, num_splits: int = 0,
           workspace: torch.Tensor | None = None, with_lse: bool = True, force_generic: bool = False,
           out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Absorbed-MLA decode over a paged latent cache.

    q_lat [B, s_q, n_h, d_c], q_rope [B, s_q, n_h, d_r]; kv_cache: bf16/fp32
    [num_blocks, block_size, d_c+d_r], or uint8 fp8 blocks (kv_dtype=MLA_FP8_E4M3,
    layout of include/mla_decode.h); block_table [B, max_blocks] int32;
    seq_lens [B] int32.  Returns (o_lat [B, s_q, n_h, d_c], lse [B, s_q, n_h] or None)."""
    _gpu(q_lat, q_rope, kv_cache, block_table, seq_lens)
    B, s_q, n_h, d_c = q_lat.shape
    d_r = q_rope.shape[-1] if d_r is None else d_r
    assert q_lat.is_contiguous() and q_rope.is_contiguous() and kv_cache.is_contiguous()
    assert q_rope.shape == (B, s_q, n_h, d_r) and q_rope.dtype == q_lat.dtype
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.shape[0] == B
    assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous() and seq_lens.shape == (B,)
    if kv_dtype is None:
        kv_dtype = _dt(kv_cache)
    max_blocks = block_table.shape[1]
    if workspace is None:
        workspace = alloc_workspace(B, s_q, n_h, d_c, max_blocks, num_splits, device=q_lat.device)
    if out is None:
        out = torch.empty((B, s_q, n_h, d_c), dtype=out_dtype, device=q_lat.device)
    if with_lse and lse is None:
        lse = torch.empty((B, s_q, n_h), dtype=torch.float32, device=q_lat.device)
    flags = MLA_FLAG_FORCE_GENERIC if force_generic else 0
    _check(lib().mla_decode_absorbed(_ptr(q_lat), _ptr(q_rope), _ptr(kv_cache), _ptr(block_table), max_blocks,
                                     _ptr(seq_lens), B, s_q, n_h, d_c, d_r, block_size, float(softmax_scale),
                                     _dt(q_lat), kv_dtype, _dt(out), num_splits, _ptr(workspace),
                                     workspace.numel(), _ptr(out), _ptr(lse) if with_lse else None, flags,
                                     _stream()), "mla_decode_absorbed")
    return out, (lse if with_lse else None)


def cache_append_workspace(T: int, d: int, d_c: int, d_r: int, device="cuda") -> torch.Tensor:
    n = lib().mla_cache_append_workspace_bytes(T, d, d_c, d_r)
    if n == 0:
        raise RuntimeError("mla_cache_append_workspace_bytes: invalid sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def cache_append(h: torch.Tensor, w_dkv_kr: torch.Tensor, positions: torch.Tensor, slot_mapping: torch.Tensor,
                 kv_cache: torch.Tensor, d_c: int, d_r: int, block_size: int = 64, kv_dtype: int | None = None,
                 rope_base: float = 10000.0, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Write c^KV = W^DKV h and k^R = RoPE(W^KR h, pos) of T new tokens into
    the paged cache (in place).  h [T, d] (token stride h.stride(0));
    w_dkv_kr [d_c + d_r, d]; positions, slot_mapping [T] int32 (slot < 0
    skips a token); kv_cache as for decode()."""
    _gpu(h, w_dkv_kr, positions, slot_mapping, kv_cache)
    T, d = h.shape
    assert h.stride(1) == 1 and w_dkv_kr.is_contiguous() and w_dkv_kr.shape == (d_c + d_r, d)
    assert w_dkv_kr.dtype == h.dtype and kv_cache.is_contiguous()
    assert positions.dtype == torch.int32 and slot_mapping.dtype == torch.int32
    assert positions.shape == (T,) and slot_mapping.shape == (T,)
    assert positions.is_contiguous() and slot_mapping.is_contiguous()
    if kv_dtype is None:
        kv_dtype = _dt(kv_cache)
    if workspace is None:
        workspace = cache_append_workspace(max(T, 1), d, d_c, d_r, device=h.device)
    _check(lib().mla_cache_append(_ptr(h), h.stride(0), _ptr(w_dkv_kr), _ptr(positions), _ptr(slot_mapping),
                                  _ptr(kv_cache), T, d, d_c, d_r, block_size, float(rope_base), _dt(h),
                                  kv_dtype, _ptr(workspace), workspace.numel(), _stream()), "mla_cache_append")
    return kv_cache


def decode_step(q_nope: torch.Tensor, w_uk: torch.Tensor, q_rope: torch.Tensor, kv_cache: torch.Tensor,
                block_table: torch.Tensor, seq_lens: torch.Tensor, w_uv: torch.Tensor, softmax_scale: float,
                kv_dtype: int | None = None, d_c: int = 512, block_size: int = 64, num_splits: int = 0,
                workspace: torch.Tensor | None = None, with_lse: bool = True, out: torch.Tensor | None = None,
                lse: torch.Tensor | None = None):
    """Whole absorbed decode step: absorb, attention, merge + up-projection.
    q_nope [B, s_q, n_h, d_h], q_rope [B, s_q, n_h, d_r], weights [n_h*d_h, d_c]
    (all bf16).  Returns (o [B, s_q, n_h, d_h] bf16, lse [B, s_q, n_h] or None)."""
    return _step(None, q_nope, w_uk, q_rope, kv_cache, block_table, seq_lens, w_uv, softmax_scale, kv_dtype, d_c,
                 block_size, num_splits, workspace, with_lse, out, lse)


def decode_step_stages(stages: int, q_nope: torch.Tensor, w_uk: torch.Tensor, q_rope: torch.Tensor,
                       kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, w_uv: torch.Tensor,
                       softmax_scale: float, kv_dtype: int | None = None, d_c: int = 512, block_size: int = 64,
                       num_splits: int = 0, workspace: torch.Tensor | None = None, with_lse: bool = True,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """decode_step restricted to the MLA_STAGE_* bits in `stages`; the stages
    of one step share `workspace` (required), `out` and `lse`."""
    if workspace is None:
        raise ValueError("decode_step_stages: the stages of a step share a caller-owned workspace")
    return _step(stages, q_nope, w_uk, q_rope, kv_cache, block_table, seq_lens, w_uv, softmax_scale, kv_dtype, d_c,
                 block_size, num_splits, workspace, with_lse, out, lse)


def decode_step_noalloc(q_nope: torch.Tensor, w_uk: torch.Tensor, q_rope: torch.Tensor, kv_cache: torch.Tensor,
                        block_table: torch.Tensor, seq_lens: torch.Tensor, w_uv: torch.Tensor, softmax_scale: float,
                        out: torch.Tensor, lse: torch.Tensor | None = None, kv_dtype: int | None = None,
                        d_c: int = 512, block_size: int = 64, num_splits: int = 0):
    """decode_step without a workspace (mla_decode_step_noalloc): `out` (and
    `lse`, if wanted) must be given, since nothing is allocated here either."""
    _gpu(q_nope, w_uk, q_rope, kv_cache, block_table, seq_lens, w_uv, out)
    B, s_q, n_h, d_h = q_nope.shape
    d_r = q_rope.shape[-1]
    for t in (q_nope, w_uk, q_rope, w_uv, kv_cache, block_table, out):
        assert t.is_contiguous()
    assert q_rope.shape == (B, s_q, n_h, d_r) and w_uk.shape == (n_h * d_h, d_c) and w_uv.shape == (n_h * d_h, d_c)
    assert out.shape == (B, s_q, n_h, d_h) and out.dtype == torch.bfloat16
    if lse is not None:
        assert lse.shape == (B, s_q, n_h) and lse.dtype == torch.float32 and lse.is_contiguous()
    if kv_dtype is None:
        kv_dtype = _dt(kv_cache)
    _check(lib().mla_decode_step_noalloc(_ptr(q_nope), _ptr(w_uk), _ptr(q_rope), _ptr(kv_cache), _ptr(block_table),
                                         block_table.shape[1], _ptr(seq_lens), _ptr(w_uv), B, s_q, n_h, d_h, d_c, d_r,
                                         block_size, float(softmax_scale), kv_dtype, num_splits, _ptr(out),
                                         _ptr(lse) if lse is not None else None, _stream()),
           "mla_decode_step_noalloc")
    return out, lse


def _step(stages, q_nope, w_uk, q_rope, kv_cache, block_table, seq_lens, w_uv, softmax_scale, kv_dtype, d_c,
          block_size, num_splits, workspace, with_lse, out, lse):
    _gpu(q_nope, w_uk, q_rope, kv_cache, block_table, seq_lens, w_uv)
    B, s_q, n_h, d_h = q_nope.shape
    d_r = q_rope.shape[-1]
    for t in (q_nope, w_uk, q_rope, w_uv, kv_cache, block_table):
        assert t.is_contiguous()
    assert q_rope.shape == (B, s_q, n_h, d_r) and w_uk.shape == (n_h * d_h, d_c) and w_uv.shape == (n_h * d_h, d_c)
    if kv_dtype is None:
        kv_dtype = _dt(kv_cache)
    max_blocks = block_table.shape[1]
    if workspace is None:
        n = lib().mla_decode_step_workspace_bytes(B, s_q, n_h, d_c, max_blocks, num_splits)
        workspace = torch.empty(n, dtype=torch.uint8, device=q_nope.device)
    if out is None:
        out = torch.empty((B, s_q, n_h, d_h), dtype=torch.bfloat16, device=q_nope.device)
    if with_lse and lse is None:
        lse = torch.empty((B, s_q, n_h), dtype=torch.float32, device=q_nope.device)
    args = (_ptr(q_nope), _ptr(w_uk), _ptr(q_rope), _ptr(kv_cache), _ptr(block_table), max_blocks, _ptr(seq_lens),
            _ptr(w_uv), B, s_q, n_h, d_h, d_c, d_r, block_size, float(softmax_scale), kv_dtype, num_splits,
            _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse) if with_lse else None)
    if stages is None:
        _check(lib().mla_decode_step(*args, _stream()), "mla_decode_step")
    else:
        _check(lib().mla_decode_step_stages(*args, int(stages), _stream()), "mla_decode_step_stages")
    return out, (lse if with_lse else None)


def decode_step_workspace(B, s_q, n_h, d_c, max_blocks_per_seq, num_splits=0, device="cuda") -> torch.Tensor:
    n = lib().mla_decode_step_workspace_bytes(B, s_q, n_h, d_c, max_blocks_per_seq, num_splits)
    return torch.empty(n, dtype=torch.uint8, device=device)


def gqa_decode(q_c: torch.Tensor, q_r: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
               seq_lens: torch.Tensor, n_g: int, softmax_scale: float, block_size: int = 64,
               out_dtype: torch.dtype = torch.bfloat16, with_lse: bool = True, force_generic: bool = False,
               out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """GQLA's GQA-path decode over a paged per-group expanded cache (layout
    of include/mla_decode.h).  q_c [B, s_q, n_h, d_h], q_r [B, s_q, n_h, d_r].
    Returns (o [B, s_q, n_h, d_h], lse [B, s_q, n_h] or None)."""
    _gpu(q_c, q_r, kv_cache, block_table, seq_lens)
    B, s_q, n_h, d_h = q_c.shape
    d_r = q_r.shape[-1]
    assert q_c.is_contiguous() and q_r.is_contiguous() and kv_cache.is_contiguous()
    assert q_r.shape == (B, s_q, n_h, d_r) and q_r.dtype == q_c.dtype
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.shape[0] == B
    assert seq_lens.dtype == torch.int32 and seq_lens.shape == (B,)
    if out is None:
        out = torch.empty((B, s_q, n_h, d_h), dtype=out_dtype, device=q_c.device)
    if with_lse and lse is None:
        lse = torch.empty((B, s_q, n_h), dtype=torch.float32, device=q_c.device)
    _check(lib().mla_gqa_decode(_ptr(q_c), _ptr(q_r), _ptr(kv_cache), _ptr(block_table), block_table.shape[1],
                                _ptr(seq_lens), B, s_q, n_h, n_g, d_h, d_r, block_size, float(softmax_scale),
                                _dt(q_c), _dt(kv_cache), _dt(out), _ptr(out), _ptr(lse) if with_lse else None,
                                MLA_FLAG_FORCE_GENERIC if force_generic else 0, _stream()), "mla_gqa_decode")
    return out, (lse if with_lse else None)


def expand_kv(c_kv: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor, d_h: int,
              out_dtype: torch.dtype | None = None):
    """k_c, v_c [T, n_h, d_h] = per-head W^UK / W^UV applied to c_kv [T, d_c]."""
    _gpu(c_kv, w_uk, w_uv)
    T, d_c = c_kv.shape
    n_h = w_uk.shape[0] // d_h
    assert c_kv.stride(1) == 1 and w_uk.is_contiguous() and w_uv.is_contiguous()
    assert w_uk.shape == (n_h * d_h, d_c) and w_uv.shape == (n_h * d_h, d_c)
    odt = c_kv.dtype if out_dtype is None else out_dtype
    k_c = torch.empty((T, n_h, d_h), dtype=odt, device=c_kv.device)
    v_c = torch.empty((T, n_h, d_h), dtype=odt, device=c_kv.device)
    _check(lib().mla_expand_kv(_ptr(c_kv), c_kv.stride(0), _ptr(w_uk), _ptr(w_uv), _ptr(k_c), _ptr(v_c), T, n_h,
                               d_c, d_h, _dt(c_kv), _dt(w_uk), _dt(k_c), _stream()), "mla_expand_kv")
    return k_c, v_c


def prefill_mha(q: torch.Tensor, k_c: torch.Tensor, k_r: torch.Tensor, v_c: torch.Tensor, softmax_scale: float,
                out_dtype: torch.dtype | None = None, with_lse: bool = True):
    """Causal MHA-mode attention: q [T, n_h, d_h+d_r], k_c/v_c [T, n_h, d_h],
    k_r [T, d_r] (shared by the heads).  Returns (o [T, n_h, d_h], lse [T, n_h])."""
    _gpu(q, k_c, k_r, v_c)
    T, n_h, dq = q.shape
    d_h = k_c.shape[-1]
    d_r = dq - d_h
    for t in (q, k_c, k_r, v_c):
        assert t.is_contiguous() and t.dtype == q.dtype
    assert k_c.shape == (T, n_h, d_h) and v_c.shape == (T, n_h, d_h) and k_r.shape == (T, d_r)
    o = torch.empty((T, n_h, d_h), dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    lse = torch.empty((T, n_h), dtype=torch.float32, device=q.device) if with_lse else None
    _check(lib().mla_prefill_mha(_ptr(q), _ptr(k_c), _ptr(k_r), _ptr(v_c), _ptr(o), _ptr(lse), T, n_h, d_h, d_r,
                                 float(softmax_scale), _dt(q), _dt(o), _stream()), "mla_prefill_mha")
    return o, lse


def combine_lse(o_part: torch.Tensor, lse_part: torch.Tensor, splits_per_row: torch.Tensor | None = None,
                out_dtype: torch.dtype = torch.float32):
    """Merge partial results: o_part [N, S, D] fp32, lse_part [N, S] fp32."""
    _gpu(o_part, lse_part, splits_per_row)
    N, S, D = o_part.shape
    assert o_part.dtype == torch.float32 and lse_part.dtype == torch.float32
    assert o_part.is_contiguous() and lse_part.is_contiguous() and lse_part.shape == (N, S)
    if splits_per_row is not None:
        assert splits_per_row.dtype == torch.int32 and splits_per_row.shape == (N,)
    out = torch.empty((N, D), dtype=out_dtype, device=o_part.device)
    lse = torch.empty((N,), dtype=torch.float32, device=o_part.device)
    _check(lib().mla_combine_lse(_ptr(o_part), _ptr(lse_part), _ptr(splits_per_row), N, S, D, _ptr(out),
                                 _ptr(lse), _dt(out), _stream()), "mla_combine_lse")
    return out, lse
