"""Python binding of libmla (weight-absorbed MLA decode on gfx950).

Argument marshalling only: every step of the decode runs in the HIP kernels
behind the C ABI declared in include/mla.h.  PyTorch provides device memory
and the current HIP stream.  There is no fallback: if libmla.so is missing
or the tensors are not on a GPU, calls raise.

    out, lse = decode(q_nope, q_rope, kv_pages, block_table, cache_seqlens,
                      softmax_scale, kv_scales=None, causal=False)
    out, lse = sparse_decode(q_nope, q_rope, kv_pages, block_table,
                             cache_seqlens, indices, softmax_scale)
    kv_append(new_kv, kv_pages, block_table, cache_seqlens, kv_scales=None)
    idx = dsa_select(block_scores, cache_seqlens, n_select=16, n_init=1, n_local=2)
    q_nope = absorb_query(q_c, w_uk_t)          # [B, Sq, H, 128] -> [B, Sq, H, 512]
    o = project_out(out, w_uv)                  # [B, Sq, H, 512] -> [B, Sq, H, 128]
    out, lse = prefill(q, k, v, softmax_scale)  # non-absorbed MHA over decompressed K/V
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1
STATUS = ["MLA_OK", "MLA_ERR_NULL", "MLA_ERR_SHAPE", "MLA_ERR_UNSUPPORTED", "MLA_ERR_ALIGN",
          "MLA_ERR_WORKSPACE", "MLA_ERR_HIP"]
EXPORTS = ["mla_workspace_size", "mla_plan", "mla_decode", "mla_sparse_decode", "mla_attend",
           "mla_combine", "mla_kv_append", "mla_dsa_select", "mla_absorb_query", "mla_project_out",
           "mla_prefill", "mla_decode_noalloc", "mla_layer_workspace_size", "mla_decode_layer",
           "mla_status_str", "mla_last_error"]

_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{name}: {detail}")
        self.status = status


def lib():
    """The loaded libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python mla_latent_kv_12_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        L.mla_workspace_size.restype = sz
        L.mla_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.mla_plan.restype = i32
        L.mla_plan.argtypes = [vp, i32, i32, i32, i32, i32, vp, sz, vp]
        L.mla_decode.restype = i32
        L.mla_decode.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32, f32, i32,
                                 vp, vp, vp, sz, i32, i32, vp]
        L.mla_sparse_decode.restype = i32
        L.mla_sparse_decode.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, vp, i32, i32, i32,
                                        i32, f32, vp, vp, vp, sz, i32, i32, vp]
        L.mla_attend.restype = i32
        L.mla_attend.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, vp, i32, i32, i32, i32,
                                 f32, i32, vp, vp, vp, sz, i32, vp]
        L.mla_combine.restype = i32
        L.mla_combine.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, sz, i32, vp]
        L.mla_kv_append.restype = i32
        L.mla_kv_append.argtypes = [vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, vp]
        L.mla_dsa_select.restype = i32
        L.mla_dsa_select.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, vp, vp]
        for fn in (L.mla_absorb_query, L.mla_project_out):
            fn.restype = i32
            fn.argtypes = [vp, vp, vp, i32, i32, vp]
        L.mla_decode_noalloc.restype = i32
        L.mla_decode_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32,
                                         f32, i32, vp, vp, i32, vp]
        L.mla_prefill.restype = i32
        L.mla_prefill.argtypes = [vp, vp, vp, i32, i32, i32, f32, i32, vp, vp, vp]
        L.mla_layer_workspace_size.restype = sz
        L.mla_layer_workspace_size.argtypes = [i32, i32, i32, i32]
        L.mla_decode_layer.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32,
                                       f32, i32, vp, vp, vp, sz, i32, vp]
        L.mla_status_str.restype = ctypes.c_char_p
        L.mla_status_str.argtypes = [i32]
        L.mla_last_error.restype = ctypes.c_char_p
        L.mla_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MLAError(status, lib().mla_last_error().decode())


def workspace_size(B: int, Sq: int, H: int, topk: int = 0, num_wg: int = 0) -> int:
    return int(lib().mla_workspace_size(B, Sq, H, topk, num_wg))


def alloc_workspace(B: int, Sq: int, H: int, topk: int = 0, num_wg: int = 0, device=None):
    n = workspace_size(B, Sq, H, topk, num_wg)
    if n == 0:
        raise MLAError(2, "invalid sizes for the workspace")
    return torch.empty(n, dtype=torch.uint8, device=device or torch.device("cuda"))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _req(t, name, dtypes, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (no CPU path exists)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, has {t.dim()}")


def _common(q_nope, q_rope, kv_pages, kv_scales, block_table, cache_seqlens, out, lse, workspace,
            topk, num_wg):
    _req(q_nope, "q_nope", (torch.bfloat16,), 4)
    _req(q_rope, "q_rope", (torch.bfloat16,), 4)
    B, Sq, H, dc = q_nope.shape
    if dc != 512 or tuple(q_rope.shape) != (B, Sq, H, 64):
        raise ValueError("q_nope must be [B,Sq,H,512] and q_rope [B,Sq,H,64]")
    _req(kv_pages, "kv_pages", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), 3)
    if tuple(kv_pages.shape[1:]) != (64, 576):
        raise ValueError("kv_pages must be [num_pages, 64, 576]")
    fp8 = kv_pages.dtype != torch.bfloat16
    if fp8:
        if kv_scales is None:
            raise ValueError("an fp8 cache needs kv_scales")
        _req(kv_scales, "kv_scales", (torch.float32,), 2)
        if tuple(kv_scales.shape) != (kv_pages.shape[0], 64):
            raise ValueError("kv_scales must be [num_pages, 64]")
    _req(block_table, "block_table", (torch.int32,), 2)
    if block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _req(cache_seqlens, "cache_seqlens", (torch.int32,), 1)
    if cache_seqlens.shape[0] != B:
        raise ValueError("cache_seqlens must be [B]")
    dev = q_nope.device
    if out is None:
        out = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)
    _req(out, "out", (torch.bfloat16,), 4)
    _req(lse, "lse", (torch.float32,), 3)
    if tuple(out.shape) != (B, Sq, H, 512) or tuple(lse.shape) != (B, Sq, H):
        raise ValueError("out must be [B,Sq,H,512] and lse [B,Sq,H]")
    if workspace is False:      # the call brings its own workspace
        return B, Sq, H, fp8, out, lse, None
    if workspace is None:
        workspace = alloc_workspace(B, Sq, H, topk, num_wg, dev)
    _req(workspace, "workspace", (torch.uint8,), 1)
    return B, Sq, H, fp8, out, lse, workspace


def plan(cache_seqlens: torch.Tensor, B: int, Sq: int, H: int, workspace: torch.Tensor,
         topk: int = 0, num_wg: int = 0):
    """Run the split-KV scheduling pass into `workspace` (see mla_plan)."""
    _req(cache_seqlens, "cache_seqlens", (torch.int32,), 1)
    _req(workspace, "workspace", (torch.uint8,), 1)
    _check(lib().mla_plan(cache_seqlens.data_ptr(), B, Sq, H, topk, num_wg, workspace.data_ptr(),
                          workspace.numel(), _stream(cache_seqlens)))


def decode(q_nope, q_rope, kv_pages, block_table, cache_seqlens, softmax_scale, kv_scales=None,
           causal=False, out=None, lse=None, workspace=None, num_wg=0, planned=False):
    """Dense absorbed MLA decode; returns (out bf16 [B,Sq,H,512], lse fp32 [B,Sq,H])."""
    B, Sq, H, fp8, out, lse, workspace = _common(q_nope, q_rope, kv_pages, kv_scales, block_table,
                                                 cache_seqlens, out, lse, workspace, 0, num_wg)
    _check(lib().mla_decode(
        q_nope.data_ptr(), q_rope.data_ptr(), kv_pages.data_ptr(),
        kv_scales.data_ptr() if fp8 else None, MLA_KV_FP8_E4M3 if fp8 else MLA_KV_BF16,
        kv_pages.shape[0], block_table.data_ptr(), block_table.shape[1], cache_seqlens.data_ptr(),
        B, Sq, H, float(softmax_scale), int(bool(causal)), out.data_ptr(), lse.data_ptr(),
        workspace.data_ptr(), workspace.numel(), int(num_wg), int(bool(planned)), _stream(q_nope)))
    return out, lse


def decode_noalloc(q_nope, q_rope, kv_pages, block_table, cache_seqlens, softmax_scale,
                   kv_scales=None, causal=False, out=None, lse=None, num_wg=0):
    """mla_decode_noalloc: mla_decode with the library's static workspace
    (nothing allocated on the device if out and lse are given)."""
    B, Sq, H, fp8, out, lse, _ = _common(q_nope, q_rope, kv_pages, kv_scales, block_table,
                                         cache_seqlens, out, lse, False, 0, num_wg)
    _check(lib().mla_decode_noalloc(
        q_nope.data_ptr(), q_rope.data_ptr(), kv_pages.data_ptr(),
        kv_scales.data_ptr() if fp8 else None, MLA_KV_FP8_E4M3 if fp8 else MLA_KV_BF16,
        kv_pages.shape[0], block_table.data_ptr(), block_table.shape[1], cache_seqlens.data_ptr(),
        B, Sq, H, float(softmax_scale), int(bool(causal)), out.data_ptr(), lse.data_ptr(),
        int(num_wg), _stream(q_nope)))
    return out, lse


def sparse_decode(q_nope, q_rope, kv_pages, block_table, cache_seqlens, indices, softmax_scale,
                  kv_scales=None, out=None, lse=None, workspace=None, num_wg=0, planned=False):
    """DSA top-k absorbed MLA decode over indices [B,Sq,topk]; returns (out, lse)."""
    _req(indices, "indices", (torch.int32,), 3)
    topk = indices.shape[2]
    B, Sq, H, fp8, out, lse, workspace = _common(q_nope, q_rope, kv_pages, kv_scales, block_table,
                                                 cache_seqlens, out, lse, workspace, topk, num_wg)
    if tuple(indices.shape[:2]) != (B, Sq):
        raise ValueError("indices must be [B, Sq, topk]")
    _check(lib().mla_sparse_decode(
        q_nope.data_ptr(), q_rope.data_ptr(), kv_pages.data_ptr(),
        kv_scales.data_ptr() if fp8 else None, MLA_KV_FP8_E4M3 if fp8 else MLA_KV_BF16,
        kv_pages.shape[0], block_table.data_ptr(), block_table.shape[1], cache_seqlens.data_ptr(),
        indices.data_ptr(), topk, B, Sq, H, float(softmax_scale), out.data_ptr(), lse.data_ptr(),
        workspace.data_ptr(), workspace.numel(), int(num_wg), int(bool(planned)), _stream(q_nope)))
    return out, lse


def attend(q_nope, q_rope, kv_pages, block_table, cache_seqlens, softmax_scale, workspace,
           kv_scales=None, indices=None, causal=False, out=None, lse=None, num_wg=0):
    """Main pass only (mla_attend); `workspace` must hold a plan for these sizes."""
    topk = 0
    if indices is not None:
        _req(indices, "indices", (torch.int32,), 3)
        topk = indices.shape[2]
    B, Sq, H, fp8, out, lse, workspace = _common(q_nope, q_rope, kv_pages, kv_scales, block_table,
                                                 cache_seqlens, out, lse, workspace, topk, num_wg)
    _check(lib().mla_attend(
        q_nope.data_ptr(), q_rope.data_ptr(), kv_pages.data_ptr(),
        kv_scales.data_ptr() if fp8 else None, MLA_KV_FP8_E4M3 if fp8 else MLA_KV_BF16,
        kv_pages.shape[0], block_table.data_ptr(), block_table.shape[1], cache_seqlens.data_ptr(),
        indices.data_ptr() if indices is not None else None, topk, B, Sq, H, float(softmax_scale),
        int(bool(causal)), out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
        int(num_wg), _stream(q_nope)))
    return out, lse


def combine(cache_seqlens, B, Sq, H, out, lse, workspace, topk=0, num_wg=0):
    """Split merge only (mla_combine) after attend()."""
    _req(cache_seqlens, "cache_seqlens", (torch.int32,), 1)
    _req(out, "out", (torch.bfloat16,), 4)
    _req(lse, "lse", (torch.float32,), 3)
    _req(workspace, "workspace", (torch.uint8,), 1)
    _check(lib().mla_combine(cache_seqlens.data_ptr(), B, Sq, H, topk, out.data_ptr(),
                             lse.data_ptr(), workspace.data_ptr(), workspace.numel(), int(num_wg),
                             _stream(out)))
    return out, lse


def kv_append(new_kv, kv_pages, block_table, cache_seqlens, kv_scales=None):
    """Write new_kv [B, Sq, 576] (bf16) into the cache slots of the Sq newest
    tokens of every sequence (mla_kv_append); quantises for an fp8 cache."""
    _req(new_kv, "new_kv", (torch.bfloat16,), 3)
    B, Sq, d = new_kv.shape
    if d != 576:
        raise ValueError("new_kv must be [B, Sq, 576]")
    _req(kv_pages, "kv_pages", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), 3)
    if tuple(kv_pages.shape[1:]) != (64, 576):
        raise ValueError("kv_pages must be [num_pages, 64, 576]")
    fp8 = kv_pages.dtype != torch.bfloat16
    if fp8:
        if kv_scales is None:
            raise ValueError("an fp8 cache needs kv_scales")
        _req(kv_scales, "kv_scales", (torch.float32,), 2)
        if tuple(kv_scales.shape) != (kv_pages.shape[0], 64):
            raise ValueError("kv_scales must be [num_pages, 64]")
    _req(block_table, "block_table", (torch.int32,), 2)
    _req(cache_seqlens, "cache_seqlens", (torch.int32,), 1)
    if block_table.shape[0] != B or cache_seqlens.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages] and cache_seqlens [B]")
    _check(lib().mla_kv_append(
        new_kv.data_ptr(), kv_pages.data_ptr(), kv_scales.data_ptr() if fp8 else None,
        MLA_KV_FP8_E4M3 if fp8 else MLA_KV_BF16, kv_pages.shape[0], block_table.data_ptr(),
        block_table.shape[1], cache_seqlens.data_ptr(), B, Sq, _stream(new_kv)))


def dsa_select(block_scores, cache_seqlens, n_select=16, n_init=1, n_local=2, indices=None):
    """Token lists [B, Sq, n_select*64] (int32) for sparse_decode from block
    scores [B, Sq, nbk] (fp32) (mla_dsa_select)."""
    _req(block_scores, "block_scores", (torch.float32,), 3)
    B, Sq, nbk = block_scores.shape
    _req(cache_seqlens, "cache_seqlens", (torch.int32,), 1)
    if cache_seqlens.shape[0] != B:
        raise ValueError("cache_seqlens must be [B]")
    if indices is None:
        indices = torch.empty((B, Sq, n_select * 64), dtype=torch.int32, device=block_scores.device)
    _req(indices, "indices", (torch.int32,), 3)
    if tuple(indices.shape) != (B, Sq, n_select * 64):
        raise ValueError("indices must be [B, Sq, n_select * 64]")
    _check(lib().mla_dsa_select(block_scores.data_ptr(), nbk, cache_seqlens.data_ptr(), B, Sq,
                                int(n_select), int(n_init), int(n_local), indices.data_ptr(),
                                _stream(block_scores)))
    return indices


def _proj(x, w, kin, kout, absorb, out):
    _req(x, "input", (torch.bfloat16,))
    _req(w, "weight", (torch.bfloat16,), 3)
    if x.dim() < 2 or x.shape[-1] != kin:
        raise ValueError(f"input must be [..., H, {kin}]")
    H = x.shape[-2]
    M = x.numel() // (H * kin)
    if tuple(w.shape) != (H, kout, kin):
        raise ValueError(f"weight must be [H, {kout}, {kin}]")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (kout,), dtype=torch.bfloat16, device=x.device)
    _req(out, "out", (torch.bfloat16,))
    if tuple(out.shape) != tuple(x.shape[:-1]) + (kout,):
        raise ValueError("out has the wrong shape")
    f = lib().mla_absorb_query if absorb else lib().mla_project_out
    _check(f(x.data_ptr(), w.data_ptr(), out.data_ptr(), M, H, _stream(x)))
    return out


def absorb_query(q_c, w_uk_t, out=None):
    """q_nope [..., H, 512] = q_c [..., H, 128] . W_UK (w_uk_t is [H, 512, 128]) (mla_absorb_query)."""
    return _proj(q_c, w_uk_t, 128, 512, True, out)


def project_out(out_latent, w_uv, out=None):
    """o [..., H, 128] = W_UV . out_latent [..., H, 512] (w_uv is [H, 128, 512]) (mla_project_out)."""
    return _proj(out_latent, w_uv, 512, 128, False, out)


def layer_workspace_size(B: int, Sq: int, H: int, num_wg: int = 0) -> int:
    return int(lib().mla_layer_workspace_size(B, Sq, H, num_wg))


def decode_layer(q_c, w_uk_t, q_rope, w_uv, kv_pages, block_table, cache_seqlens, softmax_scale,
                 kv_scales=None, causal=False, o=None, lse=None, workspace=None, num_wg=0):
    """The absorbed decode layer (mla_decode_layer): q_c [B,Sq,H,128] -> o [B,Sq,H,128]
    through W_UK (w_uk_t [H,512,128]), the dense decode and W_UV (w_uv [H,128,512]);
    returns (o, lse)."""
    _req(q_c, "q_c", (torch.bfloat16,), 4)
    B, Sq, H, dq = q_c.shape
    if dq != 128:
        raise ValueError("q_c must be [B,Sq,H,128]")
    _req(w_uk_t, "w_uk_t", (torch.bfloat16,), 3)
    _req(w_uv, "w_uv", (torch.bfloat16,), 3)
    if tuple(w_uk_t.shape) != (H, 512, 128) or tuple(w_uv.shape) != (H, 128, 512):
        raise ValueError("w_uk_t must be [H,512,128] and w_uv [H,128,512]")
    dev = q_c.device
    # argument checks of the decode part (q_nope lives in the workspace)
    _req(q_rope, "q_rope", (torch.bfloat16,), 4)
    if tuple(q_rope.shape) != (B, Sq, H, 64):
        raise ValueError("q_rope must be [B,Sq,H,64]")
    _req(kv_pages, "kv_pages", (torch.bfloat16, torch.uint8, torch.float8_e4m3fn), 3)
    if tuple(kv_pages.shape[1:]) != (64, 576):
        raise ValueError("kv_pages must be [num_pages, 64, 576]")
    fp8 = kv_pages.dtype != torch.bfloat16
    if fp8:
        if kv_scales is None:
            raise ValueError("an fp8 cache needs kv_scales")
        _req(kv_scales, "kv_scales", (torch.float32,), 2)
        if tuple(kv_scales.shape) != (kv_pages.shape[0], 64):
            raise ValueError("kv_scales must be [num_pages, 64]")
    _req(block_table, "block_table", (torch.int32,), 2)
    _req(cache_seqlens, "cache_seqlens", (torch.int32,), 1)
    if block_table.shape[0] != B or cache_seqlens.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages] and cache_seqlens [B]")
    if o is None:
        o = torch.empty((B, Sq, H, 128), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)
    _req(o, "o", (torch.bfloat16,), 4)
    _req(lse, "lse", (torch.float32,), 3)
    if tuple(o.shape) != (B, Sq, H, 128) or tuple(lse.shape) != (B, Sq, H):
        raise ValueError("o must be [B,Sq,H,128] and lse [B,Sq,H]")
    if workspace is None:
        n = layer_workspace_size(B, Sq, H, num_wg)
        if n == 0:
            raise MLAError(2, "invalid sizes for the layer workspace")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _req(workspace, "workspace", (torch.uint8,), 1)
    _check(lib().mla_decode_layer(
        q_c.data_ptr(), w_uk_t.data_ptr(), q_rope.data_ptr(), w_uv.data_ptr(), kv_pages.data_ptr(),
        kv_scales.data_ptr() if fp8 else None, MLA_KV_FP8_E4M3 if fp8 else MLA_KV_BF16,
        kv_pages.shape[0], block_table.data_ptr(), block_table.shape[1], cache_seqlens.data_ptr(),
        B, Sq, H, float(softmax_scale), int(bool(causal)), o.data_ptr(), lse.data_ptr(),
        workspace.data_ptr(), workspace.numel(), int(num_wg), _stream(q_c)))
    return o, lse


def prefill(q, k, v, softmax_scale, causal=True, out=None, lse=None):
    """Non-absorbed MHA over per-head q, k [B,T,H,192] and v [B,T,H,128] (mla_prefill);
    returns (out bf16 [B,T,H,128], lse fp32 [B,T,H])."""
    _req(q, "q", (torch.bfloat16,), 4)
    _req(k, "k", (torch.bfloat16,), 4)
    _req(v, "v", (torch.bfloat16,), 4)
    B, T, H, d = q.shape
    if d != 192 or tuple(k.shape) != (B, T, H, 192) or tuple(v.shape) != (B, T, H, 128):
        raise ValueError("q, k must be [B,T,H,192] and v [B,T,H,128]")
    if out is None:
        out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    _req(out, "out", (torch.bfloat16,), 4)
    _req(lse, "lse", (torch.float32,), 3)
    _check(lib().mla_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, float(softmax_scale),
                             int(bool(causal)), out.data_ptr(), lse.data_ptr(), _stream(q)))
    return out, lse
