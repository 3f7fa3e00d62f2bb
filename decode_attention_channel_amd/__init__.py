"""Channel-pruned (LeanK-style) single-token decode attention for MI355X (gfx950).

Thin Python layer over the C ABI of ``include/leank.h`` (libleank.so): the
functions carry the C names, take torch tensors on the GPU and pass their
pointers plus the current HIP stream.  torch provides device memory and
streams only; every step runs in the library's HIP kernels.

    mask, kept_count, kept_idx = leank_build_mask(alpha, prune_pct, align)
    cache = LayerCache(kept_count[layer].cpu(), kept_idx[layer], batch,
                       n_q_heads, n_kv_heads, n_sink, window, max_ctx)
    leank_pack_k(cache, k_prefill, v_prefill)        # appends, tracks length
    leank_pack_k(cache, k_step, v_step)              # one decode step's token
    out = leank_decode_attn(cache, q)                # float32 [B, Hq, 128]
    out = leank_decode_step(cache, q, k_tok, v_tok)  # append + attend, fused
"""

import ctypes
import math

import torch

from ._lib import (  # noqa: F401
    CHANNEL_QUANTUM,
    HEAD_DIM,
    MAX_GROUP,
    MAX_KV_HEADS,
    PAGE_ROWS,
    QUANT_GROUP,
    LayerCacheDesc,
    LeankError,
    check,
    lib,
    ptr,
    status_string,
    stream_handle,
)

__all__ = [
    "LayerCache",
    "LayerCacheDesc",
    "LeankError",
    "leank_build_mask",
    "leank_plan_layer",
    "leank_plan_layer_q",
    "leank_plan_layer_paged",
    "leank_plan_layer_paged_q",
    "leank_pack_k",
    "leank_workspace_bytes",
    "leank_workspace_init",
    "leank_decode_attn",
    "leank_decode_bytes",
    "leank_pack_k_rows",
    "leank_decode_attn_rows",
    "leank_decode_step",
    "leank_decode_step_noalloc",
    "leank_decode_step_rows",
    "leank_pair_retention",
    "leank_head_hf_ratio",
    "leank_rank_correlation",
    "status_string",
]


def _normalize_device(device):
    device = torch.device(device)
    if device.type == "cuda" and device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    return device


def _require(t, dtype, name, ndim=None, device=None, allow_cpu=False):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not (t.is_cuda or allow_cpu):
        raise TypeError(f"{name} must be a {dtype} tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def leank_build_mask(alpha, prune_pct, align, stream=None):
    """Channel mask from alpha float32 [L, H_kv, d] (synchronous): on the
    GPU for a device tensor (leank_build_mask), on the host for a CPU tensor
    (leank_build_mask_host).

    Returns (mask uint8 [L,H,d], kept_count int32 [L,H], kept_idx int16 [L,H,d]),
    all on alpha's device.
    """
    _require(alpha, torch.float32, "alpha", ndim=3, allow_cpu=True)
    n_layers, n_heads, d = alpha.shape
    mask = torch.empty((n_layers, n_heads, d), dtype=torch.uint8, device=alpha.device)
    kept_count = torch.empty((n_layers, n_heads), dtype=torch.int32, device=alpha.device)
    kept_idx = torch.empty((n_layers, n_heads, d), dtype=torch.int16, device=alpha.device)
    if alpha.device.type == "cpu":
        status = lib().leank_build_mask_host(ptr(alpha), n_layers, n_heads, d, int(prune_pct),
                                             int(align), ptr(mask), ptr(kept_count), ptr(kept_idx))
        check(status, "leank_build_mask_host")
    else:
        status = lib().leank_build_mask(ptr(alpha), n_layers, n_heads, d, int(prune_pct),
                                        int(align), ptr(mask), ptr(kept_count), ptr(kept_idx),
                                        stream_handle(stream))
        check(status, "leank_build_mask")
    return mask, kept_count, kept_idx


def leank_plan_layer(kept_count, batch, n_q_heads, n_kv_heads, head_dim, n_sink, window, max_ctx):
    """Host plan of one layer's cache (head grouping, offsets, byte sizes)."""
    return leank_plan_layer_q(kept_count, batch, n_q_heads, n_kv_heads, head_dim, n_sink, window,
                              max_ctx, 0)


def leank_plan_layer_paged(kept_count, batch, n_q_heads, n_kv_heads, head_dim, n_sink, window,
                           max_ctx, n_pages):
    """Host plan with the middle in pages of 64 rows from a pool of n_pages."""
    counts = [int(c) for c in kept_count]
    if len(counts) != n_kv_heads:
        raise ValueError("kept_count must hold one count per KV head")
    arr = (ctypes.c_int32 * max(1, len(counts)))(*counts)
    desc = LayerCacheDesc()
    check(lib().leank_plan_layer_paged(arr, batch, n_q_heads, n_kv_heads, head_dim, n_sink, window,
                                       int(max_ctx), int(n_pages), ctypes.byref(desc)),
          "leank_plan_layer_paged")
    return desc


def leank_plan_layer_paged_q(kept_count, batch, n_q_heads, n_kv_heads, head_dim, n_sink, window,
                             max_ctx, n_pages, quant_bits):
    """Host plan with a low-bit middle in pages of 64 rows (one K group each)."""
    counts = [int(c) for c in kept_count]
    if len(counts) != n_kv_heads:
        raise ValueError("kept_count must hold one count per KV head")
    arr = (ctypes.c_int32 * max(1, len(counts)))(*counts)
    desc = LayerCacheDesc()
    check(lib().leank_plan_layer_paged_q(arr, batch, n_q_heads, n_kv_heads, head_dim, n_sink,
                                         window, int(max_ctx), int(n_pages), int(quant_bits),
                                         ctypes.byref(desc)),
          "leank_plan_layer_paged_q")
    return desc


def leank_plan_layer_q(kept_count, batch, n_q_heads, n_kv_heads, head_dim, n_sink, window,
                       max_ctx, quant_bits):
    """Host plan with low-bit middle streams (quant_bits 4 or 8; 0 = bf16)."""
    counts = [int(c) for c in kept_count]
    if len(counts) != n_kv_heads:
        raise ValueError("kept_count must hold one count per KV head")
    arr = (ctypes.c_int32 * max(1, len(counts)))(*counts)
    desc = LayerCacheDesc()
    if quant_bits:
        status = lib().leank_plan_layer_q(arr, batch, n_q_heads, n_kv_heads, head_dim, n_sink,
                                          window, int(max_ctx), int(quant_bits),
                                          ctypes.byref(desc))
        check(status, "leank_plan_layer_q")
    else:
        status = lib().leank_plan_layer(arr, batch, n_q_heads, n_kv_heads, head_dim, n_sink,
                                        window, int(max_ctx), ctypes.byref(desc))
        check(status, "leank_plan_layer")
    return desc


class LayerCache:
    """One layer's channel-pruned KV cache, with buffers allocated by torch.

    ``length`` is the number of tokens appended so far (the library itself
    keeps no state).
    """

    def __init__(self, kept_count, kept_idx, batch, n_q_heads, n_kv_heads, n_sink, window,
                 max_ctx, head_dim=HEAD_DIM, device=None, quant_bits=0, n_pages=0,
                 block_table=None):
        """quant_bits 4 or 8: low-bit middle streams.  n_pages > 0: the
        middle in pages of 64 rows from a pool of n_pages pages, mapped by
        block_table (int32 [batch, pages_per_row] on the device; default:
        batch row b's pages contiguous from page b * pages_per_row)."""
        device = _normalize_device(device if device is not None else kept_idx.device)
        if n_pages:
            self.desc = leank_plan_layer_paged_q(kept_count, batch, n_q_heads, n_kv_heads, head_dim,
                                                 n_sink, window, max_ctx, n_pages, quant_bits)
        else:
            self.desc = leank_plan_layer_q(kept_count, batch, n_q_heads, n_kv_heads, head_dim,
                                           n_sink, window, max_ctx, quant_bits)
        _require(kept_idx, torch.int16, "kept_idx", ndim=2, device=device)
        if tuple(kept_idx.shape) != (n_kv_heads, head_dim):
            raise ValueError("kept_idx must be [n_kv_heads, head_dim]")
        self.kept_idx = kept_idx
        self.device = device

        def buf(nbytes):
            return torch.empty(max(1, nbytes // 2), dtype=torch.bfloat16, device=device)

        self.k_sl = buf(self.desc.k_sl_bytes)
        self.v_sl = buf(self.desc.v_sl_bytes)
        self.k_prun = buf(self.desc.k_prun_bytes)
        self.v_mid = buf(self.desc.v_mid_bytes)
        self.desc.kept_idx = kept_idx.data_ptr()
        self.desc.k_sl = self.k_sl.data_ptr()
        self.desc.v_sl = self.v_sl.data_ptr()
        self.desc.k_prun = self.k_prun.data_ptr()
        self.desc.v_mid = self.v_mid.data_ptr()
        self.quant = {}
        if quant_bits:
            for name in ("k_q", "k_qp", "k_stage", "v_q", "v_qp"):
                nbytes = getattr(self.desc, name + "_bytes")
                t = torch.empty(max(16, nbytes), dtype=torch.uint8, device=device)
                self.quant[name] = t
                setattr(self.desc, name, t.data_ptr())
        self.pool = None
        self.block_table = None
        if n_pages:
            self.pool = torch.empty(max(8, self.desc.pool_bytes // 2), dtype=torch.bfloat16,
                                    device=device)
            ppr = self.desc.pages_per_row
            if block_table is None:
                block_table = torch.arange(batch * ppr, dtype=torch.int32,
                                           device=device).reshape(batch, ppr)
            _require(block_table, torch.int32, "block_table", ndim=2, device=device)
            if tuple(block_table.shape) != (batch, ppr):
                raise ValueError(f"block_table must be [batch, {ppr}]")
            self.block_table = block_table
            self.desc.pool = self.pool.data_ptr()
            self.desc.block_table = block_table.data_ptr() if block_table.numel() else 0
        self.length = 0
        self._workspace = None

    # shape shortcuts
    @property
    def batch(self):
        return self.desc.batch

    @property
    def n_q_heads(self):
        return self.desc.n_q_heads

    @property
    def n_kv_heads(self):
        return self.desc.n_kv_heads

    @property
    def max_ctx(self):
        return self.desc.max_ctx

    @property
    def kept_count(self):
        return [self.desc.kept_count[h] for h in range(self.desc.n_kv_heads)]

    def workspace(self):
        """A zero-filled workspace sized for max_ctx (allocated once)."""
        if self._workspace is None:
            nbytes = leank_workspace_bytes(self, self.max_ctx)
            self._workspace = torch.zeros(max(16, nbytes), dtype=torch.uint8, device=self.device)
        return self._workspace

    @property
    def quant_bits(self):
        return self.desc.quant_bits

    def nbytes(self):
        d = self.desc
        return (d.k_sl_bytes + d.v_sl_bytes + d.k_prun_bytes + d.v_mid_bytes + d.k_q_bytes
                + d.k_qp_bytes + d.k_stage_bytes + d.v_q_bytes + d.v_qp_bytes + d.pool_bytes)


def _desc(cache):
    return ctypes.byref(cache.desc if isinstance(cache, LayerCache) else cache)


def leank_pack_k(cache, k_new, v_new, pos0=None, stream=None):
    """Append K, V bf16 [B, H_kv, n, 128] at position pos0 (default: cache.length)."""
    if pos0 is None:
        pos0 = cache.length
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _require(t, torch.bfloat16, name, ndim=4, device=cache.device)
        if tuple(t.shape[:2]) != (cache.batch, cache.n_kv_heads) or t.shape[3] != HEAD_DIM:
            raise ValueError(f"{name} must be [batch, n_kv_heads, n, {HEAD_DIM}]")
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new differ in shape")
    n_new = k_new.shape[2]
    status = lib().leank_pack_k(_desc(cache), ptr(k_new), ptr(v_new), int(pos0), int(n_new),
                                stream_handle(stream))
    check(status, "leank_pack_k")
    cache.length = int(pos0) + int(n_new)


def leank_workspace_bytes(cache, ctx_len):
    out = ctypes.c_size_t(0)
    check(lib().leank_workspace_bytes(_desc(cache), int(ctx_len), ctypes.byref(out)),
          "leank_workspace_bytes")
    return int(out.value)


def leank_workspace_init(workspace, stream=None):
    check(lib().leank_workspace_init(ptr(workspace), workspace.numel() * workspace.element_size(),
                                     stream_handle(stream)), "leank_workspace_init")


def leank_decode_bytes(cache, ctx_len):
    out = ctypes.c_int64(0)
    check(lib().leank_decode_bytes(_desc(cache), int(ctx_len), ctypes.byref(out)),
          "leank_decode_bytes")
    return int(out.value)


def leank_decode_attn(cache, q, ctx_len=None, scale=None, out=None, workspace=None, stream=None):
    """Decode attention for q bf16 [B, Hq, 128]; returns float32 [B, Hq, 128]."""
    if ctx_len is None:
        ctx_len = cache.length
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    _require(q, torch.bfloat16, "q", ndim=3, device=cache.device)
    if tuple(q.shape) != (cache.batch, cache.n_q_heads, HEAD_DIM):
        raise ValueError("q must be [batch, n_q_heads, 128]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    else:
        _require(out, torch.float32, "out", ndim=3, device=cache.device)
        if out.shape != q.shape:
            raise ValueError("out must match q's shape")
    if workspace is None:
        workspace = cache.workspace()
    status = lib().leank_decode_attn(_desc(cache), ptr(q), int(ctx_len), float(scale), ptr(out),
                                     ptr(workspace), workspace.numel() * workspace.element_size(),
                                     stream_handle(stream))
    check(status, "leank_decode_attn")
    return out


# ---------------------------------------------------------------- ragged batches

def leank_pack_k_rows(cache, k_new, v_new, row_pos, row_count=None, stream=None):
    """Append row_count[b] tokens of K, V bf16 [B, H_kv, n, 128] at row_pos[b] per row.

    row_pos: int64 [B] on the GPU (each row's current length); row_count:
    int32 [B] on the GPU with values in [0, n], or None for n everywhere.
    Rows whose positions fall outside the cache are left unchanged.
    """
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _require(t, torch.bfloat16, name, ndim=4, device=cache.device)
        if tuple(t.shape[:2]) != (cache.batch, cache.n_kv_heads) or t.shape[3] != HEAD_DIM:
            raise ValueError(f"{name} must be [batch, n_kv_heads, n, {HEAD_DIM}]")
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new differ in shape")
    _require(row_pos, torch.int64, "row_pos", ndim=1, device=cache.device)
    if row_pos.numel() != cache.batch:
        raise ValueError("row_pos needs one entry per batch row")
    if row_count is not None:
        _require(row_count, torch.int32, "row_count", ndim=1, device=cache.device)
        if row_count.numel() != cache.batch:
            raise ValueError("row_count needs one entry per batch row")
    status = lib().leank_pack_k_rows(_desc(cache), ptr(k_new), ptr(v_new), ptr(row_pos),
                                     ptr(row_count), int(k_new.shape[2]), stream_handle(stream))
    check(status, "leank_pack_k_rows")


def leank_decode_attn_rows(cache, q, ctx_lens, max_ctx_len=None, scale=None, out=None,
                           workspace=None, stream=None):
    """Decode attention with row b over its first ctx_lens[b] tokens (int32 [B] on the GPU).

    max_ctx_len bounds every entry of ctx_lens (default: the cache capacity).
    """
    if max_ctx_len is None:
        max_ctx_len = cache.max_ctx
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    _require(q, torch.bfloat16, "q", ndim=3, device=cache.device)
    if tuple(q.shape) != (cache.batch, cache.n_q_heads, HEAD_DIM):
        raise ValueError("q must be [batch, n_q_heads, 128]")
    _require(ctx_lens, torch.int32, "ctx_lens", ndim=1, device=cache.device)
    if ctx_lens.numel() != cache.batch:
        raise ValueError("ctx_lens needs one entry per batch row")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = cache.workspace()
    status = lib().leank_decode_attn_rows(_desc(cache), ptr(q), ptr(ctx_lens), int(max_ctx_len),
                                          float(scale), ptr(out), ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          stream_handle(stream))
    check(status, "leank_decode_attn_rows")
    return out


# ---------------------------------------------------------------- fused decode step

def _step_token(cache, t, name):
    _require(t, torch.bfloat16, name, device=cache.device)
    shape = tuple(t.shape)
    if shape not in ((cache.batch, cache.n_kv_heads, HEAD_DIM),
                     (cache.batch, cache.n_kv_heads, 1, HEAD_DIM)):
        raise ValueError(f"{name} must be [batch, n_kv_heads, 128] (or with a length-1 token axis)")


def _step_common(cache, q, k_new, v_new, scale, out, workspace, need_workspace=True):
    _require(q, torch.bfloat16, "q", ndim=3, device=cache.device)
    if tuple(q.shape) != (cache.batch, cache.n_q_heads, HEAD_DIM):
        raise ValueError("q must be [batch, n_q_heads, 128]")
    _step_token(cache, k_new, "k_new")
    _step_token(cache, v_new, "v_new")
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    else:
        _require(out, torch.float32, "out", ndim=3, device=cache.device)
        if out.shape != q.shape:
            raise ValueError("out must match q's shape")
    if workspace is None and need_workspace:
        workspace = cache.workspace()
    return scale, out, workspace


def leank_decode_step(cache, q, k_new, v_new, pos=None, scale=None, out=None, workspace=None,
                      stream=None):
    """Append one token per row (K, V bf16 [B, H_kv, 128]) at pos (default:
    cache.length) and return q's attention over the pos + 1 tokens, float32
    [B, Hq, 128] -- the result of leank_pack_k then leank_decode_attn, in
    the two decode kernels."""
    if pos is None:
        pos = cache.length
    scale, out, workspace = _step_common(cache, q, k_new, v_new, scale, out, workspace)
    status = lib().leank_decode_step(_desc(cache), ptr(q), ptr(k_new), ptr(v_new), int(pos),
                                     float(scale), ptr(out), ptr(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     stream_handle(stream))
    check(status, "leank_decode_step")
    cache.length = int(pos) + 1
    return out


def leank_decode_step_noalloc(cache, q, k_new, v_new, pos=None, scale=None, out=None,
                              stream=None):
    """leank_decode_step with the split-K records in the library's own
    device scratch (no workspace, no allocation in the library; out must be
    given by a caller that cannot allocate either).  Calls that overlap on
    one device race."""
    if pos is None:
        pos = cache.length
    scale, out, _ = _step_common(cache, q, k_new, v_new, scale, out, None, need_workspace=False)
    status = lib().leank_decode_step_noalloc(_desc(cache), ptr(q), ptr(k_new), ptr(v_new),
                                             int(pos), float(scale), ptr(out),
                                             stream_handle(stream))
    check(status, "leank_decode_step_noalloc")
    cache.length = int(pos) + 1
    return out


def leank_decode_step_rows(cache, q, k_new, v_new, row_pos, max_ctx_len=None, scale=None,
                           out=None, workspace=None, stream=None):
    """Fused step with row b appending at row_pos[b] (int64 [B] on the GPU)
    and attending over row_pos[b] + 1 tokens; max_ctx_len bounds
    row_pos[b] + 1 (default: the cache capacity).  A row outside that range
    is left unchanged and gets zeros."""
    if max_ctx_len is None:
        max_ctx_len = cache.max_ctx
    scale, out, workspace = _step_common(cache, q, k_new, v_new, scale, out, workspace)
    _require(row_pos, torch.int64, "row_pos", ndim=1, device=cache.device)
    if row_pos.numel() != cache.batch:
        raise ValueError("row_pos needs one entry per batch row")
    status = lib().leank_decode_step_rows(_desc(cache), ptr(q), ptr(k_new), ptr(v_new),
                                          ptr(row_pos), int(max_ctx_len), float(scale), ptr(out),
                                          ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          stream_handle(stream))
    check(status, "leank_decode_step_rows")
    return out


# ---------------------------------------------------------------- host analysis helpers

def _host_array(x, dtype):
    import numpy as np

    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def leank_pair_retention(mask):
    """Per channel-pair retention of a mask uint8 [L, H, d] -> float64 [d/2]."""
    import numpy as np

    m = _host_array(mask, np.uint8)
    n_layers, n_heads, d = m.shape
    out = np.zeros(d // 2, dtype=np.float64)
    check(lib().leank_pair_retention(m.ctypes.data, n_layers, n_heads, d, out.ctypes.data),
          "leank_pair_retention")
    return out


def leank_head_hf_ratio(alpha, n_hf_pairs):
    """Per-head share of |alpha| on the n_hf_pairs highest-frequency pairs -> float64 [L, H]."""
    import numpy as np

    a = _host_array(alpha, np.float32)
    n_layers, n_heads, d = a.shape
    out = np.zeros((n_layers, n_heads), dtype=np.float64)
    check(lib().leank_head_hf_ratio(a.ctypes.data, n_layers, n_heads, d, int(n_hf_pairs),
                                    out.ctypes.data), "leank_head_hf_ratio")
    return out


def leank_rank_correlation(a, b):
    """(Pearson of the values, Pearson of the ranks) of two alpha arrays."""
    import numpy as np

    x = _host_array(a, np.float32).ravel()
    y = _host_array(b, np.float32).ravel()
    if x.size != y.size:
        raise ValueError("a and b differ in size")
    pear, rank = ctypes.c_double(0.0), ctypes.c_double(0.0)
    check(lib().leank_rank_correlation(x.ctypes.data, y.ctypes.data, x.size, ctypes.byref(pear),
                                       ctypes.byref(rank)), "leank_rank_correlation")
    return pear.value, rank.value
