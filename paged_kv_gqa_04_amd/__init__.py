"""Paged grouped-query-attention decode for AMD Instinct MI355X (gfx950).

The compute lives in ``libpkv.so`` (hand-written HIP kernels behind the C ABI
of ``include/pkv.h``); this package binds it with ctypes under the same
function names. ``Plan`` and ``decode_step`` are conveniences that use torch
for the workspace allocation and the current stream only.
"""

from __future__ import annotations

from ._pkv import (  # noqa: F401
    COUNTER_STRIDE,
    DTYPES,
    LIB_PATH,
    MODE_NAMES,
    MERGES,
    MODES,
    PKV_BF16,
    PKV_ERR_HIP,
    PKV_ERR_INVALID,
    PKV_ERR_POOL,
    PKV_ERR_STATE,
    PKV_ERR_UNSUPPORTED,
    PKV_ERR_WORKSPACE,
    PKV_F16,
    PKV_MERGE_FUSED,
    PKV_MERGE_KERNEL,
    PKV_MODE_AUTO,
    PKV_MODE_SPLIT,
    PKV_MODE_UNSPLIT,
    PKV_MODE_BUCKETED,
    PKV_MODE_WORKQUEUE,
    PKV_OK,
    STATIC_SCRATCH_BYTES,
    PkvError,
    make_opts,
    make_shape,
    pkv_append,
    pkv_append_prepare,
    pkv_decode,
    pkv_decode_append,
    pkv_decode_marked,
    pkv_decode_static,
    pkv_last_error,
    pkv_paged_read,
    pkv_plan_create,
    pkv_plan_destroy,
    pkv_plan_layout_get,
    pkv_plan_queue_get,
    pkv_plan_stats_get,
    pkv_plan_update,
    pkv_plan_upload,
    pkv_plan_upload_needed,
    pkv_plan_workspace_bytes,
    pkv_pool_alloc,
    pkv_pool_create,
    pkv_pool_destroy,
    pkv_pool_free,
    pkv_pool_free_pages,
    pkv_pool_release_row,
    pkv_status_string,
    pkv_stream_read,
    pkv_version,
)


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


class Plan:
    """Owns a plan handle and (once uploaded) a torch-allocated workspace."""

    def __init__(self, shape, seq_lens_host, opts=None):
        self.handle = pkv_plan_create(shape, seq_lens_host, opts)
        self.workspace = None

    def stats(self) -> dict:
        return pkv_plan_stats_get(self.handle)

    def layout(self) -> dict:
        return pkv_plan_layout_get(self.handle)

    def workspace_bytes(self) -> int:
        return pkv_plan_workspace_bytes(self.handle)

    def update(self, seq_lens_host) -> None:
        pkv_plan_update(self.handle, seq_lens_host)

    def upload(self, device="cuda", stream=None, force=False) -> None:
        """Bind the workspace (allocated here, grown when the plan needs
        more) and copy the queue image into it. Copies nothing when the
        workspace already holds the plan's current image (re-planned with no
        change to it: pkv_plan_upload_needed), unless `force`."""
        import torch
        nb = self.workspace_bytes()
        grown = bool(nb) and (self.workspace is None or self.workspace.numel() < nb)
        if grown:
            self.workspace = torch.empty(nb, dtype=torch.uint8, device=device)
        elif not force and not pkv_plan_upload_needed(self.handle):
            return
        ptr = self.workspace if nb else 0
        pkv_plan_upload(self.handle, ptr, nb, _stream() if stream is None else stream)

    def decode(self, q, k_pool, v_pool, block_table, seq_lens, out, stream=None) -> None:
        pkv_decode(self.handle, q, k_pool, v_pool, block_table, seq_lens, out,
                   _stream() if stream is None else stream)

    def decode_append(self, q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, out,
                      new_seq_lens=None, stream=None) -> None:
        pkv_decode_append(self.handle, q, k_new, v_new, k_pool, v_pool, block_table, seq_lens,
                          out, new_seq_lens, _stream() if stream is None else stream)

    def close(self) -> None:
        if self.handle:
            pkv_plan_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_step(q, k_pool, v_pool, block_table, seq_lens, seq_lens_host, *,
                num_pages=None, sm_scale=0.0, mode="auto", num_splits=0,
                chunk_pages=0, queue_seed=0, merge="fused", out=None):
    """Plan, upload and run one decode step on torch tensors; returns
    ``(out, stats)``. ``q``: [B, Hq, d]; pools: [num_pages, Hkv, 16, d];
    ``block_table``: int32 [B, stride]; ``seq_lens``: int32 [B] (device) with
    the same values as ``seq_lens_host``."""
    import torch
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    dt = "bf16" if q.dtype == torch.bfloat16 else "f16"
    shape = make_shape(B, Hq, Hkv, d, block_table.shape[1],
                       k_pool.shape[0] if num_pages is None else num_pages, dt, sm_scale)
    opts = make_opts(mode, num_splits, chunk_pages, 0, queue_seed, merge)
    if out is None:
        out = torch.empty_like(q)
    with Plan(shape, seq_lens_host, opts) as plan:
        plan.upload(device=q.device)
        plan.decode(q, k_pool, v_pool, block_table, seq_lens, out)
        stats = plan.stats()
        torch.cuda.current_stream().synchronize()
    return out, stats


class Pool:
    """Host page allocator over a pool of ``num_pages`` pages (see pkv.h)."""

    def __init__(self, num_pages: int):
        self.handle = pkv_pool_create(num_pages)

    def free_pages(self) -> int:
        return pkv_pool_free_pages(self.handle)

    def alloc(self, n: int):
        return pkv_pool_alloc(self.handle, n)

    def free(self, pages) -> None:
        pkv_pool_free(self.handle, pages)

    def prepare(self, seq_lens_host, block_table_host, page_size: int = 16) -> int:
        return pkv_append_prepare(self.handle, seq_lens_host, block_table_host, page_size)

    def release_row(self, block_table_row, seq_len: int, page_size: int = 16) -> None:
        pkv_pool_release_row(self.handle, block_table_row, seq_len, page_size)

    def close(self) -> None:
        if self.handle:
            pkv_pool_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover
            pass
