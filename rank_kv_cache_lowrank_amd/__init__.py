"""MI355X (gfx950) decode attention over a low-rank latent KV cache.

The kernels and the C ABI live in ``csrc/`` (built into ``liblowrank_attn.so``
by ``build.build()``); ``_lib`` is the ctypes binding with the same entry-point
names as ``include/lowrank_attn.h``.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LR_BF16, LR_EHIP, LR_EINVAL, LR_EUNSUPPORTED, LR_EWORKSPACE, LR_F32, LR_I4G32, LR_OK,
    Cache, LowRankError, Model, latent_storage, load, lowrank_abi_version, lowrank_attn_decode,
    lowrank_attn_decode_workspace_size, lowrank_attn_decode_noalloc, NOALLOC_SCRATCH_BYTES, lowrank_attn_prefill, lowrank_attn_prefill_workspace_size,
    lowrank_kv_append, lowrank_decode_step, lowrank_kv_dequant, lowrank_kv_rebase, lowrank_basis_update,
    lowrank_basis_update_workspace_size, lowrank_rank_allocate,
    lowrank_rank_allocate_workspace_size, lowrank_sens_svd, lowrank_sens_svd_workspace_size,
    lowrank_sens_svd_batched, lowrank_sens_svd_batched_workspace_size,
    lowrank_kv_store,
    lowrank_last_error, prefill_workspace, workspace)
