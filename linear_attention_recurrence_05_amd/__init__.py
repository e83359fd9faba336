"""Python binding of libkda, the gfx950 KDA gated delta-rule recurrence.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/kda.h``.  PyTorch supplies device memory
and streams.  If ``libkda.so`` has not been built, importing works but every
call raises :class:`KdaLibraryMissing` -- there is no fallback path.

Functions named like the C entry points take torch tensors in the layouts
``kda.h`` documents and pass their device pointers through unchanged:

    kda_chunk_prefill(q, k, v, z, beta, A, g_min, S0, o, S_T, workspace, stream)
    kda_decode_step(q, k, v, z, beta, A, g_min, S, o, stream)
    kda_decode_tokens(q, k, v, z, beta, A, g_min, S, S_out, o, stream)
    kda_chunk_prefill_paged(q, k, v, z, beta, A, g_min, pool, slots_in, slots_out, o,
                            workspace, stream)
    kda_decode_step_paged(q, k, v, z, beta, A, g_min, pool, slots, o, stream)
    kda_decode_tokens_paged(q, k, v, z, beta, A, g_min, pool, slots_in, slots_out, o, stream)
    kda_gate_chunk_cumsum(z, A, g_min, G, stream)
    kda_intra_chunk(q, k, z, beta, A, g_min, Tm, Aqk, gamma, stream)
    kda_chunk_prefill_workspace_bytes(B, T, H, d_k, d_v, dtype)
    kda_chunk_prefill_segments(B, T, H, d_k, d_v, dtype)
    kda_chunk_prefill_plan(B, T, H, d_k, d_v, dtype)
    kda_chunk_backward(q, k, v, z, beta, A, g_min, S0, dO, dS_T, dq, dk, dv, dz, dbeta, dA,
                       dS0, workspace, stream)
    kda_chunk_backward_workspace_bytes(B, T, H, d_k, d_v, dtype)
    kda_chunk_prefill_segmented(q, k, v, z, beta, A, g_min, S0, o, S_T, n_seg, workspace, stream)
    kda_chunk_prefill_segmented_workspace_bytes(B, T, H, d_k, d_v, n_seg, dtype)

``chunk_prefill``, ``chunk_prefill_segmented``, ``chunk_backward``, ``decode_step`` and
``decode_tokens`` additionally allocate the outputs (and
the workspace) with ``torch.empty`` before calling the same entry points.
"""
from __future__ import annotations

from ._lib import (KDA_BF16, KDA_CHUNK, KDA_F32, KDA_MAX_DECODE_TOKENS, KdaError,
                   KdaLibraryMissing, abi_version, chunk_backward, chunk_prefill,
                   chunk_prefill_segmented, decode_step, decode_tokens, kda_chunk_backward,
                   kda_chunk_backward_workspace_bytes, kda_chunk_prefill_segmented,
                   kda_chunk_prefill_segmented_workspace_bytes,
                   kda_chunk_prefill, kda_chunk_prefill_noalloc, kda_chunk_prefill_paged,
                   kda_chunk_prefill_paged_workspace_bytes, kda_chunk_prefill_plan,
                   kda_chunk_prefill_segments, kda_chunk_prefill_workspace_bytes,
                   kda_decode_step, kda_decode_step_paged, kda_decode_tokens,
                   kda_decode_tokens_paged, kda_gate_chunk_cumsum, kda_intra_chunk, lib,
                   library_path, status_string)

__all__ = ["KDA_BF16", "KDA_CHUNK", "KDA_F32", "KDA_MAX_DECODE_TOKENS", "KdaError",
           "KdaLibraryMissing", "abi_version", "chunk_backward", "chunk_prefill",
           "chunk_prefill_segmented", "kda_chunk_backward", "kda_chunk_backward_workspace_bytes",
           "kda_chunk_prefill_segmented", "kda_chunk_prefill_segmented_workspace_bytes", "decode_step", "decode_tokens",
           "kda_chunk_prefill", "kda_chunk_prefill_noalloc", "kda_chunk_prefill_paged", "kda_chunk_prefill_paged_workspace_bytes",
           "kda_chunk_prefill_plan", "kda_chunk_prefill_segments",
           "kda_chunk_prefill_workspace_bytes",
           "kda_decode_step", "kda_decode_step_paged", "kda_decode_tokens",
           "kda_decode_tokens_paged", "kda_gate_chunk_cumsum", "kda_intra_chunk", "lib",
           "library_path", "status_string"]
