"""MI355X (gfx950) MLA latent-cache decode: C-ABI library + thin binding.

The hot path is three library calls, each a hand-written HIP kernel set:
``mla_absorb_q`` (fold W_UK into the query), ``mla_decode_attention`` (split-KV
attention over the paged latent cache plus the LSE-weighted merge) and
``mla_decompress_v`` (one W_UV decompression).  Upstream of attention,
``mla_cache_append`` writes the new tokens' RmsNorm'd and rope'd latent rows
into the paged cache and rotates the query rope part; ``mla_prefill_attention``
runs the naive (multi-head) form for prefill and chunked prefill;
``mla_decode_attention_dcp`` runs one rank's share of context-parallel decode
and ``mla_lse_combine`` merges the ranks' shares; ``mla_prolog`` is the fused
prolog from hidden states to absorbed queries and cache rows.  See include/mla.h for the
contract of every entry point.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MLA_BF16,
    MLA_DATA_BAD_BLOCK,
    MLA_DATA_BAD_SLOT,
    MLA_DATA_LEN_BELOW_TQ,
    MLA_DATA_LEN_OVER_TABLE,
    MLA_DATA_NEG_LEN,
    MLA_F32,
    MLA_ROPE_INTERLEAVED,
    MLA_ROPE_NEOX,
    MlaError,
    as_dims,
    lib,
    mla_absorb_q,
    mla_cache_append,
    mla_decode_attention,
    mla_decode_attention_dcp,
    mla_decode_attention_noalloc,
    mla_decode_resolve_splits,
    mla_decode_status,
    mla_decode_workspace_size,
    mla_decompress_v,
    mla_default_scale,
    mla_dims,
    mla_lse_combine,
    mla_prefill_attention,
    mla_prefill_workspace_size,
    mla_prolog,
    mla_prolog_dims,
    mla_prolog_workspace_size,
    mla_status_string,
)
