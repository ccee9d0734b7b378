"""libstarattn: the Star Attention two-phase attention hot path on one MI355X.

The compute runs in the HIP library ``libstarattn.so`` (built from ``csrc/``);
``_binding`` exposes its C ABI under the same names, ``runner`` keeps the
device buffers of one attention layer and sequences the calls.
"""
from ._binding import (  # noqa: F401
    SA_ANCHOR_FIRST, SA_ANCHOR_PREVIOUS, SA_BF16, SA_MAX_BATCH, decode_seqs, sa_decode_batch_workspace_bytes,
    sa_decode_seq, sa_decode_step_batched, SA_CALL_PHASE1, SA_CALL_PHASE2, SA_EHIP, SA_EINVAL, SA_ENOTSUP,
    SA_EWORKSPACE, SA_F32, SA_OK, StarAttnError, make_desc, sa_abi_version, sa_attn_desc, sa_decode_append,
    sa_last_error, sa_phase1_encode, sa_phase1_encode_anchor, sa_phase1_encode_anchor_at, sa_anchor_at_workspace_bytes,
    sa_phase2_merge, sa_phase2_partial, sa_phase2_step, sa_phase2_step_noalloc, SA_NOALLOC_SCRATCH_BYTES,
    sa_workspace_bytes,
)
