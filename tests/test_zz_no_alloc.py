"""sa_phase2_step_noalloc (the step without a workspace argument, whose chunk
partials live in the library's fixed device array) against sa_phase2_step with
a caller workspace, through the C ABI: two calls in a row, the second with a
smaller input, each compared bit for bit (outputs, LSE and the appended tail
rows) on identical layer states."""
import numpy as np
import pytest
import torch

import workloads as W
from harness import log, to_device
import long_context_attention_amd as sa
from long_context_attention_amd.runner import StarLayer

pytestmark = pytest.mark.gpu


def _pair(w, seed):
    """Two layers holding the same encoded context, and the workload's inputs on the device."""
    x = {k: to_device(v) for k, v in W.all_tensors(w, seed).items()}
    layers = [StarLayer.for_workload(w) for _ in range(2)]
    for layer in layers:
        layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    return layers, x


def _noalloc_step(layer, q, k, v):
    t = q.shape[0]
    out, lse = layer.out[:t], layer.lse[:t]
    sa.sa_phase2_step_noalloc(layer.desc, q, k, v, t, layer.k_cache, layer.v_cache, layer.L, layer.b, layer.k_tail,
                              layer.v_tail, layer.tail_cap, layer.tail_len, out, lse)
    layer.tail_len += t
    return out, lse


def _compare(name, ref_layer, ref, got_layer, got):
    torch.cuda.synchronize()
    for what, a, b in (("out", ref[0], got[0]), ("lse", ref[1], got[1]),
                       ("k_tail", ref_layer.k_tail, got_layer.k_tail), ("v_tail", ref_layer.v_tail, got_layer.v_tail)):
        assert torch.all(torch.isfinite(a.float())) or what == "lse", f"{name} {what}: non-finite reference"
        assert torch.equal(a, b), f"{name} {what}: differs from sa_phase2_step"


def test_noalloc_step_matches_step_with_workspace():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    # Call 1: a 40-token query step (the tile kernel, 320 rows per KV head) on 4 blocks of 512.
    wa = W.Workload("noalloc_a", 130, "bf16", 32, 4, 128, 4 * 512, 512, 512, 40, 2, 5.0e5, True)
    # Call 2, smaller: one decode step on 2 blocks of 256 (the streaming decode kernel, which
    # appends the new row itself), after a query step through sa_phase2_step.
    wb = W.Workload("noalloc_b", 131, "bf16", 8, 2, 128, 2 * 256, 256, 256, 3, 2, 1.0e4, True)
    need_a = sa.sa_workspace_bytes(sa.SA_CALL_PHASE2, StarLayer.for_workload(wa).desc, wa.ctx_len, wa.block_len,
                                   wa.n_query, wa.tail_cap)
    need_b = sa.sa_workspace_bytes(sa.SA_CALL_PHASE2, StarLayer.for_workload(wb).desc, wb.ctx_len, wb.block_len,
                                   1, wb.tail_cap)
    log(f"no-alloc: workspace of call 1 {need_a} B, call 2 {need_b} B (array {sa.SA_NOALLOC_SCRATCH_BYTES} B)")
    assert 0 < need_b < need_a <= sa.SA_NOALLOC_SCRATCH_BYTES

    (ra, na), xa = _pair(wa, 0)
    log("no-alloc call 1: query step, 40 tokens")
    ref = ra.step_fused(xa["q_qry"], xa["k_qry"], xa["v_qry"])
    got = _noalloc_step(na, xa["q_qry"], xa["k_qry"], xa["v_qry"])
    _compare("call 1", ra, ref, na, got)

    (rb, nb), xb = _pair(wb, 1)
    for layer in (rb, nb):
        layer.step_fused(xb["q_qry"], xb["k_qry"], xb["v_qry"])
    log("no-alloc call 2: decode step on a smaller layer")
    ref = rb.step_fused(xb["q_dec"][:1], xb["k_dec"][:1], xb["v_dec"][:1])
    got = _noalloc_step(nb, xb["q_dec"][:1], xb["k_dec"][:1], xb["v_dec"][:1])
    _compare("call 2", rb, ref, nb, got)
    assert np.isfinite(got[1].cpu().numpy()).all()
