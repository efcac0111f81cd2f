"""MI355X-native MoE expert-parallel dispatch / combine (DeepEP-style token exchange).

The hot path -- dispatch layout, dispatch (with fused BF16->FP8 e4m3 pack),
combine (fp32 weighted gather-reduce to BF16) and the backward pair -- runs in
hand-written HIP kernels for gfx950 behind the C ABI declared in include/ep.h.

Submodules:
  ep         ctypes binding of libep.so (same names as the C ABI) plus a small
             torch-tensor convenience wrapper (argument marshalling only)
  workloads  seeded synthetic inputs (routing, activations, gradients)
  build      compiles libep.so with hipcc for gfx950

Nothing is loaded at import time; ``ep.load()`` raises if libep.so is missing.

Usage (torch tensors on the GPU; every call is asynchronous on torch's
current stream, and the outputs are caller-owned tensors)::

    from combine_get_dispatch_amd import ep
    buf = ep.Buffer(num_tokens, hidden, num_topk, num_experts, num_ranks, cap_rows)
    # x [T, H] bf16, topk_idx [T, k] int32 (-1 = no expert), topk_w [T, k] fp32
    layout, recv_x, recv_scales, recv_w, handle = buf.dispatch_with_layout(
        x, topk_idx, topk_w, use_fp8=True)
    # ... the experts turn rank d's rows [d*cap_rows, d*cap_rows + rank_rows[d])
    #     of recv_x / recv_scales into expert_out [R*cap_rows, H] bf16 ...
    y = buf.combine(expert_out, handle, topk_w)            # [T, H] bf16
    grad_rows = buf.combine_backward(grad_y, handle)       # backward of combine
    grad_x = buf.dispatch_backward(grad_expert_in, handle, topk_w)
    assert buf.status() == 0                               # sticky device status

The rank-deduplicated exchange (``dispatch_dedup_with_layout``: one row per
(token, destination rank) with the row's local expert indices and weights)
and the low-latency form (``dispatch_low_latency``: fixed per-(expert,
source) regions, one launch, graph-capturable) return handles that
``combine`` and the backward pair take the same way.
"""
__all__ = ["ep", "workloads", "build"]
