"""Routed-expert MoE layer forward on one AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of libmoe.so
(include/moe.h); ``binding`` is the thin ctypes layer over it with the same
call names.  Importing ``binding`` fails if the library has not been built
(``python -m routing_dispatch_expert_logits_amd.build``); there is no other
execution path.
"""
__all__ = ["binding", "build"]
