"""Routed mixture-of-experts layer for AMD Instinct MI355X (gfx950).

The layer (routing plan, activation gather, grouped expert FFN, fixed-order
combine) runs in hand-written HIP kernels behind a C ABI
(``include/moe_routed.h``, library ``libmoe_routed.so``). ``abi`` is its
ctypes binding; ``synth`` draws seeded synthetic inputs; ``build`` compiles
the library.
"""
