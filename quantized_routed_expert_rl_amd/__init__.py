"""Routed mixture-of-experts FFN for AMD MI355X (gfx950).

The hot path lives in the HIP library ``librlmoe.so`` behind the C ABI of
``include/rl_moe.h``; ``binding`` marshals arguments to it.
"""
