"""Paged K8/V4 KV cache and long-context decode attention for MI355X (gfx950).

``long_context_decode_flash_amd.kvq`` is the binding of the HIP library (``libkvq.so``, built
by ``build.py``); ``long_context_decode_flash_amd.workloads`` draws the seeded synthetic inputs.
"""
