"""MI355X-native low-bit KV-cache encode and packed-cache decode attention.

* ``KVCache`` (in ``cache``): torch-facing wrapper; one device buffer per cache.
* ``_binding``: ctypes binding of include/kvq.h (the C ABI of libkvq.so).
* ``synth``: seeded synthetic inputs (no method arithmetic).
* ``build``: compiles libkvq.so for gfx950 with hipcc.

Nothing here computes on the CPU: the encode, dequant and attention steps run
in the HIP kernels of libkvq.so, and a missing library raises.
"""


def __getattr__(name):
    if name == "KVCache":
        from .cache import KVCache
        return KVCache
    raise AttributeError(name)
