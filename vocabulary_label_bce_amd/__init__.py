"""MI355X-native fused full-vocabulary binary cross-entropy (CutBCE hot path).

The compute lives in a HIP library for gfx950 (``csrc/``, built to ``libcutbce.so``) behind a C ABI
(``include/cutbce.h``). ``binding`` marshals arguments to it with ctypes; ``ops`` wraps forward/backward in a
``torch.autograd.Function``. ``workloads`` draws seeded synthetic inputs. Importing this package does not load
the library; the first call into ``binding`` does, and raises if it has not been built.
"""
__all__ = ["binding", "ops", "workloads", "build"]
