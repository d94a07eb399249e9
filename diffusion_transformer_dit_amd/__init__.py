"""MI355X-native (gfx950) DiT block forward + flow-match Euler denoising step.

The computation lives in libdit.so (hand-written HIP kernels behind the C ABI
of include/dit.h); `native` is its ctypes binding and `runtime` wraps it for
torch-owned device memory.  `inputs` draws the seeded synthetic workloads.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs", "native", "runtime"]


def __getattr__(name):
    # the binding loads libdit.so lazily, so `import diffusion_transformer_dit_amd`
    # works before the library is built (the build step imports the package)
    if name in ("native", "runtime"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
