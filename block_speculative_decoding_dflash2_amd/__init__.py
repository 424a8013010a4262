"""DFlash2 block draft -> select -> verify step on AMD Instinct MI355X (gfx950).

The computation lives in libdflash2.so (HIP kernels behind the C ABI of
include/dflash2.h); this package is its Python binding.  The binding names
load the library on first use and raise ImportError when it has not been
built (`python -m block_speculative_decoding_dflash2_amd.build`); there is
no CPU fallback."""
import importlib

_FROM_LIB = ("DFlash2Error", "EXPORTED", "LIB_PATH", "dflash2_create", "dflash2_destroy",
             "dflash2_draft_block", "dflash2_draft_losses", "dflash2_draft_losses_workspace_size", "dflash2_last_error", "dflash2_select_path", "dflash2_select_path_stop",
             "dflash2_verify_accept", "dflash2_verify_sample", "dflash2_verify_sample_workspace_size",
             "dflash2_verify_workspace_size", "dflash2_workspace_size")
_FROM_RUNNER = ("DFlash2", "config_struct", "to_device", "verify_accept", "verify_sample", "verify_sample_workspace",
                "verify_workspace")

__all__ = list(_FROM_LIB + _FROM_RUNNER) + ["metrics"]


def __getattr__(name):
    if name in _FROM_LIB:
        return getattr(importlib.import_module("._lib", __name__), name)
    if name in _FROM_RUNNER:
        return getattr(importlib.import_module(".runner", __name__), name)
    if name == "metrics":
        return importlib.import_module(".metrics", __name__)
    raise AttributeError(name)
