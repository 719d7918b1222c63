"""Batch-1 decode megakernel for a hybrid Gated-DeltaNet + full-attention decoder on MI355X.

The compute path is the HIP library ``libmk.so`` (C ABI: ``include/mk.h``); this package only
marshals arguments to it (``binding``) and builds it (``build``).  PyTorch provides device
memory and streams.  Importing does not need a GPU; calling into a missing library raises.
"""
from .binding import (MkError, lib_path, load_library, mk_config_from, mk_workspace_bytes,
                      mk_check_tensors, Model)

__all__ = ["MkError", "lib_path", "load_library", "mk_config_from", "mk_workspace_bytes",
           "mk_check_tensors", "Model"]
