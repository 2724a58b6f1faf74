"""Sink attention (GQA + learned per-head sink) for AMD MI355X (gfx950).

The compute path is the HIP library ``libsinkattn.so`` built from ``csrc/``;
``binding`` marshals torch tensors into its C ABI.  Importing this package
does not load the library; the first call does, and raises if it is missing.
"""

__version__ = "0.1.0"


def __getattr__(name):
    if name in ("prefill_varlen", "decode_splitkv", "merge_lse", "decode_workspace_bytes",
                "library", "SinkAttnError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
