"""Gated DeltaNet gated-delta-rule recurrence on MI355X (gfx950).

The compute path is a HIP library (``libgdn.so``, C ABI in ``include/gdn.h``).
``linear_attention_recurrence_rule_amd.gdn`` is the thin Python binding over it.
"""
