"""MI355X-native dynamic MoE megakernel (event-tensor scheduled).

Importing the package loads nothing native; ``dynamic_moe_task_amd.binding``
loads ``libetc.so`` (the C-ABI library built from ``csrc/``) on first use and
raises if it is missing.  ``workloads`` holds the seeded synthetic input
generators and carries none of the layer's arithmetic.
"""
__all__ = ["binding", "workloads"]
