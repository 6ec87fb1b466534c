"""MI355X-native routed mixture-of-experts layer.

Importing the package loads nothing native; ``mixture_experts_route_amd.native``
loads the HIP library (``libmoe_route.so``) and raises if it is missing.
``mixture_experts_route_amd.synth`` holds the seeded synthetic-input generators.
"""

__all__ = ["native", "synth"]
