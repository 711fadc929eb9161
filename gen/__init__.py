"""Seeded synthetic inputs shared by the CPU reference and the GPU path.

Holds workload shapes and input generators only; no step of the attention
method lives here.
"""

from .configs import BY_INDEX, WORKLOADS, Workload  # noqa: F401
from .fourier import generate, generate_head, kmeans_uniforms, next_step, token_coords  # noqa: F401
