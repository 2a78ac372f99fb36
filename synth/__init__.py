"""Seeded synthetic inputs shared as data by the HIP path's tests and by the oracle.

Holds model shapes, the weights-file writer and the prompt / uniform generators.
It contains none of the model's arithmetic.
"""
from .configs import ModelShape, Workload, WORKLOADS, workload, tiny_variant, TINY, M15B  # noqa: F401
from .weights import write_weights, cached_weights, tensor_specs, file_size  # noqa: F401
from .inputs import prompts, uniforms  # noqa: F401
