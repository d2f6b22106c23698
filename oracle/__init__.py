"""CPU oracle of the decode step.  TEST INFRASTRUCTURE: imported only by the
tests, the smoke check and the benchmark's CPU-baseline leg; the GPU library
never uses it."""
from .lo import Oracle, bf16_to_f32  # noqa: F401
