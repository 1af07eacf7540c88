"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench."""
from .inputs import (Problem, block_diag, config1, config2, config3, config3_heads,  # noqa: F401
                     config3_samples, config4, config5, gram, head_grams, random_problem, rng,
                     wishart_gram)
