"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench."""
from .inputs import (Problem, config1, config2, config3, config3_samples, config4, config5,  # noqa: F401
                     gram,
                     random_problem, rng, wishart_gram)
