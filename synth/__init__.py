"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench."""
from .inputs import (Problem, config1, config2, config3, config4, config5, gram,  # noqa: F401
                     random_problem, rng, wishart_gram)
