"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks."""
from .records import (TOPK, VOCAB, BigSpec, big_chunk, full_step_chunk,
                      full_step_lengths, lmhead_chunk, lmhead_weights,
                      quick_check, stress_chunk, tiny, zipf_bias)
