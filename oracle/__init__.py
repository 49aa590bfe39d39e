"""CPU oracle of the Julia-1 decision-model forward pass.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path must not.
"""
