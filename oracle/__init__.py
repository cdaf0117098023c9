"""Double-precision CPU oracle for Reformer's LSH-attention forward pass.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline may import it. The GPU library shares no code with it.
"""
