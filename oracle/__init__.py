"""fp64 CPU oracle of the selective scan (S6).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP path.  Written from the pages'
definitions (plain recurrence in C, materialised form in numpy/mpmath); shares
no code with the GPU kernels.
"""
