"""CPU oracle for the MoE decode FFN layer -- TEST INFRASTRUCTURE ONLY.

Importable only by the test suite, the smoke check and the benchmark's
CPU-baseline leg.  The GPU library never imports or links anything here.
"""
