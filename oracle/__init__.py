"""fp64 CPU oracle of the Spark-Attn layer -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's cpu_baseline leg
may import this package.  It shares no code with the HIP library.
"""
from .spark_oracle import *  # noqa: F401,F403
