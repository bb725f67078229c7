"""Spark-Attn block-sparse attention layer for MI355X (gfx950).

The compute lives in libspark.so (hand-written HIP kernels behind the C ABI of
include/spark.h); this package is its thin ctypes binding plus the seeded
synthetic workload generator.
"""
from ._lib import (  # noqa: F401
    SparkError, SparkArgs, lib, last_error, make_args, n_blocks, topk_from_ratio, workspace_bytes,
    spark_reblock, spark_select, spark_summarize, spark_attn, spark_layer, spark_moments,
    spark_msqrt, spark_whiten, spark_split, spark_gather, EXPORTED,
)

__version__ = "1.0.0"
