"""CPU oracle for the batch-1 MoE + FP8 LM-head decode path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, fp64 numpy statement
of what the decode path computes.  Only the test suite, the smoke check of the
package entry point and the CPU-baseline leg of the benchmark may import it.
The product path (the HIP library and its Python binding) never imports, calls
or links anything here, and this package imports nothing from the product.

Sources (web pages on NVIDIA's Ling-3.0-flash decode work on one DGX Spark):
  [saipien]   saipien.org/?p=9636
  [ncij]      ncijnetwork.com, "NVIDIA shows 3 ways to speed up MoE inference
              on DGX Spark, lifting Ling-3.0-flash throughput 42.5%"
  [genai]     generativeaipub.com, "NVIDIA engineers boost MoE inference"
  [sns]       sns.style, "NVIDIA Measures 42.5% More GSM8K Decode Throughput
              on DGX Spark"
Each function names the page section it follows.  Where the pages leave a step
open the docstring states the reading taken.

Parity status per function is listed in each module header; every function
here is pinned by a CPU test against something other than itself.
"""

from . import formats, moe, head, compare, sample, w4a8  # noqa: F401
