"""CPU oracle for the EXL3 decode-row projection (rot_in, then the trellis linear).

TEST INFRASTRUCTURE ONLY. The GPU library never imports, links or calls anything
here, and this package imports nothing from the GPU library. Only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.

It is a plain, slow evaluation of the definitions in numpy:
  numfmt   - fp16 / bf16 / fp32 storage formats and round-to-nearest-even
  trellis  - the bit reader (two independent readers) and the mul1-style codebook
  rotation - the 128-point Walsh-Hadamard transform and rot_in's fp32 steps
  linear   - the float64 projection, the fp32 finish and a dense brute force

The method is the one described on the TensorFold pull request "hip exl3: the
input rotation and trellis linear for decode rows, under the kernel contract"
(section "What this changes"). Where that page leaves a step open, the reading
taken here is stated in the docstring of the function that implements it.
"""

from . import numfmt, trellis, rotation, linear  # noqa: F401
