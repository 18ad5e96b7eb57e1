"""Plain, slow CPU oracle for the quantized KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code with the HIP kernels or their host runtime.

What it computes, and from which passage (the pages are cited by title and
section):

* ``rotation``  -- the orthonormal Hadamard rotation of each 256-value head
  vector, per 256-channel half for 512-wide heads (SJ-KVaRN, section 2.2
  "Rotation"), and the randomized Walsh-Hadamard transform on 128 values:
  sign flip, transform, sign flip (KV cache math, "How a 4-bit cache gets
  away with it: rotate first").
* ``tq6``       -- the rotated 6-bit staging format, 98 bytes per 128 values
  (SJ-KVaRN section 2.1, item 2 "Staging").
* ``sinkhorn``  -- Sinkhorn-style balancing of a 128-token x 256-channel tile
  by alternating row and column passes in the log domain (SJ-KVaRN section
  2.2 "Balancing").
* ``rounding``  -- per-row rounding with each row's own fp16 scale and zero
  point (SJ-KVaRN section 2.2 "Rounding", section 2.3 "Scalar body").
* ``record``    -- the byte layout of one sealed 128-token body record.
* ``cache``     -- the four regions (sink, staging ring, exact tail, sealed
  body) and the journaled adaptive seal rule (SJ-KVaRN sections 2.1, 4.3).
* ``attention`` -- float64 decode attention over every region under one
  softmax, in the original domain (SJ-KVaRN section 2.1; KV Cache Precision
  Tail, section 2), and block attention, where each of the newest n_q
  tokens' queries sees the cached tokens up to its own position (prefill
  chunks and verify blocks, HAL #582 section 3b).
* ``sizes``     -- the bytes-per-token and effective-bits arithmetic the pages
  print (SJ-KVaRN sections 1, 3, 7.2, 8.4; KV cache math; HAL #582 section 1).
* ``tq5``       -- the rotated 5-bit comparator block, 82 bytes per 128 values
  (SJ-KVaRN section 6), quantised like the 6-bit staging format.
* ``tbq4``      -- the TBQ4 comparator codec: 128-point randomized
  Walsh-Hadamard rotation, fp16 norm, 16 Lloyd-Max centroids of N(0, 1/128),
  66-byte blocks (KV cache math, "rotate first" and the size table).

Where the pages leave a step open, the plainest reading is taken and stated
in the function that implements it.
"""
