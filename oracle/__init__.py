"""CPU oracle for the Ecco entropy-coded block codec.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the codec computes, written from the pith.science review of
"Ecco: Improving Memory Bandwidth and Capacity for LLMs via Entropy-aware Cache
Compression" (arXiv 2505.06901): the sections "The pith / What carries the
argument", "Core claim", the referee report, "Assumptions & free parameters",
the authors' abstract and the figure captions (Fig. 4, Fig. 6, Fig. 8, Fig. 9).

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it.  The GPU product path never does, and the two
share no code: the oracle derives its own canonical codes, midpoints and
reconstruction values from the same input tables.

Floating-point precision: the pages fix FP16 tensors and FP8 group scales but
not the arithmetic in between.  Every step that decides an integer (argmax,
pattern choice, centroid index, codebook choice, outlier ranking) or produces a
stored bit pattern is done in IEEE binary32 with round-to-nearest-even and no
fused multiply-add, the precision the GPU kernels use; the GEMV reference and
all reported metrics use float64.

Modules
-------
fp        FP8 E4M3FN / FP16 / FP32 conversions
huffman   canonical prefix codes, Kraft sums, optimal length-limited lengths
kmeans    exact 1-D k-means (dynamic programming) and Lloyd k-means
train     pattern and codebook learning (the offline calibration step)
codec     encode / decode of 512-bit blocks, vectorised over groups
literal   the same encode / decode written one group at a time in pure Python
gemv      float64 GEMV over oracle-decoded weights
metrics   reconstruction error, compression ratio, padding and entropy figures
"""

from . import fp, huffman, kmeans, codec, literal, gemv, metrics, train  # noqa: F401
from .codec import Tables, tensor_scale, encode_groups, decode_blocks  # noqa: F401
