"""CPU oracle for the quantized video-DiT linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, step-by-step NumPy
statement of what the method computes.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library (it imports nothing from ``bit_quantized_linear_vq_amd``), and the
library never calls it.

Steps and the passages they follow:

* ``numerics``  storage-dtype conversions (fp16/bf16 <-> fp32, round-to-nearest-even).
* ``detect``    outlier input channels by modified z-score of channel L2 norms
                (Q-ARVD page, Methodology: outlier-aware adaptive dual-scale quantization).
* ``quantizer`` symmetric absmax quantizer; per-tensor activations, per-channel weights
                (Q-ARVD page, Methodology and Technical details); dual-scale split
                Q_dual(W) = [Q_outlier(W_outliers) | Q_normal(W_normal)] (same passage);
                offline 4-bit weights (6Bit-Diffusion page, Methodology B.1, DMPQ).
* ``fwht``      128-point block Hadamard rotation (6Bit-Diffusion page, Methodology B.1:
                online block Hadamard transform against outliers).
* ``gemm``      exact integer GEMM and the dequantization epilogue
                (Q-ARVD page, Technical details: activation quantization and GEMM/dequantization kernels).
* ``route``     relative-L1 routing statistic Gamma and the INT8-vs-4-bit decision
                (6Bit-Diffusion page, Key Insights 1 and Methodology B.1, DMPQ).
* ``linear``    the whole layer, chaining the steps above.
* ``control``   one block's runtime decision at a timestep: TDC skip test on the cached
                residual deltas, PDR precision overrides, then the DMPQ route
                (6Bit-Diffusion page, Methodology B.1-B.3).
* ``decompose`` residual re-quantization of selected tokens, added back through a
                second accumulator (SemanticDialect page, Methodology 2.2).
* ``calib``     static per-tensor activation scale by clipping-percentile search
                (Q-ARVD page, Technical details: learned clipping percentile and scale).
* ``dense``     the unquantized FP16/BF16 layer of the precision override (6Bit-Diffusion
                page, Methodology B.3, PDR).
* ``mx``        MX block formats (FP4 E2M1, FP6 E2M3, E8M0 block scales of 32) and their
                exact GEMM: the 4-bit floating-point route of the 6Bit-Diffusion page
                (Methodology B.1) in the form gfx950's scaled MFMA consumes.
"""
from . import numerics, detect, quantizer, fwht, gemm, route, linear, decompose, mx, calib, control, dense  # noqa: F401
