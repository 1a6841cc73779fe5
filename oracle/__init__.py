"""CPU oracle for the blockwise-scaled FP8 linear layer (quantizers + scaled GEMM).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The GPU library (``blockwise_scaled_fp8_quant_amd``) never imports it
and shares no code, header, table or constant generator with it; the two meet
only through the seeded input generators in ``workloads``.

Plain, slow and obviously correct: NumPy, float32 where the method's steps are
fp32 IEEE operations (scale, reciprocal, scaled value), float64 for the
dequantized GEMM, the E4M3 encode written two independent ways.

Pins (checked by the ``-m "not gpu"`` tests, against things other than this code):
  e4m3.decode_table   OCP E4M3 closed forms for named codes; PyTorch's
                      float8_e4m3fn decoding of all 256 codes; monotonicity.
  e4m3.encode_*       the two encoders agree on a boundary-exhaustive set and on
                      random fp32 patterns; both agree with PyTorch's
                      float8_e4m3fn cast wherever that cast is defined (|v| <= 464);
                      round trip on all 254 finite codes; half-ulp bound.
  quant.*             scaled small integers quantize exactly (closed form); the
                      |x - dec(q) s| <= s (ulp/2 + fp32 slack) bound; every
                      non-degenerate tile reaches the code 448; tile isolation;
                      transpose invariants; block scale == max of its 1x128 scales.
  gemm.*              explicit triple loops in pure Python on tiny shapes; special
                      cases (unit scales -> plain FP8 matmul; one nonzero code per
                      row -> one scaled product; scaled small integers -> exact
                      integer result).
  gemm.operand_norms  the parity bar's denominators: an exact rational per-element
  mx.operand_norms    loop reading each scale from the documented layout; closed
                      forms (unit codes with power-of-two scales; one nonzero code per
                      row); planted layout / decoding mistakes must fail these pins.
  mx.*                MXFP8 (OCP MX v1.0, E4M3 elements, blocks of 32): E8M0 decode
                      against PyTorch's float8_e8m0fnu for all 256 codes; the shared
                      exponent against a brute-force power-of-two search for every
                      finite bf16 amax; block maxima land in [256, 512) and the
                      reconstruction error stays within half an E4M3 ulp (or the
                      saturation distance); scaled small integers are exact; the
                      GEMM against pure-Python triple loops and, with unit scales,
                      the plain FP8 matmul.
Parity unpinned: agreement with Puro's own training numerics (their scale
format, their MXFP8 path) -- the pages print no code, values or error figures.
"""
from . import e4m3, gemm, mx, quant  # noqa: F401
