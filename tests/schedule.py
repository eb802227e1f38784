"""The kernels' online-softmax schedule and the parity bars, as test constants."""

# The kernels' online-softmax schedule, fixed by the readings and used as test constants (the
# library's own report of it is asserted to match, never fed into the reference):
#   - 64-key tiles, in increasing key order (one k-scale per tile);
#   - FP16 P against a reference maximum lazy by 8 log2 units (P <= 256);
#   - e4m3 P (FP8 PV and the FP4 method) against the exact running maximum: P = e4m3(448 * p);
#   - the denominator sums the unrounded fp32 probabilities.
BLOCK_N = 64
TAU = {"fp16": 8.0, "fp8": 0.0}
TAU_FP4 = 0
ROWSUM_ROUNDED = False

# Parity bars.  O against the emulation run with the schedule above: relative L1 <= 1e-3 (over
# all compared rows), and per row no more than ROW_TOL -- the kernel differs from the emulation only
# by fp32 rounding (v_exp_f32, MFMA summation order, fused products, and on the FP16 path the
# fp32 rounding of each tile's exponent offset, below half an integer score unit), which can flip
# the rounding of an fp16 or e4m3 P element now and then but cannot move a whole row.  O against the plain
# reading (exact running maximum, tau = 0) within the same 1e-3 bar: for e4m3 P that is the
# schedule itself; for FP16 P the lazy maximum moves only where P is rounded (measured <= 3e-4
# on the CPU, pinned by test_oracle_attn.py::test_qe_fp16_lazy_maximum_within_parity_bar).
# Measured on the GPU over the small, ragged and full-size cases: worst rows 1.2e-3 (FP16 P, an early
# causal row: its keys span two tiles whose exponent offsets round differently) and 1.6e-2 (e4m3 P:
# early causal rows see a handful of keys, where one flipped e4m3 rounding moves a row by percents);
# aggregates up to 1.7e-4 (FP16) and 4e-5 (e4m3).  A wrong row reads of the order of 1.
QE_TOL = 1e-3
ROW_TOL = {"fp16": 3e-3, "fp8": 5e-2}
PLAIN_TOL = 1e-3
