"""Error bounds of the GPU parity tests.

The workloads' accuracy target: bf16 max-abs 2e-2, relative RMS 1e-2 and lse max-abs 2e-2;
fp32 1e-5 for each.  Every other bound below comes from the kernels' rounding model
(error_model.py): it is about twice the error the model predicts on that test's own inputs.
test_error_models.py checks this on the CPU: a bound held by one test lies between 2 and 2.5
times its prediction, and a bound shared by a list of cases lies between 2 and 3 times the
largest prediction among them.
"""

TOL = {"f32": dict(max_abs=1e-5, rel_rms=1e-5, lse=1e-5),
       "bf16": dict(max_abs=2e-2, rel_rms=1e-2, lse=2e-2)}

# Forward with inputs of standard deviation 2 and 3 (causal, RoPE): the bf16 rounding of the
# rotated, scaled q and of the rotated k moves each logit by ~2^-9 of its size (~sigma^2),
# the output by that times |v| (~sigma).  Predicted max-abs 8.3e-2 / 0.307, relative RMS
# 5.0e-3 / 7.1e-3, lse 2.8e-2 / 7.9e-2.
LARGE_LOGITS = {2.0: dict(max_abs=0.17, rel_rms=1.1e-2, lse=0.06),
                3.0: dict(max_abs=0.62, rel_rms=1.5e-2, lse=0.16)}

# Logits rising to ~72 nats, every term of q.k with the same sign, so the roundings of q'
# add up instead of cancelling: predicted lse error 6.7e-2 (output within the workload bounds).
RISING_LSE = 0.14

# Every logit near 2^15 (base 2), no RoPE: q' = c * log2(e) / sqrt(d_h) rounds with one
# common relative error of 2.2e-3, which scales every logit and so lse (~22663 nats) by it:
# predicted lse error 49.0.  Only logit differences reach the output (workload bounds).
OFFSET_LSE = 100.0

# Decode over keys whose logits rise by 8.5 (base 2) per block for 8 blocks (lse up to 55):
# predicted lse error 3.3e-2.
DECODE_RISING_LSE = 0.07

# Backward, per gradient tensor: relative RMS, and max-abs relative to the tensor's largest
# reference magnitude (the gradients of early keys sum over thousands of queries, so an
# absolute bound would not carry across lengths).  Where the reference's largest magnitude
# is below scale_floor (an exactly zero gradient, e.g. window 1) the max-abs bound is
# max_rel * scale_floor and the relative RMS is not taken.  Predicted over the backward
# cases: max-abs up to 8.0e-3 of the largest magnitude, relative RMS up to 4.2e-3.
BWD = dict(rel_rms=1.0e-2, max_rel=1.6e-2, scale_floor=1e-2)

# FP8 prefill output: relative RMS and max-abs relative to the largest reference magnitude
# (floored at 1e-2).  The probabilities are rounded to E4M3 (3 mantissa bits) against the
# kernel's lazily held reference, so even the largest probability of a row carries a full
# rounding: predicted over the fp8 cases, max-abs up to 4.2e-2 of the largest magnitude and
# relative RMS up to 2.6e-2.  The logits are exact products of E4M3 values, so lse has no
# rounding of the model's kind (predicted below 1e-6); its bound covers the fp32 sums and
# the hardware exp2 / log2, measured below 6e-5.
FP8 = dict(rel_rms=5.5e-2, max_rel=8.5e-2, lse=1e-3)
