"""Plain, slow, fp64 CPU oracle of fine-grained (Mx1-slice / column-sparse) attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call anything in this package.  The library
path (sparse_self_attention_amd) never imports it, and the oracle imports
nothing from the library: the two share no code.

Every function states the passage of the pages it follows (page title plus the
section, figure or comment it falls in).

Readings of passages that the pages leave open:
  * attention is scaled dot-product with scale = 1/sqrt(D), non-causal, no bias;
  * the sparse forward renormalises over the kept keys only (the restricted
    softmax, not a masked full softmax);
  * the pooling threshold "exp(k . q_avg / sqrt D) / D < tau" is read with D as
    the lost softmax denominator: a key is skipped when its pooled softmax
    probability is below tau;
  * a group with no kept keys outputs zeros and lse = -inf;
  * top-k ties go to the lowest key index; index lists are ascending;
  * the cached mask keeps slice (g, j) when some query of group g gives key j a
    full-attention softmax probability of at least tau; tau <= 0 keeps every
    key and a group may keep none;
  * the Chipmunk sparse delta uses the full-softmax form the review asks for:
    probabilities with a stale lse, no renormalisation over the selected keys;
  * the FP8 value path takes bf16 block means, power-of-two channel scales, a
    reference point on the 1/8 grid of log2 units moved by whole log2 units only
    when a byte would pass the largest finite code, and ExpCast bytes with the
    probability scaled by 2^8 (bias 120 instead of 56); oracle/fp8.py states each;
  * the 4-bit QK^T path quantises queries and keys to MXFP4 (E2M1, blocks of 32 along the head
    dimension, power-of-two scales, block maximum to 6); oracle/fp4.py explains why FourOverSix's
    max-to-4 candidate never wins with power-of-two scales.
"""
from .attention import dense_attention_ref, sparse_attention_ref, sparse_attention_probs_ref  # noqa: F401
from .mask import (group_mean_ref, group_scores_ref, topk_select_ref, thresh_select_ref,  # noqa: F401
                   mask_ref)
from .cached import (row_lse_ref, slice_max_logprob_ref, cached_mask_ref, colsum_scores_ref,  # noqa: F401
                     colsum_mask_ref, delta_fresh_ref, delta_forward_ref)
from .fp8 import (e4m3_decode_table, e4m3_encode, bf16_round, channel_scale_exponent,  # noqa: F401
                  vsmooth_quantize_ref, expcast_byte, dequantize_ref, fp8_attention_ref)
from .fp4 import (e2m1_decode_table, e2m1_encode, mx4_quantize_ref, mx4_dequantize_ref,  # noqa: F401
                  fp4_attention_ref)
