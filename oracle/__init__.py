"""CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The GPU library never
calls it and shares no code with it; the two meet only in the seeded input
generator (``fa_inputs``), which holds no attention arithmetic.

Contents
--------
codecs      decode bf16 and IEEE fp16 bit patterns and OCP E4M3FN codes to float64 from
            their bit fields; dequantise 64-row block-scaled fp8 tensors.
attention   the plain definition O = softmax(scale*Q*K^T)*V with its
            log-sum-exp, in float64, score matrix materialised, two passes
            (max, then exp/sum); the split-KV partials over key ranges and
            their log-sum-exp-weighted merge; single-query decode with
            grouped key/value heads, also over a padded cache with a length
            per sequence; packed batches of sequences with
            unequal query and key lengths (causal masking aligned at the
            sequence end); the gradients dQ, dK, dV of the
            definition (the chain rule through the row softmax, P recomputed
            from Q and K), also for selected query rows (dQ) or selected
            key rows (dK, dV) only, and over packed sequences of unequal
            lengths; the elementwise error bound of
            an fp8-P kernel; attention with only P rounded to E4M3FN (the
            yardstick for an fp8 kernel's mean error).
rotation    incoherent processing for fp8: the random-sign Walsh-Hadamard
            rotation of Q and K along the head dimension, and 64-row block
            quantisation to E4M3FN with a scale of max|x| / 448 or the
            smallest power of two that keeps max|x| / scale <= 448.

Every function is pinned by ``tests/test_oracle*.py`` against brute force,
a library routine (torch's float64 scaled-dot-product attention on the CPU)
and closed-form invariants.  Nothing in here is "parity unpinned".
"""
from .codecs import decode_bf16, decode_e4m3fn, decode_f16, dequant_fp8_rows, round_to_e4m3fn  # noqa: F401
from .attention import (  # noqa: F401
    attention, attention_rows, split_bounds, split_partials, merge_partials,
    decode_attention, decode_attention_gqa, fp8_p_error_bound, fp8_p_attention,
    attention_backward, attention_backward_rows, attention_backward_keys, attention_backward_varlen,
    attention_varlen,
    decode_attention_ragged,
)
from .rotation import (  # noqa: F401
    hadamard_matrix, incoherent_rotation, quantize_e4m3_blocks, smallest_pow2_scale,
)
