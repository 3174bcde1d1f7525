"""float64 CPU oracle of the FLARE++ mixer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the benchmark's
CPU-baseline leg. The GPU library never imports or calls anything here.
"""
from .flarepp_oracle import (RMS_EPS, linear, merge_heads, mixer_block, out_project, project, rms_normalize_scaled, sigmoid, split_heads, simplified_mix, simplified_mix_head, mix_backward, mix_head_backward, mix_head_backward_blocked, rms_normalize_backward, sdpa_backward, sdpa_backward_tokens, decode, encode, encode_sharded, flare, gate,
                             mix, mix_head, mixing_matrix, rms_normalize, routing_factors, sdpa,
                             sdpa_tokens, sdpa_tokens_stats, softmax_rows, synthesis)

__all__ = ["RMS_EPS", "linear", "merge_heads", "mixer_block", "out_project", "project", "rms_normalize_scaled", "sigmoid", "split_heads", "simplified_mix", "simplified_mix_head", "mix_backward", "mix_head_backward", "mix_head_backward_blocked", "rms_normalize_backward", "sdpa_backward", "sdpa_backward_tokens", "decode", "encode", "encode_sharded", "flare", "gate", "mix",
           "mix_head", "mixing_matrix", "rms_normalize", "routing_factors", "sdpa", "sdpa_tokens", "sdpa_tokens_stats",
           "softmax_rows", "synthesis"]
