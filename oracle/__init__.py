"""Plain fp64 CPU oracle for the speculative-decoding verify pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls, links
or executes this package: only the test suite, ``__graft_entry__.smoke()`` and
the benchmark's ``cpu_baseline`` leg use it.  It shares no code, header,
table or constant generator with the HIP library (``verify_pass_sv_amd``) and
never imports it.

Every function is written from the method as the source pages state it and
cites the passage it follows.  Page short names used in the citations:

* "Speculative Decoding Clearly Explained" -- the thread/article that walks
  through draft, verify, accept from left to right, and correct.
* "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling" -- the
  long article (sections "Why batch-one decoding is memory-bound", "How Uzu
  optimizes bytes and tokens per pass", "Producing several tokens from one
  model pass", ...).
* "Local LLM 4x Faster -- Not Through Hardware, but Through Speculative
  Decoding" -- the summary article (153 GB/s / 5.2 GB bound, int8 path, RHT).
* "@trymirai timeline" -- the Mirai Labs post timeline (16-32 token budgets,
  Gumbel-max coupling).

Where the pages leave a step open, the reading taken is stated in the
function's docstring.  Parity status of each function is recorded in its
module header.
"""

from .formats import bf16_bits_to_f64, f16_to_f64
from .philox import philox4x32_10, uniforms24, accept_uniforms
from .qgemm import (unpack_w4, dequant_w4, qgemm_w4, dequant_w8, qgemm_w8,
                    qgemm_w4_i8, group_int_partials)
from .hadamard import sylvester, rht, quantize_per_token, hadamard_i8
from .accept import (row_lse, accept_trial, verify_accept, AcceptResult,
                     NEAR_TIE_ACCEPT, accept_on_probs)
from .sampling import (truncated_probs, greedy_choice, accept_trial_sampled,
                       verify_accept_sampled, sample_drafts, NEAR_TIE_TOP_P)
from .coupled import (gumbel_noise, coupled_choice, coupled_trial, verify_coupled,
                      coupled_drafts, NEAR_TIE_COUPLED)
from .tree import tree_trial, verify_tree
from .lmhead import (group_softmax_stats, merge_group_stats, lm_head_logits, lm_head_verify,
                     NEAR_TIE_LMHEAD)
from .chain import bf16_rne, glue as chain_glue, glue_candidates as chain_glue_candidates
from .roofline import (tokens_per_s_bound, w4_bytes_per_weight,
                       decoder_stack_shapes, stack_weight_count,
                       stack_weight_bytes_w4, stack_weight_bytes_w8)

__all__ = [
    "bf16_bits_to_f64", "f16_to_f64", "philox4x32_10", "uniforms24",
    "accept_uniforms", "unpack_w4", "dequant_w4", "qgemm_w4", "dequant_w8",
    "qgemm_w8", "qgemm_w4_i8", "group_int_partials", "sylvester", "rht",
    "quantize_per_token", "hadamard_i8", "row_lse", "accept_trial",
    "verify_accept", "AcceptResult", "NEAR_TIE_ACCEPT", "accept_on_probs",
    "truncated_probs", "greedy_choice", "accept_trial_sampled",
    "verify_accept_sampled", "sample_drafts", "NEAR_TIE_TOP_P", "gumbel_noise",
    "coupled_choice", "coupled_trial", "verify_coupled", "coupled_drafts",
    "NEAR_TIE_COUPLED", "tree_trial", "verify_tree", "group_softmax_stats",
    "merge_group_stats", "lm_head_logits", "lm_head_verify", "NEAR_TIE_LMHEAD",
    "tokens_per_s_bound", "bf16_rne", "chain_glue", "chain_glue_candidates",
    "w4_bytes_per_weight", "decoder_stack_shapes", "stack_weight_count",
    "stack_weight_bytes_w4", "stack_weight_bytes_w8",
]
