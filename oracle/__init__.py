"""CPU oracle of the drafter hot path -- test infrastructure only.

Importable by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg;
never by the product package.
"""
from .dflash_oracle import *  # noqa: F401,F403
from .dflash_oracle import (bf16_round, rmsnorm, rope, silu, argmax_lowest,  # noqa: F401
                            target_layer_ids, fuse_context, inject_kv, block_attention,
                            decoder_layer, draft_block, verify_greedy, prefill,
                            append_context, verify_append_draft, loss_weights, cross_entropy,
                            train_forward,
                            softmax_t, gumbel_sample, sample_inverse_cdf, verify_stochastic,
                            ROUNDING_POINTS)
