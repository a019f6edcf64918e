"""MI355X-native exact byte-level BPE tokenization (gfx950 HIP kernels behind a C ABI).

The public entry points mirror include/toktier.h; see ``binding`` for the argument conventions.
"""
from .binding import (EXPORTS, FAMILIES, KERNELS, TOKTIER_CL100K, TOKTIER_DEEPSEEK, TOKTIER_GPT2, TOKTIER_IGNORE_MERGES,
                      TOKTIER_O200K,
                      BucketPlan, HipEvents, Plan, RepairSession, Tokenizer, ToktierError, Vocab, lib, toktier_encode_batch, toktier_encode_batch_spans,
                      toktier_encode_batch_static,
                      toktier_encode_batch_timed, toktier_free_vocab, toktier_last_status, toktier_load_vocab,
                      toktier_load_vocab_ex, toktier_pretokenize_batch, toktier_repair_append,
                      toktier_repair_scratch_bytes, toktier_unicode_table_sha256,
                      toktier_vocab_info, toktier_workspace_bytes, toktier_workspace_bytes_ex)

__all__ = ["EXPORTS", "FAMILIES", "KERNELS", "TOKTIER_CL100K", "TOKTIER_DEEPSEEK", "TOKTIER_GPT2", "TOKTIER_IGNORE_MERGES",
           "TOKTIER_O200K",
           "BucketPlan", "HipEvents", "Plan", "RepairSession", "Tokenizer", "ToktierError", "Vocab", "lib", "toktier_encode_batch",
           "toktier_encode_batch_spans", "toktier_encode_batch_static", "toktier_encode_batch_timed", "toktier_free_vocab", "toktier_last_status",
           "toktier_load_vocab", "toktier_load_vocab_ex", "toktier_pretokenize_batch", "toktier_repair_append",
           "toktier_repair_scratch_bytes", "toktier_unicode_table_sha256",
           "toktier_vocab_info", "toktier_workspace_bytes", "toktier_workspace_bytes_ex"]
