"""MI355X-native coalesced attention: one rank's mixed workload of whole
sequences and distributed-attention shards run as one varlen, non-causal
softmax-attention launch, plus the merge of KV-split partials and the
recompute-from-LSE backward.

Importing the package loads nothing native. ``coalesced_attention_amd.zl``
is the thin binding over the C-ABI library ``libzl.so`` and fails loudly
when that library is missing; ``coalesced_attention_amd.workloads`` builds
the seeded synthetic inputs.
"""

__all__ = ["zl", "workloads"]
