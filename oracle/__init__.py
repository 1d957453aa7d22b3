"""Float64 CPU oracle for the top-K KL distillation loss over an LM head.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code, tables or helpers with the GPU library and imports nothing from it.

Sources (web pages about arXiv 2608.03796, "Efficient Knowledge Distillation
for LLMs: Offline Top-K Logits and a Fused Chunked KL Loss"):

* [wiki]  llm-wiki study note "LLM 지식 증류 효율화: Offline Top-K Logits와
  Fused Chunked KL Loss로 교사를 메모리에서 꺼내는 방법", sections
  "표준 KD의 손실 함수" (the KD objective KL(P_T || P_S) summed over the
  vocabulary), "핵심 아이디어 1: Offline Top-K Logits" (the cache of K
  (vocab index, logit) pairs per position), "전통적인 KL 손실의 문제" (the
  dense PyTorch form).
* [mv]    mind-verse.de "Optimierung der Wissensdestillation für effiziente
  Sprachmodellkompression", section "2. Ein zusammengeführter, chunked
  KL-Verlust": the dense variant rebuilds a dense teacher probability matrix
  from the cached top-K logits (zero elsewhere) and compares it with the
  student's dense log-probabilities; the three variants compute the same value.
* [abs]   the paper's abstract (chatpaper.ai / Hugging Face papers mirror):
  offline KD caches the teacher's top-K logits once.

Every function here materialises full logit rows (in row blocks) in float64 on
the exact stored input values.  Readings where the pages are silent are listed
in each function's docstring.

Pins: each function is checked in ``tests/test_oracle_pins.py`` and
``tests/test_oracle_variant_pins.py`` against closed forms, library routines,
brute force and finite differences.  No function here
is "parity unpinned".
"""
from .kl import (  # noqa: F401
    logsumexp_rows,
    teacher_probs,
    kl_forward,
    kl_backward,
    kl_dense_reconstruction,
)
from .topk import topk_cache, round_to_bf16, bf16_bits  # noqa: F401
from .variants import counted_rows, variant_forward, variant_backward, renorm_forward, renorm_backward  # noqa: F401
