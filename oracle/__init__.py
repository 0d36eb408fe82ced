"""CPU oracle for the fused linear log-prob — TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct reference that the HIP path is
checked against. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``rollout_rlk_linear_amd``) never imports, links or calls anything here, and
this package never imports the product path: the two share no code, header,
table or helper. The seeded input generators live in ``workloads.py`` and
hold none of the method's arithmetic.

What is computed (sources are the three pages on RL-Kernel):

* "VIME Qwen3-8B TP4/CP2 200-round consistency experiment", section
  "User-facing operator matrix": the linear-logp operator stands in for VIME's
  ``calculate_log_probs_and_entropy``, so per token it returns the log-prob of
  the target token and the entropy of the softmax over the vocabulary, with
  logits given by a linear LM head (hidden times the vocabulary weight).
* "RL-Kernel evidence h100-cp-gradient.json", ``validation.runtime_readbacks
  .frameworks['megatron/training'].modules.logp`` (backend
  ``rlkernel.linear_logp.bitwise.v1``): the operator runs in the training
  framework, whose actor-train phase differentiates through it, so a backward
  pass (gradients of hidden and weight) belongs to the op.

Modules:

* ``linear_logp`` — numpy float64 forward, backward, vocabulary-slice partials
  and their merge; every function names the definition it writes out.
* ``brute`` — exact rational logits plus 50-digit decimal exp/ln for tiny
  vocabularies; pins ``linear_logp`` from outside float64.
* ``lora_linear`` — numpy float64 forward and backward of the LoRA linear of
  the page "RL-Kernel h3-runtime-integration-b200 report.json" (key
  ``lora_gate``) and that page's norm-wise relative error.

Every function here is pinned by ``tests/test_oracle.py`` and
``tests/test_oracle_lora.py`` against closed forms, brute force, finite
differences and invariants. No function here is
"parity unpinned".
"""

from .linear_logp import (  # noqa: F401
    decode_bf16,
    forward,
    forward_f64,
    backward,
    backward_f64,
    slice_partials,
    slice_partials_f64,
    merge_partials,
    finalize_partials,
)
from .lora_linear import lora_backward, lora_forward, rel_err  # noqa: F401
