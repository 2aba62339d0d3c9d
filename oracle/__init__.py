"""CPU oracle for the QLoRA adapted linear layer -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the GPU library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product path.

Every function cites the passage of the source pages it follows.  The pages
are cited by title:

* "LoRA and QLoRA fine-tuning: mechanics, and when not to fine-tune"
  (netleverage.com) -- below "Mechanics"
* "Fine-Tuning on a Budget: LoRA and QLoRA" (adversariallm.ai) -- "Budget"
* "LoRA and QLoRA explained" (sciencenewstoday.org) -- "Explained"
* "LoRA vs QLoRA: Parameter-Efficient Fine-Tuning Explained" (vidman.ai) --
  "PEFT Explained"

Parity status: every function is pinned by a ``-m "not gpu"`` test against
facts the pages or mathematics fix, except the tail probability ``DELTA`` of
the outermost NF4 level, which the pages leave open (parity unpinned; see
``nf4_levels``).
"""

from .qlora_oracle import *  # noqa: F401,F403
