"""CPU oracle for one DFlash 2 draft-verify cycle tail.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (``block_draft_verification_amd``) and never imports it.

Each function is a plain, slow, obviously checkable statement of what one step
of the cycle computes, in float64 unless the step itself fixes another
precision.  Sources, by page:

* tamsi.dev, "DFlash 2 — 3× plus de tokens sur Qwen3.8-27B, même sortie"
  (sections "L'idée, sans le papier" and "Les chiffres qui comptent…");
* myaiexp.com, "DFlash 2" (section 主な機能 / main features, FAQ);
* latenode.com, "DFlash 2: un drafter de 3.43× que cae a 1.45× bajo carga"
  (opening section, "El desacuerdo empieza…", FAQ);
* postsingularityinstitute.com, "Qwen 3.8 27B + DFlash2: 140 Token/Sec?"
  (Résumé, "Apport & nouveautés");
* 0xbakeer.com, DFlash 2 sources list ("Prior art referenced by DFlash 2").

The pages state no formulas; where a step is left open the reading taken is
stated in the function's docstring.  Philox follows Salmon, Moraes, Dror and
Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).

Parity status: every public function here is pinned by ``tests/test_oracle_*``
against closed forms, brute force, library routines or distribution tests;
none is "parity unpinned".
"""

from .conv import conv2tap
from .head import head_logits, head_topk
from .selector import pair_scores, select_path
from .verify import verify_greedy, verify_sample, uniforms
from .philox import philox4x64_10

__all__ = [
    "conv2tap",
    "head_logits",
    "head_topk",
    "pair_scores",
    "select_path",
    "verify_greedy",
    "verify_sample",
    "uniforms",
    "philox4x64_10",
]
