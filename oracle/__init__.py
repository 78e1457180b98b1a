"""Oracle for response-replay attention: plain, slow, float64, CPU.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this package.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

Sources (the method's definition):
* LongStraw review page (paper.oopus.info), section 2 "core method" and the
  mind map of section 7 ("Qwen3.6-27B implementation": CP8 block-cyclic page
  ownership; global-LSE softmax recomposition of the forward);
* LongStraw abstract (cortexa.online): exact attention composition,
  response-only objective, prompt state detached;
* DeepRead summary page, "Method": stored prompt state is stopgrad, only the
  response's explicit gradient is kept.

The method reaches exactly (up to rounding order) plain causal softmax
attention of the response rows over [prompt; response], so the forward and
backward here are that plain definition written out in float64 with the score
row fully materialised (two-pass softmax, no online rescaling, no blocking).
See ``attention.py`` for the readings taken where the pages are silent.
"""
from .attention import (  # noqa: F401
    as_f64,
    replay_forward,
    replay_backward,
    partial_stats,
    lse_merge,
    response_kv_grads,
)
from .page_table import split_pages  # noqa: F401
