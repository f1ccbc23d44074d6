"""Plain float64 CPU oracle for decode attention over compressed KV caches.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  The library in
``long_context_decode_amd/`` never imports, calls or links anything here, and
nothing here imports the library: the two share no code.  Inputs reach both
sides from the seeded generators in ``synth/``, which hold none of the method's
arithmetic.

Everything is written for clarity, not speed: numpy in float64, one query / one
head at a time where that reads more plainly, no blocking or fusion.

Sources, cited by page title and section:

* [KVC]  "Compressão e Poda Dinâmica de KV Cache: StreamingLLM, SnapKV, PyramidKV e
  DuoAttention" (produtoramaxvision.com.br blog post).
* [SINK] "attention sinks" (tonho.wtf encyclopedia entry on StreamingLLM).
* [KVL]  "O KV cache", lesson 7.2 of llmdeepdive.com.

Pins: each function is checked in ``tests/test_oracle_*.py`` against something
other than itself (printed worked examples under ``tests/golden/``, closed forms,
invariants, special cases that reduce to textbook routines, brute force on tiny
inputs).  No function here is "parity unpinned".
"""
from .kv_memory import kv_cache_bytes  # noqa: F401
from .rope import apply_rope, rope_inv_freq  # noqa: F401
from .attention import (  # noqa: F401
    attend_one,
    causal_attention,
    decode_gqa,
    decode_gqa_rope,
    softmax,
)
from .streaming import (  # noqa: F401
    in_cache_positions,
    retained_tokens,
    ring_slot,
    streaming_decode,
)
from .snapkv import (  # noqa: F401
    observation_attention,
    pool1d,
    select_topk,
    snapkv_compress,
)
from .h2o import H2OBlockHead, H2OHead, h2o_prompt_scores, h2o_prompt_select  # noqa: F401
from .pyramid import pyramid_budgets  # noqa: F401
from .duo import duo_attended_tokens, duo_decode  # noqa: F401
