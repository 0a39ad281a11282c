"""CPU fp64 oracle for grouped-query attention over a bf16 KV cache.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
statement of what the HIP library computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library and its Python binding never do, and this package
never imports them.  It shares no code with the GPU path: the only common
module is ``workloads`` (seeded input generators, no method arithmetic).

Every function works in float64 on the exact values of the bf16 inputs and
cites the passage it follows.  The pages are cited by title:

* [transformer架构]  "Agentic RL入门3：transformer架构" (xiaored5.github.io)
* [注意力变体与MoE]  "注意力变体与 MoE" (notes.cassieliang.com)
* [attention]        "attention" (my-site-6ix.pages.dev, posts/attention)
* [稀疏注意力]        "稀疏注意力：省了什么，没省什么" (geekvape-learning, C11 第5课)
* [注意力机制进化史]  "注意力机制进化史：从MHA、MQA、GQA、MLA到NSA、MoBA！" (CSDN)

Pinned by ``tests/test_oracle_*.py`` against closed forms, printed values
(``tests/golden/``), invariants and an independent library routine.  The only
parts without an external pin ("parity unpinned") are the shape of the YaRN
middle band (the pages say "linear transition" without a formula), QSA's
block-key normalisation (read as L2 to unit length; the page only says
"normalise") and the particular numerical values of the synthetic outputs,
which only this oracle defines.
"""
from . import rope, attention, sparse, qsa, kv_bytes  # noqa: F401
