"""CPU oracle for AI.IF join prefill -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation of what the prefill path
computes, written from the Quail pages. It is imported only by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``; the
product path (the HIP library and its binding) never imports, links or runs
anything here, and this package imports nothing from the product.

Pages cited in this package (by title):
  [pt] "Motor de inferência Quail atinge 1 bilhão de tokens por minuto por GPU"
       (stamatios.com), sections "O problema", "Resultados", "Como funciona",
       "Futuro e método".
  [fa] "Quail: یک میلیارد توکن در دقیقه روی یک GPU" (news.ditty.ir), body and
       its key-points list.
  [it] "Quail, il motore di inferenza che supera il miliardo di token al minuto
       su una H100" (flash24.org).
  [de] "Inferenz-Engine Quail schafft eine Milliarde Token pro Minute auf einer
       H100" (flash24.org).
  [pl] "Wyścig o koszt inferencji: Quail osiąga miliard tokenów na minutę ..."
       (flash24.org), section "Praca nad silnikiem, nie nad krzemem".

What the oracle computes (the plain definition the method must reproduce):
per pair, a monolithic causal forward pass over the concatenated tokens
[anchor ‖ suffix], then the 8-column head at the last position, argmax, and the
boolean. The method's three shortcuts -- anchor KV computed once, cascade
attention with an LSE merge, the head cut to 8 columns -- are exact rewrites of
that definition ([pt] "Como funciona", bullets on the query-aware KV cache,
zero decode and simplified cascade attention), so the definition is the oracle.
The cascade form itself is also provided (``attention.cascade_attention``) so
the tests can pin the rewrite against the definition.

Parity status of each function is stated in its module header.
"""
from . import codecs, attention, model, plan, prefix, joinorder  # noqa: F401
