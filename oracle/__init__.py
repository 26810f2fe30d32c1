"""CPU oracle for the compressed-KV GQA decode path — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, deliberately unoptimised restatement of what the source pages define:

  * QEvict ("Resumo Técnico: QEvict"): window partition, cumulative attention scores, three-tier routing under a
    fixed budget, write-once INT2 quantization ledger, promotion/demotion, attention over the mixed cache;
  * CriticalKV ("Resumo Técnico: CriticalKV"): observation-window attention A, projected-value norm |V W_O|_1,
    two-stage selection (Algorithm 1);
  * DBTrimKV ("Make Each Token Count ..."): geometric retention beta^(t-i), one global top-M, per-head
    variable-length paged lists.

Floating point is fp64 throughout, except where a float decides an integer (the INT2 code and the fp16 scale /
zero of a group): those decisions are taken in fp32 exactly as the GPU takes them, because the result must be
byte-exact on both sides.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this package.
The product library never imports, links or calls it, and it shares no code with the HIP path.
"""
