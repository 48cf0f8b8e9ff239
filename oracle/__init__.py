"""CPU oracle for the DSA-indexer exact Top-K (test infrastructure).

This package is the correctness authority for the GPU library, nothing more:
only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import it.  It shares no code with the GPU path (no kernels, headers,
helpers or constants); its inputs come from the ``synth`` generators.

What it computes, in float64 on exactly decoded inputs (DoSA pages: the
podcast transcript of "DOSA: Dots Sparse Attention", Method section, problem
statement; the indexer score as defined for the DSA indexer):

    S(t, s) = sum_h w[t, h] * max(0, q[t, h] . k[s])

for every query t and every key s it can see (causal), then a full sort by
(score descending, key index ascending) and the first K keys.  Separately it
implements the DoSA certificate (seed threshold, nonnegative proxy
projections, joint residual bound, negative-head aggregate) in float64, used
to check that bounds dominate scores and that pruning never removes a key the
dense Top-K would keep.

Modules:
    formats      -- fp8 E4M3FN / bf16 / fp32 decoders written from the format definitions
    indexer      -- dense scores and exact Top-K (the plain definition)
    certificate  -- the pruning certificate in float64
"""
