"""CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP library and imports
nothing from it.

Everything here is plain numpy in float64 and follows the pages step by step:

  [SD-review]  "Fast Inference from Transformers via Speculative Decoding"
               (paper review, Leviathan / Kalman / Matias, ICML 2023)
  [PTD]        "Progressive Tree Drafting (PTD)" technical summary
  [SD-EAGLE]   "Speculative Decoding and EAGLE" lesson

Modules
  philox     Philox4x64-10 from its published definition (Salmon et al.,
             "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) and the map
             from a 64-bit word to a float64 uniform in (0, 1).
  tree       ancestor mask and depth from a parent array
             ([SD-EAGLE] "Tree Attention Verification"; [PTD] Method 1,
             "Attention Masking").
  attention  tree-masked attention over a KV cache ([SD-EAGLE] "Tree
             Attention Verification"; [PTD] Method 4, "Verification").
  accept     temperature softmax, the chain accept/reject/resample rule
             ([SD-review] §2; [SD-EAGLE] "The Exactness Rule" and "Build
             it"), the tree rule ([PTD] Method 4, "Acceptance Logic") for
             siblings drawn without replacement, i.i.d., or as fixed
             candidates, and the greedy rule ([SD-EAGLE] "The Exactness
             Rule", greedy case).
  kv_commit  the KV-cache commit after a verify step ([SD-review] §4;
             [SD-EAGLE] "Tree Attention Verification").
  tree_expand  one level of draft-tree construction ([SD-EAGLE] "EAGLE: tree
             drafting and feature reuse"; [PTD] Method 2).
  layer      one target-model layer over the draft nodes: norm, q/k/v
             projection, rotary encoding at depth positions, tree attention,
             output projection, gated MLP ([SD-EAGLE] "Two-Model Setup" step
             2; [PTD] Method 4, "Verification").

Pins (tests marked "not gpu" check each function against something other than
itself): Philox known-answer vectors and numpy's independent Philox; the
hand-derived mask of the six-node tree drawn in [SD-EAGLE]; chain attention ==
torch's causal scaled-dot-product attention; tree attention == causal attention
over each root-to-node path; the exact output law of the accept rule (== p, to
1e-12, by enumeration of draws and decision branches); the closed form
E[tokens] = (1 - a^(K+1)) / (1 - a); empirical TV / chi-square tests; the
greedy rule; inverse CDF == numpy.searchsorted; attention over the committed
cache prefix == the tree-masked verify rows; the layer over a chain == a plain
causal layer written with torch, and over a tree == that layer on each
root-to-node path.  No function here is "parity
unpinned".
"""
