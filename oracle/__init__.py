"""Reference oracle for the Stable LatentMoE forward layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow CPU implementation
of what the layer computes, written from the published descriptions of the
method.  Only the test suite, the smoke check and the benchmark's
``cpu_baseline`` leg may import it; the product path (the HIP library and its
Python binding) never imports, calls or links anything in here, and this
package never imports the product.

Sources (cited by page title and section throughout):

* [K3-LatentMoE] dimsnsums.com, "Kimi K3 — LatentMoE" explainer:
  opening section (896 routed experts, 16 active, 2 shared), section
  "Why does the router need three moves?" (latent projection, RMSNorm,
  SiTU-GLU, and the Quantile Balancing paragraph that follows it).
* [Stable-LatentMoE] codewithdark-git.github.io, "Stable LatentMoE" concept
  page: "Key Components" item 4 (SiTU, MXFP4/MXFP8 friendliness) and the
  "Sparsity Comparison" table.
* [K3-structure-5] xhh.club, "Kimi K3 模型结构（5）：宽度维度，Stable LatentMoE":
  the "延伸解读" subsections (half-width latent, the three stabilisers,
  QB vs DeepSeek-V3, parameter scale and deployment) and the Q&A pairs on
  SiTU-GLU, Quantile Balancing, routing, RMSNorm and the shared expert.

Modules:

* :mod:`oracle.qb`     -- fixed-point keys, top-k selection, Quantile
  Balancing (coordinate rounds + exact completion), outputs.
* :mod:`oracle.layer`  -- router, SiTU-GLU, RMSNorm, MXFP4 decoding and the
  whole latent-MoE layer in float64.
* :mod:`oracle.grad`   -- gradients of the layer (autograd over a float64
  PyTorch CPU restatement of the forward pass, selection held fixed) and the
  plain SGD weight update.

Parity status of each function is stated in its docstring.  The pages print
no worked numeric example of the whole layer; its composition is pinned on
weights that are scaled permutation matrices, where the expected output can
be written out by hand.
"""
