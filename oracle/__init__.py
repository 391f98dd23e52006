"""CPU oracle for query-aware selective sparse attention (ESA and MoBA).

TEST INFRASTRUCTURE ONLY. This package is the slow, plain, float64 statement
of what the GPU library computes. Only the test suite, the smoke check and the
bench's CPU-baseline leg may import it; the product path (the HIP library and
its Python binding) never does, and the oracle imports nothing from the
product. It shares no code with the GPU path: the only common dependency is
the seeded input generator in ``synth``, which holds none of the method's
arithmetic.

Every function cites the passage of the source pages it follows. The pages
(web write-ups of the two methods) are referred to as:

* ESA write-up -- "Efficient Selective Attention" article
  (hlszyjy.com/post/6872.html) and its shorter re-post
  (qqssy.cn/itzixun/132520.html);
* MoBA write-up -- "Mixture of Block Attention" article
  (dtcms.com/wzjs/567377.html), sections 1-4;
* CCA write-up -- "CCA-Attention" ICML 2025 article
  (m.jxzklqfsx.com/article/817694.html);
* attention blog -- "from MLA to CSA" essay (pwwt.cn/news/4222848).

Where a page drops an equation, the reading taken here is stated in the
function's docstring. Parity status per function is listed in the module
docstrings: every function is pinned by a CPU test against something other
than itself except where a module says "parity unpinned".
"""
from . import attention, moba, esa, numerics, cost

__all__ = ["attention", "moba", "esa", "numerics", "cost"]
