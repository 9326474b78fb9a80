"""CPU oracle for the hyper-connection residual-stream layer (mHC and xHC).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers, tables or
pre/post-processing); it receives the seeded inputs as plain arrays.

``hc_oracle`` is plain NumPy in float64, written step by step from the
pages' definitions so that it can be checked against them by eye.
``hc_grad`` repeats one xHC sublayer's forward with PyTorch CPU tensors in
float64 and differentiates it (the reference for a backward pass); its
gradients are pinned to central differences of ``hc_oracle``.  Sources,
cited by page title and section:

* [explainer]  "xHC: sixteen residual streams, four written at a time"
               (sections "mHC: keep the mixing doubly stochastic",
               "What xHC changes", "Which constraint survives").
* [xHC paper]  "xHC: Expanded Hyper-Connections" (paragraphs
               "Manifold-Constrained HC", "Mapping generation",
               "Mapping application", "Temporal feature augmentation").
* [summary]    "小红书xHC：时序特征增强 + 稀疏写回" (sections 3.1, 3.3,
               3.4.1-3.4.3), which keeps the shapes of every map.

Every function has a pin in ``tests/test_oracle_*.py`` (closed forms,
invariants, special cases, brute force); none is "parity unpinned".
"""
from .hc_oracle import *  # noqa: F401,F403
