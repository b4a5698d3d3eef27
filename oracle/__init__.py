"""Oracle for the per-layer MoE block: a plain, slow fp64 CPU reference.

TEST INFRASTRUCTURE. Only the tests, the smoke check in __graft_entry__ and
the cpu_baseline leg of bench.py may import or run anything in this package.
The library's product path never does, and this package shares no code with
the HIP kernels or the C++ runtime (it reads only the byte formats).

Sources (cited by page and section; the pages are the text of web pages about
arXiv 2609.18063, "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
with Trained Routing Prediction"):
  [Guide]  xyznot.com reading guide of the paper (Turkish, English abstract).
  [News]   ai.info news article "Edge0 serve un MoE da 35B a 20 token al
           secondo in 3 GiB" (Italian).
  [Cache]  twodots.gr article "MoE μοντέλα στην άκρη" (Greek; a different
           paper, used only for the next-token expert reuse figure).

What is pinned and what is not is listed in the header of oracle/moe.py.
"""
from .moe import *  # noqa: F401,F403
