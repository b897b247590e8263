"""Plain, slow, fp64 CPU oracle for attention over a block-paged KV cache.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The native library never calls it and shares no code with it.

Pages it follows (cited by title and section):
  * "PagedAttention Nedir? Büyük Dil Modelleri GPU Belleğini Nasıl Daha
    Verimli Kullanıyor?" (bitcanli.com) - called "the explainer" below;
  * "Makale Bülteni — PagedAttention ve vLLM" (cmlonder.com radar,
    2026-09-25) - "the PagedAttention newsletter";
  * "Makale Bülteni — vAttention" (cmlonder.com radar, 2026-10-29) - "the
    vAttention newsletter".

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against something other than itself (a worked example on the pages, a closed
form, brute force in exact decimal arithmetic, a library routine, or an
invariant the pages state). None is "parity unpinned".
"""
from . import allocator, attention, fp8, prefix_cache  # noqa: F401
