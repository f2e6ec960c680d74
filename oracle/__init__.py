"""CPU oracle for paged KV caching and PagedAttention decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path; both take their inputs from the separate ``workloads`` package.

What it computes, plainly and slowly:

* ``allocator`` -- a pure-Python block allocator: fixed-size blocks, a free
  list, per-block reference counts, per-sequence block tables, copy-on-write
  on the first write to a shared partial block.
* ``kvcache``   -- host mirrors of the K/V pools written bit-for-bit at the
  slots the allocator hands out, a block-copy for copy-on-write, and an
  independent dense per-sequence shadow cache that is never paged.
* ``attention`` -- fp64 softmax(q K^T * scale) V over a sequence's logical
  tokens (gathered through its block table), plus split-K partials and the
  exact partial combine.
* ``capacity``  -- the capacity arithmetic the source pages print.

Sources (cited by title and section throughout):
  [lesson]   "PagedAttention e continuous batching" (llmdeepdive lesson 7.8),
             section "01 · Conceito", paragraphs 1-9;
  [tutorial] "Paged Attention em Large Language Models LLMs" (acheiumaia),
             sections "Configurando as Constantes", "Cache KV Ingênuo";
  [preview]  "04 — Hacia PagedAttention (vista previa)" (lynx-cortex phase 22),
             sections "Lo que funciona en la Fase 22", "Problema 1-3",
             "La idea de PagedAttention" (steps 1-5, "Propiedades"),
             "Lo que deberías llevarte", "Lo que la Fase 22 construye".

Readings taken where the pages are silent are listed in each module and
collected in the design notes.  Every function here is pinned by a
``-m "not gpu"`` test to something other than itself (page numbers,
closed forms, invariants, a library attention routine, a hand-worked
allocator trace); none is "parity unpinned".
"""

from .allocator import AllocError, OracleAllocator  # noqa: F401
from .attention import (  # noqa: F401
    combine_partials,
    decode_attention,
    decode_partials,
    storage_to_f64,
)
from .kvcache import DenseShadow, MirrorPool  # noqa: F401
