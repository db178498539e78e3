"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy (float64 for arithmetic) restatement of
what the paged KV cache computes, written from the pages' descriptions:

  - "PagedAttention de vLLM : comment la gestion de la VRAM soutient
    l'inférence des grands modèles" (deepsonar.com.cn), §2.1-§2.4, §2.6, §VII;
  - "vLLM transforme la mémoire GPU en système d'exploitation pour LLM"
    (chester-dev.com), section on PagedAttention turning history into blocks;
  - "PagedAttention : comment optimiser la mémoire GPU lors de l'inférence des
    LLM" (deeplearn.tn), worked allocation example, block-table table,
    PagedAttention vs. FlashAttention.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package.  It shares no code with the HIP library and never
imports it; the library never imports this.

Parity status per function (what pins it, see tests/test_oracle_pins.py):
  kvbytes.kv_bytes_per_token   printed values on the page (327,680 B; 2.5 GiB; 250 GiB; x8 MHA)
  lowp.*                       hand-checked bit patterns, ties-to-even cases, a library cast
  allocator.BlockAllocator     worked examples (block size 4 table #42/#7; table 7,2,19,4),
                               waste bound, refcount invariants, brute-force enumeration
  pool.*                       definition of the layouts; element-by-element brute force
  attention.paged_decode       dense attention without a block table (library SDPA in fp64),
                               closed forms, placement and sharing invariance, GQA = MHA
  attention.lse_merge          equality with the one-shot softmax
"""
from . import lowp, kvbytes, allocator, pool, attention, replay  # noqa: F401
