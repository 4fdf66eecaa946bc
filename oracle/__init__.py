"""CPU oracle (numpy, float64) for sliding-window attention over a two-pool
paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library or its Python binding.  It
shares no code with the HIP path.

Parity status of each function (what pins it, see tests/test_oracle_pins.py):
  codecs.*            pinned: torch's dtype casts over every bf16 input pattern
  pool_config         pinned: the MiMo-V2-Flash worked example on the SWA note
  translate_loc       pinned: sentinel/tombstone invariants + page-level rebuild
  window_table        pinned: page-level rebuild (slot = page * P + offset)
  kv_store            pinned: round trip and untouched-row invariants
  validate            pinned: hand-counted violations of a hand-built batch
  evict               pinned: hand-worked ranges (both modes, interval, protected
                      prefix), idempotence, and the next window has no tombstone
  unified_*,          pinned: the envelope formula equals view base + kernel id
  envelope_offset     row for row, a byte-exact cross-check of the strided
                      views against rows placed by the envelope formula, the
                      tail pad bound, tombstone clamping, a planted
                      multiplier-1 mistake, and layout-invariant attention
  alloc_extend,       pinned: a hand-worked batch (all three parts, no prefix,
  alloc_decode,       a one-token chunk), a token-by-token allocator written
  alloc_paired,       independently, page size 1 = slicing the free list,
  pages_needed        decode = extend of one token, paired offsets and mapping
  first_key (chunked  pinned: chunk >= T is causal attention, chunk 1 is the
  local attention)    W = 0 closed form, a masked-matrix brute force, the
                      block-diagonal pair count
  ring_*              pinned: the window's positions never share a ring row
                      while they span at most R (brute force), a planted
                      too-small ring collides, ring attention equals two-pool
                      attention on the same rows
  attention           pinned: full-causal reduction, plain-softmax reduction,
                      pure-Python brute force, W=0 and identical-key closed
                      forms, GQA expansion, pair-count ratio ~ 2W/T.
  The sink formula, the 1/sqrt(D) scale and the GQA head map are readings of
  ours (the pages do not spell them out): pinned only through the special cases
  above, i.e. parity unpinned by the pages themselves for those three readings.
"""

from . import codecs, swa_oracle  # noqa: F401
from .swa_oracle import (  # noqa: F401
    NoSpaceError,
    OracleError,
    alloc_decode,
    alloc_extend,
    alloc_paired,
    attend,
    attention,
    decode,
    evict,
    evict_range,
    extend,
    kv_bytes_per_token,
    kv_store,
    first_key,
    pages_bound,
    pages_needed,
    ring_capacity,
    ring_req_to_token,
    ring_rows,
    ring_slot,
    pool_config,
    scored_pairs,
    translate_loc,
    unified_geometry,
    unified_kernel_ids,
    unified_mapping,
    unified_view_base,
    unified_views,
    envelope_offset,
    validate,
    window_range,
    window_table,
)
