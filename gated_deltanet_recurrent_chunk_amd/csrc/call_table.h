// call_table.h -- device access to a call's per-sequence table (CallTable, plan.h).
//
// The table travels inside the kernel arguments (inline arrays, read through scalar
// loads from the kernel-argument segment) or, for large batches, as a copy in device
// memory that the host staged into the workspace.  Kernels see one interface either
// way.  Chunks and tiles are derived from a sequence's entry, never looked up.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace gdn {

typedef __attribute__((address_space(4))) const SeqEntry const_seq_entry;
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(4))) const CallTable const_table;

// The call's table, read in place in the kernel-argument segment: every argument block
// that carries one has it as its first member, at offset 0 of the segment.  Its
// address comes from the segment pointer, never from the address of the kernel's
// parameter (which the compiler may copy to private memory once an address of it
// escapes, and a private address is no global one).
__device__ __forceinline__ const_table* kernarg_table() {
  return (const_table*)__builtin_amdgcn_kernarg_segment_ptr();
}

// Entry s (wave-uniform): scalar loads.
__device__ __forceinline__ SeqEntry seq_entry(const_table* t, int s) {
  const const_seq_entry* e = (t->seqs ? (const const_seq_entry*)t->seqs : t->inl_seqs) + s;
  SeqEntry r;
  r.src = e->src;
  r.dst = e->dst;
  r.row0 = e->row0;
  r.p0 = e->p0;
  r.len = e->len;
  r.unit0 = e->unit0;
  r.n_units = e->n_units;
  r.page0 = e->page0;
  r.pad = 0;
  return r;
}

// The sequence that unit u (a chunk or a tile, wave-uniform) belongs to.  Inline
// tables hold at most kInlineSeqs entries and are searched; staged ones carry the map.
__device__ __forceinline__ int unit_sequence(const_table* t, int u) {
  if (t->unit_seq) return *((const const_i32*)t->unit_seq + u);
  int s = 0;
  const int n = t->n_seqs;
#pragma unroll
  for (int i = 1; i < kInlineSeqs; ++i)
    if (i < n && u >= t->inl_seqs[i].unit0) s = i;
  return s;
}

// The page list as a plain global pointer (for vector loads, counted by vmcnt).
__device__ __forceinline__ const int32_t* page_list(const_table* t) {
  return t->pages ? t->pages : (const int32_t*)t->inl_pages;
}

// One chunk of a sequence: packed rows [row, row + len), absolute end position, and
// the checkpoint page index (into the page list) when the chunk ends on a block
// boundary, else -1.
struct ChunkPos {
  int64_t row;
  int32_t len;
  int32_t page_index;
};

// The chunk starting at absolute position pos of the sequence (pos is p0 or a cut).
__device__ __forceinline__ ChunkPos chunk_at(const SeqEntry& e, uint32_t pos, uint32_t block) {
  const uint32_t end = (uint32_t)e.p0 + (uint32_t)e.len;
  const uint32_t stop = next_cut(pos, end, block);
  ChunkPos c;
  c.row = e.row0 + (int64_t)(pos - (uint32_t)e.p0);
  c.len = (int32_t)(stop - pos);
  c.page_index = (block && stop % block == 0) ? e.page0 + (int32_t)boundary_ordinal((uint32_t)e.p0, stop, block) : -1;
  return c;
}

}  // namespace gdn
