// Private tables of libcpattn: layouts inside the metadata blob that the host
// builder writes and the kernels read.  Not part of the public ABI.
#pragma once
#include <stdint.h>

namespace cpattn {

// One zigzag chunk = one block of one sequence, in original token order.
// Its rows are contiguous both in the all-gathered buffer and in original
// order, so every copy of the path is a set of contiguous row runs.
struct Chunk {
  int32_t b;        // sequence
  int32_t t0;       // first extend token of the block within sequence b
  int32_t g_row;    // first row in the all-gathered (rank-major, padded) buffer
  int32_t o_row;    // first row in original order (sequences concatenated)
  int32_t n_rows;   // block size
  int32_t pos0;     // sequence position of t0 (prefix_b + t0): KV-pool slot index
  int32_t pad0, pad1;
};
static_assert(sizeof(Chunk) == 32, "Chunk layout");

// One attention segment: q_len query rows of one zigzag half of one
// sequence (or of one document of the AllGather-KV slice) against kv_len
// keys of that sequence, starting at key kv_start of its page-table row.
struct Seg {
  int32_t q_row0;      // first local row in Q/O
  int32_t q_len;       // rows that attend
  int32_t q_rows;      // rows owned; rows in [q_len, q_rows) are written as zeros
  int32_t kv_len;      // keys 0..kv_len-1 are visible (before the causal mask)
  int32_t causal_off;  // kv_len - q_len: row i sees keys j <= i + causal_off
  int32_t page_row;    // row of the CSR page table (the sequence)
  int32_t causal;      // 1: bottom-right causal mask, 0: none
  int32_t kv_start;    // key j of the segment is position kv_start + j of the page-table row
};
static_assert(sizeof(Seg) == 32, "Seg layout");

// One attention work item: positions [p0, p0+np) of segment seg, for one KV
// head (the head comes from the workgroup index), visiting n_tiles key tiles.
struct Work {
  int32_t seg;
  int32_t p0;
  int32_t np;
  int32_t n_tiles;
};
static_assert(sizeof(Work) == 16, "Work layout");

// Attention tiling shared by the work-list builder and the kernel.
constexpr int kAttnRows = 256;     // (position, head) rows per workgroup: 8 waves x 32
constexpr int kAttnKeys = 64;      // keys per KV tile
constexpr int kMaxGroup = kAttnRows;  // H_q / H_kv upper bound (one position per workgroup)

constexpr uint32_t kBlobMagic = 0x31415043u;  // "CPA1"
constexpr int64_t kBlobAlign = 256;

// Job counters of the attention launch, inside the blob's 256-byte header:
// words 0-7 are the next place in each of the 8 job queues, word 8 counts the
// workgroups that have taken a ticket.  The builder writes them as zero and
// every launch leaves them zero.
constexpr int64_t kCtrOffset = 128;
constexpr int kCtrWords = 9;
static_assert(kCtrOffset + 4 * kCtrWords <= kBlobAlign, "counters fit in the header");

// Error helpers (cp_meta.cpp).
int set_error(int code, const char* fmt, ...);
void clear_error();

}  // namespace cpattn
