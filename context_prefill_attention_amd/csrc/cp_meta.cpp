// Host-side zigzag context-parallel metadata (no device access).
//
// Follows the sglang zigzag.py source page: the block layout of its module
// docstring, ZigzagCPStrategy.can_apply (validity) and
// ZigzagCPStrategy.build_metadata (split_list, per_rank_actual_token,
// max_rank_len, zigzag_index, cp_reverse_index, reverse_split_len, per-half
// kv and q lengths, cu_seqlens).  Everything lands in one caller-owned host
// blob that the caller copies to the device in one transfer; the "Zigzag cp
// #3" pull request page motivates this (lengths as host values, no per-call
// tensor construction, no device-to-host sync).
//
// Besides the page's lists the blob holds this library's tables: the chunk
// table (contiguous row runs for rerange and scatter), the attention segment
// table and a longest-first attention work list.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/cpattn.h"
#include "cp_internal.h"

namespace cpattn {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

namespace {

constexpr int64_t kI32Max = 2147483647LL;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Byte layout of a blob: offsets of each array, assigned in order.
struct Layout {
  int64_t cursor = kBlobAlign;  // the first 256 bytes hold a small header
  int64_t take(int64_t bytes) {
    int64_t off = cursor;
    cursor = align_up(cursor + std::max<int64_t>(bytes, 0), kBlobAlign);
    return off;
  }
};

struct Header {
  uint32_t magic;
  int32_t version, kind, n_chunks, n_seg, n_work, cp_size, bs;
};
static_assert(sizeof(Header) <= kCtrOffset, "the header stays clear of the job counters");

// Work list for one attention call: segments cut into items of q_tile
// positions, each with the number of key tiles it visits, ordered longest
// first so that the hardware's in-order dispatch approximates LPT scheduling.
void build_work(const std::vector<Seg>& segs, int q_tile, std::vector<Work>& work) {
  work.clear();
  for (int s = 0; s < (int)segs.size(); ++s) {
    const Seg& g = segs[s];
    for (int p0 = 0; p0 < g.q_rows; p0 += q_tile) {
      const int np = std::min(q_tile, g.q_rows - p0);
      int64_t kv_end;
      if (p0 >= g.q_len) {
        kv_end = 0;  // only rows past q_len: written as zeros, no keys visited
      } else if (g.causal) {
        const int64_t last = std::min<int64_t>(p0 + np, g.q_len) - 1;
        kv_end = std::min<int64_t>(g.kv_len, last + g.causal_off + 1);
      } else {
        kv_end = g.kv_len;
      }
      work.push_back(Work{s, p0, np, (int32_t)((kv_end + kAttnKeys - 1) / kAttnKeys)});
    }
  }
  std::stable_sort(work.begin(), work.end(),
                   [](const Work& a, const Work& b) { return a.n_tiles > b.n_tiles; });
}

// Mean key tiles per work item, rounded down (0 for an empty list).
int32_t mean_item_tiles(const std::vector<Work>& work) {
  if (work.empty()) return 0;
  int64_t sum = 0;
  for (const Work& w : work) sum += w.n_tiles;
  return (int32_t)(sum / (int64_t)work.size());
}

int check_group(int32_t g, bool allow_zero) {
  if (g < (allow_zero ? 0 : 1) || g > kMaxGroup)
    return set_error(CP_ERR_UNSUPPORTED, "attn_group=%d outside [%d, %d]", g,
                     allow_zero ? 0 : 1, kMaxGroup);
  return CP_OK;
}

constexpr int32_t kKvAlignMax = 1 << 30;   // kv_align when every segment starts at key 0

void write_i32(void* blob, int64_t off, const std::vector<int32_t>& v) {
  if (!v.empty()) std::memcpy(static_cast<char*>(blob) + off, v.data(), v.size() * 4);
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" int cp_meta_build(int32_t cp_size, int32_t cp_rank, int32_t bs,
                             const int32_t* extend_lens, const int32_t* seq_lens,
                             int64_t num_tokens, int32_t attn_group,
                             void* blob, int64_t blob_capacity, cp_meta_t* meta) {
  clear_error();
  if (!meta) return set_error(CP_ERR_INVALID_ARG, "meta is NULL");
  if (cp_size < 2)
    return set_error(CP_ERR_INVALID_ARG, "cp_size=%d: zigzag CP needs at least 2 ranks", cp_size);
  if (cp_rank < 0 || cp_rank >= cp_size)
    return set_error(CP_ERR_INVALID_ARG, "cp_rank=%d outside [0, %d)", cp_rank, cp_size);
  if (bs < 1) return set_error(CP_ERR_INVALID_ARG, "bs=%d must be >= 1", bs);
  if (!extend_lens) return set_error(CP_ERR_INVALID_ARG, "extend_lens is NULL");
  if (int rc = check_group(attn_group, true)) return rc;
  const int nblk = 2 * cp_size;
  if ((int64_t)bs * nblk > kI32Max) return set_error(CP_ERR_OVERFLOW, "bs*2*cp_size overflows int32");

  // Validity (can_apply): every sequence and the batch give each block >= 1 token.
  std::vector<int64_t> ext(bs), seq;
  int64_t sum_ext = 0;
  for (int b = 0; b < bs; ++b) {
    if (extend_lens[b] < nblk)
      return set_error(CP_ERR_INVALID_ARG, "extend_lens[%d]=%d is shorter than 2*cp_size=%d",
                       b, extend_lens[b], nblk);
    ext[b] = extend_lens[b];
    sum_ext += ext[b];
  }
  if (num_tokens < sum_ext)
    return set_error(CP_ERR_INVALID_ARG, "num_tokens=%lld is smaller than sum(extend_lens)=%lld",
                     (long long)num_tokens, (long long)sum_ext);
  if (seq_lens) {
    seq.resize(bs);
    for (int b = 0; b < bs; ++b) {
      if (seq_lens[b] < 0) return set_error(CP_ERR_INVALID_ARG, "seq_lens[%d] < 0", b);
      seq[b] = seq_lens[b];
    }
  }
  // The batch's surplus rows belong to the last sequence (its full length
  // grows by the same amount, so its cached prefix is unchanged).
  const int64_t surplus = num_tokens - sum_ext;
  ext[bs - 1] += surplus;
  if (seq_lens) seq[bs - 1] += surplus;
  if (num_tokens > kI32Max) return set_error(CP_ERR_OVERFLOW, "num_tokens >= 2^31");

  std::vector<int64_t> prefix(bs, 0);
  for (int b = 0; b < bs; ++b) {
    if (seq_lens) prefix[b] = std::max<int64_t>(seq[b] - ext[b], 0);
    if (prefix[b] + ext[b] > kI32Max)
      return set_error(CP_ERR_OVERFLOW, "sequence %d: prefix + extend >= 2^31", b);
  }

  // Block j of sequence b: base tokens, plus one for the first L mod 2cp blocks.
  auto blk = [&](int b, int j) -> int64_t {
    const int64_t base = ext[b] / nblk, rem = ext[b] % nblk;
    return base + (j < rem ? 1 : 0);
  };
  auto early = [](int r) { return r; };
  auto late = [nblk](int r) { return nblk - 1 - r; };

  // Rows each rank contributes to the all-gather; the max is the pad target.
  std::vector<int32_t> per_rank(cp_size);
  int64_t mrl = 0;
  for (int r = 0; r < cp_size; ++r) {
    int64_t n = 0;
    for (int b = 0; b < bs; ++b) n += blk(b, early(r)) + blk(b, late(r));
    per_rank[r] = (int32_t)n;
    mrl = std::max(mrl, n);
  }
  if (mrl * cp_size > kI32Max)
    return set_error(CP_ERR_OVERFLOW, "all-gathered rows cp_size*max_rank_len >= 2^31");

  std::vector<int32_t> split_list(bs * nblk), zigzag_index(2 * bs);
  for (int b = 0; b < bs; ++b)
    for (int j = 0; j < nblk; ++j) split_list[b * nblk + j] = (int32_t)blk(b, j);
  for (int b = 0; b < bs; ++b) {
    zigzag_index[b] = b * nblk + early(cp_rank);
    zigzag_index[bs + b] = b * nblk + late(cp_rank);
  }

  // Where each original chunk sits in the all-gathered buffer.  Rank r's
  // local rows are [early block of seq 0..bs-1, late block of seq 0..bs-1],
  // so the gathered chunk position of (b, block j) is owner*2bs + b for an
  // early block and owner*2bs + bs + b for a late one.
  std::vector<int32_t> reverse_index(bs * nblk), reverse_split(bs * nblk);
  std::vector<Chunk> chunks(bs * nblk);
  {
    // cum_early[r][b] / cum_late[r][b]: rows of rank r's early / late blocks
    // of sequences before b.
    std::vector<int64_t> cum_early((size_t)cp_size * (bs + 1)), cum_late((size_t)cp_size * (bs + 1));
    for (int r = 0; r < cp_size; ++r) {
      int64_t* ce = &cum_early[(size_t)r * (bs + 1)];
      int64_t* cl = &cum_late[(size_t)r * (bs + 1)];
      ce[0] = cl[0] = 0;
      for (int b = 0; b < bs; ++b) {
        ce[b + 1] = ce[b] + blk(b, early(r));
        cl[b + 1] = cl[b] + blk(b, late(r));
      }
    }
    int64_t o_row = 0;
    for (int b = 0; b < bs; ++b) {
      int64_t t0 = 0;
      for (int j = 0; j < nblk; ++j) {
        const bool is_early = j < cp_size;
        const int owner = is_early ? j : nblk - 1 - j;
        const int pos = owner * 2 * bs + (is_early ? b : bs + b);
        // gathered row: the owner's region, then early rows of earlier
        // sequences (early block) or all early rows plus late rows of earlier
        // sequences (late block)
        const int64_t* ce = &cum_early[(size_t)owner * (bs + 1)];
        const int64_t* cl = &cum_late[(size_t)owner * (bs + 1)];
        const int64_t g = (int64_t)owner * mrl + (is_early ? ce[b] : ce[bs] + cl[b]);
        const int c = b * nblk + j;
        reverse_index[c] = pos;
        reverse_split[pos] = (int32_t)blk(b, j);
        chunks[c] = Chunk{b, (int32_t)t0, (int32_t)g, (int32_t)(o_row + t0),
                          (int32_t)blk(b, j), (int32_t)(prefix[b] + t0), 0, 0};
        t0 += blk(b, j);
      }
      o_row += ext[b];
    }
  }

  // Per-half lengths: each local block sees its sequence's prefix and every
  // block up to and including itself.
  std::vector<int32_t> kv_prev(bs), kv_next(bs), q_prev(bs), q_next(bs), cu_prev(bs + 1),
      cu_next(bs + 1), prefix32(bs), ext32(bs);
  int32_t max_kv = 0;
  cu_prev[0] = cu_next[0] = 0;
  for (int b = 0; b < bs; ++b) {
    int64_t upto_early = 0, upto_late = 0;
    for (int j = 0; j <= late(cp_rank); ++j) {
      if (j <= early(cp_rank)) upto_early += blk(b, j);
      upto_late += blk(b, j);
    }
    kv_prev[b] = (int32_t)(prefix[b] + upto_early);
    kv_next[b] = (int32_t)(prefix[b] + upto_late);
    q_prev[b] = (int32_t)blk(b, early(cp_rank));
    q_next[b] = (int32_t)blk(b, late(cp_rank));
    cu_prev[b + 1] = cu_prev[b] + q_prev[b];
    cu_next[b + 1] = cu_next[b] + q_next[b];
    prefix32[b] = (int32_t)prefix[b];
    ext32[b] = (int32_t)ext[b];
    max_kv = std::max(max_kv, std::max(kv_prev[b], kv_next[b]));
  }
  const int32_t total_prev = cu_prev[bs], total_next = cu_next[bs];

  // Attention segments in local row order: prev halves, then next halves.
  std::vector<Seg> segs;
  for (int b = 0; b < bs; ++b)
    segs.push_back(Seg{cu_prev[b], q_prev[b], q_prev[b], kv_prev[b], kv_prev[b] - q_prev[b], b, 1, 0});
  for (int b = 0; b < bs; ++b)
    segs.push_back(Seg{total_prev + cu_next[b], q_next[b], q_next[b], kv_next[b],
                       kv_next[b] - q_next[b], b, 1, 0});
  std::vector<Work> work;
  const int q_tile = attn_group > 0 ? kAttnRows / attn_group : 0;
  if (attn_group > 0) build_work(segs, q_tile, work);

  Layout lay;
  cp_meta_t m;
  std::memset(&m, 0, sizeof(m));
  m.version = CP_META_VERSION;
  m.kind = CP_META_ZIGZAG;
  m.cp_size = cp_size;
  m.cp_rank = cp_rank;
  m.bs = bs;
  m.attn_group = attn_group;
  m.total_seq_lens = num_tokens;
  m.max_rank_len = (int32_t)mrl;
  m.total_q_prev_tokens = total_prev;
  m.total_q_next_tokens = total_next;
  m.max_seqlen_q_prev = *std::max_element(q_prev.begin(), q_prev.end());
  m.max_seqlen_q_next = *std::max_element(q_next.begin(), q_next.end());
  m.n_local_rows = total_prev + total_next;
  m.n_chunks = bs * nblk;
  int32_t max_chunk = 0;
  for (const Chunk& c : chunks) max_chunk = std::max(max_chunk, c.n_rows);
  m.max_chunk_rows = max_chunk;
  m.n_seg = (int32_t)segs.size();
  m.n_work = (int32_t)work.size();
  m.mean_item_tiles = mean_item_tiles(work);
  m.max_kv_len = max_kv;
  m.q_tile = q_tile;
  m.kv_align = kKvAlignMax;
  m.off_split_list = lay.take(4LL * bs * nblk);
  m.off_zigzag_index = lay.take(4LL * 2 * bs);
  m.off_cp_reverse_index = lay.take(4LL * bs * nblk);
  m.off_reverse_split_len = lay.take(4LL * bs * nblk);
  m.off_per_rank_actual_token = lay.take(4LL * cp_size);
  m.off_kv_len_prev = lay.take(4LL * bs);
  m.off_kv_len_next = lay.take(4LL * bs);
  m.off_q_prev = lay.take(4LL * bs);
  m.off_q_next = lay.take(4LL * bs);
  m.off_cu_seqlens_q_prev = lay.take(4LL * (bs + 1));
  m.off_cu_seqlens_q_next = lay.take(4LL * (bs + 1));
  m.off_prefix = lay.take(4LL * bs);
  m.off_extend = lay.take(4LL * bs);
  m.off_chunks = lay.take((int64_t)sizeof(Chunk) * chunks.size());
  m.off_segs = lay.take((int64_t)sizeof(Seg) * segs.size());
  m.off_work = lay.take((int64_t)sizeof(Work) * work.size());
  m.blob_bytes = lay.cursor;
  *meta = m;
  if (!blob) return CP_OK;  // size query
  if (blob_capacity < m.blob_bytes)
    return set_error(CP_ERR_BUFFER_TOO_SMALL, "blob_capacity=%lld < blob_bytes=%lld",
                     (long long)blob_capacity, (long long)m.blob_bytes);

  std::memset(blob, 0, (size_t)m.blob_bytes);
  Header h{kBlobMagic, CP_META_VERSION, CP_META_ZIGZAG, m.n_chunks, m.n_seg, m.n_work, cp_size, bs};
  std::memcpy(blob, &h, sizeof(h));
  write_i32(blob, m.off_split_list, split_list);
  write_i32(blob, m.off_zigzag_index, zigzag_index);
  write_i32(blob, m.off_cp_reverse_index, reverse_index);
  write_i32(blob, m.off_reverse_split_len, reverse_split);
  write_i32(blob, m.off_per_rank_actual_token, per_rank);
  write_i32(blob, m.off_kv_len_prev, kv_prev);
  write_i32(blob, m.off_kv_len_next, kv_next);
  write_i32(blob, m.off_q_prev, q_prev);
  write_i32(blob, m.off_q_next, q_next);
  write_i32(blob, m.off_cu_seqlens_q_prev, cu_prev);
  write_i32(blob, m.off_cu_seqlens_q_next, cu_next);
  write_i32(blob, m.off_prefix, prefix32);
  write_i32(blob, m.off_extend, ext32);
  char* base = static_cast<char*>(blob);
  std::memcpy(base + m.off_chunks, chunks.data(), sizeof(Chunk) * chunks.size());
  std::memcpy(base + m.off_segs, segs.data(), sizeof(Seg) * segs.size());
  if (!work.empty()) std::memcpy(base + m.off_work, work.data(), sizeof(Work) * work.size());
  return CP_OK;
}

extern "C" int cp_allgather_meta_build(int32_t q_total, int32_t q_real, int32_t kv_len,
                                       int32_t attn_group, void* blob, int64_t blob_capacity,
                                       cp_meta_t* meta) {
  clear_error();
  if (!meta) return set_error(CP_ERR_INVALID_ARG, "meta is NULL");
  if (q_total < 1) return set_error(CP_ERR_INVALID_ARG, "q_total=%d must be >= 1", q_total);
  if (q_real < 0 || q_real > q_total)
    return set_error(CP_ERR_INVALID_ARG, "q_real=%d outside [0, q_total=%d]", q_real, q_total);
  if (kv_len < 1)
    return set_error(CP_ERR_INVALID_ARG, "kv_len=%d: the real K/V prefix must be non-empty", kv_len);
  if (int rc = check_group(attn_group, false)) return rc;

  std::vector<Seg> segs{Seg{0, q_real, q_total, kv_len, 0, 0, 0, 0}};
  std::vector<Work> work;
  const int q_tile = kAttnRows / attn_group;
  build_work(segs, q_tile, work);

  Layout lay;
  cp_meta_t m;
  std::memset(&m, 0, sizeof(m));
  m.version = CP_META_VERSION;
  m.kind = CP_META_ALLGATHER;
  m.bs = 1;
  m.attn_group = attn_group;
  m.n_local_rows = q_total;
  m.n_seg = 1;
  m.n_work = (int32_t)work.size();
  m.mean_item_tiles = mean_item_tiles(work);
  m.max_kv_len = kv_len;
  m.q_tile = q_tile;
  m.kv_align = kKvAlignMax;
  const int64_t empty = lay.take(0);
  m.off_split_list = m.off_zigzag_index = m.off_cp_reverse_index = m.off_reverse_split_len = empty;
  m.off_per_rank_actual_token = m.off_kv_len_prev = m.off_kv_len_next = empty;
  m.off_q_prev = m.off_q_next = m.off_cu_seqlens_q_prev = m.off_cu_seqlens_q_next = empty;
  m.off_prefix = m.off_extend = m.off_chunks = empty;
  m.off_segs = lay.take((int64_t)sizeof(Seg));
  m.off_work = lay.take((int64_t)sizeof(Work) * work.size());
  m.blob_bytes = lay.cursor;
  *meta = m;
  if (!blob) return CP_OK;
  if (blob_capacity < m.blob_bytes)
    return set_error(CP_ERR_BUFFER_TOO_SMALL, "blob_capacity=%lld < blob_bytes=%lld",
                     (long long)blob_capacity, (long long)m.blob_bytes);
  std::memset(blob, 0, (size_t)m.blob_bytes);
  Header h{kBlobMagic, CP_META_VERSION, CP_META_ALLGATHER, 0, 1, m.n_work, 0, 1};
  std::memcpy(blob, &h, sizeof(h));
  char* base = static_cast<char*>(blob);
  std::memcpy(base + m.off_segs, segs.data(), sizeof(Seg));
  std::memcpy(base + m.off_work, work.data(), sizeof(Work) * work.size());
  return CP_OK;
}

extern "C" int cp_allgather_packed_meta_build(int32_t n_docs, const int32_t* doc_cu,
                                              int32_t q_start, int32_t q_total, int32_t attn_group,
                                              void* blob, int64_t blob_capacity, cp_meta_t* meta) {
  clear_error();
  if (!meta) return set_error(CP_ERR_INVALID_ARG, "meta is NULL");
  if (n_docs < 1) return set_error(CP_ERR_INVALID_ARG, "n_docs=%d must be >= 1", n_docs);
  if (!doc_cu) return set_error(CP_ERR_INVALID_ARG, "doc_cu is NULL");
  if (doc_cu[0] != 0) return set_error(CP_ERR_INVALID_ARG, "doc_cu[0]=%d must be 0", doc_cu[0]);
  for (int b = 0; b < n_docs; ++b)
    if (doc_cu[b + 1] < doc_cu[b])
      return set_error(CP_ERR_INVALID_ARG, "doc_cu must be non-decreasing (doc_cu[%d]=%d > doc_cu[%d]=%d)",
                       b, doc_cu[b], b + 1, doc_cu[b + 1]);
  if (doc_cu[n_docs] < 1) return set_error(CP_ERR_INVALID_ARG, "the packed documents are empty");
  if (q_total < 1) return set_error(CP_ERR_INVALID_ARG, "q_total=%d must be >= 1", q_total);
  if (q_start < 0) return set_error(CP_ERR_INVALID_ARG, "q_start=%d must be >= 0", q_start);
  if ((int64_t)q_start + q_total > INT32_MAX)
    return set_error(CP_ERR_OVERFLOW, "q_start + q_total exceeds int32");
  if (int rc = check_group(attn_group, false)) return rc;

  // One segment per document that meets the local rows [q_start, q_end);
  // local rows in the pad suffix join the last segment (or form their own
  // segment without keys if no document meets the slice).
  const int32_t q_end = q_start + q_total, real = doc_cu[n_docs];
  std::vector<Seg> segs;
  int32_t max_kv = 0;
  for (int b = 0; b < n_docs; ++b) {
    const int32_t lo = std::max(doc_cu[b], q_start), hi = std::min(doc_cu[b + 1], q_end);
    if (lo >= hi) continue;
    const int32_t kv = doc_cu[b + 1] - doc_cu[b];
    segs.push_back(Seg{lo - q_start, hi - lo, hi - lo, kv, kv - (hi - lo), 0, 0, doc_cu[b]});
    max_kv = std::max(max_kv, kv);
  }
  if (q_end > real) {
    const int32_t pad0 = std::max(real, q_start) - q_start;
    if (!segs.empty() && segs.back().q_row0 + segs.back().q_rows == pad0)
      segs.back().q_rows += q_total - pad0;
    else
      segs.push_back(Seg{pad0, 0, q_total - pad0, 0, 0, 0, 0, 0});
  }
  std::vector<Work> work;
  const int q_tile = kAttnRows / attn_group;
  build_work(segs, q_tile, work);

  Layout lay;
  cp_meta_t m;
  std::memset(&m, 0, sizeof(m));
  m.version = CP_META_VERSION;
  m.kind = CP_META_ALLGATHER;
  m.bs = 1;   // one page-table row: the ordered global K/V
  int32_t align = kKvAlignMax;
  for (const Seg& g : segs)
    if (g.kv_start != 0) align = std::min(align, g.kv_start & -g.kv_start);
  m.attn_group = attn_group;
  m.n_local_rows = q_total;
  m.n_seg = (int32_t)segs.size();
  m.n_work = (int32_t)work.size();
  m.mean_item_tiles = mean_item_tiles(work);
  m.max_kv_len = max_kv;
  m.q_tile = q_tile;
  m.kv_align = align;
  const int64_t empty = lay.take(0);
  m.off_split_list = m.off_zigzag_index = m.off_cp_reverse_index = m.off_reverse_split_len = empty;
  m.off_per_rank_actual_token = m.off_kv_len_prev = m.off_kv_len_next = empty;
  m.off_q_prev = m.off_q_next = m.off_cu_seqlens_q_prev = m.off_cu_seqlens_q_next = empty;
  m.off_prefix = m.off_extend = m.off_chunks = empty;
  m.off_segs = lay.take((int64_t)sizeof(Seg) * segs.size());
  m.off_work = lay.take((int64_t)sizeof(Work) * work.size());
  m.blob_bytes = lay.cursor;
  *meta = m;
  if (!blob) return CP_OK;
  if (blob_capacity < m.blob_bytes)
    return set_error(CP_ERR_BUFFER_TOO_SMALL, "blob_capacity=%lld < blob_bytes=%lld",
                     (long long)blob_capacity, (long long)m.blob_bytes);
  std::memset(blob, 0, (size_t)m.blob_bytes);
  Header h{kBlobMagic, CP_META_VERSION, CP_META_ALLGATHER, 0, m.n_seg, m.n_work, 0, 1};
  std::memcpy(blob, &h, sizeof(h));
  char* base = static_cast<char*>(blob);
  std::memcpy(base + m.off_segs, segs.data(), sizeof(Seg) * segs.size());
  std::memcpy(base + m.off_work, work.data(), sizeof(Work) * work.size());
  return CP_OK;
}

extern "C" const char* cp_last_error(void) { return g_err; }

extern "C" const char* cp_version(void) { return "cpattn 0.1 gfx950"; }
