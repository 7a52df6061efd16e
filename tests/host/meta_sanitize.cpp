// Host-only stress of the metadata builders under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with g++ by tests/test_host_sanitize.py).
//
// Seeded random arguments, valid and invalid, for cp_meta_build,
// cp_allgather_meta_build and cp_allgather_packed_meta_build.  Each call is
// made twice: first with no blob (size query), then into a heap buffer of
// exactly meta.blob_bytes, so any write past the reported size is caught by
// the sanitizer.  A third call with one byte less must report
// CP_ERR_BUFFER_TOO_SMALL.  On success, every table the kernels index (chunks,
// segments, work list) must lie inside the blob and every index in it must
// stay within the bounds the copy and attention kernels assume.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/cpattn.h"
#include "../../context_prefill_attention_amd/csrc/cp_internal.h"

using cpattn::Chunk;
using cpattn::Seg;
using cpattn::Work;

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;

uint64_t next_u64() {   // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 2685821657736338717ull;
}

int rnd(int lo, int hi) {   // uniform in [lo, hi]
  return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1));
}

int g_fail = 0;

void fail(const char* what, int c) {
  if (g_fail < 20) std::fprintf(stderr, "case %d: %s\n", c, what);
  ++g_fail;
}

template <typename T>
const T* table(const std::vector<unsigned char>& blob, int64_t off, int64_t n, const cp_meta_t& m,
               int c) {
  if (n < 0 || off < 0 || off % 256 != 0 || off + n * (int64_t)sizeof(T) > m.blob_bytes) {
    fail("table outside the blob", c);
    return nullptr;
  }
  return reinterpret_cast<const T*>(blob.data() + off);
}

// Bounds the kernels rely on: segments within the local rows, work items
// within their segment, no tile past the segment's keys.
void check_attention_tables(const std::vector<unsigned char>& blob, const cp_meta_t& m, int c) {
  const Seg* segs = table<Seg>(blob, m.off_segs, m.n_seg, m, c);
  const Work* work = table<Work>(blob, m.off_work, m.n_work, m, c);
  if (!segs || !work) return;
  for (int i = 0; i < m.n_seg; ++i) {
    const Seg& s = segs[i];
    if (s.q_row0 < 0 || s.q_len < 0 || s.q_len > s.q_rows || s.q_row0 + (int64_t)s.q_rows > m.n_local_rows)
      fail("segment rows out of range", c);
    if (s.kv_len < 0 || s.kv_start < 0 || s.page_row < 0 || s.page_row >= m.bs)
      fail("segment keys or page row out of range", c);
    if (s.causal && s.causal_off != s.kv_len - s.q_len) fail("causal offset", c);
  }
  for (int i = 0; i < m.n_work; ++i) {
    const Work& w = work[i];
    if (w.seg < 0 || w.seg >= m.n_seg) {
      fail("work item names no segment", c);
      continue;
    }
    const Seg& s = segs[w.seg];
    if (w.p0 < 0 || w.np < 1 || w.np > m.q_tile || w.p0 + (int64_t)w.np > s.q_rows)
      fail("work item rows out of range", c);
    if (w.n_tiles < 0 || (int64_t)w.n_tiles * cpattn::kAttnKeys > (int64_t)s.kv_len + cpattn::kAttnKeys - 1)
      fail("work item tiles past the segment's keys", c);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int n_cases = argc > 1 ? std::atoi(argv[1]) : 20000;
  int counts[3][8] = {};
  for (int c = 0; c < n_cases; ++c) {
    const int kind = c % 3;
    std::vector<int32_t> a, b;
    cp_meta_t m0, m1;
    int rc0 = 0, rc1 = 0, rc2 = 0;
    std::memset(&m0, 0, sizeof(m0));
    std::memset(&m1, 0, sizeof(m1));
    if (kind == 0) {
      // zigzag metadata
      const int cp = rnd(0, 9), rank = rnd(-1, cp), bs = rnd(0, 5);
      a.resize(bs > 0 ? bs : 1);
      b.resize(a.size());
      int64_t sum = 0;
      for (int i = 0; i < bs; ++i) {
        a[i] = rnd(0, 1) ? rnd(2 * (cp > 0 ? cp : 1), 400) : rnd(-3, 3 * cp + 2);
        b[i] = a[i] + (rnd(0, 2) == 0 ? rnd(-5, 300) : 0);
        sum += a[i];
      }
      const bool with_seq = rnd(0, 1);
      const int64_t ntok = rnd(0, 4) == 0 ? sum + rnd(-3, 40) : sum;
      const int group = rnd(0, 10) == 0 ? rnd(-2, 300) : rnd(0, 9);
      rc0 = cp_meta_build(cp, rank, bs, a.data(), with_seq ? b.data() : nullptr, ntok, group, nullptr, 0, &m0);
      if (rc0 == CP_OK) {
        std::vector<unsigned char> blob((size_t)m0.blob_bytes);
        rc1 = cp_meta_build(cp, rank, bs, a.data(), with_seq ? b.data() : nullptr, ntok, group, blob.data(),
                            m0.blob_bytes, &m1);
        if (rc1 != CP_OK || std::memcmp(&m0, &m1, sizeof(m0)) != 0) fail("size query and build differ", c);
        if (m1.blob_bytes > 0) {
          std::vector<unsigned char> small((size_t)m1.blob_bytes - 1);
          cp_meta_t m2;
          rc2 = cp_meta_build(cp, rank, bs, a.data(), with_seq ? b.data() : nullptr, ntok, group, small.data(),
                              m1.blob_bytes - 1, &m2);
          if (rc2 != CP_ERR_BUFFER_TOO_SMALL) fail("undersized blob accepted", c);
        }
        if (rc1 == CP_OK) {
          const Chunk* ch = table<Chunk>(blob, m1.off_chunks, m1.n_chunks, m1, c);
          for (int i = 0; ch && i < m1.n_chunks; ++i) {
            if (ch[i].b < 0 || ch[i].b >= m1.bs || ch[i].n_rows < 0 ||
                ch[i].g_row + (int64_t)ch[i].n_rows > (int64_t)m1.cp_size * m1.max_rank_len ||
                ch[i].o_row + (int64_t)ch[i].n_rows > m1.total_seq_lens || ch[i].pos0 < 0)
              fail("chunk out of range", c);
          }
          table<int32_t>(blob, m1.off_split_list, (int64_t)m1.bs * 2 * m1.cp_size, m1, c);
          table<int32_t>(blob, m1.off_cu_seqlens_q_next, m1.bs + 1, m1, c);
          if (group > 0) check_attention_tables(blob, m1, c);
        }
      }
    } else if (kind == 1) {
      // AllGather-KV, one document
      const int q_total = rnd(-1, 700), q_real = rnd(-1, q_total + 1), kv = rnd(-1, 900);
      const int group = rnd(0, 10) == 0 ? rnd(-2, 300) : rnd(1, 9);
      rc0 = cp_allgather_meta_build(q_total, q_real, kv, group, nullptr, 0, &m0);
      if (rc0 == CP_OK) {
        std::vector<unsigned char> blob((size_t)m0.blob_bytes);
        rc1 = cp_allgather_meta_build(q_total, q_real, kv, group, blob.data(), m0.blob_bytes, &m1);
        if (rc1 != CP_OK || std::memcmp(&m0, &m1, sizeof(m0)) != 0) fail("size query and build differ", c);
        if (m1.blob_bytes > 0) {
          std::vector<unsigned char> small((size_t)m1.blob_bytes - 1);
          cp_meta_t m2;
          if (cp_allgather_meta_build(q_total, q_real, kv, group, small.data(), m1.blob_bytes - 1, &m2) !=
              CP_ERR_BUFFER_TOO_SMALL)
            fail("undersized blob accepted", c);
        }
        if (rc1 == CP_OK) check_attention_tables(blob, m1, c);
      }
    } else {
      // AllGather-KV over packed documents
      const int n_docs = rnd(-1, 8);
      a.assign(n_docs > 0 ? n_docs + 1 : 1, 0);
      for (int i = 1; i <= n_docs; ++i) a[i] = a[i - 1] + (rnd(0, 12) == 0 ? rnd(-3, 0) : rnd(0, 300));
      if (rnd(0, 15) == 0) a[0] = rnd(-2, 2);
      const int q_start = rnd(-1, 1200), q_total = rnd(-1, 600);
      const int group = rnd(0, 10) == 0 ? rnd(-2, 300) : rnd(1, 9);
      const int32_t* cu = rnd(0, 30) == 0 ? nullptr : a.data();
      rc0 = cp_allgather_packed_meta_build(n_docs, cu, q_start, q_total, group, nullptr, 0, &m0);
      if (rc0 == CP_OK) {
        std::vector<unsigned char> blob((size_t)m0.blob_bytes);
        rc1 = cp_allgather_packed_meta_build(n_docs, cu, q_start, q_total, group, blob.data(), m0.blob_bytes, &m1);
        if (rc1 != CP_OK || std::memcmp(&m0, &m1, sizeof(m0)) != 0) fail("size query and build differ", c);
        if (m1.blob_bytes > 0) {
          std::vector<unsigned char> small((size_t)m1.blob_bytes - 1);
          cp_meta_t m2;
          if (cp_allgather_packed_meta_build(n_docs, cu, q_start, q_total, group, small.data(),
                                             m1.blob_bytes - 1, &m2) != CP_ERR_BUFFER_TOO_SMALL)
            fail("undersized blob accepted", c);
        }
        if (rc1 == CP_OK) {
          check_attention_tables(blob, m1, c);
          if (m1.kv_align < 1 || (m1.kv_align & (m1.kv_align - 1)) != 0) fail("kv_align not a power of two", c);
        }
      }
    }
    if (rc0 > 0 || rc0 < -5) fail("unknown status", c);
    ++counts[kind][rc0 <= 0 && rc0 >= -5 ? -rc0 : 7];
    if (rc0 != CP_OK && cp_last_error()[0] == '\0') fail("rejection without a message", c);
  }
  for (int k = 0; k < 3; ++k)
    std::printf("builder %d: ok %d invalid %d unsupported %d too_small %d overflow %d\n", k, counts[k][0],
                counts[k][1], counts[k][2], counts[k][3], counts[k][4]);
  std::printf("%s: %d cases, %d failures\n", g_fail ? "FAIL" : "ok", n_cases, g_fail);
  return g_fail ? 1 : 0;
}
