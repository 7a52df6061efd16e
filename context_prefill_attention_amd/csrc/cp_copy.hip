// Zigzag rerange and KV-pool scatter: bandwidth-bound row copies (gfx950).
//
// Both operations move whole rows.  Every zigzag chunk (one block of one
// sequence) is a contiguous run of rows in the all-gathered buffer and in
// original token order (sglang zigzag.py source page: gather_kv_cache splits
// the gathered rows by reverse_split_len and reorders them by
// cp_reverse_index; _all_gather_reorganized pads every rank to max_rank_len).
// The rerange is therefore one contiguous memcpy per chunk, and the scatter
// one contiguous copy per (chunk, pool page) run into that page's slots
// (materialize_full_kv writes the full-sequence K/V at the extend tokens'
// cache locations).
//
// Launch shape: a 1-D grid; each workgroup owns one fixed-size byte range of
// one chunk (one-tensor rerange, 16 KiB), of one chunk in K and in V (paired
// rerange, 2 KiB of each) or of one page run of a chunk in K and in V
// (scatter, 2 KiB of each), so its lookups are a few divisions and no search.
// Each lane moves 16-byte vectors with its loads in flight before the
// stores.  In the paired kernels half of the lanes copy K and the other half
// the same bytes of V.  The scatter's small ranges keep many pool pages in
// flight at once, which pays when the pages are written in random order
// (measured against 16 KiB ranges of K and V per workgroup: 16 % faster with
// a permuted page table, 8 % with the identity table); the paired rerange
// runs 4 % faster than two one-tensor launches.
#include <hip/hip_runtime.h>

#include "../../include/cpattn.h"
#include "cp_internal.h"

namespace cpattn {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;                                   // 16-B vectors per lane in flight
constexpr int64_t kCopyBytesPerWG = 16LL * kCopyThreads * kCopyUnroll;   // 16 KiB
constexpr int kScatterThreads = 256;      // lanes 0-127 copy K, 128-255 the same bytes of V
constexpr int64_t kScatterBytesPerWG = 16LL * (kScatterThreads / 2);   // 2 KiB of each

// One workgroup copies bytes [part*16KiB, (part+1)*16KiB) of chunk c.
__global__ __launch_bounds__(kCopyThreads) void rerange_kernel(
    const Chunk* __restrict__ chunks, int32_t parts_per_chunk, int32_t forward,
    const unsigned char* __restrict__ src, unsigned char* __restrict__ dst, int64_t row_bytes) {
  const int c = blockIdx.x / parts_per_chunk;
  const int part = blockIdx.x - c * parts_per_chunk;
  const Chunk ch = chunks[c];
  const int64_t nbytes = (int64_t)ch.n_rows * row_bytes;
  const int64_t start = (int64_t)part * kCopyBytesPerWG;
  if (start >= nbytes) return;
  const int64_t g_off = (int64_t)ch.g_row * row_bytes, o_off = (int64_t)ch.o_row * row_bytes;
  const unsigned char* s = src + (forward ? g_off : o_off) + start;
  unsigned char* d = dst + (forward ? o_off : g_off) + start;
  const int64_t avail = nbytes - start;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t off = (int64_t)(u * kCopyThreads + threadIdx.x) * 16;
    if (off < avail) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s + off));
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t off = (int64_t)(u * kCopyThreads + threadIdx.x) * 16;
    if (off < avail) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(d + off));
  }
}

// K and V together (rows a multiple of 16 bytes): the same chunk/part split
// with parts of kPairBytesPerWG; half the lanes copy the part's bytes of K,
// the other half the same bytes of V, so one launch moves both tensors.
constexpr int kPairUnroll = 1;
constexpr int64_t kPairBytesPerWG = 16LL * (kCopyThreads / 2) * kPairUnroll;   // 2 KiB of each
__global__ __launch_bounds__(kCopyThreads) void rerange_pair_kernel(
    const Chunk* __restrict__ chunks, int32_t parts_per_chunk, int32_t forward,
    const unsigned char* __restrict__ k_src, unsigned char* __restrict__ k_dst,
    const unsigned char* __restrict__ v_src, unsigned char* __restrict__ v_dst, int64_t row_bytes) {
  constexpr int kHalf = kCopyThreads / 2;
  const int c = blockIdx.x / parts_per_chunk;
  const int part = blockIdx.x - c * parts_per_chunk;
  const Chunk ch = chunks[c];
  const int64_t nbytes = (int64_t)ch.n_rows * row_bytes;
  const int64_t start = (int64_t)part * kPairBytesPerWG;
  if (start >= nbytes) return;
  const int64_t g_off = (int64_t)ch.g_row * row_bytes, o_off = (int64_t)ch.o_row * row_bytes;
  const bool is_v = threadIdx.x >= kHalf;
  const int lane = threadIdx.x - (is_v ? kHalf : 0);
  const unsigned char* s = (is_v ? v_src : k_src) + (forward ? g_off : o_off) + start;
  unsigned char* d = (is_v ? v_dst : k_dst) + (forward ? o_off : g_off) + start;
  const int64_t avail = nbytes - start;
  u32x4 v[kPairUnroll];
#pragma unroll
  for (int u = 0; u < kPairUnroll; ++u) {
    const int64_t off = (int64_t)(u * kHalf + lane) * 16;
    if (off < avail) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s + off));
  }
#pragma unroll
  for (int u = 0; u < kPairUnroll; ++u) {
    const int64_t off = (int64_t)(u * kHalf + lane) * 16;
    if (off < avail) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(d + off));
  }
}

// Rows whose size is not a multiple of 16 bytes (positions, narrow
// per-token tensors): the same chunk/part split, copied in elements of T,
// the widest power of two up to 8 bytes that divides the row size, so every
// access stays aligned.  These tensors are small; one element per lane and
// step is enough.
template <typename T>
__global__ __launch_bounds__(kCopyThreads) void rerange_narrow_kernel(
    const Chunk* __restrict__ chunks, int32_t parts_per_chunk, int32_t forward,
    const unsigned char* __restrict__ src, unsigned char* __restrict__ dst, int64_t row_bytes) {
  const int c = blockIdx.x / parts_per_chunk;
  const int part = blockIdx.x - c * parts_per_chunk;
  const Chunk ch = chunks[c];
  const int64_t nbytes = (int64_t)ch.n_rows * row_bytes;
  const int64_t start = (int64_t)part * kCopyBytesPerWG;
  if (start >= nbytes) return;
  const int64_t g_off = (int64_t)ch.g_row * row_bytes, o_off = (int64_t)ch.o_row * row_bytes;
  const T* s = reinterpret_cast<const T*>(src + (forward ? g_off : o_off) + start);
  T* d = reinterpret_cast<T*>(dst + (forward ? o_off : g_off) + start);
  const int64_t n = (nbytes - start < kCopyBytesPerWG ? nbytes - start : kCopyBytesPerWG) / (int64_t)sizeof(T);
  for (int64_t i = threadIdx.x; i < n; i += kCopyThreads) d[i] = s[i];
}

// Scatter.  Within one chunk, the tokens that share a pool page are a
// contiguous run of rows on both sides: consecutive rows of the gathered
// buffer and consecutive slots of that page.  The grid is laid out as
// (chunk, j-th page the chunk touches, 2 KiB slice of that run), so a
// workgroup copies one contiguous byte range of K and of V, with a single
// page-table lookup, exactly like the rerange.  Workgroups whose slice lies
// past the end of their run exit at once.
__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(
    const Chunk* __restrict__ chunks, int32_t pages_per_chunk, int32_t slices_per_page,
    const unsigned char* __restrict__ kg, const unsigned char* __restrict__ vg,
    unsigned char* __restrict__ kp, unsigned char* __restrict__ vp, int64_t row_bytes,
    int32_t num_pages, int32_t page_size, const int32_t* __restrict__ indptr,
    const int32_t* __restrict__ indices) {
  const int per_chunk = pages_per_chunk * slices_per_page;
  const int c = blockIdx.x / per_chunk;
  const int rem = blockIdx.x - c * per_chunk;
  const int j = rem / slices_per_page;
  const int slice = rem - j * slices_per_page;
  const Chunk ch = chunks[c];
  // the run: positions [lo, hi) of page-table entry e = pos0/ps + j
  const int e = ch.pos0 / page_size + j;
  const int64_t page_first = (int64_t)e * page_size;
  const int64_t lo = max((int64_t)ch.pos0, page_first);
  const int64_t hi = min((int64_t)ch.pos0 + ch.n_rows, page_first + page_size);
  if (lo >= hi) return;
  const int64_t nbytes = (int64_t)(hi - lo) * row_bytes;
  const int64_t start = (int64_t)slice * kScatterBytesPerWG;
  if (start >= nbytes) return;
  // the page id: an entry outside the sequence's row of the table, or an id
  // outside the pool, leaves its slots untouched (nothing is written)
  const int row0 = indptr[ch.b];
  if (e >= indptr[ch.b + 1] - row0) return;
  const int page = indices[row0 + e];
  if (page < 0 || page >= num_pages) return;
  const int64_t src_off = ((int64_t)ch.g_row + (lo - ch.pos0)) * row_bytes + start;
  const int64_t dst_off = ((int64_t)page * page_size + (lo - page_first)) * row_bytes + start;
  constexpr int kHalf = kScatterThreads / 2;
  const bool is_v = threadIdx.x >= kHalf;
  const int64_t off = (int64_t)(threadIdx.x - (is_v ? kHalf : 0)) * 16;
  const unsigned char* src = is_v ? vg : kg;
  unsigned char* dst = is_v ? vp : kp;
  if (off < nbytes - start) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + src_off + off));
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dst + dst_off + off));
  }
}

// HIP rejects a launch whose grid holds more than 2^32-1 work-items.
constexpr int64_t kMaxCopyGrid = 4294967295LL / kCopyThreads;
constexpr int64_t kMaxScatterGrid = 4294967295LL / kScatterThreads;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" int cp_zigzag_rerange(const void* d_blob, const cp_meta_t* meta, int32_t direction,
                                 const void* src, void* dst, int64_t row_bytes, hipStream_t stream) {
  clear_error();
  if (!meta || !d_blob) return set_error(CP_ERR_INVALID_ARG, "meta or d_blob is NULL");
  if (meta->version != CP_META_VERSION || meta->kind != CP_META_ZIGZAG)
    return set_error(CP_ERR_INVALID_ARG, "metadata is not zigzag metadata of this version");
  if (direction != CP_RERANGE_GATHERED_TO_ORIG && direction != CP_RERANGE_ORIG_TO_GATHERED)
    return set_error(CP_ERR_INVALID_ARG, "direction=%d", direction);
  if (row_bytes <= 0) return set_error(CP_ERR_INVALID_ARG, "row_bytes=%lld must be positive", (long long)row_bytes);
  if (!src || !dst) return set_error(CP_ERR_INVALID_ARG, "src or dst is NULL");
  if (!aligned16(src) || !aligned16(dst))
    return set_error(CP_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  const int64_t chunk_bytes = (int64_t)meta->max_chunk_rows * row_bytes;
  const int64_t parts = (chunk_bytes + kCopyBytesPerWG - 1) / kCopyBytesPerWG;
  const int64_t grid = parts * meta->n_chunks;
  if (parts > 2147483647LL || grid > kMaxCopyGrid)
    return set_error(CP_ERR_OVERFLOW, "rerange grid too large (%lld workgroups of %d threads)",
                     (long long)grid, kCopyThreads);
  if (grid == 0) return CP_OK;
  const Chunk* chunks = reinterpret_cast<const Chunk*>(static_cast<const char*>(d_blob) + meta->off_chunks);
  const int32_t fwd = direction == CP_RERANGE_GATHERED_TO_ORIG;
  const unsigned char* sp = static_cast<const unsigned char*>(src);
  unsigned char* dp = static_cast<unsigned char*>(dst);
  const dim3 g((unsigned)grid), b(kCopyThreads);
  if (row_bytes % 16 == 0)
    hipLaunchKernelGGL(rerange_kernel, g, b, 0, stream, chunks, (int32_t)parts, fwd, sp, dp, row_bytes);
  else if (row_bytes % 8 == 0)
    hipLaunchKernelGGL(rerange_narrow_kernel<uint64_t>, g, b, 0, stream, chunks, (int32_t)parts, fwd, sp, dp, row_bytes);
  else if (row_bytes % 4 == 0)
    hipLaunchKernelGGL(rerange_narrow_kernel<uint32_t>, g, b, 0, stream, chunks, (int32_t)parts, fwd, sp, dp, row_bytes);
  else if (row_bytes % 2 == 0)
    hipLaunchKernelGGL(rerange_narrow_kernel<uint16_t>, g, b, 0, stream, chunks, (int32_t)parts, fwd, sp, dp, row_bytes);
  else
    hipLaunchKernelGGL(rerange_narrow_kernel<uint8_t>, g, b, 0, stream, chunks, (int32_t)parts, fwd, sp, dp, row_bytes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CP_ERR_HIP, "rerange launch: %s", hipGetErrorString(e));
  return CP_OK;
}

extern "C" int cp_zigzag_rerange_kv(const void* d_blob, const cp_meta_t* meta, int32_t direction,
                                    const void* k_src, void* k_dst, const void* v_src, void* v_dst,
                                    int64_t row_bytes, hipStream_t stream) {
  clear_error();
  if (!meta || !d_blob) return set_error(CP_ERR_INVALID_ARG, "meta or d_blob is NULL");
  if (meta->version != CP_META_VERSION || meta->kind != CP_META_ZIGZAG)
    return set_error(CP_ERR_INVALID_ARG, "metadata is not zigzag metadata of this version");
  if (direction != CP_RERANGE_GATHERED_TO_ORIG && direction != CP_RERANGE_ORIG_TO_GATHERED)
    return set_error(CP_ERR_INVALID_ARG, "direction=%d", direction);
  if (row_bytes <= 0) return set_error(CP_ERR_INVALID_ARG, "row_bytes=%lld must be positive", (long long)row_bytes);
  if (!k_src || !k_dst || !v_src || !v_dst) return set_error(CP_ERR_INVALID_ARG, "a K or V pointer is NULL");
  if (!aligned16(k_src) || !aligned16(k_dst) || !aligned16(v_src) || !aligned16(v_dst))
    return set_error(CP_ERR_INVALID_ARG, "K and V buffers must be 16-byte aligned");
  if (row_bytes % 16 != 0) {   // narrow rows: the one-tensor copy, twice
    if (int rc = cp_zigzag_rerange(d_blob, meta, direction, k_src, k_dst, row_bytes, stream)) return rc;
    return cp_zigzag_rerange(d_blob, meta, direction, v_src, v_dst, row_bytes, stream);
  }
  const int64_t chunk_bytes = (int64_t)meta->max_chunk_rows * row_bytes;
  const int64_t parts = (chunk_bytes + kPairBytesPerWG - 1) / kPairBytesPerWG;
  const int64_t grid = parts * meta->n_chunks;
  if (parts > 2147483647LL || grid > kMaxCopyGrid)
    return set_error(CP_ERR_OVERFLOW, "rerange grid too large (%lld workgroups of %d threads)",
                     (long long)grid, kCopyThreads);
  if (grid == 0) return CP_OK;
  const Chunk* chunks = reinterpret_cast<const Chunk*>(static_cast<const char*>(d_blob) + meta->off_chunks);
  hipLaunchKernelGGL(rerange_pair_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0, stream, chunks,
                     (int32_t)parts, (int32_t)(direction == CP_RERANGE_GATHERED_TO_ORIG),
                     static_cast<const unsigned char*>(k_src), static_cast<unsigned char*>(k_dst),
                     static_cast<const unsigned char*>(v_src), static_cast<unsigned char*>(v_dst), row_bytes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CP_ERR_HIP, "rerange launch: %s", hipGetErrorString(e));
  return CP_OK;
}

extern "C" int cp_kv_scatter(const void* d_blob, const cp_meta_t* meta,
                             const void* k_gathered, const void* v_gathered,
                             void* k_pool, void* v_pool, int32_t num_pages, int32_t page_size,
                             int32_t H_kv, int32_t D,
                             const int32_t* kv_page_indptr, const int32_t* kv_page_indices,
                             hipStream_t stream) {
  clear_error();
  if (!meta || !d_blob) return set_error(CP_ERR_INVALID_ARG, "meta or d_blob is NULL");
  if (meta->version != CP_META_VERSION || meta->kind != CP_META_ZIGZAG)
    return set_error(CP_ERR_INVALID_ARG, "metadata is not zigzag metadata of this version");
  if (H_kv < 1 || D < 1) return set_error(CP_ERR_INVALID_ARG, "H_kv=%d D=%d", H_kv, D);
  const int64_t row_bytes = (int64_t)H_kv * D * 2;
  if (row_bytes % 16 != 0)
    return set_error(CP_ERR_UNSUPPORTED, "H_kv*D*2=%lld must be a multiple of 16", (long long)row_bytes);
  if (page_size < 1) return set_error(CP_ERR_INVALID_ARG, "page_size=%d", page_size);
  if (num_pages < 1) return set_error(CP_ERR_INVALID_ARG, "num_pages=%d", num_pages);
  if (!k_gathered || !v_gathered || !k_pool || !v_pool || !kv_page_indptr || !kv_page_indices)
    return set_error(CP_ERR_INVALID_ARG, "a device pointer is NULL");
  if (!aligned16(k_gathered) || !aligned16(v_gathered) || !aligned16(k_pool) || !aligned16(v_pool))
    return set_error(CP_ERR_INVALID_ARG, "K/V buffers must be 16-byte aligned");
  // A chunk of n rows touches at most ceil((n - 1) / ps) + 1 pages; a page's
  // run is at most ps rows, i.e. ceil(ps * row_bytes / 2 KiB) slices.
  const int64_t pages_per_chunk =
      meta->max_chunk_rows > 0 ? (meta->max_chunk_rows - 1 + page_size - 1) / page_size + 1 : 0;
  const int64_t slices_per_page = ((int64_t)page_size * row_bytes + kScatterBytesPerWG - 1) / kScatterBytesPerWG;
  const int64_t grid = pages_per_chunk * slices_per_page * meta->n_chunks;
  if (pages_per_chunk > 2147483647LL || slices_per_page > 2147483647LL ||
      pages_per_chunk * slices_per_page > 2147483647LL || grid > kMaxScatterGrid)
    return set_error(CP_ERR_OVERFLOW, "scatter grid too large (%lld workgroups of %d threads)",
                     (long long)grid, kScatterThreads);
  if (grid == 0) return CP_OK;
  const Chunk* chunks = reinterpret_cast<const Chunk*>(static_cast<const char*>(d_blob) + meta->off_chunks);
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)grid), dim3(kScatterThreads), 0, stream, chunks,
                     (int32_t)pages_per_chunk, (int32_t)slices_per_page,
                     static_cast<const unsigned char*>(k_gathered),
                     static_cast<const unsigned char*>(v_gathered), static_cast<unsigned char*>(k_pool),
                     static_cast<unsigned char*>(v_pool), row_bytes, num_pages, page_size,
                     kv_page_indptr, kv_page_indices);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CP_ERR_HIP, "scatter launch: %s", hipGetErrorString(e));
  return CP_OK;
}
