// Zigzag rerange and KV-pool scatter: bandwidth-bound row copies (gfx950).
//
// Both operations move whole rows.  Every zigzag chunk (one block of one
// sequence) is a contiguous run of rows in the all-gathered buffer and in
// original token order (sglang zigzag.py source page: gather_kv_cache splits
// the gathered rows by reverse_split_len and reorders them by
// cp_reverse_index; _all_gather_reorganized pads every rank to max_rank_len).
// The rerange is therefore one contiguous memcpy per chunk and the scatter
// one row copy per token into its KV-pool slot (materialize_full_kv writes
// the full-sequence K/V at the extend tokens' cache locations).
//
// Launch shape: a 1-D grid; each workgroup owns one fixed-size byte range
// (rerange) or row block (scatter) of one chunk, so the chunk lookup is one
// division and no search.  Each lane moves 16-byte vectors with several loads
// in flight before the stores, which is what keeps HBM3E busy.
#include <hip/hip_runtime.h>

#include "../../include/cpattn.h"
#include "cp_internal.h"

namespace cpattn {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;                                   // 16-B vectors per lane in flight
constexpr int64_t kCopyBytesPerWG = 16LL * kCopyThreads * kCopyUnroll;   // 16 KiB

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

constexpr int kScatterRows = 16;   // token rows per workgroup
constexpr int kScatterUnroll = 4;  // 16-B vectors of K and of V per lane in flight

// One workgroup copies rows [part*16, part*16+16) of chunk c, for K and V.
// The destination row of every token is looked up once, into LDS.  Vector i
// of the block (i = lane + k*threads) is row i / vpr, column i % vpr; each
// lane steps its (row, column) pair by the thread count without dividing.
__global__ __launch_bounds__(kCopyThreads) void scatter_kernel(
    const Chunk* __restrict__ chunks, int32_t parts_per_chunk,
    const unsigned char* __restrict__ kg, const unsigned char* __restrict__ vg,
    unsigned char* __restrict__ kp, unsigned char* __restrict__ vp, int64_t row_bytes,
    int32_t num_pages, int32_t page_size, const int32_t* __restrict__ indptr,
    const int32_t* __restrict__ indices) {
  __shared__ int64_t dst_row[kScatterRows];
  const int c = blockIdx.x / parts_per_chunk;
  const int part = blockIdx.x - c * parts_per_chunk;
  const Chunk ch = chunks[c];
  const int r0 = part * kScatterRows;
  if (r0 >= ch.n_rows) return;
  const int nrows = min(kScatterRows, ch.n_rows - r0);
  if (threadIdx.x < nrows) {
    const int pos = ch.pos0 + r0 + threadIdx.x;
    const int page = indices[indptr[ch.b] + pos / page_size];
    // a page id outside the pool is skipped rather than written out of bounds
    dst_row[threadIdx.x] = (page >= 0 && page < num_pages) ? (int64_t)page * page_size + pos % page_size : -1;
  }
  __syncthreads();
  const int vpr = (int)(row_bytes / 16);   // the host keeps kScatterRows * vpr within int32
  const int total = vpr * nrows;
  const int dr = kCopyThreads / vpr, dc = kCopyThreads - dr * vpr;
  int r = (int)threadIdx.x / vpr;
  int col = (int)threadIdx.x - r * vpr;
  const unsigned char* ks = kg + ((int64_t)ch.g_row + r0) * row_bytes;
  const unsigned char* vs = vg + ((int64_t)ch.g_row + r0) * row_bytes;
  for (int i0 = 0; i0 < total; i0 += kCopyThreads * kScatterUnroll) {
    u32x4 a[kScatterUnroll], b[kScatterUnroll];
    int rr[kScatterUnroll], cc[kScatterUnroll];
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
      rr[u] = r;
      cc[u] = col;
      if (i0 + u * kCopyThreads + (int)threadIdx.x < total) {
        const int64_t so = (int64_t)r * row_bytes + col * 16;
        a[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + so));
        b[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + so));
      }
      r += dr;
      col += dc;
      if (col >= vpr) {
        col -= vpr;
        ++r;
      }
    }
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
      if (i0 + u * kCopyThreads + (int)threadIdx.x < total && dst_row[rr[u]] >= 0) {
        const int64_t dof = dst_row[rr[u]] * row_bytes + cc[u] * 16;
        __builtin_nontemporal_store(a[u], reinterpret_cast<u32x4*>(kp + dof));
        __builtin_nontemporal_store(b[u], reinterpret_cast<u32x4*>(vp + dof));
      }
    }
  }
}

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
  if (parts > 2147483647LL || grid > 2147483647LL)
    return set_error(CP_ERR_OVERFLOW, "rerange grid too large");
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
  if (row_bytes / 16 * kScatterRows > 2147483647LL)
    return set_error(CP_ERR_OVERFLOW, "H_kv*D*2=%lld is too large a row", (long long)row_bytes);
  if (page_size < 1) return set_error(CP_ERR_INVALID_ARG, "page_size=%d", page_size);
  if (num_pages < 1) return set_error(CP_ERR_INVALID_ARG, "num_pages=%d", num_pages);
  if (!k_gathered || !v_gathered || !k_pool || !v_pool || !kv_page_indptr || !kv_page_indices)
    return set_error(CP_ERR_INVALID_ARG, "a device pointer is NULL");
  if (!aligned16(k_gathered) || !aligned16(v_gathered) || !aligned16(k_pool) || !aligned16(v_pool))
    return set_error(CP_ERR_INVALID_ARG, "K/V buffers must be 16-byte aligned");
  const int64_t parts = (meta->max_chunk_rows + kScatterRows - 1) / kScatterRows;
  const int64_t grid = parts * meta->n_chunks;
  if (grid > 2147483647LL) return set_error(CP_ERR_OVERFLOW, "scatter grid too large");
  if (grid == 0) return CP_OK;
  const Chunk* chunks = reinterpret_cast<const Chunk*>(static_cast<const char*>(d_blob) + meta->off_chunks);
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0, stream, chunks,
                     (int32_t)parts, static_cast<const unsigned char*>(k_gathered),
                     static_cast<const unsigned char*>(v_gathered), static_cast<unsigned char*>(k_pool),
                     static_cast<unsigned char*>(v_pool), row_bytes, num_pages, page_size,
                     kv_page_indptr, kv_page_indices);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CP_ERR_HIP, "scatter launch: %s", hipGetErrorString(e));
  return CP_OK;
}
