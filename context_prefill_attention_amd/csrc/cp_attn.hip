// Host entry point of the fused zigzag CP prefill attention (gfx950):
// validates every argument before anything is enqueued, picks the page-id
// mode of the kernel in cp_attn_kernel.h and launches one grid over the
// work list of the metadata blob.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/cpattn.h"
#include "cp_attn_kernel.h"
#include "cp_internal.h"

namespace cpattn {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" int cp_prefill_attn(const void* q, const void* k_pool, const void* v_pool, void* out,
                               int32_t H_q, int32_t H_kv, int32_t D, float scale,
                               const void* d_blob, const cp_meta_t* meta,
                               int32_t num_pages, int32_t page_size, const int32_t* kv_page_indptr,
                               const int32_t* kv_page_indices, hipStream_t stream) {
  clear_error();
  if (!meta || !d_blob) return set_error(CP_ERR_INVALID_ARG, "meta or d_blob is NULL");
  if (meta->version != CP_META_VERSION ||
      (meta->kind != CP_META_ZIGZAG && meta->kind != CP_META_ALLGATHER))
    return set_error(CP_ERR_INVALID_ARG, "unknown metadata kind/version");
  if (H_q < 1 || H_kv < 1 || H_q % H_kv != 0)
    return set_error(CP_ERR_INVALID_ARG,
                     "num_heads (%d) must be a multiple of num_kv_heads (%d)", H_q, H_kv);
  if (meta->attn_group != H_q / H_kv)
    return set_error(CP_ERR_INVALID_ARG, "metadata work list was built for H_q/H_kv=%d, not %d",
                     meta->attn_group, H_q / H_kv);
  if (D != 64 && D != 128) return set_error(CP_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  // A lane's load offset inside one 64-key tile is kept in 32 bits.
  if ((int64_t)H_kv * D * 2 * kAttnKeys > 2147483647LL)
    return set_error(CP_ERR_UNSUPPORTED, "H_kv=%d is too many KV heads for D=%d", H_kv, D);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return set_error(CP_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (page_size < 1 || (page_size & (page_size - 1)) != 0 || page_size > (1 << 20))
    return set_error(CP_ERR_UNSUPPORTED, "page_size=%d must be a power of two", page_size);
  if (num_pages < 1) return set_error(CP_ERR_INVALID_ARG, "num_pages=%d", num_pages);
  if (!q || !k_pool || !v_pool || !out || !kv_page_indptr || !kv_page_indices)
    return set_error(CP_ERR_INVALID_ARG, "a device pointer is NULL");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return set_error(CP_ERR_INVALID_ARG, "q, k_pool, v_pool and out must be 16-byte aligned");
  const int64_t grid = (int64_t)meta->n_work * H_kv;
  if (grid > 2147483647LL) return set_error(CP_ERR_OVERFLOW, "attention grid too large");
  if (grid == 0) return CP_OK;
  AttnArgs args;
  args.q = static_cast<const unsigned char*>(q);
  args.k_pool = static_cast<const unsigned char*>(k_pool);
  args.v_pool = static_cast<const unsigned char*>(v_pool);
  args.out = static_cast<unsigned char*>(out);
  const char* base = static_cast<const char*>(d_blob);
  args.segs = reinterpret_cast<const Seg*>(base + meta->off_segs);
  args.work = reinterpret_cast<const Work*>(base + meta->off_work);
  args.indptr = kv_page_indptr;
  args.indices = kv_page_indices;
  args.h_q = H_q;
  args.h_kv = H_kv;
  args.group = H_q / H_kv;
  args.num_pages = num_pages;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  args.page_shift = shift;
  args.scale_log2 = scale * 1.4426950408889634f;
  // Page mode: one page per tile (>= 64 keys), whole pages per tile (16 or
  // 32 keys, segments starting on page boundaries), or a lookup per lane.
  const int pm = shift >= 6 ? kPageTile
                 : (shift >= 4 && meta->kv_align >= page_size ? (1 << shift) : kPageLane);
  const dim3 g((unsigned)grid), b(kThreads);
#define CP_LAUNCH(DD, PMV) hipLaunchKernelGGL((attn_kernel<DD, PMV>), g, b, 0, stream, args)
  if (D == 128) {
    switch (pm) {
      case kPageTile: CP_LAUNCH(128, kPageTile); break;
      case 32: CP_LAUNCH(128, 32); break;
      case 16: CP_LAUNCH(128, 16); break;
      default: CP_LAUNCH(128, kPageLane); break;
    }
  } else {
    switch (pm) {
      case kPageTile: CP_LAUNCH(64, kPageTile); break;
      case 32: CP_LAUNCH(64, 32); break;
      case 16: CP_LAUNCH(64, 16); break;
      default: CP_LAUNCH(64, kPageLane); break;
    }
  }
#undef CP_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CP_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return CP_OK;
}
