// Host entry point of the fused zigzag CP prefill attention (gfx950):
// validates every argument before anything is enqueued, picks the page-id
// mode of the kernel in cp_attn_kernel.h and launches one grid over the
// work list of the metadata blob.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/cpattn.h"
#include "cp_attn_kernel.h"
#include "cp_internal.h"

namespace cpattn {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Items must average this many key tiles for run-time job hand-out to pay
// for its ticket (one device-scope atomic before a workgroup's first load).
constexpr int kDynamicMinTiles = 48;

// Compute units of the device that runs `stream` (the current device for
// the null stream), queried once per device.
int compute_units(hipStream_t stream, int* n_cu) {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(CP_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= (int)cache.size()) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n < 1)
      return set_error(CP_ERR_HIP, "compute-unit count of device %d: %s", dev, hipGetErrorString(e));
    cache[dev] = n;
  }
  *n_cu = cache[dev];
  return CP_OK;
}

// Job counters of cp_prefill_attn_noalloc: one array per device (each GPU
// holds its own copy for the life of the process), zero at load and left zero
// by every launch.  In host code `scratch` names a host-side stand-in; the
// kernels get the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned int scratch[kCtrWords];

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
int scratch_address(hipStream_t stream, unsigned int** out) {
  static std::mutex mu;
  static std::vector<unsigned int*> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(CP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (stream) {
    int sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return set_error(CP_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
    if (sdev != dev)
      return set_error(CP_ERR_INVALID_ARG, "the stream belongs to device %d, the current device is %d",
                       sdev, dev);
  }
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= (int)cache.size()) cache.resize(dev + 1, nullptr);
  if (!cache[dev]) {
    unsigned int* p = nullptr;
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(CP_ERR_HIP, "address of the job counters on device %d: %s", dev, hipGetErrorString(e));
    cache[dev] = p;
  }
  *out = cache[dev];
  return CP_OK;
}

// Where a launch keeps its job counters.
enum class CtrHome { kBlob, kStatic };

// Validation, scheduling and launch shared by both entry points.
int prefill_attn(const void* q, const void* k_pool, const void* v_pool, void* out, int32_t H_q,
                 int32_t H_kv, int32_t D, float scale, const void* d_blob, const cp_meta_t* meta,
                 int32_t num_pages, int32_t page_size, const int32_t* kv_page_indptr,
                 const int32_t* kv_page_indices, hipStream_t stream, CtrHome home) {
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
  // One job per (work item, KV head).  Jobs [0, n_static) go to workgroups
  // [0, n_static); with run-time scheduling the other workgroups take the
  // remaining jobs from the blob's counters, and n_spare more let the faster
  // XCDs take more than their share (those that find nothing left end at once).
  const int64_t n_jobs = (int64_t)meta->n_work * H_kv;
  if (n_jobs == 0) return CP_OK;
  // HIP rejects a launch whose grid holds more than 2^32-1 work-items.
  if (n_jobs > 4294967295LL / kThreads)
    return set_error(CP_ERR_OVERFLOW, "attention grid too large (%lld workgroups of %d threads)",
                     (long long)n_jobs, kThreads);
  int n_cu = 0;
  if (int rc = compute_units(stream, &n_cu)) return rc;
  const bool dynamic = n_jobs > n_cu && meta->mean_item_tiles >= kDynamicMinTiles;
  const int64_t n_static = dynamic ? n_cu : n_jobs;
  const int64_t n_spare = dynamic ? std::max<int64_t>(8, (n_jobs - n_static) / 8) : 0;
  const int64_t grid = n_jobs + n_spare;
  if (grid > 4294967295LL / kThreads)
    return set_error(CP_ERR_OVERFLOW, "attention grid too large (%lld workgroups of %d threads)",
                     (long long)grid, kThreads);
  unsigned int* ctr = nullptr;
  if (home == CtrHome::kStatic) {
    if (int rc = scratch_address(stream, &ctr)) return rc;
  } else {
    // the caller's blob, written by this launch (the public entry point takes it non-const)
    ctr = reinterpret_cast<unsigned int*>(const_cast<char*>(static_cast<const char*>(d_blob)) + kCtrOffset);
  }
  AttnArgs args;
  args.q = static_cast<const unsigned char*>(q);
  args.k_pool = static_cast<const unsigned char*>(k_pool);
  args.v_pool = static_cast<const unsigned char*>(v_pool);
  args.out = static_cast<unsigned char*>(out);
  const char* base = static_cast<const char*>(d_blob);
  args.ctr = ctr;
  args.n_jobs = (int32_t)n_jobs;
  args.n_static = (int32_t)n_static;
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

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" int cp_prefill_attn(const void* q, const void* k_pool, const void* v_pool, void* out,
                               int32_t H_q, int32_t H_kv, int32_t D, float scale,
                               void* d_blob, const cp_meta_t* meta,
                               int32_t num_pages, int32_t page_size, const int32_t* kv_page_indptr,
                               const int32_t* kv_page_indices, hipStream_t stream) {
  return prefill_attn(q, k_pool, v_pool, out, H_q, H_kv, D, scale, d_blob, meta, num_pages, page_size,
                      kv_page_indptr, kv_page_indices, stream, CtrHome::kBlob);
}

extern "C" int cp_prefill_attn_noalloc(const void* q, const void* k_pool, const void* v_pool, void* out,
                                       int32_t H_q, int32_t H_kv, int32_t D, float scale,
                                       const void* d_blob, const cp_meta_t* meta,
                                       int32_t num_pages, int32_t page_size,
                                       const int32_t* kv_page_indptr, const int32_t* kv_page_indices,
                                       hipStream_t stream) {
  return prefill_attn(q, k_pool, v_pool, out, H_q, H_kv, D, scale, d_blob, meta, num_pages, page_size,
                      kv_page_indptr, kv_page_indices, stream, CtrHome::kStatic);
}
