// Fused zigzag context-parallel prefill attention for gfx950 (MI355X).
//
// One launch covers every segment of a metadata blob: both zigzag halves of
// every sequence (causal, bottom-right aligned: row i of a q_len-row half
// sees key j <= i + kv_len - q_len) or the one AllGather-KV slice
// (non-causal, keys [0, kv_len) of the global K/V).  Sources: sglang zigzag.py
// source page (run_attention: the prev and next halves with their own
// cu_seqlens_q and kv_len; build_metadata: kv_len_prev/next); the AITer GQA
// report (KV head of query head h is h / (H_q/H_kv), scale 1/sqrt(D)); the
// vllm-omni AllGather-KV pull request (local Q against global K/V, the pad
// suffix is never read).
//
// Work decomposition.  A workgroup (8 waves, 512 lanes) owns one KV head and
// 256 (position, query head) rows: q_tile = 256/G consecutive positions times
// the G query heads that share the KV head, head-minor.  Every K/V tile staged
// in LDS is therefore used by all G heads of the group.  Workgroup w takes KV
// head w % H_kv and work item w / H_kv: consecutive workgroups are dispatched
// round-robin over the 8 XCDs, so with H_kv in {1,2,4,8} each XCD sees one
// KV head (or a fixed subset) and its 4 MB L2 holds that head's K/V stream.
// Work items come longest-first from the host.
//
// Per wave: 32 rows.  Scores are computed transposed, S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 d from LDS, B = Q^T held in
// registers for the whole key loop), so lane l owns query column l%32 and
// 16 of the 32 keys of a block; the two lane halves of a column split the
// keys.  Row max needs one exchange between the halves (v_permlane32_swap);
// row sums stay per half until the end.  The probabilities are already in
// the B-operand layout of O^T = V^T P^T, so P never leaves registers; V^T
// comes from LDS through ds_read_b64_tr_b16.  O^T keeps each query in one
// lane, so the online-softmax rescale is lane-local as well.
//
// LDS: K and V tiles of 64 keys x D, double buffered (64 KiB at D = 128), rows
// of D*2 bytes with the 16-byte chunk index XOR-swizzled by the row so that
// both the K reads (16 rows, same chunk) and the transposed V reads (4 rows x
// 4 chunks) hit distinct banks.  Tiles arrive by direct global->LDS loads
// (global_load_lds_dwordx4) issued one tile ahead; the page ids they need are
// fetched two tiles ahead, so no load result is waited on before the end of
// the tile that hides it.
//
// Online softmax: the running max is raised only when a row's max grows by
// more than 2^8 (in exp2 units), so the O/l rescale is a rare wave-uniform
// branch instead of 64 multiplies per tile.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/cpattn.h"
#include "cp_internal.h"

namespace cpattn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

struct AttnArgs {
  const unsigned char* q;
  const unsigned char* k_pool;
  const unsigned char* v_pool;
  unsigned char* out;
  const Seg* segs;
  const Work* work;
  const int32_t* indptr;
  const int32_t* indices;
  int32_t h_q, h_kv, group, num_pages;
  int32_t page_shift;
  float scale_log2;  // softmax scale * log2(e): scores go through exp2
};

// 16-byte chunk slot of (row, chunk) inside a row of NC chunks.  For NC = 16
// the row's low 4 bits are permuted (bits 0-1 to 2-3) and XORed into the
// chunk: 16 consecutive rows at one chunk land in 16 different slots, and
// 4 consecutive rows x 4 aligned chunks do too.
template <int NC>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (NC == 16) {
    const int r = row & 15;
    return chunk ^ (((r & 3) << 2) | (r >> 2));
  } else {
    return chunk ^ ((row >> 1) & (NC - 1));
  }
}

__device__ __forceinline__ float wave_half_max(float x) {
  // max of x over lanes l and l^32 (v_permlane32_swap exchanges the halves)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 h = __builtin_convertvector(v, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnArgs a) {
  constexpr int NC = D / 8;               // 16-byte chunks per K/V row
  constexpr int KSTEPS = D / 16;          // k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;            // 32-row blocks of O^T
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = kAttnKeys * ROW_BYTES;
  constexpr int LOADS = TILE_BYTES / (kThreads * 16);  // 16-byte direct loads per lane per K (or V) tile
  static_assert(LOADS >= 1 && TILE_BYTES % (kThreads * 16) == 0, "loader shape");
  // [buf][K,V] tiles.  A direct global->LDS load writes 1 KiB per wave
  // instruction, lane i at +16*i; the lane picks the global chunk that the
  // swizzle puts in that slot.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2][TILE_BYTES];

  const int h_kv = a.h_kv, group = a.group;
  const int kvh = blockIdx.x % h_kv;
  const Work w = a.work[blockIdx.x / h_kv];
  const Seg s = a.segs[w.seg];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;

  // This lane's query row: position pos of the item, query head hg of the group.
  const int rho = wave * 32 + col;
  const int pos = rho / group, hg = rho - pos * group;
  const bool valid = rho < w.np * group;            // row exists in this item
  const int qp = w.p0 + pos;                        // segment-local position
  const bool live = valid && qp < s.q_len;          // row attends (else written as 0)
  const int64_t qrow = (int64_t)(s.q_row0 + qp) * a.h_q + (int64_t)kvh * group + hg;
  // Last visible key of this row; rows that do not attend use the segment's
  // last key so that their (zero-query) scores stay finite.
  const int limit = (s.causal && live) ? qp + s.causal_off : s.kv_len - 1;
  // Smallest limit of the item's rows: tiles ending at or below it need no mask.
  const int item_limit = s.causal ? w.p0 + s.causal_off : s.kv_len - 1;

  bf16x8 qop[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    if (live) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(a.q + (qrow * D + ks * 16 + half * 8) * 2);
      qop[ks] = __builtin_bit_cast(bf16x8, v);
    } else {
      qop[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }

  // Zero both buffers once: rows past kv_len are never loaded, and must hold
  // finite values (the masked scores select -inf, the zero probabilities
  // multiply V).  Later partial tiles keep finite rows of an earlier tile.
  {
    u32x4* z = reinterpret_cast<u32x4*>(&smem[0][0][0]);
#pragma unroll
    for (int i = tid; i < 4 * TILE_BYTES / 16; i += kThreads) z[i] = u32x4{0, 0, 0, 0};
  }

  // Loader geometry: direct load u of this lane writes LDS byte
  // (u*8 + wave)*1024 + 16*lane of the tile, i.e. one 16-byte slot of key row
  // ld_row[u]; it fetches the chunk that the swizzle places in that slot.
  const int32_t* ptab = a.indices + a.indptr[s.page_row];
  const int shift = a.page_shift;
  const int ps_mask = (1 << shift) - 1;
  const int64_t tok_stride = (int64_t)h_kv * ROW_BYTES;
  int ld_row[LOADS];
  int64_t ld_off[LOADS];   // byte offset of the chunk within a token row of the pool
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int o = (u * kWaves + wave) * 1024 + lane * 16;
    const int row = o / ROW_BYTES, slot = (o % ROW_BYTES) / 16;
    ld_row[u] = row;
    ld_off[u] = (int64_t)kvh * ROW_BYTES + (int64_t)(swz<NC>(row, slot)) * 16;  // swz is an involution
  }
  // Page ids: with pages of >= 64 keys a tile lies in one page and its id is
  // one scalar load; smaller pages give each lane its row's page.
  const bool page_per_tile = shift >= 6;
  auto page_id = [&](int t, int u) -> int {
    const int key = t * kAttnKeys + ld_row[u];
    if (page_per_tile) return ptab[(t * kAttnKeys) >> shift];
    return key < s.kv_len ? ptab[key >> shift] : 0;
  };
  auto issue_tile = [&](int t, int buf, const int* pg) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int key = t * kAttnKeys + ld_row[u];
      const int page = pg[u];
      if (key < s.kv_len && page >= 0 && page < a.num_pages) {
        const int64_t off = ((int64_t)page << shift | (key & ps_mask)) * tok_stride + ld_off[u];
        __builtin_amdgcn_global_load_lds(a.k_pool + off,
            (__attribute__((address_space(3))) void*)&smem[buf][0][(u * kWaves + wave) * 1024], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(a.v_pool + off,
            (__attribute__((address_space(3))) void*)&smem[buf][1][(u * kWaves + wave) * 1024], 16, 0, 0);
      }
    }
  };

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;
  // Rescale threshold: the running max is only raised when a row's max grows
  // by more than 8 in log2 units, so probabilities stay <= 2^8 and O/l are
  // rescaled rarely (the result is the same softmax with another reference).
  const float tau = 8.f / c;
  const int n_tiles = w.n_tiles;

  int pg_next[LOADS];   // page ids of the tile after the one being computed
  __syncthreads();      // zero fill done before any direct load lands
  if (n_tiles > 0) {
    int pg0[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) pg0[u] = page_id(0, u);
    issue_tile(0, 0, pg0);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) pg_next[u] = n_tiles > 1 ? page_id(1, u) : -1;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
    __syncthreads();
  }

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    // Issue the next tile's direct loads and fetch the page ids of the tile
    // after; nothing waits on either until the end of this iteration.
    if (t + 1 < n_tiles) issue_tile(t + 1, buf ^ 1, pg_next);
    int pg_after[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) pg_after[u] = (t + 2 < n_tiles) ? page_id(t + 2, u) : -1;

    // S^T for the 64 keys of this tile: two 32-key blocks.
    const unsigned char* kt = smem[buf][0];
    const unsigned char* vt = smem[buf][1];
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x16{};
      const int row = kb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(kt + row * ROW_BYTES + swz<NC>(row, ks * 2 + half) * 16);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qop[ks], sc[kb], 0, 0, 0);
      }
    }

    // Mask keys past each row's limit (only tiles that reach past the item's
    // smallest limit can hold such keys).
    const int kbase = t * kAttnKeys;
    if (kbase + kAttnKeys - 1 > item_limit) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kbase + kb * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
          if (key > limit) sc[kb][j] = -INFINITY;
        }
    }

    // Online softmax in base 2: p = exp2(s*c - m*c), m a reference no smaller
    // than 8/c below the row max seen so far.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[kb][j]);
    mx = wave_half_max(mx);
    const bool grow = mx > m_run + tau;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;
    float rs = 0.f;
    uint32_t pk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][j], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][j + 1], c, -mc));
        rs += p0 + p1;
        pk[kb][j >> 1] = pack_bf16x2(p0, p1);
      }
    l_run += rs;

    // O^T += V^T P^T over the 64 keys, four 16-key steps.  Step st uses C
    // elements 8*(st&1) .. +7 of key block st>>1, i.e. keys
    // 16*st + 8*(i/4) + 4*half + i%4 for operand slot i.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint32_t* pp = &pk[st >> 1][(st & 1) * 4];
      const bf16x8 pop = __builtin_bit_cast(bf16x8, u32x4{pp[0], pp[1], pp[2], pp[3]});
      // transposed V reads: 16-lane group gsub covers d0 .. d0+15 of a 32-d block
      const int j = lane & 15;
      const int gsub = (lane >> 4) & 1;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        i16x4 lo, hi;
        {
          const int row = st * 16 + half * 4 + (j >> 2);
          const int chunk = db * 4 + gsub * 2 + ((j & 3) >> 1);
          const int off = row * ROW_BYTES + swz<NC>(row, chunk) * 16 + (j & 1) * 8;
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((__attribute__((address_space(3))) unsigned char*)vt + off));
        }
        {
          const int row = st * 16 + 8 + half * 4 + (j >> 2);
          const int chunk = db * 4 + gsub * 2 + ((j & 3) >> 1);
          const int off = row * ROW_BYTES + swz<NC>(row, chunk) * 16 + (j & 1) * 8;
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((__attribute__((address_space(3))) unsigned char*)vt + off));
        }
        const i16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pop, o[db], 0, 0, 0);
      }
    }

#pragma unroll
    for (int u = 0; u < LOADS; ++u) pg_next[u] = pg_after[u];
    __builtin_amdgcn_s_waitcnt(0);   // next tile's direct loads from this wave have landed
    __syncthreads();                 // ... and from every wave; this tile's reads are done
  }

  // Epilogue: O = O^T / l.  Lane (col, half) holds d = 32*db + 8*(j/4) + 4*half + j%4.
  if (!valid) return;
  const float l_tot = wave_half_sum(l_run);
  const float inv = live ? 1.f / l_tot : 0.f;
  unsigned char* orow = a.out + qrow * D * 2;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = db * 32 + jj * 8 + half * 4;
      u32x2 v;
      v[0] = pack_bf16x2(o[db][jj * 4 + 0] * inv, o[db][jj * 4 + 1] * inv);
      v[1] = pack_bf16x2(o[db][jj * 4 + 2] * inv, o[db][jj * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d * 2) = v;
    }
}

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
  if (D == 128)
    hipLaunchKernelGGL(attn_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(attn_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CP_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return CP_OK;
}
