// Fused zigzag context-parallel prefill attention for gfx950 (MI355X).
//
// One launch covers every segment of a metadata blob: both zigzag halves of
// every sequence (causal, bottom-right aligned: row i of a q_len-row half
// sees key j <= i + kv_len - q_len) or the AllGather-KV slice (non-causal,
// each local query row against the keys of its own document of the ordered
// global K/V).  Sources: sglang zigzag.py
// source page (run_attention: the prev and next halves with their own
// cu_seqlens_q and kv_len; build_metadata: kv_len_prev/next); the AITer GQA
// report (KV head of query head h is h / (H_q/H_kv), scale 1/sqrt(D)); the
// vllm-omni AllGather-KV pull request (local Q against global K/V, the pad
// suffix is never read).
//
// Work decomposition.  A workgroup (8 waves, 512 lanes) owns one KV head and
// 256 (position, query head) rows: q_tile = 256/G consecutive positions times
// the G query heads that share the KV head, head-minor.  Every K/V tile staged
// in LDS is therefore used by all G heads of the group.  Job j is KV head
// j % H_kv of work item j / H_kv; work items come longest-first from the host.
// Consecutive workgroups are dispatched round-robin over the 8 XCDs, so with
// H_kv in {1,2,4,8} and job j run on XCD j % 8, each XCD sees one KV head (or
// a fixed subset) and its 4 MB L2 holds that head's K/V stream.
//
// Scheduling.  Workgroup b runs job b (static), or, when the host asks for
// run-time scheduling, the first round (b < n_static, one per CU) runs job b
// and every later workgroup takes a ticket: jobs n_static.. are dealt to 8
// queues, queue q holding n_static + q + 8t in order, and a workgroup draws
// from the queue of the XCD it runs on, which keeps the head-per-XCD pattern.
// The XCDs of one chip do not run at one speed (the same tiles take a few
// per cent longer on some), so with a fixed split the chip waits for its
// slowest XCD; here an XCD whose queue is empty draws from the next queue
// with jobs left, and the spare workgroups of the grid give the faster XCDs
// the slots to do so.
//
// Per wave: 32 rows.  Scores are computed transposed, S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 d from LDS, B = Q^T held in
// registers for the whole key loop), so lane l owns query column l%32 and
// 16 of the 32 keys of a block; the two lane halves of a column split the
// keys.  The probabilities are already in the B-operand layout of
// O^T = V^T P^T, so P never leaves registers; V^T comes from LDS through
// ds_read_b64_tr_b16.  O^T keeps each query in one lane, so the softmax and
// its rescale are lane-local apart from one exchange between the lane halves
// (v_permlane32_swap) per 32-key block.
//
// LDS: a ring of four K and V tile stages, 64 keys x D each (128 KiB at
// D = 128), rows of D*2 bytes with the 16-byte chunk index XOR-swizzled by
// the row so that both the K reads (16 rows, same chunk) and the transposed V
// reads (4 rows x 4 chunks) hit distinct banks.  Tiles arrive by direct
// global->LDS loads (global_load_lds_dwordx4) issued two tiles ahead; the
// page ids they need are fetched three tiles ahead, so no load result is
// waited on before the barrier that publishes its tile.
//
// Software pipeline: each step handles the QK product of tile t and the PV
// product of tile t-1, in two halves of 16 MFMAs; each half also carries the
// softmax of one 32-key block, whose VALU work is independent of that half's
// MFMAs, so the two overlap within the wave.  The two waves sharing a SIMD
// meet at every step's barrier; raising a wave's issue priority during
// half 1 lets the one that lags close the gap.
//
// Online softmax: probabilities are taken against a lazy reference maximum,
// raised only when a lane's sum over one 32-key block would exceed 2^32 (or
// is not finite), so the O/l rescale is a rare wave-uniform branch instead of
// 64 multiplies per block.  Row sums are accumulated in fp32 from the
// unrounded probabilities.
//
// Device code only; the host entry point (cp_prefill_attn in cp_attn.hip)
// validates the arguments, picks the page mode and launches it.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

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
  // Run-time scheduling: the job counters in the blob header (queues 0-7 and
  // the ticket count), the number of jobs and of statically placed ones
  // (n_static == n_jobs: every workgroup runs its own index, no counters).
  unsigned int* ctr;
  int32_t n_jobs, n_static;
};

// Job of workgroup b; called by all 64 lanes of wave 0, returns the same
// value in each (-1: nothing left).  Ticket takers draw from the queue of
// their XCD (hardware register XCC_ID) with one atomic; when it is empty,
// lanes 0-7 read the 8 queue counters at once and the wave draws from the
// first queue after its own with jobs left, again until all are empty (each
// failed draw finds one more queue empty, so at most 8 rounds).
__device__ __forceinline__ int take_job(unsigned int* ctr, int n_jobs, int n_static, int lane) {
  const int b = (int)blockIdx.x;
  if (b < n_static) return b;
  const int n_dyn = n_jobs - n_static;
  // jobs of queue q: n_static + q + 8t for t < n_q(q)
  auto n_q = [&](int q) -> unsigned int { return q < n_dyn ? (unsigned int)(n_dyn - q + 7) / 8u : 0u; };
  const int x = (int)(__builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 7);   // XCC_ID[3:0]
  unsigned int t = 0;
  if (lane == 0 && n_q(x) > 0) t = atomicAdd(&ctr[x], 1u);
  t = __builtin_amdgcn_readfirstlane(t);
  if (t < n_q(x)) return n_static + x + 8 * (int)t;
  for (int round = 0; round < 8; ++round) {
    unsigned int c = 0xffffffffu;
    if (lane < 8) c = __hip_atomic_load(&ctr[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t left = __builtin_amdgcn_ballot_w64(lane < 8 && c < n_q(lane));
    if (left == 0) break;
    const uint64_t rot = ((left >> x) | (left << (8 - x))) & 0xff;   // bit k: queue (x + k) % 8
    const int q = (x + (int)__builtin_ctzll(rot)) & 7;
    unsigned int t2 = 0;
    if (lane == q) t2 = atomicAdd(&ctr[q], 1u);
    t2 = __builtin_amdgcn_readlane(t2, q);
    if (t2 < n_q(q)) return n_static + q + 8 * (int)t2;
  }
  return -1;
}

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

constexpr int kStages = 4;   // LDS ring depth (tiles); loads run two tiles ahead

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (lgkm and exp counters left unconstrained).
// Encoding: vmcnt bits 3:0 and 15:14, expcnt bits 6:4, lgkmcnt bits 11:8.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Page modes.  PM == kPageTile: pages hold >= 64 keys, a tile lies in one
// page (or, after an unaligned segment start, two) and its id is one scalar
// load.  PM in {16, 32}: pages of PM keys and every segment starts on a
// page boundary, so a tile holds 64/PM whole pages whose ids are again
// scalar loads.  PM == kPageLane (pages under 16 keys, or unaligned
// segments): every lane looks up its own row's page with a vector load.
constexpr int kPageLane = 0, kPageTile = 1;

template <int D, int PM>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnArgs a) {
  constexpr int NC = D / 8;               // 16-byte chunks per K/V row
  constexpr int KSTEPS = D / 16;          // k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;            // 32-row blocks of O^T
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = kAttnKeys * ROW_BYTES;    // one K (or V) tile
  constexpr int LOADS = TILE_BYTES / (kThreads * 16);  // 16-byte direct loads per lane per K (or V) tile
  constexpr bool PAGE_PER_TILE = PM == kPageTile;
  constexpr int GP = PM >= 16 ? PM : 0;                // page size of the group modes
  constexpr int NPP = GP ? kAttnKeys / GP : 1;         // pages per tile in the group modes
  static_assert(LOADS >= 1 && TILE_BYTES % (kThreads * 16) == 0, "loader shape");
  // K and V rings of kStages tiles, one array per stage: the compiler can
  // then tell the stage being read from the stages whose direct loads are
  // still in flight and does not wait for those loads before the read.  A
  // direct global->LDS load writes 1 KiB per wave instruction, lane i at
  // +16*i; the lane picks the global chunk that the swizzle puts in that slot.
  __shared__ __attribute__((aligned(1024))) unsigned char k_s0[TILE_BYTES], k_s1[TILE_BYTES],
      k_s2[TILE_BYTES], k_s3[TILE_BYTES], v_s0[TILE_BYTES], v_s1[TILE_BYTES], v_s2[TILE_BYTES],
      v_s3[TILE_BYTES];
  static_assert(kStages == 4, "one array per ring stage");
  auto kbuf = [&](auto stc) -> unsigned char* {
    constexpr int st = decltype(stc)::value;
    if constexpr (st == 0) return k_s0; else if constexpr (st == 1) return k_s1;
    else if constexpr (st == 2) return k_s2; else return k_s3;
  };
  auto vbuf = [&](auto stc) -> unsigned char* {
    constexpr int st = decltype(stc)::value;
    if constexpr (st == 0) return v_s0; else if constexpr (st == 1) return v_s1;
    else if constexpr (st == 2) return v_s2; else return v_s3;
  };

  const int h_kv = a.h_kv, group = a.group;
  // Ticket takers also count themselves in ctr[8]; the count's result is only
  // looked at when this workgroup ends, so its round trip overlaps the job.
  // The last of them (every draw of this launch is done by then) clears the
  // counters for the next launch.
  __shared__ int job_slot;
  const unsigned int n_takers = gridDim.x - (unsigned int)a.n_static;
  unsigned int taker_no = 0;   // thread 0 of a ticket taker: 1 + its place in the count
  if (threadIdx.x < 64) {
    const int jb = take_job(a.ctr, a.n_jobs, a.n_static, threadIdx.x);
    if (threadIdx.x == 0) {
      job_slot = jb;
      if ((int)blockIdx.x >= a.n_static) taker_no = atomicAdd(&a.ctr[8], 1u) + 1u;
    }
  }
  auto clear_counters = [&]() {
    if (threadIdx.x == 0 && n_takers != 0u && taker_no == n_takers) {
#pragma unroll
      for (int i = 0; i < kCtrWords; ++i)
        __hip_atomic_store(&a.ctr[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  __syncthreads();
  const int job = __builtin_amdgcn_readfirstlane(job_slot);
  if (job < 0) {
    clear_counters();
    return;
  }
  const int kvh = job % h_kv;
  const Work w = a.work[job / h_kv];
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
  const int n_tiles = w.n_tiles;
  // first tile that holds a key past some row's limit
  const int t_mask = min(n_tiles, max(0, (item_limit + 1) / kAttnKeys));

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

  // Loader geometry: direct load u of this lane writes LDS byte
  // (u*8 + wave)*1024 + 16*lane of the tile, i.e. one 16-byte slot of key row
  // ld_row[u]; it fetches the chunk that the swizzle places in that slot.
  // The page table is read-only for the whole kernel: read it through the
  // constant address space so that wave-uniform lookups become scalar loads.
  typedef const __attribute__((address_space(4))) int32_t cint32;
  cint32* ptab = (cint32*)(a.indices) + a.indptr[s.page_row];
  const int shift = a.page_shift;
  const int ps_mask = (1 << shift) - 1;
  const uint32_t tok_stride = (uint32_t)h_kv * ROW_BYTES;
  // Key j of the segment is position kv0 + j of its page-table row (kv0 > 0
  // for all but the first document of a packed AllGather-KV slice).  When kv0
  // is not a multiple of the tile size, a tile may straddle two pages.
  const int kv0 = s.kv_start;
  const bool straddle = (kv0 & (kAttnKeys - 1)) != 0;
  const int n_entries = a.indptr[s.page_row + 1] - a.indptr[s.page_row];
  int ld_row[LOADS];
  uint32_t ld_lane[LOADS];   // chunk offset from the head-0 start of the lane's token row
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int o = (u * kWaves + wave) * 1024 + lane * 16;
    const int row = o / ROW_BYTES, slot = (o % ROW_BYTES) / 16;
    ld_row[u] = row;
    ld_lane[u] = (uint32_t)(kvh * ROW_BYTES + swz<NC>(row, slot) * 16);  // swz is an involution
  }
  // Every tile issues exactly LOADS direct loads of K and LOADS of V per
  // lane (and, with small pages, LOADS page-id loads), whatever the row: rows
  // past kv_len or with a page id outside the pool are redirected to key 0 of
  // the sequence (always real and finite) and masked out of the scores.  The
  // per-wave vector-memory counts are then exact and the waits below can
  // leave the younger tiles in flight.
  // With pages of >= 64 keys: the page of the tile's first key and, if the
  // tile may straddle a page boundary, the next one.
  // Group modes: the tile's NPP pages as scalars (pg.p[j] = page of keys
  // j*GP .. j*GP+GP-1 of the tile); lane lookups: the page of each of this
  // lane's rows.
  constexpr int NPG = PAGE_PER_TILE ? 2 : (GP != 0 ? NPP : LOADS);
  struct Pages { int p[NPG]; };
  // Every page-table read stays inside the segment's row [0, n_entries): a
  // row shorter than its keys need repeats its last entry (those keys then
  // read a wrong page, never memory outside the table), and an empty row
  // reads as page -1, which the loads redirect like any invalid page id.
  const int last_entry = max(n_entries - 1, 0);
  auto entry = [&](int e) -> int { return n_entries > 0 ? ptab[min(e, last_entry)] : -1; };
  auto fetch_pages = [&](int t) -> Pages {
    Pages pg;
    if constexpr (PAGE_PER_TILE) {
      const int e0 = (kv0 + min(t, n_tiles - 1) * kAttnKeys) >> shift;
      pg.p[0] = entry(e0);
      pg.p[1] = entry(straddle ? e0 + 1 : e0);   // an address choice: nothing waits for pg.p[0] here
    } else if constexpr (GP != 0) {
      const int e0 = (kv0 + min(t, n_tiles - 1) * kAttnKeys) >> shift;
#pragma unroll
      for (int j = 0; j < NPP; ++j) pg.p[j] = entry(e0 + j);
    } else {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int key = max(0, min(t * kAttnKeys + ld_row[u], s.kv_len - 1));
        pg.p[u] = entry((kv0 + key) >> shift);
      }
    }
    return pg;
  };
  const int page0 = entry(0);
  const bool page0_ok = page0 >= 0 && page0 < a.num_pages;
  // Per-lane part of a load address when a whole tile lies in one page.
  uint32_t ld_const[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) ld_const[u] = (uint32_t)ld_row[u] * tok_stride + ld_lane[u];
  // The same from the first key row of the lane's wave instruction, for the
  // group modes, whose base moves to that row's page.
  constexpr int kRowsPerLoad = 1024 / ROW_BYTES;
  static_assert(GP == 0 || GP % kRowsPerLoad == 0, "a wave instruction's rows lie in one page");
  uint32_t ld_gconst[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u)
    ld_gconst[u] = (uint32_t)(ld_row[u] - (u * kWaves + wave) * kRowsPerLoad) * tok_stride + ld_lane[u];
  auto issue_tile = [&](int t, auto stc, const Pages& pg) {
    unsigned char* kd = kbuf(stc);
    unsigned char* vd = vbuf(stc);
    // Common case: every key of the tile is real and its page id valid, and
    // the tile lies in one page or runs on into the next pool page (adjacent
    // pages, as a contiguous K/V tensor read through the identity table
    // gives), so each address is a wave-uniform base plus a per-lane constant.
    const int first = kv0 + t * kAttnKeys;   // page-table position of the tile's key 0
    if constexpr (PAGE_PER_TILE) {
      if ((t + 1) * kAttnKeys <= s.kv_len && pg.p[0] >= 0 && pg.p[0] < a.num_pages &&
          ((first & ps_mask) + kAttnKeys <= ps_mask + 1 || (pg.p[1] == pg.p[0] + 1 && pg.p[1] < a.num_pages))) {
        // wave-uniform tile base (scalar registers) plus a 32-bit per-lane
        // offset: the loads take the scalar-base address form, no vector adds
        const uint64_t base =
            (((uint64_t)pg.p[0] << shift) | (uint32_t)(first & ps_mask)) * tok_stride;
        const unsigned char* k_base = a.k_pool + base;
        const unsigned char* v_base = a.v_pool + base;
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
          __builtin_amdgcn_global_load_lds(k_base + (int64_t)ld_const[u],
              (__attribute__((address_space(3))) void*)&kd[(u * kWaves + wave) * 1024], 16, 0, 0);
          __builtin_amdgcn_global_load_lds(v_base + (int64_t)ld_const[u],
              (__attribute__((address_space(3))) void*)&vd[(u * kWaves + wave) * 1024], 16, 0, 0);
        }
        return;
      }
    }
    if constexpr (GP != 0) {
      // Group modes: the rows of one wave instruction lie in one page (GP is
      // a multiple of the rows it covers), so with all keys real and the
      // pages valid each load is again a scalar base plus a per-lane constant.
      if ((t + 1) * kAttnKeys <= s.kv_len) {
        int pu[LOADS];
        bool ok = true;
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
          const int j = (u * kWaves + wave) * kRowsPerLoad / GP;   // wave-uniform
          int pj = pg.p[0];
#pragma unroll
          for (int i = 1; i < NPP; ++i) pj = j == i ? pg.p[i] : pj;
          pu[u] = pj;
          ok = ok && pj >= 0 && pj < a.num_pages;
        }
        if (ok) {
#pragma unroll
          for (int u = 0; u < LOADS; ++u) {
            const int row0 = (u * kWaves + wave) * kRowsPerLoad;
            const uint64_t base =
                (((uint64_t)pu[u] << shift) | (uint32_t)((first + row0) & ps_mask)) * tok_stride;
            __builtin_amdgcn_global_load_lds(a.k_pool + base + (int64_t)ld_gconst[u],
                (__attribute__((address_space(3))) void*)&kd[(u * kWaves + wave) * 1024], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(a.v_pool + base + (int64_t)ld_gconst[u],
                (__attribute__((address_space(3))) void*)&vd[(u * kWaves + wave) * 1024], 16, 0, 0);
          }
          return;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int key = t * kAttnKeys + ld_row[u];
      const int pos = kv0 + key;
      int page;
      if constexpr (PAGE_PER_TILE) {
        page = (pos >> shift) == (first >> shift) ? pg.p[0] : pg.p[1];
      } else if constexpr (GP != 0) {
        // Page j = ld_row[u] / GP of the tile holds this lane's row, chosen
        // by a tree of selects on the bits of j (a flat compare chain would
        // be turned into an indexed array in memory).
        const int j = ld_row[u] / GP;
        static_assert(NPP == 2 || NPP == 4, "group modes hold 2 or 4 pages per tile");
        const int q0 = pg.p[0] ^ ((pg.p[0] ^ pg.p[1]) & -(j & 1));
        if constexpr (NPP == 2) {
          page = q0;
        } else {
          const int q1 = (j & 1) ? pg.p[3] : pg.p[2];
          page = (j & 2) ? q1 : q0;
        }
      } else {
        page = pg.p[u];
      }
      const bool ok = key < s.kv_len && page >= 0 && page < a.num_pages;
      const int64_t tok = ok ? ((int64_t)page << shift | (pos & ps_mask))
                             : (page0_ok ? (int64_t)page0 << shift : 0);
      const int64_t off = tok * tok_stride + ld_lane[u];
      __builtin_amdgcn_global_load_lds(a.k_pool + off,
          (__attribute__((address_space(3))) void*)&kd[(u * kWaves + wave) * 1024], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(a.v_pool + off,
          (__attribute__((address_space(3))) void*)&vd[(u * kWaves + wave) * 1024], 16, 0, 0);
    }
  };
  // Wait until tile t's direct loads have landed, given what this wave
  // issued after them: the loads of tile t+1, if it exists.  With small
  // pages the page ids fetched in this step are vector loads too; the
  // compiler may place them before or after the loads of tile t+1, so none
  // of them is counted as allowed to stay outstanding.
  auto wait_tile = [&](int t) {
    if (t + 1 < n_tiles) wait_vmcnt<2 * LOADS>();
    else wait_vmcnt<0>();
  };

  // LDS read offsets of this lane, fixed for the whole loop (stage, block
  // and step offsets are immediates):
  //   K: key row kb*32 + col, chunk 2*ks + half       (kb adds 32 rows)
  //   V: key row 16*st + 8*e + 4*half + j/4, chunk 4*db + 2*gsub + (j%4)/2,
  //      8-byte half j%2                              (st adds 16 rows)
  // 16 rows do not change the swizzle, so both row offsets are additive.
  uint32_t kofs[KSTEPS], vofs[DBLK][2];
  {
    const int j = lane & 15, gsub = (lane >> 4) & 1;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) kofs[ks] = col * ROW_BYTES + swz<NC>(col, ks * 2 + half) * 16;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = 8 * e + half * 4 + (j >> 2);
        const int chunk = db * 4 + gsub * 2 + ((j & 3) >> 1);
        vofs[db][e] = row * ROW_BYTES + swz<NC>(row, chunk) * 16 + (j & 1) * 8;
      }
  }

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;
  // Rescale threshold: the running max is only raised when a lane's sum of
  // one block's probabilities against the current reference exceeds 2^32, so
  // O and l are rescaled rarely (the result is the same softmax with another
  // reference).
  constexpr float kSumLimit = 4294967296.f;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // S^T of key block kb (keys 32*kb .. 32*kb+31) of the tile in stage st:
  // KSTEPS MFMAs over d, K from LDS, Q^T from registers.
  auto qk_blk = [&](auto stc, auto kbc) -> f32x16 {
    constexpr int kb = decltype(kbc)::value;
    const unsigned char* kt = kbuf(stc) + kb * 32 * ROW_BYTES;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kt + kofs[ks]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qop[ks], acc, 0, 0, 0);
    }
    return acc;
  };
  // O^T += V^T P^T over key block kb of the tile in stage st, P of that
  // block in pb (8 registers of packed bf16 pairs, C-element order).  Two
  // 16-key steps; step kk uses C elements 8*kk .. 8*kk+7 of the block, i.e.
  // keys 32*kb + 16*kk + 8*(i/4) + 4*half + i%4 for operand slot i.
  auto pv_at = [&](unsigned char* vt, auto kbc, const uint32_t* pb) {
    constexpr int kb = decltype(kbc)::value;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kst = kb * 2 + kk;
      const uint32_t* pp = pb + kk * 4;
      const bf16x8 pop = __builtin_bit_cast(bf16x8, u32x4{pp[0], pp[1], pp[2], pp[3]});
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((__attribute__((address_space(3))) unsigned char*)vt + vofs[db][0] + kst * 16 * ROW_BYTES));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((__attribute__((address_space(3))) unsigned char*)vt + vofs[db][1] + kst * 16 * ROW_BYTES));
        const i16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pop, o[db], 0, 0, 0);
      }
    }
  };
  auto pv_blk = [&](auto stc, auto kbc, const uint32_t* pb) { pv_at(vbuf(stc), kbc, pb); };
  // Keys of block kb of tile t past each row's limit leave the scores.
  auto mask_blk = [&](int t, int kb, f32x16& sb) {
    const int rel = limit - t * kAttnKeys - kb * 32 - half * 4;   // visible key offsets within the block
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((j >> 2) * 8 + (j & 3) > rel) sb[j] = -INFINITY;
  };
  // Probabilities of one block against reference mr (exp2 domain), packed to
  // bf16 pairs in pb; returns their fp32 sum.
  auto probs_blk = [&](const f32x16& sb, float mr, uint32_t* pb) -> float {
    const float mc = mr * c;
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[j], c, -mc));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[j + 1], c, -mc));
      pb[j >> 1] = pack_bf16x2(p0, p1);
      r0 = j ? r0 + p0 : p0;
      r1 = j ? r1 + p1 : p1;
    }
    return r0 + r1;
  };
  // Online softmax of one 32-key block with a lazy reference: probabilities
  // against the current reference; if some lane's block sum exceeds 2^32 (or
  // is not finite), the rare raise of that wave's references to their rows'
  // maxima.  A raise rescales O and l, which at that point hold only terms
  // taken with the old reference, and recomputes this block's probabilities;
  // every other block's P has either been added to O already or is computed
  // later.  The test reads the sums themselves, so the common path stays one
  // basic block.  Between raises every probability stays below 2^32, far
  // from fp32 overflow in O and l.
  auto sm_blk = [&](const f32x16& sb, uint32_t* pb) {
    const float mc = m_run * c;
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[j], c, -mc));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[j + 1], c, -mc));
      pb[j >> 1] = pack_bf16x2(p0, p1);
      r0 = j ? r0 + p0 : p0;
      r1 = j ? r1 + p1 : p1;
    }
    float rs = r0 + r1;
    if (__builtin_amdgcn_ballot_w64(!(rs <= kSumLimit)) != 0) {   // rare: raise the references
      // The first pass's results count as used here, so the compiler keeps
      // that pass ahead of the branch, next to the MFMAs it overlaps, rather
      // than sinking it into the common path (which also splits O's
      // registers into two copies).
      asm volatile("" ::"v"(rs));
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(pb[j]));
      float mx = sb[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sb[j]);
      mx = wave_half_max(mx);
      const float m_new = fmaxf(m_run, mx);   // rows whose max did not grow keep theirs
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      rs = probs_blk(sb, m_new, pb);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    l_run += rs;
  };

  // Barrier between pipeline steps: this wave's LDS reads are complete, the
  // direct loads of the tile the next step computes have landed (the caller's
  // vmcnt wait), and no wave passes until all have.  A plain s_barrier: the
  // usual __syncthreads would also wait for the younger tiles still in flight.
  auto step_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Pipeline.  Tile t lives in ring stage t % 4.  Step t issues the page ids
  // of tile t+3 and the loads of tile t+2, then runs two halves, each one
  // basic block in which MFMAs and the softmax VALU work are independent:
  //   half 1: S^T block 0 of tile t, PV of block 0 of tile t-1, softmax of
  //           block 1 of tile t-1;
  //   half 2: S^T block 1 of tile t, PV of block 1 of tile t-1, softmax of
  //           block 0 of tile t.
  // The barrier at the end of step t publishes tile t+1 and retires every
  // read of tile t-1's stage, which step t+1 refills with tile t+3.
  // Between steps, s1 holds S^T block 1 of the last tile and pk[0..7] the
  // probabilities of its block 0; pk[8..15] hold block 1's once computed.
  uint32_t pk[16];
  if (n_tiles > 0) {
    Pages pg0 = fetch_pages(0), pg1 = fetch_pages(1);
    issue_tile(0, I0{}, pg0);
    Pages pg_next = fetch_pages(2);
    if (n_tiles > 1) issue_tile(1, I1{}, pg1);
    wait_tile(0);
    step_barrier();

    f32x16 s1;
    // Step 0: no previous tile.
    {
      const Pages pg_after = fetch_pages(3);
      if (2 < n_tiles) issue_tile(2, I2{}, pg_next);
      pg_next = pg_after;
      f32x16 s0 = qk_blk(I0{}, I0{});
      s1 = qk_blk(I0{}, I1{});
      if (t_mask == 0) {
        mask_blk(0, 0, s0);
        mask_blk(0, 1, s1);
      }
      sm_blk(s0, pk);
      wait_tile(1);
      step_barrier();
    }

    // Step t >= 1; MASKED tiles hold keys past some row's limit.
    auto step = [&](auto stc, auto maskc, int t) {
      constexpr int st = decltype(stc)::value;   // t % kStages
      constexpr bool MASKED = decltype(maskc)::value;
      using SP = std::integral_constant<int, (st + kStages - 1) % kStages>;   // stage of tile t-1
      const Pages pg_after = fetch_pages(t + 3);
      if (t + 2 < n_tiles) issue_tile(t + 2, std::integral_constant<int, (st + 2) % kStages>{}, pg_next);
      pg_next = pg_after;
      // A wave still in half 1 outranks one already in half 2 for the
      // SIMD's issue slots, so the wave that lags catches up before the
      // step barrier instead of both arriving at it far apart.
      __builtin_amdgcn_s_setprio(1);
      f32x16 s0 = qk_blk(stc, I0{});
      pv_blk(SP{}, I0{}, pk);
      sm_blk(s1, pk + 8);
      __builtin_amdgcn_s_setprio(0);
      s1 = qk_blk(stc, I1{});
      if constexpr (MASKED) mask_blk(t, 0, s0);
      pv_blk(SP{}, I1{}, pk + 8);
      sm_blk(s0, pk);
      if constexpr (MASKED) mask_blk(t, 1, s1);
      wait_tile(t + 1);
      step_barrier();
    };

    int t = 1;
    const int t_full_end = max(1, t_mask);          // tiles [1, t_mask) need no mask
    // Both loops are unrolled by the ring depth, so every stage index is a
    // constant.  After the first, t % 4 == 1; the second runs the remaining
    // tiles (a few fully visible ones, which the mask leaves unchanged, then
    // the diagonal) four at a time, and the last 0-3 tiles follow one by one.
    for (; t + 3 < t_full_end; t += 4) {
      step(I1{}, std::false_type{}, t);
      step(I2{}, std::false_type{}, t + 1);
      step(I3{}, std::false_type{}, t + 2);
      step(I0{}, std::false_type{}, t + 3);
    }
    for (; t + 3 < n_tiles; t += 4) {
      step(I1{}, std::true_type{}, t);
      step(I2{}, std::true_type{}, t + 1);
      step(I3{}, std::true_type{}, t + 2);
      step(I0{}, std::true_type{}, t + 3);
    }
    if (t < n_tiles) step(I1{}, std::true_type{}, t);
    if (t + 1 < n_tiles) step(I2{}, std::true_type{}, t + 1);
    if (t + 2 < n_tiles) step(I3{}, std::true_type{}, t + 2);
    // The last tile's PV products and its block-1 softmax, from its stage.
    const int st_last = (n_tiles - 1) & (kStages - 1);
    unsigned char* v_last = st_last == 0 ? v_s0 : st_last == 1 ? v_s1 : st_last == 2 ? v_s2 : v_s3;
    pv_at(v_last, I0{}, pk);
    sm_blk(s1, pk + 8);
    pv_at(v_last, I1{}, pk + 8);
  }

  // Epilogue: O = O^T / l.  Lane (col, half) holds d = 32*db + 8*(j/4) + 4*half + j%4.
  // (Thread 0 always holds a valid row: it reaches clear_counters below.)
  if (!valid) return;
  const float l_tot = wave_half_sum(l_run);   // the two lane halves summed different keys
  const float inv = live ? 1.f / l_tot : 0.f;
  unsigned char* orow = a.out + qrow * D * 2;
  // Stored as held, each store would write 8 bytes to each of 32 rows, and
  // the CU issues such stores slowly (the last wave of a workgroup ended
  // some 3 us after the first).  The lane halves of a row (same validity,
  // both active) swap 8-byte pieces so that each lane stores 16 bytes: half
  // 0 gets d 16*jp + 0..7 of block db, half 1 d 16*jp + 8..15, and a wave
  // issues 8 stores instead of 16.
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      uint32_t x[2], y[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        x[e] = pack_bf16x2(o[db][jp * 8 + 2 * e] * inv, o[db][jp * 8 + 2 * e + 1] * inv);
        y[e] = pack_bf16x2(o[db][jp * 8 + 4 + 2 * e] * inv, o[db][jp * 8 + 4 + 2 * e + 1] * inv);
        auto r = __builtin_amdgcn_permlane32_swap(x[e], y[e], false, false);
        x[e] = r[0];
        y[e] = r[1];
      }
      const int d = db * 32 + jp * 16 + half * 8;
      *reinterpret_cast<u32x4*>(orow + d * 2) = u32x4{x[0], x[1], y[0], y[1]};
    }
  clear_counters();
}

}  // namespace
}  // namespace cpattn
