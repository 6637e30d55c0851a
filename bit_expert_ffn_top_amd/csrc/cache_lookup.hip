// Expert-cache lookup and the grouping of (token, k-slot) pairs by expert.
//
// T*k <= 64 (the decode and verify steps): one wavefront, see below.
// Small inputs (T*k <= 1024): one workgroup.
//   slot = table[idx]; a bitmap of missed experts in LDS gives the ascending
//   distinct miss list by prefix popcount; each missed pair's position in the
//   (expert, t, i) order is the count of missed pairs that sort before it.
// Large inputs (prefill chunks): a three-pass counting sort that is stable in
// (t, i) order and needs no sort of keys:
//   1. per chunk of 32 tokens, a histogram of the selected pairs per expert;
//   2. a workgroup per expert scans its histogram entries over the chunks
//      (exclusive, in place); one workgroup then scans the experts' totals
//      into the groups' starts;
//   3. per chunk, one wavefront walks its tokens in order from cursors
//      start + chunk prefix; the k pairs of a token name distinct experts,
//      so the lanes bump distinct LDS cursors.
#include "moe_internal.h"
#include "route_device.h"

namespace bitffn {
namespace {

constexpr int kMaxE = MOE_MAX_EXPERTS;

__global__ __launch_bounds__(1024) void lookup_small_kernel(
    const int32_t* __restrict__ idx, int n, const int32_t* __restrict__ table, int E,
    int32_t* __restrict__ slot, int32_t* __restrict__ miss_expert,
    int32_t* __restrict__ miss_pair, int32_t* __restrict__ n_miss) {
  __shared__ uint32_t bitmap[kMaxE / 32];
  __shared__ int32_t s_exp[kSmallLookupPairs];
  __shared__ int32_t s_cnt;
  const int tid = threadIdx.x;
  if (tid < kMaxE / 32) bitmap[tid] = 0;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  int e = -1;
  bool miss = false;
  if (tid < n) {
    e = idx[tid];
    const int s = table[e];
    slot[tid] = s;
    miss = s < 0;
    if (miss) {
      atomicOr(&bitmap[e >> 5], 1u << (e & 31));
      atomicAdd(&s_cnt, 1);
    }
    s_exp[tid] = miss ? e : -1;
  }
  __syncthreads();
  // ascending distinct missed experts
  if (tid < E) {
    const uint32_t word = bitmap[tid >> 5];
    if ((word >> (tid & 31)) & 1u) {
      int pos = __popc(word & ((1u << (tid & 31)) - 1u));
      for (int w = 0; w < (tid >> 5); ++w) pos += __popc(bitmap[w]);
      miss_expert[pos] = tid;
    }
  }
  // missed pairs ordered by (expert, pair id)
  if (miss && miss_pair != nullptr) {
    int pos = 0;
    for (int q = 0; q < n; ++q) {
      const int eq = s_exp[q];
      pos += (eq >= 0) && (eq < e || (eq == e && q < tid));
    }
    miss_pair[pos] = tid;
  }
  if (tid == 0) {
    int distinct = 0;
    for (int w = 0; w < kMaxE / 32; ++w) distinct += __popc(bitmap[w]);
    n_miss[0] = distinct;
    n_miss[1] = s_cnt;
  }
}

// T*k <= 64: one wavefront, lane p = pair p (the shared miss-list builder).
__global__ __launch_bounds__(64) void lookup_wave_kernel(
    const int32_t* __restrict__ idx, int n, const int32_t* __restrict__ table,
    int32_t* __restrict__ slot, int32_t* __restrict__ miss_expert,
    int32_t* __restrict__ miss_pair, int32_t* __restrict__ n_miss) {
  const int p = threadIdx.x;
  int e = 0, s = -1;
  if (p < n) {
    e = idx[p];
    s = table[e];
    slot[p] = s;
  }
  wave_miss_lists(p, n, e, s, miss_expert, miss_pair, n_miss);
}

__device__ __forceinline__ bool selected(int s, bool select_hits, int n_slots) {
  return select_hits ? (s >= 0 && s < n_slots) : (s < 0);
}

// pass 1: per-chunk histograms
__global__ __launch_bounds__(256) void group_count_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ slot_of_pair,
    const int32_t* __restrict__ table, int T, int k, int E, bool select_hits, int n_slots,
    int32_t* __restrict__ chunk_counts) {
  __shared__ int32_t hist[kMaxE];
  const int chunk = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int t0 = chunk * kGroupChunkTokens;
  const int t1 = min(T, t0 + kGroupChunkTokens);
  for (int p = t0 * k + threadIdx.x; p < t1 * k; p += blockDim.x) {
    const int e = idx[p];
    const int s = slot_of_pair ? slot_of_pair[p] : table[e];
    if (selected(s, select_hits, n_slots)) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    chunk_counts[static_cast<int64_t>(chunk) * E + e] = hist[e];
}

// pass 2a: for each expert (one workgroup), the exclusive prefix of its
// counts over the chunks, in place, and its total.  Thread i owns a run of
// consecutive chunks; the run sums meet in a fixed-order scan in LDS.
constexpr int kScanThreads = 256;

__global__ __launch_bounds__(kScanThreads) void group_scan_chunks_kernel(
    int n_chunks, int E, int32_t* __restrict__ chunk_counts, int32_t* __restrict__ totals) {
  __shared__ int32_t s_run[kScanThreads];
  const int e = blockIdx.x;
  const int i = threadIdx.x;
  const int per = (n_chunks + kScanThreads - 1) / kScanThreads;
  const int c0 = min(n_chunks, i * per), c1 = min(n_chunks, c0 + per);
  int run = 0;
  for (int c = c0; c < c1; ++c) run += chunk_counts[static_cast<int64_t>(c) * E + e];
  s_run[i] = run;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {   // inclusive Hillis-Steele
    const int v = i >= off ? s_run[i - off] : 0;
    __syncthreads();
    s_run[i] += v;
    __syncthreads();
  }
  int acc = s_run[i] - run;   // exclusive start of this thread's run
  for (int c = c0; c < c1; ++c) {
    int32_t* p = chunk_counts + static_cast<int64_t>(c) * E + e;
    const int v = *p;
    *p = acc;
    acc += v;
  }
  if (i == kScanThreads - 1) totals[e] = s_run[i];
}

// pass 2b: over the experts (one workgroup): start of every group (into
// `starts`, and `offsets` if wanted), the distinct list, the counts and the
// tile bases.  Fixed-order Hillis-Steele scans.
__global__ __launch_bounds__(1024) void group_scan_kernel(
    int E, int T, const int32_t* __restrict__ totals, int32_t* __restrict__ starts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ distinct,
    int32_t* __restrict__ counts_out, int32_t* __restrict__ tile_base, int tile_m,
    int32_t* __restrict__ tile_group) {
  __shared__ int32_t s_tot[kMaxE];
  __shared__ int32_t s_nz[kMaxE];
  __shared__ int32_t s_tiles[kMaxE];
  const int e = threadIdx.x;
  const int tot = e < E ? totals[e] : 0;
  if (e < kMaxE) {
    s_tot[e] = tot;
    s_nz[e] = tot > 0 ? 1 : 0;
    s_tiles[e] = (tot + tile_m - 1) / tile_m;
  }
  __syncthreads();
  for (int off = 1; off < kMaxE; off <<= 1) {
    int a = 0, b = 0, c = 0;
    if (e < kMaxE && e >= off) {
      a = s_tot[e - off];
      b = s_nz[e - off];
      c = s_tiles[e - off];
    }
    __syncthreads();
    if (e < kMaxE && e >= off) {
      s_tot[e] += a;
      s_nz[e] += b;
      s_tiles[e] += c;
    }
    __syncthreads();
  }
  if (e < E) {
    const int start = s_tot[e] - tot;  // exclusive
    starts[e] = start;
    if (offsets) offsets[e] = start;
    if (distinct && tot > 0) distinct[s_nz[e] - 1] = e;
    if (tile_base) {
      const int nt = (tot + tile_m - 1) / tile_m;
      const int tb = s_tiles[e] - nt;
      tile_base[e] = tb;
      if (tile_group)
        for (int i = 0; i < nt; ++i) tile_group[tb + i] = e;
    }
  }
  if (e == 0) {
    const int total = s_tot[E - 1];
    if (offsets) offsets[E] = total;
    if (counts_out) {
      counts_out[0] = s_nz[E - 1];
      counts_out[1] = total;
    }
    if (tile_base) {
      const int base = s_tiles[E - 1];
      const int nt = (T + tile_m - 1) / tile_m;
      tile_base[E] = base;
      tile_base[E + 1] = base + nt;
      if (tile_group)
        for (int i = 0; i < nt; ++i) tile_group[base + i] = E;
    }
  }
}

// pass 3: stable scatter, one wavefront per chunk of tokens
__global__ __launch_bounds__(64) void group_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ slot_of_pair,
    const int32_t* __restrict__ table, int T, int k, int E, bool select_hits, int n_slots,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ starts,
    int32_t* __restrict__ perm, int32_t* __restrict__ pos, int32_t* __restrict__ group_slot) {
  static_assert(MOE_MAX_TOPK <= 64, "a token's pairs in one step of the wavefront");
  constexpr int kChunkPairs = kGroupChunkTokens * MOE_MAX_TOPK;
  constexpr int kPerLane = kChunkPairs / 64;
  __shared__ int32_t cursor[kMaxE];
  __shared__ int32_t s_start[kMaxE];     // each group's first position
  __shared__ int32_t s_e[kChunkPairs];   // the chunk's experts and slots, in pair order
  __shared__ int32_t s_s[kChunkPairs];
  const int chunk = blockIdx.x;
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) {
    const int st = starts[e];
    s_start[e] = st;
    cursor[e] = st + chunk_start[static_cast<int64_t>(chunk) * E + e];
  }
  const int t0 = chunk * kGroupChunkTokens;
  const int t1 = min(T, t0 + kGroupChunkTokens);
  const int n = (t1 - t0) * k;                       // pairs of this chunk
  const int64_t p0 = static_cast<int64_t>(t0) * k;
  // every expert id and slot of the chunk requested at once (two rounds when
  // the slots come from the table), then the ordered pass reads LDS only
  int ev[kPerLane];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int q = lane + 64 * j;
    ev[j] = q < n ? idx[p0 + q] : 0;
  }
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int q = lane + 64 * j;
    if (q < n) {
      s_e[q] = ev[j];
      s_s[q] = slot_of_pair ? slot_of_pair[p0 + q] : table[ev[j]];
    }
  }
  __syncthreads();
  // Tokens in order (k <= 64: one token per step of the wavefront).  The
  // workgroup is one wavefront, whose LDS accesses take effect in program
  // order, so a later token's cursor increment follows an earlier one's
  // without a barrier (a barrier here would also wait for every store).
  for (int t = t0; t < t1; ++t) {
    const int i = lane;
    if (i < k) {
      const int q = (t - t0) * k + i;
      const int p = t * k + i;
      const int e = s_e[q];
      const int s = s_s[q];
      int at = -1;
      if (selected(s, select_hits, n_slots)) {
        at = atomicAdd(&cursor[e], 1);
        if (perm) perm[at] = p;
        if (group_slot && at == s_start[e]) group_slot[e] = s;   // the group's first pair
      }
      if (pos) pos[p] = at;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(256) void lookup_slots_kernel(const int32_t* __restrict__ idx, int n,
                                                           const int32_t* __restrict__ table,
                                                           int32_t* __restrict__ slot) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p < n) slot[p] = table[idx[p]];
}

}  // namespace

hipError_t launch_lookup_slots(const int32_t* idx, int T, int k, const int32_t* table,
                               int32_t* slot, hipStream_t s) {
  const int n = T * k;
  if (n == 0) return hipSuccess;
  lookup_slots_kernel<<<(n + 255) / 256, 256, 0, s>>>(idx, n, table, slot);
  return hipGetLastError();
}

hipError_t launch_lookup_small(const int32_t* idx, int T, int k, const int32_t* table, int E,
                               int32_t* slot, int32_t* miss_expert, int32_t* miss_pair,
                               int32_t* n_miss, hipStream_t s) {
  if (T * k <= 64) {
    lookup_wave_kernel<<<1, 64, 0, s>>>(idx, T * k, table, slot, miss_expert, miss_pair, n_miss);
    return hipGetLastError();
  }
  lookup_small_kernel<<<1, 1024, 0, s>>>(idx, T * k, table, E, slot, miss_expert, miss_pair,
                                         n_miss);
  return hipGetLastError();
}

size_t group_workspace_bytes(int T, int E) {
  const int64_t n_chunks = (T + kGroupChunkTokens - 1) / kGroupChunkTokens;
  return static_cast<size_t>(align256(n_chunks * E * 4) + align256(2 * kMaxE * 4));
}

GroupWorkspace group_workspace(void* ws, int T, int E) {
  const int64_t n_chunks = (T + kGroupChunkTokens - 1) / kGroupChunkTokens;
  char* p = static_cast<char*>(ws);
  GroupWorkspace g;
  g.chunk_counts = reinterpret_cast<int32_t*>(p);
  g.totals = reinterpret_cast<int32_t*>(p + align256(n_chunks * E * 4));
  return g;
}

hipError_t launch_group_pairs(const int32_t* idx, const int32_t* slot_of_pair,
                              const int32_t* table, int T, int k, int E, bool select_hits,
                              int n_slots, GroupWorkspace gws, int32_t* offsets, int32_t* perm,
                              int32_t* pos, int32_t* distinct, int32_t* counts_out,
                              int32_t* tile_base, int tile_m, int32_t* tile_group,
                              int32_t* group_slot, hipStream_t s) {
  const int n_chunks = (T + kGroupChunkTokens - 1) / kGroupChunkTokens;
  group_count_kernel<<<n_chunks, 256, 0, s>>>(idx, slot_of_pair, table, T, k, E, select_hits,
                                              n_slots, gws.chunk_counts);
  group_scan_chunks_kernel<<<E, kScanThreads, 0, s>>>(n_chunks, E, gws.chunk_counts,
                                                      gws.totals);
  group_scan_kernel<<<1, 1024, 0, s>>>(E, T, gws.totals, gws.totals + kMaxE, offsets, distinct,
                                       counts_out, tile_base, tile_m > 0 ? tile_m : 1,
                                       tile_group);
  group_scatter_kernel<<<n_chunks, 64, 0, s>>>(idx, slot_of_pair, table, T, k, E, select_hits,
                                               n_slots, gws.chunk_counts, gws.totals + kMaxE, perm, pos,
                                               group_slot);
  return hipGetLastError();
}

}  // namespace bitffn
