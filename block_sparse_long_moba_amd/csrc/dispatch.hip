// Dispatch: regroup (row, head, slot) choices by chosen block, MoE style.
//
// MoBA summary page (paper-graph-ui), section 3.4, "Implementation", step 2:
// queries that chose an earlier block are collected per block so each block's
// keys and values are read once for all of them; the query's own block is
// handled separately (causal, contiguous) and is not dispatched.
//
// Bins are (kv head of the pass p, global block gb) -> p*NBb + gb. Three
// passes: per-workgroup LDS histograms added into global counts (the mean
// gate's matrix-core kernel already adds its own and marks them counted, and
// then this pass returns at once), one exclusive scan (items, and tiles of
// the attention kernel's query rows), and a scatter that reserves a range
// per (workgroup, bin) and fills it, through an LDS staging area grouped by
// bin where the workgroup's entries fit (else from LDS cursors, one scattered
// store per item); a record per tile follows the scan. Item order inside a bin is unspecified; every consumer
// treats a bin's items independently.
#include "moba_internal.h"

namespace moba {
namespace {

// Division by a runtime divisor d >= 1 of numerators n < 2^31: with
// m = floor((2^32 - 1) / d), umulhi(n, m) is floor(n / d) or one less
// (its error is below n (1 + 1/d) / 2^32 < 1), and one correction step
// makes it exact.
struct Div {
  uint32_t m, d;
  __device__ uint32_t div(uint32_t n) const {
    const uint32_t q = __umulhi(n, m);
    return q + (n - q * d >= d ? 1u : 0u);
  }
};

// One workgroup per (block, kDispRows rows): the idx entries of those rows
// (all query heads of the pass) form one contiguous run, read in order, one
// entry per lane. Entry f of the run is slot f % k of (row, head) f / k; its
// bin is (kv head of the pass) * c + (chosen block) for earlier blocks
// 0 <= block < c, and the item is the entry's index in idx.
// COUNT: adds the LDS histogram to the global bin counts (skipped when the
// gate counted already: *counted != 0). SCATTER: reserves a range per
// (workgroup, bin) and writes the items into it.
constexpr int kUnroll = 8;

template <bool SCATTER>
__global__ __launch_bounds__(256) void dispatch_kernel(const int32_t *__restrict__ idx,
                                                       const int4 *__restrict__ info, int64_t NBb,
                                                       int Hp, int G, int k, Div by_kG, Div by_P,
                                                       const uint32_t *__restrict__ counted,
                                                       uint32_t *__restrict__ bin_count,
                                                       const uint32_t *__restrict__ bin_off,
                                                       uint32_t *__restrict__ cursor,
                                                       uint32_t *__restrict__ items) {
  if (!SCATTER && *counted) return;
  const int64_t gb = blockIdx.x;
  const int4 bi = info[gb];
  if (bi.x < 0 || (int)blockIdx.y * kDispatchRows >= bi.z) return;
  const int c = bi.w;
  if (c == 0 || k == 1) return;  // no earlier blocks to dispatch
  const int P = Hp / G;
  const int nbins = P * c;       // local bin (p, j) -> p*c + j
  if (nbins > kLdsBins) return;  // never with a passed table check (the plan bounds P*c)
  extern __shared__ uint32_t hist[];  // P * (largest block count) entries
  for (int i = threadIdx.x; i < nbins; i += 256) hist[i] = 0;
  __syncthreads();
  const int rows = min(kDispatchRows, bi.z - (int)blockIdx.y * kDispatchRows);
  const int64_t f0 = (bi.y + (int64_t)blockIdx.y * kDispatchRows) * Hp * k;
  const uint32_t nf = (uint32_t)(rows * Hp * k);
  const int32_t *run = idx + f0;
  // bin of entry f: kv head (f / (k G)) mod P of the pass, block j
  auto bin_of = [&](uint32_t f, int j) {
    const uint32_t rg = by_kG.div(f);
    return (int)(rg - by_P.div(rg) * (uint32_t)P) * c + j;
  };
  // kUnroll entries per thread in flight at a time
  for (uint32_t f0l = threadIdx.x; f0l < nf; f0l += 256 * kUnroll) {
    int j[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) j[u] = f0l + 256 * u < nf ? run[f0l + 256 * u] : -1;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (j[u] >= 0 && j[u] < c) atomicAdd(&hist[bin_of(f0l + 256 * u, j[u])], 1u);
  }
  __syncthreads();
  const int64_t first = gb - c;  // global index of the sequence's block 0
  if (!SCATTER) {
    for (int i = threadIdx.x; i < nbins; i += 256) {
      const uint32_t cnt = hist[i];
      if (cnt) atomicAdd(&bin_count[(int64_t)(i / c) * NBb + first + i % c], cnt);
    }
    return;
  }
  for (int i = threadIdx.x; i < nbins; i += 256) {
    const uint32_t cnt = hist[i];
    if (cnt) {
      const int64_t b = (int64_t)(i / c) * NBb + first + i % c;
      hist[i] = bin_off[b] + atomicAdd(&cursor[b], cnt);
    }
  }
  __syncthreads();
  for (uint32_t f0l = threadIdx.x; f0l < nf; f0l += 256 * kUnroll) {
    int j[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) j[u] = f0l + 256 * u < nf ? run[f0l + 256 * u] : -1;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (j[u] >= 0 && j[u] < c) {
        const uint32_t f = f0l + 256 * u;
        const uint32_t pos = atomicAdd(&hist[bin_of(f, j[u])], 1u);
        items[pos] = (uint32_t)(f0 + f);
      }
  }
}

// Zeroes the bin counts unless the gate counted (*counted != 0).
__global__ __launch_bounds__(256) void dispatch_clear_kernel(const uint32_t *__restrict__ counted,
                                                             uint32_t *__restrict__ bin_count,
                                                             int64_t nbins) {
  if (*counted) return;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nbins) bin_count[i] = 0;
}

// Inclusive scan of one uint32 per thread over 1024 threads.
__device__ uint32_t scan1024(uint32_t x, uint32_t *wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    uint32_t v = lane < 16 ? wsum[lane] : 0u;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      uint32_t y = __shfl_up(v, o);
      if (lane >= o) v += y;
    }
    if (lane < 16) wsum[lane] = v;
  }
  __syncthreads();
  uint32_t r = x + (w > 0 ? wsum[w - 1] : 0u);
  __syncthreads();
  return r;
}

// Scatter with the workgroup's items staged in LDS, grouped by bin, so that
// each (workgroup, bin) range of items is written by consecutive lanes to
// consecutive addresses. A workgroup of 1024 threads takes R rows of one
// block (R * Hp * k <= kStageEntries); each thread keeps its kStagePer idx
// entries in registers. The LDS histogram's atomics return each entry's rank
// within its bin; an exclusive scan of the counts gives every bin's start in
// the staging area, one global atomic per (workgroup, bin) its range in
// items, and the entry is placed at start + rank. The staged entries are then
// written out in staging order.
constexpr int kStageThreads = 1024;
constexpr int kStagePer = 32;                               // idx entries per thread
constexpr int kStageEntries = kStageThreads * kStagePer;    // 32768 (128 KiB staged)
constexpr int kStageBins = 2048;                            // local bins (P * c)
constexpr int kStageFBits = 15;                             // bits of a local entry index

__global__ __launch_bounds__(kStageThreads) void dispatch_staged_kernel(
    const int32_t *__restrict__ idx, const int4 *__restrict__ info, int64_t NBb, int Hp, int G,
    int k, int R, Div by_kG, Div by_P, const uint32_t *__restrict__ bin_off,
    uint32_t *__restrict__ cursor, uint32_t *__restrict__ items) {
  const int64_t gb = blockIdx.x;
  const int4 bi = info[gb];
  const int r0 = (int)blockIdx.y * R;
  if (bi.x < 0 || r0 >= bi.z) return;
  const int c = bi.w;
  if (c == 0 || k == 1) return;  // no earlier blocks to dispatch
  const int P = Hp / G;
  const int nbins = P * c;
  if (nbins > kStageBins) return;  // never: the launcher picks this kernel only when they fit
  __shared__ uint32_t start[kStageBins];  // counts, then each bin's first staging slot
  __shared__ uint32_t delta[kStageBins];  // item position - staging slot, per bin
  __shared__ uint32_t stage[kStageEntries];
  __shared__ uint32_t wsum[16];
  const int tid = threadIdx.x;
  for (int i = tid; i < nbins; i += kStageThreads) start[i] = 0;
  __syncthreads();
  const int rows = min(R, bi.z - r0);
  const int64_t f0 = (bi.y + (int64_t)r0) * Hp * k;
  const uint32_t nf = (uint32_t)(rows * Hp * k);  // <= kStageEntries
  const int32_t *run = idx + f0;
  int32_t j[kStagePer];
#pragma unroll
  for (int u = 0; u < kStagePer; ++u) {
    const uint32_t f = (uint32_t)(u * kStageThreads + tid);
    j[u] = f < nf ? run[f] : -1;
  }
  // (local bin, rank within the bin) of each entry; ~0 for no earlier block
  uint32_t br[kStagePer];
#pragma unroll
  for (int u = 0; u < kStagePer; ++u) {
    br[u] = ~0u;
    if (j[u] >= 0 && j[u] < c) {
      const uint32_t f = (uint32_t)(u * kStageThreads + tid);
      const uint32_t rg = by_kG.div(f);
      const uint32_t bin = (rg - by_P.div(rg) * (uint32_t)P) * (uint32_t)c + (uint32_t)j[u];
      br[u] = (bin << 16) | atomicAdd(&start[bin], 1u);
    }
  }
  __syncthreads();
  // exclusive scan of the counts: two bins per thread
  const uint32_t c0 = 2 * tid < nbins ? start[2 * tid] : 0u;
  const uint32_t c1 = 2 * tid + 1 < nbins ? start[2 * tid + 1] : 0u;
  const uint32_t incl = scan1024(c0 + c1, wsum);
  const uint32_t s0 = incl - c0 - c1;
  const int64_t first = gb - c;
  if (2 * tid < nbins) {
    start[2 * tid] = s0;
    if (c0) {
      const int64_t b = (int64_t)((2 * tid) / c) * NBb + first + (2 * tid) % c;
      delta[2 * tid] = bin_off[b] + atomicAdd(&cursor[b], c0) - s0;
    }
  }
  if (2 * tid + 1 < nbins) {
    start[2 * tid + 1] = s0 + c0;
    if (c1) {
      const int64_t b = (int64_t)((2 * tid + 1) / c) * NBb + first + (2 * tid + 1) % c;
      delta[2 * tid + 1] = bin_off[b] + atomicAdd(&cursor[b], c1) - (s0 + c0);
    }
  }
  if (tid == kStageThreads - 1) wsum[0] = incl;  // entries staged
  __syncthreads();
  const uint32_t nstaged = wsum[0];
#pragma unroll
  for (int u = 0; u < kStagePer; ++u)
    if (br[u] != ~0u) {
      const uint32_t bin = br[u] >> 16;
      stage[start[bin] + (br[u] & 0xffffu)] =
          (bin << kStageFBits) | (uint32_t)(u * kStageThreads + tid);
    }
  __syncthreads();
  for (uint32_t s = tid; s < nstaged; s += kStageThreads) {
    const uint32_t e = stage[s];
    items[delta[e >> kStageFBits] + s] = (uint32_t)(f0 + (e & ((1u << kStageFBits) - 1u)));
  }
}

// Exclusive scans of the bin counts (item offsets) and of their tile counts
// (tiles of `rows` query rows); resets the scatter cursors.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const uint32_t *__restrict__ count,
                                                             int64_t nbins, uint32_t rows,
                                                             uint32_t *__restrict__ off,
                                                             uint32_t *__restrict__ tile_off,
                                                             uint32_t *__restrict__ cursor) {
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t carry[2];
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int64_t base = 0; base < nbins; base += 1024) {
    const int64_t b = base + threadIdx.x;
    const uint32_t n = b < nbins ? count[b] : 0u;
    const uint32_t nt = (n + rows - 1) / rows;
    const uint32_t in = scan1024(n, wsum) + carry[0];
    const uint32_t it = scan1024(nt, wsum) + carry[1];
    if (b < nbins) {
      off[b] = in - n;
      tile_off[b] = it - nt;
      cursor[b] = 0;
    }
    __syncthreads();
    if (threadIdx.x == 1023) { carry[0] = in; carry[1] = it; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    off[nbins] = carry[0];
    tile_off[nbins] = carry[1];
  }
}

// Record of attention tile i: {first item, rows, bin, first token of the
// bin's block}, for the bin b owning the tile (largest b with tile_off[b] <= i).
__global__ __launch_bounds__(256) void tile_rec_kernel(const uint32_t *__restrict__ tile_off,
                                                       const uint32_t *__restrict__ bin_off,
                                                       const int4 *__restrict__ info, int64_t NBb,
                                                       int64_t nbins, int64_t max_tiles,
                                                       uint32_t rows, int4 *__restrict__ tile_rec) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= max_tiles || i >= tile_off[nbins]) return;
  int64_t lo = 0, hi = nbins - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (tile_off[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const uint32_t r0 = bin_off[lo] + (uint32_t)(i - tile_off[lo]) * rows;
  const uint32_t n = min(rows, bin_off[lo + 1] - r0);
  tile_rec[i] = make_int4((int)r0, (int)n, (int)lo, info[lo % NBb].y);
}

}  // namespace

Div make_div(uint32_t d) { return Div{0xffffffffu / d, d}; }

hipError_t launch_dispatch(const Problem &pb, const Work &w, hipStream_t s) {
  const int64_t nbins = (int64_t)pb.P * pb.NBb;
  dispatch_clear_kernel<<<dim3((unsigned)((nbins + 255) / 256)), 256, 0, s>>>(w.counted, w.bin_count,
                                                                             nbins);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)pb.NBb, (unsigned)((pb.B + kDispatchRows - 1) / kDispatchRows));
  const Div by_kG = make_div((uint32_t)(pb.k * pb.G)), by_P = make_div((uint32_t)pb.P);
  const size_t lds = sizeof(uint32_t) * (size_t)pb.P * pb.maxblk;
  dispatch_kernel<false><<<grid, 256, lds, s>>>(w.idx, w.blk_info, pb.NBb, pb.Hp, pb.G, pb.k, by_kG,
                                              by_P, w.counted, w.bin_count, w.bin_off, w.cursor,
                                              w.items);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dispatch_scan_kernel<<<1, 1024, 0, s>>>(w.bin_count, nbins, (uint32_t)pb.rows, w.bin_off,
                                          w.tile_off, w.cursor);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  tile_rec_kernel<<<dim3((unsigned)((w.max_tiles + 255) / 256)), 256, 0, s>>>(
      w.tile_off, w.bin_off, w.blk_info, pb.NBb, nbins, w.max_tiles, (uint32_t)pb.rows,
      w.tile_rec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int per_row = pb.Hp * pb.k;
  if (per_row <= kStageEntries && (int64_t)pb.P * pb.maxblk <= kStageBins) {
    // as many rows per workgroup as the staging area holds, spread evenly
    const int rmax = kStageEntries / per_row;
    const int nwg = (pb.B + rmax - 1) / rmax;
    const int R = (pb.B + nwg - 1) / nwg;
    dispatch_staged_kernel<<<dim3((unsigned)pb.NBb, (unsigned)nwg), kStageThreads, 0, s>>>(
        w.idx, w.blk_info, pb.NBb, pb.Hp, pb.G, pb.k, R, by_kG, by_P, w.bin_off, w.cursor,
        w.items);
    return hipGetLastError();
  }
  dispatch_kernel<true><<<grid, 256, lds, s>>>(w.idx, w.blk_info, pb.NBb, pb.Hp, pb.G, pb.k, by_kG,
                                             by_P, w.counted, w.bin_count, w.bin_off, w.cursor,
                                             w.items);
  return hipGetLastError();
}

}  // namespace moba
