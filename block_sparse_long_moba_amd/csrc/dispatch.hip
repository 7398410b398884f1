// Dispatch: regroup (row, head, slot) choices by chosen block, MoE style.
//
// MoBA summary page (paper-graph-ui), section 3.4, "Implementation", step 2:
// queries that chose an earlier block are collected per block so each block's
// keys and values are read once for all of them; the query's own block is
// handled separately (causal, contiguous) and is not dispatched.
//
// Bins are (kv head of the pass p, global block gb) -> p*NBb + gb. Three
// passes: per-workgroup LDS histograms added into global counts, one
// exclusive scan (items, and tiles of the attention kernel's query rows), and
// a scatter that reserves a range per (workgroup, bin) and fills it from LDS
// cursors; a record per tile follows the scan. Item order inside a bin is
// unspecified; every consumer treats a bin's items independently.
#include "moba_internal.h"

namespace moba {
namespace {

template <bool SCATTER>
__global__ __launch_bounds__(256) void dispatch_kernel(const int32_t *__restrict__ idx,
                                                       const int4 *__restrict__ info, int64_t NBb,
                                                       int Hp, int G, int k,
                                                       uint32_t *__restrict__ bin_count,
                                                       const uint32_t *__restrict__ bin_off,
                                                       uint32_t *__restrict__ cursor,
                                                       uint32_t *__restrict__ items) {
  const int64_t gb = blockIdx.x;
  const int4 bi = info[gb];
  if (bi.x < 0 || (int)blockIdx.y * kDispatchTokens >= bi.z) return;
  const int c = bi.w;
  if (c == 0 || k == 1) return;  // no earlier blocks to dispatch
  const int P = Hp / G;
  const int nbins = P * c;       // local bin (p, j) -> p*c + j
  if (nbins > kLdsBins) return;  // only if max_seqlen understated the longest sequence
  __shared__ uint32_t hist[kLdsBins];
  for (int i = threadIdx.x; i < nbins; i += 256) hist[i] = 0;
  __syncthreads();
  const int nh = min(k, c + 1) - 1;  // earlier-block entries per (row, head)
  const int rows = min(kDispatchTokens, bi.z - (int)blockIdx.y * kDispatchTokens);
  const int64_t t0 = bi.y + (int64_t)blockIdx.y * kDispatchTokens;
  const int n = rows * Hp;
  for (int rr = threadIdx.x; rr < n; rr += 256) {
    const int hl = rr % Hp;
    const int64_t row = (t0 + rr / Hp) * Hp + hl;
    const int32_t *sel = idx + row * k;
    const int base = (hl / G) * c;
    for (int s = 0; s < nh; ++s) {
      const int j = sel[s];
      if (j >= 0 && j < c) atomicAdd(&hist[base + j], 1u);
    }
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
  for (int rr = threadIdx.x; rr < n; rr += 256) {
    const int hl = rr % Hp;
    const int64_t row = (t0 + rr / Hp) * Hp + hl;
    const int32_t *sel = idx + row * k;
    const int base = (hl / G) * c;
    for (int s = 0; s < nh; ++s) {
      const int j = sel[s];
      if (j >= 0 && j < c) {
        const uint32_t pos = atomicAdd(&hist[base + j], 1u);
        items[pos] = (uint32_t)(row * k + s);
      }
    }
  }
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

hipError_t launch_dispatch(const Problem &pb, const Work &w, hipStream_t s) {
  const int64_t nbins = (int64_t)pb.P * pb.NBb;
  hipError_t e = launch_fill_u32(w.bin_count, 0u, nbins, s);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)pb.NBb, (unsigned)((pb.B + kDispatchTokens - 1) / kDispatchTokens));
  dispatch_kernel<false><<<grid, 256, 0, s>>>(w.idx, w.blk_info, pb.NBb, pb.Hp, pb.G, pb.k,
                                              w.bin_count, w.bin_off, w.cursor, w.items);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dispatch_scan_kernel<<<1, 1024, 0, s>>>(w.bin_count, nbins, (uint32_t)pb.rows, w.bin_off,
                                          w.tile_off, w.cursor);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  tile_rec_kernel<<<dim3((unsigned)((w.max_tiles + 255) / 256)), 256, 0, s>>>(
      w.tile_off, w.bin_off, w.blk_info, pb.NBb, nbins, w.max_tiles, (uint32_t)pb.rows,
      w.tile_rec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dispatch_kernel<true><<<grid, 256, 0, s>>>(w.idx, w.blk_info, pb.NBb, pb.Hp, pb.G, pb.k,
                                             w.bin_count, w.bin_off, w.cursor, w.items);
  return hipGetLastError();
}

}  // namespace moba
