// Memory-bound stages: block table, mean-pooled keys, value transpose, and
// the log-sum-exp merge of partial outputs.
#include <math.h>

#include <algorithm>

#include "moba_internal.h"

namespace moba {
namespace {

constexpr float kLog2eF = 1.4426950408889634f;

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *p, uint32_t value, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = value;
}

// Inclusive scan of one value per thread over a 1024-thread workgroup.
__device__ int block_scan_incl_1024(int x, int *wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int v = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int y = __shfl_up(v, o);
      if (lane >= o) v += y;
    }
    if (lane < 16) wsum[lane] = v;
  }
  __syncthreads();
  int r = x + (w > 0 ? wsum[w - 1] : 0);
  __syncthreads();
  return r;
}

// blk_first[s] = sum over earlier sequences of ceil(L/B) ("Context
// Partitioning" of the MoBA summary page, section 3.4: blocks restart in every
// sequence, the last one may be short). One workgroup of 1024 threads.
// Also keeps a copy of cu_seqlens next to the table for later stages, and
// checks what the host could not: cu_seqlens must start at 0, never decrease
// and end at T, and no sequence may have more than max_blocks blocks (the
// bound the workspace plan and the launch shapes were sized for). A failed
// check sets the status word; the fill kernel then marks every block invalid,
// so that no later kernel reads rows through the table.
__global__ __launch_bounds__(1024) void seqtable_scan_kernel(const int32_t *cu, int S, int B,
                                                             int64_t T, int max_blocks,
                                                             int32_t *blk_first,
                                                             int32_t *cu_copy,
                                                             int32_t *status) {
  __shared__ int wsum[16];
  __shared__ int carry;
  __shared__ int flags;
  if (threadIdx.x == 0) { carry = 0; flags = 0; }
  __syncthreads();
  int bad = 0;
  for (int base = 0; base < S; base += 1024) {
    int s = base + threadIdx.x;
    int v = 0;
    if (s < S) {
      const int L = cu[s + 1] - cu[s];
      if (L < 0) bad |= kStatusBadSeqlens;
      v = L > 0 ? (L + B - 1) / B : 0;
      if (v > max_blocks) bad |= kStatusTooManyBlocks;
    }
    if (s <= S) cu_copy[s] = cu[s];
    int incl = block_scan_incl_1024(v, wsum) + carry;
    if (s < S) blk_first[s] = incl - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry = incl;
    __syncthreads();
  }
  if (bad) atomicOr(&flags, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    blk_first[S] = carry;
    cu_copy[S] = cu[S];
    int f = flags;
    if (cu[0] != 0 || (int64_t)cu[S] != T) f |= kStatusBadSeqlens;
    *status = f;
  }
}

// blk_info[gb] = {sequence, first row, rows, local block index}; -1 past the
// end, and for every block when the status word reports bad input.
__global__ __launch_bounds__(256) void seqtable_fill_kernel(const int32_t *cu,
                                                            const int32_t *blk_first, int S,
                                                            int B, int64_t NBb,
                                                            const int32_t *status, int4 *info) {
  int64_t gb = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gb >= NBb) return;
  if (*status != 0 || gb >= blk_first[S]) {
    info[gb] = make_int4(-1, 0, 0, 0);
    return;
  }
  int lo = 0, hi = S - 1;  // largest s with blk_first[s] <= gb (skips empty sequences)
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (blk_first[mid] <= gb) lo = mid; else hi = mid - 1;
  }
  int j = (int)(gb - blk_first[lo]);
  int len = cu[lo + 1] - cu[lo];
  int rows = min(B, len - j * B);
  info[gb] = make_int4(lo, cu[lo] + j * B, rows, j);
}

// Fills n 32-bit words with `pattern` when the status word reports bad input
// (outputs of a call whose table check failed become NaN instead of stale
// memory); otherwise every workgroup returns at once.
__global__ __launch_bounds__(256) void poison_kernel(const int32_t *status, uint32_t *p, int64_t n,
                                                     uint32_t pattern) {
  if (*status == 0) return;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    p[i] = pattern;
}

template <typename T> struct Vec16;
template <> struct Vec16<__bf16> {
  static constexpr int N = 8;
  __device__ static void load(const __bf16 *p, float *f) {
    uint4 u = *(const uint4 *)p;
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void load(const float *p, float *f) {
    float4 u = *(const float4 *)p;
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
  }
};

// kbar[gb][g][:] = mean of the block's key rows ("Affinity Scoring", section
// 3.4 of the MoBA summary page; step 1 of its implementation). One workgroup
// per (block, kv head): 16 row groups x 16 column threads, fp64 accumulation so
// the stored fp32 mean is the correctly rounded block mean up to one rounding.
// Also writes the bf16 split hi = bf16(mean), lo = bf16(mean - hi) that the
// gate's matrix-core scores use (two bf16 products recover ~16 mantissa bits).
template <typename T>
__global__ __launch_bounds__(256) void meanpool_kernel(const T *__restrict__ k, RowHead ks,
                                                       const int4 *__restrict__ info, int Hkv,
                                                       float *__restrict__ kbar,
                                                       __bf16 *__restrict__ kbar_split) {
  constexpr int N = Vec16<T>::N;        // elements per 16-byte load
  constexpr int COLS = kHeadDim / N;    // threads per row: 16 (bf16) or 32 (fp32)
  constexpr int RG = 256 / COLS;        // row groups
  const int gb = blockIdx.x, g = blockIdx.y;
  const int4 bi = info[gb];
  if (bi.x < 0) return;
  const int col = threadIdx.x % COLS, rg = threadIdx.x / COLS;
  double acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.0;
  const int64_t stride = ks.t;
  const T *base = k + bi.y * ks.t + g * ks.h + col * N;
  int r = rg;
  for (; r + 3 * RG < bi.z; r += 4 * RG) {
    float f[4][N];
#pragma unroll
    for (int u = 0; u < 4; ++u) Vec16<T>::load(base + (int64_t)(r + u * RG) * stride, f[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += (double)f[u][i];
  }
  for (; r < bi.z; r += RG) {
    float f[N];
    Vec16<T>::load(base + (int64_t)r * stride, f);
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] += (double)f[i];
  }
  __shared__ double red[RG][kHeadDim];
#pragma unroll
  for (int i = 0; i < N; ++i) red[rg][col * N + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < RG; ++i) s += red[i][threadIdx.x];
    const float mean = (float)(s / (double)bi.z);
    kbar[((int64_t)gb * Hkv + g) * kHeadDim + threadIdx.x] = mean;
    const __bf16 hi = (__bf16)mean;
    const __bf16 lo = (__bf16)(mean - (float)hi);
    __bf16 *sp = kbar_split + ((int64_t)gb * Hkv + g) * 2 * kHeadDim + threadIdx.x;
    sp[0] = hi;
    sp[kHeadDim] = lo;
  }
}

// kmax / kmin[gb][g][:] = elementwise max / min of the block's key rows, the
// block representations of the extra picks by max and min pooling (MoBA
// review page, authors' rebuttals on mean pooling and on QUEST). Same
// workgroup shape as the mean; max and min are exact, and the bf16 hi / lo
// splits serve the matrix-core gate as for the mean.
template <typename T>
__global__ __launch_bounds__(256) void minmaxpool_kernel(const T *__restrict__ k, RowHead ks,
                                                         const int4 *__restrict__ info, int Hkv,
                                                         float *__restrict__ kmax,
                                                         float *__restrict__ kmin,
                                                         __bf16 *__restrict__ kmax_split,
                                                         __bf16 *__restrict__ kmin_split) {
  constexpr int N = Vec16<T>::N;
  constexpr int COLS = kHeadDim / N;
  constexpr int RG = 256 / COLS;
  const int gb = blockIdx.x, g = blockIdx.y;
  const int4 bi = info[gb];
  if (bi.x < 0) return;
  const int col = threadIdx.x % COLS, rg = threadIdx.x / COLS;
  float mx[N], mn[N];
#pragma unroll
  for (int i = 0; i < N; ++i) { mx[i] = -INFINITY; mn[i] = INFINITY; }
  const int64_t stride = ks.t;
  const T *base = k + bi.y * ks.t + g * ks.h + col * N;
  for (int r = rg; r < bi.z; r += RG) {
    float f[N];
    Vec16<T>::load(base + (int64_t)r * stride, f);
#pragma unroll
    for (int i = 0; i < N; ++i) { mx[i] = fmaxf(mx[i], f[i]); mn[i] = fminf(mn[i], f[i]); }
  }
  __shared__ float red[2][RG][kHeadDim];
#pragma unroll
  for (int i = 0; i < N; ++i) { red[0][rg][col * N + i] = mx[i]; red[1][rg][col * N + i] = mn[i]; }
  __syncthreads();
  if (threadIdx.x < 2 * kHeadDim) {
    const int which = threadIdx.x / kHeadDim, e = threadIdx.x % kHeadDim;
    float v = red[which][0][e];
#pragma unroll
    for (int i = 1; i < RG; ++i) v = which ? fminf(v, red[1][i][e]) : fmaxf(v, red[0][i][e]);
    const int64_t o = ((int64_t)gb * Hkv + g) * kHeadDim;
    (which ? kmin : kmax)[o + e] = v;
    const __bf16 hi = (__bf16)v;
    const __bf16 lo = (__bf16)(v - (float)hi);
    __bf16 *sp = (which ? kmin_split : kmax_split) + 2 * o + e;
    sp[0] = hi;
    sp[kHeadDim] = lo;
  }
}

// vt[p][gb][e][j] = v[first row of gb + j][g0 + p][e], zero past the block's
// rows: each block's values transposed so the attention kernels can feed them
// to the matrix cores with keys along the contraction. One 64-key tile per
// workgroup, transposed through LDS. The same workgroup also raises
// knorm[p][gb] to the largest Euclidean norm of its key rows, so that knorm
// ends as the largest key norm of the block (zeroed before the launch; norms
// are non-negative, so their bit patterns order like the values). It bounds
// every score of the block for a given query (|<q, k>| <= |q| |k|) and lets
// the attention kernels skip the exact tile maxima where the bound is small
// enough.
template <typename T>
__global__ __launch_bounds__(256) void vtrans_kernel(const T *__restrict__ v, RowHead vs,
                                                     const T *__restrict__ k, RowHead ks,
                                                     int g0, int64_t NBb, int B,
                                                     const int4 *__restrict__ info,
                                                     T *__restrict__ vt,
                                                     float *__restrict__ knorm) {
  constexpr int N = 16 / sizeof(T);
  constexpr int VPR = kHeadDim / N;   // 16-byte vectors per source row
  constexpr int PITCH = kHeadDim + 2; // LDS row pitch in elements
  const int ntile = B / kKeyTile;
  const int64_t gb = blockIdx.x / ntile;
  const int jt = blockIdx.x % ntile;
  const int p = blockIdx.y;
  const int4 bi = info[gb];
  if (bi.x < 0) return;
  __shared__ T tile[kKeyTile * PITCH];
  __shared__ float wmax[4];
  float nmax = 0.f;  // largest squared key norm among this thread's rows
  for (int c = threadIdx.x; c < kKeyTile * VPR; c += 256) {
    int r = c / VPR, col = c % VPR;
    int j = jt * kKeyTile + r;
    T tmp[N];
    float ss = 0.f;
    if (j < bi.z) {
      const int64_t row = bi.y + j;
      *(uint4 *)tmp = *(const uint4 *)(v + row * vs.t + (g0 + p) * vs.h + col * N);
      T kv[N];
      *(uint4 *)kv = *(const uint4 *)(k + row * ks.t + (g0 + p) * ks.h + col * N);
#pragma unroll
      for (int i = 0; i < N; ++i) ss = fmaf((float)kv[i], (float)kv[i], ss);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) tmp[i] = (T)0.0f;
    }
    // a row's VPR vectors are consecutive threads of one wave
#pragma unroll
    for (int o = 1; o < VPR; o <<= 1) ss += __shfl_xor(ss, o);
    nmax = fmaxf(nmax, ss);
#pragma unroll
    for (int i = 0; i < N; ++i) tile[r * PITCH + col * N + i] = tmp[i];
  }
#pragma unroll
  for (int o = 32; o >= VPR; o >>= 1) nmax = fmaxf(nmax, __shfl_xor(nmax, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = nmax;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax((unsigned *)&knorm[(int64_t)p * NBb + gb],
              __float_as_uint(sqrtf(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])))));
  constexpr int OVPR = kKeyTile / N;  // 16-byte vectors per output row
  T *dst = vt + (((int64_t)p * NBb + gb) * kHeadDim) * B + jt * kKeyTile;
  for (int c = threadIdx.x; c < kHeadDim * OVPR; c += 256) {
    int e = c / OVPR, col = c % OVPR;
    T tmp[N];
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[i] = tile[(col * N + i) * PITCH + e];
    *(uint4 *)(dst + (int64_t)e * B + col * N) = *(const uint4 *)tmp;
  }
}

__device__ __forceinline__ int seq_of_row(const int32_t *cu, int S, int64_t t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}


// Log-sum-exp combination of the per-block partial outputs (step 4 of the
// implementation in section 3.4 of the MoBA summary page: rescale each part by
// its normaliser). Slots are combined in ascending block order.
// One row (token, head) per group of LANES threads, 16 bytes of the row each;
// slot loads are issued four at a time so several are in flight per thread.
template <typename TO>
__global__ __launch_bounds__(256) void merge_kernel(const TO *__restrict__ part_o,
                                                    const float *__restrict__ part_lse,
                                                    const int32_t *__restrict__ cu, int S,
                                                    int64_t T_, int h0, int Hp, int B,
                                                    int k, const int32_t *__restrict__ status,
                                                    TO *__restrict__ out, RowHead os,
                                                    float *__restrict__ lse_out) {
  constexpr int N = 16 / sizeof(TO);       // elements per thread
  constexpr int LANES = kHeadDim / N;      // threads per row: 16 (bf16) or 32 (fp32)
  constexpr int ROWS = 256 / LANES;
  const int64_t row = (int64_t)blockIdx.x * ROWS + threadIdx.x / LANES;
  if (row >= T_ * Hp) return;
  const int lane = threadIdx.x % LANES;
  const int64_t t = row / Hp;
  const int hl = (int)(row % Hp);
  if (*status != 0) {  // bad cu_seqlens or block bound: no partial is valid
    TO nan[N];
#pragma unroll
    for (int j = 0; j < N; ++j) nan[j] = (TO)NAN;
    *(uint4 *)(out + t * os.t + (h0 + hl) * os.h + lane * N) = *(const uint4 *)nan;
    if (lane == 0 && lse_out) lse_out[(int64_t)(h0 + hl) * T_ + t] = NAN;
    return;
  }
  const int s = seq_of_row(cu, S, t);
  const int c = (int)((t - cu[s]) / B);
  const int nsel = min(k, c + 1);
  // a slot whose lse is -inf holds no block (a gate that picked fewer blocks
  // than it had slots) and is skipped
  // the row's lanes load its slots' lse values together (slot i0 + lane),
  // then reduce them with shuffles inside the row's lane group
  const float *pl = part_lse + row * k;
  float m = -INFINITY;
  for (int i0 = 0; i0 < nsel; i0 += LANES)
    m = fmaxf(m, i0 + lane < nsel ? pl[i0 + lane] : -INFINITY);
#pragma unroll
  for (int o = LANES / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, LANES));
  float sum = 0.f;
  for (int i0 = 0; i0 < nsel; i0 += LANES) {
    const float x = i0 + lane < nsel ? pl[i0 + lane] : -INFINITY;
    if (x > -INFINITY) sum += __builtin_amdgcn_exp2f((x - m) * kLog2eF);
  }
#pragma unroll
  for (int o = LANES / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o, LANES);
  const float L = m + logf(sum);
  float acc[N];
#pragma unroll
  for (int j = 0; j < N; ++j) acc[j] = 0.f;
  const TO *po = part_o + row * k * kHeadDim + lane * N;
  // all slots of the row in flight at once (16 per batch); lane u of the
  // group holds the weight of slot i0 + u, 0 for a slot past nsel or without
  // a block (whose row is not loaded)
  for (int i0 = 0; i0 < nsel; i0 += 16) {
    const float x = lane < 16 && i0 + lane < nsel ? pl[i0 + lane] : -INFINITY;
    const float wl = x > -INFINITY ? __builtin_amdgcn_exp2f((x - L) * kLog2eF) : 0.f;
    float wgt[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) wgt[u] = __shfl(wl, u, LANES);
    uint4 raw[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      raw[u] = wgt[u] != 0.f ? *(const uint4 *)(po + (int64_t)(i0 + u) * kHeadDim)
                             : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const TO *v = (const TO *)&raw[u];
#pragma unroll
      for (int j = 0; j < N; ++j) acc[j] += wgt[u] * (float)v[j];
    }
  }
  TO res[N];
#pragma unroll
  for (int j = 0; j < N; ++j) res[j] = (TO)acc[j];
  *(uint4 *)(out + t * os.t + (h0 + hl) * os.h + lane * N) = *(const uint4 *)res;
  if (lane == 0 && lse_out) lse_out[(int64_t)(h0 + hl) * T_ + t] = L;
}

// NaN in every output row of the pass and its lse when the sequence-table
// scan rejected the input (*status != 0); returns at once otherwise. Chunk c
// of row (t, hl) is 16 bytes of out.
template <typename TO>
__global__ __launch_bounds__(256) void nan_rows_kernel(const int32_t *__restrict__ status,
                                                       int64_t T_, int h0, int Hp,
                                                       TO *__restrict__ out, RowHead os,
                                                       float *__restrict__ lse_out) {
  if (*status == 0) return;
  constexpr int N = 16 / sizeof(TO);
  constexpr int C = kHeadDim / N;
  TO nan[N];
#pragma unroll
  for (int j = 0; j < N; ++j) nan[j] = (TO)NAN;
  const int64_t n = T_ * Hp * C;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / C;
    const int c = (int)(i % C);
    const int64_t t = row / Hp;
    const int hl = (int)(row % Hp);
    *(uint4 *)(out + t * os.t + (h0 + hl) * os.h + c * N) = *(const uint4 *)nan;
    if (c == 0 && lse_out) lse_out[(int64_t)(h0 + hl) * T_ + t] = NAN;
  }
}

}  // namespace

hipError_t launch_nan_rows(const Problem &pb, const Work &w, int g0, void *out, float *lse,
                           hipStream_t s) {
  const int64_t chunks = pb.T * pb.Hp * (pb.bf16 ? 16 : 32);
  if (chunks == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((chunks + 255) / 256, 1024));
  const int h0 = g0 * pb.G;
  if (pb.bf16)
    nan_rows_kernel<__bf16><<<grid, 256, 0, s>>>(w.status, pb.T, h0, pb.Hp, (__bf16 *)out, pb.os,
                                                 lse);
  else
    nan_rows_kernel<float><<<grid, 256, 0, s>>>(w.status, pb.T, h0, pb.Hp, (float *)out, pb.os,
                                                lse);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, uint32_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_u32_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(p, value, n);
  return hipGetLastError();
}

hipError_t launch_seqtable(const int32_t *cu, int S, int B, int64_t T, int max_blocks,
                           int64_t NBb, int32_t *blk_first, int32_t *cu_copy, int32_t *status,
                           int4 *blk_info, hipStream_t s) {
  seqtable_scan_kernel<<<1, 1024, 0, s>>>(cu, S, B, T, max_blocks, blk_first, cu_copy, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  seqtable_fill_kernel<<<dim3((unsigned)((NBb + 255) / 256)), dim3(256), 0, s>>>(
      cu, blk_first, S, B, NBb, status, blk_info);
  return hipGetLastError();
}

hipError_t launch_poison(const int32_t *status, void *p, int64_t words, uint32_t pattern,
                         hipStream_t s) {
  if (words <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>((words + 255) / 256, 1024);
  poison_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(status, (uint32_t *)p, words, pattern);
  return hipGetLastError();
}

hipError_t launch_meanpool(const Problem &pb, const Work &w, const void *k, hipStream_t s) {
  dim3 grid((unsigned)pb.NBb, (unsigned)pb.Hkv);
  if (pb.bf16)
    meanpool_kernel<__bf16><<<grid, 256, 0, s>>>((const __bf16 *)k, pb.ks, w.blk_info, pb.Hkv,
                                                  w.kbar, w.kbar_split);
  else
    meanpool_kernel<float><<<grid, 256, 0, s>>>((const float *)k, pb.ks, w.blk_info, pb.Hkv,
                                                 w.kbar, w.kbar_split);
  return hipGetLastError();
}

hipError_t launch_minmaxpool(const Problem &pb, const Work &w, const void *k, hipStream_t s) {
  dim3 grid((unsigned)pb.NBb, (unsigned)pb.Hkv);
  if (pb.bf16)
    minmaxpool_kernel<__bf16><<<grid, 256, 0, s>>>((const __bf16 *)k, pb.ks, w.blk_info, pb.Hkv,
                                                    w.kmax, w.kmin, w.kmax_split, w.kmin_split);
  else
    minmaxpool_kernel<float><<<grid, 256, 0, s>>>((const float *)k, pb.ks, w.blk_info, pb.Hkv,
                                                   w.kmax, w.kmin, w.kmax_split, w.kmin_split);
  return hipGetLastError();
}

hipError_t launch_vtrans(const void *v, RowHead vs, const void *k, RowHead ks, int bf16, int g0,
                         int P, int64_t NBb, int B, const int4 *blk_info, void *vt, float *knorm,
                         hipStream_t s) {
  dim3 grid((unsigned)(NBb * (B / kKeyTile)), (unsigned)P);
  const hipError_t e = launch_fill_u32((uint32_t *)knorm, 0u, (int64_t)P * NBb, s);
  if (e != hipSuccess) return e;
  if (bf16)
    vtrans_kernel<__bf16><<<grid, 256, 0, s>>>((const __bf16 *)v, vs, (const __bf16 *)k, ks, g0,
                                               NBb, B, blk_info, (__bf16 *)vt, knorm);
  else
    vtrans_kernel<float><<<grid, 256, 0, s>>>((const float *)v, vs, (const float *)k, ks, g0,
                                              NBb, B, blk_info, (float *)vt, knorm);
  return hipGetLastError();
}

hipError_t launch_merge(const Problem &pb, const Work &w, int g0, void *out, float *lse,
                        hipStream_t s) {
  const int32_t *cu = w.cu;
  const int64_t rows = pb.T * pb.Hp;
  if (rows == 0) return hipSuccess;
  const int rows_per_wg = pb.bf16 ? 16 : 8;
  dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  const int h0 = g0 * pb.G;
  if (pb.bf16)
    merge_kernel<__bf16><<<grid, 256, 0, s>>>((const __bf16 *)w.part_o, w.part_lse, cu, pb.S,
                                              pb.T, h0, pb.Hp, pb.B, pb.k, w.status,
                                              (__bf16 *)out, pb.os, lse);
  else
    merge_kernel<float><<<grid, 256, 0, s>>>((const float *)w.part_o, w.part_lse, cu, pb.S, pb.T,
                                             h0, pb.Hp, pb.B, pb.k, w.status, (float *)out,
                                             pb.os, lse);
  return hipGetLastError();
}

}  // namespace moba
