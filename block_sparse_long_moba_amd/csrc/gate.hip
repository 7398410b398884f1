// Gate: parameter-free top-k block selection per query head.
//
// MoBA summary page (paper-graph-ui), section 3.4: "Affinity Scoring"
// (s_j = <q, mean-pooled keys of block j>, no scaling), "Top-k Gating" (keep
// the k best; the query's own block is always kept and, in the reading used
// here, counts toward k), "Causality Enforcement" mechanism 1 (later blocks
// are never candidates). Review page (paperhub.cn), authors' rebuttal W1:
// each query head selects on its own.
//
// Two implementations of the mean gate: the matrix-core gate below (bf16
// inputs, GQA groups of a multiple of 4 query heads) and this vector gate
// (every other shape). Vector gate: one workgroup = 64 consecutive rows of
// one block x 4 query heads (one wave per head, one lane per row). Every row
// of the workgroup has the same own block c, so the candidate list 0..c-1 is
// uniform across the workgroup and the pooled-key rows are wave-uniform
// reads. Scores are fp32 dot products (q upcast exactly from bf16, kbar
// fp32), so a selection can differ from an exact one only where the k-th and
// (k+1)-th scores agree to ~1e-6.
#include <limits.h>

#include "moba_internal.h"

namespace moba {
namespace {

template <typename T> __device__ __forceinline__ void load_row_f32(const T *p, float *f);
template <> __device__ __forceinline__ void load_row_f32<__bf16>(const __bf16 *p, float *f) {
#pragma unroll
  for (int v = 0; v < kHeadDim / 8; ++v) {
    uint4 u = ((const uint4 *)p)[v];
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[8 * v + 2 * i] = __uint_as_float(w[i] << 16);
      f[8 * v + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}
template <> __device__ __forceinline__ void load_row_f32<float>(const float *p, float *f) {
#pragma unroll
  for (int v = 0; v < kHeadDim / 4; ++v) {
    float4 u = ((const float4 *)p)[v];
    f[4 * v] = u.x; f[4 * v + 1] = u.y; f[4 * v + 2] = u.z; f[4 * v + 3] = u.w;
  }
}

// Keeps ts[0..KMAX) sorted by (score desc, index asc). Candidates arrive in
// ascending block order, so a newcomer ranks below every kept entry with an
// equal score (ties go to the lower index) and a strict comparison suffices;
// kept entries only ever shift down by one, so their relative order holds.
template <int KMAX>
__device__ __forceinline__ void topk_insert(float (&ts)[KMAX], int (&ti)[KMAX], float s, int j) {
  if (s > ts[KMAX - 1]) {
#pragma unroll
    for (int i = KMAX - 1; i > 0; --i) {
      const bool up = s > ts[i - 1];
      const bool here = s > ts[i];
      ts[i] = up ? ts[i - 1] : (here ? s : ts[i]);
      ti[i] = up ? ti[i - 1] : (here ? j : ti[i]);
    }
    if (s > ts[0]) { ts[0] = s; ti[0] = j; }
  }
}

template <typename T, int KMAX>
__global__ __launch_bounds__(256) void gate_kernel(const T *__restrict__ q,
                                                   const float *__restrict__ kbar,
                                                   const int4 *__restrict__ info, RowHead qs,
                                                   int Hkv, int G, int h0, int Hp, int k,
                                                   int32_t *__restrict__ idx) {
  const int64_t gb = blockIdx.x;
  const int4 bi = info[gb];
  if (bi.x < 0 || (int)blockIdx.y * kGateTokens >= bi.z) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = blockIdx.z * 4 + wave;
  if (hl >= Hp) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.y * kGateTokens + lane;
  const bool active = r < bi.z;
  const int64_t t = bi.y + (active ? r : 0);
  const int c = bi.w;                // own (current) block, local index
  const int64_t first = gb - c;      // global index of the sequence's block 0
  const int h = h0 + hl;
  const int g = h / G;
  const int pick = k - 1;            // earlier blocks to choose
  int32_t *dst = idx + ((int64_t)t * Hp + hl) * k;

  if (pick >= c) {  // every earlier block fits: nothing to rank
    if (active) {
      for (int j = 0; j < c; ++j) dst[j] = j;
      dst[c] = c;
      for (int j = c + 1; j < k; ++j) dst[j] = -1;
    }
    return;
  }

  float qf[kHeadDim];
  load_row_f32<T>(q + t * qs.t + h * qs.h, qf);
  float ts[KMAX];
  int ti[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) { ts[i] = -INFINITY; ti[i] = INT_MAX; }

  const float *kb = kbar + (first * Hkv + g) * kHeadDim;
  const int64_t kstride = (int64_t)Hkv * kHeadDim;
  for (int j = 0; j < c; ++j, kb += kstride) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int e = 0; e < kHeadDim; e += 4) {
      const float4 kv = *(const float4 *)(kb + e);
      a0 = fmaf(qf[e], kv.x, a0);
      a1 = fmaf(qf[e + 1], kv.y, a1);
      a2 = fmaf(qf[e + 2], kv.z, a2);
      a3 = fmaf(qf[e + 3], kv.w, a3);
    }
    topk_insert<KMAX>(ts, ti, (a0 + a1) + (a2 + a3), j);
  }

  // chosen indices in ascending order (entries past `pick` become sentinels)
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
    if (i >= pick) ti[i] = INT_MAX;
#pragma unroll
  for (int pass = 0; pass < KMAX; ++pass)
#pragma unroll
    for (int i = pass & 1; i + 1 < KMAX; i += 2) {
      const int a = ti[i], b = ti[i + 1];
      ti[i] = min(a, b);
      ti[i + 1] = max(a, b);
    }
  if (active) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < pick) dst[i] = ti[i] == INT_MAX ? -1 : ti[i];  // -1 only for NaN scores
    dst[pick] = c;
  }
}

// ---- Matrix-core gate (bf16 inputs, GQA groups of a multiple of 4 heads).
//
// Scores S^T = Kbar Q^T run on the MFMA with Kbar split into bf16 hi + lo
// parts (q is exact in bf16; the two products carry ~16 mantissa bits of
// Kbar, so a score is within ~1e-5 relative of the fp32 dot product). Each
// lane then holds 16 block scores of one query row per 32-block tile.
// Top-k: every score becomes an order-preserving 32-bit key whose low
// idx_bits hold (2^idx_bits - 1 - j), so a larger key means a higher score and,
// for equal scores, a lower block index. Dropping the low score bits can only
// reorder scores that agree to better than 2^-(23 - idx_bits) relative. A key
// enters the lane's descending list with one v_med3_u32 per slot (all slots
// computed from the old list); the two half-lists of a row (lanes n and n+32)
// are merged at the end.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kGateChunk = 64;                // candidate blocks per LDS chunk
constexpr int kGatePitch = 2 * kHeadDim + 8;  // bf16 per LDS row: hi | lo | pad (528 B)
constexpr int kGateRows = 64;                 // tokens per workgroup (2 halves x 32)

__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int KMAX>
__device__ __forceinline__ void key_insert(uint32_t (&ts)[KMAX], uint32_t x) {
  uint32_t nt[KMAX];
  nt[0] = max(ts[0], x);
#pragma unroll
  for (int i = 1; i < KMAX; ++i) nt[i] = med3_u32(ts[i - 1], ts[i], x);
#pragma unroll
  for (int i = 0; i < KMAX; ++i) ts[i] = nt[i];
}

__device__ __forceinline__ uint32_t score_key(float s, uint32_t keep, uint32_t low) {
  const uint32_t u = __float_as_uint(s + 0.0f);  // -0 becomes +0
  const uint32_t ordered = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return (ordered & keep) | low;
}

template <int KMAX>
__global__ __launch_bounds__(512) void gate_mfma_kernel(const __bf16 *__restrict__ q,
                                                        const __bf16 *__restrict__ kbar_split,
                                                        const int4 *__restrict__ info, RowHead qs,
                                                        int Hkv, int G, int h0, int Hp, int k,
                                                        int idx_bits, int32_t *__restrict__ idx) {
  const int64_t gb = blockIdx.x;
  const int4 bi = info[gb];
  if (bi.x < 0 || (int)blockIdx.y * kGateRows >= bi.z) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, n = lane & 31, hh = lane >> 5;
  const int hl = blockIdx.z * 4 + (wave & 3);
  const int h = h0 + hl;
  const int g = (h0 + blockIdx.z * 4) / G;  // the 4 heads share one kv head
  const int c = bi.w;
  const int64_t first = gb - c;
  const int pick = k - 1;
  const int r = blockIdx.y * kGateRows + (wave >> 2) * 32 + n;
  const bool active = r < bi.z;
  const int64_t t = bi.y + (active ? r : 0);
  int32_t *dst = idx + (t * Hp + hl) * k;

  if (pick >= c) {  // every earlier block fits: nothing to rank
    if (active && hh == 0) {
      for (int j = 0; j < c; ++j) dst[j] = j;
      dst[c] = c;
      for (int j = c + 1; j < k; ++j) dst[j] = -1;
    }
    return;
  }

  bf16x8 qv[kHeadDim / 16];
  const __bf16 *qrow = q + t * qs.t + h * qs.h + 8 * hh;
#pragma unroll
  for (int kk = 0; kk < kHeadDim / 16; ++kk) qv[kk] = *(const bf16x8 *)(qrow + 16 * kk);

  __shared__ __attribute__((aligned(16))) __bf16 kl[kGateChunk * kGatePitch];
  uint32_t ts[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) ts[i] = 0u;
  const uint32_t maxi = (1u << idx_bits) - 1u, keep = ~maxi;
  const __bf16 *ksrc = kbar_split + (first * Hkv + g) * 2 * kHeadDim;
  const int64_t krow_stride = (int64_t)Hkv * 2 * kHeadDim;

  for (int j0 = 0; j0 < c; j0 += kGateChunk) {
    __syncthreads();  // the previous chunk has been consumed
    for (int x = threadIdx.x; x < kGateChunk * 32; x += 512) {
      const int row = x >> 5, col = x & 31;  // 32 16-byte pieces per row: hi then lo
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j0 + row < c) v = *(const uint4 *)(ksrc + (j0 + row) * krow_stride + col * 8);
      *(uint4 *)(kl + row * kGatePitch + col * 8) = v;
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (j0 + 32 * st >= c) break;
      floatx16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      const __bf16 *ar = kl + (32 * st + n) * kGatePitch + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < kHeadDim / 16; ++kk) {
        const bf16x8 ahi = *(const bf16x8 *)(ar + 16 * kk);
        const bf16x8 alo = *(const bf16x8 *)(ar + kHeadDim + 16 * kk);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, qv[kk], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qv[kk], acc, 0, 0, 0);
      }
      const int jb = j0 + 32 * st + 4 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = jb + 8 * (i >> 2) + (i & 3);  // accumulator i holds block j
        key_insert<KMAX>(ts, j < c ? score_key(acc[i], keep, maxi - (uint32_t)j) : 0u);
      }
    }
  }
  // merge the two half-lists of the row (lanes n and n + 32)
  uint32_t other[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) other[i] = __shfl_xor(ts[i], 32);
#pragma unroll
  for (int i = 0; i < KMAX; ++i) key_insert<KMAX>(ts, other[i]);
  // chosen indices in ascending order (entries past `pick` become sentinels)
  int sel[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) sel[i] = i < pick ? (int)(maxi - (ts[i] & maxi)) : INT_MAX;
#pragma unroll
  for (int pass = 0; pass < KMAX; ++pass)
#pragma unroll
    for (int i = pass & 1; i + 1 < KMAX; i += 2) {
      const int a = sel[i], b = sel[i + 1];
      sel[i] = min(a, b);
      sel[i + 1] = max(a, b);
    }
  if (active && hh == 0) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < pick) dst[i] = sel[i];
    dst[pick] = c;
  }
}

// Bits needed for a local block index (at least 1).
int index_bits(int maxblk) {
  int b = 1;
  while ((1 << b) < maxblk) ++b;
  return b;
}

// ---- Matrix-core gate with the pooled keys resident in LDS.
//
// Same scores, keys and tie rule as gate_mfma_kernel; the workgroup (16 waves)
// covers up to kResRows rows of one block for 4 query heads of one kv head and
// first stages the hi / lo pooled keys of all c earlier blocks into LDS once
// (one 528-byte row per block: hi, lo and 16 bytes of padding, so the 16 rows
// a half-wave reads at one column fall in 16 different bank groups and every
// operand offset is a constant). Each wave then takes (32-row group, head) tasks in turn and
// scores all c candidates of a task with no barrier. The top-k list of each
// lane holds exactly KMAX = k - 1 keys when KMAX is an instantiated size
// (EXACT): the two half-lists of a row (lanes n and n + 32) are then merged
// by one max per slot against the reversed other list, which leaves the KMAX
// largest keys of their union (in bitonic order; only the set matters). The
// own block's padding in the last 32-block chunk is masked only there.
// With bin_count non-NULL the workgroup also counts its choices per block in
// LDS and adds them to the dispatch stage's bin counts (bin p * NBb + global
// block, p the kv head of the pass), so that stage need not read idx twice.
constexpr int kResRows = 512;        // rows per workgroup
constexpr int kResWaves = 16;
constexpr int kResMaxBlocks = 288;   // earlier blocks held in LDS (148.5 KiB)

template <int KMAX, bool EXACT>
__global__ __launch_bounds__(1024, 1) void gate_resident_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kbar_split,
    const int4 *__restrict__ info, int64_t NBb, RowHead qs, int Hkv, int G, int h0, int Hp, int k,
    int idx_bits, int32_t *__restrict__ idx, uint32_t *__restrict__ bin_count) {
  // blocks with the most earlier blocks first
  const int64_t gb = NBb - 1 - (int64_t)blockIdx.x;
  const int4 bi = info[gb];
  const int row0 = (int)blockIdx.y * kResRows;
  if (bi.x < 0 || row0 >= bi.z) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, n = lane & 31, hh = lane >> 5;
  const int c = bi.w;
  const int64_t first = gb - c;
  const int hl0 = (int)blockIdx.z * 4;
  const int g = (h0 + hl0) / G;  // the 4 heads share one kv head
  const int pick = k - 1;
  const int rows = min(kResRows, bi.z - row0);
  const int ntasks = ((rows + 31) >> 5) * 4;
  uint32_t *const bins = bin_count ? bin_count + (int64_t)(hl0 / G) * NBb + first : nullptr;

  if (pick >= c) {  // every earlier block fits: nothing to rank
    if (bins)  // every (row, head) chose every earlier block
      for (int j = threadIdx.x; j < c; j += kResWaves * 64) atomicAdd(&bins[j], 4u * rows);
    for (int task = wave; task < ntasks; task += kResWaves) {
      const int r = row0 + (task >> 2) * 32 + n;
      if (hh || r >= bi.z) continue;
      int32_t *dst = idx + ((int64_t)(bi.y + r) * Hp + hl0 + (task & 3)) * k;
      for (int j = 0; j < c; ++j) dst[j] = j;
      dst[c] = c;
      for (int j = c + 1; j < k; ++j) dst[j] = -1;
    }
    return;
  }

  __shared__ __attribute__((aligned(16))) __bf16 kl[kResMaxBlocks * kGatePitch];
  __shared__ uint32_t hist[kResMaxBlocks];
  for (int j = threadIdx.x; j < c; j += kResWaves * 64) hist[j] = 0;
  {
    const __bf16 *ksrc = kbar_split + (first * Hkv + g) * 2 * kHeadDim;
    const int64_t krow = (int64_t)Hkv * 2 * kHeadDim;
    const int cpad = (c + 31) & ~31;
    for (int x = threadIdx.x; x < cpad * 32; x += kResWaves * 64) {
      const int row = x >> 5, piece = x & 31;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < c) v = *(const uint4 *)(ksrc + row * krow + piece * 8);
      *(uint4 *)(kl + row * kGatePitch + piece * 8) = v;
    }
  }
  __syncthreads();

  // A key's low bits hold maxi - j' with j' = j - 4 hh, which is the same
  // for both lane halves of a chunk position (so it is formed by the scalar
  // unit) and orders each half-list's blocks like j; before the two
  // half-lists meet, the upper half subtracts 4 from its real keys.
  const uint32_t maxi = (1u << idx_bits) - 1u, keep = ~maxi;
  // the query row of a task (this lane's half of it); the next task's row is
  // fetched while the current one is scored
  auto qrow_of = [&](int task) {
    const int r = min(row0 + (task >> 2) * 32 + n, bi.z - 1);
    return q + (bi.y + r) * qs.t + (h0 + hl0 + (task & 3)) * qs.h + 8 * hh;
  };
  bf16x8 qn[kHeadDim / 16];
  {
    const __bf16 *qrow = qrow_of(wave);
#pragma unroll
    for (int kk = 0; kk < kHeadDim / 16; ++kk) qn[kk] = *(const bf16x8 *)(qrow + 16 * kk);
  }
  for (int task = wave; task < ntasks; task += kResWaves) {
    const int hl = hl0 + (task & 3);
    const int r = row0 + (task >> 2) * 32 + n;
    const bool active = r < bi.z;
    const int64_t t = bi.y + (active ? r : 0);
    bf16x8 qv[kHeadDim / 16];
#pragma unroll
    for (int kk = 0; kk < kHeadDim / 16; ++kk) qv[kk] = qn[kk];
    if (task + kResWaves < ntasks) {
      const __bf16 *qrow = qrow_of(task + kResWaves);
#pragma unroll
      for (int kk = 0; kk < kHeadDim / 16; ++kk) qn[kk] = *(const bf16x8 *)(qrow + 16 * kk);
    }
    uint32_t ts[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) ts[i] = 0u;
    for (int j0 = 0; j0 < c; j0 += 32) {
      floatx16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      const __bf16 *ar = kl + (j0 + n) * kGatePitch + 8 * hh;  // this lane's block row
#pragma unroll
      for (int kk = 0; kk < kHeadDim / 16; ++kk) {
        const bf16x8 ahi = *(const bf16x8 *)(ar + 16 * kk);
        const bf16x8 alo = *(const bf16x8 *)(ar + kHeadDim + 16 * kk);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, qv[kk], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qv[kk], acc, 0, 0, 0);
      }
      const uint32_t lb = maxi - (uint32_t)j0;
      if (j0 + 32 <= c) {
#pragma unroll
        for (int i = 0; i < 16; ++i)  // accumulator i holds block j0 + 8(i/4) + 4hh + i%4
          key_insert<KMAX>(ts, score_key(acc[i], keep, lb - (uint32_t)(8 * (i >> 2) + (i & 3))));
      } else {
        const int jb = j0 + 4 * hh;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = jb + 8 * (i >> 2) + (i & 3);
          key_insert<KMAX>(ts, j < c ? score_key(acc[i], keep,
                                                 lb - (uint32_t)(8 * (i >> 2) + (i & 3)))
                                     : 0u);
        }
      }
    }
    // the row's two half-lists (lanes n and n + 32); empty entries stay 0
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (hh) ts[i] = ts[i] ? ts[i] - 4u : 0u;
    uint32_t other[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) other[i] = __shfl_xor(ts[i], 32);
    if constexpr (EXACT) {
#pragma unroll
      for (int i = 0; i < KMAX; ++i) ts[i] = max(ts[i], other[KMAX - 1 - i]);
    } else {
#pragma unroll
      for (int i = 0; i < KMAX; ++i) key_insert<KMAX>(ts, other[i]);
    }
    // chosen indices in ascending order (entries past `pick` become sentinels;
    // with EXACT every entry is chosen)
    int sel[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) sel[i] = i < pick ? (int)(maxi - (ts[i] & maxi)) : INT_MAX;
#pragma unroll
    for (int pass = 0; pass < KMAX; ++pass)
#pragma unroll
      for (int i = pass & 1; i + 1 < KMAX; i += 2) {
        const int a = sel[i], b = sel[i + 1];
        sel[i] = min(a, b);
        sel[i + 1] = max(a, b);
      }
    if (active && hh == 0) {
      int32_t *dst = idx + (t * Hp + hl) * k;
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i < pick) {
          dst[i] = sel[i];
          if (bins) atomicAdd(&hist[sel[i]], 1u);
        }
      dst[pick] = c;
    }
  }
  if (bins) {
    __syncthreads();
    for (int j = threadIdx.x; j < c; j += kResWaves * 64)
      if (hist[j]) atomicAdd(&bins[j], hist[j]);
  }
}


// Whether the matrix-core gate keeps every earlier block in LDS (then it also
// counts the dispatch bins).
bool gate_resident(const Problem &pb) {
  // every earlier block fits in LDS, and lists of up to 16 keys fit the
  // registers of 16 waves
  return pb.bf16 && pb.G % 4 == 0 && index_bits(pb.maxblk) <= 12 &&
         pb.maxblk - 1 <= kResMaxBlocks && pb.k - 1 <= 16;
}

hipError_t launch_gate_mfma(const Problem &pb, const Work &w, const __bf16 *q, int g0,
                            hipStream_t s, int bits, uint32_t *bin_count) {
  const int h0 = g0 * pb.G;
  const int pick = pb.k - 1;
  if (gate_resident(pb)) {
    dim3 grid((unsigned)pb.NBb, (unsigned)((pb.B + kResRows - 1) / kResRows), (unsigned)(pb.Hp / 4));
#define MOBA_GATE_RES(KM, EX)                                                                   \
  gate_resident_kernel<KM, EX><<<grid, kResWaves * 64, 0, s>>>(                                \
      q, w.kbar_split, w.blk_info, pb.NBb, pb.qs, pb.Hkv, pb.G, h0, pb.Hp, pb.k, bits, w.idx,   \
      bin_count)
    switch (pick) {
      case 1: MOBA_GATE_RES(1, true); break;
      case 2: MOBA_GATE_RES(2, true); break;
      case 3: MOBA_GATE_RES(3, true); break;
      case 4: MOBA_GATE_RES(4, true); break;
      case 5: MOBA_GATE_RES(5, true); break;
      case 6: MOBA_GATE_RES(6, true); break;
      case 7: MOBA_GATE_RES(7, true); break;
      case 8: MOBA_GATE_RES(8, true); break;
      case 11: MOBA_GATE_RES(11, true); break;
      case 12: MOBA_GATE_RES(12, true); break;
      case 15: MOBA_GATE_RES(15, true); break;
      case 16: MOBA_GATE_RES(16, true); break;
      default:
        if (pick <= 0) MOBA_GATE_RES(1, true);  // topk 1: select-all path only
        else if (pick <= 12) MOBA_GATE_RES(12, false);
        else MOBA_GATE_RES(16, false);
    }
#undef MOBA_GATE_RES
    return hipGetLastError();
  }
  dim3 grid((unsigned)pb.NBb, (unsigned)((pb.B + kGateRows - 1) / kGateRows), (unsigned)(pb.Hp / 4));
#define MOBA_GATE_MFMA(KM)                                                                       \
  gate_mfma_kernel<KM><<<grid, 512, 0, s>>>(q, w.kbar_split, w.blk_info, pb.qs, pb.Hkv, pb.G, h0, \
                                            pb.Hp, pb.k, bits, w.idx)
  if (pick <= 4) MOBA_GATE_MFMA(4);
  else if (pick <= 8) MOBA_GATE_MFMA(8);
  else if (pick <= 12) MOBA_GATE_MFMA(12);
  else if (pick <= 16) MOBA_GATE_MFMA(16);
  else if (pick <= 24) MOBA_GATE_MFMA(24);
  else if (pick <= kMaxHistPick) MOBA_GATE_MFMA(kMaxHistPick);
  else MOBA_GATE_MFMA(4);  // only with the select-all path
#undef MOBA_GATE_MFMA
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gate_t(const Problem &pb, const Work &w, const T *q, int g0, hipStream_t s) {
  dim3 grid((unsigned)pb.NBb, (unsigned)((pb.B + kGateTokens - 1) / kGateTokens),
            (unsigned)((pb.Hp + 3) / 4));
  const int h0 = g0 * pb.G;
  const int pick = pb.k - 1;
  if (pick <= 4)
    gate_kernel<T, 4><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.qs, pb.Hkv, pb.G, h0, pb.Hp,
                                           pb.k, w.idx);
  else if (pick <= 8)
    gate_kernel<T, 8><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.qs, pb.Hkv, pb.G, h0, pb.Hp,
                                           pb.k, w.idx);
  else if (pick <= 16)
    gate_kernel<T, 16><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.qs, pb.Hkv, pb.G, h0, pb.Hp,
                                            pb.k, w.idx);
  else if (pick <= kMaxHistPick)
    gate_kernel<T, kMaxHistPick><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.qs, pb.Hkv, pb.G,
                                                      h0, pb.Hp, pb.k, w.idx);
  else  // only reached when every sequence has at most topk blocks (select-all path)
    gate_kernel<T, 4><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.qs, pb.Hkv, pb.G, h0, pb.Hp,
                                           pb.k, w.idx);
  return hipGetLastError();
}

}  // namespace

// ---- Fixed gates (MoBA summary page, section 3.4 "Context Partitioning": a
// sliding window is a gate that always picks the most recent blocks, an
// attention sink one that picks the initial and the recent blocks). Slots of
// (row, query head): the n_sink initial blocks and the k - n_sink most recent
// blocks up to the own block, ascending; rows with at most k blocks so far
// take all of them. Every head gets the same selection.
__global__ __launch_bounds__(256) void gate_window_kernel(const int32_t *__restrict__ cu, int S,
                                                          int64_t T, int B, int Hp, int k,
                                                          int n_sink,
                                                          const int32_t *__restrict__ status,
                                                          int32_t *__restrict__ idx) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (t, hl)
  if (row >= T * Hp || *status != 0) return;
  const int64_t t = row / Hp;
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int c = (int)((t - cu[lo]) / B);
  const int w = k - n_sink;
  int32_t *dst = idx + row * k;
  int n = 0;
  const int s_end = min(n_sink, c + 1);       // sink blocks 0 .. s_end-1
  for (int j = 0; j < s_end; ++j) dst[n++] = j;
  for (int j = max(s_end, c - w + 1); j <= c; ++j) dst[n++] = j;  // recent blocks
  for (; n < k; ++n) dst[n] = -1;
}

// ---- Pooled-key gate (MoBA review page, authors' rebuttals on mean pooling
// and on QUEST): on top of the mean-pooled top-k, the best blocks by
// max-pooled and by min-pooled keys are selected too. The three rankings run
// through the ordinary gate kernels (same scores, order and tie rule) into
// scratch lists; this kernel forms their union per (row, query head) in the
// k slots: earlier blocks ascending, -1 for slots left empty by coinciding
// picks (their partial lse is set to -inf so the merge skips them), the own
// block at position min(k, c + 1) - 1, then -1.
__global__ __launch_bounds__(256) void gate_union_kernel(
    const int32_t *__restrict__ lm, int km, const int32_t *__restrict__ lx, int kx,
    const int32_t *__restrict__ ln, int kn, const int32_t *__restrict__ cu, int S, int64_t T,
    int B, int Hp, int k, const int32_t *__restrict__ status, int32_t *__restrict__ idx,
    float *__restrict__ part_lse) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= T * Hp || *status != 0) return;
  const int64_t t = row / Hp;
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int c = (int)((t - cu[lo]) / B);
  const int32_t *a = lm + row * km, *b = lx + row * kx, *d = ln + row * kn;
  int ia = 0, ib = 0, id = 0;
  const int nsel = min(k, c + 1);
  int32_t *dst = idx + row * k;
  float *pl = part_lse + row * k;
  int n = 0;
  // three ascending lists of earlier blocks (each ends at its own-block entry
  // or a -1): merge without duplicates
  for (;;) {
    const int va = ia < km && a[ia] >= 0 && a[ia] < c ? a[ia] : INT_MAX;
    const int vb = ib < kx && b[ib] >= 0 && b[ib] < c ? b[ib] : INT_MAX;
    const int vd = id < kn && d[id] >= 0 && d[id] < c ? d[id] : INT_MAX;
    const int v = min(va, min(vb, vd));
    if (v == INT_MAX || n >= nsel - 1) break;
    dst[n++] = v;
    ia += va == v; ib += vb == v; id += vd == v;
  }
  for (; n < nsel - 1; ++n) { dst[n] = -1; pl[n] = -INFINITY; }
  dst[n++] = c;
  for (; n < k; ++n) dst[n] = -1;
}

hipError_t launch_gate_window(const Problem &pb, const Work &w, int n_sink, hipStream_t s) {
  const int64_t rows = pb.T * pb.Hp;
  if (rows == 0) return hipSuccess;
  hipError_t e = launch_fill_u32(w.counted, 0u, 1, s);  // the dispatch counts
  if (e != hipSuccess) return e;
  gate_window_kernel<<<dim3((unsigned)((rows + 255) / 256)), 256, 0, s>>>(
      w.cu, pb.S, pb.T, pb.B, pb.Hp, pb.k, n_sink, w.status, w.idx);
  return hipGetLastError();
}

hipError_t launch_gate_impl(const Problem &pb, const Work &w, const void *q, int g0, hipStream_t s,
                            bool count);

hipError_t launch_gate_pooled(const Problem &pb, const Work &w, const void *q, int g0,
                              int extra_max, int extra_min, hipStream_t s) {
  const int64_t rows = pb.T * pb.Hp;
  if (rows == 0) return hipSuccess;
  hipError_t e0 = launch_fill_u32(w.counted, 0u, 1, s);  // the dispatch counts the union
  if (e0 != hipSuccess) return e0;
  // scratch lists in the partial-output region (unused until the attention);
  // a ranking with nothing to pick gets no list (length 0)
  const int pm = pb.k - extra_max - extra_min - 1;
  const int km = pm > 0 ? pm + 1 : 0, kx = extra_max > 0 ? extra_max + 1 : 0,
            kn = extra_min > 0 ? extra_min + 1 : 0;
  int32_t *lm = (int32_t *)w.part_o, *lx = lm + rows * km, *ln = lx + rows * kx;
  struct Ranking { float *f; __bf16 *split; int32_t *list; int k; };
  const Ranking rk[3] = {{w.kbar, w.kbar_split, lm, km}, {w.kmax, w.kmax_split, lx, kx},
                         {w.kmin, w.kmin_split, ln, kn}};
  for (const Ranking &r : rk) {
    if (r.k == 0) continue;
    Problem p2 = pb;
    p2.k = r.k;
    Work w2 = w;
    w2.kbar = r.f;
    w2.kbar_split = r.split;
    w2.idx = r.list;
    hipError_t e = launch_gate_impl(p2, w2, q, g0, s, false);
    if (e != hipSuccess) return e;
  }
  gate_union_kernel<<<dim3((unsigned)((rows + 255) / 256)), 256, 0, s>>>(
      lm, km, lx, kx, ln, kn, w.cu, pb.S, pb.T, pb.B, pb.Hp, pb.k, w.status, w.idx, w.part_lse);
  return hipGetLastError();
}

// Mean gate; with `count` the matrix-core kernel that keeps the pooled keys
// resident also fills the dispatch bin counts and marks them counted.
hipError_t launch_gate_impl(const Problem &pb, const Work &w, const void *q, int g0, hipStream_t s,
                            bool count) {
  // matrix-core gate: bf16, groups of a multiple of 4 heads, at most 4096
  // blocks per sequence (12 index bits keep 20 score bits in the keys)
  const int bits = index_bits(pb.maxblk);
  const bool counts = count && gate_resident(pb);
  hipError_t e = launch_fill_u32(w.counted, counts ? 1u : 0u, 1, s);
  if (e != hipSuccess) return e;
  if (counts && (e = launch_fill_u32(w.bin_count, 0u, (int64_t)pb.P * pb.NBb, s)) != hipSuccess)
    return e;
  if (pb.bf16 && pb.G % 4 == 0 && bits <= 12)
    return launch_gate_mfma(pb, w, (const __bf16 *)q, g0, s, bits,
                            counts ? w.bin_count : nullptr);
  return pb.bf16 ? launch_gate_t<__bf16>(pb, w, (const __bf16 *)q, g0, s)
                 : launch_gate_t<float>(pb, w, (const float *)q, g0, s);
}

hipError_t launch_gate(const Problem &pb, const Work &w, const void *q, int g0, hipStream_t s) {
  return launch_gate_impl(pb, w, q, g0, s, true);
}

}  // namespace moba
