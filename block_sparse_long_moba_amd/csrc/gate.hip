// Gate: parameter-free top-k block selection per query head.
//
// MoBA summary page (paper-graph-ui), section 3.4: "Affinity Scoring"
// (s_j = <q, mean-pooled keys of block j>, no scaling), "Top-k Gating" (keep
// the k best; the query's own block is always kept and, in the reading used
// here, counts toward k), "Causality Enforcement" mechanism 1 (later blocks
// are never candidates). Review page (paperhub.cn), authors' rebuttal W1:
// each query head selects on its own.
//
// One workgroup = 64 consecutive rows of one block x 4 query heads (one wave
// per head, one lane per row). Every row of the workgroup has the same own
// block c, so the candidate list 0..c-1 is uniform across the workgroup and
// the pooled-key rows are wave-uniform reads. Scores are fp32 dot products
// (q upcast exactly from bf16, kbar fp32), so a selection can differ from an
// exact one only where the k-th and (k+1)-th scores agree to ~1e-6.
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
                                                   const int4 *__restrict__ info, int Hq,
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
  load_row_f32<T>(q + (t * Hq + h) * kHeadDim, qf);
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

template <typename T>
hipError_t launch_gate_t(const Problem &pb, const Work &w, const T *q, int g0, hipStream_t s) {
  dim3 grid((unsigned)pb.NBb, (unsigned)((pb.B + kGateTokens - 1) / kGateTokens),
            (unsigned)((pb.Hp + 3) / 4));
  const int h0 = g0 * pb.G;
  const int pick = pb.k - 1;
  if (pick <= 4)
    gate_kernel<T, 4><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.Hq, pb.Hkv, pb.G, h0, pb.Hp,
                                           pb.k, w.idx);
  else if (pick <= 8)
    gate_kernel<T, 8><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.Hq, pb.Hkv, pb.G, h0, pb.Hp,
                                           pb.k, w.idx);
  else if (pick <= 16)
    gate_kernel<T, 16><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.Hq, pb.Hkv, pb.G, h0, pb.Hp,
                                            pb.k, w.idx);
  else if (pick <= kMaxHistPick)
    gate_kernel<T, kMaxHistPick><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.Hq, pb.Hkv, pb.G,
                                                      h0, pb.Hp, pb.k, w.idx);
  else  // only reached when every sequence has at most topk blocks (select-all path)
    gate_kernel<T, 4><<<grid, 256, 0, s>>>(q, w.kbar, w.blk_info, pb.Hq, pb.Hkv, pb.G, h0, pb.Hp,
                                           pb.k, w.idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate(const Problem &pb, const Work &w, const void *q, int g0, hipStream_t s) {
  return pb.bf16 ? launch_gate_t<__bf16>(pb, w, (const __bf16 *)q, g0, s)
                 : launch_gate_t<float>(pb, w, (const float *)q, g0, s);
}

}  // namespace moba
