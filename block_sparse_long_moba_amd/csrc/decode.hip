// Decode-phase MoBA: one new query per sequence over its KV cache.
//
// MoBA summary page (paper-graph-ui), section 3.4: the gate ("Affinity
// Scoring", "Top-k Gating", "Causality Enforcement") and the block attention
// apply unchanged to a single query; the review page's GSM-Infinite table
// reports the "MoBA prefill, MoBA decode" configuration. The query of
// sequence s is the token at its last cache row L_s - 1, so its own block c
// is the cache's last (possibly partial) block, attended up to that row; the
// pooled keys of the earlier blocks come from the cache (moba_meanpool).
//
// Three kernels: the gate ranks a query's candidates by counting (exactly the
// (score desc, index asc) order of the prefill gate), the attention runs one
// workgroup per (sequence, kv head, block) for every query head of the group
// that chose the block (the block's keys and values are read once for all of
// them), and the merge combines the per-block parts by log-sum-exp.
#include <limits.h>

#include <algorithm>
#include <type_traits>

#include "moba_internal.h"

namespace moba {
namespace {

constexpr float kLog2eDec = 1.4426950408889634f;
constexpr float kLn2Dec = 0.6931471805599453f;
constexpr int kDecKeyLanes = 16;                 // lanes per key row (8 dims each)
constexpr int kDecGroups = 256 / kDecKeyLanes;   // key groups per workgroup
constexpr int kDecWaves = 4;                     // waves per workgroup

template <typename T> struct Row8;
template <> struct Row8<__bf16> {
  using Raw = uint4;  // the 8 elements as loaded (half the registers of floats)
  __device__ static Raw load_raw(const __bf16 *p) { return *(const uint4 *)p; }
  __device__ static void unpack(const Raw &u, float *f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void load(const __bf16 *p, float *f) { unpack(load_raw(p), f); }
  __device__ static void store(__bf16 *p, const float *f) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)f[i];
    *(bf16x8 *)p = v;
  }
};
template <> struct Row8<float> {
  struct Raw { float4 a, b; };
  __device__ static Raw load_raw(const float *p) {
    return Raw{((const float4 *)p)[0], ((const float4 *)p)[1]};
  }
  __device__ static void unpack(const Raw &r, float *f) {
    f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
    f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
  }
  __device__ static void load(const float *p, float *f) { unpack(load_raw(p), f); }
  __device__ static void store(float *p, const float *f) {
    ((float4 *)p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    ((float4 *)p)[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
};

// Gate: one workgroup per (sequence, query head). Scores <q, kbar_j> of the
// earlier blocks j < c in fp32 (the prefill vector gate's arithmetic); block j
// is picked iff fewer than min(k-1, c) candidates rank above it under
// (score desc, index asc); picks are written ascending, then the own block c,
// then -1. A sequence with an empty cache gets -1 everywhere.
template <typename T>
__global__ __launch_bounds__(256) void decode_gate_kernel(const T *__restrict__ q,
                                                          const float *__restrict__ kbar,
                                                          const int32_t *__restrict__ cu,
                                                          const int32_t *__restrict__ blk_first,
                                                          int Hq, int Hkv, int B, int k,
                                                          const int32_t *__restrict__ status,
                                                          int32_t *__restrict__ idx) {
  if (*status != 0) return;  // the table check failed: the merge writes NaN
  const int s = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int L = cu[s + 1] - cu[s];
  int32_t *dst = idx + ((int64_t)s * Hq + h) * k;
  if (L == 0) {
    for (int i = tid; i < k; i += 256) dst[i] = -1;
    return;
  }
  const int c = (L - 1) / B;
  const int pick = min(k - 1, c);
  const int g = h / (Hq / Hkv);
  __shared__ float qs[kHeadDim];
  __shared__ float sc[kLdsBins];
  __shared__ int wcnt[4];
  if (tid < kHeadDim) {
    float f[8];
    if ((tid & 7) == 0) {
      Row8<T>::load(q + ((int64_t)s * Hq + h) * kHeadDim + tid, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) qs[tid + i] = f[i];
    }
  }
  __syncthreads();
  // scores: 16 lanes per block (8 dimensions each, a coalesced 512-byte row),
  // 128 blocks per round
  const float *kb0 = kbar + ((int64_t)blk_first[s] * Hkv + g) * kHeadDim;
  const int64_t kstride = (int64_t)Hkv * kHeadDim;
  const int sub = tid & 15, grp = tid >> 4;
  float qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = qs[8 * sub + i];
  for (int j0 = 0; j0 < c; j0 += 128) {
    float dsum[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + 16 * u + grp, c - 1);
      const float4 x0 = *(const float4 *)(kb0 + j * kstride + 8 * sub);
      const float4 x1 = *(const float4 *)(kb0 + j * kstride + 8 * sub + 4);
      dsum[u] = ((qv[0] * x0.x + qv[1] * x0.y) + (qv[2] * x0.z + qv[3] * x0.w)) +
                ((qv[4] * x1.x + qv[5] * x1.y) + (qv[6] * x1.z + qv[7] * x1.w));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float v = dsum[u];
      v += __shfl_xor(v, 8, 16);
      v += __shfl_xor(v, 4, 16);
      v += __shfl_xor(v, 2, 16);
      v += __shfl_xor(v, 1, 16);
      const int j = j0 + 16 * u + grp;
      if (sub == 0 && j < c) sc[j] = v;
    }
  }
  __syncthreads();
  // block j is chosen iff fewer than pick candidates rank above it; the
  // chosen blocks are written in ascending order (positions by ballot)
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int base = 0;
  for (int j0 = 0; j0 < c; j0 += 256) {
    const int j = j0 + tid;
    bool f = false;
    if (j < c) {
      const float sj = sc[j];
      int rank = 0;
      for (int i = 0; i < c; ++i) {
        const float si = sc[i];
        rank += (si > sj) || (si == sj && i < j);
      }
      f = rank < pick;
    }
    const uint64_t m = __ballot(f);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wcnt[w];
    if (f) dst[off + __popcll(m & below)] = j;
    base += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();
  }
  if (tid == 0) {
    dst[pick] = c;
    for (int i = pick + 1; i < k; ++i) dst[i] = -1;
  }
}

// Sum over each row of 16 lanes by DPP (in-register lane exchange): pairs,
// quads, then the two quads of each half (mirror within 8) and the two halves
// (mirror within 16). Each step adds two equal-valued operands in either
// order, so every lane of the row ends with the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                      0xf, 0xf, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror: the other quad
  x += dpp(x, std::integral_constant<int, 0x140>{});  // row_mirror: the other half row
  return x;
}

// Attention: one workgroup per (sequence, kv head g, block j <= c). 16 lanes
// cover one key row (8 dims each, 256 contiguous bytes); 16 key groups walk
// the block's rows (the own block up to the query's row) with an online
// softmax per group, combined at the end through LDS. Writes the part of
// slot (s, h, position of j in h's selection): o (fp32) and lse.
// MH: query heads per sweep over the block (registers hold q and the output
// accumulators of MH heads; 4 covers the 8B head shape's groups in one sweep)
template <typename T, int MH>
__global__ __launch_bounds__(256) void decode_attn_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ idx, int Hq, int Hkv, int B,
    int k, int ns, float scale_log2, const int32_t *__restrict__ status,
    float *__restrict__ part_o, float *__restrict__ part_lse) {
  if (*status != 0) return;
  const int s = blockIdx.x, g = blockIdx.y, j = blockIdx.z / ns, sp = blockIdx.z % ns;
  const int tid = threadIdx.x;
  const int L = cu[s + 1] - cu[s];
  if (L == 0 || j > (L - 1) / B) return;
  const int G = Hq / Hkv;
  // query heads of the group that chose block j, in head order, with the
  // slot of j in their selection (a head lists a block at most once): the
  // first wave tests the G*k entries 64 at a time and compacts the matches
  __shared__ int heads[64], slots[64], nheads;
  if (tid < 64) {
    const int32_t *rows = idx + ((int64_t)s * Hq + g * G) * k;  // G rows of k, contiguous
    int n = 0;
    for (int base = 0; base < G * k && n < 64; base += 64) {
      const int e = base + tid;
      const bool hit = e < G * k && rows[e] == j;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(hit);
      const int pos = n + __builtin_popcountll(mask & ((1ull << tid) - 1ull));
      if (hit && pos < 64) {
        heads[pos] = g * G + e / k;
        slots[pos] = e % k;
      }
      n += __builtin_popcountll(mask);
    }
    if (tid == 0) nheads = min(n, 64);
  }
  __syncthreads();
  const int nh = nheads;
  if (nh == 0) return;
  const int li = tid % kDecKeyLanes, kg = tid / kDecKeyLanes;
  // keys [k0, k1) of the block: split sp of ns (the own block may end early;
  // an empty split still writes its part, with lse -inf)
  const int chunk = B / ns;
  const int k0 = sp * chunk, k1 = min(min(B, L - j * B), k0 + chunk);
  const int nk = max(0, k1 - k0);
  const int64_t r0 = cu[s] + (int64_t)j * B + k0;
  const int64_t kstride = (int64_t)Hkv * kHeadDim;
  const T *kb = kc + (r0 * Hkv + g) * kHeadDim + 8 * li;
  const T *vb = vc + (r0 * Hkv + g) * kHeadDim + 8 * li;
  // per-wave states (the 4 key groups of a wave are merged with shuffles
  // first), combined across the 4 waves through LDS
  __shared__ float gm[kDecWaves][MH], gl[kDecWaves][MH];
  __shared__ float gacc[kDecWaves][MH][kHeadDim];
  const int wv = tid >> 6;
  for (int h0 = 0; h0 < nh; h0 += MH) {
    const int nq = min(MH, nh - h0);
    float qv[MH][8], m[MH], l[MH], acc[MH][8];
#pragma unroll
    for (int qi = 0; qi < MH; ++qi) {
      m[qi] = -INFINITY;
      l[qi] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[qi][e] = 0.f;
      if (qi < nq) {
        Row8<T>::load(q + ((int64_t)s * Hq + heads[h0 + qi]) * kHeadDim + 8 * li, qv[qi]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[qi][e] *= scale_log2;  // scores in log2 units
      }
    }
    // one online-softmax update per group of NU keys: their scores, one
    // maximum, one rescale of the state, then the NU weighted values (rows
    // are unpacked from their loaded form one at a time)
    using Raw = typename Row8<T>::Raw;
    auto consume = [&](auto nu_c, const Raw *kr, const Raw *vr) {
      constexpr int NU = decltype(nu_c)::value;
#pragma unroll
      for (int qi = 0; qi < MH; ++qi) {
        if (qi >= nq) break;
        float d[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          float kf[8];
          Row8<T>::unpack(kr[u], kf);
          float x = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) x = fmaf(qv[qi][e], kf[e], x);
          d[u] = row16_sum(x);
        }
        float mn = m[qi];
#pragma unroll
        for (int u = 0; u < NU; ++u) mn = fmaxf(mn, d[u]);
        const float alpha = __builtin_amdgcn_exp2f(m[qi] - mn);
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qi][e] *= alpha;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const float p = __builtin_amdgcn_exp2f(d[u] - mn);
          ps += p;
          float vf[8];
          Row8<T>::unpack(vr[u], vf);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[qi][e] = fmaf(p, vf[e], acc[qi][e]);
        }
        l[qi] = fmaf(l[qi], alpha, ps);
        m[qi] = mn;
      }
    };
    // four rows per group in flight, then the rest one by one
    constexpr int U = 4;
    int key = kg;
    for (; key + (U - 1) * kDecGroups < nk; key += U * kDecGroups) {
      Raw kr[U], vr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kr[u] = Row8<T>::load_raw(kb + (int64_t)(key + u * kDecGroups) * kstride);
        vr[u] = Row8<T>::load_raw(vb + (int64_t)(key + u * kDecGroups) * kstride);
      }
      consume(std::integral_constant<int, U>{}, kr, vr);
    }
    for (; key < nk; key += kDecGroups) {
      const Raw kr = Row8<T>::load_raw(kb + (int64_t)key * kstride);
      const Raw vr = Row8<T>::load_raw(vb + (int64_t)key * kstride);
      consume(std::integral_constant<int, 1>{}, &kr, &vr);
    }
#pragma unroll
    for (int qi = 0; qi < MH; ++qi) {
      if (qi >= nq) break;
      // merge the online-softmax states of lanes li, li+16, li+32, li+48
#pragma unroll
      for (int o = kDecKeyLanes; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(m[qi], o), l2 = __shfl_xor(l[qi], o);
        const float M = fmaxf(m[qi], m2);
        const float a1 = m[qi] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[qi] - M);
        const float a2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
        l[qi] = l[qi] * a1 + l2 * a2;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qi][e] = acc[qi][e] * a1 + __shfl_xor(acc[qi][e], o) * a2;
        m[qi] = M;
      }
      if ((tid & 63) < kDecKeyLanes) {
#pragma unroll
        for (int e = 0; e < 8; ++e) gacc[wv][qi][8 * li + e] = acc[qi][e];
        if (li == 0) { gm[wv][qi] = m[qi]; gl[wv][qi] = l[qi]; }
      }
    }
    __syncthreads();
    for (int x = tid; x < nq * kHeadDim; x += 256) {
      const int qi = x / kHeadDim, e = x % kHeadDim;
      float M = -INFINITY;
      for (int gi = 0; gi < kDecWaves; ++gi) M = fmaxf(M, gm[gi][qi]);
      float Ls = 0.f, o = 0.f;
      for (int gi = 0; gi < kDecWaves; ++gi) {
        const float wgt = gm[gi][qi] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(gm[gi][qi] - M);
        Ls += gl[gi][qi] * wgt;
        o += gacc[gi][qi][e] * wgt;
      }
      const int64_t sl = (((int64_t)s * Hq + heads[h0 + qi]) * k + slots[h0 + qi]) * ns + sp;
      part_o[sl * kHeadDim + e] = M == -INFINITY ? 0.f : o / Ls;
      if (e == 0) part_lse[sl] = M == -INFINITY ? -INFINITY : (M + __log2f(Ls)) * kLn2Dec;
    }
    __syncthreads();
  }
}

// Merge: one workgroup of 256 threads per (sequence, query head): the
// log-sum-exp combination of its min(k, c+1) parts in ascending block order.
// The part lse values are reduced by all threads; wave w adds the rows of
// parts w, w + 4, ... (two elements per lane, eight rows in flight), and the
// four waves' sums are added in wave order.
template <typename T>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float *__restrict__ part_o,
                                                           const float *__restrict__ part_lse,
                                                           const int32_t *__restrict__ cu,
                                                           int S, int Hq, int B, int k, int ns,
                                                           const int32_t *__restrict__ status,
                                                           T *__restrict__ out,
                                                           float *__restrict__ lse) {
  const int s = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  T *dst = out + ((int64_t)s * Hq + h) * kHeadDim;
  if (*status != 0) {  // bad cu_seqlens or an understated block bound
    if (tid < kHeadDim) dst[tid] = (T)NAN;
    if (tid == 0 && lse) lse[(int64_t)h * S + s] = NAN;
    return;
  }
  const int L = cu[s + 1] - cu[s];
  if (L == 0) {
    if (tid < kHeadDim) dst[tid] = (T)0.f;
    if (tid == 0 && lse) lse[(int64_t)h * S + s] = -INFINITY;
    return;
  }
  __shared__ float red[4];
  __shared__ float2 wsum[4][kHeadDim / 2];
  const int n = min(k, (L - 1) / B + 1) * ns;  // parts of the selected blocks, in block order
  const int64_t base = ((int64_t)s * Hq + h) * k * ns;
  const float *pl = part_lse + base;
  float M = -INFINITY;
  for (int i = tid; i < n; i += 256) M = fmaxf(M, pl[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int i = tid; i < n; i += 256)
    if (pl[i] > -INFINITY) sum += __builtin_amdgcn_exp2f((pl[i] - M) * kLog2eDec);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  sum = (red[0] + red[1]) + (red[2] + red[3]);
  const float Lt = M + __logf(sum);
  // part rows (written for every part, empty ones too) loaded unconditionally
  float2 o = make_float2(0.f, 0.f);
  for (int i0 = wave; i0 < n; i0 += 32) {
    float2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + 4 * u, n - 1);
      x[u] = *(const float2 *)(part_o + (base + i) * kHeadDim + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + 4 * u;
      if (i < n && pl[i] > -INFINITY) {
        const float wt = __builtin_amdgcn_exp2f((pl[i] - Lt) * kLog2eDec);
        o.x += wt * x[u].x;
        o.y += wt * x[u].y;
      }
    }
  }
  wsum[wave][lane] = o;
  __syncthreads();
  if (tid < kHeadDim / 2) {
    float2 r = wsum[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) { r.x += wsum[w][tid].x; r.y += wsum[w][tid].y; }
    dst[2 * tid] = (T)r.x;
    dst[2 * tid + 1] = (T)r.y;
  }
  if (tid == 0 && lse) lse[(int64_t)h * S + s] = Lt;
}

}  // namespace

int decode_splits(int S, int Hq, int Hkv, int B, int k, int maxblk) {
  // split a block's keys over several workgroups while the (sequence, kv
  // head, chosen block) items are too few to keep the memory system busy
  const int64_t items = (int64_t)S * Hkv * std::min<int64_t>(maxblk, (int64_t)(Hq / Hkv) * k);
  int ns = 1;
  while (ns < 8 && items * ns < 2048 && B % (2 * ns * kDecGroups) == 0) ns *= 2;
  return ns;
}

hipError_t launch_decode(const Problem &pb, const Work &w, const void *q, const void *kc,
                         const void *vc, void *out, float *lse, hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  const int ns = decode_splits(pb.S, pb.Hq, pb.Hkv, pb.B, pb.k, pb.maxblk);
  const dim3 gg((unsigned)pb.S, (unsigned)pb.Hq);
  const dim3 ga((unsigned)pb.S, (unsigned)pb.Hkv, (unsigned)(pb.maxblk * ns));
  float *po = (float *)w.part_o;
  const float sl2 = pb.scale * kLog2eDec;
  if (pb.bf16) {
    decode_gate_kernel<__bf16><<<gg, 256, 0, s>>>((const __bf16 *)q, w.kbar, w.cu, w.blk_first,
                                                  pb.Hq, pb.Hkv, pb.B, pb.k, w.status, w.idx);
    if (pb.G <= 4)
      decode_attn_kernel<__bf16, 4><<<ga, 256, 0, s>>>((const __bf16 *)q, (const __bf16 *)kc,
                                                       (const __bf16 *)vc, w.cu, w.idx, pb.Hq,
                                                       pb.Hkv, pb.B, pb.k, ns, sl2, w.status, po, w.part_lse);
    else
      decode_attn_kernel<__bf16, 8><<<ga, 256, 0, s>>>((const __bf16 *)q, (const __bf16 *)kc,
                                                       (const __bf16 *)vc, w.cu, w.idx, pb.Hq,
                                                       pb.Hkv, pb.B, pb.k, ns, sl2, w.status, po, w.part_lse);
    decode_merge_kernel<__bf16><<<gg, 256, 0, s>>>(po, w.part_lse, w.cu, pb.S, pb.Hq, pb.B, pb.k,
                                                   ns, w.status, (__bf16 *)out, lse);
  } else {
    decode_gate_kernel<float><<<gg, 256, 0, s>>>((const float *)q, w.kbar, w.cu, w.blk_first,
                                                 pb.Hq, pb.Hkv, pb.B, pb.k, w.status, w.idx);
    if (pb.G <= 4)
      decode_attn_kernel<float, 4><<<ga, 256, 0, s>>>((const float *)q, (const float *)kc,
                                                      (const float *)vc, w.cu, w.idx, pb.Hq,
                                                      pb.Hkv, pb.B, pb.k, ns, sl2, w.status, po, w.part_lse);
    else
      decode_attn_kernel<float, 8><<<ga, 256, 0, s>>>((const float *)q, (const float *)kc,
                                                      (const float *)vc, w.cu, w.idx, pb.Hq,
                                                      pb.Hkv, pb.B, pb.k, ns, sl2, w.status, po, w.part_lse);
    decode_merge_kernel<float><<<gg, 256, 0, s>>>(po, w.part_lse, w.cu, pb.S, pb.Hq, pb.B, pb.k,
                                                  ns, w.status, (float *)out, lse);
  }
  return hipGetLastError();
}

}  // namespace moba
