// Backward pass of the block-sparse attention on the matrix cores (bf16).
//
// MoBA summary page (paper-graph-ui), section 3.4: every query attends, with
// one softmax, over the union of its own block (causally) and the earlier
// blocks its gate chose. The choice is discrete, so gradients reach q, k and v
// through that attention only and the gate receives none. With
// P = softmax(scale q K^T) over the union, O = P V and D = <dO, O> per
// (row, head):
//   dS = P (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// P is recomputed from the forward pass's log-sum-exp; nothing of the forward
// pass is stored besides O and the lse.
//
// Two orientations, no atomics, fixed summation order:
// - rows resident (bwd_dq_kernel): the forward pass's work split (own block:
//   256 query rows of one head per workgroup, causal; earlier blocks: a tile of
//   up to 256 gathered rows of one bin), keys streamed through LDS in tiles of
//   64. Per tile S^T = K Q^T, dP^T = V dO^T, dS, and dQ^T += K^T dS^T (K^T
//   read from the K tile through the LDS transpose read). Each (row, head,
//   slot) gets an fp32 partial dQ; a sum over the slots follows.
// - keys resident (bwd_dkdv_kernel): one workgroup per (kv head, block, chunk
//   of 256 keys), 8 waves of 32 keys with V in registers and K in LDS as
//   MFMA B operands. The block's own rows (for each query head of the kv head,
//   causally) and then the rows of its bin stream through LDS in tiles of 32
//   rows, stored row-major; the transposed operands come from the same tiles
//   through the LDS transpose read. Per tile S = Q K^T, dP = dO V^T, dS,
//   dV^T += dO^T P and dK^T += Q^T dS; dK and dV are written once (a bin
//   too large for one workgroup is split into segments whose fp32 partials
//   a second kernel adds in segment order).
// Lane layouts: v_mfma_f32_32x32x16_bf16, lane l holds A[m = l%32][k = 8(l/32)
// .. +7] and B[k = 8(l/32) .. +7][n = l%32]; accumulator i of lane l is
// C[8(i/4) + 4(l/32) + i%4][l%32]. Feeding M-row m from source row perm(m)
// (bits 2 and 3 swapped) makes accumulator i of lane half hh hold source row
// 16(i/8) + 8hh + i%8: two runs of 8 consecutive rows, exactly the 8-wide K
// slices the next product takes from the same lane.
#include <math.h>
#include <stdlib.h>

#include "bwd.h"

namespace moba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer descriptor word 3 (gfx9 family)
constexpr int kDqRows = kRowsBf16;        // query rows per dQ workgroup (8 waves x 32)
constexpr int kKvRows = 32;               // rows per dK/dV tile

enum { BWD_HIST = 0, BWD_DIAG = 1 };

struct BwdArgs {
  const __bf16 *q, *k, *v, *dout;
  const float *lse, *delta;  // [Hq][T]
  int64_t T;
  int Hq, Hkv, G, B, topk;
  float c2, scale;  // c2 = scale * log2(e)
  int g0, h0, Hp;
  int64_t NBb, nbins;
  const int4 *info;
  const uint32_t *tile_off, *bin_off, *items;
  const int4 *tile_rec;
  float *dq_part;
  __bf16 *dk, *dv;
  const void *zeros;  // 256 zero bytes: the rows past the end of a dK/dV tile
  // bin segments of the dK/dV stage
  const uint32_t *ext_off, *slot_off;
  float *part;
  int64_t seg_rows, extra_wg, part_half;  // part_half: floats of the dK half of part
};

__device__ __forceinline__ floatx16 mfma(const bf16x8 &a, const bf16x8 &b, const floatx16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int perm32(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// dK/dV tiles: M row (or K index) 16 c + 8 a + 4 b + e (a, b in {0, 1},
// e < 4) takes tile row 16 c + 4 e + 2 b + a, so that accumulator i = 8 c + j
// of lane half hh holds row 16 c + 4 (j % 4) + 2 hh + j / 4: its 8 rows are
// the K slice the lane passes on, read 4 rows apart by the transpose reads.
__device__ __forceinline__ int perm_tr(int m) {
  return (m & 16) | ((m & 3) << 2) | (((m >> 2) & 1) << 1) | ((m >> 3) & 1);
}
// Inverse: the position 16 c + 8 b + 4 a + e that tile row 16 c + 4 e + 2 b + a
// takes in that order.
__device__ __forceinline__ int perm_tr_pos(int r) {
  return (r & 16) | (((r >> 1) & 1) << 3) | ((r & 1) << 2) | ((r >> 2) & 3);
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t *lds_short4_t;
// ds_read_b64_tr_b16 at an 8-byte-aligned LDS address
__device__ __forceinline__ bf16x4 tr_read(const char *p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t)p));
}

// Raw buffer descriptor from wave-uniform values; offsets past `bytes` read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, int64_t bytes) {
  const uint64_t v = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)(bytes < 0x7fffffff ? bytes : 0x7fffffff));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, n,
                                           kBufferWord3);
}

// Wait for every vector memory load of the wave (and its LDS accesses).
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x70); }
// Wait until at most N vector memory loads of this wave are outstanding (and
// for its LDS accesses).
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(N | 0x70);
}

typedef __attribute__((address_space(1))) const void *global_ptr_t;

// Workgroup barrier that orders LDS only: this wave's LDS accesses complete,
// then s_barrier. Unlike __syncthreads it does not wait for the wave's
// outstanding vector memory loads, so direct-to-LDS loads of later tiles
// stay in flight; every wave waits for its own loads of the next tile before
// it. The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void store_bf16x4(__bf16 *p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *(bf16x4 *)p = v;
}

// D[h][t] = <dO[t][h], O[t][h]> in fp32; 16 lanes per (row, head), rows
// ordered head-major so a workgroup writes 16 consecutive entries.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const __bf16 *__restrict__ out,
                                                        const __bf16 *__restrict__ dout,
                                                        int64_t T, int Hq,
                                                        float *__restrict__ delta) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= T * Hq) return;
  const int lane = threadIdx.x & 15;
  const int h = (int)(row / T);
  const int64_t t = row - (int64_t)h * T;
  const int64_t off = (t * Hq + h) * kHeadDim + lane * 8;
  const bf16x8 o = *(const bf16x8 *)(out + off);
  const bf16x8 g = *(const bf16x8 *)(dout + off);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (float)o[j] * (float)g[j];
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 8);
  if (lane == 0) delta[row] = s;
}

// ---- dQ: rows resident, keys streamed.
//
// LDS: three stages of {K tile, V tile}, 16 KiB each, as three separate
// arrays: 64 rows x 16 chunks of 16 B, chunk c of row r at position
// c ^ swz(r) with swz(r) = 4 (r % 4) + (r / 4) % 4. Every wave fills 2 KiB of
// each with direct loads, two tiles ahead. K^T, the A operand of
// dQ^T += K^T dS^T, comes from the K tile through ds_read_b64_tr_b16: for
// 16-lane group G and read h, lane s addresses key 16 c + 8 (s / 32) + 4 h +
// (s % 16) / 4 (of a 32-key half), columns 32 dt + 16 G%2 + 4 (s % 4) .. +3,
// and lane l receives the keys of its K slice 8 hh + 4 h .. +3 at column
// 32 dt + l % 32. The four keys of a read differ in swz by 4 each and the
// four chunks a half-wave reads in swz's low bits, so the 32 lanes hit 64
// different banks. A body ends when each wave's loads of the next tile have
// landed, with an LDS-only barrier that leaves the tile after in flight; the
// loop is unrolled by the stages so that the compiler sees that a body's
// direct loads and its LDS reads never overlap.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int MODE>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(const BwdArgs a) {
  constexpr int TILE = 16384, STAGE = 2 * TILE, LPW = 2;
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage2[STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int r = wave * 32 + n;  // this lane's query row inside the tile

  int g, p, nkt, nrows, hq, qpos = 0;
  int64_t t, kbeg, slot, gb;
  if (MODE == BWD_HIST) {
    // the forward pass's tiles of its earlier-block attention, XCD-contiguous
    const uint32_t ntiles = a.tile_off[a.nbins];
    const uint32_t per = (ntiles + 7) >> 3;
    const uint32_t jj = blockIdx.x >> 3;
    if (jj >= per) return;
    const uint32_t tile = (blockIdx.x & 7) * per + jj;
    if (tile >= ntiles) return;
    const int4 rec = a.tile_rec[tile];
    p = (int)((uint32_t)rec.z / a.NBb);
    gb = (uint32_t)rec.z % a.NBb;
    nrows = rec.y;
    slot = a.items[(uint32_t)rec.x + (r < nrows ? r : 0)];
    const int64_t th = slot / a.topk;
    t = th / a.Hp;
    hq = a.h0 + (int)(th % a.Hp);
    g = a.g0 + p;
    kbeg = rec.w;
    nkt = a.B / kKeyTile;
  } else {
    // (kv head of the pass, block, query tile with the most keys first, query
    // head of the group); every XCD takes a contiguous run
    const int nq = (a.B + kDqRows - 1) / kDqRows;
    const uint32_t total = (uint32_t)(a.Hp * a.NBb * nq);
    const uint32_t per = (total + 7) >> 3;
    const uint32_t jj = blockIdx.x >> 3;
    if (jj >= per) return;
    const uint32_t wi = (blockIdx.x & 7) * per + jj;
    if (wi >= total) return;
    uint32_t rest = wi / (uint32_t)a.G;
    const int qt = nq - 1 - (int)(rest % (uint32_t)nq);
    rest /= (uint32_t)nq;
    gb = rest % (uint32_t)a.NBb;
    const int hl = (int)(rest / (uint32_t)a.NBb) * a.G + (int)(wi % (uint32_t)a.G);
    const int4 bi = a.info[gb];
    if (bi.x < 0 || qt * kDqRows >= bi.z) return;
    hq = a.h0 + hl;
    g = hq / a.G;
    p = g - a.g0;
    nrows = min(kDqRows, bi.z - qt * kDqRows);
    const int qfirst = qt * kDqRows;
    qpos = qfirst + r;
    t = bi.y + qfirst + (r < nrows ? r : 0);
    nkt = (min(bi.z, qfirst + kDqRows) + kKeyTile - 1) / kKeyTile;
    kbeg = bi.y;
    const int nsel = min(a.topk, bi.w + 1);  // the own block is the last chosen slot
    slot = (t * a.Hp + hl) * a.topk + nsel - 1;
  }

  // this lane's query row and output gradient as B operands (k = d)
  bf16x8 qB[8], doB[8];
  {
    const int64_t off = (t * a.Hq + hq) * kHeadDim + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qB[kk] = *(const bf16x8 *)(a.q + off + 16 * kk);
      doB[kk] = *(const bf16x8 *)(a.dout + off + 16 * kk);
    }
  }
  const float lse2 = a.lse[(int64_t)hq * a.T + t] * kLog2e;
  const float Dr = a.delta[(int64_t)hq * a.T + t];
  const float c2 = a.c2;

  // direct-load sources (byte offsets from the tile base): regions of 4 rows
  const int64_t kstride = (int64_t)a.Hkv * kHeadDim;
  uint32_t kso[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int krow = (wave * LPW + j) * 4 + (lane >> 4);
    kso[j] = (uint32_t)krow * (uint32_t)kstride * 2u + (uint32_t)(((lane & 15) ^ swz(krow)) * 16);
  }
  const int lw = wave * LPW * 1024;  // this wave's share of a tile
  const __bf16 *kt0 = a.k + kbeg * kstride + (int64_t)g * kHeadDim;
  const __bf16 *vt0 = a.v + kbeg * kstride + (int64_t)g * kHeadDim;
  const int64_t span = (a.T - kbeg) * kstride * 2;  // bytes to the end of the tensor (upper bound)
  const __amdgpu_buffer_rsrc_t krs = uniform_rsrc(kt0, span);
  const __amdgpu_buffer_rsrc_t vrs = uniform_rsrc(vt0, span);
  auto issue = [&](char *st, int kt) {
    const uint32_t soff = (uint32_t)kt * kKeyTile * (uint32_t)kstride * 2u;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(st + lw + j * 1024), 16, kso[j], soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(st + TILE + lw + j * 1024), 16, kso[j], soff, 0, 0);
    }
  };
  // LDS read offsets of this lane's A operands: K and V rows (perm32) for S
  // and dP; the transpose reads of K^T per (dt, h)
  const int pr = perm32(n);
  uint32_t krd[8], trk[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) krd[kk] = pr * 256 + (((2 * kk + hh) ^ swz(pr)) * 16);
  {
    const int jq = (lane & 15) >> 2, gq = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = 8 * hh + 4 * h + jq;  // + 32 st + 16 c, which leave swz unchanged
        const int chunk = 4 * dt + 2 * gq + ((lane & 3) >> 1);
        trk[2 * dt + h] = key * 256 + ((chunk ^ swz(key)) * 16) + 8 * (lane & 1);
      }
  }

  floatx16 dq[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[dt][i] = 0.f;

  auto compute = [&](const char *Ks, int kt) {
    const char *Vs = Ks + TILE;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      floatx16 sc, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) { sc[i] = 0.f; dp[i] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        sc = mfma(*(const bf16x8 *)(Ks + st * 8192 + krd[kk]), qB[kk], sc);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        dp = mfma(*(const bf16x8 *)(Vs + st * 8192 + krd[kk]), doB[kk], dp);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 b;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * c + j;
          float pv = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, -lse2));
          if (MODE == BWD_DIAG && kt * kKeyTile + 32 * st + 16 * c + 8 * hh + j > qpos) pv = 0.f;
          b[j] = (__bf16)(pv * (dp[i] - Dr));
        }
        const char *kb = Ks + (32 * st + 16 * c) * 256;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x4 lo = tr_read(kb + trk[2 * dt]);
          const bf16x4 hi = tr_read(kb + trk[2 * dt + 1]);
          dq[dt] = mfma((bf16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), b, dq[dt]);
        }
      }
      // keep the two halves apart: interleaving them costs registers
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // body of key tile kt (stage cur), loading tile kt + 2 into stage nx2
  auto body = [&](const char *cur, char *nx2, int kt) {
    // the last two bodies load the last tile again into a stage nobody reads,
    // so that every body issues the same loads
    issue(nx2, min(kt + 2, nkt - 1));
    compute(cur, kt);
    // this wave's loads of tile kt + 1 (issued a body ago) have landed
    wait_vm<2 * LPW>();
    lds_barrier();
  };

  issue(stage0, 0);
  issue(stage1, min(1, nkt - 1));
  wait_all_loads();
  __syncthreads();
  int kt = 0;
  for (; kt + 3 <= nkt; kt += 3) {
    body(stage0, stage2, kt);
    body(stage1, stage0, kt + 1);
    body(stage2, stage1, kt + 2);
  }
  if (kt < nkt) body(stage0, stage2, kt);
  if (kt + 1 < nkt) body(stage1, stage0, kt + 1);
  wait_all_loads();  // the last bodies' repeated loads

  if (r >= nrows) return;
  float *dst = a.dq_part + slot * kHeadDim + 4 * hh;
  const float sc = a.scale;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa)
      *(float4 *)(dst + 32 * dt + 8 * aa) =
          make_float4(dq[dt][4 * aa] * sc, dq[dt][4 * aa + 1] * sc, dq[dt][4 * aa + 2] * sc,
                      dq[dt][4 * aa + 3] * sc);
}

__device__ __forceinline__ int seq_of(const int32_t *cu, int S, int64_t t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// dQ[t][h] = sum of the partials of its slots: the own block (last chosen
// slot) first, then the earlier blocks in slot order (those the dispatch
// stage routed: 0 <= block < own). 32 lanes per (row, head).
__global__ __launch_bounds__(256) void bwd_dq_sum_kernel(const float *__restrict__ dq_part,
                                                         const int32_t *__restrict__ idx,
                                                         const int32_t *__restrict__ cu, int S,
                                                         int64_t T, int Hq, int h0, int Hp, int B,
                                                         int k, const int32_t *__restrict__ status,
                                                         __bf16 *__restrict__ dq) {
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= T * Hp) return;
  const int lane = threadIdx.x & 31;
  const int64_t t = row / Hp;
  const int hl = (int)(row % Hp);
  if (*status != 0) {  // the table check failed: no partial is valid
    store_bf16x4(dq + (t * Hq + h0 + hl) * kHeadDim + lane * 4, NAN, NAN, NAN, NAN);
    return;
  }
  const int s = seq_of(cu, S, t);
  const int c = (int)((t - cu[s]) / B);
  const int nsel = min(k, c + 1);
  const float *base = dq_part + row * k * kHeadDim + lane * 4;
  const int32_t *sel = idx + row * k;
  float4 acc = *(const float4 *)(base + (int64_t)(nsel - 1) * kHeadDim);
  // the earlier slots' rows are all loaded at once (16 per batch; a slot the
  // dispatch did not route holds stale workspace bytes and is not added)
  for (int i0 = 0; i0 < nsel - 1; i0 += 16) {
    float4 x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      x[u] = i0 + u < nsel - 1 ? *(const float4 *)(base + (int64_t)(i0 + u) * kHeadDim)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (i0 + u >= nsel - 1) break;
      const int j = sel[i0 + u];
      if (j >= 0 && j < c) {
        acc.x += x[u].x; acc.y += x[u].y; acc.z += x[u].z; acc.w += x[u].w;
      }
    }
  }
  store_bf16x4(dq + (t * Hq + h0 + hl) * kHeadDim + lane * 4, acc.x, acc.y, acc.z, acc.w);
}

// ---- dK, dV: keys resident, rows streamed.
//
// LDS: three stages of {Q tile, dO tile}, each 32 rows of 256 B at a pitch
// of 272 B, as three separate arrays; four slots of the 32 rows' lse (log2
// units) and D; two slots of the rows' Q and dO addresses; the waves' K rows
// (pitch 272 B). The padding puts row r at bank group 4r mod 64, so the 16
// rows that 16 lanes read at one chunk column fall in 16 different 16-byte
// bank groups. The transposed operands (Q^T, dO^T as A operands of dK^T and
// dV^T) come from the same tiles through ds_read_b64_tr_b16: in each 16-lane
// group, output lane 4p+q receives as element j element q of the 8 bytes that
// lane 4j+p addressed. Row r of a tile feeds the MFMAs' M row (or K index)
// perm_tr so that one transpose read takes rows 4 apart, whose bank groups
// are 16 apart: conflict-free. Every lane's operand addresses a base plus
// compile-time offsets.
//
// The Q and dO tiles of a stage are 2 x 32 x 17 slots of 16 B (the 17th slot
// of a row is padding), filled by 17 wave-wide direct loads of 64 slots,
// three each on waves 0, 2 and 3 and two each on waves 4..7. A row past the
// end of the tile loads from a zeroed 256-byte area and gets lse = +inf and
// D = 0, so its probabilities and dS are exactly 0. Tile x's rows are fetched
// two tiles ahead: in the body of tile x - 2, wave 1 (lanes 0..31, one row
// each) loads the items of tile x + 1 and the lse and D of tile x into
// registers; every wave issues tile x's Q and dO loads from the row addresses
// in LDS; at the end of the body wave 1 stores the lse and D, decodes the
// items into (token, head) and stores the addresses of those rows' Q and dO;
// wave 1 issues no direct loads, so that nothing it waits for is a tile
// load. A body ends when each wave's loads of the next tile have
// landed, with a barrier that leaves the loads of the tile after in flight.
// The loop is unrolled by the three stages so that every access names its
// stage array: the compiler then sees that a body's direct loads and its LDS
// reads never overlap and adds no waits between them.
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int NP = 272;                   // pitch of a tile row
  constexpr int SLOTS = 17;                 // 16-byte slots per tile row
  constexpr int QN = 0, DN = kKvRows * NP;  // Q and dO tiles of a stage
  constexpr int STAGE = 2 * kKvRows * NP;
  static_assert(2 * kKvRows * SLOTS == 17 * 64, "17 direct loads per tile");
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage2[STAGE];
  __shared__ __attribute__((aligned(16))) float lse_d[4][2 * kKvRows];  // [slot][lse 32, D 32]
  // addresses of the Q and dO rows of a tile (the zeroed area past its end)
  __shared__ __attribute__((aligned(16))) const char *raddr[2][2][kKvRows];  // [slot][Q, dO][row]
  __shared__ __attribute__((aligned(1024))) char klds[8 * 32 * NP];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int nch = (a.B + kKvKeys - 1) / kKvKeys;
  // The first extra_wg workgroups take the segments beyond the first of the
  // split bins (extra segment e = 8 * ((x / 8) / nch) + x % 8, chunk
  // (x / 8) % nch), the others the first segment of every bin (bin
  // 8 * ((x' / 8) / nch) + x' % 8 with x' = x - extra_wg): every XCD takes
  // every 8th bin or segment, the chunks of one back to back.
  int64_t b;
  int kc, seg;
  if ((int64_t)blockIdx.x < a.extra_wg) {
    const int64_t xg = blockIdx.x >> 3;
    const int64_t se = (xg / nch) * 8 + (blockIdx.x & 7);
    kc = (int)(xg % nch);
    if (se >= (int64_t)a.ext_off[a.nbins]) return;
    int64_t lo = 0, hi = a.nbins - 1;  // the bin whose extra segments include se
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if ((int64_t)a.ext_off[mid] <= se) lo = mid; else hi = mid - 1;
    }
    b = lo;
    seg = (int)(se - a.ext_off[b]) + 1;
  } else {
    const int64_t x = blockIdx.x - a.extra_wg;
    const int64_t xg = x >> 3;
    b = (xg / nch) * 8 + (x & 7);
    kc = (int)(xg % nch);
    seg = 0;
    if (b >= a.nbins) return;
  }
  const int nseg = (int)(a.ext_off[b + 1] - a.ext_off[b]) + 1;
  const int p = (int)(b / a.NBb);
  const int64_t gb = b % a.NBb;
  const int4 bi = a.info[gb];
  if (bi.x < 0 || kc * kKvKeys >= bi.z) return;
  const int g = a.g0 + p;
  const int k0 = kc * kKvKeys;
  const int kw = k0 + 32 * wave;  // first key of this wave, local to the block
  const int key = kw + n;
  const bool kvalid = key < bi.z;

  // K rows of this wave's keys in LDS (32 rows at pitch NP; each lane reads
  // back what it wrote), V rows in registers, both as MFMA B operands (k = d);
  // a lane past the block's end takes the block's first row (its results are
  // dropped)
  char *const kw_lds = klds + wave * 32 * NP;
  bf16x8 vB[8];
  {
    const int64_t off = ((int64_t)(bi.y + (kvalid ? key : 0)) * a.Hkv + g) * kHeadDim + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      *(bf16x8 *)(kw_lds + n * NP + (2 * kk + hh) * 16) = *(const bf16x8 *)(a.k + off + 16 * kk);
      vB[kk] = *(const bf16x8 *)(a.v + off + 16 * kk);
    }
  }
  const int krd = n * NP + hh * 16;  // + 32 kk
  floatx16 dk[4], dv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dk[dt][i] = 0.f; dv[dt][i] = 0.f; }

  // tiles: the own block's rows from k0 on, per query head of the kv head
  // (first segment only), then the segment's items of the bin
  const int own_per_head = (bi.z - k0 + kKvRows - 1) / kKvRows;
  const int n_own = seg == 0 ? a.G * own_per_head : 0;
  const uint32_t ibeg = a.bin_off[b] + (uint32_t)(seg * a.seg_rows);
  const uint32_t iend = (uint32_t)min((int64_t)a.bin_off[b + 1], (int64_t)ibeg + a.seg_rows);
  const int ntiles = n_own + (int)((iend - ibeg + kKvRows - 1) / kKvRows);

  // ---- row staging (wave 1, lanes 0..31: row n of a tile)
  const bool stager = wave == 1 && lane < kKvRows;
  const uint32_t ilast = iend > 0 ? iend - 1 : 0u;
  // the item of row n of tile x, clamped to an existing entry (own tiles and
  // rows past the bin read one whose value goes unused)
  auto item_load = [&](int x) -> uint32_t {
    const uint32_t j = ibeg + (uint32_t)max(x - n_own, 0) * kKvRows + n;
    return a.items[j < ilast ? j : ilast];
  };
  // (token, head) of row n of tile x; token -1 past the tile's end
  auto row_of = [&](int x, uint32_t item) -> int2 {
    if (x < n_own) {
      const int gi = x / own_per_head;
      const int rl = k0 + (x - gi * own_per_head) * kKvRows + n;
      return rl < bi.z ? make_int2(bi.y + rl, a.h0 + p * a.G + gi) : make_int2(-1, 0);
    }
    const uint32_t j = ibeg + (uint32_t)(x - n_own) * kKvRows + n;
    if (x >= ntiles || j >= iend) return make_int2(-1, 0);
    // the divisors pass through an empty asm so that the compiler does not
    // keep their reciprocals in vector registers for the whole loop
    uint32_t dk_ = (uint32_t)a.topk, dh_ = (uint32_t)a.Hp;
    asm volatile("" : "+s"(dk_), "+s"(dh_));
    const uint32_t th = item / dk_;
    const uint32_t t = th / dh_;
    return make_int2((int)t, a.h0 + (int)(th - t * dh_));
  };
  const int npos = perm_tr_pos(n);  // where row n's lse and D go in a slot
  auto lse_store = [&](int x, int2 rw, float l, float d) {
    float *L = lse_d[x & 3];
    L[npos] = rw.x >= 0 ? l * kLog2e : INFINITY;
    L[kKvRows + npos] = rw.x >= 0 ? d : 0.f;
  };
  auto lse_off = [&](int2 rw) { return rw.x >= 0 ? (int64_t)rw.y * a.T + rw.x : (int64_t)0; };
  auto raddr_store = [&](int x, int2 rw) {
    const int64_t o = ((int64_t)rw.x * a.Hq + rw.y) * kHeadDim;
    raddr[x & 1][0][n] = rw.x >= 0 ? (const char *)(a.q + o) : (const char *)a.zeros;
    raddr[x & 1][1][n] = rw.x >= 0 ? (const char *)(a.dout + o) : (const char *)a.zeros;
  };

  // ---- direct loads of the Q and dO tiles: this wave's loads are slots
  // 64 ld + lane for ld = ld0 .. ld0 + nld - 1
  const int wv = wave == 0 ? 0 : wave - 1;  // 0..6 over the loading waves
  const int nld = wave == 1 ? 0 : wv < 3 ? 3 : 2;
  const int ld0 = wv < 3 ? 3 * wv : 9 + 2 * (wv - 3);
  auto issue = [&](char *st, int x) {
    const char *const *ra = &raddr[x & 1][0][0];
    const char *gp[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      if (u >= nld) break;
      const int sx = 64 * (ld0 + u) + lane;
      const bool is_do = sx >= kKvRows * SLOTS;
      const int y = is_do ? sx - kKvRows * SLOTS : sx;
      const int row = y / SLOTS;
      const int chunk = min(y - row * SLOTS, 15);  // the padding slot repeats chunk 15
      gp[u] = ra[(is_do ? kKvRows : 0) + row] + 16 * chunk;
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      if (u >= nld) break;
      __builtin_amdgcn_global_load_lds((global_ptr_t)gp[u], (lds_ptr_t)(st + 1024 * (ld0 + u)), 16,
                                       0, 0);
    }
  };

  // LDS read offsets: Q / dO rows as A operands of S and dP (row perm_tr(n));
  // transpose reads of Q^T / dO^T as A operands of dK^T and dV^T: for MFMA
  // (dt, c) read h of lane s takes the 8 bytes at row 16 c + 4 ((s % 16) / 4)
  // + 2 (s / 32) + h, columns 32 dt + 16 ((s / 16) % 2) + 4 (s % 4) .. +3,
  // which hands lane l the rows of its K indices 8 hh + 4 h .. +3 at column
  // 32 dt + l % 32
  const int qrd = perm_tr(n) * NP + hh * 16;  // + 32 kk: chunk 2 kk + hh
  const int trl = (4 * ((lane & 15) >> 2) + 2 * hh) * NP + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  const float c2 = a.c2;
  auto tr_a = [&](const char *tile, int dt, int c) {
    const bf16x4 lo = tr_read(tile + trl + 16 * c * NP + 64 * dt);
    const bf16x4 hi = tr_read(tile + trl + (16 * c + 1) * NP + 64 * dt);
    return (bf16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  auto compute = [&](const char *S_, int it) {
    if (kw >= bi.z) return;  // every key of this wave is past the block's end
    const bool own = it < n_own;
    int rt = 0;  // local position of the tile's first row (own tiles)
    if (own) {
      const int gi = it / own_per_head;
      rt = k0 + (it - gi * own_per_head) * kKvRows;
      if (rt + kKvRows - 1 < kw) return;  // every row precedes every key of this wave
    }
    const float *L = lse_d[it & 3];
    floatx16 s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) { s[i] = 0.f; dp[i] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      s = mfma(*(const bf16x8 *)(S_ + QN + qrd + 32 * kk), *(const bf16x8 *)(kw_lds + krd + 32 * kk),
               s);
    // probabilities in place of the scores
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float4 l0 = *(const float4 *)(L + 16 * c + 8 * hh);
      const float4 l1 = *(const float4 *)(L + 16 * c + 8 * hh + 4);
      const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * c + j;
        s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lv[j]));
      }
    }
    if (own) {
      // causal mask of the own block: key > row, with row = rt + 16 c +
      // 4 (j % 4) + 2 hh + j / 4 for score 8 c + j of this lane
      const int kr = key - rt - 2 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kr > 16 * (i >> 3) + 4 * (i & 3) + ((i >> 2) & 1)) s[i] = 0.f;
    }
    bf16x8 pb[2], db[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[c][j] = (__bf16)s[8 * c + j];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) dp = mfma(*(const bf16x8 *)(S_ + DN + qrd + 32 * kk), vB[kk], dp);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        dv[dt] = mfma(tr_a(S_ + DN, dt, c), pb[c], dv[dt]);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float4 d0 = *(const float4 *)(L + kKvRows + 16 * c + 8 * hh);
      const float4 d1 = *(const float4 *)(L + kKvRows + 16 * c + 8 * hh + 4);
      const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) db[c][j] = (__bf16)(s[8 * c + j] * (dp[8 * c + j] - dd[j]));
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        dk[dt] = mfma(tr_a(S_ + QN, dt, c), db[c], dk[dt]);
      }
  };

  // body of tile it: cur is its stage, nx2 the stage of tile it + 2
  int2 st_rw;  // stager lanes: row n of tile it + 2 at the start of body it
  auto body = [&](char *cur, char *nx2, int it) {
    // assigned and read on the stager lanes only
    uint32_t st_item;
    float st_l, st_d;
    if (stager) {
      st_item = item_load(it + 3);
      const int64_t o = lse_off(st_rw);
      st_l = a.lse[o];
      st_d = a.delta[o];
    }
    issue(nx2, it + 2);
    compute(cur, it);
    // this wave's loads from before this body's Q/dO loads have landed:
    // tile it + 1's (issued a body ago)
    if (nld == 3) wait_vm<3>(); else if (nld == 2) wait_vm<2>(); else wait_vm<0>();
    if (stager) {
      // the staged values are first touched here, after the compute (the
      // empty asm keeps the compiler from converting them right after
      // their loads, which would wait for the loads there)
      asm volatile("" : "+v"(st_l), "+v"(st_d), "+v"(st_item));
      lse_store(it + 2, st_rw, st_l, st_d);
      st_rw = row_of(it + 3, st_item);
      raddr_store(it + 3, st_rw);
    }
    lds_barrier();
  };

  if (ntiles > 0) {
    // prologue: rows of tiles 0 and 1 with their lse and D, their loads, then
    // the rows of tile 2
    if (stager) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int2 rw = row_of(x, item_load(x));
        raddr_store(x, rw);
        const int64_t o = lse_off(rw);
        lse_store(x, rw, a.lse[o], a.delta[o]);
      }
    }
    __syncthreads();
    issue(stage0, 0);
    issue(stage1, 1);
    __syncthreads();  // every wave has read both address slots
    if (stager) {
      st_rw = row_of(2, item_load(2));
      raddr_store(2, st_rw);
    }
    wait_all_loads();
    __syncthreads();
    int it = 0;
    for (; it + 3 <= ntiles; it += 3) {
      body(stage0, stage2, it);
      body(stage1, stage0, it + 1);
      body(stage2, stage1, it + 2);
    }
    if (it < ntiles) body(stage0, stage2, it);
    if (it + 1 < ntiles) body(stage1, stage0, it + 1);
    wait_all_loads();  // the last bodies' prefetches (rows past the end)
  }

  if (!kvalid) return;
  const float sc = a.scale;
  if (nseg > 1) {
    // fp32 partial of this segment, summed with the bin's other segments by
    // bwd_dkdv_sum_kernel
    const int64_t slot = a.slot_off[b] + seg;
    float *pk = a.part + ((slot * nch + kc) * kKvKeys + (key - k0)) * kHeadDim + 4 * hh;
    float *pv = pk + a.part_half;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        *(float4 *)(pk + 32 * dt + 8 * aa) =
            make_float4(dk[dt][4 * aa] * sc, dk[dt][4 * aa + 1] * sc, dk[dt][4 * aa + 2] * sc,
                        dk[dt][4 * aa + 3] * sc);
        *(float4 *)(pv + 32 * dt + 8 * aa) =
            make_float4(dv[dt][4 * aa], dv[dt][4 * aa + 1], dv[dt][4 * aa + 2], dv[dt][4 * aa + 3]);
      }
    return;
  }
  const int64_t o = ((int64_t)(bi.y + key) * a.Hkv + g) * kHeadDim + 4 * hh;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      store_bf16x4(a.dk + o + 32 * dt + 8 * aa, dk[dt][4 * aa] * sc, dk[dt][4 * aa + 1] * sc,
                   dk[dt][4 * aa + 2] * sc, dk[dt][4 * aa + 3] * sc);
      store_bf16x4(a.dv + o + 32 * dt + 8 * aa, dv[dt][4 * aa], dv[dt][4 * aa + 1],
                   dv[dt][4 * aa + 2], dv[dt][4 * aa + 3]);
    }
}

// Exclusive scans over the bins of a pass: ext_off (segments beyond the
// first, ceil(rows / seg_rows) - 1 per bin) and slot_off (partial slots: all
// segments of a split bin, none for a bin of one segment).
__global__ __launch_bounds__(1024) void dkdv_seg_scan_kernel(const uint32_t *__restrict__ bin_off,
                                                             int64_t nbins, int64_t seg_rows,
                                                             uint32_t *__restrict__ ext_off,
                                                             uint32_t *__restrict__ slot_off) {
  __shared__ uint32_t wsum[2][16];
  __shared__ uint32_t carry[2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int64_t base = 0; base < nbins; base += 1024) {
    const int64_t bb = base + threadIdx.x;
    uint32_t x[2] = {0u, 0u};
    if (bb < nbins) {
      const int64_t rows = (int64_t)bin_off[bb + 1] - bin_off[bb];
      const int64_t nseg = rows > seg_rows ? (rows + seg_rows - 1) / seg_rows : 1;
      x[0] = (uint32_t)(nseg - 1);
      x[1] = nseg > 1 ? (uint32_t)nseg : 0u;
    }
    uint32_t incl[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      uint32_t y = x[v];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(y, o);
        if (lane >= o) y += t;
      }
      if (lane == 63) wsum[v][w] = y;
      incl[v] = y;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        uint32_t y = lane < 16 ? wsum[v][lane] : 0u;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const uint32_t t = __shfl_up(y, o);
          if (lane >= o) y += t;
        }
        if (lane < 16) wsum[v][lane] = y;
      }
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 2; ++v) incl[v] += (w > 0 ? wsum[v][w - 1] : 0u) + carry[v];
    if (bb < nbins) {
      ext_off[bb] = incl[0] - x[0];
      slot_off[bb] = incl[1] - x[1];
    }
    __syncthreads();
    if (threadIdx.x == 1023) { carry[0] = incl[0]; carry[1] = incl[1]; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    ext_off[nbins] = carry[0];
    slot_off[nbins] = carry[1];
  }
}

// dK, dV of the keys of a split bin: the sum of its segments' partials in
// segment order, rounded to bf16. One workgroup per (bin, key chunk); 8
// rows of 32 lanes (4 dims each) at a time.
__global__ __launch_bounds__(256) void bwd_dkdv_sum_kernel(const BwdArgs a) {
  const int nch = (a.B + kKvKeys - 1) / kKvKeys;
  const int64_t b = blockIdx.x / nch;
  const int kc = (int)(blockIdx.x % nch);
  if (b >= a.nbins) return;
  const int nseg = (int)(a.ext_off[b + 1] - a.ext_off[b]) + 1;
  if (nseg == 1) return;
  const int p = (int)(b / a.NBb);
  const int4 bi = a.info[b % a.NBb];
  const int k0 = kc * kKvKeys;
  if (bi.x < 0 || k0 >= bi.z) return;
  const int g = a.g0 + p;
  const int e = (threadIdx.x & 31) * 4;
  const int64_t slot0 = a.slot_off[b];
  for (int kl = threadIdx.x >> 5; kl < min(kKvKeys, bi.z - k0); kl += 8) {
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    for (int sg = 0; sg < nseg; ++sg) {
      const float *pk = a.part + (((slot0 + sg) * nch + kc) * kKvKeys + kl) * kHeadDim + e;
      const float4 x = *(const float4 *)pk;
      const float4 y = *(const float4 *)(pk + a.part_half);
      sk.x += x.x; sk.y += x.y; sk.z += x.z; sk.w += x.w;
      sv.x += y.x; sv.y += y.y; sv.z += y.z; sv.w += y.w;
    }
    const int64_t o = ((int64_t)(bi.y + k0 + kl) * a.Hkv + g) * kHeadDim + e;
    store_bf16x4(a.dk + o, sk.x, sk.y, sk.z, sk.w);
    store_bf16x4(a.dv + o, sv.x, sv.y, sv.z, sv.w);
  }
}

BwdArgs make_args(const Problem &pb, const Work &w, const BwdWork &bw, const BwdIo &io, int g0) {
  BwdArgs a{};
  a.q = (const __bf16 *)io.q;
  a.k = (const __bf16 *)io.k;
  a.v = (const __bf16 *)io.v;
  a.dout = (const __bf16 *)io.dout;
  a.lse = io.lse;
  a.delta = bw.delta;
  a.T = pb.T;
  a.Hq = pb.Hq; a.Hkv = pb.Hkv; a.G = pb.G; a.B = pb.B; a.topk = pb.k;
  a.scale = pb.scale;
  a.c2 = pb.scale * kLog2e;
  a.g0 = g0; a.h0 = g0 * pb.G; a.Hp = pb.Hp;
  a.NBb = pb.NBb;
  a.nbins = (int64_t)pb.P * pb.NBb;
  a.info = w.blk_info;
  a.tile_off = w.tile_off; a.bin_off = w.bin_off; a.items = w.items; a.tile_rec = w.tile_rec;
  a.dq_part = bw.dq_part;
  a.dk = (__bf16 *)io.dk;
  a.dv = (__bf16 *)io.dv;
  a.zeros = bw.zeros;
  a.ext_off = bw.ext_off;
  a.slot_off = bw.slot_off;
  a.part = bw.part;
  const DkdvSplit sp = dkdv_split(pb.T, pb.Hp, pb.k, pb.B);
  a.seg_rows = sp.seg_rows;
  a.extra_wg = (sp.extra_bound + 7) / 8 * 8 * sp.nch;
  a.part_half = 2 * sp.extra_bound * sp.nch * kKvKeys * kHeadDim;
  return a;
}

}  // namespace

DkdvSplit dkdv_split(int64_t T, int Hp, int k, int B) {
  DkdvSplit sp;
  int64_t seg = 262144;
  if (const char *env = getenv("MOBA_DKDV_SEGMENT_ROWS")) {
    const long long v = atoll(env);
    if (v >= kKvRows) seg = v / kKvRows * kKvRows;
  }
  sp.seg_rows = seg;
  sp.extra_bound = T * Hp * (int64_t)(k > 1 ? k - 1 : 0) / seg;  // dispatched rows / seg
  sp.nch = (B + kKvKeys - 1) / kKvKeys;
  return sp;
}

BwdExtra bwd_extra(size_t base, int64_t nbins, const DkdvSplit &sp) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  BwdExtra x;
  size_t off = al(base);
  x.zeros = off;    off = al(off + kBwdZeroBytes);
  x.ext_off = off;  off = al(off + sizeof(uint32_t) * (size_t)(nbins + 1));
  x.slot_off = off; off = al(off + sizeof(uint32_t) * (size_t)(nbins + 1));
  x.part = off;
  off = al(off + sizeof(float) * 2 * (size_t)(2 * sp.extra_bound) * sp.nch * kKvKeys * kHeadDim);
  x.end = off;
  return x;
}

hipError_t launch_bwd_delta(const Problem &pb, const void *out, const void *dout, float *delta,
                            hipStream_t s) {
  const int64_t rows = pb.T * pb.Hq;
  if (rows == 0) return hipSuccess;
  bwd_delta_kernel<<<dim3((unsigned)((rows + 15) / 16)), 256, 0, s>>>(
      (const __bf16 *)out, (const __bf16 *)dout, pb.T, pb.Hq, delta);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const Problem &pb, const Work &w, const BwdWork &bw, const BwdIo &io,
                         int g0, int which, hipStream_t s) {
  const BwdArgs a = make_args(pb, w, bw, io, g0);
  if (which & 1) {
    const int64_t nq = (pb.B + kDqRows - 1) / kDqRows;
    const int64_t gdiag = (pb.Hp * pb.NBb * nq + 7) / 8 * 8;
    bwd_dq_kernel<BWD_DIAG><<<dim3((unsigned)gdiag), 512, 0, s>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((which & 2) && pb.k > 1) {
    const int64_t ghist = (w.max_tiles + 7) / 8 * 8;
    bwd_dq_kernel<BWD_HIST><<<dim3((unsigned)ghist), 512, 0, s>>>(a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_bwd_dq_sum(const Problem &pb, const Work &w, const BwdWork &bw,
                             const BwdIo &io, int g0, hipStream_t s) {
  const int64_t rows = pb.T * pb.Hp;
  if (rows == 0) return hipSuccess;
  bwd_dq_sum_kernel<<<dim3((unsigned)((rows + 7) / 8)), 256, 0, s>>>(
      bw.dq_part, w.idx, w.cu, pb.S, pb.T, pb.Hq, g0 * pb.G, pb.Hp, pb.B, pb.k, w.status,
      (__bf16 *)io.dq);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const Problem &pb, const Work &w, const BwdWork &bw, const BwdIo &io,
                           int g0, hipStream_t s) {
  const BwdArgs a = make_args(pb, w, bw, io, g0);
  const int64_t nch = (pb.B + kKvKeys - 1) / kKvKeys;
  const int64_t grid = (a.nbins + 7) / 8 * 8 * nch;
  hipError_t e = launch_fill_u32((uint32_t *)bw.zeros, 0u, kBwdZeroBytes / 4, s);
  if (e != hipSuccess) return e;
  dkdv_seg_scan_kernel<<<1, 1024, 0, s>>>(a.bin_off, a.nbins, a.seg_rows, bw.ext_off,
                                          bw.slot_off);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_dkdv_kernel<<<dim3((unsigned)(a.extra_wg + grid)), 512, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.extra_wg > 0) {
    bwd_dkdv_sum_kernel<<<dim3((unsigned)(a.nbins * nch)), 256, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // a failed table check leaves every block out: dk and dv become NaN
  const int64_t words = pb.T * pb.Hkv * kHeadDim / 2;
  if ((e = launch_poison(w.status, io.dk, words, kNanBf16x2, s)) != hipSuccess) return e;
  return launch_poison(w.status, io.dv, words, kNanBf16x2, s);
}

}  // namespace moba
