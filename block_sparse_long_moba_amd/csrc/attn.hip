// Block attention on the matrix cores (MFMA), flash-style online softmax.
//
// MoBA summary page (paper-graph-ui), section 3.4 "Implementation", step 3:
// attention of each query over its own block with a causal mask, and over each
// earlier block it chose without one, each producing a partial output and its
// log-sum-exp; "Causality Enforcement" mechanism 2 for the own block. The same
// tile engine runs dense causal attention ("Standard Attention Baseline").
//
// Workgroup: 4 waves, 128 query rows (32 per wave), one kv head. Keys stream
// through LDS in tiles of 64 (double buffered). Each wave computes the
// transposed score tile S^T = K Q^T (keys on the MFMA's M side, queries on N)
// so a lane holds 16 scores of a single query: row max and row sum need no
// cross-lane work except one exchange with the lane 32 away. The K rows are
// fed to the MFMA in a permuted order chosen so that the 16 scores a lane
// holds are exactly the 8-key groups the P V product needs on its K side: the
// probabilities go from the accumulators straight into the next MFMA's B
// operand. O^T = V^T P^T then keeps one query per lane, so the rescale by the
// running max is a per-lane multiply. Values come pre-transposed (d-major) so
// the V^T operand is a contiguous 16-byte LDS read.
#include <math.h>

#include "moba_internal.h"

namespace moba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 inputs: v_mfma_f32_32x32x16_bf16 (A: 32x16, B: 16x32, fp32 accumulate).
// Lane l holds A[m = l%32][k = 8*(l/32) .. +7] and B[k = 8*(l/32) .. +7][n = l%32];
// accumulator i of lane l is C[8*(i/4) + 4*(l/32) + i%4][l%32].
struct PolBf16 {
  using T = __bf16;
  static constexpr int KP = kHeadDim + 8;  // LDS pitch of a key row (272 B)
  static constexpr int VP = kKeyTile + 8;  // LDS pitch of a V^T row (144 B)
  static constexpr int kOcc = 2;
  struct Q { bf16x8 v[kHeadDim / 16]; };
  // K row fed to M-row m: swapping bits 2 and 3 makes accumulator i of lane
  // half hh hold key 16*(i/8) + 8*hh + i%8 of the 32-key sub-tile.
  __device__ static int perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
  __device__ static int key_of(int st, int i, int hh) {
    return 32 * st + 16 * (i >> 3) + 8 * hh + (i & 7);
  }
  __device__ static void load_q(Q &q, const T *row, int hh) {
#pragma unroll
    for (int kk = 0; kk < kHeadDim / 16; ++kk) q.v[kk] = *(const bf16x8 *)(row + 16 * kk + 8 * hh);
  }
  __device__ static void qk(floatx16 &acc, const T *Ks, int st, const Q &q, int n, int hh) {
    const T *kr = Ks + (32 * st + perm(n)) * KP + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < kHeadDim / 16; ++kk) {
      const bf16x8 a = *(const bf16x8 *)(kr + 16 * kk);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.v[kk], acc, 0, 0, 0);
    }
  }
  __device__ static void pv(floatx16 (&o)[4], const T *Vs, const float (&p)[2][16], int n, int hh) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 b;
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = (__bf16)p[st][8 * c2 + j];
        const int key0 = 32 * st + 16 * c2 + 8 * hh;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 a = *(const bf16x8 *)(Vs + (32 * dt + n) * VP + key0);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[dt], 0, 0, 0);
        }
      }
  }
};

// fp32 inputs: v_mfma_f32_32x32x2f32 (lane l holds A[l%32][l/32], B[l/32][l%32]).
struct PolF32 {
  using T = float;
  static constexpr int KP = kHeadDim + 4;  // 528 B
  static constexpr int VP = kKeyTile + 4;  // 272 B
  static constexpr int kOcc = 1;
  struct Q { float v[kHeadDim / 2]; };
  // accumulator i of lane half hh holds key 2*i + hh of the 32-key sub-tile
  __device__ static int perm(int m) { return 8 * (m >> 3) + 2 * (m & 3) + ((m >> 2) & 1); }
  __device__ static int key_of(int st, int i, int hh) { return 32 * st + 2 * i + hh; }
  __device__ static void load_q(Q &q, const T *row, int hh) {
#pragma unroll
    for (int kk = 0; kk < kHeadDim / 2; ++kk) q.v[kk] = row[2 * kk + hh];
  }
  __device__ static void qk(floatx16 &acc, const T *Ks, int st, const Q &q, int n, int hh) {
    const T *kr = Ks + (32 * st + perm(n)) * KP + hh;
#pragma unroll
    for (int kk = 0; kk < kHeadDim / 2; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[2 * kk], q.v[kk], acc, 0, 0, 0);
  }
  __device__ static void pv(floatx16 (&o)[4], const T *Vs, const float (&p)[2][16], int n, int hh) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * st + 2 * i + hh;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[(32 * dt + n) * VP + key], p[st][i],
                                                       o[dt], 0, 0, 0);
      }
  }
};

// Global -> register -> LDS staging of one key tile (64 K rows) and one V^T
// tile (d rows x 64 keys), 16-byte vectors.
template <class Pol> struct Stage {
  using T = typename Pol::T;
  static constexpr int N = 16 / sizeof(T);
  static constexpr int KVPR = kHeadDim / N;                // vectors per K row
  static constexpr int VVPR = kKeyTile / N;                // vectors per V^T row
  static constexpr int KV = kKeyTile * KVPR / 256;
  static constexpr int VV = kHeadDim * VVPR / 256;
  uint4 kr[KV], vr[VV];
  __device__ void load(const T *kbase, int64_t kstride, int64_t row0, int64_t rows_total,
                       const T *vtile, int64_t vstride) {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int64_t row = row0 + c / KVPR;
      kr[i] = row < rows_total ? *(const uint4 *)(kbase + row * kstride + (c % KVPR) * N)
                               : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VV; ++i) {
      const int c = threadIdx.x + 256 * i;
      vr[i] = *(const uint4 *)(vtile + (int64_t)(c / VVPR) * vstride + (c % VVPR) * N);
    }
  }
  __device__ void store(T *Ks, T *Vs) const {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int c = threadIdx.x + 256 * i;
      *(uint4 *)(Ks + (c / KVPR) * Pol::KP + (c % KVPR) * N) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VV; ++i) {
      const int c = threadIdx.x + 256 * i;
      *(uint4 *)(Vs + (c / VVPR) * Pol::VP + (c % VVPR) * N) = vr[i];
    }
  }
};

enum { MODE_HIST = 0, MODE_DIAG = 1, MODE_DENSE = 2 };

struct AttnArgs {
  const void *q, *k, *vt;
  int64_t T;
  int Hq, Hkv, G, B, topk;
  float scale_log2;
  int g0, h0, Hp;
  int64_t NBb;
  const int4 *info;
  // historical blocks
  const uint32_t *tile_off, *tile_bin, *bin_off, *items;
  int64_t nbins;
  // partial outputs (MoBA) or final outputs (dense)
  float *part_o, *part_lse;
  const int32_t *cu, *blk_first64;
  int S, nqt;
  int64_t NBb64;
  void *out;
  float *lse;
};

template <typename TO> __device__ __forceinline__ void store4(TO *p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float *p, float a, float b, float c, float d) {
  *(float4 *)p = make_float4(a, b, c, d);
}
template <> __device__ __forceinline__ void store4<__bf16>(__bf16 *p, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *(bf16x4 *)p = v;
}

template <class Pol, int MODE>
__global__ __launch_bounds__(256, Pol::kOcc) void attn_kernel(const AttnArgs a) {
  using T = typename Pol::T;
  constexpr int KS = kKeyTile * Pol::KP, VS = kHeadDim * Pol::VP;
  __shared__ __attribute__((aligned(16))) T lds[2 * (KS + VS)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int r = wave * 32 + n;  // this lane's query row inside the tile

  const T *q = (const T *)a.q;
  int g, nkt, nrows, hq;
  int64_t t, kbeg, slot = 0, vstep, vstride;
  int qpos = 0, qfirst = 0;     // causal modes: positions relative to kbeg
  const T *vt0;

  if (MODE == MODE_HIST) {
    // XCD-aware order: workgroup i runs on XCD i % 8; give every XCD a
    // contiguous run of tiles so the tiles of one block share its L2.
    const uint32_t ntiles = a.tile_off[a.nbins];
    const uint32_t per = (ntiles + 7) >> 3;
    const uint32_t jj = blockIdx.x >> 3;
    if (jj >= per) return;
    const uint32_t tile = (blockIdx.x & 7) * per + jj;
    if (tile >= ntiles) return;
    const uint32_t bin = a.tile_bin[tile];
    const int p = (int)(bin / a.NBb);
    const int64_t gb = bin % a.NBb;
    const int4 bi = a.info[gb];
    const uint32_t r0 = a.bin_off[bin] + (tile - a.tile_off[bin]) * kRowTile;
    nrows = (int)min((uint32_t)kRowTile, a.bin_off[bin + 1] - r0);
    slot = a.items[r0 + (r < nrows ? r : 0)];
    const int64_t th = slot / a.topk;
    t = th / a.Hp;
    hq = a.h0 + (int)(th % a.Hp);
    g = a.g0 + p;
    kbeg = bi.y;
    nkt = a.B / kKeyTile;
    vt0 = (const T *)a.vt + ((int64_t)p * a.NBb + gb) * kHeadDim * a.B;
    vstep = kKeyTile;
    vstride = a.B;
  } else if (MODE == MODE_DIAG) {
    const int nq = (a.B + kRowTile - 1) / kRowTile;
    const int qt = nq - 1 - (int)(blockIdx.x / a.NBb);  // most keys first
    const int64_t gb = blockIdx.x % a.NBb;
    const int4 bi = a.info[gb];
    if (bi.x < 0 || qt * kRowTile >= bi.z) return;
    const int hl = blockIdx.y;
    hq = a.h0 + hl;
    g = hq / a.G;
    nrows = min(kRowTile, bi.z - qt * kRowTile);
    qfirst = qt * kRowTile;
    qpos = qfirst + r;
    t = bi.y + qfirst + (r < nrows ? r : 0);
    const int kend = min(bi.z, qfirst + kRowTile);
    nkt = (kend + kKeyTile - 1) / kKeyTile;
    kbeg = bi.y;
    const int nsel = min(a.topk, bi.w + 1);  // own block is the last chosen slot
    slot = (t * a.Hp + hl) * a.topk + nsel - 1;
    vt0 = (const T *)a.vt + ((int64_t)(g - a.g0) * a.NBb + gb) * kHeadDim * a.B;
    vstep = kKeyTile;
    vstride = a.B;
  } else {  // MODE_DENSE
    const int qt = a.nqt - 1 - (int)(blockIdx.x / a.S);
    const int s = blockIdx.x % a.S;
    const int L = a.cu[s + 1] - a.cu[s];
    if (qt * kRowTile >= L) return;
    hq = blockIdx.y;
    g = hq / a.G;
    nrows = min(kRowTile, L - qt * kRowTile);
    qfirst = qt * kRowTile;
    qpos = qfirst + r;
    t = a.cu[s] + qfirst + (r < nrows ? r : 0);
    const int kend = min(L, qfirst + kRowTile);
    nkt = (kend + kKeyTile - 1) / kKeyTile;
    kbeg = a.cu[s];
    vt0 = (const T *)a.vt + ((int64_t)g * a.NBb64 + a.blk_first64[s]) * kHeadDim * kKeyTile;
    vstep = (int64_t)kHeadDim * kKeyTile;
    vstride = kKeyTile;
  }
  const bool valid = r < nrows;

  typename Pol::Q qr;
  Pol::load_q(qr, q + (t * a.Hq + hq) * kHeadDim, hh);

  const T *kbase = (const T *)a.k + (int64_t)g * kHeadDim;
  const int64_t kstride = (int64_t)a.Hkv * kHeadDim;
  floatx16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  Stage<Pol> stage;
  stage.load(kbase, kstride, kbeg, a.T, vt0, vstride);
  stage.store(lds, lds + KS);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const T *Ks = lds + (kt & 1) * (KS + VS);
    const T *Vs = Ks + KS;
    if (kt + 1 < nkt)
      stage.load(kbase, kstride, kbeg + (int64_t)(kt + 1) * kKeyTile, a.T, vt0 + (kt + 1) * vstep,
                 vstride);

    float sv[2][16];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      floatx16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      Pol::qk(acc, Ks, st, qr, n, hh);
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[st][i] = acc[i] * a.scale_log2;
    }
    if (MODE != MODE_HIST && kt * kKeyTile + kKeyTile - 1 > qfirst) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * kKeyTile + Pol::key_of(st, i, hh) > qpos) sv[st][i] = -INFINITY;
    }
    float mt = sv[0][0];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sv[st][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt);
    const float mref = mnew == -INFINITY ? 0.f : mnew;  // no row here is fully masked; stay finite
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[st][i] = __builtin_amdgcn_exp2f(sv[st][i] - mref);
        rs += sv[st][i];
      }
    l += rs;
    Pol::pv(o, Vs, sv, n, hh);

    if (kt + 1 < nkt) {
      T *Kn = lds + ((kt + 1) & 1) * (KS + VS);
      stage.store(Kn, Kn + KS);
    }
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.f / lt;
  const float lse = (m + __log2f(lt)) * kLn2;
  if (!valid) return;
  if (MODE != MODE_DENSE) {
    float *dst = a.part_o + slot * kHeadDim + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa)
        store4<float>(dst + 32 * dt + 8 * aa, o[dt][4 * aa] * inv, o[dt][4 * aa + 1] * inv,
                      o[dt][4 * aa + 2] * inv, o[dt][4 * aa + 3] * inv);
    if (hh == 0) a.part_lse[slot] = lse;
  } else {
    T *dst = (T *)a.out + (t * a.Hq + hq) * kHeadDim + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa)
        store4<T>(dst + 32 * dt + 8 * aa, o[dt][4 * aa] * inv, o[dt][4 * aa + 1] * inv,
                  o[dt][4 * aa + 2] * inv, o[dt][4 * aa + 3] * inv);
    if (hh == 0 && a.lse) a.lse[(int64_t)hq * a.T + t] = lse;
  }
}

AttnArgs base_args(const Problem &pb, const Work &w, const void *q, const void *k, int g0) {
  AttnArgs a{};
  a.q = q; a.k = k; a.vt = w.vt;
  a.T = pb.T; a.Hq = pb.Hq; a.Hkv = pb.Hkv; a.G = pb.G; a.B = pb.B; a.topk = pb.k;
  a.scale_log2 = pb.scale * kLog2e;
  a.g0 = g0; a.h0 = g0 * pb.G; a.Hp = pb.Hp;
  a.NBb = pb.NBb; a.info = w.blk_info;
  a.tile_off = w.tile_off; a.tile_bin = w.tile_bin; a.bin_off = w.bin_off; a.items = w.items;
  a.nbins = (int64_t)pb.P * pb.NBb;
  a.part_o = w.part_o; a.part_lse = w.part_lse;
  return a;
}

template <int MODE>
hipError_t launch_mode(bool bf16, dim3 grid, const AttnArgs &a, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (bf16)
    attn_kernel<PolBf16, MODE><<<grid, 256, 0, s>>>(a);
  else
    attn_kernel<PolF32, MODE><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_diag(const Problem &pb, const Work &w, const void *q, const void *k, int g0,
                            hipStream_t s) {
  const AttnArgs a = base_args(pb, w, q, k, g0);
  const int nq = (pb.B + kRowTile - 1) / kRowTile;
  return launch_mode<MODE_DIAG>(pb.bf16, dim3((unsigned)(pb.NBb * nq), (unsigned)pb.Hp), a, s);
}

hipError_t launch_attn_hist(const Problem &pb, const Work &w, const void *q, const void *k, int g0,
                            hipStream_t s) {
  if (pb.k <= 1) return hipSuccess;
  const AttnArgs a = base_args(pb, w, q, k, g0);
  const int64_t grid = (w.max_tiles + 7) / 8 * 8;
  return launch_mode<MODE_HIST>(pb.bf16, dim3((unsigned)grid), a, s);
}

hipError_t launch_dense(const void *q, const void *k, const void *vt, const int32_t *cu,
                        const int32_t *blk_first64, int bf16, int64_t T, int S, int maxlen, int Hq,
                        int Hkv, int64_t NBb64, float scale, void *out, float *lse,
                        hipStream_t s) {
  AttnArgs a{};
  a.q = q; a.k = k; a.vt = vt;
  a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.scale_log2 = scale * kLog2e;
  a.cu = cu; a.blk_first64 = blk_first64; a.S = S;
  a.nqt = (maxlen + kRowTile - 1) / kRowTile;
  a.NBb64 = NBb64;
  a.out = out; a.lse = lse;
  return launch_mode<MODE_DENSE>(bf16 != 0, dim3((unsigned)((int64_t)S * a.nqt), (unsigned)Hq),
                                 a, s);
}

}  // namespace moba
