// Block attention on the matrix cores (MFMA), flash-style online softmax.
//
// MoBA summary page (paper-graph-ui), section 3.4 "Implementation", step 3:
// attention of each query over its own block with a causal mask, and over each
// earlier block it chose without one, each producing a partial output and its
// log-sum-exp; "Causality Enforcement" mechanism 2 for the own block. The same
// tile engine runs dense causal attention ("Standard Attention Baseline").
//
// Workgroup: waves of 32 query rows of one kv head (bf16: 8 waves, 256 rows;
// fp32: 4 waves, 128 rows). Keys stream through LDS in tiles of 64 (double
// buffered). Each wave computes the
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

#include <type_traits>
#include <utility>

#include "moba_internal.h"

namespace moba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int64_t min_i64(int64_t a, int64_t b) { return a < b ? a : b; }

// bf16 inputs: v_mfma_f32_32x32x16_bf16 (A: 32x16, B: 16x32, fp32 accumulate).
// Lane l holds A[m = l%32][k = 8*(l/32) .. +7] and B[k = 8*(l/32) .. +7][n = l%32];
// accumulator i of lane l is C[8*(i/4) + 4*(l/32) + i%4][l%32].
struct PolBf16 {
  using T = __bf16;
  static constexpr int kRows = kRowsBf16;        // query rows per workgroup
  static constexpr int kThreads = 2 * kRows;     // waves of 32 rows
  static constexpr int kOcc = 1;                 // workgroups per CU (8 waves)
  static constexpr int kStages = 2;              // K and V^T tile buffers in LDS (4 spills VGPRs)
  static constexpr int kLoadAhead = 1;           // tiles between a load's issue and its use
  static constexpr int KP = kHeadDim + 8;  // LDS pitch of a key row (272 B)
  static constexpr int VP = kKeyTile + 8;  // LDS pitch of a V^T row (144 B)
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

// Own-block attention, bf16: half the rows per workgroup and two workgroups
// per CU. The own block's runs are short (1 to B/64 key tiles, the first
// ones among them), so the first loads of a run (query rows, first key and
// value tiles) are a large share of its time; the other workgroup on the CU
// computes meanwhile.
struct PolBf16Own : PolBf16 {
  static constexpr int kRows = kRowTile;
  static constexpr int kThreads = 2 * kRows;
  static constexpr int kOcc = 2;
};

// fp32 inputs: v_mfma_f32_32x32x2f32 (lane l holds A[l%32][l/32], B[l/32][l%32]).
struct PolF32 {
  using T = float;
  static constexpr int kRows = kRowsF32;         // query rows per workgroup
  static constexpr int kThreads = 2 * kRows;     // waves of 32 rows
  static constexpr int kOcc = 1;
  static constexpr int KP = kHeadDim + 4;  // 528 B
  static constexpr int VP = kKeyTile + 4;  // 272 B
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
// tile (d rows x 64 keys), 16-byte vectors. Per-thread offsets are computed
// once; each tile only moves a uniform base pointer. CHECK guards K rows past
// the end of the tensor (own-block and dense tiles can run past it).
template <class Pol, bool CHECK> struct Stage {
  using T = typename Pol::T;
  static constexpr int N = 16 / sizeof(T);
  static constexpr int KVPR = kHeadDim / N;                // vectors per K row
  static constexpr int VVPR = kKeyTile / N;                // vectors per V^T row
  static constexpr int NT = Pol::kThreads;
  static constexpr int KV = kKeyTile * KVPR / NT;
  static constexpr int VV = kHeadDim * VVPR / NT;
  uint4 kr[KV], vr[VV];
  uint32_t koff[KV], voff[VV];
  __device__ void init(uint32_t kstride, uint32_t vstride) {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int c = threadIdx.x + NT * i;
      koff[i] = (uint32_t)(c / KVPR) * kstride + (c % KVPR) * N;
    }
#pragma unroll
    for (int i = 0; i < VV; ++i) {
      const int c = threadIdx.x + NT * i;
      voff[i] = (uint32_t)(c / VVPR) * vstride + (c % VVPR) * N;
    }
  }
  // krows: tile rows that exist in the tensor (only read when CHECK)
  __device__ void load(const T *ktile, int krows, const T *vtile) {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int row = (threadIdx.x + NT * i) / KVPR;
      kr[i] = (!CHECK || row < krows) ? *(const uint4 *)(ktile + koff[i]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VV; ++i) vr[i] = *(const uint4 *)(vtile + voff[i]);
  }
  __device__ void store(T *Ks, T *Vs) const {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int c = threadIdx.x + NT * i;
      *(uint4 *)(Ks + (c / KVPR) * Pol::KP + (c % KVPR) * N) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VV; ++i) {
      const int c = threadIdx.x + NT * i;
      *(uint4 *)(Vs + (c / VVPR) * Pol::VP + (c % VVPR) * N) = vr[i];
    }
  }
};

// The reference max moves only when a tile's max exceeds it by more than this
// (log2 units), so probabilities stay <= 2^8 and the rescale of the output
// accumulators is rare. The result is exact: l uses the same reference.
constexpr float kRescaleSlack = 8.0f;
// A run of tiles whose every score is within this distance (log2 units) of
// the first tile's max goes without the other tiles' maxima: its
// probabilities stay <= 2^64, far inside the fp32 and bf16 ranges, and the
// result is the same (l uses the same reference).
constexpr float kBoundSlack = 64.0f;

// MODE_OWN_MERGE: the own block, merged with the earlier blocks' partial
// results into the final output (bf16).
enum { MODE_HIST = 0, MODE_DIAG = 1, MODE_DENSE = 2, MODE_OWN_MERGE = 3 };

struct AttnArgs {
  const void *q, *k, *vt;
  const float *knorm;  // largest key norm of every block, laid out like vt's blocks
  RowHead qs, ks, os;  // strides of q, k and (dense) out
  int64_t T;
  int Hq, Hkv, G, B, topk;
  float scale_log2;
  int g0, h0, Hp;
  int64_t NBb;
  const int4 *info;
  // historical blocks
  const uint32_t *tile_off, *bin_off, *items;
  const int4 *tile_rec;
  int64_t nbins;
  // partial outputs (MoBA) or final outputs (dense, own block merged)
  void *part_o;
  float *part_lse;
  // dense: 64-row key tiles of each sequence (first tile index) and the
  // query tiles {sequence, first row, rows, tile index in the sequence}
  const int32_t *blk_first64;
  const int4 *qtiles;
  int64_t NBq, NBb64;
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

// Causal mask of one 64-key tile (own block / dense): key > query -> -inf.
template <class Pol>
__device__ __forceinline__ void mask_tile(float (&sv)[2][16], int kt, int qpos, int hh) {
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (kt * kKeyTile + Pol::key_of(st, i, hh) > qpos) sv[st][i] = -INFINITY;
}

// Scaled max of one tile of raw scores (the scale is positive, so it commutes
// with the max); both lane halves of a query get the same value.
__device__ __forceinline__ float tile_max(const float (&sv)[2][16], float c2) {
  float mt = sv[0][0];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sv[st][i]);
  return fmaxf(mt, __shfl_xor(mt, 32)) * c2;
}

// Lazy move of the reference max given a tile's scaled max mt (rare rescale
// of O and l). Returns -m (finite) for the exponent of this tile.
__device__ __forceinline__ float move_max(float mt, float &m, float &l, floatx16 (&o)[4]) {
  const bool moved = mt > m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(moved)) {
    const float alpha = moved ? __builtin_amdgcn_exp2f(m - mt) : 1.f;
    m = moved ? mt : m;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
  }
  return m == -INFINITY ? 0.f : -m;  // finite even if nothing was visible yet
}

// Online softmax, first half: tile max, lazy move of the reference max.
__device__ __forceinline__ float softmax_rescale(const float (&sv)[2][16], float c2, float &m,
                                                 float &l, floatx16 (&o)[4]) {
  return move_max(tile_max(sv, c2), m, l, o);
}

// Online-softmax update for one tile of raw scores (q.k, unscaled): leaves the
// probabilities exp2(c2*s - m) in sv and adds them to l (fp32 path).
__device__ __forceinline__ void softmax_step(float (&sv)[2][16], float c2, float &m, float &l,
                                             floatx16 (&o)[4]) {
  const float nm = softmax_rescale(sv, c2, m, l, o);
  float rs = 0.f;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[st][i] = __builtin_amdgcn_exp2f(fmaf(sv[st][i], c2, nm));
      rs += sv[st][i];
    }
  l += rs;
}

// ---- bf16 tile loop: direct global->LDS loads, swizzled LDS, QK of the next
// tile issued before the softmax of the current one.
//
// LDS: NS K buffers (64 rows x 16 chunks of 16 B) then NS V^T buffers (128
// rows x 8 chunks), 16 KiB each. Chunk c of K row r is stored at position
// c ^ (r & 15), chunk c of V^T row r at c ^ ((r >> 1) & 7): the 16 lanes that
// read one chunk column of 16 consecutive rows then hit 16 different 16-byte
// bank groups. A direct load writes 16 B per lane at LDS base + 16 * lane, so
// each lane fetches the global chunk that belongs at its fixed LDS position.
template <int NS> struct Direct {
  static constexpr int BUF = 16384;
  static constexpr int K(int i) { return i * BUF; }
  static constexpr int V(int i) { return (NS + i) * BUF; }
  static constexpr int BYTES = 2 * NS * BUF;
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;
// Word 3 of a raw buffer descriptor on gfx9-family parts (gfx950 included).
constexpr int kBufferWord3 = 0x00020000;

// Raw buffer descriptor from wave-uniform values (kept in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, int64_t bytes) {
  const uint64_t v = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)min_i64(bytes, 0x7fffffff));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, n,
                                           kBufferWord3);
}

// Wait until at most N vector memory loads of this wave are outstanding.
// (Also waits for every LDS and scalar-cache access of the wave. Written
// with the builtin so the compiler knows what is still pending afterwards.)
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);  // expcnt(7) lgkmcnt(0)
}
// Same with N = c * PER for a wave-uniform c in [0, MAXC].
template <int PER, int MAXC> __device__ __forceinline__ void wait_vm_groups(int c) {
  if constexpr (MAXC == 0) {
    wait_vm<0>();
  } else {
    if (c >= MAXC) wait_vm<MAXC * PER>();
    else wait_vm_groups<PER, MAXC - 1>(c);
  }
}

// Tile pipeline: key tile kt lives in K buffer kt % NS and V^T buffer
// kt % NS. Body kt computes the scores of tile kt + 1 and the exp and P V of
// tile kt, and issues the loads of V^T tile kt + A and K tile kt + A + 1; at
// its end each wave waits for its loads that the next body reads (V^T tile
// kt + 1, K tile kt + 2), then the workgroup synchronises. A buffer is
// refilled only after the barrier that ends the last body reading it, which
// needs NS >= A + 1.

// c2 |q| for the query row a lane holds (each lane half holds half of it).
__device__ __forceinline__ float q_bound(const PolBf16::Q &qr, float c2) {
  float ss = 0.f;
#pragma unroll
  for (int kk = 0; kk < kHeadDim / 16; ++kk)
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf((float)qr.v[kk][j], (float)qr.v[kk][j], ss);
  ss += __shfl_xor(ss, 32);
  return c2 * sqrtf(ss);
}

// kn_run: the largest key norm over the run's tiles; qnc2 = c2 |q| of this
// lane's query, so that qnc2 * kn_run bounds every scaled score of the run.
// pre() runs after the prologue's loads are issued and returns how many
// loads it issued itself (0 or NPRE per lane); those may stay in flight
// until the end of the first body.
template <int MODE, int NW, int NS, int A, int NPRE = 0, class Pre = int (*)()>
__device__ __forceinline__ void tiles_direct(char *lds, const __bf16 *ktile0, uint32_t kstride,
                                             int64_t rows_after, const __bf16 *vt0, int64_t vstep,
                                             uint32_t vstride, int nkt, const PolBf16::Q &qr,
                                             int qfirst, int qpos, float c2, float kn_run,
                                             float qnc2, floatx16 (&o)[4], float &m, float &l,
                                             Pre &&pre = nullptr) {
  constexpr bool CAUSAL = MODE != MODE_HIST;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int n = lane & 31, hh = lane >> 5;
  // direct-load sources (byte offsets from the tile base): each tile is 16
  // regions of 1 KiB (K: 4 rows, V^T: 8 rows per region); wave w fills regions
  // w*LPW .. w*LPW+LPW-1 of both, at buffer + LPW KiB * w (a wave-uniform
  // address, so M0 is set by scalar code)
  constexpr int LPW = 16 / NW;  // loads per wave per tile and tensor
  uint32_t kso[LPW], vso[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int region = wave * LPW + j;
    const int krow = region * 4 + (lane >> 4);
    kso[j] = (uint32_t)krow * kstride * 2u + (uint32_t)(((lane & 15) ^ (krow & 15)) * 16);
    const int vrow = region * 8 + (lane >> 3);
    vso[j] = (uint32_t)vrow * vstride * 2u + (uint32_t)(((lane & 7) ^ ((vrow >> 1) & 7)) * 16);
  }
  char *const lds_w = lds + wave * LPW * 1024;
  // LDS read offsets (bytes) of this lane's MFMA A operands
  const int pr = PolBf16::perm(n);
  uint32_t krd[8], vrd[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) krd[kk] = pr * 256 + (((2 * kk + hh) ^ (pr & 15)) * 16);
#pragma unroll
  for (int c = 0; c < 4; ++c) vrd[c] = n * 128 + (((2 * c + hh) ^ ((n >> 1) & 7)) * 16);

  // Buffer descriptors over this workgroup's keys and values: loads take a
  // constant per-lane offset plus a scalar per-tile offset, and offsets past
  // num_records read zeros (K rows past the end of the tensor; those keys lie
  // beyond every query of the tile and are masked anyway).
  const __amdgpu_buffer_rsrc_t krs = uniform_rsrc(ktile0, rows_after * kstride * 2);
  const __amdgpu_buffer_rsrc_t vrs =
      uniform_rsrc(vt0, (int64_t)(nkt - 1) * vstep * 2 + (int64_t)kHeadDim * vstride * 2);
  auto issue_k = [&](int kt, int buf) {
    const uint32_t soff = (uint32_t)kt * kKeyTile * kstride * 2u;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(lds_w + buf + j * 1024), 16, kso[j],
                                               soff, 0, 0);
  };
  auto issue_v = [&](int kt, int buf) {
    const uint32_t soff = (uint32_t)(kt * vstep) * 2u;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(lds_w + buf + j * 1024), 16, vso[j],
                                               soff, 0, 0);
  };
  auto qk = [&](floatx16 (&acc)[2], int kbuf) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[st][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 av = *(const bf16x8 *)(lds + kbuf + st * 8192 + krd[kk]);
        acc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qr.v[kk], acc[st], 0, 0, 0);
      }
    }
  };
  // exp2 of one tile's scores, chunk by chunk straight into the P V product;
  // the row sum adds the fp32 probabilities (lse keeps fp32 accuracy), as a
  // tree per chunk of 8.
  auto exp_pv = [&](const floatx16 (&sc)[2], float nm, int vbuf) {
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 b;
        float pj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pj[j] = __builtin_amdgcn_exp2f(fmaf(sc[st][8 * c + j], c2, nm));
          b[j] = (__bf16)pj[j];
        }
        rs += ((pj[0] + pj[1]) + (pj[2] + pj[3])) + ((pj[4] + pj[5]) + (pj[6] + pj[7]));
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 av = *(const bf16x8 *)(lds + vbuf + dt * 4096 + vrd[2 * st + c]);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, o[dt], 0, 0, 0);
        }
      }
    l += rs;
    // l is next needed in the next body; keep its sum in this body, among
    // the MFMAs (it would otherwise be sunk past the workgroup barrier)
    asm volatile("" : "+v"(l));
  };
  auto mask = [&](floatx16 (&sc)[2], int kt) {
    if (CAUSAL && kt * kKeyTile + kKeyTile - 1 > qfirst) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * kKeyTile + PolBf16::key_of(st, i, hh) > qpos) sc[st][i] = -INFINITY;
    }
  };
  auto smax = [&](const floatx16 (&sc)[2]) {
    float sv[2][16];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[st][i] = sc[st][i];
    return tile_max(sv, c2);
  };
  // set after the first tile: whether this lane's row needs every tile's max
  // (row_max) and whether any row of the wave does (exact_max)
  bool row_max = true, exact_max = true;
  static_assert((NS == 2 || NS == 4) && NS >= A + 1 && A >= 1, "pipeline shape");
  using D = Direct<NS>;
  // Loads issued by body j (j < 0: the prologue's share of the pipeline).
  auto loads_of = [&](int j) { return (j + A < nkt ? 1 : 0) + (j + A + 1 < nkt ? 1 : 0); };
  // One tile: tile kt's raw scores are in cur (masked already for kt = 0);
  // mt_cur is the first tile's scaled max for kt = 0 and -inf after it. A
  // later tile's causal mask and, in waves with a row that needs it, its max
  // are applied at the start of its body, outside the scheduled region. With
  // HAS_NEXT the next tile's scores are produced in the same branch-free
  // region as this tile's exp and P V.
  // PH = kt % NS selects the buffers at compile time.
  auto body = [&](auto has_next, auto phase, int kt, floatx16 (&cur)[2],
                  floatx16 (&nxt)[2], float mt_cur, float &mt_nxt) {
    constexpr bool HAS_NEXT = decltype(has_next)::value;
    constexpr int PH = decltype(phase)::value;
    if (kt + A < nkt) issue_v(kt + A, D::V((PH + A) % NS));
    if (kt + A + 1 < nkt) issue_k(kt + A + 1, D::K((PH + A + 1) % NS));
    // the causal mask of a later tile, here rather than in the region: its
    // branch (taken only on the tiles that cross the diagonal) would split
    // the region and undo the interleave of the other tiles
    if (kt > 0) mask(cur, kt);
    // this tile's max: the first tile's comes from the prologue; later ones
    // are computed here only in waves with a row that needs them
    float mt = mt_cur;
    if (exact_max && kt > 0) {
      const float x = smax(cur);
      mt = row_max ? x : -INFINITY;
    }
    const float nm = move_max(mt, m, l, o);
    // ---- branch-free region
    if (HAS_NEXT) qk(nxt, D::K((PH + 1) % NS));
    exp_pv(cur, nm, D::V(PH));
    // schedule: LDS operand reads run 4 MFMAs ahead; the VALU work is spread
    // evenly between all MFMAs of the region
    constexpr int kAhead = 4;
    constexpr int nmfma = HAS_NEXT ? 32 : 16;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < nmfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kAhead < nmfma) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, HAS_NEXT ? 4 : 6, 0);
    }
    if (HAS_NEXT) mt_nxt = -INFINITY;
    // loads issued by bodies kt + 2 - A .. kt may stay in flight
    int later = 0;
#pragma unroll
    for (int j = 2 - A; j <= 0; ++j) later += loads_of(kt + j);
    wait_vm_groups<LPW, 2 * (A - 1)>(later);
    __syncthreads();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using std::integral_constant;

  issue_k(0, D::K(0));
  if (nkt > 1) issue_k(1, D::K(1));
  issue_v(0, D::V(0));
  int npre = 0;
  if constexpr (NPRE > 0) npre = pre();
  if (NPRE > 0 && npre) wait_vm<NPRE>();  // only pre()'s loads may be in flight
  else wait_vm<0>();
  __syncthreads();
  // the prologue's share: V^T tiles 1 .. A-1 and K tiles 2 .. A
#pragma unroll
  for (int i = 1; i < A; ++i) {
    if (i < nkt) issue_v(i, D::V(i % NS));
    if (i + 1 < nkt) issue_k(i + 1, D::K((i + 1) % NS));
  }
  floatx16 sa[2], sb[2];
  qk(sa, D::K(0));
  mask(sa, 0);
  float ma = smax(sa), mb = 0.f;
  // Every score of the row's run is at most qnc2 * kn_run; within
  // kBoundSlack of the first tile's max the row keeps that max as its
  // reference. Otherwise each tile's max moves the reference lazily. The
  // choice depends on the row alone (both lanes of a row agree), so a row's
  // result does not depend on the other rows of its wave; the wave computes
  // tile maxima only when one of its rows needs them.
  row_max = qnc2 * kn_run > ma + kBoundSlack;
  exact_max = __builtin_amdgcn_ballot_w64(row_max) != 0;
  // body 0 refills K buffer 0 when A + 1 == NS: every wave must have read it
  if ((A + 1) % NS == 0) __syncthreads();
  // even bodies hold the current tile's scores in sa, odd ones in sb
  auto run = [&](auto has_next, auto phase, int kt) {
    constexpr int PH = decltype(phase)::value;
    if constexpr (PH % 2 == 0) body(has_next, phase, kt, sa, sb, ma, mb);
    else body(has_next, phase, kt, sb, sa, mb, ma);
  };
  using P0 = integral_constant<int, 0>;
  using P1 = integral_constant<int, 1>;
  using P2 = integral_constant<int, 2>;
  using P3 = integral_constant<int, 3>;
  auto full = [&](int kt) {
    run(T_{}, P0{}, kt);
    run(T_{}, P1{}, kt + 1);
    if constexpr (NS > 2) {
      run(T_{}, P2{}, kt + 2);
      run(T_{}, P3{}, kt + 3);
    }
  };
  int kt = 0;
  for (; kt + NS < nkt; kt += NS) full(kt);
  // 1 .. NS tiles left, kt % NS == 0
  const int left = nkt - kt;
  if constexpr (NS > 2) {
    if (left == 4) {
      run(T_{}, P0{}, kt);
      run(T_{}, P1{}, kt + 1);
      run(T_{}, P2{}, kt + 2);
      run(F_{}, P3{}, kt + 3);
      return;
    }
    if (left == 3) {
      run(T_{}, P0{}, kt);
      run(T_{}, P1{}, kt + 1);
      run(F_{}, P2{}, kt + 2);
      return;
    }
  }
  if (left == 2) {
    run(T_{}, P0{}, kt);
    run(F_{}, P1{}, kt + 1);
  } else {
    run(F_{}, P0{}, kt);
  }
}

// ---- generic tile loop (fp32 path): register-staged loads into padded LDS.
template <class Pol, int MODE>
__device__ __forceinline__ void tiles_staged(typename Pol::T *lds, const typename Pol::T *ktile,
                                             uint32_t kstride, int64_t rows_after,
                                             const typename Pol::T *vt0, int64_t vstep,
                                             uint32_t vstride, int nkt, const typename Pol::Q &qr,
                                             int qfirst, int qpos, float c2, floatx16 (&o)[4],
                                             float &m, float &l) {
  using T = typename Pol::T;
  constexpr int KS = kKeyTile * Pol::KP, VS = kHeadDim * Pol::VP;
  constexpr bool CHECK = MODE != MODE_HIST;  // earlier blocks are always whole and in range
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  Stage<Pol, CHECK> stage;
  stage.init(kstride, vstride);
  stage.load(ktile, (int)min_i64(rows_after, kKeyTile), vt0);
  stage.store(lds, lds + KS);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const T *Ks = lds + (kt & 1) * (KS + VS);
    const T *Vs = Ks + KS;
    if (kt + 1 < nkt) {
      const int64_t r0 = (int64_t)(kt + 1) * kKeyTile;
      stage.load(ktile + r0 * kstride, (int)min_i64(rows_after - r0, kKeyTile),
                 vt0 + (kt + 1) * vstep);
    }
    float sv[2][16];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      floatx16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      Pol::qk(acc, Ks, st, qr, n, hh);
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[st][i] = acc[i];
    }
    if (MODE != MODE_HIST && kt * kKeyTile + kKeyTile - 1 > qfirst) mask_tile<Pol>(sv, kt, qpos, hh);
    softmax_step(sv, c2, m, l, o);
    Pol::pv(o, Vs, sv, n, hh);
    if (kt + 1 < nkt) {
      T *Kn = lds + ((kt + 1) & 1) * (KS + VS);
      stage.store(Kn, Kn + KS);
    }
    __syncthreads();
  }
}

// The own block's results of a workgroup's rows, merged with the rows'
// earlier-block partial results (part_o / part_lse, written by the
// earlier-block attention of this pass) into out and lse, with the
// arithmetic of merge_kernel in the same order: the maximum lse,
// exp(lse - max) summed per slot group s % 16 and the 16 group sums pairwise
// (i, i + 8), (i, i + 4), (i, i + 2), (i, i + 1), then the weighted parts
// added in ascending slot order with the own block's last. The own block's
// part enters rounded to bf16, as it would be read back from part_o, so the
// result has the bits of the own-block kernel followed by merge_kernel.
// Called by every lane after the tile loop's last barrier (LDS is free).
// Phase A: each lane of row n (two per row, in the MFMA layout: lane half hh
// holds the 4-column chunks 4 hh + 8 j) computes the row's weights and puts
// them, the row's lse and its rounded own part in the wave's LDS area.
// Phase B: 16 lanes per row, lane j holding columns 8 j .. 8 j + 7 of rows
// g, g + 4, ..., g + 28 (g = lane / 16), read the partial rows 16 bytes per
// lane, as merge_kernel does, and write out.
struct MergeLds {
  static constexpr int OWN = 0;        // 32 rows x 256 B: the own part, bf16
  static constexpr int W = 8192;       // 32 rows x 16 weights of the first 16 slots
  static constexpr int L = W + 2048;   // 32 rows: the merged lse
  static constexpr int WO = L + 128;   // 32 rows: the own part's weight
  static constexpr int WAVE = 16384;   // bytes per wave
};
__device__ __forceinline__ void merge_own(const AttnArgs &a, char *lds, const floatx16 (&o)[4],
                                          float inv, float lse_own, int64_t t0, int wave_row0,
                                          int nrows, int hq, int hl, int nsel) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  constexpr int kBatch = 2;  // slots in flight per lane (8 rows each)
  const int lane = threadIdx.x & 63;
  const int nh = nsel - 1;   // earlier-block slots
  char *const base = lds + (threadIdx.x >> 6) * MergeLds::WAVE;
  auto slot0_of = [&](int row) { return ((t0 + row) * a.Hp + hl) * (int64_t)a.topk; };
  {  // phase A
    const int n = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[dt][4 * aa + e] * inv);
        *(bf16x4 *)(base + MergeLds::OWN + n * 256 + (32 * dt + 8 * aa + 4 * hh) * 2) = v;
      }
    if (wave_row0 + n < nrows) {
      const float *pl = a.part_lse + slot0_of(wave_row0 + n);
      float x16[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) x16[u] = u < nh ? pl[u] : u == nh ? lse_own : -INFINITY;
      auto x_of = [&](int sl) { return sl < nh ? pl[sl] : sl == nh ? lse_own : -INFINITY; };
      float m = -INFINITY;
#pragma unroll
      for (int u = 0; u < 16; ++u) m = fmaxf(m, x16[u]);
      for (int sl = 16; sl < nsel; ++sl) m = fmaxf(m, x_of(sl));
      float su[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        su[u] = x16[u] > -INFINITY ? __builtin_amdgcn_exp2f((x16[u] - m) * kLog2e) : 0.f;
      for (int i0 = 16; i0 < nsel; i0 += 16) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float x = x_of(i0 + u);
          if (x > -INFINITY) su[u] += __builtin_amdgcn_exp2f((x - m) * kLog2e);
        }
      }
#pragma unroll
      for (int w = 8; w > 0; w >>= 1)
#pragma unroll
        for (int u = 0; u < w; ++u) su[u] += su[u + w];
      const float L = m + logf(su[0]);
      if (hh == 0) {
        float wt[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          wt[u] = u < nh && x16[u] > -INFINITY ? __builtin_amdgcn_exp2f((x16[u] - L) * kLog2e)
                                               : 0.f;
#pragma unroll
        for (int u = 0; u < 16; u += 4)
          *(float4 *)(base + MergeLds::W + n * 64 + 4 * u) =
              make_float4(wt[u], wt[u + 1], wt[u + 2], wt[u + 3]);
        *(float *)(base + MergeLds::L + 4 * n) = L;
        *(float *)(base + MergeLds::WO + 4 * n) = __builtin_amdgcn_exp2f((lse_own - L) * kLog2e);
      }
    }
  }
  __syncthreads();
  // phase B
  const int g = lane >> 4, j = lane & 15;
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.f;
  bool ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ok[i] = wave_row0 + g + 4 * i < nrows;
  const __bf16 *po = (const __bf16 *)a.part_o + 8 * j;
  auto weight = [&](int i, int sl) {
    const int n = g + 4 * i;
    if (sl < 16) return *(const float *)(base + MergeLds::W + n * 64 + 4 * sl);
    const float x = a.part_lse[slot0_of(wave_row0 + n) + sl];
    const float L = *(const float *)(base + MergeLds::L + 4 * n);
    return x > -INFINITY ? __builtin_amdgcn_exp2f((x - L) * kLog2e) : 0.f;
  };
  for (int sl = 0; sl < nh; sl += kBatch) {
    float w[kBatch][8];
    bf16x8 v[kBatch][8];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[b][i] = ok[i] && sl + b < nh ? weight(i, sl + b) : 0.f;
        v[b][i] = w[b][i] != 0.f
                      ? *(const bf16x8 *)(po + (slot0_of(wave_row0 + g + 4 * i) + sl + b) * kHeadDim)
                      : bf16x8{};
      }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = fmaf(w[b][i], (float)v[b][i][c], acc[i][c]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!ok[i]) continue;
    const int n = g + 4 * i;
    const float wo = *(const float *)(base + MergeLds::WO + 4 * n);
    const bf16x8 vo = *(const bf16x8 *)(base + MergeLds::OWN + n * 256 + 16 * j);
    bf16x8 res;
#pragma unroll
    for (int c = 0; c < 8; ++c) res[c] = (__bf16)fmaf(wo, (float)vo[c], acc[i][c]);
    const int64_t t = t0 + wave_row0 + n;
    *(bf16x8 *)((__bf16 *)a.out + t * a.os.t + hq * a.os.h + 8 * j) = res;
    if (j == 0 && a.lse) a.lse[(int64_t)hq * a.T + t] = *(const float *)(base + MergeLds::L + 4 * n);
  }
}

template <class Pol> struct LdsBytes {
  static constexpr int value = 2 * (kKeyTile * Pol::KP + kHeadDim * Pol::VP) * (int)sizeof(typename Pol::T);
};
// bf16: the tile buffers, then (earlier blocks) 8 KiB per wave where the
// next tile's query rows land
constexpr int kQStage = Direct<PolBf16::kStages>::BYTES;
template <> struct LdsBytes<PolBf16> {
  static constexpr int value = kQStage + PolBf16::kThreads / 64 * 8192;
};
template <> struct LdsBytes<PolBf16Own> {
  static constexpr int value = Direct<PolBf16Own::kStages>::BYTES;
};

// One work item of the attention kernel: bx stands for the workgroup index.
template <class Pol, int MODE>
__device__ __forceinline__ void attn_tile(const AttnArgs &a, char *lds, const uint32_t bx) {
  constexpr int ROWS = Pol::kRows;
  using T = typename Pol::T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int r = wave * 32 + n;  // this lane's query row inside the tile

  const T *q = (const T *)a.q;
  int g, nkt, nrows, hq;
  int64_t t, kbeg, slot = 0, vstep, vstride;
  int qpos = 0, qfirst = 0;     // causal modes: positions relative to kbeg
  const T *vt0;
  float kn_run;                 // largest key norm over the keys of the run
  int nsel = 0;                 // own block: the row's slots (the own block's is the last)

  if (MODE == MODE_HIST) {
    // (float32; bf16 runs hist_tile.) XCD-aware order: workgroup i runs on
    // XCD i % 8; give every XCD a contiguous run of tiles so the tiles of
    // one block share its L2.
    const uint32_t ntiles = a.tile_off[a.nbins];
    const uint32_t per = (ntiles + 7) >> 3;
    const uint32_t jj = bx >> 3;
    if (jj >= per) return;
    const uint32_t tile = (bx & 7) * per + jj;
    if (tile >= ntiles) return;
    const int4 rec = a.tile_rec[tile];
    const int p = (int)((uint32_t)rec.z / a.NBb);
    const int64_t gb = (uint32_t)rec.z % a.NBb;
    nrows = rec.y;
    slot = a.items[(uint32_t)rec.x + (r < nrows ? r : 0)];
    const int64_t th = slot / a.topk;
    t = th / a.Hp;
    hq = a.h0 + (int)(th % a.Hp);
    g = a.g0 + p;
    kbeg = rec.w;
    nkt = a.B / kKeyTile;
    vt0 = (const T *)a.vt + ((int64_t)p * a.NBb + gb) * kHeadDim * a.B;
    kn_run = a.knorm[(int64_t)p * a.NBb + gb];
    vstep = kKeyTile;
    vstride = a.B;
  } else if (MODE == MODE_DIAG || MODE == MODE_OWN_MERGE) {
    // Work item w runs over (kv head of the pass, block, query tile with the
    // most keys first, query head of the group). Workgroup i runs on XCD
    // i % 8 and every XCD takes a contiguous run of w, so the tiles that read
    // one block's keys and values run together and share that XCD's L2.
    const int nq = (a.B + ROWS - 1) / ROWS;
    const uint32_t total = (uint32_t)(a.Hp * a.NBb * nq);
    const uint32_t per = (total + 7) >> 3;
    const uint32_t jj = bx >> 3;
    if (jj >= per) return;
    const uint32_t wi = (bx & 7) * per + jj;
    if (wi >= total) return;
    uint32_t rest = wi / (uint32_t)a.G;
    const int qt = nq - 1 - (int)(rest % (uint32_t)nq);
    rest /= (uint32_t)nq;
    const int64_t gb = rest % (uint32_t)a.NBb;
    const int hl = (int)(rest / (uint32_t)a.NBb) * a.G + (int)(wi % (uint32_t)a.G);
    const int4 bi = a.info[gb];
    if (bi.x < 0 || qt * ROWS >= bi.z) return;
    hq = a.h0 + hl;
    g = hq / a.G;
    nrows = min(ROWS, bi.z - qt * ROWS);
    qfirst = qt * ROWS;
    qpos = qfirst + r;
    t = bi.y + qfirst + (r < nrows ? r : 0);
    const int kend = min(bi.z, qfirst + ROWS);
    nkt = (kend + kKeyTile - 1) / kKeyTile;
    kbeg = bi.y;
    nsel = min(a.topk, bi.w + 1);  // own block is the last chosen slot
    slot = (t * a.Hp + hl) * a.topk + nsel - 1;
    vt0 = (const T *)a.vt + ((int64_t)(g - a.g0) * a.NBb + gb) * kHeadDim * a.B;
    kn_run = a.knorm[(int64_t)(g - a.g0) * a.NBb + gb];  // the whole block: a valid bound
    vstep = kKeyTile;
    vstride = a.B;
  } else {  // MODE_DENSE
    // query tiles from the last (most keys) to the first
    const int4 bi = a.qtiles[a.NBq - 1 - (int64_t)bx];
    if (bi.x < 0) return;
    hq = blockIdx.y;
    g = hq / a.G;
    nrows = bi.z;
    qfirst = bi.w * ROWS;
    qpos = qfirst + r;
    t = bi.y + (r < nrows ? r : 0);
    nkt = (qfirst + nrows + kKeyTile - 1) / kKeyTile;  // keys up to the tile's last row
    kbeg = bi.y - qfirst;                              // the sequence's first row
    vt0 = (const T *)a.vt + ((int64_t)g * a.NBb64 + a.blk_first64[bi.x]) * kHeadDim * kKeyTile;
    // blocks of 64 keys here: the largest norm over the run's
    const float *kn = a.knorm + (int64_t)g * a.NBb64 + a.blk_first64[bi.x];
    kn_run = 0.f;
    for (int i = threadIdx.x & 63; i < nkt; i += 64) kn_run = fmaxf(kn_run, kn[i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kn_run = fmaxf(kn_run, __shfl_xor(kn_run, off));
    vstep = (int64_t)kHeadDim * kKeyTile;
    vstride = kKeyTile;
  }
  const bool valid = r < nrows;

  typename Pol::Q qr;
  Pol::load_q(qr, q + t * a.qs.t + hq * a.qs.h, hh);

  const T *kbase = (const T *)a.k + g * a.ks.h;
  const int64_t kstride = a.ks.t;
  floatx16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const T *ktile = kbase + kbeg * kstride;
  const int64_t rows_after = a.T - kbeg;  // K rows from kbeg to the end of the tensor
  if constexpr (std::is_same<T, __bf16>::value)
    tiles_direct<MODE, Pol::kThreads / 64, Pol::kStages, Pol::kLoadAhead>(
        lds, ktile, (uint32_t)kstride, rows_after, vt0, vstep, (uint32_t)vstride, nkt, qr, qfirst,
        qpos, a.scale_log2, kn_run, q_bound(qr, a.scale_log2), o, m, l);
  else
    tiles_staged<Pol, MODE>((T *)lds, ktile, (uint32_t)kstride, rows_after, vt0, vstep,
                            (uint32_t)vstride, nkt, qr, qfirst, qpos, a.scale_log2, o, m, l);

  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.f / lt;
  const float lse = (m + __log2f(lt)) * kLn2;
  if constexpr (MODE == MODE_OWN_MERGE) {
    static_assert(std::is_same<T, __bf16>::value, "merged own block: bf16 only");
    static_assert(Pol::kThreads / 64 * MergeLds::WAVE <= LdsBytes<Pol>::value, "merge LDS");
    merge_own(a, lds, o, inv, lse, t - (valid ? r : 0), wave * 32, nrows, hq, hq - a.h0, nsel);
    return;
  }
  if (!valid) return;
  if constexpr (MODE != MODE_DENSE) {
    T *dst = (T *)a.part_o + slot * kHeadDim + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa)
        store4<T>(dst + 32 * dt + 8 * aa, o[dt][4 * aa] * inv, o[dt][4 * aa + 1] * inv,
                  o[dt][4 * aa + 2] * inv, o[dt][4 * aa + 3] * inv);
    if (hh == 0) a.part_lse[slot] = lse;
  } else {
    T *dst = (T *)a.out + t * a.os.t + hq * a.os.h + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa)
        store4<T>(dst + 32 * dt + 8 * aa, o[dt][4 * aa] * inv, o[dt][4 * aa + 1] * inv,
                  o[dt][4 * aa + 2] * inv, o[dt][4 * aa + 3] * inv);
    if (hh == 0 && a.lse) a.lse[(int64_t)hq * a.T + t] = lse;
  }
}

// Earlier-block tiles per workgroup (bf16).
constexpr uint32_t kHistTilesPerWg = 2;

typedef __attribute__((address_space(1))) const void *global_ptr_t;

// One earlier-block tile (bf16): rec is its record, slot this lane's row's
// slot; the query rows come from q, or (q_lds) from the wave's staging area
// where the previous tile gathered them. With next_slot >= 0 (uniform
// next != 0) the tile gathers the next tile's query rows (lane's row:
// next_slot) into the staging area, behind its own first loads. Piece j of
// lane l is chunk 2 j + hh of the lane's row, at 1024 j + 16 l: the MFMA
// operand layout, read back without exchange between lanes.
__device__ __forceinline__ void hist_tile(const AttnArgs &a, char *lds, const int4 rec,
                                          int64_t slot, bool q_lds, bool next, int64_t next_slot) {
  using Pol = PolBf16;
  using T = __bf16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hh = lane >> 5;
  const int r = wave * 32 + (lane & 31);
  char *const qst = lds + kQStage + wave * 8192;
  const int p = (int)((uint32_t)rec.z / a.NBb);
  const int64_t gb = (uint32_t)rec.z % a.NBb;
  const int nrows = rec.y;
  const int nkt = a.B / kKeyTile;
  const int64_t kbeg = rec.w;
  const T *vt0 = (const T *)a.vt + ((int64_t)p * a.NBb + gb) * kHeadDim * a.B;
  const float kn_run = a.knorm[(int64_t)p * a.NBb + gb];  // bins and norms share p * NBb + block
  auto row_of = [&](int64_t sl) {
    const int64_t th = sl / a.topk;
    return (const T *)a.q + th / a.Hp * a.qs.t + (a.h0 + (int)(th % a.Hp)) * a.qs.h;
  };
  Pol::Q qr;
  if (q_lds) {
#pragma unroll
    for (int j = 0; j < kHeadDim / 16; ++j) qr.v[j] = *(const bf16x8 *)(qst + 1024 * j + 16 * lane);
  } else {
    Pol::load_q(qr, row_of(slot), hh);
  }
  const T *ktile = (const T *)a.k + (a.g0 + p) * a.ks.h + kbeg * a.ks.t;
  floatx16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m = -INFINITY, l = 0.f;
  tiles_direct<MODE_HIST, Pol::kThreads / 64, Pol::kStages, Pol::kLoadAhead, kHeadDim / 16>(
      lds, ktile, (uint32_t)a.ks.t, a.T - kbeg, vt0, (int64_t)kKeyTile, (uint32_t)a.B, nkt, qr, 0,
      0, a.scale_log2, kn_run, q_bound(qr, a.scale_log2), o, m, l, [&]() {
        if (!next) return 0;
        const T *row = row_of(next_slot) + 8 * hh;
#pragma unroll
        for (int j = 0; j < kHeadDim / 16; ++j)
          __builtin_amdgcn_global_load_lds((global_ptr_t)(row + 16 * j),
                                           (lds_ptr_t)(qst + 1024 * j), 16, 0, 0);
        return kHeadDim / 16;
      });
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.f / lt;
  if (r < nrows) {
    T *dst = (T *)a.part_o + slot * kHeadDim + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int aa = 0; aa < 4; ++aa)
        store4<T>(dst + 32 * dt + 8 * aa, o[dt][4 * aa] * inv, o[dt][4 * aa + 1] * inv,
                  o[dt][4 * aa + 2] * inv, o[dt][4 * aa + 3] * inv);
    if (hh == 0) a.part_lse[slot] = (m + __log2f(lt)) * kLn2;
  }
}

template <class Pol, int MODE>
__global__ __launch_bounds__(Pol::kThreads, Pol::kOcc) void attn_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[LdsBytes<Pol>::value];
  if constexpr (MODE == MODE_HIST && std::is_same<typename Pol::T, __bf16>::value) {
    // Workgroup i takes tiles j, j + 1 of XCD x's range (x = i % 8,
    // j = 2 (i / 8)): XCD-aware, so the tiles of one block run together on
    // one XCD and share its L2. Both records and both items of each lane's
    // row are read at the start; the second tile's query rows are gathered
    // while the first tile runs, and its loads start while the first tile's
    // partial results are still being written.
    const uint32_t ntiles = a.tile_off[a.nbins];
    const uint32_t per = (ntiles + 7) >> 3;
    const uint32_t j = (blockIdx.x >> 3) * kHistTilesPerWg;
    const uint32_t tile = (blockIdx.x & 7) * per + j;
    if (j >= per || tile >= ntiles) return;
    const bool second = j + 1 < per && tile + 1 < ntiles;
    const int r = (int)(threadIdx.x >> 6) * 32 + (int)(threadIdx.x & 31);
    const int4 rec0 = a.tile_rec[tile];
    const int4 rec1 = second ? a.tile_rec[tile + 1] : rec0;
    const int64_t slot0 = a.items[(uint32_t)rec0.x + min(r, rec0.y - 1)];
    const int64_t slot1 = a.items[(uint32_t)rec1.x + min(r, rec1.y - 1)];
    hist_tile(a, lds, rec0, slot0, false, second, slot1);
    if (second) hist_tile(a, lds, rec1, slot1, true, false, 0);
  } else {
    attn_tile<Pol, MODE>(a, lds, blockIdx.x);
  }
}

AttnArgs base_args(const Problem &pb, const Work &w, const void *q, const void *k, int g0) {
  AttnArgs a{};
  a.q = q; a.k = k; a.vt = w.vt; a.knorm = w.knorm;
  a.qs = pb.qs; a.ks = pb.ks; a.os = pb.os;
  a.T = pb.T; a.Hq = pb.Hq; a.Hkv = pb.Hkv; a.G = pb.G; a.B = pb.B; a.topk = pb.k;
  a.scale_log2 = pb.scale * kLog2e;
  a.g0 = g0; a.h0 = g0 * pb.G; a.Hp = pb.Hp;
  a.NBb = pb.NBb; a.info = w.blk_info;
  a.tile_off = w.tile_off; a.tile_rec = w.tile_rec; a.bin_off = w.bin_off; a.items = w.items;
  a.nbins = (int64_t)pb.P * pb.NBb;
  a.part_o = w.part_o; a.part_lse = w.part_lse;
  return a;
}

template <int MODE>
hipError_t launch_mode(bool bf16, dim3 grid, const AttnArgs &a, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (bf16)
    attn_kernel<PolBf16, MODE><<<grid, PolBf16::kThreads, 0, s>>>(a);
  else
    attn_kernel<PolF32, MODE><<<grid, PolF32::kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_diag(const Problem &pb, const Work &w, const void *q, const void *k, int g0,
                            hipStream_t s) {
  const AttnArgs a = base_args(pb, w, q, k, g0);
  const int rows = pb.bf16 ? PolBf16Own::kRows : PolF32::kRows;
  const int64_t nq = (pb.B + rows - 1) / rows;
  const int64_t grid = (pb.Hp * pb.NBb * nq + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  if (pb.bf16)
    attn_kernel<PolBf16Own, MODE_DIAG><<<dim3((unsigned)grid), PolBf16Own::kThreads, 0, s>>>(a);
  else
    attn_kernel<PolF32, MODE_DIAG><<<dim3((unsigned)grid), PolF32::kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_own_merge(const Problem &pb, const Work &w, const void *q, const void *k,
                                int g0, void *out, float *lse, hipStream_t s) {
  if (!pb.bf16) return hipErrorInvalidValue;
  AttnArgs a = base_args(pb, w, q, k, g0);
  a.out = out;
  a.lse = lse;
  const int64_t nq = (pb.B + PolBf16Own::kRows - 1) / PolBf16Own::kRows;
  const int64_t grid = (pb.Hp * pb.NBb * nq + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  attn_kernel<PolBf16Own, MODE_OWN_MERGE><<<dim3((unsigned)grid), PolBf16Own::kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_hist(const Problem &pb, const Work &w, const void *q, const void *k, int g0,
                            hipStream_t s) {
  if (pb.k <= 1) return hipSuccess;
  const AttnArgs a = base_args(pb, w, q, k, g0);
  const int64_t per = (w.max_tiles + 7) / 8;  // tiles per XCD, at most
  const int64_t grid = pb.bf16 ? 8 * ((per + kHistTilesPerWg - 1) / kHistTilesPerWg) : 8 * per;
  return launch_mode<MODE_HIST>(pb.bf16, dim3((unsigned)grid), a, s);
}

hipError_t launch_dense(const void *q, const void *k, const void *vt, const float *knorm,
                        const int32_t *blk_first64, const int4 *qtiles, int bf16, int64_t T,
                        int64_t NBq, int Hq, int Hkv, int64_t NBb64, float scale, void *out,
                        float *lse, hipStream_t s) {
  AttnArgs a{};
  a.q = q; a.k = k; a.vt = vt; a.knorm = knorm;
  a.qs = RowHead{(int64_t)Hq * kHeadDim, kHeadDim};  // contiguous [T][H][d]
  a.ks = RowHead{(int64_t)Hkv * kHeadDim, kHeadDim};
  a.os = a.qs;
  a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.scale_log2 = scale * kLog2e;
  a.blk_first64 = blk_first64; a.qtiles = qtiles; a.NBq = NBq;
  a.NBb64 = NBb64;
  a.out = out; a.lse = lse;
  return launch_mode<MODE_DENSE>(bf16 != 0, dim3((unsigned)NBq, (unsigned)Hq), a, s);
}

}  // namespace moba
