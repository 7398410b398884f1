// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moba.h"

namespace moba {

constexpr int kHeadDim = 128;       // head dimension of the GPU path
constexpr int kKeyTile = 64;        // keys per LDS tile in the attention kernels
constexpr int kRowTile = 128;       // smallest query-row tile of the attention kernels
constexpr int kRowsBf16 = 256;      // bf16 attention workgroup: 8 waves x 32 rows
constexpr int kRowsF32 = 128;       // fp32 attention workgroup: 4 waves x 32 rows
inline int attn_rows(int bf16) { return bf16 ? kRowsBf16 : kRowsF32; }
constexpr int kGateTokens = 64;     // tokens per gate workgroup (one wave per query head)
constexpr int kDispatchTokens = 64; // tokens per dispatch workgroup
constexpr int kMaxHistPick = 32;    // largest topk-1 kept in registers by the gate
constexpr int kWorkCounters = 8;    // one per XCD
constexpr int kMaxExtraPick = 16;   // pooled gate: extra blocks per max / min ranking
constexpr int kLdsBins = 16384;     // LDS histogram bins of the dispatch stage (64 KiB)

// Everything a launcher needs to know about one call.
struct Problem {
  int64_t T;        // total rows
  int S;            // sequences
  int maxlen;       // upper bound on a sequence length
  int Hq, Hkv, G;   // heads, G = Hq / Hkv
  int bf16;         // element type: 1 = bf16, 0 = fp32
  int B, k;         // block size, topk
  float scale;      // softmax scale
  int64_t NBb;      // upper bound on the number of blocks
  int P, Hp;        // kv heads and query heads per pass
  int maxblk;       // ceil(maxlen / B)
  int rows;         // query rows per attention workgroup (and per dispatch tile)
};

// Device buffers carved out of a workspace (see moba_layout_t).
struct Work {
  int32_t *blk_first;   // [S+1]
  int32_t *cu;          // [S+1] copy of cu_seqlens
  int4 *blk_info;       // [NBb] {seq, first row, rows, local block}
  float *kbar;          // [NBb][Hkv][d]
  __bf16 *kbar_split;   // [NBb][Hkv][2][d]: bf16 hi and lo parts, kbar ~= hi + lo
  float *kmax, *kmin;   // [NBb][Hkv][d] max- and min-pooled keys
  __bf16 *kmax_split, *kmin_split;  // [NBb][Hkv][2][d] their bf16 hi and lo parts
  void *vt;             // [P][NBb][d][B]
  int32_t *idx;         // [T][Hp][k]
  uint32_t *bin_count;  // [P*NBb]
  uint32_t *bin_off;    // [P*NBb + 1]
  uint32_t *tile_off;   // [P*NBb + 1]
  uint32_t *cursor;     // [P*NBb]
  uint32_t *work;       // [kWorkCounters] tile counters of the persistent attention (per XCD)
  int4 *tile_rec;       // [max tiles] {first item, rows, bin, first token of the block}
  uint32_t *items;      // [T*Hp*(k-1)]
  void *part_o;         // [T*Hp*k][d], element type of the inputs
  float *part_lse;      // [T*Hp*k]
  int64_t max_tiles;
};

// Launchers (enqueue only; return the launch status).
hipError_t launch_fill_u32(uint32_t *p, uint32_t value, int64_t n, hipStream_t s);
hipError_t launch_seqtable(const int32_t *cu, int S, int B, int64_t NBb, int32_t *blk_first,
                           int32_t *cu_copy, int4 *blk_info, hipStream_t s);
hipError_t launch_meanpool(const Problem &pb, const Work &w, const void *k, hipStream_t s);
hipError_t launch_minmaxpool(const Problem &pb, const Work &w, const void *k, hipStream_t s);
hipError_t launch_gate(const Problem &pb, const Work &w, const void *q, int g0, hipStream_t s);
hipError_t launch_gate_window(const Problem &pb, const Work &w, int n_sink, hipStream_t s);
hipError_t launch_gate_pooled(const Problem &pb, const Work &w, const void *q, int g0,
                              int extra_max, int extra_min, hipStream_t s);
hipError_t launch_dispatch(const Problem &pb, const Work &w, hipStream_t s);
hipError_t launch_vtrans(const void *v, int bf16, int64_t T, int Hkv, int g0, int P,
                         int64_t NBb, int B, const int4 *blk_info, void *vt, hipStream_t s);
hipError_t launch_attn_diag(const Problem &pb, const Work &w, const void *q, const void *k,
                            int g0, hipStream_t s);
hipError_t launch_attn_hist(const Problem &pb, const Work &w, const void *q, const void *k,
                            int g0, hipStream_t s);
hipError_t launch_merge(const Problem &pb, const Work &w, int g0, void *out, float *lse,
                        hipStream_t s);
int decode_splits(int S, int Hq, int Hkv, int B, int k, int maxblk);
hipError_t launch_decode(const Problem &pb, const Work &w, const void *q, const void *kc,
                         const void *vc, void *out, float *lse, hipStream_t s);
hipError_t launch_dense(const void *q, const void *k, const void *vt, const int32_t *cu,
                        const int32_t *blk_first64, int bf16, int64_t T, int S, int maxlen,
                        int Hq, int Hkv, int64_t NBb64, float scale, void *out, float *lse,
                        hipStream_t s);

}  // namespace moba
