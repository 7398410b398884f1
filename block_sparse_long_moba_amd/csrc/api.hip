// C ABI of MoBA (forward pass and its stages, gate variants, backward pass,
// decode, dense causal baseline): argument checks, workspace plans, and the
// order in which the stages are enqueued. Declared in include/moba.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "bwd.h"
#include "moba_internal.h"

using namespace moba;

namespace {

// a fixed buffer per thread: reporting an error allocates nothing
thread_local char g_last_error[512];

moba_status_t fail(moba_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
moba_status_t fail(moba_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

moba_status_t hip_fail(hipError_t e, const char *where) {
  return fail(MOBA_ERROR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define MOBA_HIP(call, where)                          \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return hip_fail(e_, where);  \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

moba_status_t check_shape(const moba_shape_t *sh) {
  if (!sh) return fail(MOBA_ERROR_INVALID_VALUE, "shape is NULL");
  if (sh->total_tokens < 0) return fail(MOBA_ERROR_INVALID_VALUE, "total_tokens < 0");
  if (sh->num_seqs < 0 || (sh->num_seqs == 0 && sh->total_tokens != 0))
    return fail(MOBA_ERROR_INVALID_VALUE, "num_seqs must be >= 1 when total_tokens > 0");
  if (sh->max_seqlen < 0) return fail(MOBA_ERROR_INVALID_VALUE, "max_seqlen < 0");
  if (sh->num_q_heads < 1 || sh->num_kv_heads < 1)
    return fail(MOBA_ERROR_INVALID_VALUE, "head counts must be >= 1");
  if (sh->num_q_heads % sh->num_kv_heads != 0)
    return fail(MOBA_ERROR_INVALID_VALUE, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                sh->num_q_heads, sh->num_kv_heads);
  if (sh->dtype != MOBA_DTYPE_FP32 && sh->dtype != MOBA_DTYPE_BF16)
    return fail(MOBA_ERROR_INVALID_VALUE, "unknown dtype %d", (int)sh->dtype);
  if (sh->head_dim < 1) return fail(MOBA_ERROR_INVALID_VALUE, "head_dim < 1");
  if (sh->head_dim != kHeadDim)
    return fail(MOBA_ERROR_UNSUPPORTED, "head_dim %d: only %d is supported", sh->head_dim, kHeadDim);
  if (sh->total_tokens >= (int64_t(1) << 31))
    return fail(MOBA_ERROR_UNSUPPORTED, "total_tokens must be < 2^31");
  return MOBA_SUCCESS;
}

moba_status_t check_moba_args(const moba_shape_t *sh, int32_t B, int32_t k) {
  moba_status_t st = check_shape(sh);
  if (st != MOBA_SUCCESS) return st;
  if (B < 1) return fail(MOBA_ERROR_INVALID_VALUE, "block_size must be >= 1");
  if (k < 1) return fail(MOBA_ERROR_INVALID_VALUE, "topk must be >= 1");
  if (B % kKeyTile != 0)
    return fail(MOBA_ERROR_UNSUPPORTED, "block_size %d: must be a multiple of %d", B, kKeyTile);
  if ((uint64_t)sh->total_tokens * (uint64_t)sh->num_q_heads * (uint64_t)k >= (uint64_t(1) << 32))
    return fail(MOBA_ERROR_UNSUPPORTED, "total_tokens * num_q_heads * topk must be < 2^32");
  const int64_t T = sh->total_tokens;
  const int64_t maxlen = sh->max_seqlen > 0 ? std::min<int64_t>(sh->max_seqlen, T) : T;
  const int64_t maxblk = ceil_div(maxlen, B);
  if (k - 1 > kMaxHistPick && k < maxblk)
    return fail(MOBA_ERROR_UNSUPPORTED,
                "topk %d: at most %d unless topk >= the block count of the longest sequence (%lld)",
                k, kMaxHistPick + 1, (long long)maxblk);
  return MOBA_SUCCESS;
}

// Table region: blk_first[S+1], a copy of cu_seqlens[S+1], the status word,
// then (16-byte aligned) blk_info[NBb].
size_t cu_copy_offset(int S) { return sizeof(int32_t) * (S + 1); }
size_t status_offset(int S) { return 2 * sizeof(int32_t) * (S + 1); }
size_t info_offset(int S) { return (status_offset(S) + sizeof(int32_t) + 15) / 16 * 16; }
size_t table_bytes(int S, int64_t NBb) { return info_offset(S) + 16 * (size_t)NBb; }

// Pointers of one table region.
struct Table {
  int32_t *first, *cu, *status;
  int4 *info;
};
Table table_at(void *base, int S) {
  char *b = (char *)base;
  return Table{(int32_t *)b, (int32_t *)(b + cu_copy_offset(S)), (int32_t *)(b + status_offset(S)),
               (int4 *)(b + info_offset(S))};
}

// The status word's meaning (see the kStatus* bits).
moba_status_t status_error(int32_t st) {
  if (st & kStatusBadSeqlens)
    return fail(MOBA_ERROR_INVALID_VALUE,
                "cu_seqlens is malformed: it must start at 0, never decrease and end at "
                "total_tokens");
  if (st & kStatusTooManyBlocks)
    return fail(MOBA_ERROR_INVALID_VALUE,
                "a sequence has more blocks than the plan allows: max_seqlen is understated");
  return MOBA_SUCCESS;
}

// Synchronises the stream and reads a status word.
moba_status_t read_status(const int32_t *status, hipStream_t s) {
  int32_t h = 0;
  MOBA_HIP(hipMemcpyAsync(&h, status, sizeof h, hipMemcpyDeviceToHost, s), "hipMemcpyAsync");
  MOBA_HIP(hipStreamSynchronize(s), "hipStreamSynchronize");
  return status_error(h);
}

// MOBA_CHECK=1 (environment): whole-pass calls check the sequence table on
// the host right after building it (one synchronisation) and return an error.
bool check_enabled() {
  const char *e = getenv("MOBA_CHECK");
  return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

// Bins region: count[nbins], offset[nbins+1], tile_offset[nbins+1],
// cursor[nbins], the counted flag (uint32), then (16-byte aligned) int4 tile
// records.
size_t tile_rec_offset(int64_t nbins) {
  return (sizeof(uint32_t) * (size_t)(4 * nbins + 2 + 1) + 15) / 16 * 16;
}
size_t bins_bytes(int64_t nbins, int64_t max_tiles) {
  return tile_rec_offset(nbins) + 16 * (size_t)max_tiles;
}

// The vt region: transposed values, then (256-byte aligned) the largest key
// norm of every block.
size_t vt_bytes(size_t es, int P, int64_t NBb, int B) {
  return align_up(es * (size_t)P * NBb * kHeadDim * B);
}

int largest_divisor_at_most(int n, int cap) {
  for (int d = std::min(n, cap); d >= 1; --d)
    if (n % d == 0) return d;
  return 1;
}

moba_status_t plan_impl(const moba_shape_t *sh, int32_t B, int32_t k, int32_t P_req,
                        moba_layout_t *L) {
  moba_status_t st = check_moba_args(sh, B, k);
  if (st != MOBA_SUCCESS) return st;
  if (!L) return fail(MOBA_ERROR_INVALID_VALUE, "layout is NULL");
  const int64_t T = sh->total_tokens;
  const int S = sh->num_seqs, Hq = sh->num_q_heads, Hkv = sh->num_kv_heads, G = Hq / Hkv;
  const size_t es = sh->dtype == MOBA_DTYPE_BF16 ? 2 : 4;
  const int64_t maxlen = sh->max_seqlen > 0 ? std::min<int64_t>(sh->max_seqlen, T) : T;
  const int64_t maxblk = std::max<int64_t>(1, ceil_div(maxlen, B));
  if (maxblk > kLdsBins)
    return fail(MOBA_ERROR_UNSUPPORTED, "a sequence may have %lld blocks; at most %d supported",
                (long long)maxblk, kLdsBins);
  int P = P_req <= 0 ? Hkv : std::min(P_req, Hkv);
  P = largest_divisor_at_most(Hkv, P);
  while (P > 1 && (int64_t)P * maxblk > kLdsBins) P = largest_divisor_at_most(Hkv, P - 1);
  const int Hp = P * G;
  const int64_t NBb = ceil_div(T, B) + S;
  const int64_t nbins = (int64_t)P * NBb;
  const int64_t hist_items = T * Hp * (k - 1);
  const int64_t max_tiles = ceil_div(hist_items, kRowTile) + nbins;  // bound for any tile size
  // own-block attention launches one workgroup per (query head, block, row tile)
  if ((int64_t)Hp * NBb * ceil_div(B, kRowTile) >= (int64_t(1) << 31))
    return fail(MOBA_ERROR_UNSUPPORTED,
                "too many own-block tiles per pass (num_q_heads * blocks * block_size / %d)",
                kRowTile);
  const int64_t slots = T * Hp * k;

  *L = moba_layout_t{};
  L->num_blocks_bound = NBb;
  L->padded_tokens = ceil_div(T, kKeyTile) * kKeyTile;
  L->kv_heads_per_pass = P;
  L->q_heads_per_pass = Hp;
  L->max_blocks_per_seq = (int32_t)maxblk;
  size_t off = 0;
  L->table_offset = off;     off = align_up(off + table_bytes(S, NBb));
  L->kbar_offset = off;      off = align_up(off + 3 * (sizeof(float) + 4) * (size_t)NBb * Hkv * kHeadDim);
  L->vt_offset = off;        off = align_up(off + vt_bytes(es, P, NBb, B) +
                                            sizeof(float) * (size_t)P * NBb);
  L->idx_offset = off;       off = align_up(off + sizeof(int32_t) * (size_t)slots);
  L->bins_offset = off;      off = align_up(off + bins_bytes(nbins, max_tiles));
  L->items_offset = off;     off = align_up(off + sizeof(uint32_t) * (size_t)std::max<int64_t>(1, hist_items));
  L->part_o_offset = off;    off = align_up(off + es * (size_t)slots * kHeadDim);
  L->part_lse_offset = off;  off = align_up(off + sizeof(float) * (size_t)slots);
  L->total_bytes = off;
  return MOBA_SUCCESS;
}

// Backward plan: the forward plan up to the items, then fp32 partial dq per
// slot (in place of the partial outputs) and D per (head, row) (in place of
// their lse). The vt region is unused.
moba_status_t bwd_plan_impl(const moba_shape_t *sh, int32_t B, int32_t k, int32_t P_req,
                            moba_layout_t *L) {
  moba_status_t st = plan_impl(sh, B, k, P_req, L);
  if (st != MOBA_SUCCESS) return st;
  const int64_t T = sh->total_tokens;
  const int64_t slots = T * L->q_heads_per_pass * k;
  size_t off = L->part_o_offset;
  off = align_up(off + sizeof(float) * (size_t)slots * kHeadDim);
  L->part_lse_offset = off;
  off = align_up(off + sizeof(float) * (size_t)T * sh->num_q_heads);
  const int64_t nbins = (int64_t)L->kv_heads_per_pass * L->num_blocks_bound;
  const DkdvSplit sp = dkdv_split(T, L->q_heads_per_pass, k, B);
  L->total_bytes = bwd_extra(off, nbins, sp).end;
  return MOBA_SUCCESS;
}

// Strides of contiguous [T][H][d] q, k, v and out.
void set_contiguous(Problem *pb) {
  pb->qs = RowHead{(int64_t)pb->Hq * kHeadDim, kHeadDim};
  pb->ks = RowHead{(int64_t)pb->Hkv * kHeadDim, kHeadDim};
  pb->vs = pb->ks;
  pb->os = pb->qs;
}

Problem make_problem(const moba_shape_t *sh, int32_t B, int32_t k, float scale,
                     const moba_layout_t *L) {
  Problem pb{};
  pb.T = sh->total_tokens;
  pb.S = sh->num_seqs;
  pb.maxlen = (int)(sh->max_seqlen > 0 ? std::min<int64_t>(sh->max_seqlen, pb.T) : pb.T);
  pb.Hq = sh->num_q_heads;
  pb.Hkv = sh->num_kv_heads;
  pb.G = pb.Hq / pb.Hkv;
  pb.bf16 = sh->dtype == MOBA_DTYPE_BF16;
  pb.B = B;
  pb.k = k;
  pb.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)kHeadDim);
  pb.NBb = L->num_blocks_bound;
  pb.P = L->kv_heads_per_pass;
  pb.Hp = L->q_heads_per_pass;
  pb.maxblk = L->max_blocks_per_seq;
  pb.rows = attn_rows(pb.bf16);
  set_contiguous(&pb);
  return pb;
}

Work carve(const Problem &pb, const moba_layout_t *L, void *ws) {
  char *b = (char *)ws;
  Work w{};
  const Table tb = table_at(b + L->table_offset, pb.S);
  w.blk_first = tb.first;
  w.cu = tb.cu;
  w.status = tb.status;
  w.blk_info = tb.info;
  w.kbar = (float *)(b + L->kbar_offset);
  const size_t nkb = (size_t)pb.NBb * pb.Hkv * kHeadDim;
  w.kbar_split = (__bf16 *)(w.kbar + nkb);
  w.kmax = (float *)(w.kbar_split + 2 * nkb);
  w.kmax_split = (__bf16 *)(w.kmax + nkb);
  w.kmin = (float *)(w.kmax_split + 2 * nkb);
  w.kmin_split = (__bf16 *)(w.kmin + nkb);
  w.vt = b + L->vt_offset;
  w.knorm = (float *)(b + L->vt_offset + vt_bytes(pb.bf16 ? 2 : 4, pb.P, pb.NBb, pb.B));
  w.idx = (int32_t *)(b + L->idx_offset);
  const int64_t nbins = (int64_t)pb.P * pb.NBb;
  uint32_t *bins = (uint32_t *)(b + L->bins_offset);
  w.bin_count = bins;
  w.bin_off = bins + nbins;
  w.tile_off = bins + 2 * nbins + 1;
  w.cursor = bins + 3 * nbins + 2;
  w.counted = bins + 4 * nbins + 2;
  w.tile_rec = (int4 *)((char *)bins + tile_rec_offset(nbins));
  w.items = (uint32_t *)(b + L->items_offset);
  w.part_o = b + L->part_o_offset;
  w.part_lse = (float *)(b + L->part_lse_offset);
  w.max_tiles = ceil_div(pb.T * pb.Hp * (pb.k - 1), pb.rows) + nbins;
  return w;
}

// Shared checks of the stage entry points: the layout must be the plan of
// these arguments (same pass size) and the workspace non-NULL. PLAN_FWD /
// PLAN_BWD: the forward / backward plan; PLAN_ANY: either (the stages before
// the attention use the regions both plans share).
enum { PLAN_FWD = 1, PLAN_BWD = 2, PLAN_ANY = 3 };
moba_status_t check_stage(const moba_shape_t *sh, int32_t B, int32_t k, const moba_layout_t *L,
                          void *ws, moba_layout_t *fresh, int which = PLAN_FWD) {
  if (!L) return fail(MOBA_ERROR_INVALID_VALUE, "layout is NULL");
  moba_status_t st = plan_impl(sh, B, k, L->kv_heads_per_pass, fresh);
  if (st != MOBA_SUCCESS) return st;
  bool ok = false;
  if ((which & PLAN_FWD) && fresh->total_bytes == L->total_bytes &&
      fresh->kv_heads_per_pass == L->kv_heads_per_pass)
    ok = true;
  if (!ok && (which & PLAN_BWD)) {
    moba_layout_t b;
    if ((st = bwd_plan_impl(sh, B, k, L->kv_heads_per_pass, &b)) != MOBA_SUCCESS) return st;
    if (b.total_bytes == L->total_bytes && b.kv_heads_per_pass == L->kv_heads_per_pass) {
      ok = true;
      *fresh = b;
    }
  }
  if (!ok) return fail(MOBA_ERROR_INVALID_VALUE, "layout does not match shape/block_size/topk");
  if (!ws && sh->total_tokens > 0) return fail(MOBA_ERROR_INVALID_VALUE, "workspace is NULL");
  return MOBA_SUCCESS;
}

moba_status_t check_pass(const moba_shape_t *sh, const moba_layout_t *L, int32_t g0) {
  if (g0 < 0 || g0 >= sh->num_kv_heads || g0 % L->kv_heads_per_pass != 0)
    return fail(MOBA_ERROR_INVALID_VALUE, "kv_head_begin %d must be a multiple of %d below %d", g0,
                L->kv_heads_per_pass, sh->num_kv_heads);
  return MOBA_SUCCESS;
}

// Backward plan: its partial-dq and D regions, and the pooled gate's scratch
// (lists at the start of the partial-dq region, at most (topk + 2) ints per
// (row, head); the per-slot lse in its last T*Hp*topk floats) kept away from D.
BwdWork carve_bwd(const Problem &pb, const moba_layout_t *L, void *ws, Work *w) {
  const size_t base = align_up(L->part_lse_offset + sizeof(float) * (size_t)pb.T * pb.Hq);
  const BwdExtra x = bwd_extra(base, (int64_t)pb.P * pb.NBb, dkdv_split(pb.T, pb.Hp, pb.k, pb.B));
  char *b = (char *)ws;
  BwdWork bw{(float *)(b + L->part_o_offset), (float *)(b + L->part_lse_offset), b + x.zeros,
             (uint32_t *)(b + x.ext_off), (uint32_t *)(b + x.slot_off), (float *)(b + x.part)};
  const int64_t slots = pb.T * pb.Hp * pb.k;
  w->part_o = bw.dq_part;
  w->part_lse = bw.dq_part + slots * (kHeadDim - 1);
  return bw;
}

bool is_bwd_plan(const moba_shape_t *sh, int32_t B, int32_t k, const moba_layout_t *L) {
  moba_layout_t f;
  return plan_impl(sh, B, k, L->kv_heads_per_pass, &f) == MOBA_SUCCESS &&
         f.total_bytes != L->total_bytes;
}

// Shared checks and set-up of the attention-gradient stages.
moba_status_t bwd_stage(const void *q, const void *k, const void *v, const void *dout,
                        const float *lse, const moba_shape_t *sh, int32_t B, int32_t topk,
                        float scale, const moba_layout_t *L, void *ws, int32_t g0, Problem *pb,
                        Work *w, BwdWork *bw, bool *nothing) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, topk, L, ws, &f, PLAN_BWD);
  if (st != MOBA_SUCCESS) return st;
  if (sh->dtype != MOBA_DTYPE_BF16) return fail(MOBA_ERROR_UNSUPPORTED, "backward pass: bf16 only");
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  *nothing = sh->total_tokens == 0;
  if (*nothing) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!q || !k || !v || !dout || !lse)
    return fail(MOBA_ERROR_INVALID_VALUE, "q, k, v, dout and lse must be non-NULL");
  *pb = make_problem(sh, B, topk, scale, L);
  *w = carve(*pb, L, ws);
  *bw = carve_bwd(*pb, L, ws, w);
  return MOBA_SUCCESS;
}

moba_status_t run_pass(const Problem &pb, const Work &w, const void *q, const void *k,
                       const void *v, int g0, void *out, float *lse, hipStream_t s,
                       const moba_gate_t &gate) {
  if (gate.kind == MOBA_GATE_WINDOW)
    MOBA_HIP(launch_gate_window(pb, w, gate.n_sink, s), "gate_window");
  else if (gate.kind == MOBA_GATE_POOLED)
    MOBA_HIP(launch_gate_pooled(pb, w, q, g0, gate.extra_max, gate.extra_min, s), "gate_pooled");
  else
    MOBA_HIP(launch_gate(pb, w, q, g0, s), "gate");
  MOBA_HIP(launch_dispatch(pb, w, s), "dispatch");
  MOBA_HIP(launch_vtrans(v, pb.vs, k, pb.ks, pb.bf16, g0, pb.P, pb.NBb, pb.B, w.blk_info, w.vt,
                         w.knorm, s),
           "vtrans");
  if (pb.bf16) {  // earlier blocks first, then the own block merged with them
    MOBA_HIP(launch_attn_hist(pb, w, q, k, g0, s), "attn_hist");
    MOBA_HIP(launch_attn_own_merge(pb, w, q, k, g0, out, lse, s), "attn_own_merge");
    MOBA_HIP(launch_nan_rows(pb, w, g0, out, lse, s), "nan_rows");
    return MOBA_SUCCESS;
  }
  MOBA_HIP(launch_attn_diag(pb, w, q, k, g0, s), "attn_diag");
  MOBA_HIP(launch_attn_hist(pb, w, q, k, g0, s), "attn_hist");
  MOBA_HIP(launch_merge(pb, w, g0, out, lse, s), "merge");
  return MOBA_SUCCESS;
}

moba_status_t check_gate(const moba_gate_t *g, int32_t topk) {
  if (!g) return fail(MOBA_ERROR_INVALID_VALUE, "gate is NULL");
  switch (g->kind) {
    case MOBA_GATE_MEAN: return MOBA_SUCCESS;
    case MOBA_GATE_WINDOW:
      if (g->n_sink < 0 || g->n_sink >= topk)
        return fail(MOBA_ERROR_INVALID_VALUE, "n_sink %d must lie in [0, topk)", g->n_sink);
      return MOBA_SUCCESS;
    case MOBA_GATE_POOLED:
      if (g->extra_max < 0 || g->extra_min < 0)
        return fail(MOBA_ERROR_INVALID_VALUE, "extra_max / extra_min must be >= 0");
      if (g->extra_max > kMaxExtraPick || g->extra_min > kMaxExtraPick)
        return fail(MOBA_ERROR_UNSUPPORTED, "extra_max / extra_min: at most %d", kMaxExtraPick);
      if (topk - g->extra_max - g->extra_min < 1)
        return fail(MOBA_ERROR_INVALID_VALUE,
                    "topk %d must exceed extra_max + extra_min (%d); the own block needs a slot",
                    topk, g->extra_max + g->extra_min);
      return MOBA_SUCCESS;
  }
  return fail(MOBA_ERROR_INVALID_VALUE, "unknown gate kind %d", (int)g->kind);
}

moba_status_t check_io(const void *q, const void *k, const void *v, const int32_t *cu,
                       const void *out, const moba_shape_t *sh) {
  if (sh->total_tokens > 0 && (!q || !k || !v || !out))
    return fail(MOBA_ERROR_INVALID_VALUE, "q, k, v and out must be non-NULL");
  if (sh->num_seqs > 0 && !cu) return fail(MOBA_ERROR_INVALID_VALUE, "cu_seqlens is NULL");
  // every head row is read and written in 16-byte vectors
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 != 0)
    return fail(MOBA_ERROR_INVALID_VALUE, "q, k, v and out must be 16-byte aligned");
  return MOBA_SUCCESS;
}

// Strides of the whole forward pass (elements): positive multiples of 16
// bytes, so every head row stays 16-byte aligned; out's (row, head) vectors
// must not overlap; one block of key rows must span less than 2 GiB, since
// the attention kernels address a block's keys with 32-bit byte offsets.
moba_status_t check_strides(const moba_shape_t *sh, int32_t B, const moba_strides_t *st) {
  const int64_t es = sh->dtype == MOBA_DTYPE_BF16 ? 2 : 4, unit = 16 / es;
  const struct { const char *name; int64_t t, h; } all[4] = {
      {"q", st->q_token, st->q_head}, {"k", st->k_token, st->k_head},
      {"v", st->v_token, st->v_head}, {"out", st->out_token, st->out_head}};
  for (const auto &x : all) {
    if (x.t <= 0 || x.h <= 0 || x.t % unit || x.h % unit)
      return fail(MOBA_ERROR_INVALID_VALUE,
                  "%s strides (%lld, %lld): must be positive multiples of %lld elements", x.name,
                  (long long)x.t, (long long)x.h, (long long)unit);
  }
  if (st->k_token > INT32_MAX / (es * B))  // k_token * es * B would reach 2^31
    return fail(MOBA_ERROR_UNSUPPORTED, "k token stride %lld: a block of %d rows spans 2 GiB or more",
                (long long)st->k_token, B);
  // out: the smaller stride must step over a whole head row, the larger one
  // over all vectors of the smaller
  int64_t s1 = st->out_head, n1 = sh->num_q_heads, s2 = st->out_token, n2 = sh->total_tokens;
  if (s1 > s2) {
    std::swap(s1, s2);
    std::swap(n1, n2);
  }
  if ((n1 > 1 && s1 < kHeadDim) || (n2 > 1 && s2 < (n1 - 1) * s1 + kHeadDim))
    return fail(MOBA_ERROR_INVALID_VALUE, "out strides (%lld, %lld): rows overlap",
                (long long)st->out_token, (long long)st->out_head);
  return MOBA_SUCCESS;
}

// Table-only stages (seqtable, meanpool) accept a layout planned with any
// topk: only the block bound and the table/kbar offsets are used.
moba_status_t check_table_stage(const moba_shape_t *sh, int32_t B, const moba_layout_t *L,
                                const void *ws) {
  moba_status_t st = check_shape(sh);
  if (st != MOBA_SUCCESS) return st;
  if (B < 1) return fail(MOBA_ERROR_INVALID_VALUE, "block_size must be >= 1");
  if (B % kKeyTile) return fail(MOBA_ERROR_UNSUPPORTED, "block_size %d: must be a multiple of %d", B, kKeyTile);
  if (!L) return fail(MOBA_ERROR_INVALID_VALUE, "layout is NULL");
  if (L->num_blocks_bound != ceil_div(sh->total_tokens, B) + sh->num_seqs)
    return fail(MOBA_ERROR_INVALID_VALUE, "layout does not match shape/block_size");
  if (!ws && sh->total_tokens > 0) return fail(MOBA_ERROR_INVALID_VALUE, "workspace is NULL");
  return MOBA_SUCCESS;
}

// Dense baseline workspace: the block table of 64-row key tiles (the
// transposed values are laid out per such tile), the table of query tiles
// (rows per attention workgroup), then the transposed values.
int64_t dense_nb64(const moba_shape_t *sh) {
  return ceil_div(sh->total_tokens, kKeyTile) + sh->num_seqs;
}
int64_t dense_nbq(const moba_shape_t *sh) {
  return ceil_div(sh->total_tokens, attn_rows(sh->dtype == MOBA_DTYPE_BF16)) + sh->num_seqs;
}
size_t dense_table_bytes(const moba_shape_t *sh) {
  return align_up(table_bytes(sh->num_seqs, dense_nb64(sh))) +
         align_up(table_bytes(sh->num_seqs, dense_nbq(sh)));
}

size_t dense_ws_bytes(const moba_shape_t *sh) {
  const size_t es = sh->dtype == MOBA_DTYPE_BF16 ? 2 : 4;
  return dense_table_bytes(sh) + vt_bytes(es, sh->num_kv_heads, dense_nb64(sh), kKeyTile) +
         align_up(sizeof(float) * (size_t)sh->num_kv_heads * dense_nb64(sh));
}

size_t workspace_limit_bytes() {
  double gib = 48.0;
  if (const char *e = getenv("MOBA_WORKSPACE_LIMIT_GIB")) {
    double v = atof(e);
    if (v > 0) gib = v;
  }
  return (size_t)(gib * (double)(size_t(1) << 30));
}

// ---- decode workspace: block table, pooled keys (with the bf16 split the
// mean-pool kernel also writes), idx[S][Hq][k], fp32 parts [S*Hq*k][d] and
// their lse.
struct DecodeLayout {
  int64_t NBb;
  int maxblk;
  size_t table, kbar, idx, part_o, part_lse, total;
};

moba_status_t decode_layout(const moba_shape_t *sh, int32_t B, int32_t k, DecodeLayout *D) {
  // decode keeps S*Hq*k slots and ranks candidates by counting: no limit on k
  moba_status_t st = check_shape(sh);
  if (st != MOBA_SUCCESS) return st;
  if (B < 1) return fail(MOBA_ERROR_INVALID_VALUE, "block_size must be >= 1");
  if (k < 1) return fail(MOBA_ERROR_INVALID_VALUE, "topk must be >= 1");
  if ((int64_t)sh->num_seqs * sh->num_q_heads * k >= (int64_t(1) << 31))
    return fail(MOBA_ERROR_UNSUPPORTED, "num_seqs * num_q_heads * topk must be < 2^31");
  const int G = sh->num_q_heads / sh->num_kv_heads;
  if (G > 64) return fail(MOBA_ERROR_UNSUPPORTED, "decode: at most 64 query heads per kv head");
  const int64_t T = sh->total_tokens;
  const int S = sh->num_seqs;
  const int64_t maxlen = sh->max_seqlen > 0 ? std::min<int64_t>(sh->max_seqlen, T) : T;
  D->maxblk = (int)std::max<int64_t>(1, ceil_div(maxlen, B));
  if (D->maxblk > kLdsBins)
    return fail(MOBA_ERROR_UNSUPPORTED, "decode: a sequence may have %d blocks; at most %d",
                D->maxblk, kLdsBins);
  D->NBb = ceil_div(T, B) + S;
  const size_t slots = (size_t)S * sh->num_q_heads * k *
                       decode_splits(S, sh->num_q_heads, sh->num_kv_heads, B, k, D->maxblk);
  size_t off = 0;
  D->table = off;    off = align_up(off + table_bytes(S, D->NBb));
  D->kbar = off;     off = align_up(off + (sizeof(float) + 4) * (size_t)D->NBb * sh->num_kv_heads * kHeadDim);
  D->idx = off;      off = align_up(off + sizeof(int32_t) * std::max<size_t>(1, slots));
  D->part_o = off;   off = align_up(off + sizeof(float) * kHeadDim * std::max<size_t>(1, slots));
  D->part_lse = off; off = align_up(off + sizeof(float) * std::max<size_t>(1, slots));
  D->total = off;
  return MOBA_SUCCESS;
}

void decode_setup(const moba_shape_t *sh, int32_t B, int32_t k, float scale, const DecodeLayout &D,
                  void *ws, Problem *pb, Work *w) {
  *pb = Problem{};
  pb->T = sh->total_tokens;
  pb->S = sh->num_seqs;
  pb->maxlen = (int)(sh->max_seqlen > 0 ? std::min<int64_t>(sh->max_seqlen, pb->T) : pb->T);
  pb->Hq = sh->num_q_heads;
  pb->Hkv = sh->num_kv_heads;
  pb->G = pb->Hq / pb->Hkv;
  pb->bf16 = sh->dtype == MOBA_DTYPE_BF16;
  pb->B = B;
  pb->k = k;
  pb->scale = scale > 0.f ? scale : 1.0f / sqrtf((float)kHeadDim);
  pb->NBb = D.NBb;
  pb->P = pb->Hkv;
  pb->Hp = pb->Hq;
  pb->maxblk = D.maxblk;
  pb->rows = attn_rows(pb->bf16);
  set_contiguous(pb);  // the cache is a contiguous [T][Hkv][d] tensor
  char *b = (char *)ws;
  *w = Work{};
  const Table tb = table_at(b + D.table, pb->S);
  w->blk_first = tb.first;
  w->cu = tb.cu;
  w->status = tb.status;
  w->blk_info = tb.info;
  w->kbar = (float *)(b + D.kbar);
  w->kbar_split = (__bf16 *)(w->kbar + (size_t)D.NBb * pb->Hkv * kHeadDim);
  w->idx = (int32_t *)(b + D.idx);
  w->part_o = b + D.part_o;
  w->part_lse = (float *)(b + D.part_lse);
}

}  // namespace

namespace moba {
moba_status_t report_error(moba_status_t st, const char *msg) { return fail(st, "%s", msg); }
}  // namespace moba

extern "C" {

const char *moba_status_string(moba_status_t s) {
  switch (s) {
    case MOBA_SUCCESS: return "MOBA_SUCCESS";
    case MOBA_ERROR_INVALID_VALUE: return "MOBA_ERROR_INVALID_VALUE";
    case MOBA_ERROR_UNSUPPORTED: return "MOBA_ERROR_UNSUPPORTED";
    case MOBA_ERROR_WORKSPACE_TOO_SMALL: return "MOBA_ERROR_WORKSPACE_TOO_SMALL";
    case MOBA_ERROR_HIP: return "MOBA_ERROR_HIP";
  }
  return "MOBA_ERROR_UNKNOWN";
}

const char *moba_last_error(void) { return g_last_error; }

moba_status_t moba_workspace_status(int32_t num_seqs, const void *workspace, hipStream_t stream) {
  if (num_seqs < 0) return fail(MOBA_ERROR_INVALID_VALUE, "num_seqs < 0");
  if (!workspace) return fail(MOBA_ERROR_INVALID_VALUE, "workspace is NULL");
  return read_status(table_at(const_cast<void *>(workspace), num_seqs).status, stream);
}

moba_status_t moba_plan(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                        int32_t kv_heads_per_pass, moba_layout_t *layout) {
  return plan_impl(shape, block_size, topk, kv_heads_per_pass, layout);
}

size_t moba_fwd_workspace_size(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                               int32_t kv_heads_per_pass) {
  moba_layout_t L;
  if (plan_impl(shape, block_size, topk, kv_heads_per_pass, &L) != MOBA_SUCCESS) return 0;
  return L.total_bytes;
}

moba_status_t moba_seqtable(const int32_t *cu, const moba_shape_t *sh, int32_t B,
                            const moba_layout_t *L, void *ws, hipStream_t s) {
  moba_status_t st = check_table_stage(sh, B, L, ws);
  if (st != MOBA_SUCCESS) return st;
  if (sh->num_seqs > 0 && !cu) return fail(MOBA_ERROR_INVALID_VALUE, "cu_seqlens is NULL");
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  const Table tb = table_at((char *)ws + L->table_offset, sh->num_seqs);
  MOBA_HIP(launch_seqtable(cu, sh->num_seqs, B, sh->total_tokens, L->max_blocks_per_seq,
                           L->num_blocks_bound, tb.first, tb.cu, tb.status, tb.info, s),
           "seqtable");
  return MOBA_SUCCESS;
}

moba_status_t moba_meanpool(const void *k, const moba_shape_t *sh, int32_t B,
                            const moba_layout_t *L, void *ws, hipStream_t s) {
  moba_status_t st = check_table_stage(sh, B, L, ws);
  if (st != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if (!k) return fail(MOBA_ERROR_INVALID_VALUE, "k is NULL");
  Problem pb = make_problem(sh, B, 1, 0.f, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_meanpool(pb, w, k, s), "meanpool");
  return MOBA_SUCCESS;
}

moba_status_t moba_gate(const void *q, const moba_shape_t *sh, int32_t B, int32_t k,
                        const moba_layout_t *L, void *ws, int32_t g0, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, k, L, ws, &f, PLAN_ANY);
  if (st != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!q) return fail(MOBA_ERROR_INVALID_VALUE, "q is NULL");
  Problem pb = make_problem(sh, B, k, 0.f, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_gate(pb, w, q, g0, s), "gate");
  return MOBA_SUCCESS;
}

moba_status_t moba_minmaxpool(const void *k, const moba_shape_t *sh, int32_t B,
                              const moba_layout_t *L, void *ws, hipStream_t s) {
  moba_status_t st = check_table_stage(sh, B, L, ws);
  if (st != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if (!k) return fail(MOBA_ERROR_INVALID_VALUE, "k is NULL");
  Problem pb = make_problem(sh, B, 1, 0.f, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_minmaxpool(pb, w, k, s), "minmaxpool");
  return MOBA_SUCCESS;
}

moba_status_t moba_gate_window(const moba_shape_t *sh, int32_t B, int32_t k, int32_t n_sink,
                               const moba_layout_t *L, void *ws, int32_t g0, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, k, L, ws, &f, PLAN_ANY);
  if (st != MOBA_SUCCESS) return st;
  const moba_gate_t gate{MOBA_GATE_WINDOW, n_sink, 0, 0};
  if ((st = check_gate(&gate, k)) != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  Problem pb = make_problem(sh, B, k, 0.f, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_gate_window(pb, w, n_sink, s), "gate_window");
  return MOBA_SUCCESS;
}

moba_status_t moba_gate_pooled(const void *q, const moba_shape_t *sh, int32_t B, int32_t k,
                               int32_t extra_max, int32_t extra_min, const moba_layout_t *L,
                               void *ws, int32_t g0, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, k, L, ws, &f, PLAN_ANY);
  if (st != MOBA_SUCCESS) return st;
  const moba_gate_t gate{MOBA_GATE_POOLED, 0, extra_max, extra_min};
  if ((st = check_gate(&gate, k)) != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!q) return fail(MOBA_ERROR_INVALID_VALUE, "q is NULL");
  Problem pb = make_problem(sh, B, k, 0.f, L);
  Work w = carve(pb, L, ws);
  if (is_bwd_plan(sh, B, k, L)) carve_bwd(pb, L, ws, &w);
  MOBA_HIP(launch_gate_pooled(pb, w, q, g0, extra_max, extra_min, s), "gate_pooled");
  return MOBA_SUCCESS;
}

moba_status_t moba_dispatch(const moba_shape_t *sh, int32_t B, int32_t k, const moba_layout_t *L,
                            void *ws, int32_t g0, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, k, L, ws, &f, PLAN_ANY);
  if (st != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  Problem pb = make_problem(sh, B, k, 0.f, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_dispatch(pb, w, s), "dispatch");
  return MOBA_SUCCESS;
}

moba_status_t moba_attn_fwd(const void *q, const void *k, const void *v, const moba_shape_t *sh,
                            int32_t B, int32_t topk, float scale, const moba_layout_t *L,
                            void *ws, int32_t g0, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, topk, L, ws, &f);
  if (st != MOBA_SUCCESS) return st;
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!q || !k || !v) return fail(MOBA_ERROR_INVALID_VALUE, "q, k, v must be non-NULL");
  Problem pb = make_problem(sh, B, topk, scale, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_vtrans(v, pb.vs, k, pb.ks, pb.bf16, g0, pb.P, pb.NBb, pb.B, w.blk_info, w.vt,
                         w.knorm, s),
           "vtrans");
  MOBA_HIP(launch_attn_diag(pb, w, q, k, g0, s), "attn_diag");
  MOBA_HIP(launch_attn_hist(pb, w, q, k, g0, s), "attn_hist");
  return MOBA_SUCCESS;
}

moba_status_t moba_attn_fwd_diag(const void *q, const void *k, const void *v,
                                 const moba_shape_t *sh, int32_t B, int32_t topk, float scale,
                                 const moba_layout_t *L, void *ws, int32_t g0, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, topk, L, ws, &f);
  if (st != MOBA_SUCCESS) return st;
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!q || !k || !v) return fail(MOBA_ERROR_INVALID_VALUE, "q, k, v must be non-NULL");
  Problem pb = make_problem(sh, B, topk, scale, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_vtrans(v, pb.vs, k, pb.ks, pb.bf16, g0, pb.P, pb.NBb, pb.B, w.blk_info, w.vt,
                         w.knorm, s),
           "vtrans");
  MOBA_HIP(launch_attn_diag(pb, w, q, k, g0, s), "attn_diag");
  return MOBA_SUCCESS;
}

moba_status_t moba_attn_fwd_hist(const void *q, const void *k, const moba_shape_t *sh, int32_t B,
                                 int32_t topk, float scale, const moba_layout_t *L, void *ws,
                                 int32_t g0, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, topk, L, ws, &f);
  if (st != MOBA_SUCCESS) return st;
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!q || !k) return fail(MOBA_ERROR_INVALID_VALUE, "q and k must be non-NULL");
  Problem pb = make_problem(sh, B, topk, scale, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_attn_hist(pb, w, q, k, g0, s), "attn_hist");
  return MOBA_SUCCESS;
}

moba_status_t moba_attn_prep(const void *k, const void *v, const moba_shape_t *sh, int32_t B,
                             int32_t topk, const moba_layout_t *L, void *ws, int32_t g0,
                             hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, topk, L, ws, &f);
  if (st != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!k || !v) return fail(MOBA_ERROR_INVALID_VALUE, "k and v must be non-NULL");
  Problem pb = make_problem(sh, B, topk, 0.f, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_vtrans(v, pb.vs, k, pb.ks, pb.bf16, g0, pb.P, pb.NBb, pb.B, w.blk_info, w.vt,
                         w.knorm, s),
           "vtrans");
  return MOBA_SUCCESS;
}

moba_status_t moba_attn_fwd_own_merge(const void *q, const void *k, const moba_shape_t *sh,
                                      int32_t B, int32_t topk, float scale,
                                      const moba_layout_t *L, void *ws, int32_t g0, void *out,
                                      float *lse, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, topk, L, ws, &f);
  if (st != MOBA_SUCCESS) return st;
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!q || !k) return fail(MOBA_ERROR_INVALID_VALUE, "q and k must be non-NULL");
  if (!out) return fail(MOBA_ERROR_INVALID_VALUE, "out is NULL");
  Problem pb = make_problem(sh, B, topk, scale, L);
  Work w = carve(pb, L, ws);
  if (pb.bf16) {
    MOBA_HIP(launch_attn_own_merge(pb, w, q, k, g0, out, lse, s), "attn_own_merge");
    MOBA_HIP(launch_nan_rows(pb, w, g0, out, lse, s), "nan_rows");
  } else {
    MOBA_HIP(launch_attn_diag(pb, w, q, k, g0, s), "attn_diag");
    MOBA_HIP(launch_merge(pb, w, g0, out, lse, s), "merge");
  }
  return MOBA_SUCCESS;
}

moba_status_t moba_merge(const moba_shape_t *sh, int32_t B, int32_t k, const moba_layout_t *L,
                         void *ws, int32_t g0, void *out, float *lse, hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, k, L, ws, &f);
  if (st != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!out) return fail(MOBA_ERROR_INVALID_VALUE, "out is NULL");
  Problem pb = make_problem(sh, B, k, 0.f, L);
  Work w = carve(pb, L, ws);
  MOBA_HIP(launch_merge(pb, w, g0, out, lse, s), "merge");
  return MOBA_SUCCESS;
}

moba_status_t moba_fwd_strided(const void *q, const void *k, const void *v, const int32_t *cu,
                               const moba_shape_t *sh, const moba_strides_t *strides, int32_t B,
                               int32_t topk, const moba_gate_t *gate_or_null, float scale,
                               void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t s) {
  const moba_gate_t mean{MOBA_GATE_MEAN, 0, 0, 0};
  const moba_gate_t *gate = gate_or_null ? gate_or_null : &mean;
  moba_status_t st = check_moba_args(sh, B, topk);
  if (st != MOBA_SUCCESS) return st;
  if ((st = check_gate(gate, topk)) != MOBA_SUCCESS) return st;
  if ((st = check_io(q, k, v, cu, out, sh)) != MOBA_SUCCESS) return st;
  if (strides && (st = check_strides(sh, B, strides)) != MOBA_SUCCESS) return st;
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  moba_layout_t L;
  if ((st = plan_impl(sh, B, topk, sh->num_kv_heads, &L)) != MOBA_SUCCESS) return st;
  // largest pass (a divisor of Hkv) whose workspace fits
  while (L.total_bytes > ws_bytes && L.kv_heads_per_pass > 1) {
    if ((st = plan_impl(sh, B, topk, L.kv_heads_per_pass - 1, &L)) != MOBA_SUCCESS) return st;
  }
  if (L.total_bytes > ws_bytes)
    return fail(MOBA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes; need at least %zu",
                ws_bytes, L.total_bytes);
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if (!ws) return fail(MOBA_ERROR_INVALID_VALUE, "workspace is NULL");
  Problem pb = make_problem(sh, B, topk, scale, &L);
  if (strides) {
    pb.qs = RowHead{strides->q_token, strides->q_head};
    pb.ks = RowHead{strides->k_token, strides->k_head};
    pb.vs = RowHead{strides->v_token, strides->v_head};
    pb.os = RowHead{strides->out_token, strides->out_head};
  }
  Work w = carve(pb, &L, ws);
  MOBA_HIP(launch_seqtable(cu, pb.S, B, pb.T, pb.maxblk, pb.NBb, w.blk_first, w.cu, w.status,
                           w.blk_info, s),
           "seqtable");
  if (check_enabled() && (st = read_status(w.status, s)) != MOBA_SUCCESS) return st;
  if (gate->kind != MOBA_GATE_WINDOW) MOBA_HIP(launch_meanpool(pb, w, k, s), "meanpool");
  if (gate->kind == MOBA_GATE_POOLED) MOBA_HIP(launch_minmaxpool(pb, w, k, s), "minmaxpool");
  for (int g0 = 0; g0 < pb.Hkv; g0 += pb.P)
    if ((st = run_pass(pb, w, q, k, v, g0, out, lse, s, *gate)) != MOBA_SUCCESS) return st;
  return MOBA_SUCCESS;
}

moba_status_t moba_fwd_gated(const void *q, const void *k, const void *v, const int32_t *cu,
                             const moba_shape_t *sh, int32_t B, int32_t topk,
                             const moba_gate_t *gate, float scale, void *out, float *lse,
                             void *ws, size_t ws_bytes, hipStream_t s) {
  if (!gate) return fail(MOBA_ERROR_INVALID_VALUE, "gate is NULL");
  return moba_fwd_strided(q, k, v, cu, sh, nullptr, B, topk, gate, scale, out, lse, ws, ws_bytes,
                          s);
}

moba_status_t moba_fwd_ex(const void *q, const void *k, const void *v, const int32_t *cu,
                          const moba_shape_t *sh, int32_t B, int32_t topk, float scale,
                          void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t s) {
  const moba_gate_t mean{MOBA_GATE_MEAN, 0, 0, 0};
  return moba_fwd_gated(q, k, v, cu, sh, B, topk, &mean, scale, out, lse, ws, ws_bytes, s);
}

moba_status_t moba_bwd_plan(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                            int32_t kv_heads_per_pass, moba_layout_t *layout) {
  if (!layout) return fail(MOBA_ERROR_INVALID_VALUE, "layout is NULL");
  return bwd_plan_impl(shape, block_size, topk, kv_heads_per_pass, layout);
}

size_t moba_bwd_workspace_size(const moba_shape_t *shape, int32_t block_size, int32_t topk,
                               int32_t kv_heads_per_pass) {
  moba_layout_t L;
  if (bwd_plan_impl(shape, block_size, topk, kv_heads_per_pass, &L) != MOBA_SUCCESS) return 0;
  return L.total_bytes;
}

moba_status_t moba_bwd(const void *q, const void *k, const void *v, const void *out,
                       const float *lse, const void *dout, const int32_t *cu,
                       const moba_shape_t *sh, int32_t B, int32_t topk, const moba_gate_t *gate,
                       float scale, void *dq, void *dk, void *dv, void *ws, size_t ws_bytes,
                       hipStream_t s) {
  moba_status_t st = check_moba_args(sh, B, topk);
  if (st != MOBA_SUCCESS) return st;
  const moba_gate_t mean{MOBA_GATE_MEAN, 0, 0, 0};
  if (!gate) gate = &mean;
  if ((st = check_gate(gate, topk)) != MOBA_SUCCESS) return st;
  if (sh->dtype != MOBA_DTYPE_BF16)
    return fail(MOBA_ERROR_UNSUPPORTED, "backward pass: bf16 only");
  if ((st = check_io(q, k, v, cu, out, sh)) != MOBA_SUCCESS) return st;
  if (sh->total_tokens > 0 && (!lse || !dout || !dq || !dk || !dv))
    return fail(MOBA_ERROR_INVALID_VALUE, "lse, dout, dq, dk and dv must be non-NULL");
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  moba_layout_t L;
  if ((st = bwd_plan_impl(sh, B, topk, sh->num_kv_heads, &L)) != MOBA_SUCCESS) return st;
  while (L.total_bytes > ws_bytes && L.kv_heads_per_pass > 1) {
    if ((st = bwd_plan_impl(sh, B, topk, L.kv_heads_per_pass - 1, &L)) != MOBA_SUCCESS) return st;
  }
  if (L.total_bytes > ws_bytes)
    return fail(MOBA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes; need at least %zu",
                ws_bytes, L.total_bytes);
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if (!ws) return fail(MOBA_ERROR_INVALID_VALUE, "workspace is NULL");
  Problem pb = make_problem(sh, B, topk, scale, &L);
  Work w = carve(pb, &L, ws);
  const BwdWork bw = carve_bwd(pb, &L, ws, &w);
  const BwdIo io{q, k, v, dout, lse, dq, dk, dv};
  MOBA_HIP(launch_seqtable(cu, pb.S, B, pb.T, pb.maxblk, pb.NBb, w.blk_first, w.cu, w.status,
                           w.blk_info, s),
           "seqtable");
  if (check_enabled() && (st = read_status(w.status, s)) != MOBA_SUCCESS) return st;
  if (gate->kind != MOBA_GATE_WINDOW) MOBA_HIP(launch_meanpool(pb, w, k, s), "meanpool");
  if (gate->kind == MOBA_GATE_POOLED) MOBA_HIP(launch_minmaxpool(pb, w, k, s), "minmaxpool");
  MOBA_HIP(launch_bwd_delta(pb, out, dout, bw.delta, s), "bwd_delta");
  for (int g0 = 0; g0 < pb.Hkv; g0 += pb.P) {
    if (gate->kind == MOBA_GATE_WINDOW)
      MOBA_HIP(launch_gate_window(pb, w, gate->n_sink, s), "gate_window");
    else if (gate->kind == MOBA_GATE_POOLED)
      MOBA_HIP(launch_gate_pooled(pb, w, q, g0, gate->extra_max, gate->extra_min, s),
               "gate_pooled");
    else
      MOBA_HIP(launch_gate(pb, w, q, g0, s), "gate");
    MOBA_HIP(launch_dispatch(pb, w, s), "dispatch");
    MOBA_HIP(launch_bwd_dq(pb, w, bw, io, g0, 3, s), "bwd_dq");
    MOBA_HIP(launch_bwd_dq_sum(pb, w, bw, io, g0, s), "bwd_dq_sum");
    MOBA_HIP(launch_bwd_dkdv(pb, w, bw, io, g0, s), "bwd_dkdv");
  }
  return MOBA_SUCCESS;
}

moba_status_t moba_bwd_delta(const void *out, const void *dout, const moba_shape_t *sh,
                             int32_t B, int32_t topk, const moba_layout_t *L, void *ws,
                             hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, topk, L, ws, &f, PLAN_BWD);
  if (st != MOBA_SUCCESS) return st;
  if (sh->dtype != MOBA_DTYPE_BF16) return fail(MOBA_ERROR_UNSUPPORTED, "backward pass: bf16 only");
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if (!out || !dout) return fail(MOBA_ERROR_INVALID_VALUE, "out and dout must be non-NULL");
  Problem pb = make_problem(sh, B, topk, 0.f, L);
  Work w = carve(pb, L, ws);
  const BwdWork bw = carve_bwd(pb, L, ws, &w);
  MOBA_HIP(launch_bwd_delta(pb, out, dout, bw.delta, s), "bwd_delta");
  return MOBA_SUCCESS;
}


moba_status_t moba_attn_bwd_dq(const void *q, const void *k, const void *v, const void *dout,
                               const float *lse, const moba_shape_t *sh, int32_t B, int32_t topk,
                               float scale, const moba_layout_t *L, void *ws, int32_t g0,
                               int32_t which, hipStream_t s) {
  Problem pb;
  Work w;
  BwdWork bw;
  bool nothing = false;
  moba_status_t st = bwd_stage(q, k, v, dout, lse, sh, B, topk, scale, L, ws, g0, &pb, &w, &bw,
                               &nothing);
  if (st != MOBA_SUCCESS || nothing) return st;
  if (which < 1 || which > 3) return fail(MOBA_ERROR_INVALID_VALUE, "which must be 1, 2 or 3");
  const BwdIo io{q, k, v, dout, lse, nullptr, nullptr, nullptr};
  MOBA_HIP(launch_bwd_dq(pb, w, bw, io, g0, which, s), "bwd_dq");
  return MOBA_SUCCESS;
}

moba_status_t moba_attn_bwd_dq_sum(const moba_shape_t *sh, int32_t B, int32_t topk,
                                   const moba_layout_t *L, void *ws, int32_t g0, void *dq,
                                   hipStream_t s) {
  moba_layout_t f;
  moba_status_t st = check_stage(sh, B, topk, L, ws, &f, PLAN_BWD);
  if (st != MOBA_SUCCESS) return st;
  if (sh->dtype != MOBA_DTYPE_BF16) return fail(MOBA_ERROR_UNSUPPORTED, "backward pass: bf16 only");
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  if ((st = check_pass(sh, L, g0)) != MOBA_SUCCESS) return st;
  if (!dq) return fail(MOBA_ERROR_INVALID_VALUE, "dq is NULL");
  Problem pb = make_problem(sh, B, topk, 0.f, L);
  Work w = carve(pb, L, ws);
  const BwdWork bw = carve_bwd(pb, L, ws, &w);
  const BwdIo io{nullptr, nullptr, nullptr, nullptr, nullptr, dq, nullptr, nullptr};
  MOBA_HIP(launch_bwd_dq_sum(pb, w, bw, io, g0, s), "bwd_dq_sum");
  return MOBA_SUCCESS;
}

moba_status_t moba_attn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout,
                                 const float *lse, const moba_shape_t *sh, int32_t B,
                                 int32_t topk, float scale, const moba_layout_t *L, void *ws,
                                 int32_t g0, void *dk, void *dv, hipStream_t s) {
  Problem pb;
  Work w;
  BwdWork bw;
  bool nothing = false;
  moba_status_t st = bwd_stage(q, k, v, dout, lse, sh, B, topk, scale, L, ws, g0, &pb, &w, &bw,
                               &nothing);
  if (st != MOBA_SUCCESS || nothing) return st;
  if (!dk || !dv) return fail(MOBA_ERROR_INVALID_VALUE, "dk and dv must be non-NULL");
  const BwdIo io{q, k, v, dout, lse, nullptr, dk, dv};
  MOBA_HIP(launch_bwd_dkdv(pb, w, bw, io, g0, s), "bwd_dkdv");
  return MOBA_SUCCESS;
}

size_t moba_decode_workspace_size(const moba_shape_t *cache_shape, int32_t block_size,
                                  int32_t topk) {
  DecodeLayout D;
  if (!cache_shape || decode_layout(cache_shape, block_size, topk, &D) != MOBA_SUCCESS) return 0;
  return D.total;
}

moba_status_t moba_decode_prepare(const void *k_cache, const int32_t *cu,
                                  const moba_shape_t *sh, int32_t B, int32_t topk, void *ws,
                                  size_t ws_bytes, hipStream_t s) {
  if (!sh) return fail(MOBA_ERROR_INVALID_VALUE, "shape is NULL");
  DecodeLayout D;
  moba_status_t st = decode_layout(sh, B, topk, &D);
  if (st != MOBA_SUCCESS) return st;
  if (ws_bytes < D.total)
    return fail(MOBA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes; need %zu", ws_bytes,
                D.total);
  if (sh->num_seqs > 0 && !cu) return fail(MOBA_ERROR_INVALID_VALUE, "cu_seqlens is NULL");
  if (sh->num_seqs == 0) return MOBA_SUCCESS;
  if (!ws) return fail(MOBA_ERROR_INVALID_VALUE, "workspace is NULL");
  if (sh->total_tokens > 0 && !k_cache) return fail(MOBA_ERROR_INVALID_VALUE, "k_cache is NULL");
  Problem pb;
  Work w;
  decode_setup(sh, B, topk, 0.f, D, ws, &pb, &w);
  MOBA_HIP(launch_seqtable(cu, pb.S, B, pb.T, pb.maxblk, pb.NBb, w.blk_first, w.cu, w.status,
                           w.blk_info, s),
           "seqtable");
  if (check_enabled() && (st = read_status(w.status, s)) != MOBA_SUCCESS) return st;
  if (sh->total_tokens > 0) MOBA_HIP(launch_meanpool(pb, w, k_cache, s), "meanpool");
  return MOBA_SUCCESS;
}

moba_status_t moba_decode(const void *q, const void *k_cache, const void *v_cache,
                          const moba_shape_t *sh, int32_t B, int32_t topk, float scale,
                          void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t s) {
  if (!sh) return fail(MOBA_ERROR_INVALID_VALUE, "shape is NULL");
  DecodeLayout D;
  moba_status_t st = decode_layout(sh, B, topk, &D);
  if (st != MOBA_SUCCESS) return st;
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  if (ws_bytes < D.total)
    return fail(MOBA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes; need %zu", ws_bytes,
                D.total);
  if (sh->num_seqs == 0) return MOBA_SUCCESS;
  if (!q || !out || !ws) return fail(MOBA_ERROR_INVALID_VALUE, "q, out and workspace must be non-NULL");
  if (sh->total_tokens > 0 && (!k_cache || !v_cache))
    return fail(MOBA_ERROR_INVALID_VALUE, "k_cache and v_cache must be non-NULL");
  Problem pb;
  Work w;
  decode_setup(sh, B, topk, scale, D, ws, &pb, &w);
  MOBA_HIP(launch_decode(pb, w, q, k_cache, v_cache, out, lse, s), "decode");
  return MOBA_SUCCESS;
}

moba_status_t moba_fwd(const void *q, const void *k, const void *v, const int32_t *cu,
                       const moba_shape_t *sh, int32_t B, int32_t topk, void *out, float *lse,
                       hipStream_t s) {
  moba_status_t st = check_moba_args(sh, B, topk);
  if (st != MOBA_SUCCESS) return st;
  if ((st = check_io(q, k, v, cu, out, sh)) != MOBA_SUCCESS) return st;
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  const size_t cap = workspace_limit_bytes();
  moba_layout_t L;
  if ((st = plan_impl(sh, B, topk, sh->num_kv_heads, &L)) != MOBA_SUCCESS) return st;
  while (L.total_bytes > cap && L.kv_heads_per_pass > 1)
    if ((st = plan_impl(sh, B, topk, L.kv_heads_per_pass - 1, &L)) != MOBA_SUCCESS) return st;
  void *ws = nullptr;
  MOBA_HIP(hipMallocAsync(&ws, L.total_bytes, s), "hipMallocAsync");
  st = moba_fwd_ex(q, k, v, cu, sh, B, topk, 0.f, out, lse, ws, L.total_bytes, s);
  hipError_t e = hipFreeAsync(ws, s);
  if (st != MOBA_SUCCESS) return st;
  if (e != hipSuccess) return hip_fail(e, "hipFreeAsync");
  return MOBA_SUCCESS;
}

size_t moba_dense_causal_workspace_size(const moba_shape_t *sh) {
  if (check_shape(sh) != MOBA_SUCCESS) return 0;
  return dense_ws_bytes(sh);
}

moba_status_t moba_dense_causal_fwd(const void *q, const void *k, const void *v, const int32_t *cu,
                                    const moba_shape_t *sh, float scale, void *out, float *lse,
                                    void *ws, size_t ws_bytes, hipStream_t s) {
  moba_status_t st = check_shape(sh);
  if (st != MOBA_SUCCESS) return st;
  if ((st = check_io(q, k, v, cu, out, sh)) != MOBA_SUCCESS) return st;
  if (!(scale >= 0.f) || isinf(scale)) return fail(MOBA_ERROR_INVALID_VALUE, "bad softmax_scale");
  const size_t need = dense_ws_bytes(sh);
  if (ws && ws_bytes < need)
    return fail(MOBA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes; need %zu", ws_bytes, need);
  if (sh->total_tokens == 0) return MOBA_SUCCESS;
  bool own = false;
  if (!ws) {
    MOBA_HIP(hipMallocAsync(&ws, need, s), "hipMallocAsync");
    own = true;
  }
  const int S = sh->num_seqs;
  const int64_t T = sh->total_tokens;
  const int64_t NB64 = dense_nb64(sh), NBq = dense_nbq(sh);
  const int bf16 = sh->dtype == MOBA_DTYPE_BF16;
  const int rows = attn_rows(bf16);
  const Table t64 = table_at(ws, S);
  const Table tq = table_at((char *)ws + align_up(table_bytes(S, NB64)), S);
  void *vt = (char *)ws + dense_table_bytes(sh);
  float *knorm = (float *)((char *)vt + vt_bytes(bf16 ? 2 : 4, sh->num_kv_heads, NB64, kKeyTile));
  const int no_bound = 0x7fffffff;  // the grid covers every query tile: no length bound
  hipError_t e = launch_seqtable(cu, S, kKeyTile, T, no_bound, NB64, t64.first, t64.cu, t64.status,
                                 t64.info, s);
  if (e == hipSuccess)
    e = launch_seqtable(cu, S, rows, T, no_bound, NBq, tq.first, tq.cu, tq.status, tq.info, s);
  if (e == hipSuccess && check_enabled()) {
    moba_status_t cst = read_status(t64.status, s);
    if (cst != MOBA_SUCCESS) {
      if (own) (void)hipFreeAsync(ws, s);
      return cst;
    }
  }
  if (e == hipSuccess)
    e = launch_vtrans(v, RowHead{(int64_t)sh->num_kv_heads * kHeadDim, kHeadDim}, k,
                      RowHead{(int64_t)sh->num_kv_heads * kHeadDim, kHeadDim}, bf16, 0,
                      sh->num_kv_heads, NB64, kKeyTile, t64.info, vt, knorm, s);
  if (e == hipSuccess)
    e = launch_dense(q, k, vt, knorm, t64.first, tq.info, bf16, T, NBq, sh->num_q_heads,
                     sh->num_kv_heads, NB64, scale > 0.f ? scale : 1.0f / sqrtf((float)kHeadDim),
                     out, lse, s);
  // a failed table check leaves every tile out: out and lse become NaN
  if (e == hipSuccess)
    e = launch_poison(t64.status, out, T * sh->num_q_heads * kHeadDim / (bf16 ? 2 : 1),
                      bf16 ? kNanBf16x2 : kNanF32, s);
  if (e == hipSuccess && lse)
    e = launch_poison(t64.status, lse, T * sh->num_q_heads, kNanF32, s);
  if (own) {
    hipError_t e2 = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return hip_fail(e, "dense_causal");
  return MOBA_SUCCESS;
}

}  // extern "C"
