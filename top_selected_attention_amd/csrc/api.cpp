// C-ABI layer: argument validation, workspace sizing and kernel dispatch.
//
// The two-phase pattern follows the CANN operator pages ("calls" section of
// each): XXX_workspace_size validates on the host and sizes the workspace;
// XXX re-validates and enqueues.  Constraints are cited where they are
// checked.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/top_selected_attention.h"
#include "tsa_internal.h"

using namespace tsa;

namespace {

constexpr size_t kAlign = 256;

// Carves aligned sub-buffers out of one workspace; with base == nullptr it
// only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

inline long cdiv(long a, long b) { return (a + b - 1) / b; }
// The kernels move tensor rows, caches and workspace buffers in 16-byte
// pieces: such pointers must be 16-byte aligned (NULL passes).
inline bool a16(const void* p) { return ((uintptr_t)p & 15) == 0; }
inline bool fits_i32(long x) { return x >= 0 && x <= 0x7fffffffL; }

int hip_status(hipError_t e) { return e == hipSuccess ? TSA_OK : TSA_ERR_HIP; }

// Records the caller's timing events around stages (no-op when n == 0).
struct StageTimer {
  void* const* ev;
  int n;
  hipStream_t st;
  hipError_t mark(int stage, int end) const {
    if (!ev || stage >= n) return hipSuccess;
    return hipEventRecord((hipEvent_t)ev[2 * stage + end], st);
  }
  // A call with no work still records every requested stage, back to back.
  hipError_t skip_all(int stages) const {
    hipError_t e = hipSuccess;
    for (int i = 0; i < stages && e == hipSuccess; i++) {
      e = mark(i, 0);
      if (e == hipSuccess) e = mark(i, 1);
    }
    return e;
  }
};

template <class A>
StageTimer timer_of(const A* a, hipStream_t st) {
  return StageTimer{a->events, a->events ? a->n_events : 0, st};
}

// ---------------------------------------------------------------------------
// Block-sparse attention
// ---------------------------------------------------------------------------

// Shape checks shared by forward, backward and compaction.
int check_bsa_common(int dtype, int ql, int kl, int B, int N1, int N2, int Sq, int Skv, int D,
                     int bq, int bkv, int mode, float scale) {
  if (dtype != TSA_BF16 && dtype != TSA_FP16) return TSA_ERR_INVALID;
  // "aclnnBlockSparseAttentionGrad", layout section: qInputLayout and
  // kvInputLayout are TND or BNSD (the operator itself builds only BNSD, per
  // its constraints; both are built here, q and k/v in the same layout).
  if ((ql != TSA_LAYOUT_BNSD && ql != TSA_LAYOUT_TND) ||
      (kl != TSA_LAYOUT_BNSD && kl != TSA_LAYOUT_TND))
    return TSA_ERR_INVALID;
  if (ql != kl) return TSA_ERR_UNSUPPORTED;
  if (B < 0 || Sq < 0 || Skv < 0 || N1 < 1 || N2 < 1) return TSA_ERR_INVALID;
  // constraints: N1 >= N2 and N1 % N2 == 0
  if (N1 % N2 != 0) return TSA_ERR_INVALID;
  // constraints: headdim = 128
  if (D != 128) return TSA_ERR_INVALID;
  if (bq < 1 || bkv < 1 || bq > 65536 || bkv > 65536) return TSA_ERR_INVALID;
  if (mode != 0 && mode != 2) return TSA_ERR_INVALID;
  // a positive scale: the kernels take the row max of the unscaled scores
  if (!std::isfinite(scale) || !(scale > 0.f)) return TSA_ERR_INVALID;
  const long QB = cdiv(Sq, bq), KB = cdiv(Skv, bkv);
  if (!fits_i32((long)B * N1 * QB * KB) || !fits_i32((long)B * N1 * QB + 1)) return TSA_ERR_INVALID;
  if (!fits_i32(QB * bq) || !fits_i32(KB * bkv)) return TSA_ERR_INVALID;
  return TSA_OK;
}

// TND: host prefix sums cu_seqlens_q / _kv [B+1] from 0 (the layout
// section: actualSeqLengths are mandatory with TND); every sequence at most
// Sq / Skv long (those give the mask's padded block counts).
template <class A>
int check_bsa_tnd(const A* a) {
  if (a->q_layout != TSA_LAYOUT_TND) return TSA_OK;
  if (!a->cu_seqlens_q || !a->cu_seqlens_kv) return TSA_ERR_NULL;
  const int32_t* cq = a->cu_seqlens_q;
  const int32_t* ck = a->cu_seqlens_kv;
  if (cq[0] != 0 || ck[0] != 0) return TSA_ERR_INVALID;
  for (int b = 0; b < a->B; b++) {
    const long sq = (long)cq[b + 1] - cq[b], sk = (long)ck[b + 1] - ck[b];
    if (sq < 0 || sk < 0 || sq > a->Sq || sk > a->Skv) return TSA_ERR_INVALID;
  }
  if (!fits_i32((long)cq[a->B] * a->N1 * a->D) || !fits_i32((long)ck[a->B] * a->N2 * a->D))
    return TSA_ERR_INVALID;
  return TSA_OK;
}

// Query / key rows the call touches (TND: the tokens; BNSD: B*Sq, B*Skv).
template <class A>
long bsa_q_rows(const A* a) {
  return a->q_layout == TSA_LAYOUT_TND ? (long)a->cu_seqlens_q[a->B] : (long)a->B * a->Sq;
}
template <class A>
long bsa_kv_rows(const A* a) {
  return a->q_layout == TSA_LAYOUT_TND ? (long)a->cu_seqlens_kv[a->B] : (long)a->B * a->Skv;
}

struct BsaWs {
  int* meta;     // TND: cu_q [B+1], cu_kv [B+1]
  int* parts;
  int* sums;
  int* row_ptr;
  int* col;
  int* rev_ptr;
  int* rev;
  int* order_q;
  int* order_kv;
  float* delta;
  // backward dK/dV segments
  int* seg_off;
  int* part_off;
  int* seg_meta;
  float* part;
};

template <class A>
size_t bsa_carve(const A* a, void* ws, BsaWs* out, bool with_delta) {
  const int QB = (int)cdiv(a->Sq, a->block_q), KB = (int)cdiv(a->Skv, a->block_kv);
  const long R = (long)a->B * a->N1 * QB, C = (long)a->B * a->N2 * KB;
  const long nparts = bsa_compact_parts_len(a->B, a->N1, a->N2, QB, KB);
  Carver c(ws);
  BsaWs w;
  w.meta = c.take<int>(2 * ((long)a->B + 1));
  w.parts = c.take<int>(nparts);
  w.sums = c.take<int>(scan_sums_len(nparts));
  w.row_ptr = c.take<int>(R + 1);
  w.col = c.take<int>(R * KB);
  w.rev_ptr = c.take<int>(C + 1);
  w.rev = c.take<int>(R * KB);
  w.order_q = c.take<int>(R);
  w.order_kv = c.take<int>(C);
  // the dK/dV segment plan is made with the lists (forward or backward), so
  // the forward's workspace layout holds it too
  const BsaDkdvShape ds = bsa_dkdv_shape(a->B, a->N1, a->N2, QB, KB, a->block_kv);
  w.seg_off = c.take<int>(ds.n_items + 1);
  w.part_off = c.take<int>(ds.n_items + 1);
  w.seg_meta = c.take<int>(2 + kBsaDkdvSlots);
  // per row: LSE in base 2 and softmax_grad, interleaved
  w.delta = with_delta ? c.take<float>(2L * a->B * a->N1 * a->Sq) : nullptr;
  w.part = with_delta ? c.take<float>(ds.max_parts * 2 * ds.nk * 128) : nullptr;
  if (out) *out = w;
  return c.off + kAlign;
}

int check_bsa_fwd(const bsa_fwd_args* a) {
  if (!a) return TSA_ERR_NULL;
  if (a->reuse_lists != 0 && a->reuse_lists != 1) return TSA_ERR_INVALID;
  int s = check_bsa_common(a->dtype, a->q_layout, a->kv_layout, a->B, a->N1, a->N2, a->Sq, a->Skv,
                           a->D, a->block_q, a->block_kv, a->sparse_mode, a->scale);
  if (s) return s;
  s = check_bsa_tnd(a);
  if (s) return s;
  if (a->atten_mask && (a->atten_mask_stride_b < 0 || a->atten_mask_stride_n < 0))
    return TSA_ERR_INVALID;
  const bool empty = bsa_q_rows(a) == 0;
  if (!empty && (!a->q || !a->out || !a->lse || !a->block_mask)) return TSA_ERR_NULL;
  if (!empty && bsa_kv_rows(a) > 0 && (!a->k || !a->v)) return TSA_ERR_NULL;
  if (!a16(a->q) || !a16(a->k) || !a16(a->v) || !a16(a->out) || !a16(a->block_mask))
    return TSA_ERR_INVALID;
  return TSA_OK;
}

int check_bsa_bwd(const bsa_bwd_args* a) {
  if (!a) return TSA_ERR_NULL;
  if (a->reuse_lists != 0 && a->reuse_lists != 1) return TSA_ERR_INVALID;
  int s = check_bsa_common(a->dtype, a->q_layout, a->kv_layout, a->B, a->N1, a->N2, a->Sq, a->Skv,
                           a->D, a->block_q, a->block_kv, a->sparse_mode, a->scale);
  if (s) return s;
  s = check_bsa_tnd(a);
  if (s) return s;
  if (a->atten_mask && (a->atten_mask_stride_b < 0 || a->atten_mask_stride_n < 0))
    return TSA_ERR_INVALID;
  const bool empty_q = bsa_q_rows(a) == 0, empty_k = bsa_kv_rows(a) == 0;
  if (!empty_q && (!a->q || !a->out || !a->dout || !a->lse || !a->dq || !a->block_mask))
    return TSA_ERR_NULL;
  if (!empty_k && (!a->k || !a->v || !a->dk || !a->dv)) return TSA_ERR_NULL;
  if (!a16(a->q) || !a16(a->k) || !a16(a->v) || !a16(a->out) || !a16(a->dout) || !a16(a->dq) ||
      !a16(a->dk) || !a16(a->dv) || !a16(a->block_mask))
    return TSA_ERR_INVALID;
  return TSA_OK;
}

// The dK/dV segment plan's outputs in the workspace (none without KV blocks).
template <class A>
BsaSegPlan seg_plan(const A* a, const BsaWs& w, const BsaParams& p) {
  const BsaDkdvShape ds = bsa_dkdv_shape(a->B, a->N1, a->N2, p.QB, p.KB, a->block_kv);
  BsaSegPlan sp{nullptr, nullptr, nullptr, ds.ksub, (int)ds.n_items};
  if (p.KB > 0) {
    sp.seg_off = w.seg_off;
    sp.part_off = w.part_off;
    sp.seg_meta = w.seg_meta;
  }
  return sp;
}

// TND: uploads cu_seqlens into the workspace and points the kernels at them.
template <class A>
hipError_t bsa_upload_seqlens(const A* a, const BsaWs& w, BsaParams* p, hipStream_t st) {
  if (a->q_layout != TSA_LAYOUT_TND) return hipSuccess;
  const int n = a->B + 1;
  int* host = new int[2 * n];
  for (int b = 0; b < n; b++) {
    host[b] = a->cu_seqlens_q[b];
    host[n + b] = a->cu_seqlens_kv[b];
  }
  hipError_t e = hipMemcpyAsync(w.meta, host, sizeof(int) * 2 * n, hipMemcpyHostToDevice, st);
  // the copy from pageable memory is staged before hipMemcpyAsync returns
  delete[] host;
  p->cu_q = w.meta;
  p->cu_kv = w.meta + n;
  return e;
}

// atten_mask fields of the kernel parameters.
template <class A>
void bsa_set_atten_mask(const A* a, BsaParams* p) {
  p->am = a->atten_mask;
  if (!p->am) return;
  p->am_sb = (long)a->atten_mask_stride_b;
  p->am_sn = (long)a->atten_mask_stride_n;
  p->am_pitch = a->Skv;
  p->am_al4 = (((uintptr_t)p->am | (uintptr_t)p->am_sb | (uintptr_t)p->am_sn |
                (uintptr_t)a->Skv | (uintptr_t)a->block_kv) & 3) == 0;
}

// Builds the forward and reverse lists, the tile order and the dK/dV
// segment plan in the workspace.  Without query or key rows every list is
// empty (and the mask, which such a call need not pass, is not read).
template <class A>
hipError_t bsa_build_lists(const A* a, const BsaWs& w, const BsaParams& p, hipStream_t st) {
  const long R = (long)a->B * a->N1 * p.QB, C = (long)a->B * a->N2 * p.KB;
  hipError_t e;
  if (R > 0 && C > 0 && bsa_q_rows(a) > 0 && bsa_kv_rows(a) > 0) {
    e = launch_bsa_compact(a->block_mask, a->B, a->N1, a->N2, p.QB, p.KB, w.parts, w.sums,
                           w.row_ptr, w.col, w.rev_ptr, w.rev, st);
  } else {
    // fill kernels rather than memset nodes, so that a captured call replays them
    e = launch_fill_i32(w.row_ptr, (int)(R + 1), 0, st);
    if (e == hipSuccess) e = launch_fill_i32(w.rev_ptr, (int)(C + 1), 0, st);
  }
  if (e == hipSuccess)
    e = launch_tile_order(w.row_ptr, (int)R, w.order_q, w.rev_ptr, (int)C, w.order_kv,
                          seg_plan(a, w, p), st);
  return e;
}

BsaParams bsa_params(int B, int N1, int N2, int Sq, int Skv, int bq, int bkv, int mode,
                     float scale) {
  BsaParams p;
  std::memset(&p, 0, sizeof(p));
  p.B = B; p.N1 = N1; p.N2 = N2; p.G = N1 / N2;
  p.Sq = Sq; p.Skv = Skv; p.D = 128;
  p.bq = bq; p.bkv = bkv;
  p.QB = (int)cdiv(Sq, bq); p.KB = (int)cdiv(Skv, bkv);
  p.causal = mode == 2;
  p.scale = scale;
  return p;
}

// ---------------------------------------------------------------------------
// NSA selected attention
// ---------------------------------------------------------------------------

template <class A>
int check_nsa(const A* a, bool tensors = true) {
  if (!a) return TSA_ERR_NULL;
  if (a->dtype != TSA_BF16 && a->dtype != TSA_FP16) return TSA_ERR_INVALID;
  // "aclnnNsaSelectedAttention", constraints: inputLayout supports only TND.
  if (a->layout == TSA_LAYOUT_BNSD || a->layout == TSA_LAYOUT_BSND) return TSA_ERR_UNSUPPORTED;
  if (a->layout != TSA_LAYOUT_TND) return TSA_ERR_INVALID;
  // constraints (TND shape ranges): B in [1, 1024], N in [1, 128], G <= 32.
  if (a->B < 1 || a->B > 1024) return TSA_ERR_INVALID;
  if (a->N1 < 1 || a->N1 > 128 || a->N2 < 1 || a->N1 % a->N2 != 0) return TSA_ERR_INVALID;
  if (a->N1 / a->N2 > 32) return TSA_ERR_INVALID;
  // constraints (TND shape ranges): the query/key and the value head dims are
  // each fixed to a value the page's extraction lost; read here as
  // D = 192 with Dv = 128 (two distinct values), and D = Dv = 128 is built too.
  if (a->Dv != 128 || (a->D != 128 && a->D != 192)) return TSA_ERR_UNSUPPORTED;
  // constraints: selected_block_size <= 128 and a multiple of 16;
  // selected_block_count in [1, 128]; their product at most 8K.
  if (a->sbs < 16 || a->sbs > 128 || a->sbs % 16 != 0) return TSA_ERR_INVALID;
  if (a->sbc < 1 || a->sbc > 128 || a->sbs * a->sbc > 8192) return TSA_ERR_INVALID;
  // constraints: sparseMode 0 or 2.
  if (a->sparse_mode != 0 && a->sparse_mode != 2) return TSA_ERR_INVALID;
  if (!std::isfinite(a->scale) || !(a->scale > 0.f)) return TSA_ERR_INVALID;
  if (!a->cu_seqlens_q || !a->cu_seqlens_kv) return TSA_ERR_NULL;
  const int32_t* cq = a->cu_seqlens_q;
  const int32_t* ck = a->cu_seqlens_kv;
  if (cq[0] != 0 || ck[0] != 0) return TSA_ERR_INVALID;
  for (int b = 0; b < a->B; b++) {
    const long sq = (long)cq[b + 1] - cq[b], sk = (long)ck[b + 1] - ck[b];
    if (sq < 0 || sk < 0) return TSA_ERR_INVALID;
    // constraints: S in [1, 128K], S >= sbs * sbc and a multiple of sbs.
    if (sk > 131072 || sq > 131072) return TSA_ERR_INVALID;
    if (sk < (long)a->sbs * a->sbc || sk % a->sbs != 0) return TSA_ERR_INVALID;
  }
  if (cq[a->B] != a->T || ck[a->B] != a->Tk) return TSA_ERR_INVALID;
  if (!fits_i32((long)a->T * a->N2 * a->sbc) || !fits_i32((long)a->T * a->N1 * a->D))
    return TSA_ERR_INVALID;
  if (a->T > 0 && !a->topk) return TSA_ERR_NULL;
  if (!tensors) return TSA_OK;  // the list calls read only shapes and topk
  if (a->T > 0 && (!a->q || !a->out || !a->lse || !a->k || !a->v)) return TSA_ERR_NULL;
  if (!a16(a->q) || !a16(a->k) || !a16(a->v) || !a16(a->out)) return TSA_ERR_INVALID;
  return TSA_OK;
}

int nsa_blocks_total(const int32_t* ck, int B, int sbs) {
  long nb = 0;
  for (int b = 0; b < B; b++) nb += cdiv((long)ck[b + 1] - ck[b], sbs);
  return (int)nb;
}

// The token-group forward and dQ kernels take head groups of up to 16 query
// heads of 128 dims (values 128); other shapes use the per-token kernels.
template <class A>
bool nsa_grouped(const A* a) {
  return a->N2 > 0 && a->N1 / a->N2 <= 16 && a->D == 128 && a->Dv == 128;
}
// Token groups per KV head: sum over sequences of ceil(Sq_b / kNsaGroup).
template <class A>
long nsa_groups_total(const A* a) {
  long ng = 0;
  for (int b = 0; b < a->B; b++) ng += cdiv((long)a->cu_seqlens_q[b + 1] - a->cu_seqlens_q[b], kNsaGroup);
  return ng;
}

struct NsaWs {
  int* meta;     // cu_q [B+1], cu_kv [B+1], blk_off [B+1], group offsets [B+1]
  int* cnt;
  int* sums;
  int* row_ptr;
  int* col;
  int* rcnt;
  int* rev_ptr;
  int* rev;
  int* ekey;      // per forward entry: reverse key and token id
  int* etok;
  int* rhist;     // reverse-list sort: (key, tile) counters and their scan sums
  int* rsums;
  NsaRevSort rs;
  int* bad;
  float* delta;
  int* seg_off;
  int* seg_sums;
  int* seg_ctr;
  float* part;
  int max_segments;
  NsaGroups grp;
};

template <class A>
size_t nsa_carve(const A* a, void* ws, NsaWs* out, bool with_delta) {
  const long R = (long)a->T * a->N2;
  const long NB = nsa_blocks_total(a->cu_seqlens_kv, a->B, a->sbs);
  const long RR = (long)a->N2 * NB;
  Carver c(ws);
  NsaWs w;
  w.meta = c.take<int>(4 * (a->B + 1));
  w.cnt = c.take<int>(R);
  w.sums = c.take<int>(scan_sums_len(R > RR ? R : RR));
  w.row_ptr = c.take<int>(R + 1);
  w.col = c.take<int>(R * a->sbc);
  w.rcnt = c.take<int>(RR);
  w.rev_ptr = c.take<int>(RR + 1);
  w.rev = c.take<int>(R * a->sbc);
  w.rs = nsa_rev_sort_plan(R * a->sbc, RR);
  w.ekey = c.take<int>(R * a->sbc);
  w.etok = c.take<int>(R * a->sbc);
  const long nh = w.rs.usable ? (long)w.rs.NK * w.rs.n_tiles : 0;
  w.rhist = c.take<int>(nh);
  w.rsums = c.take<int>(w.rs.usable ? scan_sums_len(nh) : 0);
  w.bad = c.take<int>(1);
  // the group lists precede the backward-only buffers, so that a forward and
  // a backward carving one workspace place them alike
  std::memset(&w.grp, 0, sizeof(w.grp));
  if (nsa_grouped(a)) {
    const long units = (long)a->N2 * nsa_groups_total(a);
    w.grp.NG = (int)nsa_groups_total(a);
    w.grp.cap = kNsaGroup * a->sbc * (int)cdiv(a->sbs, kNsaGroupChunk);
    w.grp.gcu = w.meta + 3 * (a->B + 1);
    w.grp.cnt = c.take<int>(units);
    w.grp.ent = c.take<int>(units * w.grp.cap * 2);
  }
  w.delta = with_delta ? c.take<float>(2L * a->T * a->N1) : nullptr;
  w.max_segments = with_delta ? nsa_max_segments(R * a->sbc, RR) : 0;
  w.seg_off = with_delta ? c.take<int>(RR + 1) : nullptr;
  w.seg_sums = with_delta ? c.take<int>(scan_sums_len(RR)) : nullptr;
  w.seg_ctr = with_delta ? c.take<int>(1) : nullptr;
  w.part = with_delta ? c.take<float>((long)w.max_segments * a->sbs * (a->D + a->Dv)) : nullptr;
  if (out) *out = w;
  return c.off + kAlign;
}

template <class A>
void nsa_geom(const A* a, const NsaWs& w, NsaGeom* g);

// Uploads cu_seqlens and block offsets into the workspace and fills the
// device geometry.
template <class A>
int nsa_setup(const A* a, const NsaWs& w, NsaGeom* g, hipStream_t st) {
  const int n = a->B + 1;
  int* host = new int[4 * n];
  host[0 * n] = 0;
  for (int b = 0; b < n; b++) {
    host[0 * n + b] = a->cu_seqlens_q[b];
    host[1 * n + b] = a->cu_seqlens_kv[b];
  }
  host[2 * n] = 0;
  host[3 * n] = 0;
  for (int b = 0; b < a->B; b++) {
    host[2 * n + b + 1] =
        host[2 * n + b] + (int)cdiv((long)a->cu_seqlens_kv[b + 1] - a->cu_seqlens_kv[b], a->sbs);
    host[3 * n + b + 1] =
        host[3 * n + b] + (int)cdiv((long)a->cu_seqlens_q[b + 1] - a->cu_seqlens_q[b], kNsaGroup);
  }
  hipError_t e = hipMemcpyAsync(w.meta, host, sizeof(int) * 4 * n, hipMemcpyHostToDevice, st);
  // the copy from pageable memory is staged before hipMemcpyAsync returns
  delete[] host;
  if (e != hipSuccess) return TSA_ERR_HIP;
  nsa_geom(a, w, g);
  return TSA_OK;
}

// Device geometry over the workspace's uploaded metadata.
template <class A>
void nsa_geom(const A* a, const NsaWs& w, NsaGeom* g) {
  const int n = a->B + 1;
  g->cu_q = w.meta;
  g->cu_kv = w.meta + n;
  g->blk_off = w.meta + 2 * n;
  g->B = a->B;
  g->T = a->T;
  g->N2 = a->N2;
  g->sbc = a->sbc;
  g->sbs = a->sbs;
  g->causal = a->sparse_mode == 2;
  g->NB = nsa_blocks_total(a->cu_seqlens_kv, a->B, a->sbs);
}

enum NsaListParts { kNsaForward = 1, kNsaReverse = 2, kNsaAll = 3 };

template <class A>
int nsa_lists(const A* a, const NsaWs& w, const NsaGeom& g, int parts, hipStream_t st) {
  if (a->validate && (parts & kNsaForward)) {
    hipError_t e = launch_fill_i32(w.bad, 1, 0, st);
    if (e == hipSuccess) e = launch_nsa_check(a->topk, g, w.bad, st);
    int bad = 0;
    if (e == hipSuccess) e = hipMemcpyAsync(&bad, w.bad, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return TSA_ERR_HIP;
    if (bad) return TSA_ERR_DATA;
  }
  hipError_t e = hipSuccess;
  if (parts & kNsaForward)
    e = launch_nsa_forward_lists(a->topk, g, w.cnt, w.sums, w.row_ptr, w.col, w.ekey, w.etok, st);
  if (e == hipSuccess && (parts & kNsaForward) && w.grp.NG > 0)
    e = launch_nsa_group_lists(g, w.row_ptr, w.col, w.grp, st);
  if (e == hipSuccess && (parts & kNsaReverse))
    e = launch_nsa_reverse_lists(g, w.row_ptr, w.col, w.sums, w.rcnt, w.rev_ptr, w.rev, w.ekey,
                                 w.etok, w.rs, w.rhist, w.rsums, st);
  return hip_status(e);
}

// ---------------------------------------------------------------------------
// Sparse flash attention
// ---------------------------------------------------------------------------

// Decode tokens of an SFA call: B * Sq (BSND) or T (TND).
long sfa_tokens(const sfa_paged_fwd_args* a) {
  return a->q_layout == TSA_LAYOUT_TND ? (long)a->T : (long)a->B * a->Sq;
}

int check_sfa(const sfa_paged_fwd_args* a) {
  if (!a) return TSA_ERR_NULL;
  if (a->dtype != TSA_BF16 && a->dtype != TSA_FP16) return TSA_ERR_INVALID;
  // "SparseAttnSharedkvMetadata", parameter list: layout_q BSND or TND
  // (cu_seqlens_q prefix sums for TND).
  if (a->q_layout != TSA_LAYOUT_BSND && a->q_layout != TSA_LAYOUT_TND) return TSA_ERR_INVALID;
  if (a->B < 0 || a->Sq < 0) return TSA_ERR_INVALID;
  if (a->q_layout == TSA_LAYOUT_TND) {
    if (!a->cu_seqlens_q) return TSA_ERR_NULL;
    if (a->T < 0 || a->cu_seqlens_q[0] != 0 || a->cu_seqlens_q[a->B] != a->T)
      return TSA_ERR_INVALID;
    for (int b = 0; b < a->B; b++)
      if (a->cu_seqlens_q[b + 1] < a->cu_seqlens_q[b]) return TSA_ERR_INVALID;
  }
  // "aclnnSparseFlashAttention", constraints: N1 in {1, 2, 4, ..., 128}.
  if (a->N1 < 1 || a->N1 > 128 || (a->N1 & (a->N1 - 1))) return TSA_ERR_INVALID;
  if (a->N2 < 1 || a->N1 % a->N2 != 0) return TSA_ERR_INVALID;
  // "SparseAttnSharedkvMetadata", parameters: one KV head only.
  if (a->N2 != 1) return TSA_ERR_UNSUPPORTED;
  // constraints: D = 512 for query/key/value, Dr = 64 for the rope parts.
  if (a->D != 512 || a->Dr != 64 || a->Dv != 512) return TSA_ERR_INVALID;
  // constraints: block_size a multiple of 16, at most 1024.
  if (a->page_size < 16 || a->page_size > 1024 || a->page_size % 16 != 0) return TSA_ERR_INVALID;
  // constraints: sparse_block_size and block_size tied by exact division
  // (read: a selected block never straddles a page).
  if (a->sparse_block_size < 1 || a->page_size % a->sparse_block_size != 0) return TSA_ERR_INVALID;
  if (a->sparse_mode != 0 && a->sparse_mode != 3) return TSA_ERR_INVALID;
  if (a->topk < 1 || a->max_pages < 1 || a->num_pages < 1) return TSA_ERR_INVALID;
  if (!std::isfinite(a->scale) || !(a->scale > 0.f)) return TSA_ERR_INVALID;
  if (!fits_i32((long)a->num_pages * a->page_size) || !fits_i32((long)a->B * a->max_pages))
    return TSA_ERR_INVALID;
  if (!fits_i32(sfa_tokens(a) * a->N1 * a->D) || !fits_i32(sfa_tokens(a) * a->topk))
    return TSA_ERR_INVALID;
  if (sfa_tokens(a) > 0 &&
      (!a->q || !a->q_rope || !a->key_cache || !a->key_rope_cache || !a->value_cache ||
       !a->block_table || !a->kv_lens || !a->topk_indices || !a->out))
    return TSA_ERR_NULL;
  // value_cache may alias key_cache (shared KV, "SparseAttnSharedkvMetadata":
  // sharedkv) or be a cache of its own with the same paging.
  if (!a16(a->q) || !a16(a->q_rope) || !a16(a->key_cache) || !a16(a->key_rope_cache) ||
      !a16(a->value_cache) || !a16(a->out))
    return TSA_ERR_INVALID;
  return TSA_OK;
}

SfaParams sfa_params(const sfa_paged_fwd_args* a) {
  SfaParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.q_rope = a->q_rope; p.kc = a->key_cache; p.krc = a->key_rope_cache;
  p.vc = a->value_cache; p.block_table = a->block_table; p.kv_lens = a->kv_lens;
  p.topk = a->topk_indices; p.out = a->out; p.lse = a->lse;
  p.B = a->B; p.Sq = a->Sq; p.N1 = a->N1; p.N2 = a->N2; p.D = a->D; p.Dr = a->Dr; p.Dv = a->Dv;
  p.ntok = sfa_tokens(a);
  p.num_pages = a->num_pages; p.page = a->page_size; p.max_pages = a->max_pages;
  p.topk_n = a->topk; p.sbs = a->sparse_block_size;
  p.causal = a->sparse_mode == 3;
  p.scale = a->scale;
  p.splits = sfa_splits(p);
  return p;
}

// ----- shared-KV two-branch decode --------------------------------------------

long skv_tokens(const sfa_sharedkv_fwd_args* a) {
  return a->q_layout == TSA_LAYOUT_TND ? (long)a->T : (long)a->B * a->Sq;
}

bool skv_page_ok(int page, int pages, int max_pages) {
  return page >= 16 && page <= 1024 && page % 16 == 0 && pages >= 1 && max_pages >= 1 &&
         fits_i32((long)pages * page);
}

int check_sfa_sharedkv(const sfa_sharedkv_fwd_args* a) {
  if (!a) return TSA_ERR_NULL;
  if (a->dtype != TSA_BF16 && a->dtype != TSA_FP16) return TSA_ERR_INVALID;
  if (a->q_layout != TSA_LAYOUT_BSND && a->q_layout != TSA_LAYOUT_TND) return TSA_ERR_INVALID;
  if (a->B < 0 || a->Sq < 0) return TSA_ERR_INVALID;
  if (a->q_layout == TSA_LAYOUT_TND) {
    if (!a->cu_seqlens_q) return TSA_ERR_NULL;
    if (a->T < 0 || a->cu_seqlens_q[0] != 0 || a->cu_seqlens_q[a->B] != a->T)
      return TSA_ERR_INVALID;
    for (int b = 0; b < a->B; b++)
      if (a->cu_seqlens_q[b + 1] < a->cu_seqlens_q[b]) return TSA_ERR_INVALID;
  }
  // "SparseAttnSharedkvMetadata", parameter list: num_heads_kv 1; the SFA
  // constraints: N1 a power of two <= 128, D 512, Dr 64.
  if (a->N1 < 1 || a->N1 > 128 || (a->N1 & (a->N1 - 1))) return TSA_ERR_INVALID;
  if (a->N2 != 1) return TSA_ERR_UNSUPPORTED;
  if (a->D != 512 || a->Dr != 64) return TSA_ERR_INVALID;
  if (!std::isfinite(a->scale) || !(a->scale > 0.f)) return TSA_ERR_INVALID;
  if ((a->has_ori_kv != 0 && a->has_ori_kv != 1) || (a->has_cmp_kv != 0 && a->has_cmp_kv != 1) ||
      !(a->has_ori_kv || a->has_cmp_kv))
    return TSA_ERR_INVALID;
  if (a->has_ori_kv) {
    if (a->ori_win_left < 0 || a->ori_win_right < 0 ||
        (long)a->ori_win_left + a->ori_win_right + 1 > 4096)
      return TSA_ERR_INVALID;
    if (!skv_page_ok(a->ori_page_size, a->ori_num_pages, a->ori_max_pages)) return TSA_ERR_INVALID;
  }
  if (a->has_cmp_kv) {
    // cmp_ratio: the parameter list's range, 4 or 128
    if (a->cmp_ratio != 4 && a->cmp_ratio != 128) return TSA_ERR_INVALID;
    if (a->cmp_topk < 1) return TSA_ERR_INVALID;
    if (!skv_page_ok(a->cmp_page_size, a->cmp_num_pages, a->cmp_max_pages)) return TSA_ERR_INVALID;
  }
  const long tok = skv_tokens(a);
  if (!fits_i32(tok * a->N1 * a->D) || !fits_i32(tok * (a->has_cmp_kv ? a->cmp_topk : 1)) ||
      !fits_i32((long)a->B * (a->has_ori_kv ? a->ori_max_pages : 1)) ||
      !fits_i32((long)a->B * (a->has_cmp_kv ? a->cmp_max_pages : 1)))
    return TSA_ERR_INVALID;
  if (tok > 0) {
    if (!a->q || !a->q_rope || !a->out || !a->seqused_kv) return TSA_ERR_NULL;
    if (a->has_ori_kv && (!a->ori_key_cache || !a->ori_key_rope_cache || !a->ori_block_table))
      return TSA_ERR_NULL;
    if (a->has_cmp_kv && (!a->cmp_key_cache || !a->cmp_key_rope_cache || !a->cmp_block_table ||
                          !a->cmp_topk_indices))
      return TSA_ERR_NULL;
  }
  if (!a16(a->q) || !a16(a->q_rope) || !a16(a->out) || !a16(a->ori_key_cache) ||
      !a16(a->ori_key_rope_cache) || !a16(a->cmp_key_cache) || !a16(a->cmp_key_rope_cache))
    return TSA_ERR_INVALID;
  return TSA_OK;
}

SfaParams skv_params(const sfa_sharedkv_fwd_args* a) {
  SfaParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.q_rope = a->q_rope; p.out = a->out; p.lse = a->lse;
  p.kv_lens = a->seqused_kv;
  p.B = a->B; p.Sq = a->Sq; p.N1 = a->N1; p.N2 = 1; p.D = a->D; p.Dr = a->Dr; p.Dv = a->D;
  p.ntok = skv_tokens(a);
  p.sbs = 1;
  p.causal = 1;  // top-k slots: rightDownCausal in compressed positions
  p.scale = a->scale;
  if (a->has_ori_kv) {
    p.kc = a->ori_key_cache; p.krc = a->ori_key_rope_cache; p.vc = a->ori_key_cache;
    p.block_table = a->ori_block_table;
    p.num_pages = a->ori_num_pages; p.page = a->ori_page_size; p.max_pages = a->ori_max_pages;
    p.win_left = a->ori_win_left;
    p.win_len = a->ori_win_left + a->ori_win_right + 1;
    p.win_pad = (p.win_len + 31) / 32 * 32;
  }
  p.cmp_ratio = 1;
  if (a->has_cmp_kv) {
    p.ckc = a->cmp_key_cache; p.ckrc = a->cmp_key_rope_cache; p.cbt = a->cmp_block_table;
    p.c_num_pages = a->cmp_num_pages; p.c_page = a->cmp_page_size;
    p.c_max_pages = a->cmp_max_pages; p.cmp_ratio = a->cmp_ratio;
    p.topk = a->cmp_topk_indices; p.topk_n = a->cmp_topk;
    if (!a->has_ori_kv) {  // no band: the one cache fields point at the compressed cache
      p.kc = p.ckc; p.krc = p.ckrc; p.vc = p.ckc; p.block_table = p.cbt;
      p.num_pages = p.c_num_pages; p.page = p.c_page; p.max_pages = p.c_max_pages;
    }
  }
  p.splits = sfa_splits(p);
  return p;
}

size_t skv_carve(const SfaParams& p, void* ws, SfaParams* out) {
  Carver c(ws);
  const long tok = p.ntok;
  float* po = c.take<float>(tok * p.splits * p.N1 * p.Dv);
  float* pl = c.take<float>(tok * p.splits * p.N1);
  int* buf = c.take<int>(skv_cu_ints(p.B) + skv_task_ints(tok, p.splits));
  if (out) {
    *out = p;
    out->part_o = po;
    out->part_lse = pl;
    out->cu_q = nullptr;
    out->cu_dev = buf;
    out->task = buf + skv_cu_ints(p.B);
  }
  return c.off + kAlign;
}

size_t sfa_carve(const SfaParams& p, void* ws, SfaParams* out) {
  Carver c(ws);
  const long tok = p.ntok;
  float* po = c.take<float>(tok * p.splits * p.N1 * p.Dv);
  float* pl = c.take<float>(tok * p.splits * p.N1);
  int* bad = c.take<int>(1);
  int* cu = c.take<int>(p.B + 1);   // TND query prefix sums, uploaded per call
  if (out) {
    *out = p;
    out->part_o = po;
    out->part_lse = pl;
    out->bad = bad;
    out->cu_q = nullptr;
    out->cu_dev = cu;
  }
  return c.off + kAlign;
}

// ----- FloydAttention ----------------------------------------------------------

// "aclnnFusedFloydAttentionGrad", shape constraints (read as B, H, N, M, K,
// D): B in [1, 2K], H in [1, 256], N a multiple of 16 in [16, 1M], M and K
// multiples of 128 in [128, 1M], D in {32, 64, 128}.
template <class A>
int check_floyd(const A* a) {
  if (!a) return TSA_ERR_NULL;
  if (a->dtype != TSA_BF16 && a->dtype != TSA_FP16) return TSA_ERR_INVALID;
  if (a->B < 1 || a->B > 2048 || a->H < 1 || a->H > 256) return TSA_ERR_INVALID;
  if (a->N < 16 || a->N > (1 << 20) || a->N % 16) return TSA_ERR_INVALID;
  if (a->M < 128 || a->M > (1 << 20) || a->M % 128) return TSA_ERR_INVALID;
  if (a->K < 128 || a->K > (1 << 20) || a->K % 128) return TSA_ERR_INVALID;
  if (a->D != 32 && a->D != 64 && a->D != 128) return TSA_ERR_INVALID;
  if (!std::isfinite(a->scale) || !(a->scale > 0.f)) return TSA_ERR_INVALID;
  // launch sizes: the largest GEMM grids and the row kernels fit 31 bits
  const long Z = (long)a->B * a->H;
  const long rows = Z * a->N * a->M;
  const double s1 = (double)Z * a->N * cdiv(a->M, 64) * cdiv(a->K, 128);
  const double s2 = (double)Z * a->M * cdiv(a->N, 64) * cdiv(a->K, 128);
  if (s1 > 2147483647.0 || s2 > 2147483647.0 || rows / 4 + 1 > 2147483647L)
    return TSA_ERR_INVALID;
  if ((double)rows * a->K * 12 > 9.0e18) return TSA_ERR_INVALID;
  if (!a->q || !a->k1 || !a->v1 || !a->k2 || !a->v2) return TSA_ERR_NULL;
  if (!a16(a->q) || !a16(a->k1) || !a16(a->v1) || !a16(a->k2) || !a16(a->v2))
    return TSA_ERR_INVALID;
  return TSA_OK;
}

// Workspace: fp32 S, (backward: fp32 dP), 16-bit P, (backward: 16-bit dS),
// fp32 [rows, D] accumulator.
template <class A>
size_t floyd_carve(const A* a, void* ws, FloydParams* p, bool bwd) {
  const long rows = (long)a->B * a->H * a->N * a->M;
  const long el = rows * a->K;
  Carver c(ws);
  FloydParams w;
  std::memset(&w, 0, sizeof(w));
  w.s = c.take<float>(el);
  w.dp = bwd ? c.take<float>(el) : nullptr;
  w.p = c.take<uint16_t>(el);
  w.ds = bwd ? c.take<uint16_t>(el) : nullptr;
  w.acc = c.take<float>(rows * a->D);
  w.Z = a->B * a->H; w.N = a->N; w.M = a->M; w.K = a->K; w.D = a->D;
  w.scale = a->scale;
  w.q = a->q; w.k1 = a->k1; w.v1 = a->v1; w.k2 = a->k2; w.v2 = a->v2;
  if (p) *p = w;
  return c.off + kAlign;
}

// ----- fixed scratch for the entry point that allocates nothing -------------

// Every GPU the library runs on holds its own copy of this array until the
// process ends.  In host code its name is only a stand-in: the device address
// comes from hipGetSymbolAddress, taken once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up on the first call on that
// device, with it current).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TSA_OK;
}

}  // namespace

// ===========================================================================
// Exported entry points
// ===========================================================================
extern "C" {

const char* tsa_status_string(int s) {
  switch (s) {
    case TSA_OK: return "ok";
    case TSA_ERR_NULL: return "a required pointer is NULL";
    case TSA_ERR_INVALID: return "a value or shape violates a documented constraint";
    case TSA_ERR_UNSUPPORTED: return "valid for the operator but not built in this library";
    case TSA_ERR_WORKSPACE: return "workspace missing, too small or not 16-byte aligned";
    case TSA_ERR_HIP: return "a HIP launch or runtime call failed";
    case TSA_ERR_DATA: return "input data out of range (validate = 1)";
    case TSA_ERR_SCRATCH:
      return "the call needs more scratch than the fixed no-allocation maximum (64 MiB)";
    default: return "unknown status";
  }
}

size_t tsa_args_sizeof(int which) {
  switch (which) {
    case 0: return sizeof(bsa_fwd_args);
    case 1: return sizeof(bsa_bwd_args);
    case 2: return sizeof(nsa_select_fwd_args);
    case 3: return sizeof(nsa_select_bwd_args);
    case 4: return sizeof(sfa_paged_fwd_args);
    case 5: return sizeof(sfa_sharedkv_fwd_args);
    case 6: return sizeof(floyd_fwd_args);
    case 7: return sizeof(floyd_bwd_args);
    default: return 0;
  }
}

// ----- BSA -----------------------------------------------------------------

int bsa_fwd_workspace_size(const bsa_fwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_bsa_fwd(a);
  if (s) return s;
  *bytes = bsa_carve(a, nullptr, nullptr, false);
  return TSA_OK;
}

int bsa_compact_workspace_size(const bsa_fwd_args* a, size_t* bytes) {
  if (!bytes || !a) return TSA_ERR_NULL;
  int s = check_bsa_common(a->dtype, a->q_layout, a->kv_layout, a->B, a->N1, a->N2, a->Sq, a->Skv,
                           a->D, a->block_q, a->block_kv, a->sparse_mode, a->scale);
  if (s) return s;
  *bytes = bsa_carve(a, nullptr, nullptr, false);
  return TSA_OK;
}

int bsa_compact(const bsa_fwd_args* a, int32_t* row_ptr, int32_t* col, int32_t* rev_ptr,
                int32_t* rev, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = bsa_compact_workspace_size(a, &need);
  if (s) return s;
  if (!row_ptr || !col || !rev_ptr || !rev || (a->B * (long)a->Sq > 0 && !a->block_mask))
    return TSA_ERR_NULL;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  BsaWs w;
  bsa_carve(a, ws, &w, false);
  const int QB = (int)cdiv(a->Sq, a->block_q), KB = (int)cdiv(a->Skv, a->block_kv);
  hipStream_t st = (hipStream_t)stream;
  if ((long)a->B * QB * KB == 0) {
    hipError_t e = launch_fill_i32(row_ptr, (int)((long)a->B * a->N1 * QB + 1), 0, st);
    if (e == hipSuccess) e = launch_fill_i32(rev_ptr, (int)((long)a->B * a->N2 * KB + 1), 0, st);
    return hip_status(e);
  }
  return hip_status(launch_bsa_compact(a->block_mask, a->B, a->N1, a->N2, QB, KB, w.parts, w.sums,
                                       row_ptr, col, rev_ptr, rev, st));
}

int bsa_fwd(const bsa_fwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = bsa_fwd_workspace_size(a, &need);
  if (s) return s;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  BsaWs w;
  bsa_carve(a, ws, &w, false);
  BsaParams p = bsa_params(a->B, a->N1, a->N2, a->Sq, a->Skv, a->block_q, a->block_kv,
                           a->sparse_mode, a->scale);
  const StageTimer tm = timer_of(a, st);
  hipError_t e = bsa_upload_seqlens(a, w, &p, st);
  if (e == hipSuccess) e = tm.mark(0, 0);
  // the lists are built even with no query rows, so that a backward reusing
  // this workspace finds valid (empty) lists
  if (e == hipSuccess && !a->reuse_lists) e = bsa_build_lists(a, w, p, st);
  if (e == hipSuccess) e = tm.mark(0, 1);
  if (e != hipSuccess) return TSA_ERR_HIP;
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out; p.lse = a->lse;
  p.row_ptr = w.row_ptr; p.col = w.col; p.order_q = w.order_q;
  bsa_set_atten_mask(a, &p);
  e = tm.mark(1, 0);
  if (e == hipSuccess && bsa_q_rows(a) > 0) e = launch_bsa_fwd(p, a->dtype == TSA_FP16, st);
  if (e == hipSuccess) e = tm.mark(1, 1);
  return hip_status(e);
}

int bsa_bwd_workspace_size(const bsa_bwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_bsa_bwd(a);
  if (s) return s;
  *bytes = bsa_carve(a, nullptr, nullptr, true);
  return TSA_OK;
}

int bsa_bwd(const bsa_bwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = bsa_bwd_workspace_size(a, &need);
  if (s) return s;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  BsaWs w;
  bsa_carve(a, ws, &w, true);
  BsaParams p = bsa_params(a->B, a->N1, a->N2, a->Sq, a->Skv, a->block_q, a->block_kv,
                           a->sparse_mode, a->scale);
  const StageTimer tm = timer_of(a, st);
  hipError_t e = bsa_upload_seqlens(a, w, &p, st);
  if (e == hipSuccess) e = tm.mark(0, 0);
  // without query or key rows the lists are empty: they are written here
  // whatever reuse_lists says, so no kernel reads lists a call never wrote
  const bool rebuild = !a->reuse_lists || bsa_q_rows(a) == 0 || bsa_kv_rows(a) == 0;
  if (e == hipSuccess && rebuild) e = bsa_build_lists(a, w, p, st);
  if (e == hipSuccess) e = tm.mark(0, 1);
  if (e != hipSuccess) return TSA_ERR_HIP;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->out; p.dout = a->dout; p.lse = (float*)a->lse;
  p.out = a->dq; p.dk = a->dk; p.dv = a->dv; p.delta = w.delta;
  p.row_ptr = w.row_ptr; p.col = w.col; p.rev_ptr = w.rev_ptr; p.rev = w.rev;
  p.order_q = w.order_q; p.order_kv = w.order_kv;
  p.seg_off = w.seg_off; p.part_off = w.part_off; p.seg_meta = w.seg_meta; p.part = w.part;
  bsa_set_atten_mask(a, &p);
  return hip_status(launch_bsa_bwd(p, a->dtype == TSA_FP16, st, tm.ev, tm.n));
}

// ----- NSA -----------------------------------------------------------------

int nsa_compact_blocks_total(const nsa_select_fwd_args* a, int32_t* nb) {
  if (!nb) return TSA_ERR_NULL;
  int s = check_nsa(a, false);
  if (s) return s;
  *nb = nsa_blocks_total(a->cu_seqlens_kv, a->B, a->sbs);
  return TSA_OK;
}

int nsa_compact_workspace_size(const nsa_select_fwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_nsa(a, false);
  if (s) return s;
  *bytes = nsa_carve(a, nullptr, nullptr, false);
  return TSA_OK;
}

int nsa_compact(const nsa_select_fwd_args* a, int32_t* row_ptr, int32_t* col, int32_t* rev_ptr,
                int32_t* rev, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = nsa_compact_workspace_size(a, &need);
  if (s) return s;
  if (!row_ptr || !col || !rev_ptr || !rev) return TSA_ERR_NULL;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  NsaWs w;
  nsa_carve(a, ws, &w, false);
  w.row_ptr = row_ptr; w.col = col; w.rev_ptr = rev_ptr; w.rev = rev;
  NsaGeom g;
  s = nsa_setup(a, w, &g, st);
  if (s) return s;
  return nsa_lists(a, w, g, kNsaAll, st);
}

int nsa_select_fwd_workspace_size(const nsa_select_fwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  if (a && a->reuse_lists != 0 && a->reuse_lists != 1) return TSA_ERR_INVALID;
  int s = check_nsa(a);
  if (s) return s;
  *bytes = nsa_carve(a, nullptr, nullptr, false);
  return TSA_OK;
}

int nsa_select_fwd(const nsa_select_fwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = nsa_select_fwd_workspace_size(a, &need);
  if (s) return s;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (a->T == 0) return hip_status(timer_of(a, st).skip_all(2));
  NsaWs w;
  nsa_carve(a, ws, &w, false);
  NsaParams p;
  std::memset(&p, 0, sizeof(p));
  const StageTimer tm = timer_of(a, st);
  if (tm.mark(0, 0) != hipSuccess) return TSA_ERR_HIP;
  if (!a->reuse_lists) {
    // the forward needs only the per-row lists; the reverse lists are left
    // to the backward (reuse_lists = 2 there)
    s = nsa_setup(a, w, &p.g, st);
    if (s) return s;
    s = nsa_lists(a, w, p.g, kNsaForward, st);
    if (s) return s;
  } else {
    nsa_geom(a, w, &p.g);
  }
  if (tm.mark(0, 1) != hipSuccess) return TSA_ERR_HIP;
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out; p.lse = a->lse;
  p.row_ptr = w.row_ptr; p.col = w.col; p.rev_ptr = w.rev_ptr; p.rev = w.rev;
  p.T = a->T; p.Tk = a->Tk; p.N1 = a->N1; p.N2 = a->N2; p.G = a->N1 / a->N2; p.D = a->D;
  p.scale = a->scale;
  p.grp = w.grp;
  hipError_t e = tm.mark(1, 0);
  if (e == hipSuccess) e = launch_nsa_fwd(p, a->dtype == TSA_FP16, st);
  if (e == hipSuccess) e = tm.mark(1, 1);
  return hip_status(e);
}

int nsa_select_bwd_workspace_size(const nsa_select_bwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_nsa(a);
  if (s) return s;
  if (a->reuse_lists < 0 || a->reuse_lists > 2) return TSA_ERR_INVALID;
  if (a->T > 0 && (!a->out || !a->dout || !a->lse || !a->dq)) return TSA_ERR_NULL;
  if (a->Tk > 0 && (!a->dk || !a->dv)) return TSA_ERR_NULL;
  if (!a16(a->dout) || !a16(a->dq) || !a16(a->dk) || !a16(a->dv)) return TSA_ERR_INVALID;
  *bytes = nsa_carve(a, nullptr, nullptr, true);
  return TSA_OK;
}

int nsa_select_bwd(const nsa_select_bwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = nsa_select_bwd_workspace_size(a, &need);
  if (s) return s;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  NsaWs w;
  nsa_carve(a, ws, &w, true);
  NsaParams p;
  std::memset(&p, 0, sizeof(p));
  const StageTimer tm = timer_of(a, st);
  if (tm.mark(0, 0) != hipSuccess) return TSA_ERR_HIP;
  // with no tokens the lists are empty: they are written here whatever
  // reuse_lists says (a forward without tokens leaves the workspace alone)
  if (a->reuse_lists == 0 || a->T == 0) {
    s = nsa_setup(a, w, &p.g, st);
    if (s) return s;
    if (a->T > 0) {
      s = nsa_lists(a, w, p.g, kNsaAll, st);
      if (s) return s;
    } else {
      if (launch_fill_i32(w.rev_ptr, (int)((long)a->N2 * p.g.NB + 1), 0, st) != hipSuccess)
        return TSA_ERR_HIP;
    }
  } else {
    nsa_geom(a, w, &p.g);
    if (a->reuse_lists == 2 && a->T > 0) {
      s = nsa_lists(a, w, p.g, kNsaReverse, st);
      if (s) return s;
    }
  }
  if (tm.mark(0, 1) != hipSuccess) return TSA_ERR_HIP;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->out; p.dout = a->dout; p.lse = (float*)a->lse;
  p.out = a->dq; p.dk = a->dk; p.dv = a->dv; p.delta = w.delta;
  p.row_ptr = w.row_ptr; p.col = w.col; p.rev_ptr = w.rev_ptr; p.rev = w.rev;
  p.T = a->T; p.Tk = a->Tk; p.N1 = a->N1; p.N2 = a->N2; p.G = a->N1 / a->N2; p.D = a->D;
  p.scale = a->scale;
  p.seg_off = w.seg_off; p.seg_sums = w.seg_sums; p.seg_ctr = w.seg_ctr; p.part = w.part;
  p.max_segments = w.max_segments;
  p.grp = w.grp;
  return hip_status(launch_nsa_bwd(p, a->dtype == TSA_FP16, st, tm.ev, tm.n));
}

// ----- SFA -----------------------------------------------------------------

int sfa_paged_fwd_workspace_size(const sfa_paged_fwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_sfa(a);
  if (s) return s;
  *bytes = sfa_carve(sfa_params(a), nullptr, nullptr);
  return TSA_OK;
}

int sfa_paged_fwd(const sfa_paged_fwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = sfa_paged_fwd_workspace_size(a, &need);
  if (s) return s;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (sfa_tokens(a) == 0) return hip_status(timer_of(a, st).skip_all(2));
  SfaParams p;
  sfa_carve(sfa_params(a), ws, &p);
  if (a->q_layout == TSA_LAYOUT_TND) {
    // the copy from pageable memory is staged before hipMemcpyAsync returns
    if (hipMemcpyAsync(p.cu_dev, a->cu_seqlens_q, sizeof(int) * (a->B + 1),
                       hipMemcpyHostToDevice, st) != hipSuccess)
      return TSA_ERR_HIP;
    p.cu_q = p.cu_dev;
  }
  if (a->validate) {
    hipError_t e = launch_fill_i32(p.bad, 1, 0, st);
    if (e == hipSuccess) e = launch_sfa_check(p, st);
    int bad = 0;
    if (e == hipSuccess) e = hipMemcpyAsync(&bad, p.bad, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return TSA_ERR_HIP;
    if (bad) return TSA_ERR_DATA;
  }
  const StageTimer tm = timer_of(a, st);
  return hip_status(launch_sfa_fwd(p, a->dtype == TSA_FP16, st, tm.ev, tm.n));
}

size_t sfa_paged_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int sfa_paged_fwd_noalloc(const sfa_paged_fwd_args* a, void* stream) {
  size_t need;
  int s = sfa_paged_fwd_workspace_size(a, &need);
  if (s) return s;
  if (need > kScratchBytes) return TSA_ERR_SCRATCH;
  void* ptr = nullptr;
  s = scratch_of_current_device(&ptr);
  if (s) return s;
  // the split partials are written in full before the combine reads them,
  // so nothing in the scratch needs clearing between calls
  return sfa_paged_fwd(a, ptr, kScratchBytes, stream);
}

// ----- FloydAttention ----------------------------------------------------------

int floyd_fwd_workspace_size(const floyd_fwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_floyd(a);
  if (s) return s;
  if (!a->out || !a->lse) return TSA_ERR_NULL;
  if (!a16(a->out)) return TSA_ERR_INVALID;
  *bytes = floyd_carve(a, nullptr, nullptr, false);
  return TSA_OK;
}

int floyd_fwd(const floyd_fwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = floyd_fwd_workspace_size(a, &need);
  if (s) return s;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  FloydParams p;
  floyd_carve(a, ws, &p, false);
  p.out = a->out;
  p.lse = a->lse;
  const StageTimer tm = timer_of(a, st);
  return hip_status(launch_floyd_fwd(p, a->dtype == TSA_FP16, st, tm.ev, tm.n));
}

int floyd_bwd_workspace_size(const floyd_bwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_floyd(a);
  if (s) return s;
  if (!a->out || !a->dout || !a->lse || !a->dq || !a->dk1 || !a->dv1 || !a->dk2 || !a->dv2)
    return TSA_ERR_NULL;
  if (!a16(a->out) || !a16(a->dout) || !a16(a->dq) || !a16(a->dk1) || !a16(a->dv1) ||
      !a16(a->dk2) || !a16(a->dv2))
    return TSA_ERR_INVALID;
  *bytes = floyd_carve(a, nullptr, nullptr, true);
  return TSA_OK;
}

int floyd_bwd(const floyd_bwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = floyd_bwd_workspace_size(a, &need);
  if (s) return s;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  FloydParams p;
  floyd_carve(a, ws, &p, true);
  p.o = a->out;
  p.dout = a->dout;
  p.lse = (float*)a->lse;
  p.dq = a->dq; p.dk1 = a->dk1; p.dv1 = a->dv1; p.dk2 = a->dk2; p.dv2 = a->dv2;
  const StageTimer tm = timer_of(a, st);
  return hip_status(launch_floyd_bwd(p, a->dtype == TSA_FP16, st, tm.ev, tm.n));
}

// ----- shared-KV two-branch decode -------------------------------------------

int sfa_sharedkv_fwd_workspace_size(const sfa_sharedkv_fwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_sfa_sharedkv(a);
  if (s) return s;
  *bytes = skv_carve(skv_params(a), nullptr, nullptr);
  return TSA_OK;
}

int sfa_sharedkv_metadata_size(const sfa_sharedkv_fwd_args* a, size_t* bytes) {
  if (!bytes) return TSA_ERR_NULL;
  int s = check_sfa_sharedkv(a);
  if (s) return s;
  const SfaParams p = skv_params(a);
  *bytes = sizeof(int) * (skv_cu_ints(p.B) + skv_task_ints(p.ntok, p.splits));
  return TSA_OK;
}

// TND prefix sums into the task buffer (host -> device), pointed at by p->cu_q.
static hipError_t skv_upload_cu(const sfa_sharedkv_fwd_args* a, SfaParams* p, hipStream_t st) {
  if (a->q_layout != TSA_LAYOUT_TND) return hipSuccess;
  // the copy from pageable memory is staged before hipMemcpyAsync returns
  hipError_t e = hipMemcpyAsync(p->cu_dev, a->cu_seqlens_q, sizeof(int) * (a->B + 1),
                                hipMemcpyHostToDevice, st);
  p->cu_q = p->cu_dev;
  return e;
}

int sfa_sharedkv_metadata(const sfa_sharedkv_fwd_args* a, void* tasks, size_t bytes,
                          void* stream) {
  size_t need;
  int s = sfa_sharedkv_metadata_size(a, &need);
  if (s) return s;
  if (!tasks || bytes < need) return TSA_ERR_WORKSPACE;
  if ((uintptr_t)tasks % 16) return TSA_ERR_INVALID;  // the list holds 16-byte records
  if (skv_tokens(a) == 0) return TSA_OK;
  hipStream_t st = (hipStream_t)stream;
  SfaParams p = skv_params(a);
  p.cu_dev = (int*)tasks;
  p.task = (int*)tasks + skv_cu_ints(p.B);
  hipError_t e = skv_upload_cu(a, &p, st);
  if (e == hipSuccess) e = launch_sfa_task(p, st);
  return hip_status(e);
}

int sfa_sharedkv_fwd(const sfa_sharedkv_fwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need;
  int s = sfa_sharedkv_fwd_workspace_size(a, &need);
  if (s) return s;
  if (!ws || !a16(ws) || ws_bytes < need) return TSA_ERR_WORKSPACE;
  if (a->tasks && (uintptr_t)a->tasks % 16) return TSA_ERR_INVALID;
  hipStream_t st = (hipStream_t)stream;
  if (skv_tokens(a) == 0) return hip_status(timer_of(a, st).skip_all(3));
  SfaParams p;
  skv_carve(skv_params(a), ws, &p);
  const bool have = a->tasks != nullptr;
  if (have) {
    // the list of an earlier sfa_sharedkv_metadata call: token entries and
    // slot ranges; no upload, no list kernel
    p.cu_dev = (int*)a->tasks;
    p.task = (int*)a->tasks + skv_cu_ints(p.B);
  } else if (skv_upload_cu(a, &p, st) != hipSuccess) {
    return TSA_ERR_HIP;
  }
  const StageTimer tm = timer_of(a, st);
  return hip_status(launch_sfa_sharedkv(p, a->dtype == TSA_FP16, have, st, tm.ev, tm.n));
}

}  // extern "C"
