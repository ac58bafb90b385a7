// Host-side declarations shared by the launchers and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {

// Records ev[2*stage + end] on st when stage < n (caller-provided timing events).
inline hipError_t mark_event(void* const* ev, int n, int stage, int end, hipStream_t st) {
  if (!ev || stage >= n) return hipSuccess;
  return hipEventRecord((hipEvent_t)ev[2 * stage + end], st);
}

// ----- scans and lists -----------------------------------------------------
int scan_sums_len(long n);
hipError_t exclusive_scan(int* data, long n, int* sums, hipStream_t st);
// Exclusive scan of data[0..n) in place, with the total written to data[n].
hipError_t exclusive_scan_total(int* data, long n, int* sums, hipStream_t st);

long bsa_compact_parts_len(int B, int N1, int N2, int QB, int KB);
// Segment plan of the dK/dV work items (see BsaParams); seg_off null: none.
struct BsaSegPlan {
  int* seg_off;
  int* part_off;
  int* seg_meta;
  int ksub, n_items;
};
// order_rows / order_cols: the n_rows forward and n_cols reverse lists' tile
// ids by list length, longest first (the attention kernels' work order);
// with plan.seg_off set, also the dK/dV segment plan over order_cols.
hipError_t launch_tile_order(const int* row_ptr, int n_rows, int* order_rows, const int* rev_ptr,
                             int n_cols, int* order_cols, const BsaSegPlan& plan, hipStream_t st);
hipError_t launch_bsa_compact(const uint8_t* mask, int B, int N1, int N2, int QB, int KB,
                              int* parts, int* sums, int* row_ptr, int* col, int* rev_ptr,
                              int* rev, hipStream_t st);

// NSA geometry as the device sees it (pointers into the workspace).
struct NsaGeom {
  const int* cu_q;     // [B+1] query prefix sums
  const int* cu_kv;    // [B+1] key prefix sums
  const int* blk_off;  // [B+1] prefix sums of ceil(Skv_b / sbs)
  int B, T, N2, sbc, sbs, causal, NB;
};


// NSA list building.  Forward: per-row sorted lists (row_ptr, col), plus
// each entry's reverse key n2*NB + global block and token id when ekey is
// given.  Reverse: per (n2, block) ascending token lists, by a stable
// counting sort of those entries when the key count allows (rs.usable),
// else by a per-list scan of the forward rows.
// Token groups of the NSA token-group forward and dQ kernels: runs of
// kNsaGroup consecutive tokens of one sequence, group g of sequence b holding
// positions [g * kNsaGroup, (g + 1) * kNsaGroup).  Each (KV head, group) has
// a chunk list: the ascending union of its tokens' selected blocks cut into
// 32-key chunks, one {key start within the sequence, token mask} entry per
// chunk that at least one token attends to (bit j = token p0 + j; a token
// listing a block twice attends to its chunks twice).
constexpr int kNsaGroup = 16;
constexpr int kNsaGroupChunk = 32;
// set in an entry's mask word when its chunk holds 16 keys, not 32 (the tail
// of a block whose size is an odd multiple of 16)
constexpr unsigned kNsaChunkHalf = 1u << 30;
struct NsaGroups {
  const int* gcu;  // [B+1] prefix sums of ceil(Sq_b / kNsaGroup)
  int NG;          // groups per KV head
  int cap;         // entries per (KV head, group): kNsaGroup * sbc * ceil(sbs / 32)
  int* cnt;        // [N2 * NG] entries of each list, unit = n2 * NG + group
  int* ent;        // [N2 * NG][cap][2]
};
hipError_t launch_nsa_group_lists(const NsaGeom& g, const int* row_ptr, const int* col,
                                  const NsaGroups& gr, hipStream_t st);

constexpr int kNsaRevMaxKeys = 16384;  // LDS counters of one sort tile (64 KB)
struct NsaRevSort {
  int NK, bits, rounds, n_tiles;
  bool usable;
};
NsaRevSort nsa_rev_sort_plan(long max_entries, long n_keys);
hipError_t launch_nsa_forward_lists(const int* topk, const NsaGeom& g, int* cnt_scan, int* sums,
                                    int* row_ptr, int* col, int* ekey, int* etok,
                                    hipStream_t st);
hipError_t launch_nsa_reverse_lists(const NsaGeom& g, const int* row_ptr, const int* col,
                                    int* sums, int* rev_scan, int* rev_ptr, int* rev,
                                    const int* ekey, const int* etok, const NsaRevSort& rs,
                                    int* hist, int* hsums, hipStream_t st);
hipError_t launch_nsa_check(const int* topk, const NsaGeom& g, int* bad, hipStream_t st);

// ----- block-sparse attention ---------------------------------------------
struct BsaParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // backward: forward output
  const void* dout;   // backward
  void* out;          // forward output / backward dq
  void* dk;
  void* dv;
  float* lse;         // forward: written; backward: read
  float* delta;       // backward: per row {LSE * log2 e, rowsum(dO * O)}, fp32 [B, N1, Sq, 2]
  const int* row_ptr;
  const int* col;
  const int* rev_ptr;
  const int* rev;
  const int* order_q;   // Q tiles (b*N1 + n1)*QB + qb, longest list first
  const int* order_kv;  // KV tiles (b*N2 + n2)*KB + kb, longest list first
  const int* cu_q;      // TND: [B+1] query prefix sums (device); null for BNSD
  const int* cu_kv;     // TND: [B+1] key prefix sums (device)
  int B, N1, N2, G, Sq, Skv, D;  // TND: Sq, Skv are the longest sequences
  int bq, bkv, QB, KB;
  int causal;
  float scale;
  // atten_mask: element (b, n1, i, j) at am[b*am_sb + n1*am_sn + i*am_pitch + j],
  // non-zero = excluded; null = none.  am_al4: every row start and every
  // chunk start is 4-byte aligned, so 4 keys load as one dword.
  const unsigned char* am;
  long am_sb, am_sn;
  int am_pitch, am_al4;
  // backward dK/dV segments (workspace): work item r (in order_kv order) has
  // seg_off[r+1] - seg_off[r] segments of at most seg_meta[0] reverse-list
  // entries; a split item's segments write fp32 partials from slot
  // part_off[r] on, which a reduction sums in segment order.  seg_meta: the
  // segment length, the count of split items and their ranks.
  int* seg_off;        // [n_items + 1]
  int* part_off;       // [n_items + 1]
  int* seg_meta;       // [2 + kBsaDkdvSlots]
  float* part;         // [kBsaMaxParts][2][keys per item][D]
};

// Workgroup slots the dK/dV segment length is sized for (two 4-wave
// workgroups on each of 256 CUs), and the partial slots that bound implies.
constexpr int kBsaDkdvSlots = 512;
constexpr int kBsaMaxParts = 2 * kBsaDkdvSlots;
// dK/dV work items of a backward: keys per item, key splits per KV tile,
// item count, and the fp32 partial slots (2 x nk x D floats each) to reserve.
struct BsaDkdvShape {
  int nk, ksub;
  long n_items, max_parts;
};
BsaDkdvShape bsa_dkdv_shape(int B, int N1, int N2, int QB, int KB, int bkv);

// Where the rows of one sequence b live in a BSA tensor: row r of head n is
// element at(n, r).  BNSD: a head's rows are contiguous, S rows per head;
// TND: rows are tokens of the sequence, the N heads of a token adjacent.
// `elems` is the elements per row of one head (D for Q/K/V/O and their
// gradients, 1 for the fp32 per-row LSE and softmax_grad).
struct BsaRowMap {
  long base;  // element offset of row 0 of head 0
  long head;  // elements between heads
  int row;    // elements between rows
  int len;    // rows of the sequence
  __device__ __forceinline__ long at(int n, int r) const { return base + n * head + (long)r * row; }
};
__device__ __forceinline__ BsaRowMap bsa_rows(const int* cu, int b, int N, int S, int elems) {
  if (cu) {
    const int s0 = cu[b];
    return BsaRowMap{(long)s0 * N * elems, elems, N * elems, cu[b + 1] - s0};
  }
  return BsaRowMap{(long)b * N * S * elems, (long)S * elems, elems, S};
}

hipError_t launch_bsa_fwd(const BsaParams& p, int fp16, hipStream_t st);
// ev / n_ev: caller timing events (stage 1 = dQ, stage 2 = dK/dV), may be null.
hipError_t launch_bsa_bwd(const BsaParams& p, int fp16, hipStream_t st, void* const* ev, int n_ev);

// ----- NSA selected attention ------------------------------------------------
struct NsaParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  void* out;          // forward output / backward dq
  void* dk;
  void* dv;
  float* lse;
  float* delta;       // backward: per row {LSE * log2 e, rowsum(dO * O)}, fp32 [T, N1, 2]
  const int* row_ptr;
  const int* col;
  const int* rev_ptr;
  const int* rev;
  NsaGeom g;
  int T, Tk, N1, N2, G, D;  // D: query/key head dim (128 or 192); values are 128 wide
  float scale;
  // backward dK/dV segments (workspace): the reverse list of (KV head,
  // block) r is cut into seg_off[r+1] - seg_off[r] segments of at most
  // kNsaSegEntries listings; segment j writes fp32 partials into slot j.
  int* seg_off;        // [N2*NB + 1] exclusive scan of segments per list, then the total
  int* seg_sums;       // scan scratch
  int* seg_ctr;        // [1] segments taken by the dK/dV workgroups
  NsaGroups grp;       // token-group chunk lists (grouped kernels only; NG = 0 otherwise)
  float* part;         // [max_segments][sbs*D (dK) + sbs*128 (dV)] fp32 partials
  int max_segments;
};

constexpr int kNsaSegEntries = 256;  // reverse-list listings per dK/dV segment at most
constexpr int kNsaDkdvMaxGrid = 768;
int nsa_max_segments(long total_entries, long nblocks);
int nsa_dkdv_grid(const NsaParams& p);

hipError_t launch_nsa_fwd(const NsaParams& p, int fp16, hipStream_t st);
hipError_t launch_nsa_bwd(const NsaParams& p, int fp16, hipStream_t st, void* const* ev, int n_ev);

// ----- sparse flash attention (paged decode) ----------------------------------
struct SfaParams {
  const void* q;
  const void* q_rope;
  const void* kc;
  const void* krc;
  const void* vc;
  const int* block_table;
  const int* kv_lens;
  const int* topk;
  void* out;
  float* lse;          // may be null
  float* part_o;       // split partials [ntok, splits, N1, Dv] fp32
  float* part_lse;     // [ntok, splits, N1]
  int* bad;            // validate flag (may be null)
  int B, Sq, N1, N2, D, Dr, Dv;
  long ntok;           // decode tokens: B * Sq (BSND) or T (TND)
  const int* cu_q;     // TND: [B+1] query prefix sums (device); null for BSND
  int* cu_dev;         // workspace slot the TND prefix sums are uploaded to
  int num_pages, page, max_pages, topk_n, sbs;
  int causal;
  int splits;
  float scale;
  // Shared-KV two-branch decode (null ckc: plain SFA).  A token's slots
  // [0, win_pad) are the band over the cache above (kc, block_table, page):
  // slot i is position qpos - win_left + i, kept for i < win_len inside
  // [0, kv_len); slots [win_pad, win_pad + topk_n) are topk's compressed ids
  // in the compressed cache (ckc / ckrc / cbt), kv_len / cmp_ratio entries,
  // rightDownCausal in compressed positions.  win_pad is a multiple of 32,
  // so no 32-slot chunk mixes the two caches.
  int win_pad, win_len, win_left;
  const void* ckc;
  const void* ckrc;
  const int* cbt;
  int c_page, c_max_pages, c_num_pages, cmp_ratio;
  // Shared-KV task list, or null (plain SFA: equal slot ranges, the token's
  // entry found from Sq / cu_q): per token {b, s, Sq_b, 0}, then per split
  // i = tk * splits + sp its slot range [lo, hi).
  int* task;
};

// The task-list buffer of the shared-KV decode: the TND prefix sums (B+1,
// padded to 4 ints), then the task list; sizes in ints.
inline long skv_cu_ints(int B) { return ((long)B + 1 + 3) / 4 * 4; }
inline long skv_task_ints(long ntok, int splits) { return ntok * 4 + ntok * splits * 2; }

int sfa_splits(const SfaParams& p);
// slots per decode token: the band (padded) plus the top-k entries
__host__ __device__ inline int sfa_total_slots(const SfaParams& p) { return p.win_pad + p.topk_n * p.sbs; }
// The shared-KV task list (metadata kernel) into p.task.
hipError_t launch_sfa_task(const SfaParams& p, hipStream_t st);
// The split and combine kernels of the shared-KV decode, with the task list
// made first unless `have_tasks`: stage 0 = task list, 1 = split attention,
// 2 = combine.
hipError_t launch_sfa_sharedkv(const SfaParams& p, int fp16, bool have_tasks, hipStream_t st,
                               void* const* ev, int n_ev);
// stage 0 = split attention, stage 1 = combine
hipError_t launch_sfa_fwd(const SfaParams& p, int fp16, hipStream_t st, void* const* ev, int n_ev);
hipError_t launch_sfa_check(const SfaParams& p, hipStream_t st);
hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t st);

// ----- FloydAttention --------------------------------------------------------

// One strided, two-level-batched GEMM: C(z1, z2, r, c) = alpha * sum_l
// A(z1, z2, r, l) B(z1, z2, l, c); strides in elements.
struct FloydGemm {
  const void* a;
  const void* b;
  void* c;
  void* c16;  // 16-bit destination of the accumulate-and-convert mode
  long a_s1, a_s2, a_sr, a_sl;
  long b_s1, b_s2, b_sl, b_sc;
  long c_s1, c_s2, c_sr, c_sc;
  int Z1, Z2, R, Cn, L;
  float alpha;
};

struct FloydParams {
  const void* q;      // [Z, N, M, D]
  const void* k1;     // [Z, N, K, D]
  const void* v1;
  const void* k2;     // [Z, M, K, D]
  const void* v2;
  const void* o;      // backward: the forward output
  const void* dout;   // backward: its gradient
  void* out;          // forward output
  float* lse;         // [Z, N, M]
  void* dq;
  void* dk1;
  void* dv1;
  void* dk2;
  void* dv2;
  // workspace
  float* s;           // scores [Z, N, M, K]
  float* dp;          // backward: dP [Z, N, M, K]
  float* acc;         // fp32 accumulator [Z, N, M, D]
  void* p;            // P [Z, N, M, K], 16-bit
  void* ds;           // backward: dS [Z, N, M, K], 16-bit
  int Z, N, M, K, D;
  float scale;
};

// forward stages: 0 = scores, 1 = softmax, 2 = P V1 + P V2
hipError_t launch_floyd_fwd(const FloydParams& p, int fp16, hipStream_t st, void* const* ev,
                            int n_ev);
// backward stages: 0 = scores and dP, 1 = P and dS, 2 = dV1 / dV2, 3 = dQ,
// 4 = dK1 / dK2
hipError_t launch_floyd_bwd(const FloydParams& p, int fp16, hipStream_t st, void* const* ev,
                            int n_ev);

}  // namespace tsa
