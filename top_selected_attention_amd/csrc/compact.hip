// Selected-block lists.
//
// Block-sparse attention ("aclnnBlockSparseAttentionGrad", function
// description): the BlockSparseMask names, per Q block, the KV blocks it
// attends to.  The forward and dQ kernels walk, per Q block, the ascending
// list of selected KV blocks (forward CSR); the dK/dV kernel walks, per KV
// block, the ascending list of Q blocks that selected it (reverse CSR).
//
// NSA selected attention ("aclnnNsaSelectedAttention", formulas section):
// per (token, KV head) the topk_indices, sorted, with wholly-masked blocks
// dropped under causal mode (forward CSR), and per (KV head, block) the
// tokens that selected it (reverse CSR).
//
// Every list is built deterministically without atomics: counts, an
// exclusive scan, then a fill in which each entry's slot is its rank.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {

// ---------------------------------------------------------------------------
// Exclusive scan of an int32 array (in place), three passes.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 4;
constexpr int kScanTile = kScanThreads * kScanPer;

// ptr[i] = scanned[i] for i < n, ptr[n] = *total.
__global__ void copy_ptr(const int* scanned, long n, const int* total, int* ptr) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) ptr[i] = scanned[i];
  else if (i == n) ptr[n] = total[0];
}

__global__ __launch_bounds__(kScanThreads) void scan_tiles(int* data, int n, int* sums) {
  const int base = blockIdx.x * kScanTile + threadIdx.x * kScanPer;
  int v[kScanPer];
  int s = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; i++) {
    v[i] = (base + i < n) ? data[base + i] : 0;
    s += v[i];
  }
  int total;
  int ex = block_excl_scan(s, &total);
#pragma unroll
  for (int i = 0; i < kScanPer; i++) {
    if (base + i < n) data[base + i] = ex;
    ex += v[i];
  }
  if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

// Single block: exclusive scan of the tile sums; sums[nt] = grand total.
__global__ __launch_bounds__(kScanThreads) void scan_sums(int* sums, int nt) {
  int carry = 0;
  for (int base = 0; base < nt; base += kScanThreads) {
    int i = base + threadIdx.x;
    int x = i < nt ? sums[i] : 0;
    int total;
    int ex = block_excl_scan(x, &total);
    if (i < nt) sums[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) sums[nt] = carry;
}

__global__ __launch_bounds__(kScanThreads) void scan_add(int* data, int n, const int* sums) {
  const int add = sums[blockIdx.x];
  const int base = blockIdx.x * kScanTile + threadIdx.x * kScanPer;
#pragma unroll
  for (int i = 0; i < kScanPer; i++)
    if (base + i < n) data[base + i] += add;
}

// Up to kScanSmallTiles tiles: one workgroup scans them in order with a
// carry, in one launch instead of three (sums[t] = offset of tile t,
// sums[nt] = total, as the three-pass path leaves them).
constexpr int kScanSmallTiles = 4;
__global__ __launch_bounds__(kScanThreads) void scan_small(int* data, int n, int nt, int* sums) {
  int carry = 0;
  for (int t = 0; t < nt; t++) {
    const int base = t * kScanTile + threadIdx.x * kScanPer;
    int v[kScanPer];
    int s = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; i++) {
      v[i] = (base + i < n) ? data[base + i] : 0;
      s += v[i];
    }
    int total;
    int ex = carry + block_excl_scan(s, &total);
#pragma unroll
    for (int i = 0; i < kScanPer; i++) {
      if (base + i < n) data[base + i] = ex;
      ex += v[i];
    }
    if (threadIdx.x == 0) sums[t] = carry;
    carry += total;
  }
  if (threadIdx.x == 0) sums[nt] = carry;
}

int scan_sums_len(long n) { return (int)((n + kScanTile - 1) / kScanTile) + 1; }

__global__ void put_total(int* data, long n, const int* total) { data[n] = total[0]; }

hipError_t exclusive_scan_total(int* data, long n, int* sums, hipStream_t st) {
  hipError_t e = exclusive_scan(data, n, sums, st);
  if (e != hipSuccess) return e;
  const int nt = (int)((n + kScanTile - 1) / kScanTile);
  hipLaunchKernelGGL(put_total, dim3(1), dim3(1), 0, st, data, n, sums + nt);
  return hipGetLastError();
}

hipError_t exclusive_scan(int* data, long n, int* sums, hipStream_t st) {
  int nt = (int)((n + kScanTile - 1) / kScanTile);
  if (nt == 0) {
    hipLaunchKernelGGL(scan_sums, dim3(1), dim3(kScanThreads), 0, st, sums, 0);
    return hipGetLastError();
  }
  if (nt <= kScanSmallTiles) {
    hipLaunchKernelGGL(scan_small, dim3(1), dim3(kScanThreads), 0, st, data, (int)n, nt, sums);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(scan_tiles, dim3(nt), dim3(kScanThreads), 0, st, data, (int)n, sums);
  hipLaunchKernelGGL(scan_sums, dim3(1), dim3(kScanThreads), 0, st, sums, nt);
  hipLaunchKernelGGL(scan_add, dim3(nt), dim3(kScanThreads), 0, st, data, (int)n, sums);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// BlockSparseMask -> forward / reverse CSR via 64 x 64 bit tiles.
//
// Rows of the mask are (b, n1, qb); the G*QB rows of the query heads of one
// KV head (b, n2) are contiguous.  A tile covers 64 rows of one such group
// and 64 KV-block columns.  Pass 1 writes per-(row, column tile) and
// per-(column, row tile) counts into one array; after its exclusive scan,
// pass 2 writes each selected entry at its rank.
// ---------------------------------------------------------------------------
struct MaskTileGeom {
  int R, KB, QB, G, RG, RTG, CT, groups;  // RG = G*QB rows per group
};

constexpr int kTileStride = 68;  // bytes per LDS tile row (odd dword count: conflict-free columns)
constexpr int kMaskWaves = 4;    // waves per tile: each takes 16 of its rows / columns

// The tile's 64 rows x 64 columns into LDS: thread t loads 16 columns
// (quarter t / 64) of row t % 64; entries past the mask's edge read 0.
__device__ __forceinline__ void load_mask_tile(const uint8_t* mask, const MaskTileGeom& g, int grp,
                                               int rt, int ct, uint8_t* tile) {
  const int r = threadIdx.x & 63, qtr = threadIdx.x >> 6;
  const int lrow = rt * 64 + r;                     // row within group
  const long row = (long)grp * g.RG + lrow;
  const int c0 = ct * 64 + 16 * qtr;
  const int nc = max(0, min(16, g.KB - c0));
  uint8_t* dst = tile + r * kTileStride + 16 * qtr;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (lrow < g.RG && nc > 0) {
    const uint8_t* src = mask + row * g.KB + c0;
    if ((g.KB & 15) == 0) {
      const uint4 u = *reinterpret_cast<const uint4*>(src);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
      for (int i = 0; i < nc; i++) w[i >> 2] |= (uint32_t)src[i] << (8 * (i & 3));
    }
  }
  for (int j = 0; j < 4; j++) *reinterpret_cast<uint32_t*>(dst + 4 * j) = w[j];
}

__global__ __launch_bounds__(64 * kMaskWaves) void bsa_mask_count(const uint8_t* mask,
                                                                  MaskTileGeom g, int* parts) {
  __shared__ uint8_t tile[64 * kTileStride];
  __shared__ int rsum[kMaskWaves][64];
  const int ct = blockIdx.x % g.CT;
  const int rtg = blockIdx.x / g.CT;
  const int grp = rtg / g.RTG, rt = rtg % g.RTG;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  load_mask_tile(mask, g, grp, rt, ct, tile);
  __syncthreads();
  // row counts within this column tile: wave w counts columns 16w .. 16w+15
  int rc = 0;
  for (int c = 16 * w; c < 16 * w + 16; c++) rc += tile[lane * kTileStride + c] != 0;
  rsum[w][lane] = rc;
  // column counts within this row tile: wave w takes columns 16w .. 16w+15
  int myc = 0;
  for (int c = 16 * w; c < 16 * w + 16; c++) {
    const unsigned long long bits = __ballot(tile[lane * kTileStride + c] != 0);
    if (lane == c) myc = __popcll(bits);
  }
  const int col = ct * 64 + lane;
  if (lane >= 16 * w && lane < 16 * w + 16 && col < g.KB)
    parts[(long)g.R * g.CT + ((long)grp * g.KB + col) * g.RTG + rt] = myc;
  __syncthreads();
  const int lrow = rt * 64 + lane;
  if (w == 0 && lrow < g.RG)
    parts[((long)grp * g.RG + lrow) * g.CT + ct] = rsum[0][lane] + rsum[1][lane] + rsum[2][lane] +
                                                   rsum[3][lane];
}

__global__ __launch_bounds__(64 * kMaskWaves) void bsa_mask_fill(
    const uint8_t* mask, MaskTileGeom g, const int* scanned, const int* sums_total, int* row_ptr,
    int* col, int* rev_ptr, int* rev) {
  __shared__ uint8_t tile[64 * kTileStride];
  const int ct = blockIdx.x % g.CT;
  const int rtg = blockIdx.x / g.CT;
  const int grp = rtg / g.RTG, rt = rtg % g.RTG;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  load_mask_tile(mask, g, grp, rt, ct, tile);
  __syncthreads();
  const long colpart0 = (long)g.R * g.CT;
  // total of the row parts = exclusive prefix of the first column part
  const int nnz = scanned[colpart0];
  const int lrow = rt * 64 + lane;
  const long row = (long)grp * g.RG + lrow;
  // every wave forms the 64 row and 64 column bases (lane = row / column);
  // wave 0 also writes the pointers
  int my_rbase = 0;
  if (lrow < g.RG) {
    my_rbase = scanned[row * g.CT + ct];
    if (ct == 0 && w == 0) row_ptr[row] = my_rbase;
  }
  const int mycol = ct * 64 + lane;
  int my_cbase = 0;
  if (mycol < g.KB) {
    my_cbase = scanned[colpart0 + ((long)grp * g.KB + mycol) * g.RTG + rt] - nnz;
    if (rt == 0 && w == 0) rev_ptr[(long)grp * g.KB + mycol] = my_cbase;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    row_ptr[g.R] = nnz;
    rev_ptr[(long)g.groups * g.KB] = sums_total[0] - nnz;
  }
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // forward entries: wave w takes rows 16w .. 16w+15, lanes are columns
  for (int r = 16 * w; r < 16 * w + 16; r++) {
    const bool bit = tile[r * kTileStride + lane] != 0;
    const unsigned long long bits = __ballot(bit);
    const int base = __shfl(my_rbase, r);
    if (bit) col[base + __popcll(bits & below)] = ct * 64 + lane;
  }
  // reverse entries: wave w takes columns 16w .. 16w+15, lanes are rows
  for (int c = 16 * w; c < 16 * w + 16; c++) {
    const bool bit = tile[lane * kTileStride + c] != 0;
    const unsigned long long bits = __ballot(bit);
    const int base = __shfl(my_cbase, c);
    if (bit) rev[base + __popcll(bits & below)] = lrow;
  }
}

MaskTileGeom mask_geom(int B, int N1, int N2, int QB, int KB) {
  MaskTileGeom g;
  g.R = B * N1 * QB;
  g.KB = KB;
  g.QB = QB;
  g.G = N1 / N2;
  g.RG = g.G * QB;
  g.RTG = (g.RG + 63) / 64;
  g.CT = (KB + 63) / 64;
  g.groups = B * N2;
  return g;
}

long bsa_compact_parts_len(int B, int N1, int N2, int QB, int KB) {
  MaskTileGeom g = mask_geom(B, N1, N2, QB, KB);
  return (long)g.R * g.CT + (long)g.groups * g.KB * g.RTG;
}

hipError_t launch_bsa_compact(const uint8_t* mask, int B, int N1, int N2, int QB, int KB,
                              int* parts, int* sums, int* row_ptr, int* col, int* rev_ptr,
                              int* rev, hipStream_t st) {
  MaskTileGeom g = mask_geom(B, N1, N2, QB, KB);
  const long nparts = bsa_compact_parts_len(B, N1, N2, QB, KB);
  const int ntiles = g.groups * g.RTG * g.CT;
  hipLaunchKernelGGL(bsa_mask_count, dim3(ntiles), dim3(64 * kMaskWaves), 0, st, mask, g, parts);
  hipError_t e = exclusive_scan(parts, nparts, sums, st);
  if (e != hipSuccess) return e;
  const int nt = (int)((nparts + kScanTile - 1) / kScanTile);
  hipLaunchKernelGGL(bsa_mask_fill, dim3(ntiles), dim3(64 * kMaskWaves), 0, st, mask, g, parts,
                     sums + nt, row_ptr, col, rev_ptr, rev);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Work order of the attention kernels: tiles by list length, longest first,
// equal lengths in tile order (head-major), so that the workgroups dealt out
// last are the short ones while tiles of one head that cost the same stay
// together (their K/V or Q/dO stay in cache).  A stable counting sort in
// LDS, one workgroup per list set (workgroup 0 the forward lists, 1 the
// reverse lists): each wave counts the buckets of its contiguous segment of
// tiles, a bucket-major scan over (bucket, wave) gives every wave its slots,
// and each wave places its tiles in index order, ranking equal buckets among
// the 64 lanes of a step with ballots.  Lengths of kOrderBins - 1 and more
// share the first bucket.  order[k] is the tile of rank k.  The order decides
// only which workgroup starts when, never a result.
// ---------------------------------------------------------------------------
constexpr int kOrderBins = 256;

// Segment plan of the BSA dK/dV work items, made by the workgroup that
// ordered the KV tiles.  The segment length S = max(1, ceil(E * ksub /
// kBsaDkdvSlots)) for E reverse-list entries in all keeps every segment
// within one workgroup slot's fair share of the work, so a KV block that
// many Q blocks selected no longer sets the kernel's length.  Work item r
// (KV tile order[r / ksub], key split r % ksub) with L entries gets
// max(1, ceil(L / S)) segments, and fp32 partial slots only when it has more
// than one: fewer than 2 * kBsaDkdvSlots slots in all (each split item has
// L > S, so ceil(L / S) < 2 L / S).  Writes exclusive prefix sums with their
// totals at [n_items], and the split items' ranks in ascending order at
// seg_meta[2..] with their count at seg_meta[1] (fewer than kBsaDkdvSlots).
__device__ void bsa_seg_plan(const int* rev_ptr, int n_tiles, const int* order, int ksub,
                             int n_items, int* seg_off, int* part_off, int* seg_meta) {
  const long E = rev_ptr[n_tiles];
  const int S = (int)max(1L, (E * ksub + kBsaDkdvSlots - 1) / kBsaDkdvSlots);
  if (threadIdx.x == 0) seg_meta[0] = S;
  int carry_s = 0, carry_p = 0, carry_x = 0;
  for (int base = 0; base < n_items; base += blockDim.x) {
    const int r = base + threadIdx.x;
    int ns = 0;
    if (r < n_items) {
      const int tile = order[r / ksub];
      ns = max(1, (rev_ptr[tile + 1] - rev_ptr[tile] + S - 1) / S);
    }
    const int np = ns > 1 ? ns : 0;
    int ts;
    const int es = block_excl_scan(ns, &ts);
    // partial slots (fewer than 2^16 in all) in the low half, split items in
    // the high half: one scan for both
    int tpx;
    const int epx = block_excl_scan(np | (np > 0 ? 1 << 16 : 0), &tpx);
    if (r < n_items) {
      seg_off[r] = carry_s + es;
      part_off[r] = carry_p + (epx & 0xffff);
      if (np > 0) seg_meta[2 + carry_x + (epx >> 16)] = r;
    }
    carry_s += ts;
    carry_p += tpx & 0xffff;
    carry_x += tpx >> 16;
  }
  if (threadIdx.x == 0) {
    seg_off[n_items] = carry_s;
    part_off[n_items] = carry_p;
    seg_meta[1] = carry_x;
  }
}

__global__ __launch_bounds__(1024) void tile_order(const int* ptr_a, int n_a, int* ord_a,
                                                   const int* ptr_b, int n_b, int* ord_b,
                                                   BsaSegPlan plan) {
  const int* ptr = blockIdx.x ? ptr_b : ptr_a;
  const int n = blockIdx.x ? n_b : n_a;
  int* ord = blockIdx.x ? ord_b : ord_a;
  __shared__ int cnt[16][kOrderBins];  // [wave][bucket]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  auto bucket = [&](int i) { return kOrderBins - 1 - min(ptr[i + 1] - ptr[i], kOrderBins - 1); };
  const int seg = (n + 15) / 16;
  const int lo = min(w * seg, n), hi = min(lo + seg, n);
  for (int i = tid; i < 16 * kOrderBins; i += 1024) (&cnt[0][0])[i] = 0;
  __syncthreads();
  for (int i = lo + lane; i < hi; i += 64) atomicAdd(&cnt[w][bucket(i)], 1);
  __syncthreads();
  // exclusive scan in (bucket, wave) order: thread t owns flat entries
  // 4t .. 4t+3, entry f = bucket * 16 + wave
  int v[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int f = 4 * tid + j;
    v[j] = cnt[f & 15][f >> 4];
    sum += v[j];
  }
  int total;
  int ex = block_excl_scan(sum, &total);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int f = 4 * tid + j;
    cnt[f & 15][f >> 4] = ex;
    ex += v[j];
  }
  __syncthreads();
  // each wave places its segment in index order, 64 tiles a step: a lane's
  // peers (the lanes of its bucket) are the AND over the bucket's 8 bits of
  // the ballot of that bit or of its complement; its rank among them is the
  // count of lower peers, and the lowest peer advances the bucket's slot
  static_assert(kOrderBins == 256, "8 bucket bits");
  const unsigned long long below = (1ull << lane) - 1;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const bool valid = i < hi;
    const int bk = valid ? bucket(i) : 0;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; bit++) {
      const bool on = (bk >> bit) & 1;
      const unsigned long long m = __ballot(valid && on);
      peers &= on ? m : ~m;
    }
    const int start = valid ? cnt[w][bk] : 0;  // every lane reads before any update
    const int rank = __popcll(peers & below);
    if (valid) ord[start + rank] = i;
    if (valid && rank == 0) cnt[w][bk] = start + __popcll(peers);
  }
  if (blockIdx.x == 1 && plan.seg_off) {
    __syncthreads();  // this workgroup's order writes are visible to all its threads
    bsa_seg_plan(ptr_b, n_b, ord_b, plan.ksub, plan.n_items, plan.seg_off, plan.part_off,
                 plan.seg_meta);
  }
}

hipError_t launch_tile_order(const int* row_ptr, int n_rows, int* order_rows, const int* rev_ptr,
                             int n_cols, int* order_cols, const BsaSegPlan& plan, hipStream_t st) {
  hipLaunchKernelGGL(tile_order, dim3(2), dim3(1024), 0, st, row_ptr, n_rows, order_rows, rev_ptr,
                     n_cols, order_cols, plan);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// NSA topk_indices -> forward / reverse CSR.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int seq_of(const int* cu, int nseq, int t) {
  int lo = 0, hi = nseq - 1;  // largest b with cu[b] <= t
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// A slot survives if its id is in range and, under causal mode, its block
// starts at or before the token's position.
__device__ __forceinline__ bool nsa_keep(int id, int pos, int nblk, int sbs, int causal) {
  return id >= 0 && id < nblk && (!causal || id * sbs <= pos);
}

// One thread per (t, n2) row: count of kept slots.
__global__ __launch_bounds__(256) void nsa_row_count(const int* topk, NsaGeom g, int* cnt) {
  const long r = (long)blockIdx.x * 256 + threadIdx.x;
  if (r >= (long)g.T * g.N2) return;
  const int t = (int)(r / g.N2);
  const int b = seq_of(g.cu_q, g.B, t);
  const int pos = t - g.cu_q[b];
  const int nblk = g.blk_off[b + 1] - g.blk_off[b];
  const int* row = topk + r * g.sbc;
  int c = 0;
  for (int i = 0; i < g.sbc; i++) c += nsa_keep(row[i], pos, nblk, g.sbs, g.causal);
  cnt[r] = c;
}

// One thread per (t, n2) row: each kept slot goes to its rank among the kept
// slots ordered by (id, slot).
__global__ __launch_bounds__(256) void nsa_row_fill(const int* topk, NsaGeom g, const int* row_ptr,
                                                    int* col, int* ekey, int* etok) {
  const long r = (long)blockIdx.x * 256 + threadIdx.x;
  if (r >= (long)g.T * g.N2) return;
  const int t = (int)(r / g.N2);
  const int n2 = (int)(r - (long)t * g.N2);
  const int b = seq_of(g.cu_q, g.B, t);
  const int pos = t - g.cu_q[b];
  const int nblk = g.blk_off[b + 1] - g.blk_off[b];
  const int* row = topk + r * g.sbc;
  const int base = row_ptr[r];
  for (int i = 0; i < g.sbc; i++) {
    const int vi = row[i];
    if (!nsa_keep(vi, pos, nblk, g.sbs, g.causal)) continue;
    int rank = 0;
    for (int j = 0; j < g.sbc; j++) {
      const int vj = row[j];
      if (nsa_keep(vj, pos, nblk, g.sbs, g.causal) && (vj < vi || (vj == vi && j < i))) rank++;
    }
    col[base + rank] = vi;
    if (ekey) {
      ekey[base + rank] = n2 * g.NB + g.blk_off[b] + vi;
      etok[base + rank] = t;
    }
  }
}

// Wave-parallel fill for rows of at most 64 slots: P lanes (a power of two
// >= sbc) per row, 64 / P rows per wave; lane i of a row ranks slot i against
// the row's other slots, fetched by lane shuffles.
__global__ __launch_bounds__(256) void nsa_row_fill_wave(const int* topk, NsaGeom g,
                                                         const int* row_ptr, int* col, int* ekey,
                                                         int* etok, int P) {
  const int lane = threadIdx.x & 63;
  const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rpw = 64 / P;
  const long r = wave * rpw + lane / P;
  const int i = lane % P;
  const bool live = r < (long)g.T * g.N2;
  int v = -1, t = 0, key = 0;
  bool keep = false;
  if (live && i < g.sbc) {
    t = (int)(r / g.N2);
    const int n2 = (int)(r - (long)t * g.N2);
    const int b = seq_of(g.cu_q, g.B, t);
    const int pos = t - g.cu_q[b];
    const int nblk = g.blk_off[b + 1] - g.blk_off[b];
    v = topk[r * g.sbc + i];
    keep = nsa_keep(v, pos, nblk, g.sbs, g.causal);
    key = n2 * g.NB + g.blk_off[b] + v;
  }
  const int base_lane = (lane / P) * P;
  int rank = 0;
  for (int j = 0; j < g.sbc; j++) {
    const int vj = __shfl(v, base_lane + j);
    const int kj = __shfl((int)keep, base_lane + j);
    rank += kj && (vj < v || (vj == v && j < i));
  }
  if (live && keep) {
    const int e = row_ptr[r] + rank;
    col[e] = v;
    if (ekey) {
      ekey[e] = key;
      etok[e] = t;
    }
  }
}

// Occurrences of block id in a sorted row.
__device__ __forceinline__ int count_in_sorted(const int* a, int n, int id) {
  int lo = 0, hi = n;
  while (lo < hi) { int m = (lo + hi) >> 1; if (a[m] < id) lo = m + 1; else hi = m; }
  int c = 0;
  while (lo + c < n && a[lo + c] == id) c++;
  return c;
}

// One 256-thread workgroup per (n2, global block): threads walk the tokens of
// the block's sequence, 256 at a time; pass 0 counts, pass 1 writes token ids
// in ascending order (a block-wide scan of the per-token counts places them).
template <int PASS>
__global__ __launch_bounds__(256) void nsa_rev(NsaGeom g, const int* row_ptr, const int* col,
                                               int* rev_cnt, const int* rev_ptr, int* rev) {
  const int r = blockIdx.x;
  if (r >= g.N2 * g.NB) return;
  const int n2 = r / g.NB, gb = r % g.NB;
  const int b = seq_of(g.blk_off, g.B, gb);
  const int id = gb - g.blk_off[b];
  const int t0 = g.cu_q[b], t1 = g.cu_q[b + 1];
  // under causal mode tokens before the block's first key cannot keep it
  const int tstart = g.causal ? max(t0, t0 + id * g.sbs) : t0;
  int out = PASS ? rev_ptr[r] : 0;
  int total = 0;
  for (int tb = tstart; tb < t1; tb += 256) {
    const int t = tb + threadIdx.x;
    int c = 0;
    if (t < t1) {
      const long rr = (long)t * g.N2 + n2;
      const int a0 = row_ptr[rr], a1 = row_ptr[rr + 1];
      // rows are short and sorted: count matches with independent loads
      for (int x = a0; x < a1; x++) c += col[x] == id;
    }
    if (PASS) {
      int tot;
      const int ex = block_excl_scan(c, &tot);
      for (int k = 0; k < c; k++) rev[out + ex + k] = t;
      out += tot;
    } else {
      total += c;
    }
  }
  if (!PASS) {
    int tot;
    block_excl_scan(total, &tot);
    if (threadIdx.x == 0) rev_cnt[r] = tot;
  }
}

// Reverse lists as a stable counting sort of the forward entries by their
// reverse key (n2 * NB + global block): entries in forward order are cut
// into tiles of `rounds` x 64; nsa_rev_hist counts each tile's keys,
// an exclusive scan over (key, tile) in key-major order gives every tile its
// first output slot per key, and nsa_rev_place writes the token ids.  Within
// a wave, lanes holding the same key (found with one ballot per key bit)
// are ranked by lane, and rounds run in order, so each list comes out in
// forward-entry order: tokens ascending, a listed duplicate twice.
__device__ __forceinline__ unsigned long long key_peers(int key, int bits, bool valid) {
  unsigned long long m = __ballot(valid);
  for (int b = 0; b < bits; b++) {
    const bool bit = (key >> b) & 1;
    const unsigned long long bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__global__ __launch_bounds__(64) void nsa_rev_hist(const int* n_entries, const int* ekey, int NK,
                                                   int bits, int rounds, int n_tiles, int* hist) {
  extern __shared__ int cnt[];
  const int lane = threadIdx.x, tile = blockIdx.x;
  const int E = n_entries[0];
  for (int k = lane; k < NK; k += 64) cnt[k] = 0;
  const long e0 = (long)tile * rounds * 64;
  for (int rd = 0; rd < rounds && e0 + rd * 64 < E; rd++) {
    const long e = e0 + rd * 64 + lane;
    const bool valid = e < E;
    const int key = valid ? ekey[e] : 0;
    const unsigned long long m = key_peers(key, bits, valid);
    if (valid && lane == __ffsll((long long)m) - 1) cnt[key] += __popcll(m);
  }
  for (int k = lane; k < NK; k += 64) hist[(long)k * n_tiles + tile] = cnt[k];
}

__global__ __launch_bounds__(64) void nsa_rev_place(const int* n_entries, const int* ekey,
                                                    const int* etok, int NK, int bits, int rounds,
                                                    int n_tiles, const int* hist, int* rev) {
  extern __shared__ int cnt[];
  const int lane = threadIdx.x, tile = blockIdx.x;
  const int E = n_entries[0];
  const long e0 = (long)tile * rounds * 64;
  if (e0 >= E) return;
  for (int k = lane; k < NK; k += 64) cnt[k] = hist[(long)k * n_tiles + tile];
  const unsigned long long below = (1ull << lane) - 1;
  for (int rd = 0; rd < rounds && e0 + rd * 64 < E; rd++) {
    const long e = e0 + rd * 64 + lane;
    const bool valid = e < E;
    const int key = valid ? ekey[e] : 0;
    const unsigned long long m = key_peers(key, bits, valid);
    const int at = valid ? cnt[key] + __popcll(m & below) : 0;
    if (valid) rev[at] = etok[e];
    if (valid && lane == __ffsll((long long)m) - 1) cnt[key] += __popcll(m);
  }
}

__global__ void nsa_rev_ptr(const int* n_entries, const int* hist, int NK, int n_tiles,
                            int* rev_ptr) {
  const long k = (long)blockIdx.x * 256 + threadIdx.x;
  if (k < NK) rev_ptr[k] = hist[k * n_tiles];
  if (k == NK) rev_ptr[k] = n_entries[0];
}

// Data check for validate = 1: counts ids outside [0, nblk).
// Token-group chunk lists: one wave per (KV head, token group).  Lane j
// holds token p0 + j's sorted row (staged in LDS) and a cursor into it; each
// step takes the smallest id at the cursors (a k-way merge), emits that
// block's 32-key chunks with the mask of the lanes at that id (under causal
// mode without the tokens placed before the chunk), and advances those
// lanes by one, so an id a token lists twice is emitted twice.
constexpr int kNoId = 0x7fffffff;
// A group whose ids span at most this many blocks, with no id listed twice by
// one token, takes the bitmap path below instead of the merge.
constexpr int kGroupBitmapIds = 1024;
// Minimum of x over lanes 0..15 (one DPP row), in every lane of that row.
__device__ __forceinline__ int row_min16(int x) {
  x = min(x, __builtin_amdgcn_update_dpp(kNoId, x, 0x128, 0xf, 0xf, false));  // row_ror:8
  x = min(x, __builtin_amdgcn_update_dpp(kNoId, x, 0x124, 0xf, 0xf, false));  // row_ror:4
  x = min(x, __builtin_amdgcn_update_dpp(kNoId, x, 0x122, 0xf, 0xf, false));  // row_ror:2
  x = min(x, __builtin_amdgcn_update_dpp(kNoId, x, 0x121, 0xf, 0xf, false));  // row_ror:1
  return x;
}
// Dynamic LDS of the list kernel: the group's rows (kNsaGroup * sbc ints),
// then its ascending chunk list (cap entries of two ints).
size_t nsa_group_lds_bytes(int sbc, int cap) {
  return sizeof(int) * ((size_t)kNsaGroup * sbc + 2 * (size_t)cap);
}
__global__ __launch_bounds__(64) void nsa_group_chunks(NsaGeom g, const int* row_ptr,
                                                       const int* col, NsaGroups gr) {
  extern __shared__ int dyn[];
  int* rows = dyn;                         // [kNsaGroup][sbc]
  int* lst = dyn + kNsaGroup * g.sbc;      // [cap][2]
  const int lane = threadIdx.x;
  const int unit = blockIdx.x;
  const int n2 = unit / gr.NG, gi = unit - n2 * gr.NG;
  const int b = seq_of(gr.gcu, g.B, gi);
  const int p0 = (gi - gr.gcu[b]) * kNsaGroup;
  const int t0 = g.cu_q[b] + p0;
  const int ntok = min(kNsaGroup, g.cu_q[b + 1] - t0);
  const int sbc = g.sbc, sbs = g.sbs;
  int r0 = 0, n = 0;
  if (lane < ntok) {
    const long row = (long)(t0 + lane) * g.N2 + n2;
    r0 = row_ptr[row];
    n = row_ptr[row + 1] - r0;
  }
  // stage the rows: slot i = j * sbc + e of the tile holds entry e of token
  // j's row; eight independent loads per lane in flight at a time
  const int tot = ntok * sbc;
  for (int i0 = 0; i0 < tot; i0 += 8 * 64) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int i = i0 + u * 64 + lane;
      const int j = min(i / sbc, kNsaGroup - 1), e = i - j * sbc;
      const int rj = __shfl(r0, j), nj = __shfl(n, j);
      v[u] = (i < tot && e < nj) ? col[rj + e] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int i = i0 + u * 64 + lane;
      if (i < tot) rows[i] = v[u];
    }
  }
  __syncthreads();
  const int cpb = (sbs + kNsaGroupChunk - 1) / kNsaGroupChunk;
  int* out = gr.ent + (long)unit * gr.cap * 2;
  static_assert(kNsaGroup <= 16, "one DPP row of lanes holds the group's tokens");
  // Mask of the tokens (bit j: token p0 + j) that attend to chunk s of block
  // id, given the tokens that listed the block: under causal mode the tokens
  // placed before the chunk's first key drop out.
  auto chunk_mask = [&](int id, unsigned sel, int s) {
    unsigned m = sel;
    if (g.causal) {
      const int d = id * sbs + kNsaGroupChunk * s - p0;  // tokens j < d sit before the chunk
      if (d >= 32) m = 0u;
      else if (d > 0) m &= ~((1u << d) - 1u);
    }
    return m;
  };
  auto half_flag = [&](int s) {
    return sbs - kNsaGroupChunk * s < kNsaGroupChunk ? kNsaChunkHalf : 0u;
  };
  int count = 0;
  // Bitmap path: every listed (token, id) ORs the token's bit into the id's
  // LDS word, then one ascending pass over the words emits each listed id's
  // chunks, placed by a wave prefix sum.  It gives the list the merge below
  // gives, without a serial step per id, when the group's ids span at most
  // kGroupBitmapIds blocks and no token lists an id twice (rows are sorted,
  // so a repeat sits next to its twin); otherwise the merge runs.
  __shared__ unsigned bm[kGroupBitmapIds];
  bool merged = false;
  {
    int lo = n > 0 ? rows[lane * sbc] : kNoId;        // lanes >= ntok have n = 0
    int hi = n > 0 ? rows[lane * sbc + n - 1] : -1;
    lo = __builtin_amdgcn_readfirstlane(row_min16(lo));
    hi = -__builtin_amdgcn_readfirstlane(row_min16(-hi));
    if (lo != kNoId && hi - lo < kGroupBitmapIds) {
      const int W = hi - lo + 1;
      for (int i = lane; i < W; i += 64) bm[i] = 0u;
      __syncthreads();
      bool odd = false;  // a repeated (or out-of-order) id
      for (int i0 = 0; i0 < tot; i0 += 64) {
        const int i = i0 + lane;
        const int j = min(i / sbc, kNsaGroup - 1), e = i - j * sbc;
        const int nj = __shfl(n, j);
        const bool live = i < tot && e < nj;
        const int v = live ? rows[i] : lo;
        if (live && ((e > 0 && rows[i - 1] >= v) || v < lo || v > hi)) odd = true;
        else if (live) atomicOr(&bm[v - lo], 1u << j);
      }
      const bool any_odd = __ballot(odd) != 0;
      __syncthreads();
      if (!any_odd) {
        for (int i0 = 0; i0 < W; i0 += 64) {
          const int i = i0 + lane;
          const unsigned sel = i < W ? bm[i] : 0u;
          int mine = 0;
          for (int s = 0; s < cpb; s++) mine += chunk_mask(lo + i, sel, s) != 0u;
          const int incl = wave_incl_scan(mine);
          int pos = count + incl - mine;
          for (int s = 0; s < cpb; s++) {
            const unsigned m = chunk_mask(lo + i, sel, s);
            if (m) {
              lst[2 * pos] = (lo + i) * sbs + kNsaGroupChunk * s;
              lst[2 * pos + 1] = (int)(m | half_flag(s));
              pos++;
            }
          }
          count += __shfl(incl, 63);
        }
        merged = true;
      }
    }
  }
  // Merge: lane j's cursor c, its id (head) and the id after it (nxt)
  int c = 0;
  int head = merged ? kNoId : (c < n ? rows[lane * sbc] : kNoId);
  int nxt = c + 1 < n ? rows[lane * sbc + 1] : kNoId;
  while (true) {
    // minimum over lanes 0..15 by row rotations (DPP), read from lane 0
    int mn = head;
    mn = min(mn, __builtin_amdgcn_update_dpp(kNoId, mn, 0x128, 0xf, 0xf, false));  // row_ror:8
    mn = min(mn, __builtin_amdgcn_update_dpp(kNoId, mn, 0x124, 0xf, 0xf, false));  // row_ror:4
    mn = min(mn, __builtin_amdgcn_update_dpp(kNoId, mn, 0x122, 0xf, 0xf, false));  // row_ror:2
    mn = min(mn, __builtin_amdgcn_update_dpp(kNoId, mn, 0x121, 0xf, 0xf, false));  // row_ror:1
    mn = __builtin_amdgcn_readfirstlane(mn);
    if (mn == kNoId) break;
    const unsigned sel = (unsigned)__ballot(lane < 16 && head == mn);
    for (int s = 0; s < cpb; s++) {
      const unsigned m = chunk_mask(mn, sel, s);
      if (m) {
        if (lane == 0) {
          lst[2 * count] = mn * sbs + kNsaGroupChunk * s;
          lst[2 * count + 1] = (int)(m | half_flag(s));
        }
        count++;
      }
    }
    if (head == mn) {
      c++;
      head = nxt;
      nxt = c + 1 < n ? rows[lane * sbc + c + 1] : kNoId;
    }
  }
  if (lane == 0) gr.cnt[unit] = count;
  __syncthreads();

  // Window balancing.  The consumer walks the list four chunks (one window)
  // per barrier, token j on wave j, so a window lasts as long as the SIMD
  // with the most work in it; waves of a workgroup go to the SIMDs in turn,
  // so token j works on SIMD j % 4.  Each window slot takes, among the next
  // 16 chunks of the ascending list not yet placed (held by lanes 0..15), the
  // one that keeps the window's largest per-SIMD token count lowest (the
  // earliest on a tie).  Any order gives each token the same set of chunks;
  // the online softmax is order-free up to rounding.
  // Candidates: lanes 0..63 hold the next 64 unplaced chunks in list order
  // (lanes past the list's end hold none).  A pick drops its lane and moves
  // the lanes after it down by one (a whole-wave DPP shift), so after 16
  // picks lanes 48..63 are empty and take the next 16 chunks.
  int cks = 0, cm = 0, ok = 0;
  if (lane < count) {
    cks = lst[2 * lane];
    cm = lst[2 * lane + 1];
    ok = 1;
  }
  int fetched = 64;
  int l0 = 0, l1 = 0, l2 = 0, l3 = 0;  // the window's tokens per SIMD
  for (int k = 0; k < count; k++) {
    if ((k & 3) == 0) l0 = l1 = l2 = l3 = 0;
    const int a = max(max(l0 + __popc((unsigned)cm & 0x1111u), l1 + __popc((unsigned)cm & 0x2222u)),
                      max(l2 + __popc((unsigned)cm & 0x4444u), l3 + __popc((unsigned)cm & 0x8888u)));
    const int key = ok && lane < 16 ? a * 16 + lane : kNoId;
    const int best = __builtin_amdgcn_readfirstlane(row_min16(key)) & 15;
    const int bks = __builtin_amdgcn_readlane(cks, best);
    const unsigned bm = (unsigned)__builtin_amdgcn_readlane(cm, best);
    if (lane == 0) {
      out[2 * k] = bks;
      out[2 * k + 1] = (int)bm;
    }
    l0 += __popc(bm & 0x1111u);
    l1 += __popc(bm & 0x2222u);
    l2 += __popc(bm & 0x4444u);
    l3 += __popc(bm & 0x8888u);
    const int nks = __builtin_amdgcn_update_dpp(0, cks, 0x130, 0xf, 0xf, false);  // wave_shl:1
    const int nm = __builtin_amdgcn_update_dpp(0, cm, 0x130, 0xf, 0xf, false);
    const int nok = __builtin_amdgcn_update_dpp(0, ok, 0x130, 0xf, 0xf, false);
    if (lane >= best) {
      cks = nks;
      cm = nm;
      ok = nok;
    }
    if ((k & 15) == 15) {
      const int e = fetched + lane - 48;
      if (lane >= 48) {
        ok = e < count;
        cks = ok ? lst[2 * e] : 0;
        cm = ok ? lst[2 * e + 1] : 0;
      }
      fetched += 16;
    }
  }
}

hipError_t launch_nsa_group_lists(const NsaGeom& g, const int* row_ptr, const int* col,
                                  const NsaGroups& gr, hipStream_t st) {
  const long units = (long)g.N2 * gr.NG;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(nsa_group_chunks, dim3((unsigned)units), dim3(64),
                     nsa_group_lds_bytes(g.sbc, gr.cap), st, g, row_ptr, col, gr);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void nsa_check_ids(const int* topk, NsaGeom g, int* bad) {
  const long r = (long)blockIdx.x * 256 + threadIdx.x;
  if (r >= (long)g.T * g.N2) return;
  const int t = (int)(r / g.N2);
  const int b = seq_of(g.cu_q, g.B, t);
  const int nblk = g.blk_off[b + 1] - g.blk_off[b];
  int c = 0;
  for (int i = 0; i < g.sbc; i++) {
    int v = topk[r * g.sbc + i];
    c += (v < 0 || v >= nblk);
  }
  if (c) bad[0] = 1;  // benign race: every writer stores the same value
}

hipError_t launch_nsa_check(const int* topk, const NsaGeom& g, int* bad, hipStream_t st) {
  const long rows = (long)g.T * g.N2;
  hipLaunchKernelGGL(nsa_check_ids, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, topk,
                     g, bad);
  return hipGetLastError();
}

hipError_t launch_nsa_forward_lists(const int* topk, const NsaGeom& g, int* cnt_scan, int* sums,
                                    int* row_ptr, int* col, int* ekey, int* etok,
                                    hipStream_t st) {
  const long rows = (long)g.T * g.N2;
  const unsigned rb = (unsigned)((rows + 255) / 256);
  // forward: counts -> scan -> fill
  hipLaunchKernelGGL(nsa_row_count, dim3(rb), dim3(256), 0, st, topk, g, cnt_scan);
  hipError_t e = exclusive_scan(cnt_scan, rows, sums, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(copy_ptr, dim3((unsigned)((rows + 256) / 256)), dim3(256), 0, st, cnt_scan,
                     rows, sums + (rows + kScanTile - 1) / kScanTile, row_ptr);
  if (g.sbc <= 64) {
    int P = 1;
    while (P < g.sbc) P <<= 1;
    const long waves = (rows + 64 / P - 1) / (64 / P);
    hipLaunchKernelGGL(nsa_row_fill_wave, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, topk,
                       g, row_ptr, col, ekey, etok, P);
  } else {
    hipLaunchKernelGGL(nsa_row_fill, dim3(rb), dim3(256), 0, st, topk, g, row_ptr, col, ekey, etok);
  }
  return hipGetLastError();
}

NsaRevSort nsa_rev_sort_plan(long max_entries, long n_keys) {
  NsaRevSort r;
  r.NK = (int)n_keys;
  r.bits = 1;
  while ((1L << r.bits) < n_keys) r.bits++;
  r.rounds = 16;
  // key-major (key, tile) counters: at most 8M of them
  while ((max_entries + 64L * r.rounds - 1) / (64L * r.rounds) * n_keys > (8L << 20)) r.rounds *= 2;
  r.n_tiles = (int)((max_entries + 64L * r.rounds - 1) / (64L * r.rounds));
  if (r.n_tiles < 1) r.n_tiles = 1;
  r.usable = n_keys >= 1 && n_keys <= kNsaRevMaxKeys;
  return r;
}

hipError_t launch_nsa_reverse_lists(const NsaGeom& g, const int* row_ptr, const int* col,
                                    int* sums, int* rev_scan, int* rev_ptr, int* rev,
                                    const int* ekey, const int* etok, const NsaRevSort& rs,
                                    int* hist, int* hsums, hipStream_t st) {
  // reverse: counts -> scan -> fill
  const long rrows = (long)g.N2 * g.NB;
  if (rrows == 0) return launch_fill_i32(rev_ptr, 1, 0, st);
  if (ekey && rs.usable) {
    const int* n_entries = row_ptr + (long)g.T * g.N2;
    const size_t lds = sizeof(int) * rs.NK;
    hipLaunchKernelGGL(nsa_rev_hist, dim3(rs.n_tiles), dim3(64), lds, st, n_entries, ekey, rs.NK,
                       rs.bits, rs.rounds, rs.n_tiles, hist);
    hipError_t e = exclusive_scan(hist, (long)rs.NK * rs.n_tiles, hsums, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(nsa_rev_place, dim3(rs.n_tiles), dim3(64), lds, st, n_entries, ekey, etok,
                       rs.NK, rs.bits, rs.rounds, rs.n_tiles, (const int*)hist, rev);
    hipLaunchKernelGGL(nsa_rev_ptr, dim3((unsigned)((rs.NK + 1 + 255) / 256)), dim3(256), 0, st,
                       n_entries, (const int*)hist, rs.NK, rs.n_tiles, rev_ptr);
    return hipGetLastError();
  }
  const unsigned wb = (unsigned)rrows;
  hipLaunchKernelGGL(nsa_rev<0>, dim3(wb), dim3(256), 0, st, g, row_ptr, col, rev_scan,
                     (const int*)nullptr, (int*)nullptr);
  hipError_t e = exclusive_scan(rev_scan, rrows, sums, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(copy_ptr, dim3((unsigned)((rrows + 256) / 256)), dim3(256), 0, st, rev_scan,
                     rrows, sums + (rrows + kScanTile - 1) / kScanTile, rev_ptr);
  hipLaunchKernelGGL(nsa_rev<1>, dim3(wb), dim3(256), 0, st, g, row_ptr, col, (int*)nullptr,
                     (const int*)rev_ptr, rev);
  return hipGetLastError();
}


}  // namespace tsa
