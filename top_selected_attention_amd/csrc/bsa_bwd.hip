// Block-sparse attention backward ("aclnnBlockSparseAttentionGrad", formula
// section):
//   softmax_grad = rowsum(dOut * Out),  dP = dOut V^T,
//   dS = P * (dP - softmax_grad),  dV = P^T dOut,
//   dQ = (dS K) scale,  dK = (dS^T Q) scale,
// over the selected blocks only, with P recomputed as exp(scale*S - LSE).
//
// Two kernels, each owning its outputs, so nothing is accumulated across
// workgroups: no atomics, one fixed summation order, bit-identical reruns.
//   * dQ: one workgroup per Q-block slice walks the Q block's KV list (the
//     forward CSR).  It first forms softmax_grad for its rows from O and dO
//     and stores it for the second kernel.
//   * dK/dV: one workgroup per KV-block slice walks the list of Q blocks that
//     selected the KV block (the reverse CSR), over all query heads of the
//     KV head's group.
// Both stage their streamed operand (K/V resp. Q/dO) in 64-row chunks through
// double-buffered, padded LDS tiles with direct global -> LDS loads, keep the
// stationary operand in registers, and feed accumulator tiles straight back
// into the next MFMA as operands (see tsa_device.h).
#include <type_traits>

#include <algorithm>

#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {

namespace {
constexpr int kD = 128;
constexpr int kTileB = ptile_bytes(64);  // one padded 64-row chunk of a [rows][128] 16-bit tensor
}  // namespace

// ---------------------------------------------------------------------------
// dQ (+ softmax_grad).  Each wave owns 32 query rows: per 32-key half of a
// chunk it forms S^T = K Q^T and dP^T = V dO^T, dS^T = P^T (dP^T - D), and
// accumulates dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------
// AM (both kernels): an element mask (atten_mask) is given.
template <class E, int NW, bool AM>
__global__ __launch_bounds__(NW * 64) void bsa_dq_kernel(BsaParams p, int qsub, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int NR = NW * 32;
  __shared__ __attribute__((aligned(1024))) char lds_kv[2][2][kTileB];  // [stage][K, V]

  const int item = blockIdx.x;
  if (item >= n_items) return;
  // work order as in the forward: Q tiles by list length, longest first
  const int qs = item % qsub;
  const int tile = p.order_q[item / qsub];
  const int qb = tile % p.QB;
  const int bn = tile / p.QB;
  const int n1 = bn % p.N1, b = bn / p.N1;
  const int n2 = n1 / p.G;
  const BsaRowMap qm = bsa_rows(p.cu_q, b, p.N1, p.Sq, kD);
  const BsaRowMap km = bsa_rows(p.cu_kv, b, p.N2, p.Skv, kD);
  const BsaRowMap sm = bsa_rows(p.cu_q, b, p.N1, p.Sq, 1);
  const int row_lo = qb * p.bq + qs * NR;
  const int row_hi = min((qb + 1) * p.bq, qm.len);
  if (row_lo >= row_hi) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);  // wave-uniform
  const int l32 = lane & 31, h = lane >> 5;
  const int wrow0 = row_lo + wid * 32;
  const int qrow = wrow0 + l32;
  const bool row_ok = qrow < row_hi;

  const long qoff = qm.at(n1, qrow);  // this lane's query row
  const T* kh = (const T*)p.k + km.at(n2, 0);
  const T* vh = (const T*)p.v + km.at(n2, 0);
  const long krow_bytes = (long)km.row * 2;

  // Stationary operands of this lane's query: Q^T and dO^T columns;
  // softmax_grad D = rowsum(dO * O) formed here and stored; LSE (base 2).
  V8 qreg[8], doreg[8];
  float dlt, lse2;
  {
    const T* qr = (const T*)p.q + qoff;
    const T* orr = (const T*)p.o + qoff;
    const T* dor = (const T*)p.dout + qoff;
    float acc = 0.f;
#pragma unroll
    for (int ds = 0; ds < 8; ds++) {
      const int off = ds * 16 + 8 * h;
      qreg[ds] = row_ok ? as_v8<V8>(ld16(qr + off)) : zero_v8<V8>();
      doreg[ds] = row_ok ? as_v8<V8>(ld16(dor + off)) : zero_v8<V8>();
      const V8 ov = row_ok ? as_v8<V8>(ld16(orr + off)) : zero_v8<V8>();
#pragma unroll
      for (int e = 0; e < 8; e++) acc += E::to_f32(doreg[ds][e]) * E::to_f32(ov[e]);
    }
    acc += __shfl_xor(acc, 32);
    dlt = acc;
    lse2 = row_ok ? p.lse[sm.at(n1, qrow)] * kLog2e : 0.f;
    // stored beside the row's LSE in base 2, the pair the dK/dV kernel reads
    if (row_ok && h == 0)
      *reinterpret_cast<float2*>(p.delta + 2 * sm.at(n1, qrow)) = make_float2(lse2, acc);
  }

  const unsigned char* amrow = nullptr;
  if constexpr (AM) amrow = p.am + b * p.am_sb + n1 * p.am_sn + (long)qrow * p.am_pitch;

  const int e0 = p.row_ptr[bn * p.QB + qb], e1 = p.row_ptr[bn * p.QB + qb + 1];
  ListWindow colw(p.col, e0, e1);
  const int cpb = (p.bkv + 63) / 64;
  const float sl2 = p.scale * kLog2e;

  auto chunk_range = [&](ChunkPos c, int& ks, int& ke) {
    const int kb = colw(c.e);
    ks = kb * p.bkv + c.s * 64;
    ke = min(min(ks + 64, (kb + 1) * p.bkv), km.len);
  };
  auto next_valid = [&](ChunkPos c) {
    ChunkAt a;
    for (a.c = c; a.c.e < e1; a.c = chunk_advance(a.c, cpb)) {
      chunk_range(a.c, a.lo, a.hi);
      if (a.lo < a.hi && !(p.causal && a.lo > row_hi - 1)) break;
    }
    return a;
  };
  // Padded K/V tiles by direct loads; a whole chunk takes a scalar base (its
  // first key row) plus per-lane offsets fixed for the walk, a ragged chunk
  // re-reads its last key.
  PStage<NW, 64> stg;
  stg.init(wid, lane, krow_bytes);
  const unsigned lds0 = lds_addr(&lds_kv[0][0][0]);
  auto load_chunk = [&](int ks, int ke, int buf) {
    const unsigned lk = lds0 + buf * 2 * kTileB, lv = lk + kTileB;
    const char* kb = (const char*)kh + (long)ks * krow_bytes;
    const char* vb = (const char*)vh + (long)ks * krow_bytes;
    if (ke - ks == 64) {
      stg.full(kb, lk, wid, lane);
      stg.full(vb, lv, wid, lane);
    } else {
      stg.ragged(kb, krow_bytes, ke - 1 - ks, lk, wid, lane);
      stg.ragged(vb, krow_bytes, ke - 1 - ks, lv, wid, lane);
    }
  };
  // per-lane bases of the operand reads: K and V rows (key l32, +32 per key
  // tile), K^T by transpose reads
  const unsigned rb = prow_base(lane), tb = ptr_base(lane);

  f32x16 dq[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int j = 0; j < 16; j++) dq[dt][j] = 0.f;
  const float lneg = -lse2;

  ChunkAt cur = next_valid(ChunkPos{e0, 0});
  if (cur.c.e < e1) load_chunk(cur.lo, cur.hi, 0);
  wait_vm();
  __syncthreads();
  int buf = 0;
  while (cur.c.e < e1) {
    const int ks = cur.lo, ke = cur.hi;
    const ChunkAt nxt = next_valid(chunk_advance(cur.c, cpb));
    if (nxt.c.e < e1) load_chunk(nxt.lo, nxt.hi, buf ^ 1);
    const char* Kr = &lds_kv[buf][0][0] + rb;
    const char* Vr = &lds_kv[buf][1][0] + rb;
    const char* Kt = &lds_kv[buf][0][0] + tb;
    const bool full =
        !AM && (ke - ks == 64) && wrow0 + 32 <= row_hi && (!p.causal || ke - 1 <= wrow0);
    // atten_mask keep bits of this lane's row: bit 16*kt + j for element j of tile kt
    uint32_t keep = 0xffffffffu;
    if constexpr (AM) keep = row_ok ? am_keep_row(amrow + ks, ke - ks, h, p.am_al4) : 0u;
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      f32x16 st, dpt;
#pragma unroll
      for (int j = 0; j < 16; j++) st[j] = dpt[j] = 0.f;
#pragma unroll
      for (int ds = 0; ds < 8; ds++) {
        st = E::mfma32(lds_read16<V8>(Kr + kt * 32 * kPadPitch + 32 * ds), qreg[ds], st);
        dpt = E::mfma32(lds_read16<V8>(Vr + kt * 32 * kPadPitch + 32 * ds), doreg[ds], dpt);
      }
      // one K and one V read per MFMA, four reads ahead
      sched_mfma_lds<16, 1, 4>();
      // dS^T = P^T * (dP^T - D), P^T = exp2(S^T * scale*log2e - LSE2);
      // element j is key ks + kt*32 + 8*(j/4) + 4*h + j%4.  Outside a full
      // chunk, key offsets above this lane's limit are masked (two copies of
      // the loop so the full path carries no compare).
      V8 bs[2];
      auto form_ds = [&](auto masked) {
        int lim = 0;
        if (masked) {
          lim = ke - 1 - ks;
          if (p.causal) lim = min(lim, qrow - ks);
          lim = row_ok ? lim - 4 * h : -1000000;
        }
#pragma unroll
        for (int j = 0; j < 16; j++) {
          float pv = fast_exp2(__builtin_fmaf(st[j], sl2, lneg));
          if (masked)
            pv = ((kt * 32 + 8 * (j >> 2) + (j & 3)) <= lim && ((keep >> (16 * kt + j)) & 1u))
                     ? pv : 0.f;
          bs[j >> 3][j & 7] = E::from_f32(pv * (dpt[j] - dlt));
        }
      };
      if (full) form_ds(std::false_type());
      else form_ds(std::true_type());
      // dQ^T += K^T dS^T over the tile's 32 keys (two 16-key steps)
#pragma unroll
      for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
          dq[dt] = E::mfma32(ptile_tr<V8>(Kt + (kt * 2 + k2) * 16 * kPadPitch + 64 * dt), bs[k2],
                             dq[dt]);
      sched_mfma_lds<8, 2, 4>();  // a transposed K^T pair per MFMA
    }
    wait_vm();
    __syncthreads();
    buf ^= 1;
    cur = nxt;
  }

  if (row_ok) {
    T* drow = (T*)p.out + qoff;
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d0 = dt * 32 + 8 * jj + 4 * h;
        *reinterpret_cast<uint2*>(drow + d0) =
            pack4<E>(dq[dt][4 * jj] * p.scale, dq[dt][4 * jj + 1] * p.scale,
                     dq[dt][4 * jj + 2] * p.scale, dq[dt][4 * jj + 3] * p.scale);
      }
  }
}

// ---------------------------------------------------------------------------
// dK / dV.  Each wave owns 32 keys of the KV block.  The block's K rows stay
// in LDS for the whole walk (read as the B operand of S); each wave keeps its
// V rows as the B operand of dP in registers.  Per 32-query chunk of a
// selecting Q block (double-buffered in LDS):
//   S = Q K^T and dP = dO V^T (queries x keys, lanes on key columns),
//   P = exp2(S * scale*log2e - LSE2), dS = P * (dP - softmax_grad),
//   dV^T += dO^T P and dK^T += Q^T dS, with dO^T / Q^T read from the staged
//   natural-layout tiles by transpose reads.
// Small chunks keep two workgroups' LDS within a CU and the live registers
// under 256, so two waves share each SIMD.
// ---------------------------------------------------------------------------
// Two waves per SIMD (register budget 256; a few spills are cheaper than
// running one wave per SIMD).
template <class E, int NW, bool AM>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void bsa_dkdv_kernel(BsaParams p, int ksub, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int NK = NW * 32;       // keys per workgroup
  constexpr int kQC = 32;           // queries per chunk
  constexpr int kQTile = ptile_bytes(kQC);
  __shared__ __attribute__((aligned(1024))) char lds_k[ptile_bytes(NK)];
  __shared__ __attribute__((aligned(1024))) char lds_qd[2][2][kQTile];  // [stage][Q, dO]
  __shared__ float lds_ld[2][64];  // per chunk row: LSE (base 2), softmax_grad

  // One workgroup per segment: segment sg belongs to work item rank (the
  // largest r with seg_off[r] <= sg), items in the order of p.order_kv
  // (KV tiles by reverse-list length, longest first), dealt round-robin over
  // the XCDs in launch order.
  const int sg = blockIdx.x;
  if (sg >= p.seg_off[n_items]) return;
  int rank = 0;
  {
    int hi = n_items - 1;
    while (rank < hi) {
      const int mid = (rank + hi + 1) >> 1;
      if (p.seg_off[mid] <= sg) rank = mid; else hi = mid - 1;
    }
  }
  const int kseg = sg - p.seg_off[rank];
  const int nseg = p.seg_off[rank + 1] - p.seg_off[rank];
  const int ksl = rank % ksub;
  const int tile = p.order_kv[rank / ksub];
  const int kb = tile % p.KB;
  const int bh = tile / p.KB;  // b * N2 + n2
  const int n2 = bh % p.N2, b = bh / p.N2;
  // rows of this sequence (BNSD: one per batch entry; TND: cu_q / cu_kv)
  const BsaRowMap qm = bsa_rows(p.cu_q, b, p.N1, p.Sq, kD);
  const BsaRowMap km = bsa_rows(p.cu_kv, b, p.N2, p.Skv, kD);
  const BsaRowMap sm = bsa_rows(p.cu_q, b, p.N1, p.Sq, 1);
  const int key_lo = kb * p.bkv + ksl * NK;
  const int key_hi = min((kb + 1) * p.bkv, km.len);
  if (key_lo >= key_hi) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);  // wave-uniform
  const int l32 = lane & 31, h = lane >> 5;
  const int wkey0 = key_lo + wid * 32;
  const int mykey = wkey0 + l32;
  const bool key_ok = mykey < key_hi;

  const long kvoff = km.at(n2, 0);
  const T* kh = (const T*)p.k + kvoff;
  const T* vh = (const T*)p.v + kvoff;

  // K rows of the workgroup into a padded LDS tile (rows past key_hi re-read
  // the last key)
  {
    PStage<NW, NK> kst;
    kst.ragged((const char*)(kh + (long)key_lo * km.row), (long)km.row * 2, key_hi - 1 - key_lo,
               lds_addr(lds_k), wid, lane);
  }
  V8 vreg[8];
#pragma unroll
  for (int ds = 0; ds < 8; ds++)
    vreg[ds] = key_ok ? as_v8<V8>(ld16(vh + (long)mykey * km.row + ds * 16 + 8 * h)) : zero_v8<V8>();

  // this segment's entries of the KV tile's reverse list
  const int c = bh * p.KB + kb;
  const int seg_len = p.seg_meta[0];
  const int e0 = p.rev_ptr[c] + kseg * seg_len;
  const int e1 = min(e0 + seg_len, p.rev_ptr[c + 1]);
  ListWindow revw(p.rev, e0, e1);
  const int cpq = (p.bq + kQC - 1) / kQC;
  const float sl2 = p.scale * kLog2e;

  // Chunk (e, s): query rows [qs, qe) (sub-chunk s) of query head n1, for
  // reverse-list entry id g*QB + qb.
  auto chunk_range = [&](ChunkPos c, int& n1, int& qs, int& qe) {
    const int id = revw(c.e);
    const int g = p.G > 1 ? id / p.QB : 0, qb = id - g * p.QB;
    n1 = n2 * p.G + g;
    qs = qb * p.bq + c.s * kQC;
    qe = min(min(qs + kQC, (qb + 1) * p.bq), qm.len);
  };
  auto next_valid = [&](ChunkPos c) {
    for (; c.e < e1; c = chunk_advance(c, cpq)) {
      int n1, qs, qe;
      chunk_range(c, n1, qs, qe);
      if (qs < qe && !(p.causal && qe - 1 < key_lo)) break;
    }
    return c;
  };
  // 32 rows of Q and of dO (padded tiles) plus their LSE / softmax_grad.  A
  // whole chunk takes a scalar base (its first row) plus per-lane offsets
  // fixed for the walk; a ragged chunk re-reads its last row.
  const long qrow_bytes = (long)qm.row * 2;
  PStage<NW, kQC> stg;
  stg.init(wid, lane, qrow_bytes);
  const unsigned lds0 = lds_addr(&lds_qd[0][0][0]);
  auto load_chunk = [&](int n1, int qs, int qe, int buf) {
    const long qoff = qm.at(n1, 0), soff = sm.at(n1, 0);
    const unsigned lq = lds0 + buf * 2 * kQTile, ld = lq + kQTile;
    const char* qb = (const char*)((const T*)p.q + qoff + (long)qs * qm.row);
    const char* db = (const char*)((const T*)p.dout + qoff + (long)qs * qm.row);
    if (qe - qs == kQC) {
      stg.full(qb, lq, wid, lane);
      stg.full(db, ld, wid, lane);
    } else {
      stg.ragged(qb, qrow_bytes, qe - 1 - qs, lq, wid, lane);
      stg.ragged(db, qrow_bytes, qe - 1 - qs, ld, wid, lane);
    }
    if (wid == 0) {
      // a direct LDS load writes lane l's dword at base + 4*l for all 64
      // lanes: the arrays hold 64 entries; entries past 32 are never read
      // lanes 2r, 2r + 1: the LSE / softmax_grad pair of the chunk's row r
      const long r = soff + (long)min(qs + (lane >> 1), qe - 1) * sm.row;
      g2lds4(p.delta + 2 * r + (lane & 1), lds_ld[buf]);
    }
  };

  // Per-lane bases of the operand reads: Q and dO rows l32, the wave's K
  // rows 32*wid + l32 (pieces 2*ds + h at +32*ds); dO^T and Q^T by transpose
  // reads.
  const unsigned rb = prow_base(lane), tb = ptr_base(lane);
  const char* Kr = lds_k + wid * 32 * kPadPitch + rb;

  f32x16 dvt[4], dkt[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int j = 0; j < 16; j++) dvt[dt][j] = dkt[dt][j] = 0.f;

  ChunkPos i = next_valid(ChunkPos{e0, 0});
  if (i.e < e1) {
    int n1, qs, qe;
    chunk_range(i, n1, qs, qe);
    load_chunk(n1, qs, qe, 0);
  }
  wait_vm();
  __syncthreads();
  int buf = 0;
  while (i.e < e1) {
    int n1, qs, qe;
    chunk_range(i, n1, qs, qe);
    const ChunkPos inext = next_valid(chunk_advance(i, cpq));
    if (inext.e < e1) {
      int n1b, qs2, qe2;
      chunk_range(inext, n1b, qs2, qe2);
      load_chunk(n1b, qs2, qe2, buf ^ 1);
    }
    const char* Qr = &lds_qd[buf][0][0] + rb;
    const char* Dr = &lds_qd[buf][1][0] + rb;
    const char* Qt = &lds_qd[buf][0][0] + tb;
    const char* Dt = &lds_qd[buf][1][0] + tb;

    // S = Q K^T and dP = dO V^T for 32 queries (rows) x this wave's 32 keys
    f32x16 s, dp;
#pragma unroll
    for (int j = 0; j < 16; j++) s[j] = dp[j] = 0.f;
#pragma unroll
    for (int ds = 0; ds < 8; ds++) {
      s = E::mfma32(lds_read16<V8>(Qr + 32 * ds), lds_read16<V8>(Kr + 32 * ds), s);
      dp = E::mfma32(lds_read16<V8>(Dr + 32 * ds), vreg[ds], dp);
    }
    // three LDS reads feed two MFMAs per step
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int u = 0; u < 8; u++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    // a chunk whose every query row is valid and at or after every key of
    // this wave needs no mask
    const bool full =
        !AM && (qe - qs == kQC) && wkey0 + 32 <= key_hi && (!p.causal || qs >= wkey0 + 31);
    // atten_mask keep bits of this lane's key column: bit j for element j
    uint32_t keep = 0xffffffffu;
    if constexpr (AM) {
      const int key = wkey0 + l32;
      keep = key < key_hi ? am_keep_col(p.am + b * p.am_sb + n1 * p.am_sn + (long)qs * p.am_pitch +
                                            key, p.am_pitch, qe - qs, h)
                          : 0u;
    }
    // element j of a lane is query 8*(j/4) + 4*h + j%4 of the chunk, column key l32
    V8 bp[2], bd[2];
    auto form = [&](auto masked) {
      int lo = 0, up = 0;
      if (masked) {
        lo = (p.causal ? wkey0 + l32 - qs : 0) - 4 * h;
        up = wkey0 + l32 < key_hi ? qe - qs - 1 - 4 * h : -1000000;
      }
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const int rbase = 8 * j4 + 4 * h;
        const float4 a4 = *reinterpret_cast<const float4*>(&lds_ld[buf][2 * rbase]);
        const float4 b4 = *reinterpret_cast<const float4*>(&lds_ld[buf][2 * rbase + 4]);
        const float lv[4] = {a4.x, a4.z, b4.x, b4.z};
        const float dv[4] = {a4.y, a4.w, b4.y, b4.w};
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int j = 4 * j4 + jj;
          float pr = fast_exp2(__builtin_fmaf(s[j], sl2, -lv[jj]));
          if (masked) {
            const int off = 8 * j4 + jj;
            pr = (off >= lo && off <= up && ((keep >> j) & 1u)) ? pr : 0.f;
          }
          bp[j >> 3][j & 7] = E::from_f32(pr);
          bd[j >> 3][j & 7] = E::from_f32(pr * (dp[j] - dv[jj]));
        }
      }
    };
    if (full) form(std::false_type());
    else form(std::true_type());
    // dV^T += dO^T P ; dK^T += Q^T dS  (16 queries per step)
#pragma unroll
    for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
      for (int dt = 0; dt < 4; dt++) {
        dvt[dt] = E::mfma32(ptile_tr<V8>(Dt + k2 * 16 * kPadPitch + 64 * dt), bp[k2], dvt[dt]);
        dkt[dt] = E::mfma32(ptile_tr<V8>(Qt + k2 * 16 * kPadPitch + 64 * dt), bd[k2], dkt[dt]);
      }
    sched_mfma_lds<16, 2, 4>();
    wait_vm();
    __syncthreads();
    buf ^= 1;
    i = inext;
  }

  if (key_ok && nseg == 1) {
    T* dkrow = (T*)p.dk + kvoff + (long)mykey * km.row;
    T* dvrow = (T*)p.dv + kvoff + (long)mykey * km.row;
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d0 = dt * 32 + 8 * jj + 4 * h;
        *reinterpret_cast<uint2*>(dkrow + d0) =
            pack4<E>(dkt[dt][4 * jj] * p.scale, dkt[dt][4 * jj + 1] * p.scale,
                     dkt[dt][4 * jj + 2] * p.scale, dkt[dt][4 * jj + 3] * p.scale);
        *reinterpret_cast<uint2*>(dvrow + d0) =
            pack4<E>(dvt[dt][4 * jj], dvt[dt][4 * jj + 1], dvt[dt][4 * jj + 2], dvt[dt][4 * jj + 3]);
      }
  } else if (key_ok) {
    // fp32 partials of a split item: [slot][dK, dV][key of the item][d]
    float* pk = p.part + ((long)(p.part_off[rank] + kseg) * 2 * NK + (mykey - key_lo)) * kD;
    float* pv = pk + (long)NK * kD;
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d0 = dt * 32 + 8 * jj + 4 * h;
        *reinterpret_cast<float4*>(pk + d0) =
            make_float4(dkt[dt][4 * jj], dkt[dt][4 * jj + 1], dkt[dt][4 * jj + 2], dkt[dt][4 * jj + 3]);
        *reinterpret_cast<float4*>(pv + d0) =
            make_float4(dvt[dt][4 * jj], dvt[dt][4 * jj + 1], dvt[dt][4 * jj + 2], dvt[dt][4 * jj + 3]);
      }
  }
}

// Sums the segments' fp32 partials of each split dK/dV work item in segment
// order (fixed order: bit-identical reruns) and writes dK (times scale) and
// dV.  Items with one segment wrote their rows themselves; the grid covers
// only the split items (their ranks listed by the segment plan), with
// kReduceParts workgroups per item, each a slice of its rows (a thread then
// sums a handful of 16-byte columns, so the segments' loads of one item are
// in flight together).
constexpr int kReduceParts = 8;
template <class E, int NW>
__global__ __launch_bounds__(256) void bsa_dkdv_reduce(BsaParams p, int ksub) {
  typedef typename E::T T;
  constexpr int NK = NW * 32;
  constexpr int kPer = 2 * NK * (kD / 4) / kReduceParts;  // 16-byte columns per workgroup
  static_assert(kPer % 256 == 0, "whole passes of the workgroup");
  if ((int)blockIdx.x >= p.seg_meta[1]) return;
  const int rank = p.seg_meta[2 + blockIdx.x];
  const int nseg = p.seg_off[rank + 1] - p.seg_off[rank];
  const int ksl = rank % ksub;
  const int tile = p.order_kv[rank / ksub];
  const int kb = tile % p.KB, bh = tile / p.KB;
  const int n2 = bh % p.N2, b = bh / p.N2;
  const BsaRowMap km = bsa_rows(p.cu_kv, b, p.N2, p.Skv, kD);
  const int key_lo = kb * p.bkv + ksl * NK;
  const int key_hi = min((kb + 1) * p.bkv, km.len);
  const float* base = p.part + (long)p.part_off[rank] * 2 * NK * kD;
  for (int i = blockIdx.y * kPer + threadIdx.x; i < (blockIdx.y + 1) * kPer; i += 256) {
    const int which = i / (NK * (kD / 4));  // 0 dK, 1 dV
    const int kk = (i / (kD / 4)) % NK, d4 = i % (kD / 4);
    const int key = key_lo + kk;
    if (key >= key_hi) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int sgi = 0; sgi < nseg; sgi++) {
      const float4 x = *reinterpret_cast<const float4*>(
          base + ((long)sgi * 2 * NK + which * NK + kk) * kD + 4 * d4);
      acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    const float sc = which ? 1.f : p.scale;
    T* dst = (T*)(which ? p.dv : p.dk) + km.at(n2, key) + 4 * d4;
    *reinterpret_cast<uint2*>(dst) = pack4<E>(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
  }
}

template <class E, int NW>
static hipError_t launch_dq_t(const BsaParams& p, hipStream_t st) {
  const int qsub = (p.bq + NW * 32 - 1) / (NW * 32);
  const int n_items = p.B * p.N1 * p.QB * qsub;
  if (n_items == 0) return hipSuccess;
  if (p.am)
    hipLaunchKernelGGL((bsa_dq_kernel<E, NW, true>), dim3(8 * ((n_items + 7) / 8)), dim3(NW * 64),
                       0, st, p, qsub, n_items);
  else
    hipLaunchKernelGGL((bsa_dq_kernel<E, NW, false>), dim3(8 * ((n_items + 7) / 8)), dim3(NW * 64),
                       0, st, p, qsub, n_items);
  return hipGetLastError();
}

// The dK/dV kernel and then the reduction of split items' partials, each a
// timed stage of its own (2 and 3).
template <class E, int NW>
static hipError_t launch_dkdv_t(const BsaParams& p, hipStream_t st, void* const* ev, int n_ev) {
  const int ksub = (p.bkv + NW * 32 - 1) / (NW * 32);
  const int n_items = p.B * p.N2 * p.KB * ksub;
  hipError_t e = mark_event(ev, n_ev, 2, 0, st);
  // the segment plan was made with the lists (launch_tile_order); at most
  // n_items + kBsaMaxParts segments, the surplus workgroups exit
  if (e == hipSuccess && n_items > 0) {
    if (p.am)
      hipLaunchKernelGGL((bsa_dkdv_kernel<E, NW, true>), dim3(n_items + kBsaMaxParts),
                         dim3(NW * 64), 0, st, p, ksub, n_items);
    else
      hipLaunchKernelGGL((bsa_dkdv_kernel<E, NW, false>), dim3(n_items + kBsaMaxParts),
                         dim3(NW * 64), 0, st, p, ksub, n_items);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 3, 0, st);
  // fewer than kBsaDkdvSlots split items, and at most half the partial slots
  const BsaDkdvShape ds = bsa_dkdv_shape(p.B, p.N1, p.N2, p.QB, p.KB, p.bkv);
  const int max_split = (int)std::min<long>(kBsaDkdvSlots, ds.max_parts / 2);
  if (e == hipSuccess && n_items > 0 && max_split > 0) {
    hipLaunchKernelGGL((bsa_dkdv_reduce<E, NW>), dim3(max_split, kReduceParts), dim3(256), 0, st,
                       p, ksub);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 3, 1, st);
  return e;
}

BsaDkdvShape bsa_dkdv_shape(int B, int N1, int N2, int QB, int KB, int bkv) {
  BsaDkdvShape s;
  const int nw = bkv <= 32 ? 1 : (bkv <= 64 ? 2 : 4);  // as launch_bwd_t picks
  s.nk = 32 * nw;
  s.ksub = (bkv + s.nk - 1) / s.nk;
  s.n_items = (long)B * N2 * KB * s.ksub;
  // partial slots: fewer than kBsaMaxParts, and fewer than twice the
  // entries of all items (R * KB bounds the reverse-list entries)
  s.max_parts = std::max(1L, std::min((long)kBsaMaxParts, 2L * B * N1 * QB * KB * s.ksub));
  return s;
}

template <class E>
static hipError_t launch_bwd_t(const BsaParams& p, hipStream_t st, void* const* ev, int n_ev) {
  hipError_t e = mark_event(ev, n_ev, 1, 0, st);
  if (e == hipSuccess)
    e = p.bq <= 32 ? launch_dq_t<E, 1>(p, st)
                   : (p.bq <= 64 ? launch_dq_t<E, 2>(p, st) : launch_dq_t<E, 4>(p, st));
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 1, st);
  if (e == hipSuccess)
    e = p.bkv <= 32 ? launch_dkdv_t<E, 1>(p, st, ev, n_ev)
                    : (p.bkv <= 64 ? launch_dkdv_t<E, 2>(p, st, ev, n_ev)
                                   : launch_dkdv_t<E, 4>(p, st, ev, n_ev));
  return e;
}

hipError_t launch_bsa_bwd(const BsaParams& p, int fp16, hipStream_t st, void* const* ev, int n_ev) {
  return fp16 ? launch_bwd_t<FP16>(p, st, ev, n_ev) : launch_bwd_t<BF16>(p, st, ev, n_ev);
}

}  // namespace tsa
