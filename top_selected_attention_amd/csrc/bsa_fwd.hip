// Block-sparse attention forward ("aclnnBlockSparseAttentionGrad", formula
// section): Out = Softmax(Mask(scale * Q K_sparse^T, atten_mask)) V_sparse,
// plus the natural-log LSE of each row.
//
// One workgroup per (b, n1, Q block) slice of up to 128 query rows; each wave
// owns 32 query rows.  The Q block's selected KV blocks are walked in 64-key
// chunks: K and V of a chunk are one contiguous slab of BNSD memory (the
// gather is a base-pointer jump), moved by direct global -> LDS loads into a
// double buffer while the previous chunk computes.
//
// The scores are computed transposed, S^T = K Q^T, on 32x32x16 MFMA: K is the
// A operand read from LDS, Q the B operand held in registers for the whole
// kernel.  In the accumulator layout a lane then owns one query column and
// 16 keys of it, so the online-softmax max and sum are in-lane plus one
// exchange with lane l^32.  P^T leaves the accumulator directly as the B
// operand of O^T += V^T P^T, with V^T read from the natural-layout V tile by
// LDS transpose reads (ds_read_b64_tr_b16).  The tiles are padded (272-byte
// rows, rows permuted within 16) so that every operand read is one base
// register plus an immediate.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {

constexpr int kD = 128;        // head dim (the page's constraint: headdim = 128)
constexpr int kKC = 64;        // keys per chunk
constexpr int kTileB = ptile_bytes(kKC);  // bytes per staged (padded) K or V chunk

// AM: an element mask (atten_mask) is given; its entries are read per chunk.
template <class E, int NW, bool AM>
__global__ __launch_bounds__(NW * 64) void bsa_fwd_kernel(BsaParams p, int qsub, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int NR = NW * 32;  // query rows per workgroup (32 per wave)
  __shared__ __attribute__((aligned(1024))) char lds_kv[2][2][kTileB];  // [stage][K, V]

  const int item = blockIdx.x;
  if (item >= n_items) return;
  // Work order: Q tiles by list length, longest first (p.order_q).
  // Workgroups go to the 8 XCDs round-robin in launch order, so every XCD
  // starts with its share of the longest lists and the short ones fill the
  // end; a head-major order left each XCD's last head's long lists for the
  // end.
  const int qs = item % qsub;
  const int tile = p.order_q[item / qsub];
  const int qb = tile % p.QB;
  const int bn = tile / p.QB;  // b * N1 + n1
  const int n1 = bn % p.N1, b = bn / p.N1;
  const int n2 = n1 / p.G;
  // rows of this sequence (BNSD: one per batch entry; TND: cu_q / cu_kv)
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
  const int qrow = wrow0 + l32;  // this lane's query column

  const T* qh = (const T*)p.q + qm.at(n1, 0);
  const T* kh = (const T*)p.k + km.at(n2, 0);
  const T* vh = (const T*)p.v + km.at(n2, 0);
  const long krow_bytes = (long)km.row * 2;

  // Q^T as the B operand of S^T = K Q^T: lane holds query l32, d = 16*ds + 8*h .. +7
  V8 qreg[8];
#pragma unroll
  for (int ds = 0; ds < 8; ds++)
    qreg[ds] = qrow < row_hi ? as_v8<V8>(ld16(qh + (long)qrow * qm.row + ds * 16 + 8 * h))
                             : zero_v8<V8>();

  // this lane's atten_mask row (positions within the sequence)
  const unsigned char* amrow = nullptr;
  if constexpr (AM) amrow = p.am + b * p.am_sb + n1 * p.am_sn + (long)qrow * p.am_pitch;

  const int tile_row = bn * p.QB + qb;
  const int e0 = p.row_ptr[tile_row], e1 = p.row_ptr[tile_row + 1];
  ListWindow colw(p.col, e0, e1);
  const int cpb = (p.bkv + kKC - 1) / kKC;
  const float sl2 = p.scale * kLog2e;

  // Chunk (e, s) covers keys [ks, ke) of KV block col[e], sub-chunk s.  Chunks that
  // are empty (ragged tail) or wholly after the slice's last row under causal
  // mode are skipped; the test is uniform across the workgroup.
  auto chunk_range = [&](ChunkPos c, int& ks, int& ke) {
    const int kb = colw(c.e);
    ks = kb * p.bkv + c.s * kKC;
    ke = min(min(ks + kKC, (kb + 1) * p.bkv), km.len);
  };
  auto next_valid = [&](ChunkPos c) {
    for (; c.e < e1; c = chunk_advance(c, cpb)) {
      int ks, ke;
      chunk_range(c, ks, ke);
      if (ks < ke && !(p.causal && ks > row_hi - 1)) break;
    }
    return c;
  };
  // Direct global -> LDS loads (no registers) into padded tiles.  Keys past
  // the chunk's end re-read its last key (finite data; their scores are
  // masked, so P = 0 exactly there).  A whole chunk takes a scalar base (its
  // first key row) plus per-lane offsets fixed for the walk.
  PStage<NW, kKC> stg;
  stg.init(wid, lane, krow_bytes);
  const unsigned lds0 = lds_addr(&lds_kv[0][0][0]);
  auto load_chunk = [&](int ks, int ke, int buf) {
    const unsigned lk = lds0 + buf * 2 * kTileB, lv = lk + kTileB;
    const char* kb = (const char*)kh + (long)ks * krow_bytes;
    const char* vb = (const char*)vh + (long)ks * krow_bytes;
    if (ke - ks == kKC) {
      stg.full(kb, lk, wid, lane);
      stg.full(vb, lv, wid, lane);
    } else {
      stg.ragged(kb, krow_bytes, ke - 1 - ks, lk, wid, lane);
      stg.ragged(vb, krow_bytes, ke - 1 - ks, lv, wid, lane);
    }
  };
  // Per-lane bases of the MFMA operand reads: K rows (key l32, +32 per key
  // tile; pieces 2*ds + h at +32*ds) and V^T by transpose reads.
  const unsigned rb = prow_base(lane), tb = ptr_base(lane);

  // Online softmax state of this lane's query, base 2.  The reference m only
  // moves when a chunk's max exceeds it by more than kLazy (so P <= 2^kLazy);
  // O and l are rescaled only then, by a wave-uniform branch.
  constexpr float kLazy = 8.f;
  float m = -INFINITY, lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int j = 0; j < 16; j++) o[dt][j] = 0.f;

  ChunkPos i = next_valid(ChunkPos{e0, 0});
  if (i.e < e1) {
    int ks, ke;
    chunk_range(i, ks, ke);
    load_chunk(ks, ke, 0);
  }
  wait_vm();
  __syncthreads();
  int buf = 0;
  while (i.e < e1) {
    int ks, ke;
    chunk_range(i, ks, ke);
    const ChunkPos inext = next_valid(chunk_advance(i, cpb));
    if (inext.e < e1) {
      int ks2, ke2;
      chunk_range(inext, ks2, ke2);
      load_chunk(ks2, ke2, buf ^ 1);
    }
    const char* Kr = &lds_kv[buf][0][0] + rb;
    const char* Vt = &lds_kv[buf][1][0] + tb;

    // S^T = K Q^T: 64 keys x 32 queries (two 32x32 tiles)
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int j = 0; j < 16; j++) st[kt][j] = 0.f;
#pragma unroll
    for (int ds = 0; ds < 8; ds++) {
      st[0] = E::mfma32(lds_read16<V8>(Kr + 32 * ds), qreg[ds], st[0]);
      st[1] = E::mfma32(lds_read16<V8>(Kr + 32 * kPadPitch + 32 * ds), qreg[ds], st[1]);
    }
    sched_mfma_lds<16, 1, 4>();
    // Element j of tile kt is key ks + kt*32 + 8*(j/4) + 4*h + j%4.  A chunk
    // wholly inside [0, ke) and at or below every row of this wave needs no
    // mask; otherwise key offsets above this lane's limit are masked (the
    // offset without the lane's 4*h is a compile-time constant per element).
    // An atten_mask clears element j of tile kt where keep bit 16*kt + j is 0.
    const bool full = !AM && (ke - ks == kKC) && (!p.causal || ke - 1 <= wrow0);
    if (!full) {
      int lim = ke - 1 - ks;
      if (p.causal) lim = min(lim, qrow - ks);
      lim -= 4 * h;
      uint32_t keep = 0xffffffffu;
      if constexpr (AM) keep = qrow < row_hi ? am_keep_row(amrow + ks, ke - ks, h, p.am_al4) : 0u;
#pragma unroll
      for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int j = 0; j < 16; j++)
          st[kt][j] = ((kt * 32 + 8 * (j >> 2) + (j & 3)) <= lim && ((keep >> (16 * kt + j)) & 1u))
                          ? st[kt][j] : -INFINITY;
    }
    float mx = vmax(st[0][0], st[1][0]);
#pragma unroll
    for (int j = 1; j < 16; j++) mx = vmax(mx, vmax(st[0][j], st[1][j]));
    mx = max_xor32(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
      const float m_new = vmax(m, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; dt++)
#pragma unroll
        for (int j = 0; j < 16; j++) o[dt][j] *= alpha;
    }
    // P^T = exp2(S^T * scale*log2e - m), fed back as the B operand of PV
    const float mneg = m == -INFINITY ? 0.f : -m;
    V8 pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const float pv = fast_exp2(__builtin_fmaf(st[kt][j], sl2, mneg));
        lsum += pv;
        pb[2 * kt + (j >> 3)][j & 7] = E::from_f32(pv);
      }
    // O^T += V^T P^T, 16 keys per step
#pragma unroll
    for (int k4 = 0; k4 < 4; k4++)
#pragma unroll
      for (int dt = 0; dt < 4; dt++)
        o[dt] = E::mfma32(ptile_tr<V8>(Vt + k4 * 16 * kPadPitch + 64 * dt), pb[k4], o[dt]);
    sched_mfma_lds<16, 2, 4>();

    wait_vm();
    __syncthreads();
    buf ^= 1;
    i = inext;
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2.
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qrow < row_hi) {
    T* orow = (T*)p.out + qm.at(n1, qrow);
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d0 = dt * 32 + 8 * jj + 4 * h;
        *reinterpret_cast<uint2*>(orow + d0) =
            pack4<E>(o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv, o[dt][4 * jj + 2] * inv,
                     o[dt][4 * jj + 3] * inv);
      }
    if (h == 0) p.lse[sm.at(n1, qrow)] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <class E, int NW>
static hipError_t launch_fwd_t(const BsaParams& p, hipStream_t st) {
  const int qsub = (p.bq + NW * 32 - 1) / (NW * 32);
  const int n_items = p.B * p.N1 * p.QB * qsub;
  const int grid = 8 * ((n_items + 7) / 8);
  if (p.am)
    hipLaunchKernelGGL((bsa_fwd_kernel<E, NW, true>), dim3(grid), dim3(NW * 64), 0, st, p, qsub,
                       n_items);
  else
    hipLaunchKernelGGL((bsa_fwd_kernel<E, NW, false>), dim3(grid), dim3(NW * 64), 0, st, p, qsub,
                       n_items);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_fwd_e(const BsaParams& p, hipStream_t st) {
  // 32 query rows per wave: up to 4 waves cover a 128-row Q block slice
  if (p.bq <= 32) return launch_fwd_t<E, 1>(p, st);
  if (p.bq <= 64) return launch_fwd_t<E, 2>(p, st);
  return launch_fwd_t<E, 4>(p, st);
}

hipError_t launch_bsa_fwd(const BsaParams& p, int fp16, hipStream_t st) {
  if (p.B * p.N1 * p.QB == 0) return hipSuccess;
  return fp16 ? launch_fwd_e<FP16>(p, st) : launch_fwd_e<BF16>(p, st);
}

}  // namespace tsa
