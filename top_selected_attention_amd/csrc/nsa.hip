// NSA selected attention ("aclnnNsaSelectedAttention", formulas section):
//   selected_key/value = Gather(key/value, topk_indices),
//   attention_out = Softmax(Mask(scale * query @ selected_key^T)) @ selected_value,
// TND layout, sparseMode 0 or 2 (causal).  The backward applies the chain of
// "aclnnBlockSparseAttentionGrad" (formula section) to the gathered keys;
// the Gather's gradient adds each gathered row's dK/dV back to its source row,
// which the dK/dV kernel does by walking, per KV block, the tokens that
// selected it (reverse list) -- one owner per output row, no atomics.
//
// Forward and dQ: one wave per (token, KV head), walking the selected blocks
// in 32-key chunks through its own LDS region -- no workgroup barrier.  The
// work is bound by gathering K/V (about 16 FLOP per gathered byte, nearly all
// of it served by L2), not by MFMA.  Head groups of up to 16 query heads use
// 16x16x32 MFMA with the group's heads as the 16 columns, and stage the next
// chunk in registers while the current one computes; larger groups (up to
// 32) use a 32-wide tile staged by direct global -> LDS loads.
#include <algorithm>

#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {

namespace {
constexpr int kD = 128;
constexpr int kChunk = 32;                 // keys per chunk (forward / dQ)
constexpr int kWaveTile = kChunk * kD * 2;  // bytes of one 32-row tile

__device__ __forceinline__ int seq_of_dev(const int* cu, int nseq, int t) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Stages 32 rows of 256 bytes into a swizzled per-wave tile; rowptr(r) gives
// the global address of row r (0 <= r < 32).
template <class RowPtr>
__device__ __forceinline__ void stage32_wave(char* tile, RowPtr rowptr) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4, pc = lane & 15;
#pragma unroll
  for (int inst = 0; inst < 8; inst++) {
    const int r = inst * 4 + sub;
    g2lds16(rowptr(r) + ((pc ^ swz(r)) << 4), tile + inst * 1024);
  }
}

// Per-wave 32-key tile of the 16-head kernels: key k sits in row
// 16*(k/16) + 2*(k%8) + (k/8)%2, rows 272 bytes apart (one 16-byte bank group
// further per row).  Stores of whole rows, reads of one piece from 16
// consecutive keys, and transposed reads of 32 bytes from 8 consecutive keys
// then all touch distinct banks, and every lane's addresses are one base plus
// compile-time offsets (no per-access address registers).
constexpr int kPitch = 272;
constexpr int kTile16 = kChunk * kPitch;
__device__ __forceinline__ int key_row(int k) { return (k & 16) | ((k & 7) << 1) | ((k >> 3) & 1); }
// Row of key 4*u + s (0 <= s < 4) is key_row(4*u) + 2*s.
__device__ __forceinline__ constexpr int key_row4(int u) {
  return 16 * (u >> 2) + 8 * (u & 1) + ((u >> 1) & 1);
}
}  // namespace

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(256) void nsa_fwd_kernel(NsaParams p, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  __shared__ __attribute__((aligned(1024))) char lds[4][2][kWaveTile];  // per wave: K, V

  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  // unit order: KV-head-major, tokens ascending; workgroups are dealt to the
  // 8 XCDs round-robin, so each XCD holds an even share of every stretch of
  // tokens (and of their unequal list lengths) while the K/V of the
  // sequences in progress stay in L2
  const int unit = item * 4 + wid;
  if (unit >= p.T * p.N2) return;
  const int n2 = unit / p.T, t = unit % p.T;
  const NsaGeom& g = p.g;
  const int b = seq_of_dev(g.cu_q, g.B, t);
  const int pos = t - g.cu_q[b];
  const int kv0 = g.cu_kv[b];
  const int G = p.G;
  char* Kt = lds[wid][0];
  char* Vt = lds[wid][1];

  const T* qrow = (const T*)p.q + ((long)t * p.N1 + n2 * G + l32) * kD;
  const bool col_ok = l32 < G;
  V8 qreg[8];
#pragma unroll
  for (int ds = 0; ds < 8; ds++)
    qreg[ds] = col_ok ? as_v8<V8>(ld16(qrow + ds * 16 + 8 * h)) : zero_v8<V8>();

  const long row = (long)t * p.N2 + n2;
  const int e0 = p.row_ptr[row], e1 = p.row_ptr[row + 1];
  ListWindow colw(p.col, e0, e1);
  const int sbs = g.sbs;
  const int cpb = (sbs + kChunk - 1) / kChunk;
  const int nchunks = (e1 - e0) * cpb;
  const float sl2 = p.scale * kLog2e;
  const long kstride = (long)p.N2 * kD * 2;  // bytes between consecutive tokens of one KV head
  const char* kbase = (const char*)p.k + ((long)kv0 * p.N2 + n2) * kD * 2;
  const char* vbase = (const char*)p.v + ((long)kv0 * p.N2 + n2) * kD * 2;

  float m = -INFINITY, lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int j = 0; j < 16; j++) o[dt][j] = 0.f;

  for (int i = 0; i < nchunks; i++) {
    const int blk = colw(e0 + i / cpb);
    const int ks = blk * sbs + (i % cpb) * kChunk;     // key position in the sequence
    const int ke = min(ks + kChunk, (blk + 1) * sbs);
    if (g.causal && ks > pos) continue;                // wholly after the token
    auto rp_k = [&](int r) { return kbase + (long)min(ks + r, ke - 1) * kstride; };
    auto rp_v = [&](int r) { return vbase + (long)min(ks + r, ke - 1) * kstride; };
    stage32_wave(Kt, rp_k);
    stage32_wave(Vt, rp_v);
    wait_vm();

    f32x16 st;
#pragma unroll
    for (int j = 0; j < 16; j++) st[j] = 0.f;
#pragma unroll
    for (int ds = 0; ds < 8; ds++)
      st = E::mfma32(tile_read16<V8>(Kt, l32, 2 * ds + h), qreg[ds], st);

    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int key = ks + 8 * (j >> 2) + 4 * h + (j & 3);
      const bool ok = key < ke && (!g.causal || key <= pos);
      const float s = ok ? st[j] * sl2 : -INFINITY;
      st[j] = s;
      mx = fmaxf(mx, s);
    }
    mx = wave_max_half_swap(mx);
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int j = 0; j < 16; j++) o[dt][j] *= alpha;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const float pv = fast_exp2(st[j] - m_use);
      lsum += pv;
      st[j] = pv;
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; k2++) {
      V8 pb;
#pragma unroll
      for (int e = 0; e < 8; e++) pb[e] = E::from_f32(st[8 * k2 + e]);
#pragma unroll
      for (int dt = 0; dt < 4; dt++) o[dt] = E::mfma32(tile_read_tr<V8>(Vt, k2, dt), pb, o[dt]);
    }
  }

  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (col_ok) {
    const long orow = (long)t * p.N1 + n2 * G + l32;
    T* op = (T*)p.out + orow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d0 = dt * 32 + 8 * jj + 4 * h;
        *reinterpret_cast<uint2*>(op + d0) = pack4<E>(o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv,
                                                      o[dt][4 * jj + 2] * inv, o[dt][4 * jj + 3] * inv);
      }
    if (h == 0) p.lse[orow] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Forward for head groups of up to 16 query heads: one wave per (token, KV
// head) on 16x16x32 MFMA (the group's heads are the 16 columns).  The next
// chunk's K and V rows are loaded into registers while the current chunk
// computes, each quarter-wave reading one whole 256-byte row (L1 tag lookups,
// not bytes, limit a gather whose 16 lanes touch 16 rows).  K is written to
// the wave's LDS tile and read back as the A operand of S^T = K Q^T; V then
// overwrites it and is read back transposed as the A operand of
// O^T += V^T P^T.  One 8.5 KB tile per wave and at most 168 VGPRs keep three
// waves on each SIMD.
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void nsa_fwd16_kernel(NsaParams p, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(1024))) char lds[4][kTile16];  // per wave: K, then V

  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  // unit order: KV-head-major, tokens ascending; workgroups are dealt to the
  // 8 XCDs round-robin, so each XCD holds an even share of every stretch of
  // tokens (and of their unequal list lengths) while the K/V of the
  // sequences in progress stay in L2
  const int unit = item * 4 + wid;
  if (unit >= p.T * p.N2) return;
  const int n2 = unit / p.T, t = unit % p.T;
  const NsaGeom& g = p.g;
  const int b = seq_of_dev(g.cu_q, g.B, t);
  const int pos = t - g.cu_q[b];
  const int kv0 = g.cu_kv[b];
  const int G = p.G;
  char* Tl = lds[wid];

  // Q^T as the B operand: lane (head l16, quarter gq) holds dims 32*ks + 8*gq .. +7
  const bool col_ok = l16 < G;
  V8 qreg[4];
  {
    const T* qrow = (const T*)p.q + ((long)t * p.N1 + n2 * G + (col_ok ? l16 : 0)) * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
      qreg[ks] = col_ok ? as_v8<V8>(ld16(qrow + 32 * ks + 8 * gq)) : zero_v8<V8>();
  }

  const long row = (long)t * p.N2 + n2;
  const int e0 = p.row_ptr[row], e1 = p.row_ptr[row + 1];
  const ShortList blocks(p.col + e0, e1 - e0);  // sbc <= 128 entries
  const int sbs = g.sbs;
  const int cpb = (sbs + kChunk - 1) / kChunk;
  const float sl2 = p.scale * kLog2e;
  const long kstride = (long)p.N2 * kD;  // elements between consecutive tokens of one KV head
  const T* kbase = (const T*)p.k + ((long)kv0 * p.N2 + n2) * kD;
  const T* vbase = (const T*)p.v + ((long)kv0 * p.N2 + n2) * kD;

  auto chunk_range = [&](ChunkPos c, int& ks, int& ke) {
    const int blk = blocks(c.e - e0);
    ks = blk * sbs + c.s * kChunk;
    ke = min(ks + kChunk, (blk + 1) * sbs);
  };
  auto next_valid = [&](ChunkPos c) {
    for (; c.e < e1; c = chunk_advance(c, cpb)) {
      int ks, ke;
      chunk_range(c, ks, ke);
      if (!(g.causal && ks > pos)) break;  // wholly after the token: skipped
    }
    return c;
  };
  // K and V chunks as 32 x 256-byte tiles, 8 16-byte pieces per lane (row
  // 4*u + lane/16, piece lane%16): every quarter-wave reads one whole row.
  // Keys past the chunk's end re-read its last key.
  const int rstride = p.N2 * kD;  // elements between consecutive tokens of one KV head
  auto load = [&](const T* base, ChunkPos c, uint4 (&r8)[8]) {
    int ks, ke;
    chunk_range(c, ks, ke);
    const T* cb = base + (long)ks * kstride + 8 * (lane & 15);
    const int last = ke - 1 - ks;  // rows past it re-read the chunk's last key
#pragma unroll
    for (int u = 0; u < 8; u++) r8[u] = ld16(cb + min(4 * u + (lane >> 4), last) * rstride);
  };
  // tile bases: row stores (key 4*u + gq, piece l16), A-operand reads (key
  // 16*kt + l16, piece 4*q4 + gq), transposed reads (keys 4*gq + l16/4 and
  // +16, bytes 32*dt + 8*(l16%4) ..)
  char* const Tw = Tl + 2 * gq * kPitch + 16 * l16;
  char* const Tr = Tl + key_row(l16) * kPitch + 16 * gq;
  char* const Tt = Tl + key_row(4 * gq + (l16 >> 2)) * kPitch + 8 * (l16 & 3);
  auto to_lds = [&](const uint4 (&r8)[8]) {
#pragma unroll
    for (int u = 0; u < 8; u++) *reinterpret_cast<uint4*>(Tw + key_row4(u) * kPitch) = r8[u];
  };

  constexpr float kLazy = 8.f;
  float m = -INFINITY, lsum = 0.f;
  f32x4_t o[8];  // O^T tiles: d = 16*dt + 4*gq + j, column head l16
#pragma unroll
  for (int dt = 0; dt < 8; dt++) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 kr[8], vr[8];
  // One step per chunk c, whose K and V loads are in flight; nx is the next
  // chunk (c itself after the last one, so the loads stay unconditional).
  // The wave's one LDS tile holds K, then V: LDS operations of a wave run in
  // order, so V's stores follow the S reads of K.
  auto step = [&](ChunkPos c, ChunkPos nx) {
    int ks, ke;
    chunk_range(c, ks, ke);
    to_lds(kr);
    load(kbase, nx, kr);
    // S^T tiles: element j of st[kt] is key ks + 16*kt + 4*gq + j, column head
    // l16; A operand = key row 16*kt + l16, dims 32*q4 + 8*gq ..
    f32x4_t st[2];
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++)
        st[kt] = E::mfma16(lds_read16<V8>(Tr + kt * 16 * kPitch + 64 * q4), qreg[q4], st[kt]);
    }
    to_lds(vr);
    load(vbase, nx, vr);
    const int lim = min(ke - 1, g.causal ? pos : 0x7fffffff) - ks;  // last kept key offset
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float v = (16 * kt + 4 * gq + j) <= lim ? st[kt][j] : -INFINITY;
        st[kt][j] = v;
        mx = fmaxf(mx, v);
      }
    mx = max_xor16_32(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; dt++) o[dt] *= alpha;
    }
    const float mneg = m == -INFINITY ? 0.f : -m;
    V8 pb;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float pv = fast_exp2(__builtin_fmaf(st[kt][j], sl2, mneg));
        lsum += pv;
        pb[4 * kt + j] = E::from_f32(pv);
      }
    // O^T += V^T P^T: V^T rows d = 16*dt + l16, keys {4gq..4gq+3, 16+4gq..16+4gq+3}
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      o[dt] = E::mfma16(lds_read_tr_pair<V8>(Tt + 32 * dt, Tt + 16 * kPitch + 32 * dt), pb, o[dt]);
  };

  ChunkPos c = next_valid(ChunkPos{e0, 0});
  if (c.e < e1) {
    load(kbase, c, kr);
    load(vbase, c, vr);
  }
  while (c.e < e1) {
    const ChunkPos nx = next_valid(chunk_advance(c, cpb));
    step(c, nx.e < e1 ? nx : c);
    c = nx;
  }

  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  if (col_ok) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const long orow = (long)t * p.N1 + n2 * G + l16;
    T* op = (T*)p.out + orow * kD;
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      *reinterpret_cast<uint2*>(op + 16 * dt + 4 * gq) =
          pack4<E>(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (gq == 0) p.lse[orow] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// dQ (+ softmax_grad): one wave per (token, KV head)
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(256) void nsa_dq_kernel(NsaParams p, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  __shared__ __attribute__((aligned(1024))) char lds[4][2][kWaveTile];

  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int unit = item * 4 + wid;
  if (unit >= p.T * p.N2) return;
  const int n2 = unit / p.T, t = unit % p.T;
  const NsaGeom& g = p.g;
  const int b = seq_of_dev(g.cu_q, g.B, t);
  const int pos = t - g.cu_q[b];
  const int kv0 = g.cu_kv[b];
  const int G = p.G;
  char* Kt = lds[wid][0];
  char* Vt = lds[wid][1];

  const bool col_ok = l32 < G;
  const long qr = (long)t * p.N1 + n2 * G + l32;
  V8 qreg[8], doreg[8];
  float acc = 0.f;
#pragma unroll
  for (int ds = 0; ds < 8; ds++) {
    const long off = qr * kD + ds * 16 + 8 * h;
    qreg[ds] = col_ok ? as_v8<V8>(ld16((const T*)p.q + off)) : zero_v8<V8>();
    doreg[ds] = col_ok ? as_v8<V8>(ld16((const T*)p.dout + off)) : zero_v8<V8>();
    const V8 ov = col_ok ? as_v8<V8>(ld16((const T*)p.o + off)) : zero_v8<V8>();
#pragma unroll
    for (int e = 0; e < 8; e++) acc += E::to_f32(doreg[ds][e]) * E::to_f32(ov[e]);
  }
  acc += __shfl_xor(acc, 32);
  const float dlt = acc;
  const float lse2 = col_ok ? p.lse[qr] * kLog2e : 0.f;
  if (col_ok && h == 0) p.delta[qr] = dlt;

  const long row = (long)t * p.N2 + n2;
  const int e0 = p.row_ptr[row], e1 = p.row_ptr[row + 1];
  ListWindow colw(p.col, e0, e1);
  const int sbs = g.sbs;
  const int cpb = (sbs + kChunk - 1) / kChunk;
  const int nchunks = (e1 - e0) * cpb;
  const float sl2 = p.scale * kLog2e;
  const long kstride = (long)p.N2 * kD * 2;
  const char* kbase = (const char*)p.k + ((long)kv0 * p.N2 + n2) * kD * 2;
  const char* vbase = (const char*)p.v + ((long)kv0 * p.N2 + n2) * kD * 2;

  f32x16 dq[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int j = 0; j < 16; j++) dq[dt][j] = 0.f;

  for (int i = 0; i < nchunks; i++) {
    const int blk = colw(e0 + i / cpb);
    const int ks = blk * sbs + (i % cpb) * kChunk;
    const int ke = min(ks + kChunk, (blk + 1) * sbs);
    if (g.causal && ks > pos) continue;
    auto rp_k = [&](int r) { return kbase + (long)min(ks + r, ke - 1) * kstride; };
    auto rp_v = [&](int r) { return vbase + (long)min(ks + r, ke - 1) * kstride; };
    stage32_wave(Kt, rp_k);
    stage32_wave(Vt, rp_v);
    wait_vm();

    f32x16 st, dpt;
#pragma unroll
    for (int j = 0; j < 16; j++) st[j] = dpt[j] = 0.f;
#pragma unroll
    for (int ds = 0; ds < 8; ds++) {
      st = E::mfma32(tile_read16<V8>(Kt, l32, 2 * ds + h), qreg[ds], st);
      dpt = E::mfma32(tile_read16<V8>(Vt, l32, 2 * ds + h), doreg[ds], dpt);
    }
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int key = ks + 8 * (j >> 2) + 4 * h + (j & 3);
      const bool ok = col_ok && key < ke && (!g.causal || key <= pos);
      const float pv = ok ? fast_exp2(st[j] * sl2 - lse2) : 0.f;
      st[j] = pv * (dpt[j] - dlt);
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; k2++) {
      V8 bs;
#pragma unroll
      for (int e = 0; e < 8; e++) bs[e] = E::from_f32(st[8 * k2 + e]);
#pragma unroll
      for (int dt = 0; dt < 4; dt++) dq[dt] = E::mfma32(tile_read_tr<V8>(Kt, k2, dt), bs, dq[dt]);
    }
  }

  if (col_ok) {
    T* dp = (T*)p.out + qr * kD;
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int d0 = dt * 32 + 8 * jj + 4 * h;
        *reinterpret_cast<uint2*>(dp + d0) =
            pack4<E>(dq[dt][4 * jj] * p.scale, dq[dt][4 * jj + 1] * p.scale,
                     dq[dt][4 * jj + 2] * p.scale, dq[dt][4 * jj + 3] * p.scale);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ for head groups of up to 16 query heads, on 16x16x32 MFMA with the same
// register-staged gather and single LDS tile as the 16-head forward:
// dP^T = V dO^T from the V tile, then K replaces it for S^T = K Q^T,
// dS^T = P^T (dP^T - softmax_grad), and dQ^T += K^T dS^T with K^T read
// transposed from the tile.
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void nsa_dq16_kernel(NsaParams p, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(1024))) char lds[4][kTile16];  // per wave: V, then K

  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int unit = item * 4 + wid;
  if (unit >= p.T * p.N2) return;
  const int n2 = unit / p.T, t = unit % p.T;
  const NsaGeom& g = p.g;
  const int b = seq_of_dev(g.cu_q, g.B, t);
  const int pos = t - g.cu_q[b];
  const int kv0 = g.cu_kv[b];
  const int G = p.G;
  char* Tl = lds[wid];

  // Q^T and dO^T as B operands: lane (head l16, quarter gq) holds dims
  // 32*ks + 8*gq .. +7; softmax_grad = rowsum(dO * O) of head l16.
  const bool col_ok = l16 < G;
  const long qr = (long)t * p.N1 + n2 * G + (col_ok ? l16 : 0);
  V8 qreg[4], doreg[4];
  float acc = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ks++) {
    const long off = qr * kD + 32 * ks + 8 * gq;
    qreg[ks] = col_ok ? as_v8<V8>(ld16((const T*)p.q + off)) : zero_v8<V8>();
    doreg[ks] = col_ok ? as_v8<V8>(ld16((const T*)p.dout + off)) : zero_v8<V8>();
    const V8 ov = col_ok ? as_v8<V8>(ld16((const T*)p.o + off)) : zero_v8<V8>();
#pragma unroll
    for (int e = 0; e < 8; e++) acc += E::to_f32(doreg[ks][e]) * E::to_f32(ov[e]);
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  const float dlt = acc;
  const float lse2 = col_ok ? p.lse[qr] * kLog2e : 0.f;
  if (col_ok && gq == 0) p.delta[qr] = dlt;

  const long row = (long)t * p.N2 + n2;
  const int e0 = p.row_ptr[row], e1 = p.row_ptr[row + 1];
  const ShortList blocks(p.col + e0, e1 - e0);  // sbc <= 128 entries
  const int sbs = g.sbs;
  const int cpb = (sbs + kChunk - 1) / kChunk;
  const float sl2 = p.scale * kLog2e;
  const long kstride = (long)p.N2 * kD;
  const T* kbase = (const T*)p.k + ((long)kv0 * p.N2 + n2) * kD;
  const T* vbase = (const T*)p.v + ((long)kv0 * p.N2 + n2) * kD;

  auto chunk_range = [&](ChunkPos c, int& ks, int& ke) {
    const int blk = blocks(c.e - e0);
    ks = blk * sbs + c.s * kChunk;
    ke = min(ks + kChunk, (blk + 1) * sbs);
  };
  auto next_valid = [&](ChunkPos c) {
    for (; c.e < e1; c = chunk_advance(c, cpb)) {
      int ks, ke;
      chunk_range(c, ks, ke);
      if (!(g.causal && ks > pos)) break;
    }
    return c;
  };
  const int rstride = p.N2 * kD;
  auto load = [&](const T* base, ChunkPos c, uint4 (&r8)[8]) {
    int ks, ke;
    chunk_range(c, ks, ke);
    const T* cb = base + (long)ks * kstride + 8 * (lane & 15);
    const int last = ke - 1 - ks;
#pragma unroll
    for (int u = 0; u < 8; u++) r8[u] = ld16(cb + min(4 * u + (lane >> 4), last) * rstride);
  };
  // tile bases: row stores (key 4*u + gq, piece l16), A-operand reads (key
  // 16*kt + l16, piece 4*q4 + gq), transposed reads (keys 4*gq + l16/4 and
  // +16, bytes 32*dt + 8*(l16%4) ..)
  char* const Tw = Tl + 2 * gq * kPitch + 16 * l16;
  char* const Tr = Tl + key_row(l16) * kPitch + 16 * gq;
  char* const Tt = Tl + key_row(4 * gq + (l16 >> 2)) * kPitch + 8 * (l16 & 3);
  auto to_lds = [&](const uint4 (&r8)[8]) {
#pragma unroll
    for (int u = 0; u < 8; u++) *reinterpret_cast<uint4*>(Tw + key_row4(u) * kPitch) = r8[u];
  };

  f32x4_t dq[8];  // dQ^T tiles: d = 16*dt + 4*gq + j, column head l16
#pragma unroll
  for (int dt = 0; dt < 8; dt++) dq[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 kr[8], vr[8];
  // One step per chunk c, whose K and V loads are in flight; nx is the next
  // chunk (c itself after the last one).  The wave's one LDS tile holds V,
  // then K (a wave's LDS operations run in order).
  auto step = [&](ChunkPos c, ChunkPos nx) {
    int ks, ke;
    chunk_range(c, ks, ke);
    // element j of st[kt] / dpt[kt]: key ks + 16*kt + 4*gq + j, column head l16
    f32x4_t st[2], dpt[2];
    to_lds(vr);
    load(vbase, nx, vr);
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      dpt[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++)
        dpt[kt] = E::mfma16(lds_read16<V8>(Tr + kt * 16 * kPitch + 64 * q4), doreg[q4], dpt[kt]);
    }
    to_lds(kr);
    load(kbase, nx, kr);
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++)
        st[kt] = E::mfma16(lds_read16<V8>(Tr + kt * 16 * kPitch + 64 * q4), qreg[q4], st[kt]);
    }
    const int lim = min(ke - 1, g.causal ? pos : 0x7fffffff) - ks;  // last kept key offset
    V8 bs;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const bool ok = col_ok && (16 * kt + 4 * gq + j) <= lim;
        const float pv = ok ? fast_exp2(__builtin_fmaf(st[kt][j], sl2, -lse2)) : 0.f;
        bs[4 * kt + j] = E::from_f32(pv * (dpt[kt][j] - dlt));
      }
    // dQ^T += K^T dS^T: K^T rows d = 16*dt + l16, keys {4gq..4gq+3, 16+4gq..16+4gq+3}
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      dq[dt] = E::mfma16(lds_read_tr_pair<V8>(Tt + 32 * dt, Tt + 16 * kPitch + 32 * dt), bs, dq[dt]);
  };

  ChunkPos c = next_valid(ChunkPos{e0, 0});
  if (c.e < e1) {
    load(vbase, c, vr);
    load(kbase, c, kr);
  }
  while (c.e < e1) {
    const ChunkPos nx = next_valid(chunk_advance(c, cpb));
    step(c, nx.e < e1 ? nx : c);
    c = nx;
  }

  if (col_ok) {
    T* dp = (T*)p.out + qr * kD;
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      *reinterpret_cast<uint2*>(dp + 16 * dt + 4 * gq) =
          pack4<E>(dq[dt][0] * p.scale, dq[dt][1] * p.scale, dq[dt][2] * p.scale,
                   dq[dt][3] * p.scale);
  }
}

// ---------------------------------------------------------------------------
// dK / dV.  The tokens that selected a (KV head, block) -- its reverse list --
// are cut into segments of at most kSegEntries listings, so a block that
// thousands of tokens selected is shared by many workgroups.  A workgroup
// walks its segments' tokens in chunks of 32 query rows (32 / G tokens x G
// heads); each wave owns 32 of the block's keys:
//   S = Q K^T, dP = dO V^T, P = exp2(S*scale*log2e - LSE2),
//   dS = P (dP - softmax_grad), dV^T += dO^T P, dK^T += Q^T dS,
// and writes fp32 partial dK/dV of its segment.  A reduction kernel then sums
// each block's segments in segment order: no atomics, a fixed summation
// order, bit-identical reruns.
// ---------------------------------------------------------------------------
constexpr int kSegEntries = 256;

// Workgroups of the dK/dV partial kernel: about three resident per CU on
// 256 CUs, a multiple of the 8 XCDs, never more than the segments.
int nsa_dkdv_grid(const NsaParams& p) {
  const int g = std::min(kNsaDkdvMaxGrid, std::max(1, p.max_segments));
  return 8 * ((g + 7) / 8);
}

int nsa_max_segments(long total_entries, long nblocks) {
  return (int)(nblocks + (total_entries + kSegEntries - 1) / kSegEntries);
}

__global__ void nsa_seg_count(const int* rev_ptr, int nblocks, int* seg_cnt) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= nblocks) return;
  const int len = rev_ptr[r + 1] - rev_ptr[r];
  seg_cnt[r] = max(1, (len + kSegEntries - 1) / kSegEntries);
}

template <class E, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void nsa_dkdv_seg_kernel(NsaParams p, int nblocks, float* part) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int kQC = 32;                  // query rows per chunk
  constexpr int kQTile = kQC * kD * 2;
  __shared__ __attribute__((aligned(1024))) char lds_k[NW * 32 * kD * 2];
  __shared__ __attribute__((aligned(1024))) char lds_q[2][kQTile];
  __shared__ __attribute__((aligned(1024))) char lds_do[2][kQTile];
  // a direct LDS load writes all 64 lanes' dwords: rows 32..63 are never read
  __shared__ float lds_lse[2][64];
  __shared__ float lds_dlt[2][64];
  __shared__ int lds_pos[2][64];
  __shared__ int lds_tok[kSegEntries];  // the segment's token ids

  const NsaGeom& g = p.g;
  const int* seg_off = p.seg_off;
  // Segments are dealt round-robin (workgroup w takes w, w + grid, ...), so
  // all workgroups move through the (KV head, sequence, block) order
  // together: the Q and dO rows in use at any time are those of one stretch
  // of sequences, which stay in MALL, rather than of every sequence and head
  // at once.
  const int w = blockIdx.x;
  const int nseg = seg_off[nblocks];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int G = p.G;
  const int tpc = max(1, kQC / G);  // tokens per chunk (G <= 32)
  const int sbs = g.sbs;
  const float sl2 = p.scale * kLog2e;
  // chunk row -> (token of the chunk, head): shifts when G is a power of two
  const bool gpow2 = (G & (G - 1)) == 0;
  const int gsh = __builtin_ctz(G);
  auto div_g = [&](int x, int& qq, int& rr) {
    if (gpow2) {
      qq = x >> gsh;
      rr = x & (G - 1);
    } else {
      qq = x / G;
      rr = x - qq * G;
    }
  };

  for (int sg = w; sg < nseg; sg += gridDim.x) {
    // segment -> block (largest r with seg_off[r] <= sg)
    int lo = 0, hi = nblocks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg_off[mid] <= sg) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int k = sg - seg_off[r];
    const int n2 = r / g.NB, gb = r % g.NB;
    const int b = seq_of_dev(g.blk_off, g.B, gb);
    const int blk = gb - g.blk_off[b];
    const int kv0 = g.cu_kv[b], q0 = g.cu_q[b];
    const int skv = g.cu_kv[b + 1] - kv0;
    const int key_lo = blk * sbs;
    const int key_hi = min((blk + 1) * sbs, skv);
    const int wkey0 = key_lo + wid * 32;
    const int e0 = p.rev_ptr[r] + k * kSegEntries;
    const int e1 = min(e0 + kSegEntries, p.rev_ptr[r + 1]);

    // K rows of the block into LDS (rows past key_hi re-read the last key);
    // V rows of this wave's keys as the B operand of dP in registers
    {
      const int sub = lane >> 4, pc = lane & 15;
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int inst = wid * 8 + u;
        const int rr = inst * 4 + sub;
        const long key = kv0 + min(key_lo + rr, key_hi - 1);
        g2lds16((const char*)((const T*)p.k + (key * p.N2 + n2) * kD) + ((pc ^ swz(rr)) << 4),
                lds_k + inst * 1024);
      }
    }
    V8 vreg[8];
    {
      const int mykey = wkey0 + l32;
      const long vrow = ((long)(kv0 + min(mykey, key_hi - 1)) * p.N2 + n2) * kD;
#pragma unroll
      for (int ds = 0; ds < 8; ds++)
        vreg[ds] = mykey < key_hi ? as_v8<V8>(ld16((const T*)p.v + vrow + ds * 16 + 8 * h))
                                  : zero_v8<V8>();
    }
    const int nchunks = (e1 - e0 + tpc - 1) / tpc;
    // the segment's token ids into LDS once, so chunk addresses need no
    // dependent global load
    for (int x = tid; x < e1 - e0; x += NW * 64) lds_tok[x] = p.rev[e0 + x];
    __syncthreads();

    // chunk row rr -> (entry c*tpc + rr/G of the segment, head rr%G); rows
    // past the chunk's tokens re-read its last valid row and are masked.
    // The token ids of all of a wave's rows are read from LDS first, then
    // the direct loads are issued.
    auto load_chunk = [&](int c, int buf) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int sub = ln >> 4, pc = ln & 15;
      const int nt = min(tpc, e1 - e0 - c * tpc);
      constexpr int U = 8 / NW;
      int tok[U], gh[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int rr = (wid * U + u) * 4 + sub;
        int tq, tr;
        div_g(rr, tq, tr);
        gh[u] = (tq < nt && rr < tpc * G) ? tr : G - 1;
        tok[u] = lds_tok[c * tpc + min(tq, nt - 1)];
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int inst = wid * U + u;
        const int rr = inst * 4 + sub;
        const long qrw = (long)tok[u] * p.N1 + n2 * G + gh[u];
        g2lds16((const char*)((const T*)p.q + qrw * kD) + ((pc ^ swz(rr)) << 4),
                lds_q[buf] + inst * 1024);
        g2lds16((const char*)((const T*)p.dout + qrw * kD) + ((pc ^ swz(rr)) << 4),
                lds_do[buf] + inst * 1024);
      }
      if (wid == 0) {
        int tq, tr;
        div_g(ln & 31, tq, tr);
        const bool valid = ln < kQC && tq < nt && ln < tpc * G;
        const int t = lds_tok[c * tpc + min(tq, nt - 1)];
        const long qrw = (long)t * p.N1 + n2 * G + (valid ? tr : G - 1);
        g2lds4(p.lse + qrw, lds_lse[buf]);
        g2lds4(p.delta + qrw, lds_dlt[buf]);
        // position of the row's token, or -1 for padding rows (always masked)
        lds_pos[buf][ln] = valid ? t - q0 : -1;
      }
    };

    f32x16 dvt[4], dkt[4];
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int j = 0; j < 16; j++) dvt[dt][j] = dkt[dt][j] = 0.f;

    if (nchunks > 0) load_chunk(0, 0);
    wait_vm();
    __syncthreads();
    int buf = 0;
    for (int c = 0; c < nchunks; c++) {
      if (c + 1 < nchunks) load_chunk(c + 1, buf ^ 1);
      // lane terms of this iteration from an opaque lane id (not kept, and
      // spilled, across iterations)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int l32i = ln & 31, hi2 = ln >> 5;
      const char* Qb = lds_q[buf];
      const char* Db = lds_do[buf];
      // S = Q K^T and dP = dO V^T: 32 rows x this wave's 32 keys
      f32x16 sc, dp;
#pragma unroll
      for (int j = 0; j < 16; j++) sc[j] = dp[j] = 0.f;
#pragma unroll
      for (int ds = 0; ds < 8; ds++) {
        sc = E::mfma32(tile_read16<V8>(Qb, l32i, 2 * ds + hi2),
                       tile_read16<V8>(lds_k, wid * 32 + l32i, 2 * ds + hi2), sc);
        dp = E::mfma32(tile_read16<V8>(Db, l32i, 2 * ds + hi2), vreg[ds], dp);
      }
      // element j of a lane is row 8*(j/4) + 4*h + j%4 of the chunk, column key l32
      const int mykey = wkey0 + l32i;
      const int need = g.causal ? mykey : 0;
      const bool key_ok = mykey < key_hi;
      V8 bp[2], bd[2];
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const int rbase = 8 * j4 + 4 * hi2;
        const float4 lse4 = *reinterpret_cast<const float4*>(&lds_lse[buf][rbase]);
        const float4 dl4 = *reinterpret_cast<const float4*>(&lds_dlt[buf][rbase]);
        const int4 ps4 = *reinterpret_cast<const int4*>(&lds_pos[buf][rbase]);
        const float lv[4] = {lse4.x, lse4.y, lse4.z, lse4.w};
        const float dv[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
        const int pv4[4] = {ps4.x, ps4.y, ps4.z, ps4.w};
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int j = 4 * j4 + jj;
          // a valid row (pos >= 0) at or after this key (causal) keeps it
          const bool ok = key_ok && pv4[jj] >= need;
          float pr = fast_exp2(__builtin_fmaf(sc[j], sl2, -lv[jj] * kLog2e));
          pr = ok ? pr : 0.f;
          bp[j >> 3][j & 7] = E::from_f32(pr);
          bd[j >> 3][j & 7] = E::from_f32(pr * (dp[j] - dv[jj]));
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS  (16 rows per step)
#pragma unroll
      for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
          dvt[dt] = E::mfma32(tile_read_tr<V8>(Db, k2, dt, ln), bp[k2], dvt[dt]);
          dkt[dt] = E::mfma32(tile_read_tr<V8>(Qb, k2, dt, ln), bd[k2], dkt[dt]);
        }
      wait_vm();
      __syncthreads();
      buf ^= 1;
    }

    // fp32 partials of this segment: [segment][key within block][d], dK then dV
    const int mykey = wkey0 + l32;
    if (mykey < key_hi) {
      float* pk = part + ((long)sg * 2 * sbs + (mykey - key_lo)) * kD;
      float* pv = pk + (long)sbs * kD;
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
    __syncthreads();  // the next segment reuses the LDS buffers
  }
}

// dK = scale * sum of a block's segment partials, dV = their sum, in segment
// order; one thread per (block, key, 4 columns).
template <class E>
__global__ __launch_bounds__(256) void nsa_dkdv_reduce(NsaParams p, const int* seg_off, int nblocks,
                                                       const float* part) {
  const NsaGeom& g = p.g;
  const int sbs = g.sbs;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long per_block = (long)sbs * (kD / 4);
  if (i >= (long)nblocks * per_block) return;
  const int r = (int)(i / per_block);
  const int key = (int)(i % per_block) / (kD / 4);
  const int d0 = 4 * ((int)(i % per_block) % (kD / 4));
  const int n2 = r / g.NB, gb = r % g.NB;
  const int b = seq_of_dev(g.blk_off, g.B, gb);
  const int blk = gb - g.blk_off[b];
  const int kv0 = g.cu_kv[b];
  const int skv = g.cu_kv[b + 1] - kv0;
  const int kpos = blk * sbs + key;
  if (kpos >= skv) return;
  float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), av = ak;
  for (int sg = seg_off[r]; sg < seg_off[r + 1]; sg++) {
    const float* pk = part + ((long)sg * 2 * sbs + key) * kD + d0;
    const float4 x = *reinterpret_cast<const float4*>(pk);
    const float4 y = *reinterpret_cast<const float4*>(pk + (long)sbs * kD);
    ak.x += x.x; ak.y += x.y; ak.z += x.z; ak.w += x.w;
    av.x += y.x; av.y += y.y; av.z += y.z; av.w += y.w;
  }
  const long orow = ((long)(kv0 + kpos) * p.N2 + n2) * kD + d0;
  typedef typename E::T T;
  *reinterpret_cast<uint2*>((T*)p.dk + orow) =
      pack4<E>(ak.x * p.scale, ak.y * p.scale, ak.z * p.scale, ak.w * p.scale);
  *reinterpret_cast<uint2*>((T*)p.dv + orow) = pack4<E>(av.x, av.y, av.z, av.w);
}

template <class E>
static hipError_t fwd_t(const NsaParams& p, hipStream_t st) {
  const int units = p.T * p.N2;
  const int n_items = (units + 3) / 4;
  if (n_items == 0) return hipSuccess;
  if (p.G <= 16)
    hipLaunchKernelGGL((nsa_fwd16_kernel<E>), dim3(8 * ((n_items + 7) / 8)), dim3(256), 0, st, p,
                       n_items);
  else
    hipLaunchKernelGGL((nsa_fwd_kernel<E>), dim3(8 * ((n_items + 7) / 8)), dim3(256), 0, st, p,
                       n_items);
  return hipGetLastError();
}

hipError_t launch_nsa_fwd(const NsaParams& p, int fp16, hipStream_t st) {
  return fp16 ? fwd_t<FP16>(p, st) : fwd_t<BF16>(p, st);
}

template <class E>
static hipError_t bwd_t(const NsaParams& p, hipStream_t st, void* const* ev, int n_ev) {
  hipError_t e = mark_event(ev, n_ev, 1, 0, st);
  const int units = p.T * p.N2;
  const int n_items = (units + 3) / 4;
  if (e == hipSuccess && n_items > 0) {
    if (p.G <= 16)
      hipLaunchKernelGGL((nsa_dq16_kernel<E>), dim3(8 * ((n_items + 7) / 8)), dim3(256), 0, st,
                         p, n_items);
    else
      hipLaunchKernelGGL((nsa_dq_kernel<E>), dim3(8 * ((n_items + 7) / 8)), dim3(256), 0, st, p,
                         n_items);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 0, st);
  const int nb = p.N2 * p.g.NB;
  if (e == hipSuccess && nb > 0) {
    // segment table: counts, then their exclusive scan (total at the end)
    hipLaunchKernelGGL(nsa_seg_count, dim3((nb + 255) / 256), dim3(256), 0, st, p.rev_ptr, nb,
                       p.seg_off);
    e = exclusive_scan_total(p.seg_off, nb, p.seg_sums, st);
  }
  if (e == hipSuccess && nb > 0) {
    const int nw = (p.g.sbs + 31) / 32;  // 1..4 waves, 32 keys each
    const int grid = nsa_dkdv_grid(p);
    if (nw <= 1)
      hipLaunchKernelGGL((nsa_dkdv_seg_kernel<E, 1>), dim3(grid), dim3(64), 0, st, p, nb,
                         p.part);
    else if (nw <= 2)
      hipLaunchKernelGGL((nsa_dkdv_seg_kernel<E, 2>), dim3(grid), dim3(128), 0, st, p, nb,
                         p.part);
    else
      hipLaunchKernelGGL((nsa_dkdv_seg_kernel<E, 4>), dim3(grid), dim3(256), 0, st, p, nb,
                         p.part);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 3, 0, st);
  if (e == hipSuccess && nb > 0) {
    const long n = (long)nb * p.g.sbs * (kD / 4);
    hipLaunchKernelGGL((nsa_dkdv_reduce<E>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       p, p.seg_off, nb, (const float*)p.part);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 3, 1, st);
  return e;
}

hipError_t launch_nsa_bwd(const NsaParams& p, int fp16, hipStream_t st, void* const* ev, int n_ev) {
  return fp16 ? bwd_t<FP16>(p, st, ev, n_ev) : bwd_t<BF16>(p, st, ev, n_ev);
}

}  // namespace tsa
