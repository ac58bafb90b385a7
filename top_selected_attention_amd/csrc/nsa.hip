// NSA selected attention ("aclnnNsaSelectedAttention", formulas section):
//   selected_key/value = Gather(key/value, topk_indices),
//   attention_out = Softmax(Mask(scale * query @ selected_key^T)) @ selected_value,
// TND layout, sparseMode 0 or 2 (causal).  The backward applies the chain of
// "aclnnBlockSparseAttentionGrad" (formula section) to the gathered keys;
// the Gather's gradient adds each gathered row's dK/dV back to its source row,
// which the dK/dV kernel does by walking, per KV block, the tokens that
// selected it (reverse list) -- one owner per output row, no atomics.
//
// Forward and dQ: head groups of up to 16 query heads of 128 dims run the
// token-group kernels below (16 consecutive tokens of a sequence share every
// K/V chunk their selections have in common, staged once per group); larger
// groups (up to 32), and query/key heads of 192 dims (values of 128), run one
// wave per (token, KV head) on a 32-wide tile, walking the token's selected
// blocks in 32-key chunks staged by direct global -> LDS loads.
#include <algorithm>
#include <type_traits>

#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {

namespace {
constexpr int kD = 128;                    // query/key head dim of the 128-dim kernels
constexpr int kDv = 128;                   // value head dim
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

}  // namespace

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
// DQK: query/key head dim, 128 or 192 (values are kDv = 128 wide).  A
// 192-dim key row is staged as two 256-byte tiles, its bytes 0..255 and
// 128..383 (dims 0..127 and 64..191): the second tile's pieces 8..15 hold
// dims 128..191, so both tiles keep the one swizzled 256-byte layout.
template <class E, int DQK>
__global__ __launch_bounds__(256) void nsa_fwd_kernel(NsaParams p, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int NKT = DQK == 128 ? 1 : 2;  // K tiles per chunk
  static_assert(DQK == 128 || DQK == 192, "query/key head dim 128 or 192");
  __shared__ __attribute__((aligned(1024))) char lds[4][NKT + 1][kWaveTile];  // per wave: K.., V

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
  char* Kt2 = lds[wid][NKT - 1];  // dims 64..191 (DQK = 192)
  char* Vt = lds[wid][NKT];

  const T* qrow = (const T*)p.q + ((long)t * p.N1 + n2 * G + l32) * DQK;
  const bool col_ok = l32 < G;
  V8 qreg[DQK / 16];
#pragma unroll
  for (int ds = 0; ds < DQK / 16; ds++)
    qreg[ds] = col_ok ? as_v8<V8>(ld16(qrow + ds * 16 + 8 * h)) : zero_v8<V8>();

  const long row = (long)t * p.N2 + n2;
  const int e0 = p.row_ptr[row], e1 = p.row_ptr[row + 1];
  ListWindow colw(p.col, e0, e1);
  const int sbs = g.sbs;
  const int cpb = (sbs + kChunk - 1) / kChunk;
  const int nchunks = (e1 - e0) * cpb;
  const float sl2 = p.scale * kLog2e;
  // bytes between consecutive tokens of one KV head
  const long kstride = (long)p.N2 * DQK * 2, vstride = (long)p.N2 * kDv * 2;
  const char* kbase = (const char*)p.k + ((long)kv0 * p.N2 + n2) * DQK * 2;
  const char* vbase = (const char*)p.v + ((long)kv0 * p.N2 + n2) * kDv * 2;

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
    auto rp_k2 = [&](int r) { return kbase + (long)min(ks + r, ke - 1) * kstride + 128; };
    auto rp_v = [&](int r) { return vbase + (long)min(ks + r, ke - 1) * vstride; };
    stage32_wave(Kt, rp_k);
    if constexpr (NKT == 2) stage32_wave(Kt2, rp_k2);
    stage32_wave(Vt, rp_v);
    wait_vm();

    f32x16 st;
#pragma unroll
    for (int j = 0; j < 16; j++) st[j] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DQK / 16; ds++)
      st = E::mfma32(ds < 8 ? tile_read16<V8>(Kt, l32, 2 * ds + h)
                            : tile_read16<V8>(Kt2, l32, 2 * (ds - 4) + h),
                     qreg[ds], st);

    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int key = ks + 8 * (j >> 2) + 4 * h + (j & 3);
      const bool ok = key < ke && (!g.causal || key <= pos);
      const float s = ok ? st[j] * sl2 : -INFINITY;
      st[j] = s;
      mx = vmax(mx, s);
    }
    mx = max_xor32(mx);
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
    T* op = (T*)p.out + orow * kDv;
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
// dQ (+ softmax_grad): one wave per (token, KV head)
// ---------------------------------------------------------------------------
// DQK as in the forward: 192-dim key rows staged as two overlapping tiles.
template <class E, int DQK>
__global__ __launch_bounds__(256) void nsa_dq_kernel(NsaParams p, int n_items) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int NKT = DQK == 128 ? 1 : 2;
  __shared__ __attribute__((aligned(1024))) char lds[4][NKT + 1][kWaveTile];

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
  char* Kt2 = lds[wid][NKT - 1];  // dims 64..191 (DQK = 192)
  char* Vt = lds[wid][NKT];

  const bool col_ok = l32 < G;
  const long qr = (long)t * p.N1 + n2 * G + l32;
  V8 qreg[DQK / 16], doreg[kDv / 16];
#pragma unroll
  for (int ds = 0; ds < DQK / 16; ds++)
    qreg[ds] = col_ok ? as_v8<V8>(ld16((const T*)p.q + qr * DQK + ds * 16 + 8 * h))
                      : zero_v8<V8>();
  float acc = 0.f;
#pragma unroll
  for (int ds = 0; ds < kDv / 16; ds++) {
    const long off = qr * kDv + ds * 16 + 8 * h;
    doreg[ds] = col_ok ? as_v8<V8>(ld16((const T*)p.dout + off)) : zero_v8<V8>();
    const V8 ov = col_ok ? as_v8<V8>(ld16((const T*)p.o + off)) : zero_v8<V8>();
#pragma unroll
    for (int e = 0; e < 8; e++) acc += E::to_f32(doreg[ds][e]) * E::to_f32(ov[e]);
  }
  acc += __shfl_xor(acc, 32);
  const float dlt = acc;
  const float lse2 = col_ok ? p.lse[qr] * kLog2e : 0.f;
  if (col_ok && h == 0) *reinterpret_cast<float2*>(p.delta + 2 * qr) = make_float2(lse2, dlt);

  const long row = (long)t * p.N2 + n2;
  const int e0 = p.row_ptr[row], e1 = p.row_ptr[row + 1];
  ListWindow colw(p.col, e0, e1);
  const int sbs = g.sbs;
  const int cpb = (sbs + kChunk - 1) / kChunk;
  const int nchunks = (e1 - e0) * cpb;
  const float sl2 = p.scale * kLog2e;
  const long kstride = (long)p.N2 * DQK * 2, vstride = (long)p.N2 * kDv * 2;
  const char* kbase = (const char*)p.k + ((long)kv0 * p.N2 + n2) * DQK * 2;
  const char* vbase = (const char*)p.v + ((long)kv0 * p.N2 + n2) * kDv * 2;

  f32x16 dq[DQK / 32];
#pragma unroll
  for (int dt = 0; dt < DQK / 32; dt++)
#pragma unroll
    for (int j = 0; j < 16; j++) dq[dt][j] = 0.f;

  for (int i = 0; i < nchunks; i++) {
    const int blk = colw(e0 + i / cpb);
    const int ks = blk * sbs + (i % cpb) * kChunk;
    const int ke = min(ks + kChunk, (blk + 1) * sbs);
    if (g.causal && ks > pos) continue;
    auto rp_k = [&](int r) { return kbase + (long)min(ks + r, ke - 1) * kstride; };
    auto rp_k2 = [&](int r) { return kbase + (long)min(ks + r, ke - 1) * kstride + 128; };
    auto rp_v = [&](int r) { return vbase + (long)min(ks + r, ke - 1) * vstride; };
    stage32_wave(Kt, rp_k);
    if constexpr (NKT == 2) stage32_wave(Kt2, rp_k2);
    stage32_wave(Vt, rp_v);
    wait_vm();

    f32x16 st, dpt;
#pragma unroll
    for (int j = 0; j < 16; j++) st[j] = dpt[j] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DQK / 16; ds++)
      st = E::mfma32(ds < 8 ? tile_read16<V8>(Kt, l32, 2 * ds + h)
                            : tile_read16<V8>(Kt2, l32, 2 * (ds - 4) + h),
                     qreg[ds], st);
#pragma unroll
    for (int ds = 0; ds < kDv / 16; ds++)
      dpt = E::mfma32(tile_read16<V8>(Vt, l32, 2 * ds + h), doreg[ds], dpt);
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
      for (int dt = 0; dt < DQK / 32; dt++)
        dq[dt] = E::mfma32(dt < 4 ? tile_read_tr<V8>(Kt, k2, dt) : tile_read_tr<V8>(Kt2, k2, dt - 2),
                           bs, dq[dt]);
    }
  }

  if (col_ok) {
    T* dp = (T*)p.out + qr * DQK;
#pragma unroll
    for (int dt = 0; dt < DQK / 32; dt++)
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
// Token-group forward and dQ (head groups of up to 16 query heads, 128-dim
// heads).  A workgroup takes kNsaGroup = 16 consecutive tokens of one
// sequence and one KV head, and walks the group's chunk list (the ascending
// union of its tokens' selected blocks in 32-key chunks, each with the mask
// of the tokens that attend to it) four chunks at a time: the waves load the
// 8 K and V tiles of the next window straight into LDS while the current
// window computes, and one barrier per window hands the buffers over.  A K/V
// row is so gathered once per group instead of once per token.  Each wave
// owns TPW tokens (TPW = 1: 16 waves, four per SIMD; TPW = 2 pairs tokens w
// and 15 - w in 8 waves, and every fragment read from LDS then feeds both
// tokens' MFMAs when both attend, which measured slower for want of waves to
// hide latency) and, for each chunk one of its tokens attends to, computes
// that token's 16-head x 32-key scores on 16x16x32 MFMA from the shared
// tiles.  A token visits its chunks in ascending block order, as the
// per-token kernels do.
// ---------------------------------------------------------------------------
namespace {
constexpr int kGrpTPW = 1;                                // tokens per wave (1 or 2)
constexpr int kGrpSlots = 4;                              // chunks per window
constexpr int kGrpTile = kChunk * 256;                    // one K or V tile, 8 KB
constexpr int kGrpLds = 2 * kGrpSlots * 2 * kGrpTile;     // two windows, 128 KB
static_assert(kNsaGroupChunk == kChunk, "list chunks are kernel chunks");

// Tiles of the token-group kernels: key k of a chunk in row k (256 bytes),
// its 16-byte piece c at piece c ^ gswz(k).  gswz is a bijection on each run
// of 16 rows, and gswz >> 1 is one on rows 0-7, on rows 8-15, on the even
// and on the odd rows of a run; so the operand reads below -- 16 rows x one
// piece, 16 rows x two adjacent pieces (32 lanes), and transpose reads of 4
// or 8 consecutive rows x one aligned piece pair -- touch distinct banks
// whether a read is served 16 or 32 lanes at a time.  A lane's read
// addresses differ only in bits the loop index XORs in, so each is the
// lane's base address XOR a constant.
__device__ __forceinline__ int gswz(int k) {
  return ((((k & 7) ^ ((k >> 3) & 1)) << 1) | ((k >> 3) & 1));
}
typedef __attribute__((address_space(3))) const uint4 lds_u4_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
template <typename V8>
__device__ __forceinline__ V8 lds16_at(unsigned a) {
  return __builtin_bit_cast(V8, *(lds_u4_t*)(uintptr_t)a);
}
template <typename V8>
__device__ __forceinline__ V8 ldstr_at(unsigned a0, unsigned a1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)a0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(uintptr_t)a1);
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(V8, v);
}
// Per-lane base of the row reads (key 16*kt + l16, logical piece 4*q4 + gq:
// base ^ 64*q4, + 4096*kt) and of the transpose reads (keys 4*gq + l16/4
// (+16), bytes 32*dt + 8*(l16%4): base ^ 32*dt, + 4096 for the second half).
__device__ __forceinline__ unsigned grp_row_base(int l16, int gq) {
  return (unsigned)(l16 * 256 + 16 * (gq ^ gswz(l16)));
}
__device__ __forceinline__ unsigned grp_tr_base(int l16, int gq) {
  const int k = 4 * gq + (l16 >> 2);
  return (unsigned)(k * 256 + 16 * (((l16 & 3) >> 1) ^ gswz(k)) + 8 * (l16 & 1));
}

struct GrpUnit {
  int n2, p0, ntok, t0, kv0;
};
__device__ __forceinline__ GrpUnit grp_unit(const NsaParams& p, int unit) {
  GrpUnit u;
  u.n2 = unit / p.grp.NG;
  const int gi = unit - u.n2 * p.grp.NG;
  const int b = seq_of_dev(p.grp.gcu, p.g.B, gi);
  u.p0 = (gi - p.grp.gcu[b]) * kNsaGroup;
  u.t0 = p.g.cu_q[b] + u.p0;
  u.ntok = min(kNsaGroup, p.g.cu_q[b + 1] - u.t0);
  u.kv0 = p.g.cu_kv[b];
  return u;
}

// A wave's share of a window's loads: of the 8 tiles (K and V of 4 slots),
// tile wid % 8 (slot tile / 2, K for even tiles, V for odd), slices
// (wid / 8) * SPW .. + SPW - 1 of its eight 1-KB slices of direct loads;
// lane l's bytes of slice sl land in row 4*sl + l/16, physical piece l%16.
// A chunk of 16 keys (a block size that is an odd multiple of 16) re-reads
// keys 0..15 into rows 16..31, which no score keeps.
template <int SPW>
struct GrpLoader {
  const char* base;  // key row 0 of the sequence's KV head
  unsigned rowb;     // bytes between consecutive tokens of one KV head
  int s0;            // first slice
  __device__ __forceinline__ void init(const NsaParams& p, const GrpUnit& u, int wid) {
    rowb = (unsigned)p.N2 * kD * 2;
    base = (const char*)((wid & 1) ? p.v : p.k) + ((long)u.kv0 * p.N2 + u.n2) * kD * 2;
    s0 = (wid >> 3) * SPW;
  }
  // chunk of keys [ks, ks + nvalid) into the tile at LDS address lds
  __device__ __forceinline__ void issue(int ks, int nvalid, unsigned lds, int lane) const {
    const char* sb = base + (long)ks * rowb;
#pragma unroll
    for (int u = 0; u < SPW; u++) {
      const int sl = s0 + u;
      const int k = 4 * sl + (lane >> 4);
      const int kk = nvalid < kChunk ? (k & 15) : k;
      g2lds16_so_at(sb, (unsigned)kk * rowb + 16u * (unsigned)((lane & 15) ^ gswz(k)),
                    lds + 1024u * sl);
    }
  }
};

// A window's four list entries, held by lanes 0..3 (read back with readlane).
struct GrpWin {
  int ks, msk;
  __device__ __forceinline__ void fetch(const int* ent, int cnt, int w, int lane) {
    const int e = w * kGrpSlots + lane;
    ks = 0;
    msk = 0;
    if (lane < kGrpSlots && e < cnt) {
      ks = ent[2 * e];
      msk = ent[2 * e + 1];
    }
  }
};
}  // namespace

template <class E, int TPW>
__global__ __launch_bounds__(kNsaGroup / TPW * 64) void nsa_fwd_grp_kernel(NsaParams p) {
  constexpr int NW = kNsaGroup / TPW;  // waves
  typedef typename E::T T;
  typedef typename E::V8 V8;
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(1024))) char lds[kGrpLds];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar branches
  const int l16 = lane & 15, gq = lane >> 4;
  const GrpUnit u = grp_unit(p, blockIdx.x);
  const NsaGeom& g = p.g;
  const int G = p.G;
  const bool col_ok = l16 < G;
  const int sbs = g.sbs;
  const float sl2 = p.scale * kLog2e;
  constexpr float kLazy = 8.f;

  // the wave's two tokens: j = wid and 15 - wid of the group
  const int jt[2] = {wid, TPW == 2 ? kNsaGroup - 1 - wid : wid};
  bool live[2];
  V8 q[2][4];
  f32x4_t o[2][8];
  float m[2], lsum[2];
#pragma unroll
  for (int i = 0; i < TPW; i++) {
    live[i] = jt[i] < u.ntok;
    const bool ok = live[i] && col_ok;
    const T* qrow = (const T*)p.q + ((long)(u.t0 + (live[i] ? jt[i] : 0)) * p.N1 + u.n2 * G +
                                     (col_ok ? l16 : 0)) * kD;
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) q[i][q4] = ok ? as_v8<V8>(ld16(qrow + 32 * q4 + 8 * gq)) : zero_v8<V8>();
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[i][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[i] = -INFINITY;
    lsum[i] = 0.f;
  }

  const int cnt = p.grp.cnt[blockIdx.x];
  const int* ent = p.grp.ent + (long)blockIdx.x * p.grp.cap * 2;
  const int nwin = (cnt + kGrpSlots - 1) / kGrpSlots;
  GrpLoader<64 / NW> ld;
  ld.init(p, u, wid);
  const unsigned lds0 = lds_addr(lds);
  const int my_slot = (wid & 7) >> 1;
  auto tile_addr = [&](int buf, int slot, int kv) {
    return lds0 + (unsigned)(((buf * kGrpSlots + slot) * 2 + kv) * kGrpTile);
  };
  auto nvalid_of = [&](unsigned msk) { return (msk & kNsaChunkHalf) ? kChunk / 2 : kChunk; };
  auto issue = [&](const GrpWin& wn, int w, int buf) {
    if (w * kGrpSlots + my_slot < cnt) {
      const int ks = __builtin_amdgcn_readlane(wn.ks, my_slot);
      const unsigned msk = (unsigned)__builtin_amdgcn_readlane(wn.msk, my_slot);
      ld.issue(ks, nvalid_of(msk), tile_addr(buf, my_slot, wid & 1), lane);
    }
  };

  const unsigned rd = grp_row_base(l16, gq), tt = grp_tr_base(l16, gq);

  // One chunk for the tokens the compile-time flags A, B (tokens 0, 1 of the
  // wave) name: straight-line code, so every LDS read can be issued ahead of
  // the MFMAs that use it.
  auto chunk = [&](auto A, auto B, unsigned Kt, int ks, int nv) {
    constexpr bool sa = decltype(A)::value, sb = decltype(B)::value;
    const unsigned Vt = Kt + kGrpTile;
    V8 f[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) f[kt][q4] = lds16_at<V8>(((Kt + rd) ^ (64u * q4)) + 4096u * kt);
    // S^T tiles: element j of st[i][kt] is key ks + 16*kt + 4*gq + j, head l16
    f32x4_t st[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      if (!(i == 0 ? sa : sb)) continue;
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        st[i][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) st[i][kt] = E::mfma16(f[kt][q4], q[i][q4], st[i][kt]);
      }
    }
    // V^T rows d = 16*dt + l16, keys {4gq..4gq+3, 16+4gq..16+4gq+3}, read
    // while the softmax runs
    V8 vf[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      vf[dt] = ldstr_at<V8>((Vt + tt) ^ (32u * dt), ((Vt + tt) ^ (32u * dt)) + 4096u);
    V8 pb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      if (!(i == 0 ? sa : sb)) continue;
      const int lim = min(nv - 1, g.causal ? u.p0 + jt[i] - ks : 0x7fffffff);
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float v = (16 * kt + 4 * gq + j) <= lim ? st[i][kt][j] : -INFINITY;
          st[i][kt][j] = v;
          mx = vmax(mx, v);
        }
      mx = max_xor16_32(mx) * sl2;
      if (__builtin_amdgcn_ballot_w64(mx > m[i] + kLazy)) {
        const float m_new = fmaxf(m[i], mx);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m[i] - m_new);
        m[i] = m_new;
        lsum[i] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) o[i][dt] *= alpha;
      }
      const float mneg = m[i] == -INFINITY ? 0.f : -m[i];
#pragma unroll
      for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float pv = fast_exp2(__builtin_fmaf(st[i][kt][j], sl2, mneg));
          lsum[i] += pv;
          pb[i][4 * kt + j] = E::from_f32(pv);
        }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      if (sa) o[0][dt] = E::mfma16(vf[dt], pb[0], o[0][dt]);
      if (sb) o[1][dt] = E::mfma16(vf[dt], pb[1], o[1][dt]);
    }
  };

  GrpWin cur, nxt;
  cur.fetch(ent, cnt, 0, lane);
  nxt.fetch(ent, cnt, 1, lane);
  if (nwin > 0) issue(cur, 0, 0);
  for (int w = 0; w < nwin; w++) {
    wait_vm();
    __syncthreads();  // window w landed; window w - 1's buffer is free
    GrpWin nn;
    nn.fetch(ent, cnt, w + 2, lane);
    if (w + 1 < nwin) issue(nxt, w + 1, (w + 1) & 1);
    const int nslot = min(kGrpSlots, cnt - w * kGrpSlots);
    for (int s = 0; s < nslot; s++) {
      const unsigned msk = (unsigned)__builtin_amdgcn_readlane(cur.msk, s);
      const bool sel0 = (msk >> jt[0]) & 1u, sel1 = TPW == 2 && ((msk >> jt[1]) & 1u);
      if (!(sel0 || sel1)) continue;
      const int ks = __builtin_amdgcn_readlane(cur.ks, s);
      const unsigned Kt = tile_addr(w & 1, s, 0);
      const int nv = nvalid_of(msk);
      if (sel0 && sel1) chunk(std::true_type{}, std::true_type{}, Kt, ks, nv);
      else if (sel0) chunk(std::true_type{}, std::false_type{}, Kt, ks, nv);
      else chunk(std::false_type{}, std::true_type{}, Kt, ks, nv);
    }
    cur = nxt;
    nxt = nn;
  }

#pragma unroll
  for (int i = 0; i < TPW; i++) {
    if (!live[i]) continue;
    float lt = lsum[i] + __shfl_xor(lsum[i], 16);
    lt += __shfl_xor(lt, 32);
    if (col_ok) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const long orow = (long)(u.t0 + jt[i]) * p.N1 + u.n2 * G + l16;
      T* op = (T*)p.out + orow * kD;
#pragma unroll
      for (int dt = 0; dt < 8; dt++)
        *reinterpret_cast<uint2*>(op + 16 * dt + 4 * gq) =
            pack4<E>(o[i][dt][0] * inv, o[i][dt][1] * inv, o[i][dt][2] * inv, o[i][dt][3] * inv);
      if (gq == 0) p.lse[orow] = lt > 0.f ? (m[i] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// dQ (+ softmax_grad) over the same token groups and chunk lists:
// S^T = K Q^T and dP^T = V dO^T from the K and V tiles, dS^T = P^T (dP^T -
// softmax_grad), dQ^T += K^T dS^T with K^T read transposed from the K tile.
template <class E, int TPW>
__global__ __launch_bounds__(kNsaGroup / TPW * 64) void nsa_dq_grp_kernel(NsaParams p) {
  constexpr int NW = kNsaGroup / TPW;  // waves
  typedef typename E::T T;
  typedef typename E::V8 V8;
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(1024))) char lds[kGrpLds];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar branches
  const int l16 = lane & 15, gq = lane >> 4;
  const GrpUnit u = grp_unit(p, blockIdx.x);
  const NsaGeom& g = p.g;
  const int G = p.G;
  const bool col_ok = l16 < G;
  const int sbs = g.sbs;
  const float sl2 = p.scale * kLog2e;

  const int jt[2] = {wid, TPW == 2 ? kNsaGroup - 1 - wid : wid};
  bool live[2];
  V8 q[2][4], dov[2][4];
  f32x4_t dq[2][8];
  float lse2[2], dlt[2];
#pragma unroll
  for (int i = 0; i < TPW; i++) {
    live[i] = jt[i] < u.ntok;
    const bool ok = live[i] && col_ok;
    const long qr = (long)(u.t0 + (live[i] ? jt[i] : 0)) * p.N1 + u.n2 * G + (col_ok ? l16 : 0);
    float acc = 0.f;
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const long off = qr * kD + 32 * q4 + 8 * gq;
      q[i][q4] = ok ? as_v8<V8>(ld16((const T*)p.q + off)) : zero_v8<V8>();
      dov[i][q4] = ok ? as_v8<V8>(ld16((const T*)p.dout + off)) : zero_v8<V8>();
      const V8 ov = ok ? as_v8<V8>(ld16((const T*)p.o + off)) : zero_v8<V8>();
#pragma unroll
      for (int e = 0; e < 8; e++) acc += E::to_f32(dov[i][q4][e]) * E::to_f32(ov[e]);
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    dlt[i] = acc;
    lse2[i] = ok ? p.lse[qr] * kLog2e : 0.f;
    if (ok && gq == 0) *reinterpret_cast<float2*>(p.delta + 2 * qr) = make_float2(lse2[i], dlt[i]);
#pragma unroll
    for (int dt = 0; dt < 8; dt++) dq[i][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int cnt = p.grp.cnt[blockIdx.x];
  const int* ent = p.grp.ent + (long)blockIdx.x * p.grp.cap * 2;
  const int nwin = (cnt + kGrpSlots - 1) / kGrpSlots;
  GrpLoader<64 / NW> ld;
  ld.init(p, u, wid);
  const unsigned lds0 = lds_addr(lds);
  const int my_slot = (wid & 7) >> 1;
  auto tile_addr = [&](int buf, int slot, int kv) {
    return lds0 + (unsigned)(((buf * kGrpSlots + slot) * 2 + kv) * kGrpTile);
  };
  auto nvalid_of = [&](unsigned msk) { return (msk & kNsaChunkHalf) ? kChunk / 2 : kChunk; };
  auto issue = [&](const GrpWin& wn, int w, int buf) {
    if (w * kGrpSlots + my_slot < cnt) {
      const int ks = __builtin_amdgcn_readlane(wn.ks, my_slot);
      const unsigned msk = (unsigned)__builtin_amdgcn_readlane(wn.msk, my_slot);
      ld.issue(ks, nvalid_of(msk), tile_addr(buf, my_slot, wid & 1), lane);
    }
  };
  const unsigned rd = grp_row_base(l16, gq), tt = grp_tr_base(l16, gq);

  // One chunk for the tokens the compile-time flags A, B name (see the forward).
  auto chunk = [&](auto A, auto B, unsigned Kt, int ks, int nv) {
    constexpr bool sa = decltype(A)::value, sb = decltype(B)::value;
    const unsigned Vt = Kt + kGrpTile;
    // element j of st[i][kt] / dpt[i][kt]: key ks + 16*kt + 4*gq + j, head l16
    f32x4_t st[2][2], dpt[2][2];
    V8 f[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) f[kt][q4] = lds16_at<V8>(((Kt + rd) ^ (64u * q4)) + 4096u * kt);
#pragma unroll
    for (int i = 0; i < 2; i++) {
      if (!(i == 0 ? sa : sb)) continue;
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        st[i][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) st[i][kt] = E::mfma16(f[kt][q4], q[i][q4], st[i][kt]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) f[kt][q4] = lds16_at<V8>(((Vt + rd) ^ (64u * q4)) + 4096u * kt);
#pragma unroll
    for (int i = 0; i < 2; i++) {
      if (!(i == 0 ? sa : sb)) continue;
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        dpt[i][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) dpt[i][kt] = E::mfma16(f[kt][q4], dov[i][q4], dpt[i][kt]);
      }
    }
    // K^T rows d = 16*dt + l16, keys {4gq..4gq+3, 16+4gq..16+4gq+3}, read
    // while dS is formed
    V8 kf[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      kf[dt] = ldstr_at<V8>((Kt + tt) ^ (32u * dt), ((Kt + tt) ^ (32u * dt)) + 4096u);
    V8 bs[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      if (!(i == 0 ? sa : sb)) continue;
      const int lim = min(nv - 1, g.causal ? u.p0 + jt[i] - ks : 0x7fffffff);
#pragma unroll
      for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const bool ok = col_ok && (16 * kt + 4 * gq + j) <= lim;
          const float pv = ok ? fast_exp2(__builtin_fmaf(st[i][kt][j], sl2, -lse2[i])) : 0.f;
          bs[i][4 * kt + j] = E::from_f32(pv * (dpt[i][kt][j] - dlt[i]));
        }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      if (sa) dq[0][dt] = E::mfma16(kf[dt], bs[0], dq[0][dt]);
      if (sb) dq[1][dt] = E::mfma16(kf[dt], bs[1], dq[1][dt]);
    }
  };

  GrpWin cur, nxt;
  cur.fetch(ent, cnt, 0, lane);
  nxt.fetch(ent, cnt, 1, lane);
  if (nwin > 0) issue(cur, 0, 0);
  for (int w = 0; w < nwin; w++) {
    wait_vm();
    __syncthreads();
    GrpWin nn;
    nn.fetch(ent, cnt, w + 2, lane);
    if (w + 1 < nwin) issue(nxt, w + 1, (w + 1) & 1);
    const int nslot = min(kGrpSlots, cnt - w * kGrpSlots);
    for (int s = 0; s < nslot; s++) {
      const unsigned msk = (unsigned)__builtin_amdgcn_readlane(cur.msk, s);
      const bool sel0 = (msk >> jt[0]) & 1u, sel1 = TPW == 2 && ((msk >> jt[1]) & 1u);
      if (!(sel0 || sel1)) continue;
      const int ks = __builtin_amdgcn_readlane(cur.ks, s);
      const unsigned Kt = tile_addr(w & 1, s, 0);
      const int nv = nvalid_of(msk);
      if (sel0 && sel1) chunk(std::true_type{}, std::true_type{}, Kt, ks, nv);
      else if (sel0) chunk(std::true_type{}, std::false_type{}, Kt, ks, nv);
      else chunk(std::false_type{}, std::true_type{}, Kt, ks, nv);
    }
    cur = nxt;
    nxt = nn;
  }

#pragma unroll
  for (int i = 0; i < TPW; i++) {
    if (!live[i] || !col_ok) continue;
    const long qr = (long)(u.t0 + jt[i]) * p.N1 + u.n2 * G + l16;
    T* dp = (T*)p.out + qr * kD;
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      *reinterpret_cast<uint2*>(dp + 16 * dt + 4 * gq) =
          pack4<E>(dq[i][dt][0] * p.scale, dq[i][dt][1] * p.scale, dq[i][dt][2] * p.scale,
                   dq[i][dt][3] * p.scale);
  }
}

// ---------------------------------------------------------------------------
// dK / dV.  The tokens that selected a (KV head, block) -- its reverse list --
// are cut into segments of at most kSegEntries listings, so a block that
// thousands of tokens selected is shared by many workgroups.  Workgroups
// take segments in list order from a counter.  A workgroup walks its
// segment's tokens in chunks of 32 query rows (32 / G tokens x G heads);
// each wave owns 32 of the block's keys:
//   S = Q K^T, dP = dO V^T, P = exp2(S*scale*log2e - LSE2),
//   dS = P (dP - softmax_grad), dV^T += dO^T P, dK^T += Q^T dS,
// and writes fp32 partial dK/dV of its segment into the segment's slot.  A
// reduction kernel then sums each block's segments in segment order: no
// atomics on the data, a fixed summation order, bit-identical reruns
// whichever workgroup ran which segment.
// ---------------------------------------------------------------------------
constexpr int kSegEntries = kNsaSegEntries;

// Workgroups of the dK/dV partial kernel: about three resident per CU on
// 256 CUs, never more than the segments.
int nsa_dkdv_grid(const NsaParams& p) {
  return std::min(kNsaDkdvMaxGrid, std::max(1, p.max_segments));
}

// every list with listings has at most len / kSegEntries + 1 segments
int nsa_max_segments(long total_entries, long nblocks) {
  return (int)(nblocks + (total_entries + kSegEntries - 1) / kSegEntries);
}

// Segments per list; also clears the dK/dV kernel's work counter.
__global__ void nsa_seg_count(const int* rev_ptr, int nblocks, int* seg_cnt, int* ctr) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r == 0) ctr[0] = 0;
  if (r >= nblocks) return;
  const int len = rev_ptr[r + 1] - rev_ptr[r];
  seg_cnt[r] = (len + kSegEntries - 1) / kSegEntries;
}

// DQK: query/key head dim (128 or 192); a 192-dim K or Q row is staged as
// two padded tiles of 128 dims each (bytes 0..255 and 128..383 of the row),
// as in the forward.  The 192 variant runs one wave per SIMD (its dK
// accumulators take 32 more registers).
//
// Q, dO and K sit in padded LDS tiles (272-byte rows, see PStage), so every
// operand read is a base register plus a constant.  A chunk's 32 rows are
// gathered rows -- row k is head k % G of the chunk's token k / G -- so each
// lane keeps, for each 1-KB slice it loads, the row's (token slot, head) and
// its 16-byte piece, fixed for the whole kernel; per chunk a load is then
// the token id (from LDS) times the row stride plus those constants, added
// as a 32-bit offset to a scalar base.
template <class E, int NW, int DQK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DQK == 128 ? 2 : 1)))
void nsa_dkdv_seg_kernel(NsaParams p) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int kQC = 32;                  // query rows per chunk
  constexpr int kQTile = ptile_bytes(kQC);
  constexpr int NK = NW * 32;              // keys per workgroup (the block)
  constexpr int NKT = DQK == 128 ? 1 : 2;  // padded tiles per K / Q row
  typedef PStage<NW, kQC> QStage;
  constexpr int NU = QStage::NU;
  __shared__ __attribute__((aligned(1024))) char lds_k[NKT][ptile_bytes(NK)];
  __shared__ __attribute__((aligned(1024))) char lds_q[2][NKT][kQTile];
  __shared__ __attribute__((aligned(1024))) char lds_do[2][kQTile];
  // per chunk row r: (LSE * log2 e, softmax_grad) at [2r], [2r + 1], loaded
  // by one direct load of 64 lanes; the row's token position, or -1 for a
  // padding row (always masked)
  __shared__ float lds_ld[2][64];
  __shared__ int lds_pos[2][kQC];
  __shared__ int lds_tok[kSegEntries];  // the segment's token ids

  const NsaGeom& g = p.g;
  // the next segment from the counter, or -1 when all are taken
  __shared__ int s_next;
  const int nblocks = p.N2 * g.NB, nseg = min(p.seg_off[nblocks], p.max_segments);
  auto next_segment = [&]() -> int {
    if (threadIdx.x == 0) s_next = atomicAdd(p.seg_ctr, 1);
    __syncthreads();
    const int k = s_next;
    __syncthreads();
    return k < nseg ? k : -1;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);  // wave-uniform
  const int l32 = lane & 31, h = lane >> 5;
  const int G = p.G;
  const int tpc = max(1, kQC / G);  // tokens per chunk (G <= 32)
  const int sbs = g.sbs;
  const float sl2 = p.scale * kLog2e;
  // byte strides of a (token, head) row of Q and dO: row t * N1 + n1 of
  // T * N1 rows, each offset below 2^32 (T * N1 * D fits 31 bits)
  constexpr unsigned qstride = DQK * 2, dstride = kDv * 2;

  // This lane's rows of the chunk tiles, fixed for the kernel and packed in
  // one register each: for slice u * NW + wid, bits 0-5 hold the row's token
  // slot + 1 (0: a row past the chunk's tpc * G), bits 8-12 its head, bits
  // 16-19 its 16-byte piece; the same for the LSE / softmax_grad load (wave
  // 0), row lane / 2.
  auto rowcode = [&](int k, int pc) {
    const bool row_ok = k < tpc * G;
    return (row_ok ? k / G + 1 : 0) | ((row_ok ? k % G : G - 1) << 8) | (pc << 16);
  };
  int rcode[NU];
#pragma unroll
  for (int u = 0; u < NU; u++) {
    int k, pc;
    pslot(1024 * (u * NW + wid) + 16 * lane, kQC, k, pc);
    rcode[u] = rowcode(k, pc);
  }
  const int lcode = rowcode(lane >> 1, 0);

  // Per-lane bases of the operand reads: Q and dO rows l32, the wave's K
  // rows 32*wid + l32 (pieces 2*ds + h at +32*ds); dO^T and Q^T by transpose
  // reads.
  const unsigned rb = prow_base(lane), tb = ptr_base(lane);
  const unsigned lq0 = lds_addr(&lds_q[0][0][0]), ld0 = lds_addr(&lds_do[0][0]);

  for (int sg = next_segment(); sg >= 0; sg = next_segment()) {
    // segment -> list (largest r with seg_off[r] <= sg) and its listings
    int r = 0;
    {
      int hi = nblocks - 1;
      while (r < hi) {
        const int mid = (r + hi + 1) >> 1;
        if (p.seg_off[mid] <= sg) r = mid; else hi = mid - 1;
      }
    }
    const int e0 = p.rev_ptr[r] + (sg - p.seg_off[r]) * kSegEntries;
    const int e1 = min(e0 + kSegEntries, p.rev_ptr[r + 1]);
    const int n2 = r / g.NB, gb = r % g.NB;
    const int b = seq_of_dev(g.blk_off, g.B, gb);
    const int blk = gb - g.blk_off[b];
    const int kv0 = g.cu_kv[b], q0 = g.cu_q[b];
    const int skv = g.cu_kv[b + 1] - kv0;
    const int key_lo = blk * sbs;
    const int key_hi = min((blk + 1) * sbs, skv);
    const int wkey0 = key_lo + wid * 32;
    const int n2G = n2 * G;

    // K rows of the block into padded tiles (rows past key_hi re-read the
    // last key); V rows of this wave's keys as the B operand of dP in
    // registers
    {
      const char* krow0 = (const char*)((const T*)p.k + ((long)(kv0 + key_lo) * p.N2 + n2) * DQK);
      PStage<NW, NK> kst;
      int ln = lane;
      asm volatile("" : "+v"(ln));  // slice offsets formed per segment, not kept
#pragma unroll
      for (int kt = 0; kt < NKT; kt++)
        kst.ragged(krow0 + 128 * kt, (long)p.N2 * DQK * 2, key_hi - 1 - key_lo,
                   lds_addr(lds_k[kt]), wid, ln);
    }
    V8 vreg[kDv / 16];
    {
      const int mykey = wkey0 + l32;
      const long vrow = ((long)(kv0 + min(mykey, key_hi - 1)) * p.N2 + n2) * kDv;
#pragma unroll
      for (int ds = 0; ds < kDv / 16; ds++)
        vreg[ds] = mykey < key_hi ? as_v8<V8>(ld16((const T*)p.v + vrow + ds * 16 + 8 * h))
                                  : zero_v8<V8>();
    }
    const int nchunks = (e1 - e0 + tpc - 1) / tpc;
    // the segment's token ids into LDS once, so chunk addresses need no
    // dependent global load
    for (int x = tid; x < e1 - e0; x += NW * 64) lds_tok[x] = p.rev[e0 + x];
    __syncthreads();

    // Chunk c: entries c*tpc .. of the segment; rows of tokens past its nt
    // re-read its last token's last head and are masked by position -1.
    auto load_chunk = [&](int c, int buf) {
      const int nt = min(tpc, e1 - e0 - c * tpc);
      const int* tk = lds_tok + c * tpc;
      const unsigned lq = lq0 + buf * (NKT * kQTile), ld = ld0 + buf * kQTile;
      // row of a code: its token (the chunk's last for a row past nt) and
      // head (the last for such a row).  The code passes through an empty
      // asm so that its fields are unpacked here, per chunk, rather than
      // hoisted out of the loop into registers of their own.
      auto row_of = [&](int code, int& t) {
        asm volatile("" : "+v"(code));
        const int tq1 = code & 63;
        const bool ok = tq1 > 0 && tq1 <= nt;
        t = tk[ok ? tq1 - 1 : nt - 1];
        return (unsigned)(t * p.N1 + n2G) + (unsigned)(ok ? (code >> 8) & 31 : G - 1);
      };
#pragma unroll
      for (int u = 0; u < NU; u++) {
        const int sl = u * NW + wid;
        if (sl < QStage::S && (QStage::kTail == 64 || sl < QStage::S - 1 || lane < QStage::kTail)) {
          int t, code = rcode[u];
          const unsigned row = row_of(code, t);
          asm volatile("" : "+v"(code));
          const unsigned pcb = (unsigned)(code >> 12) & 0xf0u;
#pragma unroll
          for (int kt = 0; kt < NKT; kt++)
            g2lds16_so_at(p.q, row * qstride + 128 * kt + pcb, lq + kt * kQTile + 1024 * sl);
          g2lds16_so_at(p.dout, row * dstride + pcb, ld + 1024 * sl);
        }
      }
      if (wid == 0) {
        int t, code = lcode;
        const unsigned row = row_of(code, t);
        asm volatile("" : "+v"(code));
        const int tq1 = code & 63;
        g2lds4_so_at(p.delta, (2 * row + (lane & 1)) * 4, lds_addr(lds_ld[buf]));
        int ln = lane;
        asm volatile("" : "+v"(ln));  // the address is formed here, not kept
        if (!(ln & 1)) lds_pos[buf][ln >> 1] = tq1 > 0 && tq1 <= nt ? t - q0 : -1;
      }
    };

    f32x16 dvt[kDv / 32], dkt[DQK / 32];
#pragma unroll
    for (int dt = 0; dt < kDv / 32; dt++)
#pragma unroll
      for (int jj = 0; jj < 16; jj++) dvt[dt][jj] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DQK / 32; dt++)
#pragma unroll
      for (int jj = 0; jj < 16; jj++) dkt[dt][jj] = 0.f;

    const char* Kr = lds_k[0] + wid * 32 * kPadPitch + rb;
    const char* Kr2 = lds_k[NKT - 1] + wid * 32 * kPadPitch + rb;  // dims 64..191 (DQK = 192)
    const int mykey = wkey0 + l32;
    const int need = g.causal ? mykey : 0;
    const bool key_ok = mykey < key_hi;

    if (nchunks > 0) load_chunk(0, 0);
    wait_vm();
    // the V rows are taken as landed here: otherwise the compiler waits for
    // them inside the loop, which also waits for the next chunk's loads
#pragma unroll
    for (int ds = 0; ds < kDv / 16; ds++) asm volatile("" : "+v"(vreg[ds]));
    __syncthreads();
    int buf = 0;
    for (int c = 0; c < nchunks; c++) {
      if (c + 1 < nchunks) load_chunk(c + 1, buf ^ 1);
      const char* Qr = &lds_q[buf][0][0] + rb;
      const char* Qr2 = &lds_q[buf][NKT - 1][0] + rb;
      const char* Dr = &lds_do[buf][0] + rb;
      const char* Qt = &lds_q[buf][0][0] + tb;
      const char* Qt2 = &lds_q[buf][NKT - 1][0] + tb;
      const char* Dt = &lds_do[buf][0] + tb;
      // S = Q K^T and dP = dO V^T: 32 rows x this wave's 32 keys
      f32x16 sc, dp;
#pragma unroll
      for (int jj = 0; jj < 16; jj++) sc[jj] = dp[jj] = 0.f;
#pragma unroll
      for (int ds = 0; ds < 8; ds++) {
        sc = E::mfma32(lds_read16<V8>(Qr + 32 * ds), lds_read16<V8>(Kr + 32 * ds), sc);
        dp = E::mfma32(lds_read16<V8>(Dr + 32 * ds), vreg[ds], dp);
      }
#pragma unroll
      for (int ds = 8; ds < DQK / 16; ds++)
        sc = E::mfma32(lds_read16<V8>(Qr2 + 32 * (ds - 4)), lds_read16<V8>(Kr2 + 32 * (ds - 4)),
                       sc);
      if constexpr (DQK == 128) {
        // three LDS reads feed two MFMAs per step
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int u = 0; u < 8; u++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
      }
      // element jj of a lane is row 8*(jj/4) + 4*h + jj%4 of the chunk, column key l32
      V8 bp[2], bd[2];
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const int rbase = 8 * j4 + 4 * h;
        const float4 a4 = *reinterpret_cast<const float4*>(&lds_ld[buf][2 * rbase]);
        const float4 b4 = *reinterpret_cast<const float4*>(&lds_ld[buf][2 * rbase + 4]);
        const int4 ps4 = *reinterpret_cast<const int4*>(&lds_pos[buf][rbase]);
        const float lv[4] = {a4.x, a4.z, b4.x, b4.z};
        const float dv[4] = {a4.y, a4.w, b4.y, b4.w};
        const int pv4[4] = {ps4.x, ps4.y, ps4.z, ps4.w};
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int e = 4 * j4 + jj;
          // a valid row (pos >= 0) at or after this key (causal) keeps it
          const bool ok = key_ok && pv4[jj] >= need;
          float pr = fast_exp2(__builtin_fmaf(sc[e], sl2, -lv[jj]));
          pr = ok ? pr : 0.f;
          bp[e >> 3][e & 7] = E::from_f32(pr);
          bd[e >> 3][e & 7] = E::from_f32(pr * (dp[e] - dv[jj]));
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS  (16 rows per step)
#pragma unroll
      for (int k2 = 0; k2 < 2; k2++) {
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
          dvt[dt] = E::mfma32(ptile_tr<V8>(Dt + k2 * 16 * kPadPitch + 64 * dt), bp[k2], dvt[dt]);
          dkt[dt] = E::mfma32(ptile_tr<V8>(Qt + k2 * 16 * kPadPitch + 64 * dt), bd[k2], dkt[dt]);
        }
#pragma unroll
        for (int dt = 4; dt < DQK / 32; dt++)
          dkt[dt] = E::mfma32(ptile_tr<V8>(Qt2 + k2 * 16 * kPadPitch + 64 * (dt - 2)), bd[k2],
                              dkt[dt]);
      }
      // a transposed dO^T / Q^T pair per MFMA, four reads ahead
      if constexpr (DQK == 128) sched_mfma_lds<16, 2, 4>();
      wait_vm();
      __syncthreads();
      buf ^= 1;
    }

    // fp32 partials of this segment: [segment][dK: key][DQK], then [dV: key][kDv]
    if (key_ok) {
      float* sb = p.part + (long)sg * sbs * (DQK + kDv);
      float* pk = sb + (long)(mykey - key_lo) * DQK;
      float* pv = sb + (long)sbs * DQK + (long)(mykey - key_lo) * kDv;
#pragma unroll
      for (int dt = 0; dt < DQK / 32; dt++)
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int d0 = dt * 32 + 8 * jj + 4 * h;
          *reinterpret_cast<float4*>(pk + d0) =
              make_float4(dkt[dt][4 * jj], dkt[dt][4 * jj + 1], dkt[dt][4 * jj + 2], dkt[dt][4 * jj + 3]);
        }
#pragma unroll
      for (int dt = 0; dt < kDv / 32; dt++)
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int d0 = dt * 32 + 8 * jj + 4 * h;
          *reinterpret_cast<float4*>(pv + d0) =
              make_float4(dvt[dt][4 * jj], dvt[dt][4 * jj + 1], dvt[dt][4 * jj + 2], dvt[dt][4 * jj + 3]);
        }
    }
    __syncthreads();  // the next segment reuses the LDS buffers
  }
}

// dK = scale * sum of a block's segment partials, dV = their sum, in segment
// order; one thread per (block, key, 4 columns).
template <class E, int DQK>
__global__ __launch_bounds__(256) void nsa_dkdv_reduce(NsaParams p, const int* seg_off,
                                                       int nblocks, const float* part) {
  const NsaGeom& g = p.g;
  const int sbs = g.sbs;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  // one thread per (block, key, 4 columns of dK and the same 4 of dV; the
  // threads of columns DQK-kDv.. handle dK only)
  constexpr int C4 = DQK / 4;
  const long per_block = (long)sbs * C4;
  if (i >= (long)nblocks * per_block) return;
  const int r = (int)(i / per_block);
  const int key = (int)(i % per_block) / C4;
  const int d0 = 4 * ((int)(i % per_block) % C4);
  const int n2 = r / g.NB, gb = r % g.NB;
  const int b = seq_of_dev(g.blk_off, g.B, gb);
  const int blk = gb - g.blk_off[b];
  const int kv0 = g.cu_kv[b];
  const int skv = g.cu_kv[b + 1] - kv0;
  const int kpos = blk * sbs + key;
  if (kpos >= skv) return;
  const bool has_v = d0 < kDv;
  float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), av = ak;
  for (int sg = seg_off[r]; sg < seg_off[r + 1]; sg++) {
    const float* sb = part + (long)sg * sbs * (DQK + kDv);
    const float4 x = *reinterpret_cast<const float4*>(sb + (long)key * DQK + d0);
    ak.x += x.x; ak.y += x.y; ak.z += x.z; ak.w += x.w;
    if (has_v) {
      const float4 y = *reinterpret_cast<const float4*>(sb + (long)sbs * DQK + (long)key * kDv + d0);
      av.x += y.x; av.y += y.y; av.z += y.z; av.w += y.w;
    }
  }
  const long krow = (long)(kv0 + kpos) * p.N2 + n2;
  typedef typename E::T T;
  *reinterpret_cast<uint2*>((T*)p.dk + krow * DQK + d0) =
      pack4<E>(ak.x * p.scale, ak.y * p.scale, ak.z * p.scale, ak.w * p.scale);
  if (has_v) *reinterpret_cast<uint2*>((T*)p.dv + krow * kDv + d0) = pack4<E>(av.x, av.y, av.z, av.w);
}

template <class E>
static hipError_t fwd_t(const NsaParams& p, hipStream_t st) {
  const int units = p.T * p.N2;
  const int n_items = (units + 3) / 4;
  if (n_items == 0) return hipSuccess;
  // 192-dim query/key heads: the 32-column kernel for every group size
  if (p.D == 192)
    hipLaunchKernelGGL((nsa_fwd_kernel<E, 192>), dim3(8 * ((n_items + 7) / 8)), dim3(256), 0, st,
                       p, n_items);
  else if (p.G <= 16 && p.grp.NG > 0)
    hipLaunchKernelGGL((nsa_fwd_grp_kernel<E, kGrpTPW>), dim3(p.N2 * p.grp.NG),
                       dim3(kNsaGroup / kGrpTPW * 64), 0, st, p);
  else
    hipLaunchKernelGGL((nsa_fwd_kernel<E, 128>), dim3(8 * ((n_items + 7) / 8)), dim3(256), 0, st,
                       p, n_items);
  return hipGetLastError();
}

hipError_t launch_nsa_fwd(const NsaParams& p, int fp16, hipStream_t st) {
  return fp16 ? fwd_t<FP16>(p, st) : fwd_t<BF16>(p, st);
}

template <class E, int DQK>
static hipError_t dkdv_launch(const NsaParams& p, int nw, int grid, hipStream_t st) {
  if (nw <= 1)
    hipLaunchKernelGGL((nsa_dkdv_seg_kernel<E, 1, DQK>), dim3(grid), dim3(64), 0, st, p);
  else if (nw <= 2)
    hipLaunchKernelGGL((nsa_dkdv_seg_kernel<E, 2, DQK>), dim3(grid), dim3(128), 0, st, p);
  else
    hipLaunchKernelGGL((nsa_dkdv_seg_kernel<E, 4, DQK>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class E>
static hipError_t bwd_t(const NsaParams& p, hipStream_t st, void* const* ev, int n_ev) {
  hipError_t e = mark_event(ev, n_ev, 1, 0, st);
  const int units = p.T * p.N2;
  const int n_items = (units + 3) / 4;
  if (e == hipSuccess && n_items > 0) {
    if (p.D == 192)
      hipLaunchKernelGGL((nsa_dq_kernel<E, 192>), dim3(8 * ((n_items + 7) / 8)), dim3(256), 0, st,
                         p, n_items);
    else if (p.G <= 16 && p.grp.NG > 0)
      hipLaunchKernelGGL((nsa_dq_grp_kernel<E, kGrpTPW>), dim3(p.N2 * p.grp.NG),
                         dim3(kNsaGroup / kGrpTPW * 64), 0, st, p);
    else
      hipLaunchKernelGGL((nsa_dq_kernel<E, 128>), dim3(8 * ((n_items + 7) / 8)), dim3(256), 0, st,
                         p, n_items);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 0, st);
  const int nb = p.N2 * p.g.NB;
  if (e == hipSuccess && nb > 0) {
    // segments per list, then their exclusive scan (total at the end)
    hipLaunchKernelGGL(nsa_seg_count, dim3((nb + 255) / 256), dim3(256), 0, st, p.rev_ptr, nb,
                       p.seg_off, p.seg_ctr);
    e = hipGetLastError();
    if (e == hipSuccess) e = exclusive_scan_total(p.seg_off, nb, p.seg_sums, st);
  }
  if (e == hipSuccess && nb > 0) {
    const int nw = (p.g.sbs + 31) / 32;  // 1..4 waves, 32 keys each
    const int grid = nsa_dkdv_grid(p);
    if (p.D == 192)
      e = dkdv_launch<E, 192>(p, nw, grid, st);
    else
      e = dkdv_launch<E, 128>(p, nw, grid, st);
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 3, 0, st);
  if (e == hipSuccess && nb > 0) {
    const long n = (long)nb * p.g.sbs * (p.D / 4);
    if (p.D == 192)
      hipLaunchKernelGGL((nsa_dkdv_reduce<E, 192>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                         0, st, p, p.seg_off, nb, (const float*)p.part);
    else
      hipLaunchKernelGGL((nsa_dkdv_reduce<E, 128>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                         0, st, p, p.seg_off, nb, (const float*)p.part);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 3, 1, st);
  return e;
}

hipError_t launch_nsa_bwd(const NsaParams& p, int fp16, hipStream_t st, void* const* ev, int n_ev) {
  return fp16 ? bwd_t<FP16>(p, st, ev, n_ev) : bwd_t<BF16>(p, st, ev, n_ev);
}

}  // namespace tsa
