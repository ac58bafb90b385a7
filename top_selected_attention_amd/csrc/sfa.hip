// Sparse flash attention over a paged, shared KV cache (decode).
//
// "aclnnSparseFlashAttention", formulas section: softmax(Q K~^T / sqrt(d_k)) V~
// with K~/V~ the selected keys/values; a score is
// scale * (q . k + q_rope . k_rope) (d_k counts the 512-wide head and the
// 64-wide rope part); constraints section: D = 512, Dr = 64.
// "SparseAttnSharedkvMetadata", parameter list: one KV head, PA_ND paged KV,
// seqused_kv (kv_lens), rightDownCausal mask mode 3 (decode token s of Sq at
// position kv_len - Sq + s); and its task list of per-core (batch, head,
// Q block, K block) ranges, which here is the split-KV work decomposition.
//
// Shared KV: the value row is the key row (value_cache aliases key_cache),
// so one gathered 1 KB row feeds both the scores and P V.  A separate value
// cache takes sfa_split_sepv_kernel, which gathers the value rows too.
//
// Split kernel: one workgroup per (decode token, split of its selected keys,
// group of 64 query heads); 8 waves = 2 groups of 32 heads x 4 quarters of
// the 512 output columns.  Selected rows are gathered 32
// at a time by direct global -> LDS loads (a 1 KB key row per instruction,
// plus its 128-byte rope row) into a three-stage ring.  On 16x16x32 MFMA, per
// wave: a partial S^T (32 keys x 32 heads) = K Q^T over its quarter of the
// 576 dims (Q^T slice held in registers), the partials of a head group summed
// through LDS, online softmax along the keys (lanes own heads), and
// O^T (128 x 32) += V^T P^T with V^T read from the same key tile by LDS
// transpose reads.  With one split the kernel writes the output; otherwise it
// writes normalised fp32 partials and their base-2 LSE, and the combine kernel
// merges them: LSE = logsumexp_s LSE_s, O = sum_s exp(LSE_s - LSE) O_s.
// The work is bound by the gather from HBM (about 114 FLOP per gathered byte
// at 64 heads, below the bf16 ridge).
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {

namespace {
constexpr int kDv = 512;          // value / key head dim
constexpr int kDr = 64;           // rope dim
constexpr int kKeys = 32;         // keys per chunk
constexpr int kMainB = kKeys * kDv * 2;   // 32 KB
constexpr int kRopeB = kKeys * kDr * 2;   // 4 KB
constexpr int kTab = 2048;                // slots resolved into LDS at a time

// 1 KB rows (64 16-byte pieces): piece c of row r at c ^ swz1k(r).  16 rows
// reading one piece hit 16 distinct bank groups, and transpose reads of 8
// rows x 2 adjacent pieces hit 16 distinct bank groups.
__device__ __forceinline__ int swz1k(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// 128-byte rope rows (8 pieces): 16 consecutive rows reading one piece hit
// distinct bank groups.
__device__ __forceinline__ int swzr(int r) { return (r >> 1) & 7; }

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Batch entry b, index s within it and query count sq of decode token tk:
// BSND has Sq tokens per entry; TND entry b holds rows cu_q[b] .. cu_q[b+1]-1
// (the largest b with cu_q[b] <= tk, which skips empty entries).
__device__ __forceinline__ void sfa_token(const SfaParams& p, int tk, int& b, int& s, int& sq) {
  if (!p.cu_q) {
    b = tk / p.Sq;
    s = tk - b * p.Sq;
    sq = p.Sq;
    return;
  }
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu_q[mid] <= tk) lo = mid; else hi = mid - 1;
  }
  b = lo;
  s = tk - p.cu_q[b];
  sq = p.cu_q[b + 1] - p.cu_q[b];
}
}  // namespace

template <class E>
__global__ __launch_bounds__(512) void sfa_split_kernel(SfaParams p, int n_items, int hgroups,
                                                        int per_split) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int NS = 3;  // gather ring: chunks c+1, c+2 in flight while c computes
  __shared__ __attribute__((aligned(1024))) char lds_main[NS][kMainB];
  __shared__ __attribute__((aligned(1024))) char lds_rope[NS][kRopeB];
  __shared__ __attribute__((aligned(16))) char lds_xs[8 * 4 * 64 * 16];  // partial score tiles
  __shared__ __attribute__((aligned(16))) int lds_tab[kTab];
  __shared__ unsigned lds_cmask[kTab / kKeys];

  const int item = xcd_remap(blockIdx.x, n_items);
  if (item < 0) return;
  // item order: token-major so a token's splits / head groups share L2
  const int hg = item % hgroups;
  const int sp = (item / hgroups) % p.splits;
  const int tk = item / (hgroups * p.splits);
  int b, s, sq;
  if (p.task) {
    const int4 ti = *reinterpret_cast<const int4*>(p.task + 4 * (long)tk);
    b = ti.x;
    s = ti.y;
    sq = ti.z;
  } else {
    sfa_token(p, tk, b, s, sq);
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  // wave = (32-head group h2, quarter qd): the quarter selects 128 of the 512
  // output columns and a quarter of the 576-dim score contraction (main dims
  // 128*qd .. +127, and rope dims 32*qd .. +31 for qd < 2); the four waves of
  // a head group sum their partial scores in the same fixed order, so all
  // four hold identical scores and softmax state.
  const int h2 = wid & 1, qd = wid >> 1;

  const int kv_len = p.kv_lens[b];
  const int qpos = kv_len - sq + s;
  const int total = sfa_total_slots(p);
  int slot_lo = sp * per_split;
  int slot_hi = min(slot_lo + per_split, total);
  if (p.task) {
    const int* rg = p.task + 4 * p.ntok + 2 * ((long)tk * p.splits + sp);
    slot_lo = rg[0];
    slot_hi = rg[1];
  }
  // the top-k slots' cache, length and causal bound: the compressed cache in
  // the shared-KV decode, else the one cache
  const bool skv = p.ckc != nullptr;
  const int t_len = skv ? kv_len / p.cmp_ratio : kv_len;
  const int t_qpos = skv ? t_len - sq + s : qpos;
  const int t_page = skv ? p.c_page : p.page;
  const int t_maxp = skv ? p.c_max_pages : p.max_pages;
  const int t_nump = skv ? p.c_num_pages : p.num_pages;
  const int* t_btab = skv ? p.cbt + (long)b * p.c_max_pages : p.block_table + (long)b * p.max_pages;

  const int hbase = hg * 64 + h2 * 32;  // heads hbase + 16*hh + l16, hh = 0, 1
  const int* topk = p.topk + (long)tk * p.topk_n;  // N2 = 1
  const int* btab = p.block_table + (long)b * p.max_pages;
  const float sl2 = p.scale * kLog2e;

  // Q^T slices as B operands: lane (g, head) holds dims 32*ks + 8*g .. +7
  V8 qm[2][4], qrp[2];
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    const int head = hbase + 16 * hh + l16;
    const bool ok = head < p.N1;
    const T* qr = (const T*)p.q + ((long)tk * p.N1 + (ok ? head : 0)) * kDv + 128 * qd;
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
      qm[hh][ks] = ok ? as_v8<V8>(ld16(qr + 32 * ks + 8 * g)) : zero_v8<V8>();
    const T* qrr = (const T*)p.q_rope + ((long)tk * p.N1 + (ok ? head : 0)) * kDr + 32 * (qd & 1);
    qrp[hh] = ok && qd < 2 ? as_v8<V8>(ld16(qrr + 8 * g)) : zero_v8<V8>();
  }

  // Physical cache rows of a run of up to kTab slots, resolved once into LDS
  // (slot -> selected block id -> position -> page -> row), with one
  // validity mask per 32-slot chunk (bit r = key r kept), so the gather loop
  // never waits on index or page-table loads.  A dropped slot holds its
  // chunk's first kept row (finite data, P = 0), or row 0 in a chunk with
  // none (never read: such chunks are skipped).
  auto fill_table = [&](int seg_lo, int seg_n) {
    constexpr int R = kTab / 512;
    int id[R];
    bool band[R];
#pragma unroll
    for (int i = 0; i < R; i++) {
      const int t = tid + 512 * i;
      const int gs = seg_lo + t;  // slot of the token
      band[i] = gs < p.win_pad;
      id[i] = t >= seg_n ? -1 : (band[i] ? 0 : topk[(gs - p.win_pad) / p.sbs]);
    }
    int lp[R], pos[R], pg[R];
    bool ok[R];
#pragma unroll
    for (int i = 0; i < R; i++) {
      const int t = tid + 512 * i;
      const int gs = seg_lo + t;
      if (band[i]) {
        pos[i] = qpos - p.win_left + gs;
        ok[i] = t < seg_n && gs < p.win_len && pos[i] >= 0 && pos[i] < kv_len;
        pg[i] = p.page;
        lp[i] = ok[i] ? min(pos[i] / p.page, p.max_pages - 1) : 0;
      } else {
        // the id is range-checked before it is scaled, so a huge id cannot
        // wrap into a small position
        const bool idok = id[i] >= 0 && id[i] <= (t_len - 1) / p.sbs;
        pos[i] = idok ? id[i] * p.sbs + (gs - p.win_pad) % p.sbs : 0;
        ok[i] = t < seg_n && idok && pos[i] < t_len && (!p.causal || pos[i] <= t_qpos);
        pg[i] = t_page;
        lp[i] = ok[i] ? min(pos[i] / t_page, t_maxp - 1) : 0;
      }
    }
    int phys[R];
#pragma unroll
    for (int i = 0; i < R; i++) phys[i] = ok[i] ? (band[i] ? btab[lp[i]] : t_btab[lp[i]]) : 0;
#pragma unroll
    for (int i = 0; i < R; i++) {
      const int t = tid + 512 * i;  // lanes 0..31 and 32..63 each cover one chunk
      const int np = band[i] ? p.num_pages : t_nump;
      const int row = ok[i] ? min(max(phys[i], 0), np - 1) * pg[i] + pos[i] % pg[i] : 0;
      const unsigned long long bal = __ballot(ok[i]);
      const unsigned half = lane < 32 ? (unsigned)bal : (unsigned)(bal >> 32);
      const int first = (half ? __builtin_ctz(half) : 0) + (lane & 32);
      const int frow = __shfl(row, first);
      lds_tab[t] = ok[i] ? row : (half ? frow : 0);
      if ((lane & 31) == 0) lds_cmask[t >> 5] = half;
    }
  };
  // 8 waves x 4 one-KB key rows, and waves 0..3 one 1-KB slice of 8 rope rows;
  // a chunk past the band reads the top-k slots' cache
  int seg_base = 0;  // first slot of the segment being gathered
  auto load_chunk = [&](int c, int buf) {
    const bool tk_cache = skv && seg_base + c * kKeys >= p.win_pad;
    const char* kc = (const char*)(tk_cache ? p.ckc : p.kc);
    const char* krc = (const char*)(tk_cache ? p.ckrc : p.krc);
    const int* tb = lds_tab + c * kKeys;
    const int4 rm = *reinterpret_cast<const int4*>(tb + wid * 4);  // same for all lanes
    const int rms[4] = {rm.x, rm.y, rm.z, rm.w};
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int r = wid * 4 + u;
      g2lds16(kc + (long)rms[u] * (kDv * 2) + ((lane ^ swz1k(r)) << 4), lds_main[buf] + r * 1024);
    }
    if (wid < 4) {
      const int r = wid * 8 + (lane >> 3);
      g2lds16(krc + (long)tb[r] * (kDr * 2) + (((lane & 7) ^ swzr(r)) << 4),
                    lds_rope[buf] + wid * 1024);
    }
  };
  // wait until only the newest NS - 2 chunks' loads (4 key rows, plus a rope
  // slice for waves 0..3, per chunk) are in flight
  auto wait_keep_newest = [&]() {
    if (wid < 4) wait_vm_le<5 * (NS - 2)>(); else wait_vm_le<4 * (NS - 2)>();
  };

  constexpr float kLazy = 8.f;
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  f32x4_t o[8][2];  // O^T tiles: rows d = 128*qd + 16*dt + 4*g + j, column head 16*hh + l16
#pragma unroll
  for (int dt = 0; dt < 8; dt++)
#pragma unroll
    for (int hh = 0; hh < 2; hh++) o[dt][hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int seg_lo = slot_lo; seg_lo < slot_hi; seg_lo += kTab) {
    const int seg_n = min(kTab, slot_hi - seg_lo);
    const int nchunks = (seg_n + kKeys - 1) / kKeys;
    __syncthreads();  // the previous segment's table and tiles are no longer read
    seg_base = seg_lo;
    fill_table(seg_lo, seg_n);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NS - 1; c++)
      if (c < nchunks) load_chunk(c, c);
    if (nchunks >= NS - 1) wait_keep_newest(); else wait_vm();
    __syncthreads();
    int buf = 0;
    for (int c = 0; c < nchunks; c++) {
      const bool issue = c + NS - 1 < nchunks;
      if (issue) load_chunk(c + NS - 1, buf == 0 ? NS - 1 : buf - 1);  // (buf + NS - 1) % NS
      // the same for every wave of the workgroup
      const unsigned mcur = __builtin_amdgcn_readfirstlane(lds_cmask[c]);
      if (mcur) {
        const char* Mt = lds_main[buf];
        const char* Rt = lds_rope[buf];
        // partial S^T tiles (16 keys x 16 heads) over this wave's quarter:
        // element j of st[kt][hh] is key 16*kt + 4*g + j, head 16*hh + l16
        f32x4_t st[2][2];
        V8 ka[2][5];  // all A operands of the chunk's scores, read before the MFMAs
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
          const int r = kt * 16 + l16;
#pragma unroll
          for (int ks = 0; ks < 4; ks++) {
            const int c16 = 16 * qd + 4 * ks + g;  // 16-byte piece of dims 128*qd + 32*ks + 8*g
            ka[kt][ks] = lds_read16<V8>(Mt + r * 1024 + ((c16 ^ swz1k(r)) << 4));
          }
          // waves without rope dims hold a zero operand: the compiler may issue the
          // rope MFMA on every wave (with a zero Q operand there), and leftover
          // register contents such as inf would turn its products into NaN
          ka[kt][4] = qd < 2 ? lds_read16<V8>(Rt + r * 128 + (((4 * qd + g) ^ swzr(r)) << 4))
                             : zero_v8<V8>();
        }
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
          st[kt][0] = st[kt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ks++) {
            st[kt][0] = E::mfma16(ka[kt][ks], qm[0][ks], st[kt][0]);
            st[kt][1] = E::mfma16(ka[kt][ks], qm[1][ks], st[kt][1]);
          }
          if (qd < 2) {
            st[kt][0] = E::mfma16(ka[kt][4], qrp[0], st[kt][0]);
            st[kt][1] = E::mfma16(ka[kt][4], qrp[1], st[kt][1]);
          }
        }
        // Partial tiles summed by reduce-scatter: wave (h2, qd) sums tile qd
        // of its head group over the four quarters, S = ((p0 + p1) + p2) + p3
        // in that order, into a slot only it read; then every wave of the
        // group reads the four sums.
        char* xs = lds_xs + lane * 16;
#pragma unroll
        for (int t = 0; t < 4; t++)
          *reinterpret_cast<f32x4_t*>(xs + (wid * 4 + t) * 1024) = st[t >> 1][t & 1];
        __syncthreads();
        {
          f32x4_t acc = *reinterpret_cast<const f32x4_t*>(xs + (h2 * 4 + qd) * 1024);
#pragma unroll
          for (int q = 1; q < 4; q++)
            acc += *reinterpret_cast<const f32x4_t*>(xs + ((2 * q + h2) * 4 + qd) * 1024);
          *reinterpret_cast<f32x4_t*>(xs + (h2 * 4 + qd) * 1024) = acc;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; t++)
          st[t >> 1][t & 1] = *reinterpret_cast<const f32x4_t*>(xs + (h2 * 4 + t) * 1024);
        V8 pb[2];
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          float mx = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const int key = kt * 16 + 4 * g + j;
              const float v = ((mcur >> key) & 1u) ? st[kt][hh][j] : -INFINITY;
              st[kt][hh][j] = v;
              mx = vmax(mx, v);
            }
          mx = max_xor16_32(mx) * sl2;
          if (__builtin_amdgcn_ballot_w64(mx > m[hh] + kLazy)) {
            const float m_new = fmaxf(m[hh], mx);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m[hh] - m_new);
            m[hh] = m_new;
            lsum[hh] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; dt++) o[dt][hh] *= alpha;
          }
          const float mneg = m[hh] == -INFINITY ? 0.f : -m[hh];
#pragma unroll
          for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const float pv = fast_exp2(__builtin_fmaf(st[kt][hh][j], sl2, mneg));
              lsum[hh] += pv;
              pb[hh][4 * kt + j] = E::from_f32(pv);
            }
        }
        // O^T += V^T P^T: V^T rows d = 128*qd + 16*dt + l16, keys
        // {4g..4g+3, 16+4g..16+4g+3} (the key order of pb)
        const int r0 = 4 * g + (l16 >> 2), r1 = r0 + 16;
        const int cq = l16 & 3;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
          const int c16 = 16 * qd + 2 * dt + (cq >> 1);
          const int b8 = 8 * (cq & 1);
          const V8 a = lds_read_tr_pair<V8>(Mt + r0 * 1024 + ((c16 ^ swz1k(r0)) << 4) + b8,
                                            Mt + r1 * 1024 + ((c16 ^ swz1k(r1)) << 4) + b8);
          o[dt][0] = E::mfma16(a, pb[0], o[dt][0]);
          o[dt][1] = E::mfma16(a, pb[1], o[dt][1]);
        }
      }
      if (issue) wait_keep_newest(); else wait_vm();
      __syncthreads();
      buf = buf == NS - 1 ? 0 : buf + 1;
    }
  }

#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    const int head = hbase + 16 * hh + l16;
    float lt = lsum[hh] + __shfl_xor(lsum[hh], 16);
    lt += __shfl_xor(lt, 32);
    if (head >= p.N1) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // element j of o[dt][hh] is d = 128*qd + 16*dt + 4*g + j
    if (p.splits == 1) {
      T* orow = (T*)p.out + ((long)tk * p.N1 + head) * kDv + 128 * qd;
#pragma unroll
      for (int dt = 0; dt < 8; dt++)
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) =
            pack4<E>(o[dt][hh][0] * inv, o[dt][hh][1] * inv, o[dt][hh][2] * inv, o[dt][hh][3] * inv);
      if (g == 0 && qd == 0 && p.lse)
        p.lse[(long)tk * p.N1 + head] = lt > 0.f ? (m[hh] + log2f(lt)) * kLn2 : -INFINITY;
    } else {
      const long pr = ((long)tk * p.splits + sp) * p.N1 + head;
      float* po = p.part_o + pr * kDv + 128 * qd;
#pragma unroll
      for (int dt = 0; dt < 8; dt++)
        *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) =
            make_float4(o[dt][hh][0] * inv, o[dt][hh][1] * inv, o[dt][hh][2] * inv, o[dt][hh][3] * inv);
      if (g == 0 && qd == 0) p.part_lse[pr] = lt > 0.f ? m[hh] + log2f(lt) : -INFINITY;
    }
  }
}

// Split kernel for a separate value cache ("aclnnSparseFlashAttention",
// constraints section: query, key and value share D = 512; the value rows
// are gathered beside the key rows).  One workgroup per (decode token, split,
// group of 64 query heads); 4 waves, each owning 16 heads and the whole
// 576-dim score contraction (no partial-score exchange).  Per chunk of 32
// selected slots the key row (1 KB), its rope row (128 B) and the value row
// (1 KB) are staged by direct loads into a two-stage ring; per wave
// S^T (32 keys x 16 heads) = K Q^T on 16x16x32 MFMA, online softmax along
// the keys, O^T (512 x 16) += V^T P^T with V^T read transposed from the
// value tile.  Same slot table, masks, partials and combine as the shared-KV
// kernel.
template <class E>
__global__ __launch_bounds__(256) void sfa_split_sepv_kernel(SfaParams p, int n_items, int hgroups,
                                                             int per_split) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  constexpr int NS = 2;
  __shared__ __attribute__((aligned(1024))) char lds_k[NS][kMainB];
  __shared__ __attribute__((aligned(1024))) char lds_v[NS][kMainB];
  __shared__ __attribute__((aligned(1024))) char lds_r[NS][kRopeB];
  __shared__ __attribute__((aligned(16))) int lds_tab[kTab];
  __shared__ unsigned lds_cmask[kTab / kKeys];

  const int item = xcd_remap(blockIdx.x, n_items);
  if (item < 0) return;
  const int hg = item % hgroups;
  const int sp = (item / hgroups) % p.splits;
  const int tk = item / (hgroups * p.splits);
  int b, s, sq;
  sfa_token(p, tk, b, s, sq);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int kv_len = p.kv_lens[b];
  const int qpos = kv_len - sq + s;
  const int total = sfa_total_slots(p);
  const int slot_lo = sp * per_split;
  const int slot_hi = min(slot_lo + per_split, total);
  const int* topk = p.topk + (long)tk * p.topk_n;
  const int* btab = p.block_table + (long)b * p.max_pages;
  const float sl2 = p.scale * kLog2e;

  // Q^T as B operands: lane (g, head l16) holds dims 32*ks + 8*g .. +7
  const int head = hg * 64 + wid * 16 + l16;
  const bool hok = head < p.N1;
  V8 qm[16], qr[2];
  {
    const T* qrow = (const T*)p.q + ((long)tk * p.N1 + (hok ? head : 0)) * kDv;
    const T* qrr = (const T*)p.q_rope + ((long)tk * p.N1 + (hok ? head : 0)) * kDr;
#pragma unroll
    for (int ks = 0; ks < 16; ks++)
      qm[ks] = hok ? as_v8<V8>(ld16(qrow + 32 * ks + 8 * g)) : zero_v8<V8>();
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
      qr[ks] = hok ? as_v8<V8>(ld16(qrr + 32 * ks + 8 * g)) : zero_v8<V8>();
  }

  // physical rows of a run of slots and per-chunk masks (bit r = key r kept);
  // a dropped slot holds its chunk's first kept row, or row 0 when none
  auto fill_table = [&](int seg_lo, int seg_n) {
#pragma unroll
    for (int i = 0; i < kTab / 256; i++) {
      const int t = tid + 256 * i;
      const int gs = seg_lo + t;
      const int id = t < seg_n ? topk[gs / p.sbs] : -1;
      const bool idok = id >= 0 && id <= (kv_len - 1) / p.sbs;
      const int pos = idok ? id * p.sbs + gs % p.sbs : 0;
      const bool ok = t < seg_n && idok && pos < kv_len && (!p.causal || pos <= qpos);
      const int lp = ok ? min(pos / p.page, p.max_pages - 1) : 0;
      const int phys = ok ? btab[lp] : 0;
      const int row = ok ? min(max(phys, 0), p.num_pages - 1) * p.page + pos % p.page : 0;
      const unsigned long long bal = __ballot(ok);
      const unsigned half = lane < 32 ? (unsigned)bal : (unsigned)(bal >> 32);
      const int first = (half ? __builtin_ctz(half) : 0) + (lane & 32);
      const int frow = __shfl(row, first);
      lds_tab[t] = ok ? row : (half ? frow : 0);
      if ((lane & 31) == 0) lds_cmask[t >> 5] = half;
    }
  };
  // 4 waves x 8 key rows and 8 value rows (one 1-KB row per instruction),
  // and one 1-KB slice of 8 rope rows per wave
  auto load_chunk = [&](int c, int buf) {
    const int* tb = lds_tab + c * kKeys;
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int r = wid * 8 + u;
      const long row = tb[r];
      g2lds16((const char*)p.kc + row * (kDv * 2) + ((lane ^ swz1k(r)) << 4), lds_k[buf] + r * 1024);
      g2lds16((const char*)p.vc + row * (kDv * 2) + ((lane ^ swz1k(r)) << 4), lds_v[buf] + r * 1024);
    }
    const int r = wid * 8 + (lane >> 3);
    g2lds16((const char*)p.krc + (long)tb[r] * (kDr * 2) + (((lane & 7) ^ swzr(r)) << 4),
            lds_r[buf] + wid * 1024);
  };

  constexpr float kLazy = 8.f;
  float m = -INFINITY, lsum = 0.f;
  f32x4_t o[32];  // O^T tiles: rows d = 16*dt + 4*g + j, column head l16
#pragma unroll
  for (int dt = 0; dt < 32; dt++) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int seg_lo = slot_lo; seg_lo < slot_hi; seg_lo += kTab) {
    const int seg_n = min(kTab, slot_hi - seg_lo);
    const int nchunks = (seg_n + kKeys - 1) / kKeys;
    __syncthreads();  // the previous run's table and tiles are no longer read
    fill_table(seg_lo, seg_n);
    __syncthreads();
    load_chunk(0, 0);
    wait_vm();
    __syncthreads();
    int buf = 0;
    for (int c = 0; c < nchunks; c++) {
      if (c + 1 < nchunks) load_chunk(c + 1, buf ^ 1);
      const unsigned mcur = __builtin_amdgcn_readfirstlane(lds_cmask[c]);
      if (mcur) {
        const char* Kt = lds_k[buf];
        const char* Vt = lds_v[buf];
        const char* Rt = lds_r[buf];
        // element j of st[kt] is key 16*kt + 4*g + j, head l16
        f32x4_t st[2];
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
          const int r = kt * 16 + l16;
          st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 16; ks++) {
            const int c16 = 4 * ks + g;
            st[kt] = E::mfma16(lds_read16<V8>(Kt + r * 1024 + ((c16 ^ swz1k(r)) << 4)), qm[ks], st[kt]);
          }
#pragma unroll
          for (int ks = 0; ks < 2; ks++)
            st[kt] = E::mfma16(lds_read16<V8>(Rt + r * 128 + (((4 * ks + g) ^ swzr(r)) << 4)),
                               qr[ks], st[kt]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const int key = kt * 16 + 4 * g + j;
            const float v = ((mcur >> key) & 1u) ? st[kt][j] : -INFINITY;
            st[kt][j] = v;
            mx = vmax(mx, v);
          }
        mx = max_xor16_32(mx) * sl2;
        if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
          const float m_new = fmaxf(m, mx);
          const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
          m = m_new;
          lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < 32; dt++) o[dt] *= alpha;
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
        // O^T += V^T P^T: V^T rows d = 16*dt + l16, keys {4g..4g+3, 16+4g..16+4g+3}
        const int r0 = 4 * g + (l16 >> 2), r1 = r0 + 16;
        const int cq = l16 & 3;
#pragma unroll
        for (int dt = 0; dt < 32; dt++) {
          const int c16 = 2 * dt + (cq >> 1);
          const int b8 = 8 * (cq & 1);
          const V8 a = lds_read_tr_pair<V8>(Vt + r0 * 1024 + ((c16 ^ swz1k(r0)) << 4) + b8,
                                            Vt + r1 * 1024 + ((c16 ^ swz1k(r1)) << 4) + b8);
          o[dt] = E::mfma16(a, pb, o[dt]);
        }
      }
      wait_vm();
      __syncthreads();
      buf ^= 1;
    }
  }

  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  if (!hok) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // element j of o[dt] is d = 16*dt + 4*g + j
  if (p.splits == 1) {
    T* orow = (T*)p.out + ((long)tk * p.N1 + head) * kDv;
#pragma unroll
    for (int dt = 0; dt < 32; dt++)
      *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) =
          pack4<E>(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (g == 0 && p.lse)
      p.lse[(long)tk * p.N1 + head] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
  } else {
    const long pr = ((long)tk * p.splits + sp) * p.N1 + head;
    float* po = p.part_o + pr * kDv;
#pragma unroll
    for (int dt = 0; dt < 32; dt++)
      *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) =
          make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (g == 0) p.part_lse[pr] = lt > 0.f ? m + log2f(lt) : -INFINITY;
  }
}

// One wave per (token, head): merges the splits' partials.
template <class E>
__global__ __launch_bounds__(256) void sfa_combine_kernel(SfaParams p) {
  typedef typename E::T T;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long ntok = p.ntok;
  if (w >= ntok * p.N1) return;
  const long tk = w / p.N1;
  const int head = (int)(w % p.N1);
  float mx = -INFINITY;
  for (int s = 0; s < p.splits; s++) mx = fmaxf(mx, p.part_lse[(tk * p.splits + s) * p.N1 + head]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < p.splits; s++) {
      const long pr = (tk * p.splits + s) * p.N1 + head;
      const float ls = p.part_lse[pr];
      if (ls == -INFINITY) continue;
      const float wgt = fast_exp2(ls - mx);
      L += wgt;
      const float4* po = reinterpret_cast<const float4*>(p.part_o + pr * kDv + 8 * lane);
      const float4 a = po[0], c = po[1];
      acc[0] += wgt * a.x; acc[1] += wgt * a.y; acc[2] += wgt * a.z; acc[3] += wgt * a.w;
      acc[4] += wgt * c.x; acc[5] += wgt * c.y; acc[6] += wgt * c.z; acc[7] += wgt * c.w;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* orow = (T*)p.out + (tk * p.N1 + head) * kDv + 8 * lane;
  *reinterpret_cast<uint2*>(orow) = pack4<E>(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(orow + 4) = pack4<E>(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if (lane == 0 && p.lse) p.lse[tk * p.N1 + head] = L > 0.f ? (mx + log2f(L)) * kLn2 : -INFINITY;
}

// validate = 1: ids, kv_lens and the pages they reach must be in range.
__global__ void sfa_check_kernel(SfaParams p) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long ntok = p.ntok;
  if (i >= ntok * p.topk_n) return;
  const long tk = i / p.topk_n;
  int b, s, sq;
  sfa_token(p, (int)tk, b, s, sq);
  const int kv_len = p.kv_lens[b];
  bool bad = kv_len < 0 || kv_len > p.max_pages * p.page;
  const int id = p.topk[i];
  if (!bad && id != -1) {
    const long pos0 = (long)id * p.sbs;
    bad = id < 0 || pos0 >= kv_len;
    if (!bad) {
      const int phys = p.block_table[(long)b * p.max_pages + pos0 / p.page];
      bad = phys < 0 || phys >= p.num_pages;
    }
  }
  if (bad) p.bad[0] = 1;  // every writer stores the same value
}

int sfa_splits(const SfaParams& p) {
  const long tokens = p.ntok;
  const int hgroups = (p.N1 + 63) / 64;
  const long wgs = tokens * hgroups;
  const int total = sfa_total_slots(p);
  if (wgs == 0) return 1;
  // aim for >= 256 workgroups (one resident per CU), at least 4 chunks per split
  long s = (256 + wgs - 1) / wgs;
  const long max_s = (total + 4 * kKeys - 1) / (4 * kKeys);
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

// Sets n ints to v (a kernel, not a memset node, so callers may capture it).
__global__ void fill_i32_kernel(int* p, int n, int v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_sfa_check(const SfaParams& p, hipStream_t st) {
  const long n = p.ntok * p.topk_n;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(sfa_check_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class E>
static hipError_t sfa_t(const SfaParams& p, hipStream_t st, void* const* ev, int n_ev) {
  const long tokens = p.ntok;
  const int hgroups = (p.N1 + 63) / 64;
  const int total = sfa_total_slots(p);
  const int per_split = ((total + p.splits - 1) / p.splits + kKeys - 1) / kKeys * kKeys;
  const long n_items = tokens * p.splits * hgroups;
  hipError_t e = mark_event(ev, n_ev, 0, 0, st);
  if (e == hipSuccess) {
    // a value cache apart from the key cache: its own gather (plain SFA only)
    if (p.vc != p.kc && p.ckc == nullptr)
      hipLaunchKernelGGL((sfa_split_sepv_kernel<E>), dim3((unsigned)(8 * ((n_items + 7) / 8))),
                         dim3(256), 0, st, p, (int)n_items, hgroups, per_split);
    else
      hipLaunchKernelGGL((sfa_split_kernel<E>), dim3((unsigned)(8 * ((n_items + 7) / 8))),
                         dim3(512), 0, st, p, (int)n_items, hgroups, per_split);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 0, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 0, st);
  if (e == hipSuccess && p.splits > 1) {
    const long waves = tokens * p.N1;
    hipLaunchKernelGGL((sfa_combine_kernel<E>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                       p);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 1, st);
  return e;
}

// Shared-KV task list ("SparseAttnSharedkvMetadata": a per-core list of
// attention tasks with their start and end points): one wave per decode
// token.  Each 32-slot chunk of the token's slots weighs its kept keys plus a
// fixed cost for the gather and barrier it always takes; the chunks are cut
// into p.splits contiguous ranges of near-equal weight (split k starts at the
// first chunk whose inclusive weight prefix exceeds k / splits of the total)
// and written as slot ranges, so each split workgroup gets a similar number
// of kept keys whatever the band clipping and empty top-k slots.
__global__ __launch_bounds__(256) void sfa_task_kernel(SfaParams p) {
  constexpr int kChunkCost = 4;
  const long tk = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tk >= p.ntok) return;
  // the token's batch entry: the largest b with cu_q[b] <= tk, i.e. the count
  // of i in [1, B) with cu_q[i] <= tk, 64 prefix sums tested at a time
  int b, s, sq;
  if (p.cu_q) {
    b = 0;
    for (int i0 = 1; i0 < p.B; i0 += 64) {
      const int i = i0 + lane;
      b += __popcll(__ballot(i < p.B && p.cu_q[i] <= tk));
    }
    s = (int)tk - p.cu_q[b];
    sq = p.cu_q[b + 1] - p.cu_q[b];
  } else {
    sfa_token(p, (int)tk, b, s, sq);
  }
  if (lane == 0) *reinterpret_cast<int4*>(p.task + 4 * tk) = make_int4(b, s, sq, 0);
  const int kv_len = p.kv_lens[b];
  const int qpos = kv_len - sq + s;
  const int t_len = kv_len / p.cmp_ratio;
  const int t_qpos = t_len - sq + s;
  const int total = sfa_total_slots(p);
  const int nch = (total + kKeys - 1) / kKeys;
  const int* topk = p.topk + tk * p.topk_n;
  const int max_id = (t_len - 1) / p.sbs;  // ids above it start past the cache
  auto weight = [&](int c) {
    if (c >= nch) return 0;
    const int lo = c * kKeys, hi = min(lo + kKeys, total);
    int kept = 0;
    if (lo < p.win_pad) {  // band slots i keep position qpos - win_left + i in [0, kv_len)
      const int a = max(lo, p.win_left - qpos);
      const int e = min(min(hi, p.win_len), kv_len - qpos + p.win_left);
      kept = max(0, e - a);
    } else {
      // slot lo + u is entry ent[u] of the token's top-k row, offset off[u]
      // within that sparse block: one division per chunk, then a walk.  The
      // id loads are unconditional (entries clamped into the row; slots past
      // hi are dropped below), so they issue back to back.
      int ent[kKeys], off[kKeys];
      {
        const int r0 = lo - p.win_pad;
        int e = r0 / p.sbs, o = r0 - e * p.sbs;
#pragma unroll
        for (int u = 0; u < kKeys; u++) {
          ent[u] = min(e, p.topk_n - 1);
          off[u] = o;
          if (++o == p.sbs) {
            o = 0;
            ++e;
          }
        }
      }
      int id[kKeys];
#pragma unroll
      for (int u = 0; u < kKeys; u++) id[u] = topk[ent[u]];
#pragma unroll
      for (int u = 0; u < kKeys; u++) {
        const bool idok = lo + u < hi && id[u] >= 0 && id[u] <= max_id;
        const int pos = idok ? id[u] * p.sbs + off[u] : 0;
        kept += idok && pos < t_len && pos <= t_qpos;
      }
    }
    return kept + kChunkCost;
  };
  // one round of 64 chunks covers 2048 slots: the weights are kept from the
  // total's pass when it is the only round
  const int w0 = weight(lane);
  long wsum = 0;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    int w = c0 == 0 ? w0 : weight(c0 + lane);
    for (int o = 32; o > 0; o >>= 1) w += __shfl_xor(w, o);
    wsum += w;
  }
  int cnt = 0;  // lane k: chunks whose inclusive prefix * splits <= k * wsum
  long carry = 0;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    long incl = wave_incl_scan(c0 == 0 ? w0 : weight(c)) + carry;
    for (int k = 1; k < p.splits; k++) {
      const unsigned long long bal = __ballot(c < nch && incl * p.splits <= (long)k * wsum);
      if (lane == k) cnt += __popcll(bal);
    }
    carry = __shfl(incl, 63);
  }
  const int nxt = __shfl(cnt, (lane + 1) & 63);
  if (lane < p.splits) {
    const int clo = lane == 0 ? 0 : cnt;
    const int chi = lane + 1 == p.splits ? nch : nxt;
    int* t = p.task + 4 * p.ntok + 2 * (tk * p.splits + lane);
    t[0] = min(clo * kKeys, total);
    t[1] = min(max(chi, clo) * kKeys, total);
  }
}

hipError_t launch_sfa_task(const SfaParams& p, hipStream_t st) {
  if (p.ntok == 0) return hipSuccess;
  hipLaunchKernelGGL(sfa_task_kernel, dim3((unsigned)((p.ntok + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_sfa_sharedkv(const SfaParams& p, int fp16, bool have_tasks, hipStream_t st,
                               void* const* ev, int n_ev) {
  hipError_t e = mark_event(ev, n_ev, 0, 0, st);
  if (e == hipSuccess && !have_tasks) e = launch_sfa_task(p, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 0, 1, st);
  // the split / combine stages are timed as stages 1 and 2
  void* const* ev2 = n_ev > 1 ? ev + 2 : nullptr;
  if (e == hipSuccess) e = fp16 ? sfa_t<FP16>(p, st, ev2, n_ev - 1) : sfa_t<BF16>(p, st, ev2, n_ev - 1);
  return e;
}

hipError_t launch_sfa_fwd(const SfaParams& p, int fp16, hipStream_t st, void* const* ev, int n_ev) {
  return fp16 ? sfa_t<FP16>(p, st, ev, n_ev) : sfa_t<BF16>(p, st, ev, n_ev);
}

}  // namespace tsa
