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
// Shared KV: the value row is the key row (value_cache may alias key_cache),
// so one gathered 1 KB row feeds both the scores and P V.
//
// Split kernel: one workgroup per (decode token, split of its selected keys,
// group of 64 query heads); 4 waves x 16 heads.  Selected rows are gathered 32
// at a time by direct global -> LDS loads (a 1 KB key row per instruction,
// plus its 128-byte rope row) into a double buffer.  On 16x16x32 MFMA, per
// wave: S^T (32 keys x 16 heads) = K Q^T over 576 dims (Q^T held in
// registers), online softmax along the keys (lanes own heads), and
// O^T (512 x 16) += V^T P^T with V^T read from the same key tile by LDS
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

// 1 KB rows (64 16-byte pieces): piece c of row r at c ^ swz1k(r).  16 rows
// reading one piece hit 16 distinct bank groups, and transpose reads of 8
// rows x 2 adjacent pieces hit 16 distinct bank groups.
__device__ __forceinline__ int swz1k(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// 128-byte rope rows (8 pieces): 16 consecutive rows reading one piece hit
// distinct bank groups.
__device__ __forceinline__ int swzr(int r) { return (r >> 1) & 7; }

typedef float f32x4_t __attribute__((ext_vector_type(4)));
}  // namespace

template <class E>
__global__ __launch_bounds__(256) void sfa_split_kernel(SfaParams p, int n_items, int hgroups,
                                                        int per_split) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  __shared__ __attribute__((aligned(1024))) char lds_main[2][kMainB];
  __shared__ __attribute__((aligned(1024))) char lds_rope[2][kRopeB];

  const int item = xcd_remap(blockIdx.x, n_items);
  if (item < 0) return;
  // item order: token-major so a token's splits / head groups share L2
  const int hg = item % hgroups;
  const int sp = (item / hgroups) % p.splits;
  const int tk = item / (hgroups * p.splits);
  const int b = tk / p.Sq, s = tk % p.Sq;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  const int kv_len = p.kv_lens[b];
  const int qpos = kv_len - p.Sq + s;
  const int total = p.topk_n * p.sbs;
  const int slot_lo = sp * per_split;
  const int slot_hi = min(slot_lo + per_split, total);
  const int nchunks = slot_hi > slot_lo ? (slot_hi - slot_lo + kKeys - 1) / kKeys : 0;

  const int head = hg * 64 + wid * 16 + l16;
  const bool head_ok = head < p.N1;
  const int* topk = p.topk + (long)tk * p.topk_n;  // N2 = 1
  const int* btab = p.block_table + (long)b * p.max_pages;
  const float sl2 = p.scale * kLog2e;

  // Q^T as the B operand: lane (g, head) holds d = 32*ks + 8*g .. +7
  V8 qreg[18];
  {
    const T* qr = (const T*)p.q + ((long)tk * p.N1 + (head_ok ? head : 0)) * kDv;
    const T* qrr = (const T*)p.q_rope + ((long)tk * p.N1 + (head_ok ? head : 0)) * kDr;
#pragma unroll
    for (int ks = 0; ks < 16; ks++)
      qreg[ks] = head_ok ? as_v8<V8>(ld16(qr + 32 * ks + 8 * g)) : zero_v8<V8>();
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
      qreg[16 + ks] = head_ok ? as_v8<V8>(ld16(qrr + 32 * ks + 8 * g)) : zero_v8<V8>();
  }

  // Row addresses of chunk c: lanes 0..31 resolve slot -> position -> page
  // -> physical row; returns the validity mask (bit r = key r is kept).
  // Invalid slots re-read the chunk's first valid row (finite data, P = 0).
  auto resolve = [&](int c, int& rowidx) -> unsigned {
    const int slot = slot_lo + c * kKeys + (lane & 31);
    bool ok = lane < 32 && slot < slot_hi;
    int pos = 0;
    if (ok) {
      const int id = topk[slot / p.sbs];
      pos = id * p.sbs + slot % p.sbs;
      ok = id >= 0 && pos < kv_len && (!p.causal || pos <= qpos);
    }
    int lp = min(max(pos / p.page, 0), p.max_pages - 1);
    int phys = ok ? min(max(btab[lp], 0), p.num_pages - 1) : 0;
    rowidx = phys * p.page + (ok ? pos % p.page : 0);
    const unsigned long long bal = __ballot(ok);
    const unsigned mask = (unsigned)(bal & 0xffffffffull);
    const int first = mask ? __builtin_ctz(mask) : 0;
    const int frow = __shfl(rowidx, first);
    if (!ok) rowidx = frow;
    return mask;
  };
  auto load_chunk = [&](int rowidx, int buf) {
    const char* kc = (const char*)p.kc;
    const char* krc = (const char*)p.krc;
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int r = wid * 8 + u;                 // one 1 KB row per instruction
      const int ri = __shfl(rowidx, r);
      g2lds16(kc + (long)ri * (kDv * 2) + ((lane ^ swz1k(r)) << 4), lds_main[buf] + r * 1024);
    }
    {
      const int r = wid * 8 + (lane >> 3);        // 8 rope rows per instruction
      const int ri = __shfl(rowidx, r);
      g2lds16(krc + (long)ri * (kDr * 2) + (((lane & 7) ^ swzr(r)) << 4),
              lds_rope[buf] + wid * 1024);
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4_t o[32];
#pragma unroll
  for (int dt = 0; dt < 32; dt++) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int rowidx;
  unsigned mask_cur = 0, mask_next = 0;
  if (nchunks > 0) {
    mask_cur = resolve(0, rowidx);
    load_chunk(rowidx, 0);
  }
  wait_vm();
  __syncthreads();
  int buf = 0;
  for (int c = 0; c < nchunks; c++) {
    if (c + 1 < nchunks) {
      mask_next = resolve(c + 1, rowidx);
      load_chunk(rowidx, buf ^ 1);
    }
    if (mask_cur) {
      const char* Mt = lds_main[buf];
      const char* Rt = lds_rope[buf];
      f32x4_t st[2];
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int r = kt * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < 16; ks++) {
          const int c16 = 4 * ks + g;
          const V8 a = lds_read16<V8>(Mt + r * 1024 + ((c16 ^ swz1k(r)) << 4));
          st[kt] = E::mfma16(a, qreg[ks], st[kt]);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          const int c8 = 4 * ks + g;
          const V8 a = lds_read16<V8>(Rt + r * 128 + ((c8 ^ swzr(r)) << 4));
          st[kt] = E::mfma16(a, qreg[16 + ks], st[kt]);
        }
      }
      // element j of tile kt is key kt*16 + 4*g + j, column = this lane's head
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int key = kt * 16 + 4 * g + j;
          const float v = ((mask_cur >> key) & 1u) ? st[kt][j] * sl2 : -INFINITY;
          st[kt][j] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 32; dt++) o[dt] *= alpha;
      V8 pb;
#pragma unroll
      for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float pv = fast_exp2(st[kt][j] - m_use);
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
        const V8 a = lds_read_tr_pair<V8>(Mt + r0 * 1024 + ((c16 ^ swz1k(r0)) << 4) + b8,
                                          Mt + r1 * 1024 + ((c16 ^ swz1k(r1)) << 4) + b8);
        o[dt] = E::mfma16(a, pb, o[dt]);
      }
    }
    wait_vm();
    __syncthreads();
    buf ^= 1;
    mask_cur = mask_next;
  }

  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  if (!head_ok) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // element j of o[dt] is d = 16*dt + 4*g + j
  if (p.splits == 1) {
    T* orow = (T*)p.out + ((long)tk * p.N1 + head) * kDv;
#pragma unroll
    for (int dt = 0; dt < 32; dt++)
      *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) =
          pack4<E>(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (g == 0 && p.lse) p.lse[(long)tk * p.N1 + head] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
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
  const long ntok = (long)p.B * p.Sq;
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
  const long ntok = (long)p.B * p.Sq;
  if (i >= ntok * p.topk_n) return;
  const long tk = i / p.topk_n;
  const int b = (int)(tk / p.Sq);
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
  const long tokens = (long)p.B * p.Sq;
  const int hgroups = (p.N1 + 63) / 64;
  const long wgs = tokens * hgroups;
  const int total = p.topk_n * p.sbs;
  if (wgs == 0) return 1;
  // aim for >= 512 workgroups (two per CU), at least 4 chunks per split
  long s = (512 + wgs - 1) / wgs;
  const long max_s = (total + 4 * kKeys - 1) / (4 * kKeys);
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

hipError_t launch_sfa_check(const SfaParams& p, hipStream_t st) {
  const long n = (long)p.B * p.Sq * p.topk_n;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(sfa_check_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class E>
static hipError_t sfa_t(const SfaParams& p, hipStream_t st, void* const* ev, int n_ev) {
  const long tokens = (long)p.B * p.Sq;
  const int hgroups = (p.N1 + 63) / 64;
  const int total = p.topk_n * p.sbs;
  const int per_split = ((total + p.splits - 1) / p.splits + kKeys - 1) / kKeys * kKeys;
  const long n_items = tokens * p.splits * hgroups;
  hipError_t e = mark_event(ev, n_ev, 0, 0, st);
  if (e == hipSuccess) {
    hipLaunchKernelGGL((sfa_split_kernel<E>), dim3((unsigned)(8 * ((n_items + 7) / 8))), dim3(256),
                       0, st, p, (int)n_items, hgroups, per_split);
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

hipError_t launch_sfa_fwd(const SfaParams& p, int fp16, hipStream_t st, void* const* ev, int n_ev) {
  return fp16 ? sfa_t<FP16>(p, st, ev, n_ev) : sfa_t<BF16>(p, st, ev, n_ev);
}

}  // namespace tsa
