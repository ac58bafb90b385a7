// FloydAttention ("aclnnFusedFloydAttentionGrad", function description and
// formula section): the query keeps two sequence axes, and the scores of row
// (n, m) against key k add two products batched over different axes:
//   S = scale * (Q K1^T + Q K2^T),  P = Softmax(S),  Y = P V1 + P V2,
// Q [Z, N, M, D], K1/V1 [Z, N, K, D] (batched over n), K2/V2 [Z, M, K, D]
// (batched over m), Z = B * H.  The backward chain: dP = dY V1^T + dY V2^T,
// dS = P (dP - rowsum(dY * Y)), dV1 = P^T dY, dV2 = P^T dY,
// dQ = (dS K1 + dS K2) scale, dK1 = dS^T Q scale, dK2 = dS^T Q scale.
//
// Built from small operators, as the page advises once M x D or K x D is
// large: every product is one launch of a strided, two-level-batched MFMA
// GEMM whose operand and output strides express the batch axis (n or m),
// with S and dP materialised in fp32 and P / dS in 16 bits in the
// workspace; a row kernel forms the softmax (P, LSE) and one forms dS.
// Deterministic: no atomics; each output element is written by one lane,
// and the two products of Y and of dQ are summed in a fixed order.
#include "tsa_device.h"
#include "tsa_internal.h"

namespace tsa {

namespace {
constexpr int kTR = 64;    // output rows per workgroup
constexpr int kTC = 128;   // output columns per workgroup
constexpr int kTL = 64;    // contraction chunk
constexpr int kP = kTL + 8;  // LDS row pitch in elements (144 bytes: 16-byte aligned rows)

template <typename T>
__device__ __forceinline__ void scatter8(T* dst, long stride, uint4 v) {
  const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
  for (int i = 0; i < 8; i++) dst[i * stride] = e[i];
}
}  // namespace

// C(z1, z2, r, c) = alpha * sum_l A(z1, z2, r, l) B(z1, z2, l, c), element
// addresses base + z1*s1 + z2*s2 + (row or l)*s + (l or col)*s.  AL: A is
// contiguous along l (else along r); BL: B contiguous along l (else along c).
// The operand tiles are staged in LDS as [row][l] and [col][l] (a transposed
// operand is scattered on the way in), then read as 16-byte MFMA operands.
// OUT: 0 fp32 store, 1 fp32 accumulate, 2 16-bit store, 3 16-bit store of
// (fp32 C + product) into c16.  L, and R (when !AL) and Cn (when !BL), are
// multiples of 8; tails of R, Cn and L are masked.
template <class E, bool AL, bool BL, int OUT>
__global__ __launch_bounds__(256) void floyd_gemm_kernel(FloydGemm g) {
  typedef typename E::T T;
  typedef typename E::V8 V8;
  __shared__ __attribute__((aligned(16))) T sa[kTR * kP];
  __shared__ __attribute__((aligned(16))) T sb[kTC * kP];

  const int nr = (g.R + kTR - 1) / kTR, nc = (g.Cn + kTC - 1) / kTC;
  long id = blockIdx.x;
  const int tr = (int)(id % nr);
  id /= nr;
  const int tc = (int)(id % nc);
  id /= nc;
  const long z2 = id % g.Z2, z1 = id / g.Z2;
  const T* A = (const T*)g.a + z1 * g.a_s1 + z2 * g.a_s2;
  const T* Bm = (const T*)g.b + z1 * g.b_s1 + z2 * g.b_s2;
  const int r0 = tr * kTR, c0 = tc * kTC;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);

  f32x16 acc[2];
#pragma unroll
  for (int ct = 0; ct < 2; ct++)
#pragma unroll
    for (int j = 0; j < 16; j++) acc[ct][j] = 0.f;

  for (int l0 = 0; l0 < g.L; l0 += kTL) {
    // A tile: kTR rows x kTL l
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int x = tid + 256 * u;
      if (AL) {
        const int r = x >> 3, pc = x & 7;
        const int gr = r0 + r, gl = l0 + 8 * pc;
        const uint4 v = (gr < g.R && gl < g.L) ? ld16(A + gr * g.a_sr + gl) : zero;
        *reinterpret_cast<uint4*>(sa + r * kP + 8 * pc) = v;
      } else {
        const int l = x >> 3, rg = x & 7;
        const int gr = r0 + 8 * rg, gl = l0 + l;
        const uint4 v = (gr < g.R && gl < g.L) ? ld16(A + gl * g.a_sl + gr) : zero;
        scatter8(sa + (8 * rg) * kP + l, kP, v);
      }
    }
    // B tile: kTC columns x kTL l
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int x = tid + 256 * u;
      if (BL) {
        const int c = x >> 3, pc = x & 7;
        const int gc = c0 + c, gl = l0 + 8 * pc;
        const uint4 v = (gc < g.Cn && gl < g.L) ? ld16(Bm + gc * g.b_sc + gl) : zero;
        *reinterpret_cast<uint4*>(sb + c * kP + 8 * pc) = v;
      } else {
        const int l = x >> 4, cg = x & 15;
        const int gc = c0 + 8 * cg, gl = l0 + l;
        const uint4 v = (gc < g.Cn && gl < g.L) ? ld16(Bm + gl * g.b_sl + gc) : zero;
        scatter8(sb + (8 * cg) * kP + l, kP, v);
      }
    }
    __syncthreads();
    // this wave: rows 32*(wid&1) .., columns 64*(wid>>1) + 32*ct ..
#pragma unroll
    for (int ks = 0; ks < kTL / 16; ks++) {
      const V8 a = lds_read16<V8>(sa + (32 * (wid & 1) + l32) * kP + 16 * ks + 8 * h);
#pragma unroll
      for (int ct = 0; ct < 2; ct++) {
        const V8 b = lds_read16<V8>(sb + (64 * (wid >> 1) + 32 * ct + l32) * kP + 16 * ks + 8 * h);
        acc[ct] = E::mfma32(a, b, acc[ct]);
      }
    }
    __syncthreads();
  }

  // element j of acc[ct]: row 32*(wid&1) + 8*(j/4) + 4*h + j%4, column l32
  const long cb = z1 * g.c_s1 + z2 * g.c_s2;
#pragma unroll
  for (int ct = 0; ct < 2; ct++) {
    const int c = c0 + 64 * (wid >> 1) + 32 * ct + l32;
    if (c >= g.Cn) continue;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int r = r0 + 32 * (wid & 1) + 8 * (j >> 2) + 4 * h + (j & 3);
      if (r >= g.R) continue;
      const long off = cb + r * g.c_sr + c * g.c_sc;
      const float v = g.alpha * acc[ct][j];
      if constexpr (OUT == 0) ((float*)g.c)[off] = v;
      if constexpr (OUT == 1) ((float*)g.c)[off] += v;
      if constexpr (OUT == 2) ((T*)g.c)[off] = E::from_f32(v);
      if constexpr (OUT == 3) ((T*)g.c16)[off] = E::from_f32(((const float*)g.c)[off] + v);
    }
  }
}

// Row softmax over the K scores of a query row: P = exp(S - max) / sum (16
// bits), LSE = max + ln(sum).  One wave per row.
template <class E>
__global__ __launch_bounds__(256) void floyd_softmax_kernel(const float* S, void* P, float* lse,
                                                           long rows, int K) {
  typedef typename E::T T;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* s = S + row * K;
  float mx = -INFINITY;
  for (int k = 4 * lane; k < K; k += 256) {
    const float4 v = *reinterpret_cast<const float4*>(s + k);
    mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float m2 = mx * kLog2e;
  float sum = 0.f;
  for (int k = 4 * lane; k < K; k += 256) {
    const float4 v = *reinterpret_cast<const float4*>(s + k);
    sum += fast_exp2(v.x * kLog2e - m2) + fast_exp2(v.y * kLog2e - m2) +
           fast_exp2(v.z * kLog2e - m2) + fast_exp2(v.w * kLog2e - m2);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  const float inv = 1.f / sum;
  T* pr = (T*)P + row * K;
  for (int k = 4 * lane; k < K; k += 256) {
    const float4 v = *reinterpret_cast<const float4*>(s + k);
    *reinterpret_cast<uint2*>(pr + k) =
        pack4<E>(fast_exp2(v.x * kLog2e - m2) * inv, fast_exp2(v.y * kLog2e - m2) * inv,
                 fast_exp2(v.z * kLog2e - m2) * inv, fast_exp2(v.w * kLog2e - m2) * inv);
  }
  if (lane == 0) lse[row] = mx + logf(sum);
}

// Per query row: softmax_grad = sum_d dY * Y, then P = exp(S - LSE) and
// dS = P (dP - softmax_grad), both in 16 bits.  One wave per row.
template <class E>
__global__ __launch_bounds__(256) void floyd_ds_kernel(const float* S, const float* dP,
                                                      const float* lse, const void* Y,
                                                      const void* dY, void* P, void* dS, long rows,
                                                      int K, int D) {
  typedef typename E::T T;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  for (int d = lane; d < D; d += 64)
    acc += E::to_f32(((const T*)dY)[row * D + d]) * E::to_f32(((const T*)Y)[row * D + d]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  const float l2 = lse[row] * kLog2e;
  const float* s = S + row * K;
  const float* dp = dP + row * K;
  T* pr = (T*)P + row * K;
  T* dsr = (T*)dS + row * K;
  for (int k = 4 * lane; k < K; k += 256) {
    const float4 v = *reinterpret_cast<const float4*>(s + k);
    const float4 w = *reinterpret_cast<const float4*>(dp + k);
    const float p0 = fast_exp2(v.x * kLog2e - l2), p1 = fast_exp2(v.y * kLog2e - l2);
    const float p2 = fast_exp2(v.z * kLog2e - l2), p3 = fast_exp2(v.w * kLog2e - l2);
    *reinterpret_cast<uint2*>(pr + k) = pack4<E>(p0, p1, p2, p3);
    *reinterpret_cast<uint2*>(dsr + k) =
        pack4<E>(p0 * (w.x - acc), p1 * (w.y - acc), p2 * (w.z - acc), p3 * (w.w - acc));
  }
}

namespace {

template <class E>
hipError_t gemm(const FloydGemm& g, bool al, bool bl, int out, hipStream_t st) {
  const long tiles = (long)((g.R + kTR - 1) / kTR) * ((g.Cn + kTC - 1) / kTC) * g.Z2 * g.Z1;
  if (tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)tiles), block(256);
#define TSA_FLOYD_GEMM(AL_, BL_, OUT_) \
  hipLaunchKernelGGL((floyd_gemm_kernel<E, AL_, BL_, OUT_>), grid, block, 0, st, g)
  if (al && bl) {
    if (out == 0) TSA_FLOYD_GEMM(true, true, 0);
    else TSA_FLOYD_GEMM(true, true, 1);
  } else if (al && !bl) {
    if (out == 0) TSA_FLOYD_GEMM(true, false, 0);
    else TSA_FLOYD_GEMM(true, false, 3);
  } else {
    TSA_FLOYD_GEMM(false, false, 2);
  }
#undef TSA_FLOYD_GEMM
  return hipGetLastError();
}

// The score products of (Q, K1, K2) into S: the first batched over n (rows
// m), the second over m (rows n) and added.  Used for S (Q, K1, K2) and for
// dP (dY, V1, V2).
template <class E>
hipError_t two_scores(const FloydParams& p, const void* q, const void* k1, const void* k2,
                      float* out, float alpha, hipStream_t st) {
  const long N = p.N, M = p.M, K = p.K, D = p.D;
  FloydGemm g{};
  g.Z1 = p.Z; g.L = p.D; g.alpha = alpha; g.c = out;
  // batched over n: rows m, columns k
  g.a = q; g.a_s1 = N * M * D; g.a_s2 = M * D; g.a_sr = D; g.a_sl = 1;
  g.b = k1; g.b_s1 = N * K * D; g.b_s2 = K * D; g.b_sl = 1; g.b_sc = D;
  g.c_s1 = N * M * K; g.c_s2 = M * K; g.c_sr = K; g.c_sc = 1;
  g.Z2 = p.N; g.R = p.M; g.Cn = p.K;
  hipError_t e = gemm<E>(g, true, true, 0, st);
  if (e != hipSuccess) return e;
  // batched over m: rows n, columns k, added
  g.a_s2 = D; g.a_sr = M * D;
  g.b = k2; g.b_s1 = M * K * D; g.b_s2 = K * D;
  g.c_s2 = K; g.c_sr = M * K;
  g.Z2 = p.M; g.R = p.N;
  return gemm<E>(g, true, true, 1, st);
}

// out16 = alpha * (X V1 + X V2) over k, X [Z, N, M, K] 16-bit, V [.., K, D]:
// the first product batched over n into the fp32 accumulator, the second over
// m added and written in 16 bits.
template <class E>
hipError_t two_values(const FloydParams& p, const void* x, const void* v1, const void* v2,
                      float* accum, void* out16, float alpha, hipStream_t st) {
  const long N = p.N, M = p.M, K = p.K, D = p.D;
  FloydGemm g{};
  g.Z1 = p.Z; g.L = p.K; g.alpha = alpha; g.c = accum; g.c16 = out16;
  g.a = x; g.a_s1 = N * M * K; g.a_s2 = M * K; g.a_sr = K; g.a_sl = 1;
  g.b = v1; g.b_s1 = N * K * D; g.b_s2 = K * D; g.b_sl = D; g.b_sc = 1;
  g.c_s1 = N * M * D; g.c_s2 = M * D; g.c_sr = D; g.c_sc = 1;
  g.Z2 = p.N; g.R = p.M; g.Cn = p.D;
  hipError_t e = gemm<E>(g, true, false, 0, st);
  if (e != hipSuccess) return e;
  g.a_s2 = K; g.a_sr = M * K;
  g.b = v2; g.b_s1 = M * K * D; g.b_s2 = K * D;
  g.c_s2 = D; g.c_sr = M * D;
  g.Z2 = p.M; g.R = p.N;
  return gemm<E>(g, true, false, 3, st);
}

// d1 = alpha * X^T Y batched over n ([K, D] per n) and d2 = alpha * X^T Y
// batched over m, X [Z, N, M, K], Y [Z, N, M, D] (16-bit outputs).
template <class E>
hipError_t two_transposed(const FloydParams& p, const void* x, const void* y, void* d1, void* d2,
                          float alpha, hipStream_t st) {
  const long N = p.N, M = p.M, K = p.K, D = p.D;
  FloydGemm g{};
  g.Z1 = p.Z; g.alpha = alpha; g.R = p.K; g.Cn = p.D;
  // over n: rows k, columns d, contraction m
  g.a = x; g.a_s1 = N * M * K; g.a_s2 = M * K; g.a_sr = 1; g.a_sl = K;
  g.b = y; g.b_s1 = N * M * D; g.b_s2 = M * D; g.b_sl = D; g.b_sc = 1;
  g.c = d1; g.c_s1 = N * K * D; g.c_s2 = K * D; g.c_sr = D; g.c_sc = 1;
  g.Z2 = p.N; g.L = p.M;
  hipError_t e = gemm<E>(g, false, false, 2, st);
  if (e != hipSuccess) return e;
  // over m: contraction n
  g.a_s2 = K; g.a_sl = M * K;
  g.b_s2 = D; g.b_sl = M * D;
  g.c = d2; g.c_s1 = M * K * D;
  g.Z2 = p.M; g.L = p.N;
  return gemm<E>(g, false, false, 2, st);
}

template <class E>
hipError_t fwd_e(const FloydParams& p, hipStream_t st, void* const* ev, int n_ev) {
  const long rows = (long)p.Z * p.N * p.M;
  hipError_t e = mark_event(ev, n_ev, 0, 0, st);
  if (e == hipSuccess) e = two_scores<E>(p, p.q, p.k1, p.k2, p.s, p.scale, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 0, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 0, st);
  if (e == hipSuccess && rows > 0) {
    hipLaunchKernelGGL(floyd_softmax_kernel<E>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                       st, (const float*)p.s, p.p, p.lse, rows, p.K);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 0, st);
  if (e == hipSuccess) e = two_values<E>(p, p.p, p.v1, p.v2, p.acc, p.out, 1.f, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 1, st);
  return e;
}

template <class E>
hipError_t bwd_e(const FloydParams& p, hipStream_t st, void* const* ev, int n_ev) {
  const long rows = (long)p.Z * p.N * p.M;
  hipError_t e = mark_event(ev, n_ev, 0, 0, st);
  if (e == hipSuccess) e = two_scores<E>(p, p.q, p.k1, p.k2, p.s, p.scale, st);
  if (e == hipSuccess) e = two_scores<E>(p, p.dout, p.v1, p.v2, p.dp, 1.f, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 0, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 0, st);
  if (e == hipSuccess && rows > 0) {
    hipLaunchKernelGGL(floyd_ds_kernel<E>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       (const float*)p.s, (const float*)p.dp, (const float*)p.lse, p.o, p.dout,
                       p.p, p.ds, rows, p.K, p.D);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark_event(ev, n_ev, 1, 1, st);
  // dV1, dV2 = P^T dY; dQ = (dS K1 + dS K2) scale; dK1, dK2 = dS^T Q scale
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 0, st);
  if (e == hipSuccess) e = two_transposed<E>(p, p.p, p.dout, p.dv1, p.dv2, 1.f, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 2, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 3, 0, st);
  if (e == hipSuccess) e = two_values<E>(p, p.ds, p.k1, p.k2, p.acc, p.dq, p.scale, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 3, 1, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 4, 0, st);
  if (e == hipSuccess) e = two_transposed<E>(p, p.ds, p.q, p.dk1, p.dk2, p.scale, st);
  if (e == hipSuccess) e = mark_event(ev, n_ev, 4, 1, st);
  return e;
}

}  // namespace

hipError_t launch_floyd_fwd(const FloydParams& p, int fp16, hipStream_t st, void* const* ev,
                            int n_ev) {
  return fp16 ? fwd_e<FP16>(p, st, ev, n_ev) : fwd_e<BF16>(p, st, ev, n_ev);
}

hipError_t launch_floyd_bwd(const FloydParams& p, int fp16, hipStream_t st, void* const* ev,
                            int n_ev) {
  return fp16 ? bwd_e<FP16>(p, st, ev, n_ev) : bwd_e<BF16>(p, st, ev, n_ev);
}

}  // namespace tsa
