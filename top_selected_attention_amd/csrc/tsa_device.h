// Device-side building blocks for gfx950 (CDNA4, wave64).
//
// MFMA operand layouts used throughout (checked on the device by an in-bounds
// probe of the builtins):
//   v_mfma_f32_32x32x16_{bf16,f16}: A (32 x 16) lane l holds row l%32 and
//     8 k-values of half l/32; B (16 x 32) lane l holds column l%32 and the 8
//     k-values of the same half; C (32 x 32, 16 fp32 per lane) element j of
//     lane l is row 8*(j/4) + 4*(l/32) + j%4, column l%32.
//   v_mfma_f32_16x16x32_{bf16,f16}: A lane l holds row l%16 and 8 k-values of
//     quarter l/16; C element j of lane l is row 4*(l/16) + j, column l%16.
// Which 8 k-values a lane holds is free as long as A and B agree; the
// kernels use that freedom to feed accumulator tiles straight back in as
// operands.
//
// ds_read_b64_tr_b16 (LDS transpose read): within each group of 16 lanes,
// output element j of lane i is element i%4 of the 4 x 16-bit values that
// lane 4*j + i/4 of the group addressed.  Pointing lane 4*j + c at
// row_j[4c .. 4c+3] therefore hands lane i the column entries
// row_0[i], .., row_3[i]: a transposed 16 x 4 tile, used to read V (and K,
// Q, dO in the backward) as the k-major MFMA operand without transposing it
// in memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element type traits: storage type, 8-wide MFMA operand, conversions.
struct BF16 {
  typedef __bf16 T;
  typedef bf16x8 V8;
  static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ T from_f32(float x) { return (T)x; }
  static __device__ __forceinline__ float to_f32(T x) { return (float)x; }
};

struct FP16 {
  typedef _Float16 T;
  typedef f16x8 V8;
  static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ T from_f32(float x) { return (T)x; }
  static __device__ __forceinline__ float to_f32(T x) { return (float)x; }
};

// 16-byte global load / store of 8 16-bit elements.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

template <typename V8>
__device__ __forceinline__ V8 as_v8(uint4 u) {
  return __builtin_bit_cast(V8, u);
}

// Two transposed LDS reads give one 8-wide operand.
template <typename V8>
__device__ __forceinline__ V8 lds_read_tr_pair(const void* p0, const void* p1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(const char*)p0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(const char*)p1);
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(V8, v);
}

template <typename V8>
__device__ __forceinline__ V8 lds_read16(const void* p) {
  return __builtin_bit_cast(V8, *reinterpret_cast<const uint4*>(p));
}

// IEEE maximum (a NaN operand gives NaN).  On gfx950 it is v_maximum3_f32,
// two operands per instruction and no canonicalising of its inputs, which
// fmaxf (maxnum) needs for values such as MFMA results.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }


// Max over lanes l and l ^ 32, and over l, l ^ 16, l ^ 32, l ^ 48, on the
// VALU lane-swap instructions (a swap of 16-lane rows 1, 3 with 0, 2, and of
// the two 32-lane halves) instead of LDS-routed shuffles.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16_32(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_xor32(vmax(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// XOR swizzle of the 16 16-byte pieces of a 256-byte LDS row (one K, V, Q or
// dO row of 128 16-bit values).  Row r stores logical piece c at c ^ swz(r).
// It keeps three read patterns free of bank conflicts: 16 consecutive rows
// reading one piece (swz is a bijection on r mod 16); 8 rows reading two
// adjacent pieces (swz(0..7) are all even); and transpose reads of 4
// consecutive rows x 4 aligned pieces (rows of an aligned group of 4 differ
// in bits 2-3 of swz).
__device__ __forceinline__ int swz(int r) {
  return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
}

// Waits for this wave's outstanding vector-memory loads (including direct
// global -> LDS loads) to land.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits until at most N of this wave's vector-memory operations are still in
// flight (they complete in issue order): the older stages of a multi-stage
// pipeline have landed while the newest N loads may still be pending.
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename V8>
__device__ __forceinline__ V8 zero_v8() {
  return __builtin_bit_cast(V8, make_uint4(0, 0, 0, 0));
}

// Four fp32 values rounded to the element type, packed into 8 bytes.
template <class E>
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  typedef typename E::T T;
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 v = {E::from_f32(a), E::from_f32(b), E::from_f32(c), E::from_f32(d)};
  return __builtin_bit_cast(uint2, v);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// lds_base + 16*l.  lds_base must be the same for every lane of the wave.
//
// Issued from inline assembly, so the compiler's wait-count pass does not see
// an LDS write in flight: it then inserts no "wait for every vector load"
// before later LDS reads, and a pipeline stage can stay in flight across the
// reads of an older stage.  The caller owns the ordering: an explicit vmcnt
// wait (wait_vm / wait_vm_le) by the issuing wave, then a barrier when other
// waves read the bytes, before any read; and the same before a buffer is
// filled again.  The global address is read when the instruction issues; M0
// (the LDS base) is saved and restored around it.
__device__ __forceinline__ void g2lds16(const void* g, void* lds_base) {
  const unsigned l = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "v"(g), "s"(l)
      : "memory");
}
// Same with 4 bytes per lane (lane l's dword lands at lds_base + 4*l).
__device__ __forceinline__ void g2lds4(const void* g, void* lds_base) {
  const unsigned l = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "v"(g), "s"(l)
      : "memory");
}

// Direct loads addressed by 32-bit LDS byte addresses (see lds_addr): the
// vector-address form and the scalar-base form (a wave-uniform base plus a
// per-lane 32-bit byte offset, so the per-lane address needs no 64-bit
// arithmetic; readfirstlane yields a signed int, so each half of the base
// goes back to unsigned before widening).
__device__ __forceinline__ void g2lds16_at(const void* g, unsigned lds) {
  const unsigned l = __builtin_amdgcn_readfirstlane(lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "v"(g), "s"(l)
      : "memory");
}
__device__ __forceinline__ void g2lds16_so_at(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned l = __builtin_amdgcn_readfirstlane(lds);
  const unsigned long long b = (unsigned long long)(uintptr_t)sbase;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
  const unsigned long long sb = ((unsigned long long)hi << 32) | lo;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "v"(voff), "s"(sb), "s"(l)
      : "memory");
}
// 4 bytes per lane from a wave-uniform base plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void g2lds4_so_at(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned l = __builtin_amdgcn_readfirstlane(lds);
  const unsigned long long b = (unsigned long long)(uintptr_t)sbase;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
  const unsigned long long sb = ((unsigned long long)hi << 32) | lo;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0\n\ts_nop 0"
      : "=&s"(saved)
      : "v"(voff), "s"(sb), "s"(l)
      : "memory");
}
// LDS byte address of a __shared__ object (a compile-time constant for a
// __shared__ array, so arithmetic on it stays in scalar registers).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// ---------------------------------------------------------------------------
// Padded tiles.  A [rows][128] 16-bit tile staged in LDS with a 272-byte row
// pitch (256 bytes of data, 16 of padding), logical row k in physical row
// prow(k), which swaps the two 2-bit fields of k mod 16 (prow is its own
// inverse).  Every MFMA operand read of a lane is then one base register
// plus a compile-time offset, and the read patterns stay free of bank
// conflicts on 64 four-byte banks:
//  * 16-byte row reads by 16 lanes of 16 consecutive rows: the physical rows
//    are a permutation of 16 consecutive ones, whose starts lie 4 banks
//    apart (272 bytes = 68 banks);
//  * transpose reads (ds_read_b64_tr_b16) by 32 lanes of the rows 4q + i,
//    i < 4, times 4 aligned pieces: the physical rows are 4 apart (16
//    banks), so the four 64-byte row segments tile the 64 banks.
// Direct global -> LDS loads fill a tile in 1-KB slices: byte o holds
// logical row prow(o / 272), piece (o % 272) / 16; padding pieces re-read
// row 0, piece 0 (never read back).  A tile of 32 rows ends half-way into
// its ninth slice, whose upper 32 lanes stay idle.
// ---------------------------------------------------------------------------
constexpr int kPadPitch = 272;
__host__ __device__ constexpr int ptile_bytes(int rows) { return rows * kPadPitch; }
__device__ __forceinline__ int prow(int k) {
  return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3);
}
// The logical row k and 16-byte piece pc that byte o of a padded tile of
// `rows` rows holds.
__device__ __forceinline__ void pslot(int o, int rows, int& k, int& pc) {
  const int r = o / kPadPitch, c = (o - r * kPadPitch) >> 4;
  const bool ok = c < 16 && r < rows;  // r >= rows: lanes of a partial slice
  k = ok ? prow(r) : 0;
  pc = ok ? c : 0;
}
// Base offset of a lane's 16-byte row reads: row lane%32 (a 32-row step is
// +32*272 bytes), piece 2*ds + lane/32 at +32*ds bytes.
__device__ __forceinline__ unsigned prow_base(int lane) {
  return (unsigned)(prow(lane & 31) * kPadPitch + 16 * (lane >> 5));
}
// Base offset of a lane's transpose reads: the k-major operand of rows
// 16*k16 + {4h..4h+3, 8+4h..8+4h+3} (h = lane/32) and column dt*32 +
// lane%32, in the row order of a 32x32 accumulator's elements 8*k2 ..
// 8*k2+7.  The 16-row step is +16*272 bytes, dt is +64, and the second row
// group (+8 rows) lies 2*272 bytes after the first.
__device__ __forceinline__ unsigned ptr_base(int lane) {
  const int g16 = lane >> 4, i16 = lane & 15, h = lane >> 5;
  return (unsigned)((4 * (i16 >> 2) + h) * kPadPitch + (2 * (g16 & 1) + ((i16 & 3) >> 1)) * 16 +
                    8 * (i16 & 1));
}
template <typename V8>
__device__ __forceinline__ V8 ptile_tr(const char* p) {
  return lds_read_tr_pair<V8>(p, p + 2 * kPadPitch);
}

// Staging of a padded tile of R rows by the NW waves of a workgroup: wave w
// loads slices w, w + NW, ...  The per-lane source offsets of a whole tile
// (rows row_bytes apart) are fixed at set-up; a ragged tile clamps its rows.
template <int NW, int R>
struct PStage {
  static constexpr int S = (ptile_bytes(R) + 1023) / 1024;        // slices
  static constexpr int kTail = (ptile_bytes(R) - 1024 * (S - 1)) / 16;  // lanes of the last
  static constexpr int NU = (S + NW - 1) / NW;
  unsigned off[NU];
  __device__ __forceinline__ void init(int wid, int lane, long row_bytes) {
#pragma unroll
    for (int u = 0; u < NU; u++) {
      int k, pc;
      pslot(1024 * (u * NW + wid) + 16 * lane, R, k, pc);
      off[u] = (unsigned)(k * row_bytes) + (unsigned)(16 * pc);
    }
  }
  // rows base, base + row_bytes, ... (wid wave-uniform)
  __device__ __forceinline__ void full(const char* base, unsigned lds, int wid, int lane) const {
#pragma unroll
    for (int u = 0; u < NU; u++) {
      const int sl = u * NW + wid;
      if (sl < S && (kTail == 64 || sl < S - 1 || lane < kTail))
        g2lds16_so_at(base, off[u], lds + 1024 * sl);
    }
  }
  // logical rows past `last` re-read row `last`
  __device__ __forceinline__ void ragged(const char* base, long row_bytes, int last, unsigned lds,
                                         int wid, int lane) const {
#pragma unroll
    for (int u = 0; u < NU; u++) {
      const int sl = u * NW + wid;
      if (sl < S && (kTail == 64 || sl < S - 1 || lane < kTail)) {
        int k, pc;
        pslot(1024 * sl + 16 * lane, R, k, pc);
        g2lds16_at(base + (long)min(k, last) * row_bytes + 16 * pc, lds + 1024 * sl);
      }
    }
  }
};

// Position in a walk over the chunks of a block list: entry e of the list
// and sub-chunk s of that entry (advanced by counting, with no division).
struct ChunkPos {
  int e, s;
};
// A chunk of a walk with its row range [lo, hi), so that the range found
// while looking for the next valid chunk is not computed again.
struct ChunkAt {
  ChunkPos c;
  int lo, hi;
};
__device__ __forceinline__ ChunkPos chunk_advance(ChunkPos c, int per_entry) {
  if (++c.s == per_entry) {
    c.s = 0;
    ++c.e;
  }
  return c;
}

// Wave-uniform lookups into an int32 list (e.g. the column ids of one row of
// a compacted block mask): 64 consecutive entries are held one per lane and
// read back with readlane, so a loop over the list issues no global load per
// step; a lookup outside the held run refills it from there.  Lookups must
// be wave-uniform.
struct ListWindow {
  const int* list;
  int base, hi, val;
  __device__ __forceinline__ ListWindow(const int* l, int lo, int hi_) : list(l), base(lo), hi(hi_) {
    fill();
  }
  __device__ __forceinline__ void fill() {
    const int e = base + (int)(threadIdx.x & 63);
    val = e < hi ? list[e] : 0;
  }
  __device__ __forceinline__ int operator()(int idx) {
    if ((unsigned)(idx - base) >= 64u) {
      base = idx;
      fill();
    }
    return __builtin_amdgcn_readlane(val, idx - base);
  }
};

// 16-byte read of logical piece c of row r from a swizzled tile.
template <typename V8>
__device__ __forceinline__ V8 tile_read16(const char* tile, int r, int c) {
  return lds_read16<V8>(tile + r * 256 + ((c ^ swz(r)) << 4));
}

// k-major operand from a swizzled [rows][128] tile by transpose reads: lane
// l gets column dt*32 + l%32 and rows k16*16 + {4h..4h+3, 8+4h..8+4h+3}
// (h = l/32), the row order that a 32x32 accumulator's elements 8*k2..8*k2+7
// have in their row index (8*(j/4) + 4*h + j%4).
template <typename V8>
__device__ __forceinline__ V8 tile_read_tr(const char* tile, int k16, int dt,
                                          int lane = threadIdx.x & 63) {
  const int g16 = lane >> 4, i16 = lane & 15, h = lane >> 5;
  const int r0 = k16 * 16 + 4 * h + (i16 >> 2);
  const int r1 = r0 + 8;
  const int c = 4 * dt + 2 * (g16 & 1) + ((i16 & 3) >> 1);
  const int b8 = 8 * (i16 & 1);
  return lds_read_tr_pair<V8>(tile + r0 * 256 + ((c ^ swz(r0)) << 4) + b8,
                              tile + r1 * 256 + ((c ^ swz(r1)) << 4) + b8);
}

// Scheduling hint for a stage of NM MFMAs fed by LDS reads: AHEAD reads are
// issued first, then each MFMA is followed by RPM more reads, so the LDS
// latency of later operands hides behind earlier MFMAs.  (Place it after the
// stage's code, in the same basic block.)
template <int NM, int RPM, int AHEAD>
__device__ __forceinline__ void sched_mfma_lds() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
  for (int u = 0; u < NM; u++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Block-wide exclusive scan of one value per thread; returns the exclusive
// prefix, *total gets the block sum.
__device__ __forceinline__ int block_excl_scan(int x, int* total) {
  __shared__ int wsum[16];  // up to 1024 threads
  __shared__ int tot;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int v = lane < nw ? wsum[lane] : 0;
    const int vi = wave_incl_scan(v);
    if (lane < nw) wsum[lane] = vi - v;
    if (lane == nw - 1) tot = vi;
  }
  __syncthreads();
  const int excl = wsum[wid] + incl - x;
  *total = tot;
  __syncthreads();  // wsum / tot are reused by the next call
  return excl;
}

// XCD-aware workgroup -> work-item remap.  Workgroups are dispatched to the 8
// XCDs round-robin (workgroup w runs on XCD w % 8).  Giving XCD x the
// contiguous range [x * per, (x + 1) * per) of the work order keeps the work
// items an XCD runs together adjacent in that order, so their shared K/V
// blocks stay in that XCD's L2.  Returns -1 for the padding workgroups.
__device__ __forceinline__ int xcd_remap(int w, int n_items, int n_xcd = 8) {
  int per = (n_items + n_xcd - 1) / n_xcd;
  int item = (w % n_xcd) * per + (w / n_xcd);
  return item < n_items ? item : -1;
}

// ---------------------------------------------------------------------------
// Element masks (u8, non-zero = excluded) inside a 64-key chunk.
// ---------------------------------------------------------------------------

// Keep bits of one query row over the keys a lane holds in a 64-key chunk
// when keys run along the accumulator's rows: bit 4*c + i stands for key
// offset 8*c + 4*h + i (c = 0..7, i = 0..3) and is set when that entry is
// zero.  `row` points at the chunk's first key in the mask row; offsets at or
// past n are not read and come out cleared.  al4: row and chunk starts are
// 4-byte aligned and rows end on a 4-byte boundary, so four keys load as
// one dword that stays inside the row.
__device__ __forceinline__ uint32_t am_keep_row(const unsigned char* row, int n, int h, int al4) {
  uint32_t keep = 0;
#pragma unroll
  for (int c = 0; c < 8; c++) {
    const int o = 8 * c + 4 * h;
    if (o >= n) continue;
    uint32_t w = 0;
    if (al4) {
      w = *reinterpret_cast<const uint32_t*>(row + o);
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++) w |= (uint32_t)(o + i < n ? row[o + i] : 1) << (8 * i);
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
      keep |= (uint32_t)(((w >> (8 * i)) & 0xffu) == 0 && o + i < n) << (4 * c + i);
  }
  return keep;
}

// Keep bits of one key column over the 16 queries a lane holds in a 32-query
// chunk when queries run along the accumulator's rows: bit j stands for
// query offset 8*(j/4) + 4*h + j%4.  `col` points at the chunk's first query
// row in the key's column; rows are `pitch` bytes apart; offsets at or past n
// are not read and come out cleared.
__device__ __forceinline__ uint32_t am_keep_col(const unsigned char* col, long pitch, int n, int h) {
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const int o = 8 * (j >> 2) + 4 * h + (j & 3);
    if (o < n && col[(long)o * pitch] == 0) keep |= 1u << j;
  }
  return keep;
}

}  // namespace tsa
