// fa_common.hpp - shared device helpers for the gfx950 attention kernels.
//
// MFMA fragment conventions (v_mfma_f32_32x32x16_bf16, wave64), checked on the
// device with a probe of known matrices:
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. 8*(l/32)+7
//   B (16 x 32): lane l holds column l%32, the same k range as A
//   C (32 x 32): lane l, register r holds column l%32,
//                row 8*(r/4) + 4*(l/32) + r%4
// Only the pairing of A's and B's k slots matters for a contraction, so any
// permutation of k applied to both operands is free; the kernels use that to
// feed a C fragment straight back in as a B operand.
//
// LDS tiles hold rows of D bf16 values (D*2 bytes) whose 16-byte chunks are
// permuted per row (chunk ^ swz(row)) so that both the row reads of the score
// product and the transposing reads of the value product hit distinct banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_launch.hpp"   // DropParams

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine x with the value held by lane (l + 32) % 64 (v_permlane32_swap
// exchanges the two half-waves; both results are symmetric in the pair).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round 8 floats to bf16 (nearest even) and pack them as one MFMA operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  bf16x2 p0 = __builtin_convertvector((f32x2){a0, a1}, bf16x2);
  bf16x2 p1 = __builtin_convertvector((f32x2){a2, a3}, bf16x2);
  bf16x2 p2 = __builtin_convertvector((f32x2){a4, a5}, bf16x2);
  bf16x2 p3 = __builtin_convertvector((f32x2){a6, a7}, bf16x2);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}
__device__ __forceinline__ bf16x4 pack_bf16x4(float a0, float a1, float a2, float a3) {
  bf16x2 p0 = __builtin_convertvector((f32x2){a0, a1}, bf16x2);
  bf16x2 p1 = __builtin_convertvector((f32x2){a2, a3}, bf16x2);
  bf16x4 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  return r;
}

// Per-row chunk permutation for a tile with rows of D bf16 values.
//  D = 128 (16 chunks, 256 B a row) and D = 256 (32 chunks, 512 B): the 4 low
//    row bits, rotated by 2, so 16 consecutive rows read at one chunk land in
//    16 different chunk slots, and 4 consecutive rows read over 4 aligned
//    chunks cover 16 different slots.
//  D = 64 (8 chunks, 128 B a row, two rows per 256 B bank window): rows of one
//    parity get 8 different slots for rows 0..15, and rows 2 apart differ in
//    chunk bit 2.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D >= 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

// Byte offset of 16-byte chunk `chunk` of row `row` inside an LDS tile.
template <int D>
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return (uint32_t)(row * (D * 2) + ((chunk ^ swz<D>(row)) << 4));
}

// Byte offset of bf16 element (row, col) inside an LDS tile.
template <int D>
__device__ __forceinline__ uint32_t elem_off(int row, int col) {
  return tile_off<D>(row, col >> 3) + (uint32_t)((col & 7) << 1);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char* base, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

// Transposing LDS read of 4 bf16 values (ds_read_b64_tr_b16).  Within each
// group of 16 lanes, lane i receives element i%4 of the 8-byte rows addressed
// by lanes i/4, 4+i/4, 8+i/4, 12+i/4 of that group, in that order.
__device__ __forceinline__ s16x4 lds_read_tr16(const char* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(base + off));
}

// Compile-time loop: calls f(std::integral_constant<int, i>) for i in [I, N).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const FA_LDS char*)p;
}

// ---- Sync-check build
// Built with -DFA_SYNC_CHECK (libfa_synccheck.so), every asm-issued LDS read
// and every global/buffer -> LDS copy completes before the next instruction,
// and every workgroup barrier first waits for all of the wave's memory
// operations.  No barrier is added or moved: waves of one workgroup take
// different paths in several kernels (ping-pong halves, per-wave causal
// skips), so a barrier anywhere else could deadlock.  The arithmetic is
// unchanged, so kernels whose ordering is right give bit-identical results in
// both builds; a tile read before its copy landed, a copy that overwrites a
// buffer another wave still reads, or an asm read used before its wait shows
// as a difference (the check build lands every copy at once and never leaves
// a read in flight).
#ifdef FA_SYNC_CHECK
constexpr bool kSyncCheck = true;
#define FA_SYNC_CHECK_LDS_WAIT "\n\ts_waitcnt lgkmcnt(0)"
#else
constexpr bool kSyncCheck = false;
#define FA_SYNC_CHECK_LDS_WAIT ""
#endif
__device__ __forceinline__ void sync_check_drain() {
  if constexpr (kSyncCheck) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void sync_check_copy_done() {
  if constexpr (kSyncCheck) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// Workgroup barrier (__syncthreads; in the sync-check build after a full drain).
__device__ __forceinline__ void block_sync() {
  sync_check_drain();
  __syncthreads();
}

// ---- LDS reads issued from inline asm
// The compiler treats the transposing-read builtin as a possible reader of
// every global -> LDS copy still in flight and drains them all (vmcnt(0))
// before each one, so copies issued for later tiles would stall the reads of
// the current tile.  These asm forms are invisible to the compiler's wait
// counters instead, which puts their ordering in the caller's hands:
//  * a value read by lds_*_issue may only be used after lds_wait<n>() with n
//    no larger than the number of asm LDS reads issued after it (LDS returns
//    in order, so the n most recent reads may still be pending; reads the
//    compiler issues in between only make the wait stricter), and after
//    lds_ready() has passed it through (so no use is scheduled earlier);
//  * the data must already be in LDS and visible (the callers read tiles that
//    a barrier after s_waitcnt vmcnt has published).
// The build scans the generated ISA and fails if any instruction touches the
// destination registers of such a read before a wait that retires it.
template <uint32_t OFF>
__device__ __forceinline__ s16x4 lds_tr16_issue(uint32_t addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" FA_SYNC_CHECK_LDS_WAIT : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <uint32_t OFF>
__device__ __forceinline__ bf16x8 lds_b128_issue(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" FA_SYNC_CHECK_LDS_WAIT : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait() {
  static_assert(N >= 0 && N < 16, "lgkmcnt is a 4-bit field");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
}
__device__ __forceinline__ void lds_ready(s16x4& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void lds_ready(bf16x8& x) { asm volatile("" : "+v"(x)); }

// The A operand (tile^T fragment) from a retired pair of transposing reads:
// the low four k values from r[0], the high four from r[1].
__device__ __forceinline__ bf16x8 tr_pair_take(s16x4 (&r)[2]) {
  lds_ready(r[0]);
  lds_ready(r[1]);
  const bf16x4 a = __builtin_bit_cast(bf16x4, r[0]), b = __builtin_bit_cast(bf16x4, r[1]);
  bf16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

// Asynchronous 16-byte global -> LDS copy (global_load_lds_dwordx4): lane l's
// 16 bytes from `src` land at lds_block + 16 l.  `lds_block` must be the same
// for every lane of the wave.  Completion is tracked by vmcnt.
__device__ __forceinline__ void global_to_lds16(const void* src, void* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (FA_LDS void*)lds_block, 16, 0, 0);
  sync_check_copy_done();
}

// Buffer descriptor over `bytes` bytes from `base` (raw, unswizzled dwords);
// loads at offsets >= bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Asynchronous 16-byte buffer -> LDS copy: lane l's 16 bytes at byte offset
// `voff` of the buffer land at lds_block + 16 l (lds_block wave-uniform).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, void* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_LDS void*)lds_block, 16, voff, 0, 0, 0);
  sync_check_copy_done();
}

// Asynchronous 4-byte buffer -> LDS copy: lane l's dword lands at lds_block + 4 l.
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, void* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_LDS void*)lds_block, 4, voff, 0, 0, 0);
  sync_check_copy_done();
}

// Wait until this wave's global loads (including global -> LDS copies) are done.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits until at most N global memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so that each
// XCD runs one contiguous range of logical tiles (neighbouring tiles share the
// same K/V rows and so the same L2).
__device__ __forceinline__ int xcd_remap(int id, int count) {
  const int x = id & 7, slot = id >> 3;
  const int q = count >> 3, r = count & 7;
  return x * q + (x < r ? x : r) + slot;
}

// Maps a hardware workgroup id to (head index bh, tile index) for a grid of
// `ntiles` tiles per head and `bhcount` heads.  Workgroups are dealt to the 8
// XCDs round-robin (id % 8).  When the head count is a multiple of 8, every XCD
// gets bhcount/8 whole heads, whose K/V rows then share that XCD's L2.  Under
// a causal mask the tiles of one XCD go out heaviest first across its heads
// (longest-processing-time order, so no CU is left with a tail of heavy tiles);
// otherwise head by head.  `heavy_high`: the highest tile index carries the
// most work (query tiles that see the most keys); otherwise the lowest (key
// tiles seen by the most queries).
__device__ __forceinline__ void tile_of(int id, int ntiles, int bhcount, bool causal, bool heavy_high,
                                        int& bh, int& tile) {
  int rank;
  if ((bhcount & 7) == 0) {
    const int x = id & 7, s = id >> 3;
    const int hpx = bhcount >> 3;
    if (causal) {
      bh = x * hpx + s % hpx;
      rank = s / hpx;
    } else {
      bh = x * hpx + s / ntiles;
      rank = s - (s / ntiles) * ntiles;
    }
  } else {
    const int L = xcd_remap(id, ntiles * bhcount);
    bh = L / ntiles;
    rank = L - bh * ntiles;
  }
  tile = heavy_high ? ntiles - 1 - rank : rank;
}

// ---- dropout on the probabilities
// The mask is recomputed wherever it is needed, never stored.  Each call of
// Philox4x32-10 (J. K. Salmon et al., "Parallel random numbers: as easy as 1,
// 2, 3", SC 2011) under the 64-bit seed as key yields eight 16-bit fields
// (field f: the low half of word f / 2 for even f, the high half for odd f).
// Element (query row i, key j) of head bh is field 4 ((j >> 3) & 1) + (j & 3)
// of the call on the counter (2 (j >> 4) + ((j >> 2) & 1), i, bh, offset), and
// is kept when that field is >= t = round(p 2^16); a kept probability is
// scaled by 2^16 / (2^16 - t).  (DropParams is declared with the launchers.)

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // One 32 x 32 -> 64-bit product per multiplier (v_mad_u64_u32): on
    // MI355X 1.32x the rate of separate high and low multiplies.
    // The three-way XORs are one v_bitop3_b32 each (truth table 0x96 is
    // a ^ b ^ c); the compiler otherwise emits two XORs.
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
    x0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), x1, k0, 0x96);
    x1 = (uint32_t)p1;
    x2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), x3, k1, 0x96);
    x3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return (u32x4){x0, x1, x2, x3};
}

// Counter word 0 of key j: one call serves the 8 keys j0 + {0..3, 8..11}
// (j0 % 16 in {0, 4}) of one row, key j0 + 8 (f >> 2) + (f & 3) taking field f.
__device__ __forceinline__ uint32_t drop_ctr0(uint32_t j) { return ((j >> 4) << 1) | ((j >> 2) & 1u); }

// Whether field F of a generator output is kept, against thr = t << 16: the
// low half of a word is compared shifted up, the high half in place (the low
// bits under it cannot lift it past a multiple of 2^16).
template <int F>
__device__ __forceinline__ bool drop_keep(const u32x4& w, uint32_t thr) {
  if constexpr ((F & 1) != 0) return w[F >> 1] >= thr;
  else return (w[F >> 1] << 16) >= thr;
}

// The generator call that serves keys j0 + 8 (f >> 2) + (f & 3), f = 0..7, of
// query row `row` in head bh (j0 % 16 in {0, 4}); drop_keep<f> reads key f's
// decision from it.
__device__ __forceinline__ u32x4 drop_word8(const DropParams& dp, int bh, int row, int j0) {
  return philox4x32_10(drop_ctr0((uint32_t)j0), (uint32_t)row, (uint32_t)bh, dp.offset, dp.key0, dp.key1);
}

// Zeroes the dropped ones of the values v[f] of keys j0 + 8 (f >> 2) + (f & 3),
// f = 0..7, of query row `row` in head bh (j0 % 16 in {0, 4}); kept values
// stay as they are (the caller applies inv_keep).  One generator call.
__device__ __forceinline__ void drop_zero8(const DropParams& dp, int bh, int row, int j0, float* v) {
  const u32x4 w = philox4x32_10(drop_ctr0((uint32_t)j0), (uint32_t)row, (uint32_t)bh, dp.offset, dp.key0, dp.key1);
  static_for<0, 8>([&](auto F) {
    constexpr int f = decltype(F)::value;
    v[f] = drop_keep<f>(w, dp.thr) ? v[f] : 0.f;
  });
}

// Keep decision of one element (query row `row`, key `key`) of head bh, as
// a mask of all ones (kept) or zero.
__device__ __forceinline__ uint32_t drop_mask1(const DropParams& dp, int bh, int row, int key) {
  const u32x4 w = philox4x32_10(drop_ctr0((uint32_t)key), (uint32_t)row, (uint32_t)bh, dp.offset, dp.key0, dp.key1);
  const int f = ((key >> 1) & 4) | (key & 3);
  const uint32_t x = (f >> 1) == 0 ? w[0] : (f >> 1) == 1 ? w[1] : (f >> 1) == 2 ? w[2] : w[3];
  return ((f & 1) ? x : (x << 16)) >= dp.thr ? 0xFFFFFFFFu : 0u;
}

// Keep bits of 16 query rows at this lane's key, for layouts where lane l
// holds key kb + l % 32 (kb % 32 == 0) and the rows row0 + 8 (r >> 2) +
// (r & 3), r = 0..15, the same in every lane of a half-wave: bit r of the
// result is the keep bit of row r.  The 8 lanes whose keys share a generator
// call (lane bits 0, 1 and 3 vary; the lane at position p = 4 bit3 + 2 bit1 +
// bit0 holds field p) draw two calls each: position p the rows 2p and 2p + 1,
// 8 keep bits apiece, packed as the 2-bit entry (row 2p, row 2p + 1) of key q
// at bits 2q, 2q + 1.  Three exchanges with lanes l ^ 1, l ^ 2 and l ^ 8
// (DPP; every lane of the wave must be active) transpose that 8 x 8 matrix of
// entries, one index bit per exchange, so each lane ends with the entries of
// its own key: two calls per lane per 16 rows instead of 16.
__device__ __forceinline__ uint32_t drop_bits16(const DropParams& dp, int bh, int key, int row0) {
  const int pos = ((key >> 1) & 4) | (key & 3);
  const uint32_t c0 = drop_ctr0((uint32_t)key);
  uint32_t m = 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 2 * pos + t;
    const u32x4 w = philox4x32_10(c0, (uint32_t)(row0 + 8 * (r >> 2) + (r & 3)), (uint32_t)bh, dp.offset,
                                  dp.key0, dp.key1);
    static_for<0, 8>([&](auto F) {
      constexpr int f = decltype(F)::value;
      m |= drop_keep<f>(w, dp.thr) ? (1u << (2 * f + t)) : 0u;
    });
  }
  // Stage s: bit s of the position and bit s of the entry index trade places.
  auto stage = [&](uint32_t y, int s, uint32_t hi_mask, int sh) __attribute__((always_inline)) {
    return ((pos >> s) & 1) ? (m & hi_mask) | ((y & hi_mask) >> sh) : (m & ~hi_mask) | ((y & ~hi_mask) << sh);
  };
  m = stage((uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false), 0, 0xCCCCu, 2);    // lane ^ 1
  m = stage((uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false), 1, 0xF0F0u, 4);    // lane ^ 2
  m = stage((uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false), 2, 0xFF00u, 8);   // lane ^ 8 (row_ror:8)
  return m;
}

// Keep bit r of a drop_bits16 result as a mask of all ones or zero.
__device__ __forceinline__ uint32_t drop_bit_mask(uint32_t bits, int r) {
  return (uint32_t)((int32_t)(bits << (31 - r)) >> 31);
}

// Bitwise select of two floats by such a mask (one v_bfi_b32).
__device__ __forceinline__ float mask_select(uint32_t m, float kept, float dropped) {
  return __uint_as_float((m & __float_as_uint(kept)) | (~m & __float_as_uint(dropped)));
}

}  // namespace fa
