// fa_bwd.hip - backward of exact attention, bf16 in/out, fp32 accumulation.
//
// Method: the forward kept only O and the per-row logsumexp; the backward
// rebuilds P_ij = exp(scale q_i k_j - LSE_i) tile by tile on chip instead of
// reading a stored P (page "FlashAttention", vagrantpi.github.io PKM note,
// "三招" item 3; page "知识点13 | FlashAttention深度攻略", blog.xiaohack.org,
// section 6; page "Flash Attention 到底做了什么？", guanweilu.cn, section on the
// backward).  The gradient formula printed on the blog page is garbled; the
// kernels use the chain rule of softmax for the loss sum(O * dO):
//   dV = P^T dO,  dP = dO V^T,  D_i = rowsum(dO * O)_i,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three launches on one stream, no atomics (results are bit-reproducible):
//   1. bwd_pre  : workspace = [-D | -LSE log2(e)], streaming O and dO once, so
//                 that P = exp2(c S + nl) is one FMA and one exp per element,
//                 and dP - D comes out of the dP product itself (its
//                 accumulator starts from -D), leaving one multiply for dS.
//   2. bwd_dkdv : one workgroup per 128 keys (32 per wave, K and V of those
//                 keys resident in registers); walks the query tiles that can
//                 see them.  S = Q K^T and dP = dO V^T use 32x32x16 MFMA with
//                 the key as the lane, so P and dS come out in the B-operand
//                 layout of dV^T += dO^T P and dK^T += Q^T dS, whose A operands
//                 are transposing LDS reads of the dO and Q tiles.
//   3. bwd_dq   : one workgroup per 128 queries (32 per wave, Q and dO of those
//                 rows resident); walks the key tiles they can see.  S^T and
//                 dP^T have the query as the lane, so the row statistics are
//                 one scalar per lane, and dS^T feeds dQ^T += K^T dS^T directly.
// fa_backward runs 2 and 3 as one grid (bwd_fused) ordered heaviest first, so
// the two passes share one tail; the split entry points launch them apart.
// At head size 256 (without dropout) both passes run eight-wave tiles whose
// wave pairs hold the same rows (two waves per SIMD instead of one): dQ by a
// score wave and a dQ wave, dK/dV by a P wave and a dS wave without the mask
// and by column halves under it (each the faster form there on MI355X).
// Both passes stage their streamed tiles with buffer -> LDS copies into two
// LDS slots (three or four in the d = 256 role-pair tiles, whose lagging wave
// still reads the previous tile).  At head size 64 these plain loops at three
// waves per SIMD measured faster than software-pipelined forms (the score
// products of the next tile issued ahead of the exp / dS work of the current
// one) at two.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  float* ws;          // [-D (B*H*N) | -LSE*log2(e) (B*H*N)]
  float* dqacc;       // single pass: fp32 dQ / scale, [B, N, H, d] (zeroed before the pass)
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int H, N, ntiles, BH;   // N: query rows per head
  int Nk;             // key rows per head
  int qoff;           // sequence position of query row 0 (causal: Nk - N)
  int64_t bhn;        // B*H*N
  float c;            // scale * log2(e)
  float scale;
  DropParams drop;    // used by the DROP instantiations only
};

// ------------------------------------------------------------------ preprocess
// CH = D/8 lanes share a row, each reading one 16-byte chunk of O and of dO.
// Rows go in [B, H, N] order (the order of the outputs), so a workgroup's
// writes of -D and -LSE log2 e are contiguous and each row read is a whole
// D*2-byte run (in [B, N, H] order each output word was a line of its own).
// A workgroup takes 64 rows: each lane group of CH lanes handles RPT = CH/4
// of them and issues all their loads before the first reduction (at D = 128
// and 256 one row per lane group left the loads too few in flight: 23 against
// 38 us and 30 against 38 us on MI355X).
constexpr int kPreRowsPerWg = 64;

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ o,
                                                      const __bf16* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ ws, int H, int N,
                                                      int64_t rows, int64_t bhn) {
  constexpr int CH = D / 8;
  constexpr int GROUPS = 256 / CH;                 // lane groups per workgroup
  constexpr int RPT = kPreRowsPerWg / GROUPS;      // rows per lane group
  static_assert(RPT * GROUPS == kPreRowsPerWg && RPT >= 1, "rows per workgroup");
  const int grp = threadIdx.x / CH;
  const int ch = threadIdx.x % CH;
  const int64_t row0 = (int64_t)blockIdx.x * kPreRowsPerWg + grp;   // rows row0 + GROUPS i
  bf16x8 x[RPT], y[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int64_t idx = row0 + GROUPS * i;   // output index (b H + h) N + n
    if (idx < rows) {
      const int64_t n = idx % N, bh = idx / N;
      const int64_t h = bh % H, b = bh / H;
      const int64_t r = (b * N + n) * H + h;  // row of the [B, N, H, d] tensors
      x[i] = *reinterpret_cast<const bf16x8*>(o + r * D + ch * 8);
      y[i] = *reinterpret_cast<const bf16x8*>(dout + r * D + ch * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int64_t idx = row0 + GROUPS * i;
    float acc = 0.f;
    if (idx < rows) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[i][e], (float)y[i][e], acc);
    }
#pragma unroll
    for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, CH);
    if (idx < rows && ch == 0) {
      ws[idx] = -acc;
      ws[bhn + idx] = -lse[idx] * kLog2e;
    }
  }
}

// Integer division rounding toward -inf / +inf (b > 0).
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ __forceinline__ int ceil_div(int a, int b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); }

// Lane base for the A operand of a row-major tile read 16 bytes per lane:
// row l%32 (+ 32 j), logical chunk 2 ks + l/32; address = base ^ (ks << 5).
template <int D>
__device__ __forceinline__ uint32_t row_frag_base(int lane) {
  const int hh = lane >> 5, l32 = lane & 31;
  return (uint32_t)(l32 * D * 2) | ((uint32_t)(hh ^ swz<D>(l32)) << 4);
}

// Lane base for the transposing read (A operand = tile^T): within each group of
// 16 lanes, lane i addresses row 4 (l/32) + i/4 and element column
// 16 ((l/16)%2) + 4 (i%4); address = base ^ (64 t [+ 32 for rows + 8]).
template <int D>
__device__ __forceinline__ uint32_t tr_frag_base(int lane) {
  const int ti = lane & 15, tg = lane >> 4;
  const int r4 = (tg >> 1) * 4 + (ti >> 2);
  const int cl = (tg & 1) * 2 + ((ti & 3) >> 1);
  return (uint32_t)(r4 * D * 2) | ((uint32_t)(cl ^ swz<D>(r4)) << 4) | ((uint32_t)(ti & 1) << 3);
}

// A fragment of tile^T: rows d = 32 t + l%32, tile rows 32 j + 16 u + 4 (l/32)
// + {0..3} and the same + 8, matching the B operand built from accumulator
// registers 8u .. 8u+7 of a C fragment of rows 32 j .. 32 j + 31.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, uint32_t base, int t, int j, int u) {
  const uint32_t rowoff = (uint32_t)((32 * j + 16 * u) * D * 2);
  const bf16x4 lo = __builtin_bit_cast(bf16x4, lds_read_tr16(tile, (base ^ (64 * t)) + rowoff));
  const bf16x4 hi = __builtin_bit_cast(bf16x4, lds_read_tr16(tile, (base ^ (64 * t + 32)) + rowoff + 8 * D * 2));
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Per-lane byte offsets of the buffer -> LDS copies of a tile of ROWS rows:
// copy i of a wave fills LDS block (wave + NW i) (NW waves in the
// workgroup); lane l holds physical chunk slot%CH of row slot/CH, i.e.
// logical chunk (slot%CH) ^ swz(row).
template <int D, int CPW, int NW = 4>
__device__ __forceinline__ void stage_offsets(uint32_t (&voff)[CPW], int wave, int lane, int64_t rs) {
  constexpr int CH = D / 8;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int slot = (wave + NW * i) * 64 + lane;
    const int row = slot / CH;
    voff[i] = (uint32_t)(row * rs * 2) + (uint32_t)(((slot % CH) ^ swz<D>(row)) * 16);
  }
}

// Write a C fragment holding rows d of one key/query column (this lane's row
// of the output tensor) scaled by `mul`, as bf16 with round-to-nearest-even.
template <int D>
__device__ __forceinline__ void store_row_frags(__bf16* row, const f32x16* acc, int hh, float mul) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = t * 32 + 8 * g4 + 4 * hh;
      *reinterpret_cast<bf16x4*>(row + d0) =
          pack_bf16x4(acc[t][4 * g4 + 0] * mul, acc[t][4 * g4 + 1] * mul,
                      acc[t][4 * g4 + 2] * mul, acc[t][4 * g4 + 3] * mul);
    }
}

// ------------------------------------------------------------------ dK, dV pass
constexpr int kKeysPerWg = 128;   // 4 waves x 32 keys
// Query rows per step: at D = 64 two 32-row blocks (one barrier and one copy
// batch per 64 rows; the blocks run one after the other in the same
// registers: 2% faster on MI355X, bitwise the same results), else one.  The
// dropout pass keeps one (with two it spills).
template <int D, bool DROP, bool ATOMIC = false>
constexpr int dkdv_rows() { return D == 64 && !DROP && !ATOMIC ? 64 : 32; }

template <int D, bool DROP, bool ATOMIC = false>
constexpr int dkdv_lds_bytes() {
  return 2 * (2 * dkdv_rows<D, DROP, ATOMIC>() * D * 2 + 512);
}

// Single pass (ATOMIC): LDS per wave for its 32 K rows (a swizzled tile, read
// transposed as the B operand of dQ += dS K) and for the dS staging of one
// 32 x 32 block ([query][key] bf16, rows padded to 80 bytes), then the four
// waves' fp32 dQ partials of the block ([wave][query][d]).
constexpr int kStRow = 80;
template <int D>
constexpr int sp_extra_lds_bytes() { return 4 * (32 * D * 2 + 32 * kStRow) + 4 * 32 * D * 4; }

// dK, dV of key tile kt of head bh (one workgroup).  ATOMIC: also the
// contribution of these keys to dQ of every query block the tile visits,
// dQ_blk += dS_blk K (unscaled), added into a.dqacc with fp32 atomics.
template <int D, bool CAUSAL, bool DROP, bool ATOMIC = false>
__device__ __forceinline__ void dkdv_tile(const BwdArgs& a, int bh, int kt, char* smem) {
  constexpr int KS = D / 16, DT = D / 32, RB = D * 2;
  constexpr int kBq = dkdv_rows<D, DROP, ATOMIC>(); // query rows per step
  constexpr int NSUB = kBq / 32;            // 32-row blocks per step
  constexpr int TILE = kBq * RB;            // one Q or dO tile
  constexpr int CPW = TILE / 1024 / 4;      // 1 KB copies per wave per tile
  constexpr int SLOT = 2 * TILE + 512;      // Q, dO, then 64 floats of -LSE log2 e and of D
  static_assert(2 * SLOT == dkdv_lds_bytes<D, DROP, ATOMIC>(), "LDS layout");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, Nk = a.Nk, qoff = a.qoff;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = ((int64_t)b * N * a.H + h) * D;      // Q, dO
  const int64_t kbase = ((int64_t)b * Nk * a.H + h) * D;    // K, V, dK, dV
  const float* dstat = a.ws + (int64_t)bh * N;
  const float* nlstat = a.ws + a.bhn + (int64_t)bh * N;

  const int k0 = kt * kKeysPerWg;
  const int kw0 = k0 + 32 * wave;
  const int mykey = kw0 + l32;

  // K^T and V^T as B operands: this lane's key, chunk 2 ks + hh.
  bf16x8 kf[KS], vf[KS];
  {
    const int64_t kr = min(mykey, Nk - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(a.k + kbase + kr * rs + (2 * ks + hh) * 8);
      vf[ks] = *reinterpret_cast<const bf16x8*>(a.v + kbase + kr * rs + (2 * ks + hh) * 8);
    }
  }
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) { dk[t] = (f32x16){}; dv[t] = (f32x16){}; }
  // Single pass: this wave's K rows as a tile (row l32 = key kw0 + l32) and
  // its dS^T staging area, after the two slots of the step loop.  The first
  // step's barrier orders these stores before any read.  Rows of keys past
  // Nk are zero: their fragments hold a copy of the last key, whose dS is not
  // zero, and only the zero row keeps them out of dQ.
  char* const ktile = smem + dkdv_lds_bytes<D, DROP, ATOMIC>() + __builtin_amdgcn_readfirstlane(wave) * (32 * RB);
  char* const stage_st = smem + dkdv_lds_bytes<D, DROP, ATOMIC>() + 4 * 32 * RB +
                         __builtin_amdgcn_readfirstlane(wave) * (32 * kStRow);
  float* const dq_part = reinterpret_cast<float*>(smem + dkdv_lds_bytes<D, DROP, ATOMIC>() + 4 * (32 * RB + 32 * kStRow));
  f32x16 dqw[DT];   // single pass: this wave's dQ partial of the step's block
  if constexpr (ATOMIC) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      *reinterpret_cast<bf16x8*>(ktile + tile_off<D>(l32, 2 * ks + hh)) = mykey < Nk ? kf[ks] : (bf16x8){};
  }

  // Under the mask query row i (sequence position i + qoff) sees keys up to
  // i + qoff: the first row that can see key k0 is k0 - qoff.
  const int qstart = CAUSAL ? max(0, k0 - qoff) : 0;
  const int nsteps = (N - qstart + kBq - 1) / kBq;

  uint32_t voff[CPW];
  stage_offsets<D, CPW>(voff, wave, lane, rs);
  // Wave-uniform (scalar) copy of the wave index for LDS destinations, which
  // must be uniform.
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  // Copies of query tile s (rows past N and statistics past N read as zero).
  auto stage = [&](int s, char* slot) {
    const int qi0 = qstart + s * kBq;
    const int rows = min(N - qi0, kBq);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + base + (int64_t)qi0 * rs, (uint32_t)(rows * rs * 2));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.dout + base + (int64_t)qi0 * rs, (uint32_t)(rows * rs * 2));
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      buffer_to_lds16(rq, voff[i], slot + (wu + 4 * i) * 1024);
      buffer_to_lds16(rg, voff[i], slot + TILE + (wu + 4 * i) * 1024);
    }
    if (wu == 0)
      buffer_to_lds4(make_rsrc(nlstat + qi0, (uint32_t)(rows * 4)), lane * 4, slot + 2 * TILE);
    else if (wu == 1)
      buffer_to_lds4(make_rsrc(dstat + qi0, (uint32_t)(rows * 4)), lane * 4, slot + 2 * TILE + 256);
  };

  const uint32_t rfb = row_frag_base<D>(lane);
  const uint32_t tfb = tr_frag_base<D>(lane);
  // S = Q K^T and dP = dO V^T for 32-row block sb of a tile: lane = key,
  // register r = query row 32 sb + 8(r/4) + 4hh + r%4 (the row swizzle
  // repeats every 16 rows, so block sb is the lane base plus a row offset).
  // The dP product starts from -D of each query row, so pacc ends as dP - D
  // (with dropout from 0: pacc = dP).
  auto scores = [&](const char* slot, int sb, f32x16& sacc, f32x16& pacc) __attribute__((always_inline)) {
    sacc = (f32x16){};
    if constexpr (DROP) {
      pacc = (f32x16){};
    } else {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 nd = *reinterpret_cast<const f32x4*>(slot + 2 * TILE + 256 + (32 * sb + 8 * g4 + 4 * hh) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) pacc[4 * g4 + e] = nd[e];
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sacc = mfma32x32x16(lds_read_b128(slot, (rfb ^ (ks << 5)) + 32 * sb * RB), kf[ks], sacc);
      pacc = mfma32x32x16(lds_read_b128(slot + TILE, (rfb ^ (ks << 5)) + 32 * sb * RB), vf[ks], pacc);
    }
  };
  const float c = a.c;
  // P, dS for 32-row block sb (rows qi0 ..) of a query tile and the dV, dK updates.
  auto update = [&](auto mask_tag, const char* slot, int sb, const f32x16& sacc, const f32x16& pacc, int qi0)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // Keep bits of this lane's 16 rows of the block (bit 4 g4 + e: row qi0 +
    // 8 g4 + 4 hh + e); lane l32 holds key kw0 + l32 with kw0 % 32 == 0.  (At
    // D = 256 the DPP exchange makes this ROCm 7.2 compiler crash in its AGPR
    // rewrite pass; that head size draws each element on its own.)
    uint32_t dbits = 0;
    if constexpr (DROP && D <= 128) dbits = drop_bits16(a.drop, bh, mykey, qi0 + 4 * hh);
    // Query rows 16 u .. 16 u + 15 of the tile (registers 8u .. 8u+7) at a time.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float p[8], ds[8];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int g4 = 2 * u + g;
        const f32x4 nl = *reinterpret_cast<const f32x4*>(slot + 2 * TILE + (32 * sb + 8 * g4 + 4 * hh) * 4);
        f32x4 nd;
        uint32_t km[4];   // keep masks (all ones: kept)
        if constexpr (DROP) {
          nd = *reinterpret_cast<const f32x4*>(slot + 2 * TILE + 256 + (32 * sb + 8 * g4 + 4 * hh) * 4);
          if constexpr (D <= 128) {
#pragma unroll
            for (int e = 0; e < 4; ++e) km[e] = drop_bit_mask(dbits, 4 * g4 + e);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) km[e] = drop_mask1(a.drop, bh, qi0 + 8 * g4 + 4 * hh + e, mykey);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float pv = fast_exp2(__builtin_fmaf(sacc[r], c, nl[e]));
          if constexpr (MASK) {
            const int qrow = qi0 + 8 * g4 + 4 * hh + e;
            const bool hide = qrow >= N || (CAUSAL && mykey > qrow + qoff);
            pv = hide ? 0.f : pv;
          }
          if constexpr (DROP) {
            // dV takes P of the kept elements (the keep multiplier s is
            // applied when dV is stored); dS = P (z dP - D) with pacc = dP:
            // P (s dP - D) where kept, -P D where dropped.
            p[4 * g + e] = __uint_as_float(km[e] & __float_as_uint(pv));
            ds[4 * g + e] = pv * mask_select(km[e], __builtin_fmaf(a.drop.inv_keep, pacc[r], nd[e]), nd[e]);
          } else {
            p[4 * g + e] = pv;
            ds[4 * g + e] = pv * pacc[r];
          }
        }
      }
      const bf16x8 pb = pack_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      const bf16x8 db = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      // dV^T += dO^T P ; dK^T += Q^T dS   (rows d, columns keys)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        dv[t] = mfma32x32x16(tr_frag<D>(slot + TILE, tfb, t, sb, u), pb, dv[t]);
        dk[t] = mfma32x32x16(tr_frag<D>(slot, tfb, t, sb, u), db, dk[t]);
      }
      if constexpr (ATOMIC) {
        // dS^T staging: element (query 16u + 8g + 4hh + e, key l32) of the block
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<__bf16*>(stage_st + (16 * u + 8 * g + 4 * hh + e) * kStRow + l32 * 2) = db[4 * g + e];
      }
    }
    if constexpr (ATOMIC) {
      // dQ (rows queries, columns d) += dS K over this wave's 32 keys: the
      // staged dS rows are the A operand, and the transposing reads of the K
      // tile (the A operand of K^T elsewhere) have the B operand's layout.
      // Lanes of the result then run along d, so each atomic instruction
      // covers two 128-byte rows of the accumulator.
      // The staging was written by this wave alone; its LDS accesses complete
      // in issue order, the asm barrier keeps the compiler from moving the
      // reads above the writes.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int t = 0; t < DT; ++t) dqw[t] = (f32x16){};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // A operand, lane = query l32: keys 16u + 4hh + 0..3 and 16u + 8 + 4hh + 0..3,
        // the key order of tr_frag's fragment
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(stage_st + l32 * kStRow + (16 * u + 4 * hh) * 2);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(stage_st + l32 * kStRow + (16 * u + 8 + 4 * hh) * 2);
        bf16x8 bq;
        bq[0] = lo[0]; bq[1] = lo[1]; bq[2] = lo[2]; bq[3] = lo[3];
        bq[4] = hi[0]; bq[5] = hi[1]; bq[6] = hi[2]; bq[7] = hi[3];
#pragma unroll
        for (int t = 0; t < DT; ++t) dqw[t] = mfma32x32x16(bq, tr_frag<D>(ktile, tfb, t, 0, u), dqw[t]);
      }
      asm volatile("" ::: "memory");
    }
  };
  // One step: publish query tile s, copy tile s+1, then (MODE 1: unmasked,
  // MODE 2: masked; MODE 0: none of the step's rows sees this wave's keys)
  // S, dP, P, dS and the dV, dK updates.
  auto step = [&](int s, auto mode_tag) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    char* slot = smem + (s & 1) * SLOT;
    wait_vmem();
    block_sync();
    if (s + 1 < nsteps) stage(s + 1, smem + ((s + 1) & 1) * SLOT);
    const int qi0 = qstart + s * kBq;
    if constexpr (MODE != 0) {
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        // masked steps: skip blocks past N or with no row that sees this
        // wave's keys (wave-uniform)
        if constexpr (MODE == 2 && NSUB > 1)
          if (qi0 + 32 * sb >= N || (CAUSAL && qi0 + 32 * sb + 31 + qoff < kw0)) continue;
        f32x16 sacc, pacc;
        scores(slot, sb, sacc, pacc);
        update(std::bool_constant<MODE == 2>{}, slot, sb, sacc, pacc, qi0 + 32 * sb);
      }
    } else if constexpr (ATOMIC) {
#pragma unroll
      for (int t = 0; t < DT; ++t) dqw[t] = (f32x16){};
    }
    if constexpr (ATOMIC) {
      // The block's dQ partials of the four waves (lane: d = 32 t + l32,
      // register r: query 8 (r / 4) + 4 hh + r % 4) meet in LDS; wave w sums
      // query rows 8 w .. 8 w + 7 and adds them to the accumulator, each
      // atomic instruction covering one row's D contiguous floats.  The next
      // step's barrier keeps the partials until every wave has read them.
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dq_part[(wave * 32 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + 32 * t + l32] = dqw[t][r];
      block_sync();
#pragma unroll
      for (int i = 0; i < 8 * D / 64; ++i) {
        const int idx = i * 64 + lane;
        const int row = 8 * wave + idx / D, col = idx % D;
        const float sum = (dq_part[row * D + col] + dq_part[(32 + row) * D + col]) +
                          (dq_part[(64 + row) * D + col] + dq_part[(96 + row) * D + col]);
        if (qi0 + row < N)
          __hip_atomic_fetch_add(a.dqacc + base + (int64_t)(qi0 + row) * rs + col, sum, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  // The steps run in sections whose loop bodies have one update path (with
  // the masked and the unmasked update behind a branch inside one loop, the
  // compiler kept dK and dV in several register sets and copied them every
  // step):
  //   [0, s_vis)        no row of the step sees this wave's keys (causal)
  //   [s_vis, s_unm)    the step straddles the diagonal: masked
  //   [s_unm, nfull)    every row sees every key of the wave: unmasked
  //   [.., nsteps)      the step has rows past N: masked
  const int nfull = (N - qstart) / kBq;
  int s_vis = 0, s_unm = 0;
  if constexpr (CAUSAL) {
    // step s: rows qi0 .. qi0 + kBq - 1 (qi0 = qstart + s kBq) at positions + qoff;
    // visible when qi0 + kBq - 1 + qoff >= kw0, unmasked when qi0 + qoff >= kw0 + 31.
    s_vis = min(nsteps, max(0, ceil_div(kw0 - qoff - (kBq - 1) - qstart, kBq)));
    s_unm = min(nsteps, max(s_vis, ceil_div(kw0 + 31 - qoff - qstart, kBq)));
    s_vis = __builtin_amdgcn_readfirstlane(s_vis);
    s_unm = __builtin_amdgcn_readfirstlane(s_unm);
  }
  using M0 = std::integral_constant<int, 0>;
  using M1 = std::integral_constant<int, 1>;
  using M2 = std::integral_constant<int, 2>;
  stage(0, smem);
  int s = 0;
  for (; s < s_vis; ++s) step(s, M0{});
  for (; s < s_unm; ++s) step(s, M2{});
  for (; s < nfull; ++s) step(s, M1{});
  for (; s < nsteps; ++s) step(s, M2{});

  if (mykey < Nk) {
    store_row_frags<D>(a.dk + kbase + (int64_t)mykey * rs, dk, hh, a.scale);
    store_row_frags<D>(a.dv + kbase + (int64_t)mykey * rs, dv, hh, DROP ? a.drop.inv_keep : 1.f);
  }
}

// ------------------------------------------------------------------ d = 256: wave pairs with split roles
// At d = 256 the dK and dV accumulators of 32 keys alone take 256 registers
// of a wave, which leaves one wave per SIMD and nothing to hide its
// latencies.  Here eight waves share the 128-key tile: waves w and w + 4 hold
// the same 32 keys (two waves per SIMD) and divide the one-wave tile's work
// by role:
//  * the P wave (w) holds K, forms S = Q K^T and P = exp2(c S - LSE log2 e),
//    hands P to its partner through LDS as fp32 and accumulates dV^T += dO^T P;
//  * the dS wave (w + 4) holds V, forms dP - D = dO V^T - D, and one step
//    later, with that step's P from its partner, dS = P (dP - D) and
//    dK^T += Q^T dS.
// Every product and elementwise operation is the one-wave tile's, in the same
// order, so dK and dV are bitwise those of the one-wave tile.  The dS wave
// runs one step behind, which puts the two waves of a SIMD out of phase (the
// exponentials of one beside the products of the other), and the query tiles
// rotate through three LDS slots: tile s + 1 is copied while the P wave reads
// tile s and the dS wave tiles s - 1 and s.  One barrier per step.  The
// launchers take this tile without the causal mask; under it the
// column-split tile below measured faster.
constexpr int kPairWaves = 8;
constexpr int kPBytes = 4 * 64 * 16 * 4;   // P of one step: 4 pairs x 64 lanes x 16 floats

template <int D>
constexpr int dkdv_pair_lds_bytes() { return 3 * (2 * 32 * D * 2 + 512) + 2 * kPBytes; }

// dK, dV of key tile kt of head bh by wave pairs (eight waves, 32 query rows
// per step).
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_tile_pair(const BwdArgs& a, int bh, int kt, char* smem) {
  constexpr int KS = D / 16, DT = D / 32, RB = D * 2;
  constexpr int kBq = 32;
  constexpr int TILE = kBq * RB;            // one Q or dO tile
  constexpr int CPW = TILE / 1024 / kPairWaves;
  constexpr int SLOT = 2 * TILE + 512;      // Q, dO, then 64 floats of -LSE log2 e and of -D
  static_assert(CPW * kPairWaves * 1024 == TILE, "the copies cover the tile");
  static_assert(3 * SLOT + 2 * kPBytes == dkdv_pair_lds_bytes<D>(), "LDS layout");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int kg = wave & 3;                                        // key group
  const int role = __builtin_amdgcn_readfirstlane(wave >> 2);    // 0: P wave, 1: dS wave
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, Nk = a.Nk, qoff = a.qoff;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = ((int64_t)b * N * a.H + h) * D;      // Q, dO
  const int64_t kbase = ((int64_t)b * Nk * a.H + h) * D;    // K, V, dK, dV
  const float* dstat = a.ws + (int64_t)bh * N;
  const float* nlstat = a.ws + a.bhn + (int64_t)bh * N;

  const int k0 = kt * kKeysPerWg;
  const int kw0 = k0 + 32 * kg;
  const int mykey = kw0 + l32;
  const int64_t krow = kbase + (int64_t)min(mykey, Nk - 1) * rs;

  const int qstart = CAUSAL ? max(0, k0 - qoff) : 0;
  const int nsteps = (N - qstart + kBq - 1) / kBq;

  auto slot_of = [&](int s) { return smem + (s % 3) * SLOT; };
  // P of step s: float4 64 g4 + lane of this pair's area holds registers
  // 4 g4 .. 4 g4 + 3 of the lane (the same lane layout in both waves).
  auto pbuf = [&](int s) {
    return reinterpret_cast<f32x4*>(smem + 3 * SLOT + (s & 1) * kPBytes) + kg * 4 * 64;
  };
  uint32_t voff[CPW];
  stage_offsets<D, CPW, kPairWaves>(voff, wave, lane, rs);
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  auto stage = [&](int s) {
    char* slot = slot_of(s);
    const int qi0 = qstart + s * kBq;
    const int rows = min(N - qi0, kBq);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + base + (int64_t)qi0 * rs, (uint32_t)(rows * rs * 2));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.dout + base + (int64_t)qi0 * rs, (uint32_t)(rows * rs * 2));
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      buffer_to_lds16(rq, voff[i], slot + (wu + kPairWaves * i) * 1024);
      buffer_to_lds16(rg, voff[i], slot + TILE + (wu + kPairWaves * i) * 1024);
    }
    if (wu == 0)
      buffer_to_lds4(make_rsrc(nlstat + qi0, (uint32_t)(rows * 4)), lane * 4, slot + 2 * TILE);
    else if (wu == 1)
      buffer_to_lds4(make_rsrc(dstat + qi0, (uint32_t)(rows * 4)), lane * 4, slot + 2 * TILE + 256);
  };
  // Start of step s for every wave: tile s published, tile s + 1 on its way.
  auto sync_stage = [&](int s) {
    wait_vmem();
    block_sync();
    if (s + 1 < nsteps) stage(s + 1);
  };
  const uint32_t rfb = row_frag_base<D>(lane);
  const uint32_t tfb = tr_frag_base<D>(lane);
  const float c = a.c;

  // Sections of steps (see dkdv_tile): [0, s_vis) no row sees this pair's
  // keys, [s_vis, s_unm) masked, [s_unm, nfull) unmasked, [nfull, nsteps)
  // masked (rows past N).
  const int nfull = (N - qstart) / kBq;
  int s_vis = 0, s_unm = 0;
  if constexpr (CAUSAL) {
    s_vis = min(nsteps, max(0, ceil_div(kw0 - qoff - (kBq - 1) - qstart, kBq)));
    s_unm = min(nsteps, max(s_vis, ceil_div(kw0 + 31 - qoff - qstart, kBq)));
    s_vis = __builtin_amdgcn_readfirstlane(s_vis);
    s_unm = __builtin_amdgcn_readfirstlane(s_unm);
  }
  stage(0);
  if (role == 0) {
    // K^T as B operand: this lane's key, chunk 2 ks + hh.
    bf16x8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(a.k + krow + (2 * ks + hh) * 8);
    f32x16 dv[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dv[t] = (f32x16){};
    // S (lane = key, register r = query row 8(r/4) + 4hh + r%4), P, its
    // publication and the dV update for step s.
    auto p_step = [&](int s, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const char* slot = slot_of(s);
      const int qi0 = qstart + s * kBq;
      f32x16 sacc = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc = mfma32x32x16(lds_read_b128(slot, rfb ^ (ks << 5)), kf[ks], sacc);
      f32x4* const po = pbuf(s);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float p[8];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int g4 = 2 * u + g;
          const f32x4 nl = *reinterpret_cast<const f32x4*>(slot + 2 * TILE + (8 * g4 + 4 * hh) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pv = fast_exp2(__builtin_fmaf(sacc[4 * g4 + e], c, nl[e]));
            if constexpr (MASK) {
              const int qrow = qi0 + 8 * g4 + 4 * hh + e;
              const bool hide = qrow >= N || (CAUSAL && mykey > qrow + qoff);
              pv = hide ? 0.f : pv;
            }
            p[4 * g + e] = pv;
          }
          po[64 * g4 + lane] = (f32x4){p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
        }
        const bf16x8 pb = pack_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        // dV^T += dO^T P (rows d, columns keys)
#pragma unroll
        for (int t = 0; t < DT; ++t) dv[t] = mfma32x32x16(tr_frag<D>(slot + TILE, tfb, t, 0, u), pb, dv[t]);
      }
    };
    int s = 0;
    for (; s < s_vis; ++s) sync_stage(s);
    for (; s < s_unm; ++s) { sync_stage(s); p_step(s, std::true_type{}); }
    for (; s < nfull; ++s) { sync_stage(s); p_step(s, std::false_type{}); }
    for (; s < nsteps; ++s) { sync_stage(s); p_step(s, std::true_type{}); }
    block_sync();   // the dS wave reads the last step's P after this barrier
    if (mykey < Nk) store_row_frags<D>(a.dv + krow, dv, hh, 1.f);
  } else {
    bf16x8 vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) vf[ks] = *reinterpret_cast<const bf16x8*>(a.v + krow + (2 * ks + hh) * 8);
    f32x16 dk[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dk[t] = (f32x16){};
    f32x16 pacc;   // dP - D of the step whose P has not arrived yet
    // dP - D for step s: the product starts from -D of each query row.
    auto dp_step = [&](int s) __attribute__((always_inline)) {
      const char* slot = slot_of(s);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 nd = *reinterpret_cast<const f32x4*>(slot + 2 * TILE + 256 + (8 * g4 + 4 * hh) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) pacc[4 * g4 + e] = nd[e];
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        pacc = mfma32x32x16(lds_read_b128(slot + TILE, rfb ^ (ks << 5)), vf[ks], pacc);
    };
    // dS = P (dP - D) with step s's P from the partner, and the dK update.
    auto dk_step = [&](int s) __attribute__((always_inline)) {
      const char* slot = slot_of(s);
      const f32x4* const pi = pbuf(s);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float ds[8];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int g4 = 2 * u + g;
          const f32x4 pv = pi[64 * g4 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[4 * g + e] = pv[e] * pacc[4 * g4 + e];
        }
        const bf16x8 db = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
        // dK^T += Q^T dS (rows d, columns keys)
#pragma unroll
        for (int t = 0; t < DT; ++t) dk[t] = mfma32x32x16(tr_frag<D>(slot, tfb, t, 0, u), db, dk[t]);
      }
    };
    int s = 0;
    for (; s < s_vis; ++s) sync_stage(s);
    if (s < nsteps) {
      sync_stage(s);
      dp_step(s);
      for (++s; s < nsteps; ++s) {
        sync_stage(s);
        dk_step(s - 1);
        dp_step(s);
      }
      block_sync();
      dk_step(nsteps - 1);
    } else {
      block_sync();
    }
    if (mykey < Nk) store_row_frags<D>(a.dk + krow, dk, hh, a.scale);
  }
}

// ------------------------------------------------------------------ d = 256: columns split over wave pairs
// At d = 256 the dK and dV accumulators of 32 keys alone take 256 registers
// of a wave, which leaves one wave per SIMD and nothing to hide one wave's
// latencies.  Here eight waves share the 128-key tile: waves w and w + 4
// hold the same 32 keys, wave w columns 0 .. 127 and wave w + 4 columns
// 128 .. 255 of K, V, dK and dV (two waves per SIMD).  Each forms its
// columns' part of S = Q K^T and dP = dO V^T, the two parts meet in LDS as
// fp32, and both waves go on from the same sums (a + b and b + a are the
// same fp32 value); each then updates its own columns of dV and dK.  The
// launchers take this tile under the causal mask.
constexpr int kSplitWaves = kPairWaves;   // launched by the same eight-wave kernels
constexpr int kXchgBytes = kSplitWaves * 64 * 32 * 4;   // 32 floats per lane and wave

template <int D>
constexpr int dkdv_split_lds_bytes() { return 2 * (2 * 32 * D * 2 + 512) + kXchgBytes; }

// Barrier once this wave's LDS stores have completed.  Global -> LDS copies
// still in flight are not waited for (__syncthreads would drain them).
__device__ __forceinline__ void lds_store_barrier() {
  sync_check_drain();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// This wave's partial S and dP go to its exchange slot (lane-major float4s:
// slot row r4 of lane l at float4 index 64 r4 + l, rows 0-3 S, 4-7 dP).
__device__ __forceinline__ void xchg_put(f32x4* slot, int lane, const f32x16& s, const f32x16& p) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    slot[64 * r4 + lane] = (f32x4){s[4 * r4], s[4 * r4 + 1], s[4 * r4 + 2], s[4 * r4 + 3]};
    slot[64 * (4 + r4) + lane] = (f32x4){p[4 * r4], p[4 * r4 + 1], p[4 * r4 + 2], p[4 * r4 + 3]};
  }
}
// Adds the partner's partial S and dP from its exchange slot.
__device__ __forceinline__ void xchg_add(const f32x4* slot, int lane, f32x16& s, f32x16& p) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const f32x4 os = slot[64 * r4 + lane], op = slot[64 * (4 + r4) + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[4 * r4 + e] += os[e];
      p[4 * r4 + e] += op[e];
    }
  }
}

// dK, dV of key tile kt of head bh with the columns split over wave pairs
// (eight waves, 32 query rows per step).
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_tile_split(const BwdArgs& a, int bh, int kt, char* smem) {
  constexpr int DH = D / 2;                 // columns per wave
  constexpr int KS = DH / 16, DT = DH / 32, RB = D * 2;
  constexpr int kBq = 32;
  constexpr int TILE = kBq * RB;            // one Q or dO tile
  constexpr int CPW = TILE / 1024 / kSplitWaves;
  constexpr int SLOT = 2 * TILE + 512;      // Q, dO, then 64 floats of -LSE log2 e and of -D
  static_assert(CPW * kSplitWaves * 1024 == TILE, "the copies cover the tile");
  static_assert(2 * SLOT + kXchgBytes == dkdv_split_lds_bytes<D>(), "LDS layout");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int kg = wave & 3;                                       // key group
  const int dh = __builtin_amdgcn_readfirstlane(wave >> 2);     // column half
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, Nk = a.Nk, qoff = a.qoff;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = ((int64_t)b * N * a.H + h) * D;      // Q, dO
  const int64_t kbase = ((int64_t)b * Nk * a.H + h) * D;    // K, V, dK, dV
  const float* dstat = a.ws + (int64_t)bh * N;
  const float* nlstat = a.ws + a.bhn + (int64_t)bh * N;
  f32x4* const xmine = reinterpret_cast<f32x4*>(smem + 2 * SLOT) + wave * 8 * 64;
  const f32x4* const xpeer = reinterpret_cast<const f32x4*>(smem + 2 * SLOT) + (wave ^ 4) * 8 * 64;

  const int k0 = kt * kKeysPerWg;
  const int kw0 = k0 + 32 * kg;
  const int mykey = kw0 + l32;

  // K^T and V^T as B operands: this lane's key, chunk 2 ks + hh of the half.
  bf16x8 kf[KS], vf[KS];
  {
    const int64_t kr = kbase + (int64_t)min(mykey, Nk - 1) * rs + dh * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(a.k + kr + (2 * ks + hh) * 8);
      vf[ks] = *reinterpret_cast<const bf16x8*>(a.v + kr + (2 * ks + hh) * 8);
    }
  }
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) { dk[t] = (f32x16){}; dv[t] = (f32x16){}; }

  const int qstart = CAUSAL ? max(0, k0 - qoff) : 0;
  const int nsteps = (N - qstart + kBq - 1) / kBq;

  uint32_t voff[CPW];
  stage_offsets<D, CPW, kSplitWaves>(voff, wave, lane, rs);
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  auto stage = [&](int s, char* slot) {
    const int qi0 = qstart + s * kBq;
    const int rows = min(N - qi0, kBq);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + base + (int64_t)qi0 * rs, (uint32_t)(rows * rs * 2));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.dout + base + (int64_t)qi0 * rs, (uint32_t)(rows * rs * 2));
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      buffer_to_lds16(rq, voff[i], slot + (wu + kSplitWaves * i) * 1024);
      buffer_to_lds16(rg, voff[i], slot + TILE + (wu + kSplitWaves * i) * 1024);
    }
    if (wu == 0)
      buffer_to_lds4(make_rsrc(nlstat + qi0, (uint32_t)(rows * 4)), lane * 4, slot + 2 * TILE);
    else if (wu == 1)
      buffer_to_lds4(make_rsrc(dstat + qi0, (uint32_t)(rows * 4)), lane * 4, slot + 2 * TILE + 256);
  };

  // Fragment bases moved to this wave's columns: byte bit 8 of both bases is
  // zero (the chunk swizzle stays below chunk 16), so + 256 dh selects logical
  // chunks 16 dh .. 16 dh + 15 under every XOR the reads apply.
  const uint32_t rfb = row_frag_base<D>(lane) + (uint32_t)(dh * DH * 2);
  const uint32_t tfb = tr_frag_base<D>(lane) + (uint32_t)(dh * DH * 2);
  // This half's part of S = Q K^T and dP = dO V^T (lane = key, register r =
  // query row 8(r/4) + 4hh + r%4); half 0's dP starts from -D of each row, so
  // the sum of the halves is dP - D.
  auto scores = [&](const char* slot, f32x16& sacc, f32x16& pacc) __attribute__((always_inline)) {
    sacc = (f32x16){};
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 nd = *reinterpret_cast<const f32x4*>(slot + 2 * TILE + 256 + (8 * g4 + 4 * hh) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) pacc[4 * g4 + e] = dh == 0 ? nd[e] : 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sacc = mfma32x32x16(lds_read_b128(slot, rfb ^ (ks << 5)), kf[ks], sacc);
      pacc = mfma32x32x16(lds_read_b128(slot + TILE, rfb ^ (ks << 5)), vf[ks], pacc);
    }
  };
  const float c = a.c;
  // P, dS of the step's rows (qi0 ..) and this half's dV, dK updates.
  auto update = [&](auto mask_tag, const char* slot, const f32x16& sacc, const f32x16& pacc, int qi0)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float p[8], ds[8];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int g4 = 2 * u + g;
        const f32x4 nl = *reinterpret_cast<const f32x4*>(slot + 2 * TILE + (8 * g4 + 4 * hh) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float pv = fast_exp2(__builtin_fmaf(sacc[r], c, nl[e]));
          if constexpr (MASK) {
            const int qrow = qi0 + 8 * g4 + 4 * hh + e;
            const bool hide = qrow >= N || (CAUSAL && mykey > qrow + qoff);
            pv = hide ? 0.f : pv;
          }
          p[4 * g + e] = pv;
          ds[4 * g + e] = pv * pacc[r];
        }
      }
      const bf16x8 pb = pack_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      const bf16x8 db = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        dv[t] = mfma32x32x16(tr_frag<D>(slot + TILE, tfb, t, 0, u), pb, dv[t]);
        dk[t] = mfma32x32x16(tr_frag<D>(slot, tfb, t, 0, u), db, dk[t]);
      }
    }
  };
  // One step (MODE 1 unmasked, 2 masked, 0 no row sees this pair's keys):
  // publish query tile s and copy tile s + 1, the partial products, the
  // exchange, then P, dS and the updates.  Every wave passes both barriers of
  // every step, whatever its mode.  The exchange slots are rewritten only
  // after the next step's first barrier, which the partner passes once it
  // has read them.
  auto step = [&](int s, auto mode_tag) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    char* slot = smem + (s & 1) * SLOT;
    wait_vmem();
    block_sync();
    if (s + 1 < nsteps) stage(s + 1, smem + ((s + 1) & 1) * SLOT);
    f32x16 sacc, pacc;
    if constexpr (MODE != 0) {
      scores(slot, sacc, pacc);
      xchg_put(xmine, lane, sacc, pacc);
    }
    lds_store_barrier();
    if constexpr (MODE != 0) {
      xchg_add(xpeer, lane, sacc, pacc);
      update(std::bool_constant<MODE == 2>{}, slot, sacc, pacc, qstart + s * kBq);
    }
  };
  // Sections with one update path each, as in dkdv_tile.
  const int nfull = (N - qstart) / kBq;
  int s_vis = 0, s_unm = 0;
  if constexpr (CAUSAL) {
    s_vis = min(nsteps, max(0, ceil_div(kw0 - qoff - (kBq - 1) - qstart, kBq)));
    s_unm = min(nsteps, max(s_vis, ceil_div(kw0 + 31 - qoff - qstart, kBq)));
    s_vis = __builtin_amdgcn_readfirstlane(s_vis);
    s_unm = __builtin_amdgcn_readfirstlane(s_unm);
  }
  using M0 = std::integral_constant<int, 0>;
  using M1 = std::integral_constant<int, 1>;
  using M2 = std::integral_constant<int, 2>;
  stage(0, smem);
  int s = 0;
  for (; s < s_vis; ++s) step(s, M0{});
  for (; s < s_unm; ++s) step(s, M2{});
  for (; s < nfull; ++s) step(s, M1{});
  for (; s < nsteps; ++s) step(s, M2{});

  if (mykey < Nk) {
    store_row_frags<DH>(a.dk + kbase + (int64_t)mykey * rs + dh * DH, dk, hh, a.scale);
    store_row_frags<DH>(a.dv + kbase + (int64_t)mykey * rs + dh * DH, dv, hh, 1.f);
  }
}

// ------------------------------------------------------------------ dQ pass
constexpr int kQPerWg = 128;   // 4 waves x 32 queries
constexpr int kBk = 64;        // keys per step

template <int D>
constexpr int dq_lds_bytes() {
  return 2 * 2 * kBk * D * 2;
}

// dQ of query tile qtile of head bh (one workgroup).
template <int D, bool CAUSAL, bool DROP>
__device__ __forceinline__ void dq_tile(const BwdArgs& a, int bh, int qtile, char* smem) {
  constexpr int NS = 2;   // K and V slots each
  constexpr int KS = D / 16, DT = D / 32, RB = D * 2;
  constexpr int TILE = kBk * RB;
  constexpr int CPW = TILE / 1024 / 4;
  static_assert(2 * NS * TILE == dq_lds_bytes<D>(), "LDS layout");
  char* const kbuf = smem;
  char* const vbuf = smem + NS * TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, Nk = a.Nk, qoff = a.qoff;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = ((int64_t)b * N * a.H + h) * D;      // Q, dO, dQ
  const int64_t kbase = ((int64_t)b * Nk * a.H + h) * D;    // K, V

  const int q0 = qtile * kQPerWg;
  const int qw0 = q0 + 32 * wave;
  const int myq = qw0 + l32;
  const int qc = min(myq, N - 1);

  bf16x8 qf[KS], gf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = *reinterpret_cast<const bf16x8*>(a.q + base + (int64_t)qc * rs + (2 * ks + hh) * 8);
    gf[ks] = *reinterpret_cast<const bf16x8*>(a.dout + base + (int64_t)qc * rs + (2 * ks + hh) * 8);
  }
  const float nl2 = a.ws[a.bhn + (int64_t)bh * N + qc];
  const float ndval = a.ws[(int64_t)bh * N + qc];   // -D of this lane's query

  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = (f32x16){};

  const int kend = CAUSAL ? min(Nk, q0 + qoff + kQPerWg) : Nk;
  const int nkt = (kend + kBk - 1) / kBk;

  uint32_t voff[CPW];
  stage_offsets<D, CPW>(voff, wave, lane, rs);
  const int wu = __builtin_amdgcn_readfirstlane(wave);   // uniform, for LDS destinations
  auto stage_rows = [&](const __bf16* src, int t, char* dst) {
    const int rows = min(Nk - t * kBk, kBk);
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(src + kbase + (int64_t)t * kBk * rs, (uint32_t)(rows * rs * 2));
#pragma unroll
    for (int i = 0; i < CPW; ++i) buffer_to_lds16(rsrc, voff[i], dst + (wu + 4 * i) * 1024);
  };
  auto kslot = [&](int t) { return kbuf + (t % NS) * TILE; };
  auto vslot = [&](int t) { return vbuf + (t % NS) * TILE; };

  const uint32_t rfb = row_frag_base<D>(lane);
  const uint32_t tfb = tr_frag_base<D>(lane);
  // S^T = K Q^T and dP^T = V dO^T for 32-key sub-tile j of a K/V slot pair:
  // lane = query, register r = key 32 j + 8(r/4) + 4hh + r%4.
  auto scores = [&](const char* kt, const char* vt, int j, f32x16& sacc, f32x16& pacc) {
    sacc = (f32x16){};
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] = DROP ? 0.f : ndval;   // pacc ends as dP^T - D (with dropout dP^T)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sacc = mfma32x32x16(lds_read_b128(kt, (rfb ^ (ks << 5)) + 32 * j * RB), qf[ks], sacc);
      pacc = mfma32x32x16(lds_read_b128(vt, (rfb ^ (ks << 5)) + 32 * j * RB), gf[ks], pacc);
    }
  };
  const float c = a.c;
  auto update = [&](auto mask_tag, const char* kt, int j, const f32x16& sacc, const f32x16& pacc, int k0) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float ds[8];
      // registers 8 u + e: keys k0 + 32 j + 16 u + 4 hh + 8 (e >> 2) + (e & 3), one call
      u32x4 w;
      if constexpr (DROP) w = drop_word8(a.drop, bh, myq, k0 + 32 * j + 16 * u + 4 * hh);
      static_for<0, 8>([&](auto E) {
        constexpr int e = decltype(E)::value;
        const int r = 8 * u + e;
        float pv = fast_exp2(__builtin_fmaf(sacc[r], c, nl2));
        if constexpr (MASK) {
          const int key = k0 + 32 * j + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool hide = key >= Nk || (CAUSAL && key > myq + qoff);
          pv = hide ? 0.f : pv;
        }
        if constexpr (DROP) {
          // dS^T = P (z dP - D) with pacc = dP: P (s dP - D) where kept, -P D
          // where dropped
          ds[e] = pv * (drop_keep<e>(w, a.drop.thr) ? __builtin_fmaf(a.drop.inv_keep, pacc[r], ndval) : ndval);
        } else {
          ds[e] = pv * pacc[r];
        }
      });
      const bf16x8 db = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      // dQ^T += K^T dS^T (rows d, columns queries)
#pragma unroll
      for (int t = 0; t < DT; ++t) dq[t] = mfma32x32x16(tr_frag<D>(kt, tfb, t, j, u), db, dq[t]);
    }
  };

  // Double-buffered K and V of the same tile; step t copies tile t+1 while it
  // works through the two 32-key units of tile t.  FULL steps are tiles that
  // every row of this wave sees whole (one unmasked update path); the other
  // steps (the diagonal, the ragged end, keys past this wave's rows) take the
  // general path.  Two loops, so that each body has one path (see dkdv_tile).
  auto step = [&](int t, auto full_tag) __attribute__((always_inline)) {
    wait_vmem();
    block_sync();
    if (t + 1 < nkt) {
      stage_rows(a.k, t + 1, kbuf + ((t + 1) & 1) * TILE);
      stage_rows(a.v, t + 1, vbuf + ((t + 1) & 1) * TILE);
    }
    const int k0 = t * kBk;
    if constexpr (decltype(full_tag)::value) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x16 sc, pc;
        scores(kbuf + (t & 1) * TILE, vbuf + (t & 1) * TILE, j, sc, pc);
        update(std::false_type{}, kbuf + (t & 1) * TILE, j, sc, pc, k0);
      }
    } else {
      if (CAUSAL && k0 > qw0 + qoff + 31) return;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x16 sc, pc;
        scores(kbuf + (t & 1) * TILE, vbuf + (t & 1) * TILE, j, sc, pc);
        if (CAUSAL && k0 + 32 * j > qw0 + qoff + 31) break;
        const bool masked = (k0 + 32 * j + 32 > Nk) || (CAUSAL && k0 + 32 * j + 31 > qw0 + qoff);
        if (masked) update(std::true_type{}, kbuf + (t & 1) * TILE, j, sc, pc, k0);
        else update(std::false_type{}, kbuf + (t & 1) * TILE, j, sc, pc, k0);
      }
    }
  };
  // Tiles 0 .. t_full - 1 lie whole below Nk and, under the mask, at or below
  // the position of this wave's first row.
  int t_full = min(nkt, Nk / kBk);
  if constexpr (CAUSAL) t_full = min(t_full, max(0, floor_div(qw0 + qoff - (kBk - 1), kBk) + 1));
  t_full = __builtin_amdgcn_readfirstlane(t_full);
  stage_rows(a.k, 0, kslot(0));
  stage_rows(a.v, 0, vslot(0));
  int t = 0;
  for (; t < t_full; ++t) step(t, std::true_type{});
  for (; t < nkt; ++t) step(t, std::false_type{});

  if (myq < N) store_row_frags<D>(a.dq + base + (int64_t)myq * rs, dq, hh, a.scale);
}

// dQ of query tile qtile of head bh by wave pairs (eight waves; waves w and
// w + 4 hold the same 32 queries).  The score wave (w) holds Q and dO and
// does all of the one-wave tile's work up to dS^T: S^T = K Q^T, dP^T - D =
// V dO^T - D, P^T and dS^T = P^T (dP^T - D), rounded to bf16 as the product
// takes it, which it hands to its partner through LDS.  The dQ wave (w + 4)
// holds the dQ accumulators and, one step behind, adds dQ^T += K^T dS^T.
// The products and elementwise operations are the one-wave tile's in the
// same order (bitwise the same dQ).  K and V rotate through four 32-key
// slot pairs, copied two steps ahead: the dQ wave reads K of the step before
// the score wave's (two steps ahead instead of one: 2-3% faster).
constexpr int kBkPair = 32;
constexpr int kDsBytes = 4 * 64 * 32;   // dS^T of one step: 4 pairs x 64 lanes x 16 bf16

template <int D>
constexpr int dq_pair_lds_bytes() { return 4 * 2 * kBkPair * D * 2 + 2 * kDsBytes; }

template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_tile_pair(const BwdArgs& a, int bh, int qtile, char* smem) {
  constexpr int KS = D / 16, DT = D / 32, RB = D * 2;
  constexpr int TILE = kBkPair * RB;       // one K or V tile
  constexpr int CPW = TILE / 1024 / kPairWaves;
  static_assert(CPW * kPairWaves * 1024 == TILE, "the copies cover the tile");
  static_assert(8 * TILE + 2 * kDsBytes == dq_pair_lds_bytes<D>(), "LDS layout");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int qg = wave & 3;                                        // query group
  const int role = __builtin_amdgcn_readfirstlane(wave >> 2);    // 0: score wave, 1: dQ wave
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, Nk = a.Nk, qoff = a.qoff;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = ((int64_t)b * N * a.H + h) * D;      // Q, dO, dQ
  const int64_t kbase = ((int64_t)b * Nk * a.H + h) * D;    // K, V

  const int q0 = qtile * kQPerWg;
  const int qw0 = q0 + 32 * qg;
  const int myq = qw0 + l32;
  const int qc = min(myq, N - 1);

  const int kend = CAUSAL ? min(Nk, q0 + qoff + kQPerWg) : Nk;
  const int nkt = (kend + kBkPair - 1) / kBkPair;

  auto slot_of = [&](int t) { return smem + (t & 3) * (2 * TILE); };   // K, then V
  // dS^T of step t: 16-byte unit 64 u + lane of this pair's area holds the
  // bf16 operand of half u (registers 8 u .. 8 u + 7) of the lane.
  auto dsbuf = [&](int t) {
    return reinterpret_cast<bf16x8*>(smem + 8 * TILE + (t & 1) * kDsBytes) + qg * 2 * 64;
  };
  uint32_t voff[CPW];
  stage_offsets<D, CPW, kPairWaves>(voff, wave, lane, rs);
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  auto stage = [&](int t) {
    char* slot = slot_of(t);
    const int rows = min(Nk - t * kBkPair, kBkPair);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kbase + (int64_t)t * kBkPair * rs, (uint32_t)(rows * rs * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kbase + (int64_t)t * kBkPair * rs, (uint32_t)(rows * rs * 2));
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      buffer_to_lds16(rk, voff[i], slot + (wu + kPairWaves * i) * 1024);
      buffer_to_lds16(rv, voff[i], slot + TILE + (wu + kPairWaves * i) * 1024);
    }
  };
  // Start of step t for every wave: this wave's copies of tile t complete
  // (those of tile t + 1, the only ones issued after them, may be in flight),
  // then the barrier publishes everyone's, and tile t + 2 goes into the slot
  // of tile t - 2.
  auto sync_stage = [&](int t) {
    if (t + 1 < nkt) wait_vmem_n<2 * CPW>();
    else wait_vmem();
    block_sync();
    if (t + 2 < nkt) stage(t + 2);
  };
  const uint32_t rfb = row_frag_base<D>(lane);
  const uint32_t tfb = tr_frag_base<D>(lane);
  const float c = a.c;

  // Steps [0, t_full) are seen whole by every row of the pair; [t_full,
  // t_act) are masked (the diagonal, keys past Nk); from t_act on no row of
  // the pair sees the step's keys.
  int t_full = min(nkt, Nk / kBkPair);
  int t_act = nkt;
  if constexpr (CAUSAL) {
    t_full = min(t_full, max(0, floor_div(qw0 + qoff - (kBkPair - 1), kBkPair) + 1));
    t_act = min(nkt, (qw0 + qoff + 31) / kBkPair + 1);
  }
  t_full = __builtin_amdgcn_readfirstlane(t_full);
  t_act = __builtin_amdgcn_readfirstlane(t_act);
  stage(0);
  if (nkt > 1) stage(1);
  if (role == 0) {
    bf16x8 qf[KS], gf[KS];
    {
      const int64_t qr = base + (int64_t)qc * rs;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(a.q + qr + (2 * ks + hh) * 8);
        gf[ks] = *reinterpret_cast<const bf16x8*>(a.dout + qr + (2 * ks + hh) * 8);
      }
    }
    const float nl2 = a.ws[a.bhn + (int64_t)bh * N + qc];
    const float ndval = a.ws[(int64_t)bh * N + qc];   // -D of this lane's query
    // S^T and dP^T - D (lane = query, register r = key 8(r/4) + 4hh + r%4 of
    // the step), then P^T, dS^T and its publication for step t.
    auto score_step = [&](int t, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const char* kt = slot_of(t);
      const int k0 = t * kBkPair;
      f32x16 sacc = (f32x16){}, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] = ndval;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sacc = mfma32x32x16(lds_read_b128(kt, rfb ^ (ks << 5)), qf[ks], sacc);
        pacc = mfma32x32x16(lds_read_b128(kt + TILE, rfb ^ (ks << 5)), gf[ks], pacc);
      }
      bf16x8* const dso = dsbuf(t);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * u + e;
          float pv = fast_exp2(__builtin_fmaf(sacc[r], c, nl2));
          if constexpr (MASK) {
            const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool hide = key >= Nk || (CAUSAL && key > myq + qoff);
            pv = hide ? 0.f : pv;
          }
          ds[e] = pv * pacc[r];
        }
        dso[64 * u + lane] = pack_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      }
    };
    int t = 0;
    for (; t < t_full; ++t) { sync_stage(t); score_step(t, std::false_type{}); }
    for (; t < t_act; ++t) { sync_stage(t); score_step(t, std::true_type{}); }
    for (; t < nkt; ++t) sync_stage(t);
    block_sync();   // the dQ wave reads the last step's dS after this barrier
  } else {
    f32x16 dq[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dq[t] = (f32x16){};
    // dQ^T += K^T dS^T (rows d, columns queries) with step t's dS^T.
    auto dq_step = [&](int t) __attribute__((always_inline)) {
      const char* kt = slot_of(t);
      const bf16x8* const dsi = dsbuf(t);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 db = dsi[64 * u + lane];
#pragma unroll
        for (int t2 = 0; t2 < DT; ++t2) dq[t2] = mfma32x32x16(tr_frag<D>(kt, tfb, t2, 0, u), db, dq[t2]);
      }
    };
    // Step t's barrier publishes the dS of step t - 1; K of step t - 1 stays
    // in its slot until the barrier of step t + 1.
    int t = 0;
    for (; t < nkt; ++t) {
      sync_stage(t);
      if (t >= 1 && t <= t_act) dq_step(t - 1);
    }
    block_sync();
    if (t_act == nkt && nkt > 0) dq_step(nkt - 1);
    if (myq < N) store_row_frags<D>(a.dq + base + (int64_t)myq * rs, dq, hh, a.scale);
  }
}

// ------------------------------------------------------------------ kernels
// Waves per SIMD the dK/dV and fused kernels are compiled for (measured on
// MI355X).  d = 64: 3 (168 registers; without the mask five dwords spill,
// still 3% faster than 2; dropout without the mask keeps 2, where 3 would
// spill 48).  d = 128: 2 (256 registers; without the mask the fused kernel's
// dQ tile, which the compiler would give about 280, spills 57 dwords, and
// is still 1.44x faster than at one wave per SIMD).  d = 256: 1 (the dK and
// dV accumulators of a wave alone take 256 registers; a few more spill
// without the mask); these one-wave tiles serve d = 256 with dropout, the
// eight-wave pair kernels the rest.
template <int D, bool CAUSAL, bool DROP>
constexpr int bwd_min_waves() {
  return D == 64 ? (CAUSAL || !DROP ? 3 : 2) : D == 128 ? 2 : 1;
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256, (bwd_min_waves<D, CAUSAL, DROP>())) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[dkdv_lds_bytes<D, DROP>()];
  int bh, kt;
  tile_of(blockIdx.x, a.ntiles, a.BH, CAUSAL, false, bh, kt);   // low key tiles see the most queries
  dkdv_tile<D, CAUSAL, DROP>(a, bh, kt, smem);
}

template <int D, bool CAUSAL, bool KV_SPLIT>
__global__ __launch_bounds__(kPairWaves * 64, 2) void bwd_dkdv_pair_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[KV_SPLIT ? dkdv_split_lds_bytes<D>() : dkdv_pair_lds_bytes<D>()];
  int bh, kt;
  tile_of(blockIdx.x, a.ntiles, a.BH, CAUSAL, false, bh, kt);
  if constexpr (KV_SPLIT) dkdv_tile_split<D, CAUSAL>(a, bh, kt, smem);
  else dkdv_tile_pair<D, CAUSAL>(a, bh, kt, smem);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPairWaves * 64, 2) void bwd_dq_pair_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[dq_pair_lds_bytes<D>()];
  int bh, qt;
  tile_of(blockIdx.x, a.ntiles, a.BH, CAUSAL, true, bh, qt);
  dq_tile_pair<D, CAUSAL>(a, bh, qt, smem);
}

// Single-pass backward: the dK/dV tiles also add their share of dQ with fp32
// atomics (two waves per SIMD at d = 64: the dQ accumulators do not fit
// beside the pass's registers at three).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, (D == 64 ? 2 : 1)) void bwd_single_pass_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[dkdv_lds_bytes<D, false, true>() + sp_extra_lds_bytes<D>()];
  int bh, kt;
  tile_of(blockIdx.x, a.ntiles, a.BH, CAUSAL, false, bh, kt);
  dkdv_tile<D, CAUSAL, false, true>(a, bh, kt, smem);
}

// Zeroes n4 float4s (the single pass's dQ accumulator).
__global__ __launch_bounds__(256) void zero_f32x4_kernel(f32x4* __restrict__ p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// dQ = scale * acc, rounded to bf16 (nearest even), 8 elements per thread.
__global__ __launch_bounds__(256) void dq_from_acc_kernel(const f32x4* __restrict__ acc, __bf16* __restrict__ dq,
                                                          int64_t n8, float scale) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x = acc[2 * i], y = acc[2 * i + 1];
  *reinterpret_cast<bf16x8*>(dq + 8 * i) = pack_bf16x8(x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale,
                                                       y[0] * scale, y[1] * scale, y[2] * scale, y[3] * scale);
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256, (D == 128 ? 2 : 3)) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[dq_lds_bytes<D>()];
  int bh, qt;
  tile_of(blockIdx.x, a.ntiles, a.BH, CAUSAL, true, bh, qt);
  dq_tile<D, CAUSAL, DROP>(a, bh, qt, smem);
}

// Both passes in one grid (a.ntiles key tiles and as many query tiles per head,
// both 128 rows), so that the light tiles of one pass fill the other's tail.
// Every XCD takes whole heads when the head count is a multiple of 8 (else the
// whole grid is one group) and hands out its tasks heaviest first by FLOPs.
// Under a causal mask the task costs, in units of 64x128 visible pairs times
// the FLOPs per pair, are 8 (2 (nt - kt) - 1) for key tile kt (4 GEMMs) and
// 6 (2 qt + 1) for query tile qt (3 GEMMs): two arithmetic sequences whose
// values never coincide, so the rank-r task is found by a binary search on the
// cost.  Without a mask the dK/dV tasks (the heavier ones) go first.
__device__ __forceinline__ void fused_task(int id, int nt, int bhcount, bool causal,
                                           bool& is_kv, int& bh, int& tile) {
  int group, rank, hpg;
  if ((bhcount & 7) == 0) {
    group = id & 7;
    rank = id >> 3;
    hpg = bhcount >> 3;
  } else {
    group = 0;
    rank = id;
    hpg = bhcount;
  }
  int which;   // task index inside its pass for this group: tile * hpg + head
  if (!causal) {
    is_kv = rank < nt * hpg;
    which = is_kv ? rank : rank - nt * hpg;
    bh = group * hpg + which % hpg;
    tile = which / hpg;
    return;
  }
  // Number of tasks with cost >= w.
  auto count_ge = [&](int w) {
    const int kvmax = 8 * (2 * nt - 1), dqmax = 6 * (2 * nt - 1);
    const int kv = w > kvmax ? 0 : min(nt, (kvmax - w) / 16 + 1);
    const int dq = w > dqmax ? 0 : min(nt, (dqmax - w) / 12 + 1);
    return (kv + dq) * hpg;
  };
  // Largest w with count_ge(w) > rank: the cost of the rank-r task.
  int lo = 1, hi = 8 * (2 * nt - 1);
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (count_ge(mid) > rank) lo = mid;
    else hi = mid - 1;
  }
  const int w = lo;
  const int pos = rank - count_ge(w + 1);   // position among the hpg tasks of cost w
  is_kv = (w % 16) == 8;
  tile = is_kv ? nt - (w / 8 + 1) / 2 : (w / 6 - 1) / 2;
  bh = group * hpg + pos;
}

// d = 256: both passes in one grid of eight-wave workgroups; KV_SPLIT takes
// the column-split dK/dV tiles, else the role pairs.
template <int D, bool CAUSAL, bool KV_SPLIT>
__global__ __launch_bounds__(kPairWaves * 64, 2) void bwd_fused_pair_kernel(BwdArgs a) {
  constexpr int KV = KV_SPLIT ? dkdv_split_lds_bytes<D>() : dkdv_pair_lds_bytes<D>();
  constexpr int LDS = KV > dq_pair_lds_bytes<D>() ? KV : dq_pair_lds_bytes<D>();
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  bool is_kv;
  int bh, tile;
  fused_task(blockIdx.x, a.ntiles, a.BH, CAUSAL, is_kv, bh, tile);
  if (is_kv) {
    if constexpr (KV_SPLIT) dkdv_tile_split<D, CAUSAL>(a, bh, tile, smem);
    else dkdv_tile_pair<D, CAUSAL>(a, bh, tile, smem);
  } else {
    dq_tile_pair<D, CAUSAL>(a, bh, tile, smem);
  }
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256, (bwd_min_waves<D, CAUSAL, DROP>())) void bwd_fused_kernel(BwdArgs a) {
  constexpr int LDS = dkdv_lds_bytes<D, DROP>() > dq_lds_bytes<D>() ? dkdv_lds_bytes<D, DROP>() : dq_lds_bytes<D>();
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  bool is_kv;
  int bh, tile;
  fused_task(blockIdx.x, a.ntiles, a.BH, CAUSAL, is_kv, bh, tile);
  if (is_kv) dkdv_tile<D, CAUSAL, DROP>(a, bh, tile, smem);
  else dq_tile<D, CAUSAL, DROP>(a, bh, tile, smem);
}

template <int D>
hipError_t run_pre(const BwdArgs& a, int B, hipStream_t st) {
  const int64_t rows = (int64_t)B * a.N * a.H;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + kPreRowsPerWg - 1) / kPreRowsPerWg)), dim3(256), 0, st,
                     a.o, a.dout, a.lse, a.ws, a.H, a.N, rows, a.bhn);
  return hipGetLastError();
}

template <int D, bool DROP = false>
hipError_t run_dkdv(BwdArgs a, int BH, bool causal, hipStream_t st) {
  a.ntiles = (a.Nk + kKeysPerWg - 1) / kKeysPerWg;
  const dim3 grid(a.ntiles * BH);
  if constexpr (D == 256 && !DROP) {
    if (causal) hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, true, true>), grid, dim3(kPairWaves * 64), 0, st, a);
    else hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, false, false>), grid, dim3(kPairWaves * 64), 0, st, a);
    return hipGetLastError();
  }
  if (causal) hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, DROP>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, DROP>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, bool DROP = false>
hipError_t run_dq(BwdArgs a, int BH, bool causal, hipStream_t st) {
  a.ntiles = (a.N + kQPerWg - 1) / kQPerWg;
  const dim3 grid(a.ntiles * BH);
  if constexpr (D == 256 && !DROP) {
    if (causal) hipLaunchKernelGGL((bwd_dq_pair_kernel<D, true>), grid, dim3(kPairWaves * 64), 0, st, a);
    else hipLaunchKernelGGL((bwd_dq_pair_kernel<D, false>), grid, dim3(kPairWaves * 64), 0, st, a);
    return hipGetLastError();
  }
  if (causal) hipLaunchKernelGGL((bwd_dq_kernel<D, true, DROP>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((bwd_dq_kernel<D, false, DROP>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, bool DROP = false>
hipError_t run_fused(BwdArgs a, int BH, bool causal, hipStream_t st) {
  // Square attention only (N == Nk): key tiles == query tiles, both 128 rows.
  a.ntiles = (a.N + kKeysPerWg - 1) / kKeysPerWg;
  const dim3 grid(2 * a.ntiles * BH);
  // d = 256: the eight-wave pair tiles; dK/dV by column halves under the
  // mask (1.092 against 1.136 ms on [2, 4096, 16, 256] with the role pairs),
  // by role pairs without it (1.908 against 2.022 ms).
  if constexpr (D == 256 && !DROP) {
    if (causal) hipLaunchKernelGGL((bwd_fused_pair_kernel<D, true, true>), grid, dim3(kPairWaves * 64), 0, st, a);
    else hipLaunchKernelGGL((bwd_fused_pair_kernel<D, false, false>), grid, dim3(kPairWaves * 64), 0, st, a);
    return hipGetLastError();
  }
  if (causal) hipLaunchKernelGGL((bwd_fused_kernel<D, true, DROP>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((bwd_fused_kernel<D, false, DROP>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

BwdArgs make_args(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, float* ws, void* dq, void* dk, void* dv, const AttnShape& s) {
  BwdArgs a{};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.ws = ws;
  a.dq = static_cast<__bf16*>(dq);
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.H = s.H;
  a.N = s.N;
  a.Nk = s.N;
  a.qoff = 0;
  a.bhn = (int64_t)s.B * s.H * s.N;
  a.BH = s.B * s.H;
  a.c = s.scale * kLog2e;
  a.scale = s.scale;
  return a;
}

}  // namespace

hipError_t launch_bwd_pre_bf16(const void* o, const void* dout, const float* lse, float* ws,
                               const AttnShape& s, hipStream_t stream) {
  const BwdArgs a = make_args(nullptr, nullptr, nullptr, o, dout, lse, ws, nullptr, nullptr, nullptr, s);
  return s.d == 64 ? run_pre<64>(a, s.B, stream)
         : s.d == 128 ? run_pre<128>(a, s.B, stream)
                      : run_pre<256>(a, s.B, stream);
}

hipError_t launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const void* dout,
                                const float* ws, void* dk, void* dv, const AttnShape& s,
                                hipStream_t stream) {
  const BwdArgs a = make_args(q, k, v, nullptr, dout, nullptr, const_cast<float*>(ws), nullptr, dk, dv, s);
  const int BH = s.B * s.H;
  return s.d == 64 ? run_dkdv<64>(a, BH, s.causal != 0, stream)
         : s.d == 128 ? run_dkdv<128>(a, BH, s.causal != 0, stream)
                      : run_dkdv<256>(a, BH, s.causal != 0, stream);
}

hipError_t launch_bwd_dqdkdv_bf16(const void* q, const void* k, const void* v, const void* dout,
                                  const float* ws, void* dq, void* dk, void* dv, const AttnShape& s,
                                  hipStream_t stream) {
  const BwdArgs a = make_args(q, k, v, nullptr, dout, nullptr, const_cast<float*>(ws), dq, dk, dv, s);
  const int BH = s.B * s.H;
  return s.d == 64 ? run_fused<64>(a, BH, s.causal != 0, stream)
         : s.d == 128 ? run_fused<128>(a, BH, s.causal != 0, stream)
                      : run_fused<256>(a, BH, s.causal != 0, stream);
}

hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* dout,
                              const float* ws, void* dq, const AttnShape& s, hipStream_t stream) {
  const BwdArgs a = make_args(q, k, v, nullptr, dout, nullptr, const_cast<float*>(ws), dq, nullptr, nullptr, s);
  const int BH = s.B * s.H;
  return s.d == 64 ? run_dq<64>(a, BH, s.causal != 0, stream)
         : s.d == 128 ? run_dq<128>(a, BH, s.causal != 0, stream)
                      : run_dq<256>(a, BH, s.causal != 0, stream);
}

hipError_t launch_bwd_cross_bf16(const void* q, const void* k, const void* v, const void* o,
                                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                 float* ws, const AttnShape& s, int Nk, hipStream_t stream) {
  hipError_t e = launch_bwd_pre_bf16(o, dout, lse, ws, s, stream);
  if (e != hipSuccess) return e;
  if (Nk == s.N) return launch_bwd_dqdkdv_bf16(q, k, v, dout, ws, dq, dk, dv, s, stream);
  BwdArgs a = make_args(q, k, v, nullptr, dout, nullptr, ws, dq, dk, dv, s);
  a.Nk = Nk;
  a.qoff = s.causal ? Nk - s.N : 0;
  const int BH = s.B * s.H;
  const bool causal = s.causal != 0;
  e = s.d == 64 ? run_dkdv<64>(a, BH, causal, stream)
         : s.d == 128 ? run_dkdv<128>(a, BH, causal, stream)
                      : run_dkdv<256>(a, BH, causal, stream);
  if (e != hipSuccess) return e;
  return s.d == 64 ? run_dq<64>(a, BH, causal, stream)
         : s.d == 128 ? run_dq<128>(a, BH, causal, stream)
                      : run_dq<256>(a, BH, causal, stream);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* ws, const AttnShape& s, hipStream_t stream) {
  hipError_t e = launch_bwd_pre_bf16(o, dout, lse, ws, s, stream);
  if (e != hipSuccess) return e;
  return launch_bwd_dqdkdv_bf16(q, k, v, dout, ws, dq, dk, dv, s, stream);
}

int64_t bwd_single_pass_acc_offset(int B, int H, int N) {
  return ((2 * (int64_t)B * H * N + 3) / 4) * 4;   // floats; 16-byte aligned
}

hipError_t launch_bwd_single_pass_bf16(const void* q, const void* k, const void* v, const void* o,
                                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                       float* ws, const AttnShape& s, hipStream_t stream) {
  float* acc = ws + bwd_single_pass_acc_offset(s.B, s.H, s.N);
  const int64_t n = (int64_t)s.B * s.N * s.H * s.d;   // a multiple of 64
  const int64_t n4 = n / 4;
  const int64_t zblocks = (n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192;
  hipLaunchKernelGGL(zero_f32x4_kernel, dim3((unsigned)zblocks), dim3(256), 0, stream, reinterpret_cast<f32x4*>(acc), n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_bwd_pre_bf16(o, dout, lse, ws, s, stream);
  if (e != hipSuccess) return e;
  BwdArgs a = make_args(q, k, v, nullptr, dout, nullptr, ws, nullptr, dk, dv, s);
  a.dqacc = acc;
  a.ntiles = (a.Nk + kKeysPerWg - 1) / kKeysPerWg;
  const dim3 grid(a.ntiles * a.BH);
  if (s.d == 64) {
    if (s.causal) hipLaunchKernelGGL((bwd_single_pass_kernel<64, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((bwd_single_pass_kernel<64, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (s.causal) hipLaunchKernelGGL((bwd_single_pass_kernel<128, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((bwd_single_pass_kernel<128, false>), grid, dim3(256), 0, stream, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(dq_from_acc_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const f32x4*>(acc), static_cast<__bf16*>(dq), n8, s.scale);
  return hipGetLastError();
}

}  // namespace fa

namespace fa {

hipError_t launch_bwd_dropout_bf16(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   float* ws, const AttnShape& s, const DropParams& drop,
                                   hipStream_t stream) {
  hipError_t e = launch_bwd_pre_bf16(o, dout, lse, ws, s, stream);
  if (e != hipSuccess) return e;
  BwdArgs a = make_args(q, k, v, nullptr, dout, nullptr, ws, dq, dk, dv, s);
  a.drop = drop;
  const int BH = s.B * s.H;
  const bool causal = s.causal != 0;
  return s.d == 64 ? run_fused<64, true>(a, BH, causal, stream)
         : s.d == 128 ? run_fused<128, true>(a, BH, causal, stream)
                      : run_fused<256, true>(a, BH, causal, stream);
}

}  // namespace fa
