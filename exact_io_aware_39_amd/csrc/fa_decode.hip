// fa_decode.hip - decode against a K/V cache: a few query rows per head
// against a long key sequence, split over the keys and combined by the
// logsumexp merge.
//
// Method: page "FlashAttention" (vagrantpi.github.io PKM note), part "⚠️ 注意"
// (in decode each step has one query token, there is no N x N matrix, the cost
// is reading K and V, and the variant for that case is FlashDecoding) and
// "三招" item 2 (online softmax: running max, running sum and unnormalised
// output rescaled by exp(m_old - m_new); the same rescaling combines whole
// chunks, LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s).
//
// gfx950 mapping:
//  * decode_split_kernel: one workgroup of 4 waves per (batch, head, key
//    chunk).  Each wave walks the chunk's 32-key blocks w, w+4, w+8, ... with
//    its own running max, sum and unnormalised output; the four waves merge
//    through LDS at the end and write the chunk's normalised O_s and LSE_s.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the (at most 32) query rows are
//    the MFMA columns, one per lane as in the forward, so the softmax state of
//    a query lives in one lane pair; unused columns hold zero queries.
//  * K and V blocks stream through a wave-private two-slot LDS ring filled by
//    buffer -> LDS copies whose descriptors end at the last key (rows past it
//    read as zero): waves never wait for each other inside the loop.  The next
//    block's copies are in flight while the current block is used, so V^T is
//    read with asm-issued transposing reads (see fa_common.hpp).
//  * decode_merge_kernel: one wave per (batch, head, query row) combines the
//    chunks; deterministic (no atomics).
//  * The bound is HBM bandwidth: every K and V byte is read exactly once; the
//    matrix cores and the vector unit run far below their limits.
#include <algorithm>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecBlk = 32;    // keys per block
constexpr int kDecSlots = 2;   // ring slots per wave

struct DecArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  float* ws_o;     // [B*H][S][Nq][D] normalised chunk outputs
  float* ws_lse;   // [B*H][S][Nq] chunk logsumexps (natural log)
  int H, Nq, Nk, S, bpc;   // bpc: 32-key blocks per chunk
  int causal;
  float c;         // scale * log2(e)
};

template <int D>
constexpr int dec_lds_bytes() { return kDecWaves * kDecSlots * 2 * kDecBlk * D * 2; }

template <int D>
__global__ __launch_bounds__(256, (D == 64 ? 2 : 1)) void decode_split_kernel(DecArgs a) {
  constexpr int CH = D / 8, KS = D / 16, DT = D / 32, RB = D * 2;
  constexpr int TILE = kDecBlk * RB;      // bytes of one K or V block
  constexpr int CPB = TILE / 1024;        // 1 KB copies per block and tensor
  constexpr int WAVE_LDS = kDecSlots * 2 * TILE;
  static_assert(kDecWaves * WAVE_LDS == dec_lds_bytes<D>(), "LDS layout");
  static_assert(dec_lds_bytes<D>() >= 2048 + kDecWaves * 32 * D * 4, "merge area");
  __shared__ __attribute__((aligned(1024))) char smem[dec_lds_bytes<D>()];

  // The wave index is made scalar: it picks each wave's K/V blocks and LDS
  // ring, and a copy's buffer descriptor and LDS destination must be uniform
  // (with a per-lane index every copy is wrapped in a loop over its values).
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x / a.S, chunk = blockIdx.x - bh * a.S;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Nq = a.Nq, Nk = a.Nk;
  const int64_t rs = (int64_t)a.H * D;   // row stride (elements)
  const __bf16* __restrict__ Kg = a.k + ((int64_t)b * Nk * a.H + h) * D;
  const __bf16* __restrict__ Vg = a.v + ((int64_t)b * Nk * a.H + h) * D;

  const int nblk = (Nk + kDecBlk - 1) / kDecBlk;
  const int blk0 = chunk * a.bpc + wave;
  const int blk_end = min(nblk, (chunk + 1) * a.bpc);
  const int nmine = blk0 < blk_end ? (blk_end - blk0 + kDecWaves - 1) / kDecWaves : 0;

  // Q^T operand: query l32 (zero past Nq), 16-byte chunk 2 ks + hh.
  bf16x8 qf[KS];
  {
    const __bf16* qrow = a.q + ((int64_t)b * Nq * a.H + h) * D + (int64_t)min(l32, Nq - 1) * rs;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + hh) * 8);
      if (l32 >= Nq) qf[ks] = (bf16x8){};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));   // wait for Q here, not in the loop
  }

  // Copy i of a block fills LDS bytes [1024 i, 1024 i + 1024) of its slot; the
  // lane's 16 bytes are physical chunk p % CH of row p / CH (p = 64 i + lane),
  // which holds logical chunk (p % CH) ^ swz(row) of that key row.
  uint32_t voff[CPB];
#pragma unroll
  for (int i = 0; i < CPB; ++i) {
    const int p = 64 * i + lane, row = p / CH;
    voff[i] = (uint32_t)(row * rs * 2) + (uint32_t)(((p % CH) ^ swz<D>(row)) * 16);
  }
  char* const ring = smem + wave * WAVE_LDS;   // slot s: K at 2 s TILE, V at (2 s + 1) TILE
  auto stage = [&](int blk, int slot) {
    const int rows = min(Nk - blk * kDecBlk, kDecBlk);
    const uint32_t bytes = (uint32_t)(rows * rs * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (int64_t)blk * kDecBlk * rs, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (int64_t)blk * kDecBlk * rs, bytes);
    char* kd = ring + 2 * slot * TILE;
#pragma unroll
    for (int i = 0; i < CPB; ++i) {
      buffer_to_lds16(rk, voff[i], kd + 1024 * i);
      buffer_to_lds16(rv, voff[i], kd + TILE + 1024 * i);
    }
  };

  // Fragment lane bases, as in the forward (one 32-key sub-tile):
  //  K (A operand of S^T): row l%32, logical chunk 2 ks + l/32.
  const uint32_t kl = (uint32_t)(l32 * RB) | ((uint32_t)(hh ^ swz<D>(l32)) << 4);
  //  V^T (A operand of O^T), transposing read: within each group of 16 lanes,
  //  lane i addresses row 16 u + r4 (+8 for the high half), r4 = 4 (l/32) +
  //  i/4, and element column 32 t + 16 ((l/16)%2) + 4 (i%4).
  uint32_t vl;
  {
    const int ti = lane & 15, tg = lane >> 4;
    const int r4 = (tg >> 1) * 4 + (ti >> 2);
    const int cl = (tg & 1) * 2 + ((ti & 3) >> 1);
    vl = (uint32_t)(r4 * RB) | ((uint32_t)(cl ^ swz<D>(r4)) << 4) | ((uint32_t)(ti & 1) << 3);
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = (f32x16){};
  float m = -INFINITY;   // running max of this lane's query, log2 units
  float l_part = 0.f;    // this half-wave's share of the running sum
  const float c = a.c;
  const int qpos = Nk - Nq + l32;   // sequence position of this lane's query (causal)

  if (nmine > 0) stage(blk0, 0);
  for (int i = 0; i < nmine; ++i) {
    const int blk = blk0 + kDecWaves * i, slot = i & 1;
    // The other slot was last read by block i-1, whose reads have all been
    // waited for; block i's copies must be complete, block i+1's may not be.
    if (i + 1 < nmine) {
      stage(blk + kDecWaves, slot ^ 1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * CPB) : "memory");
    } else {
      wait_vmem();
    }
    const char* kt = ring + 2 * slot * TILE;
    const char* vt = kt + TILE;

    f32x16 s = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma32x32x16(lds_read_b128(kt, kl ^ (ks << 5)), qf[ks], s);

    // Keys past the end, and under the mask keys after the query's position.
    const int k0 = blk * kDecBlk;
    const bool edge = (k0 + kDecBlk > Nk) || (a.causal && k0 + kDecBlk - 1 > Nk - Nq);
    if (edge) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool hide = key >= Nk || (a.causal && key > qpos);
        s[r] = hide ? -INFINITY : s[r];
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m, mx == -INFINITY ? -INFINITY : mx * c);
    if (__any(m_new != m)) {
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      m = m_new;
    }
    const float nm = (m == -INFINITY) ? 0.f : -m;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(__builtin_fmaf(s[r], c, nm));
      p[r] = (s[r] == -INFINITY) ? 0.f : e;
      l_part += p[r];
    }
    bf16x8 pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      pb[u] = pack_bf16x8(p[8 * u + 0], p[8 * u + 1], p[8 * u + 2], p[8 * u + 3],
                          p[8 * u + 4], p[8 * u + 5], p[8 * u + 6], p[8 * u + 7]);

    // O^T += V^T P^T: keys 16 u .. 16 u + 15 of the block per k-step.
    const uint32_t vbase = lds_addr(vt);
    s16x4 rd[2][DT][2];
    static_for<0, 2>([&](auto U) {
      constexpr int u = decltype(U)::value;
      static_for<0, DT>([&](auto T) {
        constexpr int t = decltype(T)::value;
        constexpr uint32_t rowoff = (uint32_t)(16 * u * RB);
        rd[u][t][0] = lds_tr16_issue<rowoff>(vbase + (vl ^ (64 * t)));
        rd[u][t][1] = lds_tr16_issue<rowoff + 8 * RB>(vbase + (vl ^ (64 * t + 32)));
      });
    });
    lds_wait<2 * DT>();
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = mfma32x32x16(tr_pair_take(rd[0][t]), pb[0], oacc[t]);
    lds_wait<0>();
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = mfma32x32x16(tr_pair_take(rd[1][t]), pb[1], oacc[t]);
  }

  // ---- merge the four waves through LDS (the rings are no longer needed)
  const float lsum = sum_halves(l_part);
  block_sync();
  float* mm = reinterpret_cast<float*>(smem);            // [wave][32] running max
  float* ll = mm + kDecWaves * 32;                       // [wave][32] running sum
  float* oo = reinterpret_cast<float*>(smem + 2048);     // [wave][32][D] unnormalised O
  if (hh == 0) {
    mm[wave * 32 + l32] = m;
    ll[wave * 32 + l32] = lsum;
  }
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * t + 8 * g4 + 4 * hh;
      *reinterpret_cast<f32x4*>(oo + (wave * 32 + l32) * D + d0) =
          (f32x4){oacc[t][4 * g4 + 0], oacc[t][4 * g4 + 1], oacc[t][4 * g4 + 2], oacc[t][4 * g4 + 3]};
    }
  block_sync();
  // Thread (q, part): query q = tid / 8, dims part, part + 8, ...
  const int q = tid >> 3, part = tid & 7;
  if (q < Nq) {
    float mw[kDecWaves], mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      mw[w] = mm[w * 32 + q];
      mstar = fmaxf(mstar, mw[w]);
    }
    const int64_t row = ((int64_t)bh * a.S + chunk) * Nq + q;
    float* out = a.ws_o + row * D;
    if (mstar == -INFINITY) {   // no key of this chunk is visible to the query
      for (int dd = part; dd < D; dd += 8) out[dd] = 0.f;
      if (part == 0) a.ws_lse[row] = -INFINITY;
    } else {
      float aw[kDecWaves], L = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        aw[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - mstar);
        L += aw[w] * ll[w * 32 + q];
      }
      const float inv = 1.f / L;
      for (int dd = part; dd < D; dd += 8) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) acc += aw[w] * oo[(w * 32 + q) * D + dd];
        out[dd] = acc * inv;
      }
      if (part == 0) a.ws_lse[row] = kLn2 * (mstar + fast_log2(L));
    }
  }
}

// One wave per (batch, head, query row): LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s, in chunk order.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecArgs a) {
  const int lane = threadIdx.x;
  const int bq = blockIdx.x;                 // bh * Nq + q
  const int bh = bq / a.Nq, q = bq - bh * a.Nq;
  const int b = bh / a.H, h = bh - b * a.H;
  const int S = a.S;
  const float* lse_s = a.ws_lse + (int64_t)bh * S * a.Nq + q;   // chunk s at lse_s[s * Nq]
  const float* o_s = a.ws_o + ((int64_t)bh * S * a.Nq + q) * D;  // chunk s at o_s[s * Nq * D]
  float mx = -INFINITY;
  for (int s = lane; s < S; s += 64) mx = fmaxf(mx, lse_s[(int64_t)s * a.Nq]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  float acc[D / 64] = {};
  float tot = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ls = lse_s[(int64_t)s * a.Nq];
      const float w = (ls == -INFINITY) ? 0.f : fast_exp2((ls - mx) * kLog2e);
      tot += w;
      if (w != 0.f) {
#pragma unroll
        for (int e = 0; e < D / 64; ++e) acc[e] += w * o_s[(int64_t)s * a.Nq * D + lane + 64 * e];
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  __bf16* orow = a.o + (((int64_t)b * a.Nq + q) * a.H + h) * D;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) orow[lane + 64 * e] = (__bf16)(acc[e] * inv);
  if (lane == 0) a.lse[(int64_t)bh * a.Nq + q] = tot > 0.f ? mx + kLn2 * fast_log2(tot) : -INFINITY;
}

template <int D>
hipError_t run_decode(const DecArgs& a, int BH, hipStream_t st) {
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)(BH * a.S)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(BH * a.Nq)), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int decode_splits(int B, int H, int Nq, int Nk) {
  (void)Nq;
  const int64_t bh = (int64_t)B * H;
  const int64_t nblk = (Nk + kDecBlk - 1) / kDecBlk;
  // About 1024 workgroups in all (4 per CU), and at least 8 blocks (two per
  // wave) in every chunk.
  int64_t s = (1024 + bh - 1) / bh;
  s = std::min<int64_t>(s, std::max<int64_t>(1, nblk / 8));
  s = std::min<int64_t>(s, kDecodeMaxSplits);
  return (int)std::max<int64_t>(1, s);
}

hipError_t launch_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                              float* ws, const DecodeShape& s, hipStream_t stream) {
  DecArgs a{};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  const int64_t bh = (int64_t)s.B * s.H;
  a.ws_o = ws;
  a.ws_lse = ws + bh * s.splits * s.Nq * s.d;
  a.H = s.H;
  a.Nq = s.Nq;
  a.Nk = s.Nk;
  a.S = s.splits;
  const int nblk = (s.Nk + kDecBlk - 1) / kDecBlk;
  a.bpc = (nblk + s.splits - 1) / s.splits;
  a.causal = s.causal;
  a.c = s.scale * kLog2e;
  if (s.d == 64) return run_decode<64>(a, (int)bh, stream);
  return run_decode<128>(a, (int)bh, stream);
}

}  // namespace fa
