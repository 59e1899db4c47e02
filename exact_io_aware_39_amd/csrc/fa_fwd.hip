// fa_fwd.hip - fused forward of exact attention, bf16 in/out, fp32 accumulation.
//
// Method (page "FlashAttention", vagrantpi.github.io PKM note, "三招"): tiles of
// K and V stream through on-chip memory while a block of query rows keeps its
// running max m, running sum l and unnormalised output on chip; when the max
// grows, the earlier sum and output are multiplied by exp(m_old - m_new); O is
// divided by l once at the end and only O and the row statistics are written.
// The loop order is the one of the FlashAttention-2 follow-up on page
// "知识点13 | FlashAttention深度攻略" (blog.xiaohack.org): query blocks are the
// parallel dimension (one workgroup each) and keys are the inner loop.
//
// gfx950 mapping (one workgroup = 4 waves = 128 query rows; 64 keys a step):
//  * S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16 so that each lane
//    of a wave owns one query row (column of S^T) and 16 of every 32 keys; the
//    per-row softmax state lives in that lane and only the row max needs one
//    exchange between the two half-waves (v_permlane32_swap).
//  * The fp32 S^T accumulator, exponentiated and rounded to bf16, is directly
//    the B operand of O^T += V^T P^T: no LDS round trip for P.
//  * V^T fragments come from row-major V tiles in LDS through the transposing
//    read ds_read_b64_tr_b16; K fragments are plain 16-byte LDS reads.
//  * K/V tiles are double buffered in LDS; the next tile's global loads are in
//    flight during the current tile's matrix work; one barrier per step.
//  * exp is exp2 with scale*log2(e) folded into one FMA.  The reference max is
//    only moved when a row's max grows by more than 2^8 (RESCALE_LOG2): any
//    finite reference gives the same O and LSE (the final divide uses the same
//    reference), so this keeps exactness while the O rescale becomes rare;
//    probabilities stay <= 2^8 before normalisation.
//  * Causal: tiles above the diagonal are never visited; waves whose 32 rows
//    cannot see any key of a step skip it; only steps that straddle the
//    diagonal (or the ragged end of the keys) evaluate the mask.
//  * Workgroups are renumbered per XCD so one head's query tiles share an L2,
//    and causal query tiles run heaviest first.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kBr = 32 * kWaves;   // query rows per workgroup
constexpr int kBc = 64;            // keys per step
constexpr float kRescaleLog2 = 8.0f;

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int H, N, nqt;
  float c;   // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int KS = D / 16;           // k-steps of the score product
  constexpr int DT = D / 32;           // 32-wide output tiles
  // Padded LDS rows: K rows are read 16 bytes at a time, 16 rows at one
  // column (a 16-byte pad puts those rows in 16 different bank groups); V rows
  // are read by the transposing 8-byte read, 4 rows x 64 bytes per half-wave
  // (a 64-byte pad puts those rows in 4 disjoint quarters of the banks).
  // Offsets stay additive, so every fragment address is a lane base plus an
  // immediate.
  constexpr int KSTR = D * 2 + 16;       // bytes per K row in LDS
  constexpr int VSTR = D * 2 + 64;       // bytes per V row in LDS
  constexpr int KT = kBc * KSTR;         // bytes of one K tile
  constexpr int STAGE = KT + kBc * VSTR; // K tile then V tile
  constexpr int CPT = kBc * CH / 256;    // chunks each thread stages per tile
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / a.nqt;
  const int qt = a.nqt - 1 - (L - bh * a.nqt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;
  const int64_t rs = (int64_t)a.H * D;                       // row stride (elements)
  const int64_t base = ((int64_t)b * N * a.H + h) * D;
  const __bf16* __restrict__ Qg = a.q + base;
  const __bf16* __restrict__ Kg = a.k + base;
  const __bf16* __restrict__ Vg = a.v + base;

  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + l32;

  // Q^T operand for this lane's row: chunk 2*ks + hh of the row, per k-step.
  bf16x8 qf[KS];
  {
    const __bf16* qrow = Qg + (int64_t)min(myq, N - 1) * rs;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + hh) * 8);
  }

  const int kend = CAUSAL ? min(N, q0 + kBr) : N;
  const int nkt = (kend + kBc - 1) / kBc;

  // Global offsets (elements) of the chunks this thread stages, for key tile 0.
  int64_t goff[CPT];
  int grow[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int idx = tid + 256 * i;
    grow[i] = idx / CH;
    goff[i] = (int64_t)grow[i] * rs + (idx % CH) * 8;
  }
  const int64_t tile_step = (int64_t)kBc * rs;
  u32x4 kreg[CPT], vreg[CPT];
  auto gload = [&](int kt) {
    const int64_t t0 = kt * tile_step;
    if (kt * kBc + kBc <= N) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        kreg[i] = *reinterpret_cast<const u32x4*>(Kg + t0 + goff[i]);
        vreg[i] = *reinterpret_cast<const u32x4*>(Vg + t0 + goff[i]);
      }
    } else {   // ragged last tile: rows past N re-read row N-1 (real, finite data)
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int over = kt * kBc + grow[i] - (N - 1);
        const int64_t off = t0 + goff[i] - (over > 0 ? (int64_t)over * rs : 0);
        kreg[i] = *reinterpret_cast<const u32x4*>(Kg + off);
        vreg[i] = *reinterpret_cast<const u32x4*>(Vg + off);
      }
    }
  };
  // Staging: thread tid writes chunk (row, ch) of each tile; the row steps by
  // 256 / CH between its chunks.
  const uint32_t kst = (tid / CH) * KSTR + (tid % CH) * 16;
  const uint32_t vst = (tid / CH) * VSTR + (tid % CH) * 16;
  auto swrite = [&](int stage) {
    char* kb = smem + stage * STAGE;
    char* vb = kb + KT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      *reinterpret_cast<u32x4*>(kb + kst + i * (256 / CH) * KSTR) = kreg[i];
      *reinterpret_cast<u32x4*>(vb + vst + i * (256 / CH) * VSTR) = vreg[i];
    }
  };
  // Lane bases of the fragment reads (the rest of each address is constant).
  //  K (A operand of S^T): row 32 j + l%32, chunk 2 ks + l/32.
  const uint32_t kfrag = l32 * KSTR + hh * 16;
  //  V^T (A operand of O^T) through the transposing read: within each group of
  //  16 lanes, lane i addresses row 4 (l/32) + i/4 and column 16 ((l/16)%2) + 4 (i%4).
  const int ti = lane & 15, tg = lane >> 4;
  const uint32_t vfrag = ((tg >> 1) * 4 + (ti >> 2)) * VSTR + ((tg & 1) * 16 + (ti & 3) * 4) * 2;

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = (f32x16){};
  float m_ref = -INFINITY;   // reference max, log2 units
  float l_part = 0.f;        // this half-wave's share of the row sum
  const float c = a.c;

  // Softmax update and O^T += V^T P^T for one step; MASK evaluates the causal /
  // ragged-end mask, the common path carries no per-element test.
  auto softmax_pv = [&](auto mask_tag, f32x16 (&s)[2], const char* vb, int k0) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float mx = -INFINITY;
    if constexpr (MASK) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * j + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool hide = key >= N || (CAUSAL && key > myq);
          s[j][r] = hide ? -INFINITY : s[j][r];
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
    mx = max_halves(mx);
    const float mcand = MASK ? ((mx == -INFINITY) ? -INFINITY : mx * c) : mx * c;
    const float m_new = fmaxf(m_ref, mcand);
    if (__any(m_new > m_ref + kRescaleLog2)) {
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      m_ref = m_new;
    }
    const float nm = -m_ref;
    bf16x8 pb[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = fast_exp2(__builtin_fmaf(s[j][r], c, nm));
        if constexpr (MASK) e = (s[j][r] == -INFINITY) ? 0.f : e;
        p[r] = e;
        l_part += e;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        pb[j][u] = pack_bf16x8(p[8 * u + 0], p[8 * u + 1], p[8 * u + 2], p[8 * u + 3],
                               p[8 * u + 4], p[8 * u + 5], p[8 * u + 6], p[8 * u + 7]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const uint32_t off = vfrag + (32 * j + 16 * u) * VSTR + t * 64;
          const bf16x4 lo = __builtin_bit_cast(bf16x4, lds_read_tr16(vb, off));
          const bf16x4 hi = __builtin_bit_cast(bf16x4, lds_read_tr16(vb, off + 8 * VSTR));
          bf16x8 va;
          va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
          va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
          oacc[t] = mfma32x32x16(va, pb[j][u], oacc[t]);
        }
  };

  gload(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int stage = kt & 1;
    swrite(stage);
    __syncthreads();
    if (kt + 1 < nkt) gload(kt + 1);

    const int k0 = kt * kBc;
    // All keys of this step lie beyond this wave's rows: nothing to add.
    if (CAUSAL && k0 > qw0 + 31) continue;

    const char* kb = smem + stage * STAGE;
    const char* vb = kb + KT;

    // ---- S^T = K Q^T for two 32-key sub-tiles (independent chains interleaved)
    f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        s[j] = mfma32x32x16(lds_read_b128(kb, kfrag + 32 * j * KSTR + 32 * ks), qf[ks], s[j]);

    const bool masked = (k0 + kBc > N) || (CAUSAL && k0 + kBc - 1 > qw0);
    if (masked) softmax_pv(std::true_type{}, s, vb, k0);
    else softmax_pv(std::false_type{}, s, vb, k0);
  }

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
  const float l = sum_halves(l_part);
  if (myq < N) {
    const float inv = 1.f / l;
    __bf16* orow = a.o + base + (int64_t)myq * rs;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = t * 32 + 8 * g4 + 4 * hh;
        *reinterpret_cast<bf16x4*>(orow + d0) =
            pack_bf16x4(oacc[t][4 * g4 + 0] * inv, oacc[t][4 * g4 + 1] * inv,
                        oacc[t][4 * g4 + 2] * inv, oacc[t][4 * g4 + 3] * inv);
      }
    if (hh == 0) a.lse[(int64_t)bh * N + myq] = kLn2 * (m_ref + fast_log2(l));
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& args, int BH, hipStream_t stream) {
  const int grid = args.nqt * BH;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const AttnShape& s, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.H = s.H;
  a.N = s.N;
  a.nqt = (s.N + kBr - 1) / kBr;
  a.c = s.scale * kLog2e;
  const int BH = s.B * s.H;
  if (s.d == 64) return s.causal ? launch<64, true>(a, BH, stream) : launch<64, false>(a, BH, stream);
  return s.causal ? launch<128, true>(a, BH, stream) : launch<128, false>(a, BH, stream);
}

}  // namespace fa
