// fa_fwd_fp8.hip - attention forward on e4m3 (FP8) inputs for gfx950.
//
// Method: the fused, tiled forward with online softmax of the page
// "FlashAttention" (vagrantpi.github.io), parts "三招" (tiling, online
// softmax), with the FP8 precision that the same page's "效果" table gives for
// FlashAttention-3 and the page "知识点13 | FlashAttention深度攻略" lists under
// "前沿研究方向".  Inputs are OCP E4M3 codes with one descale per tensor.
//
// Both products run on the 32x32x64 FP8 MFMA:
//  * S^T = K Q^T: Q^T is the B operand held in registers, K rows come from LDS.
//    The K rows of a 64-key tile are fed to the A operand in a permuted order,
//    so that the 32 scores a lane holds are 32 consecutive keys (lane l holds
//    query l % 32 and keys 32 (l / 32) .. 32 (l / 32) + 31 of the tile).
//  * O^T += V^T P^T: P = 2^8 exp(S - m) (m a reference at most 0.75 below
//    the running row maximum in log2 units, so 2^8 p <= 2^8.75 < 448, the
//    largest e4m3 value) is rounded to e4m3 and those 32 consecutive keys are
//    the lane's B operand as they stand; V^T comes from a transposed copy of V
//    ([B H, d, Nk rounded up to 64], made by a pre-pass kernel), so that the A
//    operand is 32 contiguous bytes of a V^T row.
// The row sum l adds the unrounded 2^8 p, so LSE = m + ln(l / 2^8) does not
// depend on the rounding, and O = dv * (sum_j Pq_j V_j) / l.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));   // 32 e4m3 values: one MFMA operand

// 32x32x64 e4m3 x e4m3 -> fp32 (format code 0 for both operands; with zero
// scale operands the compiler emits the unscaled instruction).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

constexpr int kF8Bc = 64;         // keys per step
constexpr int kF8Waves = 4;       // waves per workgroup, 32 query rows each
constexpr float kF8PLog2 = 8.0f;  // p is rounded as 2^8 p
// The reference max moves only when some row's max exceeds it by more than
// this (log2 units): then 2^8 p <= 2^8.75 < 448, the largest e4m3 value, so
// no probability overflows, and most steps skip the rescale of O.
constexpr float kF8Slack = 0.75f;

struct Fp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* vt;   // [B H, D, Nkp] transposed V, keys >= Nk zero
  __bf16* o;
  float* lse;
  int H, N, Nk, Nkp, nqt, BH, qoff;
  float c;    // scale * dq * dk * log2(e)
  float dv;
};

// 16-byte chunk swizzles (physical chunk = logical chunk ^ swizzle(row)).
//  K tile, rows of D bytes: the 8 lanes of a read group address rows
//  {0,1,2,3,32,33,34,35} + const, which the swizzle spreads over distinct
//  16-byte bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128) return (row & 3) | (((row >> 5) & 1) << 2);
  else return ((row >> 1) & 1) | (((row >> 5) & 1) << 1);
}
//  V^T tile, rows (one per d) of 64 bytes: a read group addresses 8
//  consecutive rows.
__device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 3; }

// 32 bytes at LDS offsets off and off ^ 16 (two 16-byte chunks of a row).
__device__ __forceinline__ i32x8 lds_read32(const char* base, uint32_t off) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(base + off);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(base + (off ^ 16u));
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Four floats to four e4m3 codes (round to nearest even), first value in the
// lowest byte.  Each conversion writes one 16-bit half of its destination and
// keeps the other; both halves are written here, so `old` (any value, e.g.
// the register's previous contents) does not reach the result.
__device__ __forceinline__ int pack_e4m3x4(int old, float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// ---- V -> V^T: one workgroup per 64 keys of one head.
template <int D>
__global__ __launch_bounds__(256) void fp8_vt_kernel(const uint8_t* __restrict__ v, uint8_t* __restrict__ vt,
                                                     int H, int Nk, int Nkp) {
  constexpr int CH = D / 16;
  __shared__ uint32_t tile[kF8Bc][D / 4 + 1];   // [key][d / 4], padded row
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int k0 = blockIdx.x * kF8Bc;
  const int64_t rs = (int64_t)H * D;
  const uint8_t* src = v + ((int64_t)b * Nk * H + h) * D;
  for (int c = threadIdx.x; c < kF8Bc * CH; c += 256) {
    const int row = c / CH, ch = c - row * CH;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (k0 + row < Nk) x = *reinterpret_cast<const u32x4*>(src + (int64_t)(k0 + row) * rs + ch * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) tile[row][4 * ch + j] = x[j];
  }
  block_sync();
  uint8_t* dst = vt + (int64_t)bh * D * Nkp + k0;
  for (int c = threadIdx.x; c < D * 4; c += 256) {
    const int d = c >> 2, kc = c & 3;   // row d of V^T, keys 16 kc .. 16 kc + 15
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * kc + 4 * j + i;
        x |= ((tile[key][d >> 2] >> (8 * (d & 3))) & 0xFFu) << (8 * i);
      }
      w[j] = x;
    }
    *reinterpret_cast<u32x4*>(dst + (int64_t)d * Nkp + 16 * kc) = w;
  }
}

// ---- forward
// Occupancy: 3 waves per SIMD at d = 128 (168 VGPRs; at the compiler's own
// choice of 170 only 2 fit, measured 4-5% slower on [4, 4096, 16, 128]) and 4
// at d = 64 (<= 116 VGPRs).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kF8Waves, (D == 128 ? 3 : 4)) void fwd_fp8_kernel(Fp8Args a) {
  constexpr int CH = D / 16;               // 16-byte chunks per K row
  constexpr int KS = D / 64;               // k-steps of the score product
  constexpr int DT = D / 32;               // 32-row output tiles
  constexpr int TILE = kF8Bc * D;          // bytes of a K tile and of a V^T tile
  constexpr int CPW = TILE / 1024 / kF8Waves;   // 1 KB copies per wave per tile
  constexpr int kBr = 32 * kF8Waves;
  static_assert(CPW >= 1, "tile copies");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];   // K0, K1, V^T0, V^T1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;

  int bh, qt;
  tile_of(blockIdx.x, a.nqt, a.BH, CAUSAL, true, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, Nk = a.Nk, Nkp = a.Nkp, qoff = a.qoff;
  const int64_t rs = (int64_t)a.H * D;     // row stride (elements = bytes for e4m3)
  const int64_t base = ((int64_t)b * N * a.H + h) * D;
  const uint8_t* __restrict__ Qg = a.q + base;
  const uint8_t* __restrict__ Kg = a.k + ((int64_t)b * Nk * a.H + h) * D;
  const uint8_t* __restrict__ Vtg = a.vt + (int64_t)bh * D * Nkp;

  const int q0 = qt * kBr;
  const int qw0 = q0 + 32 * wave;
  const int myq = qw0 + l32;

  // Q^T operand: bytes 64 ks + 32 (l / 32) .. + 31 of the lane's row.
  i32x8 qf[KS];
  {
    const uint8_t* qrow = Qg + (int64_t)min(myq, N - 1) * rs;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 32 * hh);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 32 * hh + 16);
      qf[ks] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  const int kend = CAUSAL ? min(Nk, q0 + qoff + kBr) : Nk;
  const int nkt = (kend + kF8Bc - 1) / kF8Bc;

  // Staging.  Copy i of this wave fills 1 KB block (wave + 4 i) of a tile;
  // lane l's 16 bytes are LDS chunk p = 64 block + l.  K: row p / CH, physical
  // chunk p % CH, holding logical chunk (p % CH) ^ k_swz(row) of key row k0 +
  // row.  V^T: row p / 4 (a d index), physical chunk p % 4, holding keys
  // k0 + 16 ((p % 4) ^ v_swz(row)) .. + 15.  The K descriptor covers the
  // tile's valid rows only (rows past Nk read as zero and are masked).
  uint32_t koff[CPW], voff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int p = 64 * (wave + kF8Waves * i) + lane;
    const int kr = p / CH, kpc = p % CH;
    koff[i] = (uint32_t)(kr * rs) + (uint32_t)((kpc ^ k_swz<D>(kr)) * 16);
    const int vr = p >> 2, vpc = p & 3;
    voff[i] = (uint32_t)(vr * Nkp) + (uint32_t)((vpc ^ v_swz(vr)) * 16);
  }
  char* const kbuf = smem;
  char* const vbuf = smem + 2 * TILE;
  const int wblk = wave * 1024;
  auto stage = [&](int kt, int buf) __attribute__((always_inline)) {
    const int k0 = kt * kF8Bc;
    const int rows = min(Nk - k0, kF8Bc);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (int64_t)k0 * rs, (uint32_t)(rows * rs));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vtg + k0, (uint32_t)(D * Nkp - k0));
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      buffer_to_lds16(rk, koff[i], kbuf + buf * TILE + wblk + kF8Waves * 1024 * i);
      buffer_to_lds16(rv, voff[i], vbuf + buf * TILE + wblk + kF8Waves * 1024 * i);
    }
  };

  // Fragment lane bases.  K (A operand of S^T, sub-tile t): MFMA row m = l %
  // 32 reads key row 32 ((m / 4) % 2) + 16 t + 4 (m / 8) + m % 4, so the
  // output row (r / 4) 8 + 4 (l / 32) + r % 4 of sub-tile t is key
  // 32 (l / 32) + 16 t + r; logical chunks 4 ks + 2 (l / 32) + {0, 1}.
  const int krow = ((l32 >> 2) & 1) * 32 + (l32 >> 3) * 4 + (l32 & 3);
  const uint32_t kl = (uint32_t)(krow * D) | ((uint32_t)((2 * hh) ^ k_swz<D>(krow)) << 4);
  //  V^T (A operand of O^T, tile dt): row 32 dt + l % 32, keys
  //  32 (l / 32) .. + 31 = logical chunks 2 (l / 32) + {0, 1}.
  const uint32_t vl = (uint32_t)(l32 * kF8Bc) | ((uint32_t)((2 * hh) ^ v_swz(l32)) << 4);

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = (f32x16){};
  float m_ref = -INFINITY;   // reference row max, log2 units
  float m_thr = -INFINITY;   // m_ref + kF8Slack: a row max above it moves the reference
  float nm = 0.f;            // exponent offset 8 - m_ref (0 while m_ref = -inf)
  float l_part = 0.f;        // this half-wave's share of sum 2^8 p
  const float c = a.c;

  auto scores = [&](const char* kb, f32x16 (&s)[2]) __attribute__((always_inline)) {
    s[0] = (f32x16){};
    s[1] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        s[t] = mfma_fp8(lds_read32(kb, (kl ^ (uint32_t)(ks << 6)) + (uint32_t)(16 * t * D)), qf[ks], s[t]);
  };

  // Softmax of one step against a reference max at most kF8Slack below the
  // running max (moved to the exact running max when it falls further
  // behind), and P as e4m3 codes.
  auto softmax = [&](auto mask_tag, f32x16 (&s)[2], int k0, i32x8& pf) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * hh + 16 * t + r;
          const bool hide = key >= Nk || (CAUSAL && key > myq + qoff);
          s[t][r] = hide ? -INFINITY : s[t][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = max_halves(mx);
    // (a row max of -inf, whose product with c could be a NaN, only occurs
    // under the mask)
    const float mcand = MASK ? ((mx == -INFINITY) ? -INFINITY : mx * c) : mx * c;
    if (__any(mcand > m_thr)) {
      const float m_new = fmaxf(m_ref, mcand);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      m_ref = m_new;
      m_thr = m_new + kF8Slack;
      nm = (m_new == -INFINITY) ? 0.f : kF8PLog2 - m_new;
    }
    float p[32];
    float lsum[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = fast_exp2(__builtin_fmaf(s[t][r], c, nm));
        if constexpr (MASK) e = (s[t][r] == -INFINITY) ? 0.f : e;
        p[16 * t + r] = e;
        lsum[r & 1] += e;
      }
    l_part += lsum[0] + lsum[1];
#pragma unroll
    for (int v = 0; v < 8; ++v) pf[v] = pack_e4m3x4(pf[v], p[4 * v], p[4 * v + 1], p[4 * v + 2], p[4 * v + 3]);
  };

  auto pv = [&](const char* vb, const i32x8& pf) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
      oacc[t] = mfma_fp8(lds_read32(vb, vl + (uint32_t)(32 * t * kF8Bc)), pf, oacc[t]);
  };

  // Step kt: K and V^T of tile kt are in buffer kt & 1; tile kt + 1 is copied
  // into the other buffer meanwhile.  `buf_tag` is that buffer index, a
  // compile-time constant in the two-step loops.
  stage(0, 0);
  // P as e4m3 codes; each step's packing starts from the previous step's
  // registers (both halves of every word are overwritten).
  i32x8 pf = {};
  auto step = [&](int kt, auto mask_tag, auto buf_tag) __attribute__((always_inline)) {
    const int cur = buf_tag;
    wait_vmem();
    block_sync();
    if (kt + 1 < nkt) stage(kt + 1, cur ^ 1);
    const int k0 = kt * kF8Bc;
    if (CAUSAL && k0 > qw0 + qoff + 31) return;   // no key of the tile is visible to this wave
    f32x16 s[2];
    scores(kbuf + cur * TILE, s);
    softmax(mask_tag, s, k0, pf);
    pv(vbuf + cur * TILE, pf);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // Tiles [0, nfree) need no mask for any row of this wave: whole tiles below
  // the wave's first row (causal) and before the ragged end.  The rest take
  // the masked path.  Every wave runs all nkt steps (each has a barrier).
  const int nfull = Nk / kF8Bc;
  const int nfree = __builtin_amdgcn_readfirstlane(
      CAUSAL ? min(nfull, max(0, (qw0 + qoff + 1) / kF8Bc)) : min(nfull, nkt));
  int kt = 0;
  for (; kt + 1 < nfree; kt += 2) {
    step(kt, std::false_type{}, B0{});
    step(kt + 1, std::false_type{}, B1{});
  }
  if (kt < nfree) step(kt++, std::false_type{}, B0{});
  for (; kt < nkt; ++kt) step(kt, std::true_type{}, kt & 1);
  wait_vmem();

  // ---- epilogue: O = dv O_acc / l, LSE = ln2 (m + log2 l - 8)
  const float l = sum_halves(l_part);
  if (myq < N) {
    const float inv = a.dv / l;
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
    if (hh == 0) a.lse[(int64_t)bh * N + myq] = kLn2 * (m_ref + fast_log2(l) - kF8PLog2);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(Fp8Args args, const uint8_t* v, uint8_t* vt, hipStream_t stream) {
  hipLaunchKernelGGL((fp8_vt_kernel<D>), dim3(args.Nkp / kF8Bc, args.BH), dim3(256), 0, stream,
                     v, vt, args.H, args.Nk, args.Nkp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  args.nqt = (args.N + 32 * kF8Waves - 1) / (32 * kF8Waves);
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3(args.nqt * args.BH), dim3(64 * kF8Waves), 0, stream,
                     args);
  return hipGetLastError();
}

}  // namespace

size_t fwd_fp8_workspace_bytes(int B, int H, int Nk, int d) {
  const size_t nkp = ((size_t)Nk + kF8Bc - 1) / kF8Bc * kF8Bc;
  return (size_t)B * H * d * nkp;
}

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, float dq, float dk, float dv,
                          void* o, float* lse, void* ws, const AttnShape& s, int Nk, hipStream_t stream) {
  Fp8Args a;
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.vt = static_cast<const uint8_t*>(ws);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.H = s.H;
  a.N = s.N;
  a.Nk = Nk;
  a.Nkp = (Nk + kF8Bc - 1) / kF8Bc * kF8Bc;
  a.BH = s.B * s.H;
  a.qoff = s.causal ? Nk - s.N : 0;
  a.c = s.scale * dq * dk * kLog2e;
  a.dv = dv;
  const uint8_t* vv = static_cast<const uint8_t*>(v);
  uint8_t* vt = static_cast<uint8_t*>(ws);
  if (s.d == 64) return s.causal ? launch<64, true>(a, vv, vt, stream) : launch<64, false>(a, vv, vt, stream);
  return s.causal ? launch<128, true>(a, vv, vt, stream) : launch<128, false>(a, vv, vt, stream);
}

}  // namespace fa
