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
//   1. bwd_pre  : D = rowsum(dO * O) in fp32, streaming both tensors once.
//   2. bwd_dkdv : one workgroup per 128 keys (32 per wave, K and V of those
//                 keys resident in registers); walks the query tiles that can
//                 see them, staging Q, dO, LSE and D through double-buffered
//                 LDS.  S = Q K^T and dP = dO V^T use 32x32x16 MFMA with the
//                 key as the lane, so P and dS come out in the B-operand
//                 layout of dV^T += dO^T P and dK^T += Q^T dS, whose A
//                 operands are transposing LDS reads of the dO and Q tiles.
//   3. bwd_dq   : one workgroup per 128 queries (32 per wave, Q and dO of those
//                 rows resident); walks the key tiles they can see.  S^T and
//                 dP^T have the query as the lane, so LSE_i and D_i are one
//                 scalar per lane, and dS^T feeds dQ^T += K^T dS^T directly.
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
  const float* dvec;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* dvec_out;
  int H, N, ntiles;
  float c;       // scale * log2(e)
  float scale;
};

// ------------------------------------------------------------------ D = rowsum(dO * O)
// CH = D/8 lanes share a row, each reading one 16-byte chunk of O and of dO;
// the whole [B, N, H, d] tensors are read front to back.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ o,
                                                      const __bf16* __restrict__ dout,
                                                      float* __restrict__ dvec, int H, int N,
                                                      int64_t rows) {
  constexpr int CH = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / CH;
  const int ch = (int)(gid % CH);
  float acc = 0.f;
  if (r < rows) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(o + r * D + ch * 8);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(dout + r * D + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
  }
#pragma unroll
  for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, CH);
  if (r < rows && ch == 0) {
    const int64_t h = r % H, bn = r / H;
    const int64_t n = bn % N, b = bn / N;
    dvec[(b * H + h) * N + n] = acc;
  }
}

// A-operand fragment of a transposed tile: element (row = d, k = tile row) of
// the 32x32x16 MFMA for output d-tile t and k-step u of a 32-row block j.
// Lane l gets d = 32 t + l%32 and tile rows 32 j + 16 u + 4 (l/32) + {0..3}
// (low half) and the same + 8 (high half), matching the B operand built from
// accumulator registers 8u .. 8u+7 of a C fragment.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int lane, int t, int j, int u) {
  const int i = lane & 15, g = lane >> 4;
  const int row = 32 * j + 16 * u + (g >> 1) * 4 + (i >> 2);
  const int col = t * 32 + (g & 1) * 16 + (i & 3) * 4;
  const bf16x4 lo = __builtin_bit_cast(bf16x4, lds_read_tr16(tile, elem_off<D>(row, col)));
  const bf16x4 hi = __builtin_bit_cast(bf16x4, lds_read_tr16(tile, elem_off<D>(row + 8, col)));
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
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
constexpr int kBq = 32;           // queries per step

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int CH = D / 8, KS = D / 16, DT = D / 32;
  constexpr int TILE = kBq * D * 2;
  constexpr int CPT = (kBq * CH + 255) / 256;   // chunks per thread per tensor
  __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];   // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float sl[2][kBq];        // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float sd[2][kBq];        // D

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / a.ntiles;
  const int kt = L - bh * a.ntiles;          // low key tiles see the most queries: run first
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = ((int64_t)b * N * a.H + h) * D;
  const float* lse = a.lse + (int64_t)bh * N;
  const float* dvec = a.dvec + (int64_t)bh * N;

  const int k0 = kt * kKeysPerWg;
  const int kw0 = k0 + 32 * wave;
  const int mykey = kw0 + l32;

  // K^T and V^T as B operands: this lane's key, chunk 2 ks + hh.
  bf16x8 kf[KS], vf[KS];
  {
    const int64_t kr = min(mykey, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(a.k + base + kr * rs + (2 * ks + hh) * 8);
      vf[ks] = *reinterpret_cast<const bf16x8*>(a.v + base + kr * rs + (2 * ks + hh) * 8);
    }
  }
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) { dk[t] = (f32x16){}; dv[t] = (f32x16){}; }

  const int qstart = CAUSAL ? k0 : 0;
  const int nsteps = (N - qstart + kBq - 1) / kBq;

  u32x4 qreg[CPT], greg[CPT];
  float lreg = 0.f, dreg = 0.f;
  auto gload = [&](int s) {
    const int qi0 = qstart + s * kBq;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i;
      if (idx < kBq * CH) {
        const int row = idx / CH, ch = idx % CH;
        const int64_t qr = min(qi0 + row, N - 1);
        qreg[i] = *reinterpret_cast<const u32x4*>(a.q + base + qr * rs + ch * 8);
        greg[i] = *reinterpret_cast<const u32x4*>(a.dout + base + qr * rs + ch * 8);
      }
    }
    if (tid < kBq) {
      const int qr = min(qi0 + tid, N - 1);
      lreg = lse[qr] * kLog2e;
      dreg = dvec[qr];
    }
  };
  auto swrite = [&](int stage) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i;
      if (idx < kBq * CH) {
        const int row = idx / CH, ch = idx % CH;
        const uint32_t off = tile_off<D>(row, ch);
        *reinterpret_cast<u32x4*>(smem[stage][0] + off) = qreg[i];
        *reinterpret_cast<u32x4*>(smem[stage][1] + off) = greg[i];
      }
    }
    if (tid < kBq) {
      sl[stage][tid] = lreg;
      sd[stage][tid] = dreg;
    }
  };

  const float c = a.c;
  gload(0);
  for (int s = 0; s < nsteps; ++s) {
    const int stage = s & 1;
    swrite(stage);
    __syncthreads();
    if (s + 1 < nsteps) gload(s + 1);

    const int qi0 = qstart + s * kBq;
    if (CAUSAL && qi0 + kBq - 1 < kw0) continue;   // every query precedes this wave's keys
    const char* qt = smem[stage][0];
    const char* gt = smem[stage][1];

    // S = Q K^T and dP = dO V^T: lane = key, register r = query row 8(r/4) + 4hh + r%4.
    f32x16 sacc = (f32x16){}, pacc = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 qa = lds_read_b128(qt, tile_off<D>(l32, 2 * ks + hh));
      const bf16x8 ga = lds_read_b128(gt, tile_off<D>(l32, 2 * ks + hh));
      sacc = mfma32x32x16(qa, kf[ks], sacc);
      pacc = mfma32x32x16(ga, vf[ks], pacc);
    }
    f32x4 lq[4], dq4[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      lq[g4] = *reinterpret_cast<const f32x4*>(&sl[stage][8 * g4 + 4 * hh]);
      dq4[g4] = *reinterpret_cast<const f32x4*>(&sd[stage][8 * g4 + 4 * hh]);
    }
    const bool masked = (qi0 + kBq > N) || (CAUSAL && kw0 + 31 > qi0);
    float p[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float lv = lq[r >> 2][r & 3], dv4 = dq4[r >> 2][r & 3];
      float pv = fast_exp2(__builtin_fmaf(sacc[r], c, -lv));
      if (masked) {
        const int qrow = qi0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool hide = qrow >= N || (CAUSAL && mykey > qrow);
        pv = hide ? 0.f : pv;
      }
      p[r] = pv;
      ds[r] = pv * (pacc[r] - dv4);
    }
    bf16x8 pb[2], db[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pb[u] = pack_bf16x8(p[8 * u], p[8 * u + 1], p[8 * u + 2], p[8 * u + 3],
                          p[8 * u + 4], p[8 * u + 5], p[8 * u + 6], p[8 * u + 7]);
      db[u] = pack_bf16x8(ds[8 * u], ds[8 * u + 1], ds[8 * u + 2], ds[8 * u + 3],
                          ds[8 * u + 4], ds[8 * u + 5], ds[8 * u + 6], ds[8 * u + 7]);
    }
    // dV^T += dO^T P ; dK^T += Q^T dS   (rows d, columns keys)
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        dv[t] = mfma32x32x16(tr_frag<D>(gt, lane, t, 0, u), pb[u], dv[t]);
        dk[t] = mfma32x32x16(tr_frag<D>(qt, lane, t, 0, u), db[u], dk[t]);
      }
  }

  if (mykey < N) {
    store_row_frags<D>(a.dk + base + (int64_t)mykey * rs, dk, hh, a.scale);
    store_row_frags<D>(a.dv + base + (int64_t)mykey * rs, dv, hh, 1.f);
  }
}

// ------------------------------------------------------------------ dQ pass
constexpr int kQPerWg = 128;   // 4 waves x 32 queries
constexpr int kBk = 64;        // keys per step

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int CH = D / 8, KS = D / 16, DT = D / 32;
  constexpr int TILE = kBk * D * 2;
  constexpr int CPT = kBk * CH / 256;
  __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];   // [stage][K, V]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / a.ntiles;
  const int qtile = a.ntiles - 1 - (L - bh * a.ntiles);   // heaviest (causal) first
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N;
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = ((int64_t)b * N * a.H + h) * D;

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
  const float lse2 = a.lse[(int64_t)bh * N + qc] * kLog2e;
  const float dval = a.dvec[(int64_t)bh * N + qc];

  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = (f32x16){};

  const int kend = CAUSAL ? min(N, q0 + kQPerWg) : N;
  const int nkt = (kend + kBk - 1) / kBk;
  u32x4 kreg[CPT], vreg[CPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / CH, ch = idx % CH;
      const int64_t key = min(kt * kBk + row, N - 1);
      kreg[i] = *reinterpret_cast<const u32x4*>(a.k + base + key * rs + ch * 8);
      vreg[i] = *reinterpret_cast<const u32x4*>(a.v + base + key * rs + ch * 8);
    }
  };
  auto swrite = [&](int stage) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / CH, ch = idx % CH;
      const uint32_t off = tile_off<D>(row, ch);
      *reinterpret_cast<u32x4*>(smem[stage][0] + off) = kreg[i];
      *reinterpret_cast<u32x4*>(smem[stage][1] + off) = vreg[i];
    }
  };

  const float c = a.c;
  gload(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int stage = kt & 1;
    swrite(stage);
    __syncthreads();
    if (kt + 1 < nkt) gload(kt + 1);

    const int k0 = kt * kBk;
    if (CAUSAL && k0 > qw0 + 31) continue;
    const char* ktile = smem[stage][0];
    const char* vtile = smem[stage][1];
    const bool masked = (k0 + kBk > N) || (CAUSAL && k0 + kBk - 1 > qw0);

    bf16x8 db[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // S^T = K Q^T and dP^T = V dO^T: lane = query, register r = key 8(r/4) + 4hh + r%4.
      f32x16 sacc = (f32x16){}, pacc = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = lds_read_b128(ktile, tile_off<D>(32 * j + l32, 2 * ks + hh));
        const bf16x8 va = lds_read_b128(vtile, tile_off<D>(32 * j + l32, 2 * ks + hh));
        sacc = mfma32x32x16(ka, qf[ks], sacc);
        pacc = mfma32x32x16(va, gf[ks], pacc);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = fast_exp2(__builtin_fmaf(sacc[r], c, -lse2));
        if (masked) {
          const int key = k0 + 32 * j + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool hide = key >= N || (CAUSAL && key > myq);
          pv = hide ? 0.f : pv;
        }
        ds[r] = pv * (pacc[r] - dval);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        db[j][u] = pack_bf16x8(ds[8 * u], ds[8 * u + 1], ds[8 * u + 2], ds[8 * u + 3],
                               ds[8 * u + 4], ds[8 * u + 5], ds[8 * u + 6], ds[8 * u + 7]);
    }
    // dQ^T += K^T dS^T (rows d, columns queries)
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          dq[t] = mfma32x32x16(tr_frag<D>(ktile, lane, t, j, u), db[j][u], dq[t]);
  }

  if (myq < N) store_row_frags<D>(a.dq + base + (int64_t)myq * rs, dq, hh, a.scale);
}

template <int D>
hipError_t run_pre(const BwdArgs& a, int B, hipStream_t st) {
  const int64_t rows = (int64_t)B * a.N * a.H;
  const int64_t threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     a.o, a.dout, a.dvec_out, a.H, a.N, rows);
  return hipGetLastError();
}

template <int D>
hipError_t run_dkdv(BwdArgs a, int BH, bool causal, hipStream_t st) {
  a.ntiles = (a.N + kKeysPerWg - 1) / kKeysPerWg;
  const dim3 grid(a.ntiles * BH);
  if (causal) hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t run_dq(BwdArgs a, int BH, bool causal, hipStream_t st) {
  a.ntiles = (a.N + kQPerWg - 1) / kQPerWg;
  const dim3 grid(a.ntiles * BH);
  if (causal) hipLaunchKernelGGL((bwd_dq_kernel<D, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((bwd_dq_kernel<D, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

BwdArgs make_args(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, const float* dvec_in, float* dvec_out, void* dq, void* dk,
                  void* dv, const AttnShape& s) {
  BwdArgs a{};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.dvec = dvec_in;
  a.dvec_out = dvec_out;
  a.dq = static_cast<__bf16*>(dq);
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.H = s.H;
  a.N = s.N;
  a.c = s.scale * kLog2e;
  a.scale = s.scale;
  return a;
}

}  // namespace

hipError_t launch_bwd_pre_bf16(const void* o, const void* dout, float* dvec, const AttnShape& s,
                               hipStream_t stream) {
  const BwdArgs a = make_args(nullptr, nullptr, nullptr, o, dout, nullptr, nullptr, dvec, nullptr,
                              nullptr, nullptr, s);
  return s.d == 64 ? run_pre<64>(a, s.B, stream) : run_pre<128>(a, s.B, stream);
}

hipError_t launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const void* dout,
                                const float* lse, const float* dvec, void* dk, void* dv,
                                const AttnShape& s, hipStream_t stream) {
  const BwdArgs a = make_args(q, k, v, nullptr, dout, lse, dvec, nullptr, nullptr, dk, dv, s);
  const int BH = s.B * s.H;
  return s.d == 64 ? run_dkdv<64>(a, BH, s.causal != 0, stream)
                   : run_dkdv<128>(a, BH, s.causal != 0, stream);
}

hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* dout,
                              const float* lse, const float* dvec, void* dq, const AttnShape& s,
                              hipStream_t stream) {
  const BwdArgs a = make_args(q, k, v, nullptr, dout, lse, dvec, nullptr, dq, nullptr, nullptr, s);
  const int BH = s.B * s.H;
  return s.d == 64 ? run_dq<64>(a, BH, s.causal != 0, stream)
                   : run_dq<128>(a, BH, s.causal != 0, stream);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* dvec, const AttnShape& s, hipStream_t stream) {
  hipError_t e = launch_bwd_pre_bf16(o, dout, dvec, s, stream);
  if (e == hipSuccess) e = launch_bwd_dkdv_bf16(q, k, v, dout, lse, dvec, dk, dv, s, stream);
  if (e == hipSuccess) e = launch_bwd_dq_bf16(q, k, v, dout, lse, dvec, dq, s, stream);
  return e;
}

}  // namespace fa
