// fa_f32.hip - float32 forward and backward on the fp32 matrix cores.
//
// Same algorithm as the bf16 kernels, in fp32 throughout: tiles of the
// streamed operand pass through LDS, the running max, running sum and the
// unnormalised output stay in registers (page "FlashAttention", vagrantpi
// PKM note, "三招" items 1-3: tiling, online softmax, recomputation).  The
// backward rebuilds P = exp(scale q k^T - LSE) and follows the chain rule of
// softmax: dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
// dQ = scale dS K, dK = scale dS^T Q.
//
// Every product runs on v_mfma_f32_16x16x4_f32 (wave64, one block):
//   A (16 x 4): lane l holds row l%16, k = l/16
//   B (4 x 16): lane l holds column l%16, k = l/16
//   C (16 x 16): lane l, register r holds row 4*(l/16) + r, column l%16
// A contraction may visit k in any order as long as A and B agree, so the
// kernels pick the order that lets each lane read four consecutive floats,
// and they feed a C fragment straight back in as the B operand of the next
// product: with S^T = K Q^T in C layout, lane l already holds P^T for keys
// 4*(l/16) + r of its query column, which is what O^T = V^T P^T needs as B
// when step r of the contraction maps lane group l/16 to key 4*(l/16) + r.
// The A operand of that product (V^T, Q^T, dO^T or K^T) is kept transposed in
// LDS so that the same four keys are one 16-byte read.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16 * kWaves;   // resident rows per workgroup, 16 per wave
constexpr int kTile = 32;            // streamed rows per LDS stage
constexpr int kPad = 4;              // floats of padding per LDS row

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dout;
  const float* lse;
  const float* dvec;
  float* out0;   // O (forward), dK (dK/dV pass) or dQ (dQ pass)
  float* out1;   // LSE (forward) or dV (dK/dV pass)
  int H, N, ntiles;
  float scale;
};

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }

// Reductions over the four lanes l, l^16, l^32, l^48 that share a column.
__device__ __forceinline__ float col_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float col_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int D>
__device__ __forceinline__ void bh_coords(const F32Args& a, int& bh, int& tile, int64_t& base) {
  bh = blockIdx.x / a.ntiles;
  tile = blockIdx.x - bh * a.ntiles;
  const int b = bh / a.H, h = bh - b * a.H;
  base = ((int64_t)b * a.N * a.H + h) * D;
}

// Stage kTile rows of `src` starting at row r0 into LDS: row-major (stride
// D + kPad) into `rm` and, if `tr` is given, transposed (stride kTile + kPad)
// into `tr`.  Rows past N read as zero.
template <int D>
__device__ __forceinline__ void stage(const float* src, int64_t base, int64_t rs, int r0, int N,
                                      float* rm, float* tr) {
  constexpr int C4 = D / 4;
  for (int idx = threadIdx.x; idx < kTile * C4; idx += kThreads) {
    const int r = idx / C4, c = (idx - r * C4) * 4;
    const int row = r0 + r;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < N) x = ld4(src + base + (int64_t)row * rs + c);
    if (rm) st4(rm + r * (D + kPad) + c, x);
    if (tr) {
      tr[(c + 0) * (kTile + kPad) + r] = x.x;
      tr[(c + 1) * (kTile + kPad) + r] = x.y;
      tr[(c + 2) * (kTile + kPad) + r] = x.z;
      tr[(c + 3) * (kTile + kPad) + r] = x.w;
    }
  }
}

// C += X Y^T over the head dimension for one 16 x 16 tile, where lane l
// supplies row l%16 of X from LDS (row-major, stride D + kPad, starting at
// row x0) and its own 16 B-operand floats of Y (row l%16 of Y at columns
// 16c + 4(l/16) .. +3, c = 0 .. D/16 - 1).
template <int D>
__device__ __forceinline__ f32x4 dot_rows(const float* xs, int x0, const float4 (&y)[D / 16], f32x4 c) {
  const int lane = threadIdx.x & 63;
  const float* xr = xs + (x0 + (lane & 15)) * (D + kPad) + 4 * (lane >> 4);
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    const float4 x = ld4(xr + 16 * cc);
    c = mma(x.x, y[cc].x, c);
    c = mma(x.y, y[cc].y, c);
    c = mma(x.z, y[cc].z, c);
    c = mma(x.w, y[cc].w, c);
  }
  return c;
}

// acc[dt] += Xt[16dt .. 16dt+15, t0 + 0 .. 15] * F, where Xt is a transposed
// LDS tile (stride kTile + kPad) and F is a C fragment (rows t0 + 4(l/16) + r
// of the contraction, column l%16) used as the B operand.
template <int D>
__device__ __forceinline__ void acc_tr(f32x4 (&acc)[D / 16], const float* xt, int t0, const f32x4& f) {
  const int lane = threadIdx.x & 63;
  const float* xr = xt + (lane & 15) * (kTile + kPad) + t0 + 4 * (lane >> 4);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const float4 x = ld4(xr + 16 * dt * (kTile + kPad));
    acc[dt] = mma(x.x, f[0], acc[dt]);
    acc[dt] = mma(x.y, f[1], acc[dt]);
    acc[dt] = mma(x.z, f[2], acc[dt]);
    acc[dt] = mma(x.w, f[3], acc[dt]);
  }
}

// Lane l's 16 B-operand floats of one row: row[16c + 4(l/16) .. +3].
template <int D>
__device__ __forceinline__ void load_row(float4 (&y)[D / 16], const float* row) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) y[cc] = ld4(row + 16 * cc + 4 * g);
}

// Store a transposed accumulator (rows = head dimension, column l%16 = the
// lane's row of the output) as the lane's slice of that output row.
template <int D>
__device__ __forceinline__ void store_row(float* row, const f32x4 (&acc)[D / 16], float mul) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    st4(row + 16 * dt + 4 * g, make_float4(acc[dt][0] * mul, acc[dt][1] * mul, acc[dt][2] * mul, acc[dt][3] * mul));
}

// Forward: wave w owns queries tile*64 + 16w + l%16 (the columns of S^T).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args a) {
  __shared__ float ks[kTile * (D + kPad)];
  __shared__ float vt[D * (kTile + kPad)];
  int bh, tile;
  int64_t base;
  bh_coords<D>(a, bh, tile, base);
  const int N = a.N, lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int64_t rs = (int64_t)a.H * D;
  const int qw = tile * kRows + 16 * w;   // first query of this wave
  const int myq = qw + (lane & 15);

  float4 qv[D / 16];
  load_row<D>(qv, a.q + base + (int64_t)min(myq, N - 1) * rs);
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int kend = CAUSAL ? min(N, tile * kRows + kRows) : N;
  for (int k0 = 0; k0 < kend; k0 += kTile) {
    block_sync();
    stage<D>(a.k, base, rs, k0, N, ks, nullptr);
    stage<D>(a.v, base, rs, k0, N, nullptr, vt);
    block_sync();
    if (CAUSAL && k0 > qw + 15) continue;   // the whole stage is above this wave's diagonal
    f32x4 s[kTile / 16];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < kTile / 16; ++t) {
      s[t] = dot_rows<D>(ks, 16 * t, qv, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 16 * t + 4 * g + r;
        s[t][r] = (key >= N || (CAUSAL && key > myq)) ? -INFINITY : s[t][r] * a.scale;
        mx = fmaxf(mx, s[t][r]);
      }
    }
    mx = col_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < kTile / 16; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[t][r] = (s[t][r] == -INFINITY) ? 0.f : expf(s[t][r] - m_new);
        ps += s[t][r];
      }
    l = l * alpha + col_sum(ps);
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int t = 0; t < kTile / 16; ++t) acc_tr<D>(o, vt, 16 * t, s[t]);
  }
  if (myq < N) {
    store_row<D>(a.out0 + base + (int64_t)myq * rs, o, 1.f / l);
    if (g == 0) a.out1[(int64_t)bh * N + myq] = m + logf(l);
  }
}

// D_i = sum_c dO_ic O_ic: one thread per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(const float* o, const float* dout,
                                                          float* dvec, int H, int N, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const float* op = o + r * D;
  const float* gp = dout + r * D;
  float acc = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; ++c) acc = __builtin_fmaf(op[c], gp[c], acc);
  const int64_t h = r % H, bn = r / H;
  const int64_t n = bn % N, b = bn / N;
  dvec[(b * H + h) * N + n] = acc;
}

// dK, dV: wave w owns keys tile*64 + 16w + l%16 (the columns of S = Q K^T)
// and walks every query that can see them, 32 per LDS stage.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_f32_kernel(F32Args a) {
  __shared__ float qs[kTile * (D + kPad)];
  __shared__ float gs[kTile * (D + kPad)];
  __shared__ float qt[D * (kTile + kPad)];
  __shared__ float gt[D * (kTile + kPad)];
  __shared__ float ls[kTile], dd[kTile];
  int bh, tile;
  int64_t base;
  bh_coords<D>(a, bh, tile, base);
  const int N = a.N, lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int64_t rs = (int64_t)a.H * D;
  const int kw = tile * kRows + 16 * w;   // first key of this wave
  const int myk = kw + (lane & 15);

  float4 kv[D / 16], vv[D / 16];
  load_row<D>(kv, a.k + base + (int64_t)min(myk, N - 1) * rs);
  load_row<D>(vv, a.v + base + (int64_t)min(myk, N - 1) * rs);
  f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* lse = a.lse + (int64_t)bh * N;
  const float* dvec = a.dvec + (int64_t)bh * N;

  const int qstart = CAUSAL ? tile * kRows : 0;   // earlier queries see none of these keys
  for (int i0 = qstart; i0 < N; i0 += kTile) {
    block_sync();
    stage<D>(a.q, base, rs, i0, N, qs, qt);
    stage<D>(a.dout, base, rs, i0, N, gs, gt);
    if (threadIdx.x < kTile) {
      const int qi = i0 + threadIdx.x;
      ls[threadIdx.x] = qi < N ? lse[qi] : 0.f;
      dd[threadIdx.x] = qi < N ? dvec[qi] : 0.f;
    }
    block_sync();
    if (CAUSAL && i0 + kTile - 1 < kw) continue;   // no query of the stage sees this wave's keys
#pragma unroll
    for (int u = 0; u < kTile / 16; ++u) {
      f32x4 s = dot_rows<D>(qs, 16 * u, kv, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 dp = dot_rows<D>(gs, 16 * u, vv, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * u + 4 * g + r;
        const int qi = i0 + row;
        const bool vis = qi < N && !(CAUSAL && myk > qi);
        const float p = vis ? expf(s[r] * a.scale - ls[row]) : 0.f;
        s[r] = p;
        dp[r] = p * (dp[r] - dd[row]);
      }
      acc_tr<D>(dv, gt, 16 * u, s);
      acc_tr<D>(dk, qt, 16 * u, dp);
    }
  }
  if (myk < N) {
    store_row<D>(a.out0 + base + (int64_t)myk * rs, dk, a.scale);
    store_row<D>(a.out1 + base + (int64_t)myk * rs, dv, 1.f);
  }
}

// dQ: wave w owns queries tile*64 + 16w + l%16 (the columns of S^T = K Q^T)
// and walks every key they can see, 32 per LDS stage.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32_kernel(F32Args a) {
  __shared__ float ks[kTile * (D + kPad)];
  __shared__ float vs[kTile * (D + kPad)];
  __shared__ float kt[D * (kTile + kPad)];
  int bh, tile;
  int64_t base;
  bh_coords<D>(a, bh, tile, base);
  const int N = a.N, lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int64_t rs = (int64_t)a.H * D;
  const int qw = tile * kRows + 16 * w;
  const int myq = qw + (lane & 15);
  const int qc = min(myq, N - 1);

  float4 qv[D / 16], gv[D / 16];
  load_row<D>(qv, a.q + base + (int64_t)qc * rs);
  load_row<D>(gv, a.dout + base + (int64_t)qc * rs);
  const float lse = a.lse[(int64_t)bh * N + qc];
  const float dvl = a.dvec[(int64_t)bh * N + qc];
  f32x4 dq[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kend = CAUSAL ? min(N, tile * kRows + kRows) : N;
  for (int k0 = 0; k0 < kend; k0 += kTile) {
    block_sync();
    stage<D>(a.k, base, rs, k0, N, ks, kt);
    stage<D>(a.v, base, rs, k0, N, vs, nullptr);
    block_sync();
    if (CAUSAL && k0 > qw + 15) continue;
#pragma unroll
    for (int t = 0; t < kTile / 16; ++t) {
      f32x4 s = dot_rows<D>(ks, 16 * t, qv, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 dp = dot_rows<D>(vs, 16 * t, gv, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 16 * t + 4 * g + r;
        const bool vis = key < N && !(CAUSAL && key > myq);
        const float p = vis ? expf(s[r] * a.scale - lse) : 0.f;
        dp[r] = p * (dp[r] - dvl);
      }
      acc_tr<D>(dq, kt, 16 * t, dp);
    }
  }
  if (myq < N) store_row<D>(a.out0 + base + (int64_t)myq * rs, dq, a.scale);
}

template <int D>
hipError_t fwd(const F32Args& a, int BH, int causal, hipStream_t st) {
  const dim3 grid(a.ntiles * BH), block(kThreads);
  if (causal) hipLaunchKernelGGL((fwd_f32_kernel<D, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((fwd_f32_kernel<D, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t bwd(const F32Args& a, int B, int BH, int causal, hipStream_t st) {
  const int64_t rows = (int64_t)B * a.N * a.H;
  hipLaunchKernelGGL((bwd_pre_f32_kernel<D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st,
                     a.o, a.dout, const_cast<float*>(a.dvec), a.H, a.N, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.ntiles * BH), block(kThreads);
  if (causal) hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_dq(const F32Args& a, int BH, int causal, hipStream_t st) {
  const dim3 grid(a.ntiles * BH), block(kThreads);
  if (causal) hipLaunchKernelGGL((bwd_dq_f32_kernel<D, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((bwd_dq_f32_kernel<D, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const AttnShape& s, hipStream_t stream) {
  F32Args a{};
  a.q = q; a.k = k; a.v = v;
  a.out0 = o; a.out1 = lse;
  a.H = s.H; a.N = s.N;
  a.ntiles = (s.N + kRows - 1) / kRows;
  a.scale = s.scale;
  const int BH = s.B * s.H;
  return s.d == 64 ? fwd<64>(a, BH, s.causal, stream) : fwd<128>(a, BH, s.causal, stream);
}

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* dvec, const AttnShape& s, hipStream_t stream) {
  F32Args a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse; a.dvec = dvec;
  a.out0 = dk; a.out1 = dv;
  a.H = s.H; a.N = s.N;
  a.ntiles = (s.N + kRows - 1) / kRows;
  a.scale = s.scale;
  const int BH = s.B * s.H;
  hipError_t e = s.d == 64 ? bwd<64>(a, s.B, BH, s.causal, stream) : bwd<128>(a, s.B, BH, s.causal, stream);
  if (e != hipSuccess) return e;
  a.out0 = dq; a.out1 = nullptr;
  return s.d == 64 ? bwd_dq<64>(a, BH, s.causal, stream) : bwd_dq<128>(a, BH, s.causal, stream);
}

}  // namespace fa
