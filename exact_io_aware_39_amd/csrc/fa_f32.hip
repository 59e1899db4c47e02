// fa_f32.hip - float32 forward and backward (correctness path, plain VALU).
//
// Same algorithm as the bf16 kernels, in fp32 throughout and without matrix
// cores: tiles of K and V pass through LDS, each thread owns one query row (or
// one key row in the dK/dV pass) and keeps its running max, running sum and
// unnormalised output in registers (page "FlashAttention", vagrantpi.github.io
// PKM note, "三招" items 1-3).  The backward rebuilds P = exp(scale q k^T - LSE)
// and follows the chain rule of softmax: dV = P^T dO, dP = dO V^T,
// D = rowsum(dO * O), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kRows = 64;   // query (or key) rows per workgroup, one per thread
constexpr int kTile = 32;   // rows of the streamed operand per step

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

template <int D>
__device__ __forceinline__ void bh_coords(const F32Args& a, int& bh, int& tile, int64_t& base) {
  bh = blockIdx.x / a.ntiles;
  tile = blockIdx.x - bh * a.ntiles;
  const int b = bh / a.H, h = bh - b * a.H;
  base = ((int64_t)b * a.N * a.H + h) * D;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(F32Args a) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  int bh, tile;
  int64_t base;
  bh_coords<D>(a, bh, tile, base);
  const int N = a.N, tid = threadIdx.x;
  const int64_t rs = (int64_t)a.H * D;
  const int myq = tile * kRows + tid;

  float q[D], o[D];
  const float* qrow = a.q + base + (int64_t)min(myq, N - 1) * rs;
#pragma unroll
  for (int c = 0; c < D; ++c) { q[c] = qrow[c]; o[c] = 0.f; }
  float m = -INFINITY, l = 0.f;

  const int kend = CAUSAL ? min(N, tile * kRows + kRows) : N;
  for (int k0 = 0; k0 < kend; k0 += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += kRows) {
      const int r = idx / D, c = idx % D;
      const int key = k0 + r;
      ks[r][c] = key < N ? a.k[base + (int64_t)key * rs + c] : 0.f;
      vs[r][c] = key < N ? a.v[base + (int64_t)key * rs + c] : 0.f;
    }
    __syncthreads();
    float s[kTile];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = __builtin_fmaf(q[c], ks[j][c], dot);
      const int key = k0 + j;
      s[j] = (key >= N || (CAUSAL && key > myq)) ? -INFINITY : dot * a.scale;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;        // nothing visible yet for this row
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float p = (s[j] == -INFINITY) ? 0.f : expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, vs[j][c], o[c]);
    }
    m = m_new;
  }
  if (myq < N) {
    float* orow = a.out0 + base + (int64_t)myq * rs;
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) orow[c] = o[c] * inv;
    a.out1[(int64_t)bh * N + myq] = m + logf(l);
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

// dK, dV for 64 keys (one per thread), walking every query that can see them.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void bwd_dkdv_f32_kernel(F32Args a) {
  __shared__ float qs[kTile][D];
  __shared__ float gs[kTile][D];
  __shared__ float kv[2][kRows][D + 1];
  __shared__ float ls[kTile], ds[kTile];
  int bh, tile;
  int64_t base;
  bh_coords<D>(a, bh, tile, base);
  const int N = a.N, tid = threadIdx.x;
  const int64_t rs = (int64_t)a.H * D;
  const int k0 = tile * kRows;
  const int myk = k0 + tid;
  for (int idx = tid; idx < kRows * D; idx += kRows) {
    const int r = idx / D, c = idx % D;
    const int key = min(k0 + r, N - 1);
    kv[0][r][c] = a.k[base + (int64_t)key * rs + c];
    kv[1][r][c] = a.v[base + (int64_t)key * rs + c];
  }
  float dk[D], dv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) { dk[c] = 0.f; dv[c] = 0.f; }
  const float* lse = a.lse + (int64_t)bh * N;
  const float* dvec = a.dvec + (int64_t)bh * N;
  const int qstart = CAUSAL ? (k0 / kTile) * kTile : 0;
  for (int i0 = qstart; i0 < N; i0 += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += kRows) {
      const int r = idx / D, c = idx % D;
      const int qi = min(i0 + r, N - 1);
      qs[r][c] = a.q[base + (int64_t)qi * rs + c];
      gs[r][c] = a.dout[base + (int64_t)qi * rs + c];
    }
    if (tid < kTile) {
      const int qi = min(i0 + tid, N - 1);
      ls[tid] = lse[qi];
      ds[tid] = dvec[qi];
    }
    __syncthreads();
    for (int r = 0; r < kTile; ++r) {
      const int qi = i0 + r;
      if (qi >= N || (CAUSAL && myk > qi)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = __builtin_fmaf(qs[r][c], kv[0][tid][c], s);
        dp = __builtin_fmaf(gs[r][c], kv[1][tid][c], dp);
      }
      const float p = expf(s * a.scale - ls[r]);
      const float dsv = p * (dp - ds[r]);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        dv[c] = __builtin_fmaf(p, gs[r][c], dv[c]);
        dk[c] = __builtin_fmaf(dsv, qs[r][c], dk[c]);
      }
    }
  }
  if (myk < N) {
    float* dkrow = a.out0 + base + (int64_t)myk * rs;
    float* dvrow = a.out1 + base + (int64_t)myk * rs;
#pragma unroll
    for (int c = 0; c < D; ++c) { dkrow[c] = dk[c] * a.scale; dvrow[c] = dv[c]; }
  }
}

// dQ for 64 queries (one per thread), walking every key they can see.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void bwd_dq_f32_kernel(F32Args a) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  __shared__ float qg[2][kRows][D + 1];
  int bh, tile;
  int64_t base;
  bh_coords<D>(a, bh, tile, base);
  const int N = a.N, tid = threadIdx.x;
  const int64_t rs = (int64_t)a.H * D;
  const int q0 = tile * kRows;
  const int myq = q0 + tid;
  for (int idx = tid; idx < kRows * D; idx += kRows) {
    const int r = idx / D, c = idx % D;
    const int qi = min(q0 + r, N - 1);
    qg[0][r][c] = a.q[base + (int64_t)qi * rs + c];
    qg[1][r][c] = a.dout[base + (int64_t)qi * rs + c];
  }
  const int qc = min(myq, N - 1);
  const float lse = a.lse[(int64_t)bh * N + qc];
  const float dvl = a.dvec[(int64_t)bh * N + qc];
  float dq[D];
#pragma unroll
  for (int c = 0; c < D; ++c) dq[c] = 0.f;
  const int kend = CAUSAL ? min(N, q0 + kRows) : N;
  for (int k0 = 0; k0 < kend; k0 += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += kRows) {
      const int r = idx / D, c = idx % D;
      const int key = min(k0 + r, N - 1);
      ks[r][c] = a.k[base + (int64_t)key * rs + c];
      vs[r][c] = a.v[base + (int64_t)key * rs + c];
    }
    __syncthreads();
    for (int j = 0; j < kTile; ++j) {
      const int key = k0 + j;
      if (key >= N || (CAUSAL && key > myq)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = __builtin_fmaf(qg[0][tid][c], ks[j][c], s);
        dp = __builtin_fmaf(qg[1][tid][c], vs[j][c], dp);
      }
      const float p = expf(s * a.scale - lse);
      const float dsv = p * (dp - dvl);
#pragma unroll
      for (int c = 0; c < D; ++c) dq[c] = __builtin_fmaf(dsv, ks[j][c], dq[c]);
    }
  }
  if (myq < N) {
    float* row = a.out0 + base + (int64_t)myq * rs;
#pragma unroll
    for (int c = 0; c < D; ++c) row[c] = dq[c] * a.scale;
  }
}

template <int D>
hipError_t fwd(const F32Args& a, int BH, int causal, hipStream_t st) {
  const dim3 grid(a.ntiles * BH), block(kRows);
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
  const dim3 grid(a.ntiles * BH), block(kRows);
  F32Args a1 = a;   // dK/dV pass: out0 = dK, out1 = dV
  if (causal) hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, true>), grid, block, 0, st, a1);
  else hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, false>), grid, block, 0, st, a1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return e;
}

template <int D>
hipError_t bwd_dq(const F32Args& a, int BH, int causal, hipStream_t st) {
  const dim3 grid(a.ntiles * BH), block(kRows);
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
