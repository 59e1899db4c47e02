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
// gfx950 mapping (32 query rows per wave; 64 keys a step):
//  * S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16 so that each lane
//    of a wave owns one query row (column of S^T) and 16 of every 32 keys; the
//    per-row softmax state lives in that lane and only the row max needs one
//    exchange between the two half-waves (v_permlane32_swap).
//  * The fp32 S^T accumulator, exponentiated and rounded to bf16, is directly
//    the B operand of O^T += V^T P^T: no LDS round trip for P.
//  * V^T fragments come from row-major V tiles in LDS through the transposing
//    read ds_read_b64_tr_b16; K fragments are plain 16-byte LDS reads.  Tile
//    rows are dense with XOR-permuted 16-byte chunks (no bank conflicts for
//    either read); every fragment address is a lane base XOR a constant.
//  * K and V tiles live in LDS rings filled by asynchronous global -> LDS
//    copies (no staging registers).  The loop form depends on the head size
//    (fwd_mode): at d = 64 one workgroup of 4 waves takes one tile per step
//    (scores, softmax, P V) with one barrier per step; at d = 128 a workgroup
//    of 8 waves pairs the two waves of each SIMD in opposite phases, so that
//    one runs its matrix products while the other runs its softmax.
//  * V^T is read with asm-issued transposing reads: the compiler would wait
//    for every copy in flight before the builtin form of that read.
//  * exp is exp2 with scale*log2(e) folded into one FMA.  The reference max is
//    only moved when a row's max grows by more than 2^8 (kRescaleLog2), or,
//    in the unmasked steps of most forms, when a row's share of the sum
//    exceeds 2^16 (the row max is then not computed at all): any
//    finite reference gives the same O and LSE (the final divide uses the same
//    reference), so this keeps exactness while the O rescale becomes rare.
//  * Causal: tiles above the diagonal are never visited; waves whose 32 rows
//    cannot see any key of a step skip it; only steps that straddle the
//    diagonal (or the ragged end of the keys) evaluate the mask.
//  * Workgroups are renumbered per XCD so whole heads share an L2; causal
//    query tiles go out heaviest first across the heads of an XCD.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBc = 64;            // keys per step
constexpr float kRescaleLog2 = 8.0f;
constexpr float kSumLimit = 65536.0f;
// Loop form per instantiation (measured on MI355X):
//  0  one tile per step: scores, softmax and P V of tile t, 4 waves per
//     workgroup, several workgroups per CU (D = 64: pairing waves by phase
//     measured slower);
//  3  ping-pong: 8 waves, two per SIMD in opposite phases; while one wave of
//     a SIMD runs the products of its step (S(t) and P V of tile t-1) the
//     other runs the softmax of its tile, and barriers swap the roles
//     (D = 128).  Waves of one SIMD that share a phase compete for the same
//     pipe; a probe of the two arrangements measured 3400 against 2100
//     cycles for two d = 128 steps.
//  With dropout (DROP) every head size takes loop 0.
template <int D, bool CAUSAL, bool DROP = false>
constexpr int fwd_mode() { return D == 128 && !DROP ? 3 : 0; }
// Waves per workgroup (32 query rows each) and per SIMD (registers: 128,
// 256 or, at D = 256, all 512; its four 32 KB K and V buffers also fill the
// LDS of a CU with one workgroup).  D = 64 runs 4 waves per SIMD: 2% faster
// on MI355X than 3 (168 registers), although a few loop-invariant values
// (used after the loop) then go to scratch; with dropout (the generator
// needs registers) it keeps 3.
// The one-tile-per-step loop at D = 64 without a mask takes 8 waves (256
// rows, half the copy instructions per row; 3% faster on MI355X than 4); with
// the mask the waves of a 256-row tile that finish their diagonal early
// would idle through the rest (3% slower), so it keeps 4.
// At D = 256 without dropout an 8-wave form (two waves per SIMD over the same
// 128 KB of K and V buffers, 37 dwords spilled) is chosen at run time for
// grids of at least kWide256Grid of its workgroups: 4-7% faster on MI355X
// there, and up to 37% slower on small grids, which have half as many
// workgroups as with 4 waves.
template <int D, bool CAUSAL, bool DROP = false>
constexpr int fwd_wg_waves() { return fwd_mode<D, CAUSAL, DROP>() == 3 || (D == 64 && !CAUSAL && !DROP) ? 8 : 4; }
template <int D, bool DROP, int W = 4>
constexpr int fwd_waves() { return D == 64 ? (DROP ? 3 : 4) : D == 128 ? 2 : (W == 8 ? 2 : 1); }
constexpr int kWide256Grid = 512;
// How unmasked steps after the first keep the reference max: lazily (P
// against the current reference first, the row max only when a row's share
// of the sum exceeds 2^16, then the step redone) or eagerly (the row max
// first, the reference moved when it grows by more than 2^8, one pass of
// exponentials).  The lazy form saves the max at D = 64 and 128 and at
// D = 256 without the mask; under the mask at D = 256 (12-15% faster) and
// with dropout (2-6%) the redo path's second copy of the exponentials (and
// of the generator calls) costs more registers than the max (measured on
// MI355X).
template <int D, bool CAUSAL, bool DROP>
constexpr bool fwd_eager_max() { return (D == 256 && CAUSAL) || DROP; }

// Buffer index carried by a step's buffer tag: the constant of a
// compile-time tag, 0 for a run-time one (whose offset is in the pointer).
template <class T>
constexpr int buffer_index() {
  if constexpr (std::is_same_v<T, int>) return 0;
  else return T::value;
}

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int H, N, nqt, BH;   // N: query rows per head
  int Nk;               // key rows per head
  int qoff;             // sequence position of query row 0 (causal: Nk - N)
  float c;   // scale * log2(e)
  DropParams drop;   // used by the DROP instantiations only
};

template <int D, bool CAUSAL, bool DROP, int WGW = fwd_wg_waves<D, CAUSAL, DROP>()>
__global__ __launch_bounds__((64 * WGW), (fwd_waves<D, DROP, WGW>())) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int KS = D / 16;           // k-steps of the score product
  constexpr int DT = D / 32;           // 32-wide output tiles
  constexpr int RB = D * 2;            // bytes per LDS row (dense, chunks swizzled)
  constexpr int TILE = kBc * RB;       // bytes of one K or V tile
  constexpr int MODE = fwd_mode<D, CAUSAL, DROP>();
  constexpr int kWaves = WGW;
  static_assert(MODE == 0 || kWaves == 8, "the ping-pong loop takes 8 waves");
  constexpr int kBr = 32 * kWaves;     // query rows per workgroup
  constexpr int CPW = TILE / 1024 / kWaves;   // 1 KB global->LDS copies per wave per tile
  // Mode 0 keeps a ring of NB tiles: copies run NB - 1 tiles ahead.  Two
  // are enough: at D = 64 a ring of three (48 KB of LDS, three workgroups
  // per CU still fit) measured the same time on MI355X (within 0.5%).
  constexpr int NB = 2;
  constexpr int NK = MODE == 3 ? 4 : NB;  // K buffers
  constexpr int NV = NK;                  // V buffers
  __shared__ __attribute__((aligned(1024))) char smem[(NK + NV) * TILE];   // K buffers, then V buffers

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;

  int bh, qt;
  tile_of(blockIdx.x, a.nqt, a.BH, CAUSAL, true, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.N, Nk = a.Nk, qoff = a.qoff;
  const int64_t rs = (int64_t)a.H * D;                       // row stride (elements)
  const int64_t base = ((int64_t)b * N * a.H + h) * D;       // Q and O
  const int64_t kvbase = ((int64_t)b * Nk * a.H + h) * D;    // K and V
  const __bf16* __restrict__ Qg = a.q + base;
  const __bf16* __restrict__ Kg = a.k + kvbase;
  const __bf16* __restrict__ Vg = a.v + kvbase;

  const int q0 = qt * kBr;
  // Mode 3: waves 0-3 take 32-row blocks 0, 2, 4, 6 of the tile and waves 4-7
  // blocks 1, 3, 5, 7, so both halves reach the diagonal together.
  // Scalar (readfirstlane): the per-wave causal tests on it then compile to
  // scalar branches instead of exec-mask regions (1% on the d = 64 causal
  // forward on MI355X).
  const int qw0 = __builtin_amdgcn_readfirstlane(q0 + 32 * (MODE == 3 ? 2 * (wave & 3) + (wave >> 2) : wave));
  const int myq = qw0 + l32;

  // Q^T operand for this lane's row: chunk 2*ks + hh of the row, per k-step.
  bf16x8 qf[KS];
  {
    const __bf16* qrow = Qg + (int64_t)min(myq, N - 1) * rs;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + hh) * 8);
  }

  const int kend = CAUSAL ? min(Nk, q0 + qoff + kBr) : Nk;
  const int nkt = (kend + kBc - 1) / kBc;

  // Staging: copy i of this wave fills LDS block (wave + 4 i) of a tile; lane
  // l's 16 bytes are physical chunk slot%CH of row slot/CH (slot = 64 block + l),
  // which holds logical chunk (slot%CH) ^ swz(row) of that key row.  The copies
  // go through a buffer descriptor that covers exactly the valid rows of the
  // tile, so rows past N read as zeros (they are masked anyway); the per-lane
  // byte offsets are the same for every tile.
  uint32_t svoff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int slot = (wave + kWaves * i) * 64 + lane;
    const int row = slot / CH;
    svoff[i] = (uint32_t)(row * rs * 2) + (uint32_t)(((slot % CH) ^ swz<D>(row)) * 16);
  }
  // LDS: NK K buffers, then NV V buffers (two each for the plain loop, four
  // for the ping-pong loop).
  char* const kbuf = smem;
  char* const vbuf = smem + NK * TILE;
  // Byte offset of this wave's first 1 KB block, as a wave-uniform (scalar) value.
  const int wblk = __builtin_amdgcn_readfirstlane(wave * 1024);
  auto stage_rows = [&](const __bf16* src, int kt, char* dst) __attribute__((always_inline)) {
    const int rows = min(Nk - kt * kBc, kBc);
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(src + (int64_t)kt * kBc * rs, (uint32_t)(rows * rs * 2));
#pragma unroll
    for (int i = 0; i < CPW; ++i) buffer_to_lds16(rsrc, svoff[i], dst + wblk + kWaves * i * 1024);
  };

  // Lane bases of the fragment reads.  The chunk field of an address (bits
  // 4 .. 4+log2(CH)-1) is zero in the row part, so swizzled addresses are the
  // lane base XOR a per-read constant, plus an immediate row offset.
  //  K (A operand of S^T): row 32 j + l%32, logical chunk 2 ks + l/32.
  const uint32_t kl = (uint32_t)(l32 * RB) | ((uint32_t)(hh ^ swz<D>(l32)) << 4);
  //  V^T (A operand of O^T), transposing read: within each group of 16 lanes,
  //  lane i addresses row 32 j + 16 u + r4 (+8 for the high half), r4 =
  //  4 (l/32) + i/4, and element column 32 t + 16 ((l/16)%2) + 4 (i%4).
  uint32_t vl;
  {
    const int ti = lane & 15, tg = lane >> 4;
    const int r4 = (tg >> 1) * 4 + (ti >> 2);
    const int cl = (tg & 1) * 2 + ((ti & 3) >> 1);
    const int sw0 = swz<D>(r4);
    vl = (uint32_t)(r4 * RB) | ((uint32_t)(cl ^ sw0) << 4) | ((uint32_t)(ti & 1) << 3);
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = (f32x16){};
  float m_ref = -INFINITY;   // reference max, log2 units
  float l_part = 0.f;        // this half-wave's share of the row sum
  const float c = a.c;

  // Moves the reference max to the exact running max of the rows (in log2
  // units) and rescales the running sum and output to it.
  auto move_reference = [&](f32x16 (&s)[2]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_ref, (mx == -INFINITY) ? -INFINITY : mx * c);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
    l_part *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
    m_ref = m_new;
  };

  // P = exp2(c S - m_ref) for one step, its row-sum share, and bf16 operands.
  // With dropout the operands carry P of the kept elements of the step's keys
  // (k0 ..) and 0 for the dropped ones (the keep multiplier is applied to O
  // once, at the end), while the row sum takes P itself.
  auto exp_tile = [&](auto mask_tag, const f32x16 (&s)[2], bf16x8 (&pb)[2][2], int k0) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const float nm = -m_ref;
    float lsum[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = fast_exp2(__builtin_fmaf(s[j][r], c, nm));
        if constexpr (MASK) e = (s[j][r] == -INFINITY) ? 0.f : e;
        p[r] = e;
        lsum[r & 1] += e;
      }
      if constexpr (DROP) {
        // register 4 g + e holds key k0 + 32 j + 8 g + 4 hh + e; one call
        // serves registers 8 c .. 8 c + 7 (groups g = 2c, 2c + 1)
#pragma unroll
        for (int c = 0; c < 2; ++c) drop_zero8(a.drop, bh, myq, k0 + 32 * j + 16 * c + 4 * hh, p + 8 * c);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        pb[j][u] = pack_bf16x8(p[8 * u + 0], p[8 * u + 1], p[8 * u + 2], p[8 * u + 3],
                               p[8 * u + 4], p[8 * u + 5], p[8 * u + 6], p[8 * u + 7]);
    }
    return lsum[0] + lsum[1];
  };

  // Softmax update for one step: P (bf16 operands) of the step's scores.
  //  MASK steps (diagonal or ragged end) hide keys and move the reference to
  //  the exact running max when it grows by more than 2^8.
  //  Other steps, in the lazy form, exponentiate against the current
  //  reference straight away and only look at the row max (and redo the
  //  step) if some row's share of the sum exceeds 2^16, which bounds every
  //  probability by 2^16; in the eager form (fwd_eager_max) they look at the
  //  row max first, as MASK steps do.
  //  The first step of a wave, when no key of it is hidden (mask_tag of
  //  value 2), sets the reference to the row max before exponentiating: the
  //  reference is -inf before it, so exponentiating first would always redo
  //  the step, and nothing has been accumulated yet to rescale.
  //  A move of the reference rescales the output accumulated so far.
  auto softmax_tile = [&](auto mask_tag, f32x16 (&s)[2], int k0, bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
    constexpr int MT = (int)decltype(mask_tag)::value;
    float lsum;
    if constexpr (MT == 2) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
      m_ref = max_halves(mx) * c;
      lsum = exp_tile(std::false_type{}, s, pb, k0);
    } else if constexpr (MT == 1) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * j + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool hide = key >= Nk || (CAUSAL && key > myq + qoff);
          s[j][r] = hide ? -INFINITY : s[j][r];
        }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
      mx = max_halves(mx);
      const float mcand = (mx == -INFINITY) ? -INFINITY : mx * c;
      if (__any(fmaxf(m_ref, mcand) > m_ref + kRescaleLog2)) move_reference(s);
      lsum = exp_tile(std::true_type{}, s, pb, k0);
    } else if constexpr (fwd_eager_max<D, CAUSAL, DROP>()) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
      if (__any(max_halves(mx) * c > m_ref + kRescaleLog2)) move_reference(s);
      lsum = exp_tile(std::false_type{}, s, pb, k0);
    } else {
      lsum = exp_tile(std::false_type{}, s, pb, k0);
      if (__any(!(lsum <= kSumLimit))) {
        move_reference(s);
        lsum = exp_tile(std::false_type{}, s, pb, k0);
      }
    }
    l_part += lsum;
  };

  // O^T += V^T P^T for one step, in four groups g = (j, u) of DT products;
  // with D = 64 the V^T reads of group g+1 are in flight while group g's
  // products issue.
  auto pv_tile = [&](const char* vb, const bf16x8 (&pb)[2][2], auto off_tag) __attribute__((always_inline)) {
    constexpr uint32_t BOFF = decltype(off_tag)::value;
    const uint32_t vbase = lds_addr(vb);
    s16x4 rd[4][DT][2];
    auto issue = [&](auto G) __attribute__((always_inline)) {
      constexpr int g = decltype(G)::value;
      constexpr uint32_t rowoff = (uint32_t)(16 * g * RB);
      static_for<0, DT>([&](auto T) {
        constexpr int t = decltype(T)::value;
        rd[g][t][0] = lds_tr16_issue<BOFF + rowoff>(vbase + (vl ^ (64 * t)));
        rd[g][t][1] = lds_tr16_issue<BOFF + rowoff + 8 * RB>(vbase + (vl ^ (64 * t + 32)));
      });
    };
    auto consume = [&](auto G) __attribute__((always_inline)) {
      constexpr int g = decltype(G)::value;
      static_for<0, DT>([&](auto T) {
        constexpr int t = decltype(T)::value;
        oacc[t] = mfma32x32x16(tr_pair_take(rd[g][t]), pb[g >> 1][g & 1], oacc[t]);
      });
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    if constexpr (D == 64) {
      issue(I0{});
      issue(I1{});
      lds_wait<2 * DT>();
      consume(I0{});
      issue(I2{});
      lds_wait<2 * DT>();
      consume(I1{});
      issue(I3{});
      lds_wait<2 * DT>();
      consume(I2{});
      lds_wait<0>();
      consume(I3{});
    } else {
      // d = 128: one group in flight (registers are the limit here).
      issue(I0{});
      lds_wait<0>();
      consume(I0{});
      issue(I1{});
      lds_wait<0>();
      consume(I1{});
      issue(I2{});
      lds_wait<0>();
      consume(I2{});
      issue(I3{});
      lds_wait<0>();
      consume(I3{});
    }
  };

  auto softmax_pv = [&](auto mask_tag, f32x16 (&s)[2], const char* vb, auto off_tag, int k0) __attribute__((always_inline)) {
    bf16x8 pb[2][2];
    softmax_tile(mask_tag, s, k0, pb);
    pv_tile(vb, pb, off_tag);
  };

  // S^T = K Q^T for the two 32-key sub-tiles of a K buffer (independent
  // accumulation chains interleaved).
  auto scores = [&](const char* kb, f32x16 (&s)[2]) __attribute__((always_inline)) {
    s[0] = (f32x16){};
    s[1] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        s[j] = mfma32x32x16(lds_read_b128(kb, (kl ^ (ks << 5)) + 32 * j * RB), qf[ks], s[j]);
  };

  if constexpr (MODE == 3) {
    // Ping-pong.  Global phase p ends with a workgroup barrier.  Waves 0-3
    // (half A) run the products of step t in phase 2t and the softmax of tile
    // t in phase 2t+1; waves 4-7 (half B; wave w and wave w+4 share a SIMD)
    // run the same sequence one phase later.  The products of step t are
    // S(t) = K(t) Q^T and P V of tile t-1 (the softmax of tile t-1 ran in
    // between), so a move of the reference in softmax(t) rescales O after
    // P V of tile t-1 has been added, as in the plain loop.  The product
    // phases run at a raised wave priority so that the matrix pipe, not the
    // other wave's vector work, gets the issue slots.
    const int half = __builtin_amdgcn_readfirstlane(wave >> 2);
    const int nlast = __builtin_amdgcn_readfirstlane(CAUSAL ? min(nkt - 1, (qw0 + qoff + 31) / kBc) : nkt - 1);
    // Phase barriers are asm so that no release fence drains the copies in
    // flight; the memory clobber keeps LDS accesses on their side.
    auto phase_end = [] {
      __builtin_amdgcn_sched_barrier(0);
      sync_check_drain();
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // Copies run two tiles ahead through four buffers each (tile t in buffer
    // t & 3).  Batch t (K(t+2) and V(t+1)) is issued at the end of a softmax
    // phase, after the vector work: by half B in phase 2t, by half A in
    // phase 2t+1.  The barrier ending phase 2t+1 leaves only each wave's
    // latest batch in flight (s_waitcnt vmcnt(2 CPW)), so batch t-1, which
    // the products of step t+1 read from phase 2t+2 on, is complete; the
    // buffers batch t overwrites were last read in phase 2t-1.  Every batch
    // is 2 CPW copies per wave: a tile past the last one is copied from an
    // empty range (no memory is read) into a buffer nobody reads again, so
    // the count of copies in flight is the same every phase.
    auto stage_or_skip = [&](const __bf16* src, int kt, char* dst) __attribute__((always_inline)) {
      const bool real = kt < nkt;
      const int rows = real ? min(Nk - kt * kBc, kBc) : 0;
      const __amdgpu_buffer_rsrc_t rsrc =
          make_rsrc(src + (int64_t)(real ? kt : 0) * kBc * rs, (uint32_t)(rows * rs * 2));
#pragma unroll
      for (int i = 0; i < CPW; ++i) buffer_to_lds16(rsrc, svoff[i], dst + wblk + kWaves * i * 1024);
    };
    auto copies = [&](int t) __attribute__((always_inline)) {
      stage_or_skip(Kg, t + 2, kbuf + ((t + 2) & 3) * TILE);
      stage_or_skip(Vg, t + 1, vbuf + ((t + 1) & 3) * TILE);
    };
    // Ends phase 2t+1: every copy but this wave's latest batch is complete.
    auto phase_end_publish = [&] __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vmem_n<2 * CPW>();
      sync_check_drain();
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    f32x16 sc[2];
    bf16x8 pb[2][2];
    // Products of step t: S(t) = K(t) Q^T when PK & 1, P V of tile t-1 when
    // PK & 2.  PK = 3: P V products on even slots, score products on odd
    // ones, LDS operands read L slots ahead; PK = 7: both, one after the
    // other (fewer registers, for the few masked steps).
    auto products = [&](int t, auto pk_tag) __attribute__((always_inline)) {
      constexpr int PK = decltype(pk_tag)::value;
      const char* kb = kbuf + (t & 3) * TILE;
      const char* vb = vbuf + ((t + 3) & 3) * TILE;
      if constexpr (PK == 3) {
        constexpr int NPV = 4 * DT, NM = 2 * NPV;
        static_assert(2 * KS == NPV, "as many S products as P V products");
        const uint32_t vbase = lds_addr(vb), kbase = lds_addr(kb);
        constexpr int L = 4;
        s16x4 rv[NPV][2];
        bf16x8 rk[NPV];
        auto issue = [&](auto I) __attribute__((always_inline)) {
          constexpr int i = decltype(I)::value;
          if constexpr ((i & 1) == 0) {
            constexpr int pidx = i >> 1, g = pidx / DT, tt = pidx % DT;
            constexpr uint32_t rowoff = (uint32_t)(16 * g * RB);
            rv[pidx][0] = lds_tr16_issue<rowoff>(vbase + (vl ^ (64 * tt)));
            rv[pidx][1] = lds_tr16_issue<rowoff + 8 * RB>(vbase + (vl ^ (64 * tt + 32)));
          } else {
            constexpr int q = i >> 1, ks = q >> 1, j = q & 1;
            rk[q] = lds_b128_issue<(uint32_t)(32 * j * RB)>(kbase + (kl ^ (ks << 5)));
          }
        };
        static_for<0, L>([&](auto I) { issue(I); });
        static_for<0, NM>([&](auto I) {
          constexpr int i = decltype(I)::value;
          if constexpr (i + L < NM) issue(std::integral_constant<int, i + L>{});
          constexpr int after = [] {
            int n = 0;
            for (int sl = i + 1; sl <= (i + L < NM - 1 ? i + L : NM - 1); ++sl) n += (sl & 1) ? 1 : 2;
            return n;
          }();
          lds_wait<after>();
          if constexpr ((i & 1) == 0) {
            constexpr int pidx = i >> 1, g = pidx / DT, tt = pidx % DT;
            oacc[tt] = mfma32x32x16(tr_pair_take(rv[pidx]), pb[g >> 1][g & 1], oacc[tt]);
          } else {
            constexpr int q = i >> 1, ks = q >> 1, j = q & 1;
            lds_ready(rk[q]);
            sc[j] = mfma32x32x16(rk[q], qf[ks], ks == 0 ? (f32x16){} : sc[j]);
          }
        });
      } else {
        if constexpr ((PK & 2) != 0) pv_tile(vb, pb, std::integral_constant<uint32_t, 0>{});
        if constexpr ((PK & 1) != 0) scores(kb, sc);
        static_assert(PK < 4 || PK == 7, "product kind");
      }
    };
    // Softmax of tile t: SK = 0 none, 1 every key visible, 2 masked, 4 the
    // wave's first step with every key visible.
    auto softmax = [&](int t, auto sk_tag) __attribute__((always_inline)) {
      constexpr int SK = decltype(sk_tag)::value;
      if constexpr (SK == 1) softmax_tile(std::false_type{}, sc, t * kBc, pb);
      if constexpr (SK == 2) softmax_tile(std::true_type{}, sc, t * kBc, pb);
      if constexpr (SK == 4) softmax_tile(std::integral_constant<int, 2>{}, sc, t * kBc, pb);
    };
    // One step: the products of step t, then the softmax of tile t, each
    // ending with its phase barrier.
    auto step = [&](int t, auto pk_tag, auto sk_tag) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(1);
      products(t, pk_tag);
      __builtin_amdgcn_s_setprio(0);
      if (half == 0) phase_end();
      else phase_end_publish();
      softmax(t, sk_tag);
      copies(t + half);
      if (half == 0) phase_end_publish();
      else phase_end();
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    using P4 = std::integral_constant<int, 4>;
    using P7 = std::integral_constant<int, 7>;
    // Leading tiles every key of which this wave's rows see.
    const int nfree = __builtin_amdgcn_readfirstlane(
        CAUSAL ? min((qw0 + qoff + 1) / kBc, Nk / kBc) : Nk / kBc);
    stage_rows(Kg, 0, kbuf);
    wait_vmem();
    block_sync();
    stage_or_skip(Kg, 1, kbuf + TILE);
    stage_or_skip(Vg, 0, vbuf);
    // Half B starts one phase late (phase 0 idle); the sections below keep
    // one path per loop body.
    if (half == 1) {
      copies(0);
      phase_end();
    }
    if (nfree > 0) step(0, P1{}, P4{});
    else step(0, P1{}, P2{});
    int t = 1;
    for (; t < nfree; ++t) step(t, P3{}, P1{});
    for (; t <= nlast; ++t) step(t, P7{}, P2{});
    // t = nlast + 1: P V of this wave's last tile; later steps only copy
    // and keep the barrier count.
    if (t < nkt) {
      step(t, P2{}, P0{});
      for (++t; t < nkt; ++t) step(t, P0{}, P0{});
      products(nkt, P0{});
    } else {
      products(nkt, P2{});
    }
    if (half == 0) phase_end();
    wait_vmem();              // no copy may land after the workgroup ends
  } else {
    // A ring of NB buffers for K and NB for V (tile t in buffer t % NB):
    // step t copies tile t + NB - 1 while it computes scores, softmax and
    // P V of tile t.  With NB = 3 every step issues one batch of 2 CPW copies
    // per wave (a tile past the last one is copied from an empty range, which
    // reads no memory, into a buffer no step reads again), so waiting until
    // one batch is left in flight completes tile t.  The buffer a step fills
    // was last read in the step before, which every wave has left at the
    // step's barrier.
    auto stage_or_skip = [&](const __bf16* src, int kt, char* dst) __attribute__((always_inline)) {
      const bool real = kt < nkt;
      const int rows = real ? min(Nk - kt * kBc, kBc) : 0;
      const __amdgpu_buffer_rsrc_t rsrc =
          make_rsrc(src + (int64_t)(real ? kt : 0) * kBc * rs, (uint32_t)(rows * rs * 2));
#pragma unroll
      for (int i = 0; i < CPW; ++i) buffer_to_lds16(rsrc, svoff[i], dst + wblk + kWaves * i * 1024);
    };
    stage_rows(Kg, 0, kbuf);
    stage_rows(Vg, 0, vbuf);
    if constexpr (NB == 3) {
      stage_or_skip(Kg, 1, kbuf + TILE);
      stage_or_skip(Vg, 1, vbuf + TILE);
    }
    // Step kt; `cur_tag` is the buffer holding tile kt (kt % NB), a
    // compile-time constant in the unrolled loops so that the buffer's LDS
    // offset is an immediate of every fragment read.
    auto step = [&](int kt, auto mask_tag, auto cur_tag) __attribute__((always_inline)) {
      constexpr bool CT = !std::is_same_v<decltype(cur_tag), int>;
      const int cur = cur_tag;
      if constexpr (NB == 3) {
        wait_vmem_n<2 * CPW>();
        block_sync();
        const int nxt = cur == 0 ? 2 : cur - 1;   // (cur + 2) % 3
        stage_or_skip(Kg, kt + 2, kbuf + nxt * TILE);
        stage_or_skip(Vg, kt + 2, vbuf + nxt * TILE);
      } else {
        wait_vmem();
        block_sync();
        if (kt + 1 < nkt) {
          stage_rows(Kg, kt + 1, kbuf + (cur ^ 1) * TILE);
          stage_rows(Vg, kt + 1, vbuf + (cur ^ 1) * TILE);
        }
      }
      const int k0 = kt * kBc;
      if (CAUSAL && k0 > qw0 + qoff + 31) return;
      f32x16 sc[2];
      scores(kbuf + cur * TILE, sc);
      const char* vb = CT ? vbuf : vbuf + cur * TILE;
      using Off = std::integral_constant<uint32_t, (uint32_t)(buffer_index<decltype(cur_tag)>() * TILE)>;
      softmax_pv(mask_tag, sc, vb, Off{}, k0);
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    // Unmasked steps kt .. end - 1 from kt = 0, NB per iteration.
    auto run_free = [&](int& kt, int end) __attribute__((always_inline)) {
      using First = std::integral_constant<int, 2>;
      if constexpr (NB == 3) {
        if (kt < end) step(kt++, First{}, B0{});
        if (kt < end) step(kt++, std::false_type{}, B1{});
        for (; kt + 2 < end; kt += 3) {
          step(kt, std::false_type{}, B2{});
          step(kt + 1, std::false_type{}, B0{});
          step(kt + 2, std::false_type{}, B1{});
        }
        if (kt < end) step(kt++, std::false_type{}, B2{});
        if (kt < end) step(kt++, std::false_type{}, B0{});
      } else if constexpr (D == 64) {
        // the loop keeps buffer 0 first (measured faster at this width)
        if (kt < end) step(kt++, First{}, B0{});
        if (kt < end) step(kt++, std::false_type{}, B1{});
        for (; kt + 1 < end; kt += 2) {
          step(kt, std::false_type{}, B0{});
          step(kt + 1, std::false_type{}, B1{});
        }
        if (kt < end) step(kt++, std::false_type{}, B0{});
      } else {
        if (kt < end) step(kt++, First{}, B0{});
        for (; kt + 1 < end; kt += 2) {
          step(kt, std::false_type{}, B1{});
          step(kt + 1, std::false_type{}, B0{});
        }
        if (kt < end) step(kt++, std::false_type{}, B1{});
      }
    };
    int kt = 0;
    if constexpr (CAUSAL) {
      // Sections with one softmax path each: first the tiles every key of
      // which all rows of this wave see (no mask); then the tiles that
      // straddle the wave's diagonal or the ragged end of the keys (masked),
      // and the tiles past its diagonal (skipped).
      run_free(kt, __builtin_amdgcn_readfirstlane(min((qw0 + qoff + 1) / kBc, Nk / kBc)));
    } else {
      // Without a mask only a ragged last tile hides keys, so the loop over
      // the full tiles has a single softmax path.  With the masked path as a
      // branch inside the loop, the compiler kept O in two register sets and
      // copied it twice per step (a fifth of the d = 128 loop's time).
      run_free(kt, Nk / kBc);
    }
    for (; kt < nkt; ++kt) step(kt, std::true_type{}, kt % NB);
    if constexpr (NB == 3) wait_vmem();   // no copy may land after the workgroup ends
  }

  // ---- epilogue: O = O_acc / l (with dropout inv_keep O_acc / l), LSE = ln2 * (m + log2 l)
  const float l = sum_halves(l_part);
  if (myq < N) {
    const float inv = (DROP ? a.drop.inv_keep : 1.f) / l;
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

template <int D, bool CAUSAL, bool DROP, int W = fwd_wg_waves<D, CAUSAL, DROP>()>
hipError_t launch(FwdArgs args, int BH, hipStream_t stream) {
  args.nqt = (args.N + 32 * W - 1) / (32 * W);
  const int grid = args.nqt * BH;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, DROP, W>), dim3(grid), dim3(64 * W), 0, stream, args);
  return hipGetLastError();
}

template <bool DROP>
hipError_t launch_any(const FwdArgs& a, const AttnShape& s, hipStream_t stream) {
  const int BH = s.B * s.H;
  if (s.d == 64) return s.causal ? launch<64, true, DROP>(a, BH, stream) : launch<64, false, DROP>(a, BH, stream);
  if (s.d == 256) {
    if constexpr (!DROP) {
      if ((int64_t)((s.N + 255) / 256) * BH >= kWide256Grid)
        return s.causal ? launch<256, true, false, 8>(a, BH, stream) : launch<256, false, false, 8>(a, BH, stream);
    }
    return s.causal ? launch<256, true, DROP>(a, BH, stream) : launch<256, false, DROP>(a, BH, stream);
  }
  return s.causal ? launch<128, true, DROP>(a, BH, stream) : launch<128, false, DROP>(a, BH, stream);
}

FwdArgs make_fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, const AttnShape& s,
                      int Nk) {
  FwdArgs a{};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.H = s.H;
  a.N = s.N;
  a.Nk = Nk;
  a.qoff = s.causal ? Nk - s.N : 0;
  a.BH = s.B * s.H;
  a.c = s.scale * kLog2e;
  return a;
}

}  // namespace

hipError_t launch_fwd_cross_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const AttnShape& s, int Nk, hipStream_t stream) {
  return launch_any<false>(make_fwd_args(q, k, v, o, lse, s, Nk), s, stream);
}

hipError_t launch_fwd_dropout_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const AttnShape& s, const DropParams& drop, hipStream_t stream) {
  FwdArgs a = make_fwd_args(q, k, v, o, lse, s, s.N);
  a.drop = drop;
  return launch_any<true>(a, s, stream);
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const AttnShape& s, hipStream_t stream) {
  return launch_fwd_cross_bf16(q, k, v, o, lse, s, s.N, stream);
}

}  // namespace fa
